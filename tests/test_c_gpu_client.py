"""The device calls from plain C: tests/c_gpu_client.c (C99, the HIP runtime's
C API for memory and the stream, no torch) is built against include/dfa.h and
libdfa.so and run as a child process on the GPU; its fused forward and
backward over the folded schedule are checked against the oracle with the
parity tests' bounds."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from oracle import schedule_ref as sr
from tests.parity_util import bhnd, check_grad, check_out

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_sequence_dfa_amd")


def to_bits(x):
    """fp32 array holding bf16 values -> raw bf16 (uint16)."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def from_bits(u, shape):
    return (u.astype(np.uint32) << 16).view(np.float32).reshape(shape)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_client_forward_backward(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sequence_dfa_amd import inputs
    if not os.path.exists(os.path.join(PKG, "libdfa.so")):
        pytest.fail("libdfa.so is not built")
    exe = str(tmp_path / "client")
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-O1", "-D__HIP_PLATFORM_AMD__",
                           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "c_gpu_client.c"), "-L", PKG, "-ldfa",
                           "-L", "/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{PKG}",
                           "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    N, P, Hq, Hkv, D = 1024, 4, 4, 2, 128
    print(f"case: C client, folded schedule N={N} P={P} Hq={Hq} Hkv={Hkv} D={D} bf16", flush=True)
    q, k, v, do = inputs.workload_tensors(8100, 1, N, Hq, Hkv, D, "bf16", with_do=True)
    for name, x in (("q", q), ("k", k), ("v", v), ("do", do)):
        to_bits(x).tofile(str(tmp_path / f"{name}.bin"))
    r = subprocess.run([exe, str(tmp_path), str(N), str(P), str(Hq), str(Hkv)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    print(r.stdout.strip(), flush=True)
    o = from_bits(np.fromfile(str(tmp_path / "o.bin"), dtype=np.uint16), (1, N, Hq, D))
    lse = np.fromfile(str(tmp_path / "lse.bin"), dtype=np.float32).reshape(1, Hq, N)
    dq = from_bits(np.fromfile(str(tmp_path / "dq.bin"), dtype=np.uint16), (1, N, Hq, D))
    dk = from_bits(np.fromfile(str(tmp_path / "dk.bin"), dtype=np.uint16), (1, N, Hkv, D))
    dv = from_bits(np.fromfile(str(tmp_path / "dv.bin"), dtype=np.uint16), (1, N, Hkv, D))
    scale = 1 / np.sqrt(D)
    ro, rl = oracle.attn_rows(q, k, v, scale)
    ra, _ = oracle.attn_rows(q, k, np.abs(v), scale)
    check_out(bhnd(o), ro, lse, rl, "bf16", "C client O", oabs=ra, n_keys=N)
    (rdq, rdk, rdv), (aq, ak, av) = oracle.attn_grads(q, k, v, do, scale, with_abs=True)
    check_grad(bhnd(dq), rdq, aq, "bf16", "C client dq")
    check_grad(bhnd(dk), rdk, ak, "bf16", "C client dk")
    check_grad(bhnd(dv), rdv, av, "bf16", "C client dv")
    # the blocks the client built are the enumerator's
    assert f"{len(sr.enumerate_schedule(sr.BALANCED, N, P))} blocks" in r.stdout

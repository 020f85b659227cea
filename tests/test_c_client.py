"""The C ABI from C: tests/c_abi_client.c is compiled as C99 with
-Wall -Werror against include/dfa.h, linked against the built libdfa.so,
and run on the CPU (schedule building, balance accounting, workspace sizes,
status strings and error paths -- the host-only calls).  Its schedules must
equal the brute-force enumerator of oracle/schedule_ref.py field by field,
and its balance figures the enumerator's."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import schedule_ref as sr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_sequence_dfa_amd")


def library():
    lib = os.path.join(PKG, "libdfa.so")
    if not os.path.exists(lib):
        from long_context_sequence_dfa_amd import _build
        _build.build()
    return lib


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"),
                    reason="needs gcc and the HIP runtime library")
def test_c_client_against_the_enumerator(tmp_path):
    library()
    exe = str(tmp_path / "client")
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-O1",
                           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_client.c"),
                           "-L", PKG, "-ldfa", f"-Wl,-rpath,{PKG}", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout[-2000:] + out.stderr[-2000:]
    lines = out.stdout.splitlines()
    i, cases = 0, 0
    while i < len(lines) and lines[i].startswith("S "):
        f = lines[i].split()
        kind, n, p, stripe, nb, total, busy = (int(x) for x in f[1:8])
        bubble, eta = float(f[8]), float(f[9])
        blocks = np.array([[int(x) for x in ln.split()[1:]] for ln in lines[i + 1:i + 1 + nb]],
                          dtype=np.int64).reshape(-1, 11)
        want = sr.enumerate_schedule(sr.STRIPED_BLOCK if stripe > 1 else kind, n, p, stripe)
        assert np.array_equal(blocks, want), (kind, n, p, stripe)
        bal = sr.balance(want, p)
        assert total == int(want[:, 9].sum()) and busy == int(round(bal["eta_blocks"] * p * p))
        assert bubble == pytest.approx(bal["bubble"], abs=1e-15)
        assert eta == pytest.approx(bal["eta_blocks"], abs=1e-15)
        r = lines[i + 1 + nb].split()
        bar = r.index("|")
        assert [int(x) for x in r[1:bar]] == list(bal["rank_pairs"])
        assert [int(x) for x in r[bar + 1:]] == list(bal["step_max"])
        i += 2 + nb
        while i < len(lines) and lines[i].startswith("W "):
            op, st, size = (int(x) for x in lines[i].split()[1:])
            assert st == 0 and size > 0, lines[i]
            i += 1
        cases += 1
    assert cases == 14
    rest = {ln.split()[1]: ln.split()[2:] for ln in lines[i:] if ln.startswith("E ")}
    assert rest["shape"][0] == "-2"
    assert rest["capacity"][0] == "-5" and int(rest["capacity"][1]) == len(sr.enumerate_schedule(sr.RING, 1024, 4))
    assert rest["null"][0] == "-1"
    texts = [ln for ln in lines[i:] if ln.startswith("T ")]
    assert len(texts) == 8 and all(len(t.split(maxsplit=2)) == 3 for t in texts)

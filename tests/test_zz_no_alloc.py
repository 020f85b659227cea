"""dfa_attn_bwd_noalloc (the backward on the library's fixed per-GPU scratch)
against dfa_attn_bwd with a caller workspace: identical gradients on two
calls in a row, the second a smaller problem (the scratch keeps the first
call's contents), and a problem larger than the scratch refused up front."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dfa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sequence_dfa_amd as m
    from long_context_sequence_dfa_amd import binding
    binding.lib()
    return m


def run_case(dfa, seed, kind, N, P, Hq, Hkv, D, dtype):
    from long_context_sequence_dfa_amd import binding, inputs
    print(f"case: no-alloc backward kind={kind} N={N} P={P} Hq={Hq} Hkv={Hkv} D={D} {dtype}", flush=True)
    q, k, v, do = inputs.workload_tensors(seed, 1, N, Hq, Hkv, D, dtype, with_do=True)
    tq, tk, tv, tdo = (inputs.to_torch(x, dtype, torch.device("cuda:0")) for x in (q, k, v, do))
    blocks = dfa.dfa_schedule_build(kind, N, P)
    o, lse = dfa.dfa_attn_fwd(tq, tk, tv, blocks)
    ref = dfa.dfa_attn_bwd(tq, tk, tv, o, tdo, lse, blocks)
    got = tuple(torch.full_like(t, float("nan")) for t in ref)
    binding.dfa_attn_bwd_noalloc(tq, tk, tv, o, tdo, lse, blocks, *got)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        # the same kernels on the same inputs: bit-identical (no atomics)
        assert torch.equal(a, b), name


def test_noalloc_backward_matches_workspace_backward(dfa):
    from oracle import schedule_ref as sr
    run_case(dfa, 7001, sr.BALANCED, 4096, 4, 8, 2, 128, "bf16")
    run_case(dfa, 7002, sr.RING, 1024, 2, 2, 2, 64, "bf16")


def test_noalloc_backward_fp32_and_striped(dfa):
    from oracle import schedule_ref as sr
    run_case(dfa, 7003, sr.STRIPED, 2048, 8, 4, 4, 128, "f32")
    run_case(dfa, 7004, sr.STRIPED, 512, 4, 2, 1, 128, "bf16")


def test_noalloc_refuses_problems_beyond_the_scratch(dfa):
    from long_context_sequence_dfa_amd import binding
    # 64 heads x 2^18 rows need 128 MiB of row statistics: refused on the
    # host before any launch (the addresses are never touched)
    N, Hq = 1 << 18, 64
    d = binding.DfaAttnDesc()
    d.dtype, d.batch, d.heads_q, d.heads_kv, d.head_dim = binding.DFA_BF16, 1, Hq, 8, 128
    d.seqlen, d.softmax_scale = N, 128 ** -0.5
    for name, h in (("q_strides", Hq), ("k_strides", 8), ("v_strides", 8), ("o_strides", Hq)):
        getattr(d, name)[:] = [N * h * 128, h * 128, 128]
    blocks = np.ascontiguousarray(binding.dfa_schedule_build(1, N, 8))
    fake = ctypes.c_void_p(1 << 20)
    st = binding.lib().dfa_attn_bwd_noalloc(ctypes.byref(d), blocks.ctypes.data_as(ctypes.c_void_p),
                                            len(blocks), fake, fake, fake, fake, fake, fake, fake,
                                            fake, fake, None)
    assert st == binding.DFA_E_WORKSPACE

"""GPU parity of the rotary position embedding (dfa_rope) against the fp64
oracle, and of attention over rotated queries and keys (forward and the
gradients mapped back through the inverse rotation)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import schedule_ref as sr
from tests.parity_util import bhnd, check_grad, check_out, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dfa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sequence_dfa_amd as m
    from long_context_sequence_dfa_amd import binding
    binding.lib()
    return m


def say(msg):
    print(msg, flush=True)


def rounded(y, dtype):
    return oracle.round_bf16(y) if dtype == "bf16" else y.astype(np.float32).astype(np.float64)


def check_rot(got, want_exact, dtype, what):
    """got: the kernel's stored values; want_exact: fp64.  Each output is one
    rounding of (nearly) the exact value: at most one unit in the last place
    apart from the oracle's own rounding, and equal to it almost everywhere."""
    ulp_rel = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -23
    err = np.abs(got - want_exact)
    assert np.all(err <= ulp_rel * np.abs(want_exact) + 1e-30), (what, float((err / (np.abs(want_exact) + 1e-30)).max()))
    same = np.mean(got == rounded(want_exact, dtype))
    assert same >= 0.99, (what, "share equal to the oracle's rounding", same)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,N,H,d,off,base", [(2, 300, 3, 128, 0, 1e4), (1, 257, 2, 64, 12345, 1e4),
                                              (1, 64, 4, 128, 262000, 5e5), (1, 5, 1, 2, 7, 1e4)])
def test_rope_kernel_parity(dfa, dtype, B, N, H, d, off, base):
    from long_context_sequence_dfa_amd import inputs
    say(f"case: rope {dtype} B={B} N={N} H={H} d={d} offset={off} base={base}")
    x = inputs.normal_tensor(6000 + N, 0, (B, N, H, d), dtype)
    tx = inputs.to_torch(x, dtype, "cuda")
    y = dfa.dfa_rope(tx, pos_offset=off, base=base)
    yi = dfa.dfa_rope(tx, pos_offset=off, base=base, inverse=True)
    back = dfa.dfa_rope(y, pos_offset=off, base=base, inverse=True)
    torch.cuda.synchronize()
    check_rot(to_np(y).astype(np.float64), oracle.rope(x, base=base, pos_offset=off), dtype, "rope")
    check_rot(to_np(yi).astype(np.float64), oracle.rope(x, base=base, pos_offset=off, inverse=True),
              dtype, "inverse")
    # turning back what was stored returns the input up to the two roundings
    # (each within one unit in the last place of the pair's length)
    ulp = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -23
    pl = np.repeat(np.sqrt(x[..., 0::2] ** 2 + x[..., 1::2] ** 2), 2, axis=-1)
    assert np.all(np.abs(to_np(back) - x) <= 2.5 * ulp * pl + 1e-30)


def test_rope_in_place_and_strided(dfa):
    from long_context_sequence_dfa_amd import inputs
    say("case: rope in place and on a [B, H, N, d] storage view")
    B, N, H, d = 1, 200, 3, 128
    x = inputs.normal_tensor(6100, 0, (B, N, H, d), "bf16")
    store = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).to(torch.bfloat16).cuda()
    tx = store.permute(0, 2, 1, 3)  # logical [B, N, H, d], storage [B, H, N, d]
    out = torch.empty_like(tx)
    dfa.dfa_rope(tx, out)
    ref = dfa.dfa_rope(tx.contiguous())
    # rows that are not 16-byte aligned (2-element offset, odd row stride): the one-pair path
    pad = torch.zeros((B, N, H, d + 2), dtype=torch.bfloat16, device="cuda")
    odd = pad[..., 2:]
    odd.copy_(tx)
    dfa.dfa_rope(odd, odd)
    dfa.dfa_rope(tx, tx)  # in place
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(tx, ref) and torch.equal(odd, ref)


def test_attention_over_rotated_inputs(dfa):
    """RoPE before the ring (the striped-attention page's placement): rotate
    q and k at their absolute positions, run the folded schedule, and map the
    gradients of the rotated tensors back with the inverse rotation."""
    from long_context_sequence_dfa_amd import inputs
    say("case: attention over rotated q, k (balanced P=4, N=1024, GQA)")
    B, N, Hq, Hkv, D, P = 1, 1024, 4, 2, 128, 4
    scale = 1 / np.sqrt(D)
    q, k, v, do = inputs.workload_tensors(6200, B, N, Hq, Hkv, D, "bf16", with_do=True)
    tq, tk, tv, tdo = (inputs.to_torch(x, "bf16", "cuda") for x in (q, k, v, do))
    blocks = dfa.dfa_schedule_build(sr.BALANCED, N, P)
    qr, kr = dfa.dfa_rope(tq), dfa.dfa_rope(tk)
    o, lse = dfa.dfa_attn_fwd(qr, kr, tv, blocks)
    dqr, dkr, dv = dfa.dfa_attn_bwd(qr, kr, tv, o, tdo, lse, blocks)
    dq, dk = dfa.dfa_rope(dqr, inverse=True), dfa.dfa_rope(dkr, inverse=True)
    torch.cuda.synchronize()
    # the oracle rotates and stores (bf16) on its own side
    oq, ok = oracle.round_bf16(oracle.rope(q)), oracle.round_bf16(oracle.rope(k))
    ro, rl = oracle.attn_rows(oq, ok, v, scale)
    ra, _ = oracle.attn_rows(oq, ok, np.abs(v), scale)
    check_out(bhnd(to_np(o)), ro, to_np(lse), rl, "bf16", "O", oabs=ra, n_keys=N)
    (gq, gk, gv), (aq, ak, av) = oracle.attn_grads(oq, ok, v, do, scale, with_abs=True)
    # back through the transpose rotation; a rotated element mixes the pair,
    # so its error magnitude is the pair's sum
    bq = oracle.rope(bhnd(gq), inverse=True)
    bk = oracle.rope(bhnd(gk), inverse=True)
    pair = lambda a: np.repeat(a[..., 0::2] + a[..., 1::2], 2, axis=-1)
    check_grad(bhnd(to_np(dq)), bhnd(bq), pair(aq), "bf16", "dq")
    check_grad(bhnd(to_np(dk)), bhnd(bk), pair(ak), "bf16", "dk")
    check_grad(bhnd(to_np(dv)), gv, av, "bf16", "dv")

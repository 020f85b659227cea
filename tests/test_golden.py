"""Fixtures under tests/golden/: values the pages print for their worked
examples (each file names its page and section), the published splitmix64
outputs, and the input generator's first values written by
tests/golden/make_inputs_golden.py.  Each is checked against the schedule
enumerator of the oracle and against the library's host-side schedule
builder and balance accounting."""
import os

import numpy as np
import pytest

from oracle import schedule_ref as sr
from long_context_sequence_dfa_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def ints(s):
    return [int(x) for x in s.split(",")]


@pytest.fixture(scope="module")
def dfa():
    import long_context_sequence_dfa_amd as m
    from long_context_sequence_dfa_amd import binding
    binding.lib()
    return m


def schedules(dfa, kind, n, p):
    """The oracle's enumeration and the library's build of one schedule."""
    ref = sr.enumerate_schedule(kind, n, p)
    lib = np.asarray(dfa.dfa_schedule_build(kind, n, p))[:, :ref.shape[1]]
    return ref, lib


def test_ring_p4_grid(dfa):
    r = rows("ring_p4_grid.txt")
    grid, walk, count = r[:4], r[4:6], r[6]
    p, c = 4, 8
    for blocks in schedules(dfa, sr.RING, p * c, p):
        for qc, kvs, pct in grid:
            mine = blocks[blocks[:, 0] == int(qc)]
            assert sorted(mine[:, 2].tolist()) == ints(kvs)
            # the printed share counts whole blocks of the row
            assert 100 * len(mine) // p == int(pct)
        for step, rank, kv_rank, what in walk:
            sel = blocks[(blocks[:, 1] == int(step)) & (blocks[:, 0] == int(rank))]
            assert (int(rank) - int(step)) % p == int(kv_rank)
            if what == "full":
                assert len(sel) == 1 and sel[0, 2] == int(kv_rank) and sel[0, 9] == c * c
            else:
                assert len(sel) == 0
        assert [int(count[0]), len(blocks), p * p] == [p, int(count[1]), int(count[2])]


def test_folded_chunks_p4(dfa):
    p, c = 4, 8
    for blocks in schedules(dfa, sr.BALANCED, 2 * p * c, p):
        for rank, lo, hi, total in rows("folded_chunks_p4.txt"):
            q_chunks = sorted({int(s) // c for s in blocks[blocks[:, 0] == int(rank)][:, 3]})
            assert q_chunks == [int(lo), int(hi)]
            assert int(lo) + int(hi) == int(total) == 2 * p - 1
        bal = sr.balance(blocks, p)
        assert len(set(bal["rank_pairs"].tolist())) == 1  # the same load on every rank


def test_striping_16_tokens(dfa):
    kinds = {"contiguous": sr.RING, "striped": sr.STRIPED}
    for kind, rank, toks in rows("striping_16x4.txt"):
        pieces = sr.rank_pieces(kinds[kind], 16, 4)[int(rank)]
        assert np.concatenate([sr.positions(pc) for pc in pieces]).tolist() == ints(toks)
        # the library's rows of that rank: q_start + i * stride
        blocks = np.asarray(dfa.dfa_schedule_build(kinds[kind], 16, 4))
        b = blocks[blocks[:, 0] == int(rank)][0]
        assert (b[3] + np.arange(b[5]) * b[7]).tolist() == ints(toks)


def test_ring_bubble_table(dfa):
    # Reading: the page's measured bubbles come within 1.5 percentage points
    # of the lock-step bubble of the exact pair counts, and the block-count
    # utilisation is exactly the printed (P+1)/(2P).
    for tokens, p, pct in rows("ring_bubble_table.txt"):
        n, p = int(tokens), int(p)
        ref, lib = schedules(dfa, sr.RING, n, p)
        bal_ref = sr.balance(ref, p)
        bal_lib = dfa.dfa_schedule_balance(lib, p)
        assert bal_lib["bubble"] == pytest.approx(bal_ref["bubble"], abs=1e-12)
        assert abs(100 * bal_ref["bubble"] - float(pct)) < 1.5
        assert bal_ref["eta_blocks"] == pytest.approx((p + 1) / (2 * p), abs=1e-15)
        assert bal_lib["eta_blocks"] == pytest.approx((p + 1) / (2 * p), abs=1e-15)
        # every rank of the striped schedule carries the same load within one
        # triangle's diagonal, so its bubble is below the page's "<1 %"
        st = sr.balance(sr.enumerate_schedule(sr.STRIPED, n, p), p)
        assert st["bubble"] < 0.01


def test_splitmix64_published_outputs():
    want = [int(r[0], 16) for r in rows("splitmix64_seed0.txt")]
    with np.errstate(over="ignore"):
        got = inputs._mix(np.arange(1, len(want) + 1, dtype=np.uint64) * inputs.GAMMA)
    assert [int(x) for x in got] == want


def test_generator_first_values():
    names = {"q": 0, "k": 1, "v": 2, "do": 3}
    cases = rows("inputs_first8.txt")
    assert len(cases) == 20
    for wl, seed, dtype, name, *vals in cases:
        scale = 1.0 / np.sqrt(128) if wl.startswith("llama7b-n32k") and name != "do" else None
        got = inputs.normal_tensor(int(seed), names[name], (8,), dtype, scale)
        assert got.tolist() == [float(v) for v in vals], (wl, name)

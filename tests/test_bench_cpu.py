"""The benchmark's host side on the CPU: it refuses more than one GPU before
touching a device, and the work it counts (visible pairs behind the
causal-effective FLOPs) matches the closed forms of each workload's schedule."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.fixture(scope="module")
def dfa():
    import long_context_sequence_dfa_amd as m
    from long_context_sequence_dfa_amd import binding
    binding.lib()
    return m


def closed_form_pairs(wl):
    """Visible (query, key) pairs per query head of the benchmark's block list."""
    n = wl["N"]
    if wl["rank"] is None:
        return n * (n + 1) // 2  # every causal pair, whichever schedule covers them
    # token striping, one rank r's share: its rows m*P + r see keys 0 .. m*P + r
    p, r = wl["P"], wl["rank"]
    c = n // p
    return sum(m * p + r + 1 for m in range(c))


@pytest.mark.parametrize("name", [w for w in bench.WORKLOADS if "docs" not in bench.WORKLOADS[w]])
def test_counted_pairs(dfa, name):
    wl = bench.WORKLOADS[name]
    blocks = np.asarray(bench.schedule(dfa, wl))
    if wl["rank"] is not None:
        blocks = blocks[blocks[:, 0] == wl["rank"]]
    assert int(blocks[:, 9].sum()) == closed_form_pairs(wl)


def test_headline_figures(dfa):
    # the Llama-7B shape at N = 32768: N(N+1)/2 pairs per head, 14 d FLOP each
    wl = bench.WORKLOADS["llama7b-n32k-balanced-p8"]
    pairs = int(np.asarray(bench.schedule(dfa, wl))[:, 9].sum())
    assert pairs == 536_887_296
    assert 14 * 128 * pairs * 32 == pytest.approx(3.0790e13, rel=1e-4)
    # one rank's share at N = 131072 over 16 ranks: 8 C^2 - 7 C with C = 8192
    wl = bench.WORKLOADS["llama7b-n131k-striped-p16-rank0"]
    b = np.asarray(bench.schedule(dfa, wl))
    assert int(b[b[:, 0] == 0][:, 9].sum()) == 8 * 8192 ** 2 - 7 * 8192 == 536_813_568

"""The algorithmic work bench.py divides by (the roofline numerators) against
counts taken from the oracle's own definitions, by brute force per query.

The attention flops count 4 d h_q per (query, head, visible key), where a
query's keys are those u <= t in its selected blocks; any top-k choice
gives the same count, since every top-k candidate is a whole block below the
local window.  Pass 1 counts 2 d h_q per visible stage-1 (or coarse) window
of each scored row (a row with more candidates than n_topk), pass 2 per
window its max pool reads for the row's candidate blocks.
"""
import numpy as np
import pytest

import bench
import oracle.reference as R


def _brute(n, n_init, n_local, n_topk, h_q=32, d=128):
    p = R.Params(n_init=n_init, n_local=n_local, n_topk=n_topk)
    B = p.block_size
    n1, n2 = R.n_windows(n, 32, 16), R.n_windows(n, 128, 64)
    keys = lse1 = lse2 = wins = 0
    for t in range(n):
        bt = t // B
        lo, hi = R.candidate_range(t, p)
        cand = list(range(lo, hi + 1))
        scored = len(cand) > n_topk
        init = [b for b in range(n_init) if b <= bt]
        local = [b for b in range(bt - n_local + 1, bt + 1) if b >= 0]
        chosen = cand[:n_topk] if scored else cand
        blocks = set(init) | set(local) | set(chosen)
        keys += sum(min(B, t + 1 - B * b) for b in blocks if B * b <= t)
        if scored:
            lse1 += R.n_visible(t, 32, 16, n1)
            lse2 += R.n_visible(t, 128, 64, n2)
            # windows 4b - 1 .. 4b + 3 of every candidate block (the pool's reach)
            wins += len({j for b in cand for j in range(4 * b - 1, 4 * b + 4) if j >= 0})
    f = lambda x: float(x) * h_q * d
    return {"attn_flops": 4 * f(keys), "lse_exact_flops": 2 * f(lse1), "lse_approx_flops": 2 * f(lse2),
            "blocks_flops": 2 * f(wins)}


@pytest.mark.parametrize("n,sel", [(9000, (1, 32, 63)), (5000, (1, 4, 11)), (3000, (2, 3, 7))])
def test_algorithmic_work_matches_brute_force(n, sel):
    got = bench.algorithmic_work(n, 32, 2, 128, *sel)
    want = _brute(n, *sel)
    for key, v in want.items():
        assert got[key] == pytest.approx(v, rel=0, abs=0.5), (key, got[key], v)


def test_visible_keys_of_the_headline_layer():
    """At n = 131072 with |I| = 96: a query in one of the first 96 blocks
    keeps every causal key (t + 1), later ones 95 whole blocks plus their own
    block's prefix (6080 + t % 64 + 1): a closed form of the count the
    attention roofline is built on (5,970 keys per query on average)."""
    n, full = 131072, 96 * 64
    closed = full * (full + 1) // 2 + (n - full) // 64 * sum(6080 + r + 1 for r in range(64))
    w = bench.algorithmic_work(n, 32, 2)
    assert w["attn_flops"] == 4 * 128 * 32 * closed
    assert closed / n == 5970.0

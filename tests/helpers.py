"""Shared test helpers: acceptance rules and small utilities (no method arithmetic)."""
from __future__ import annotations

import numpy as np

REL_TIE = 1e-3       # selection tie band (relative), from the acceptance criteria
ATT_MAX_ABS = 2e-2   # attention max-abs tolerance for bf16 I/O with fp32 accumulation
ATT_REL_RMS = 1e-2   # additional relative-RMS bound (outputs have small norms at 128K)


def check_selection(gpu_blocks, oracle_blocks, info, t, p, rel=REL_TIE):
    """Compare one (row, group) selection with the oracle.

    Returns (ok, exempt, n_band) where ``exempt`` says the oracle's k-th and
    (k+1)-th candidate scores differ by less than ``rel`` relative (the row
    may then differ inside the band), and ``n_band`` counts candidates within
    the band around the k-th score.  Outside the band every decision must
    match; init and local blocks and the count must always match."""
    g = [b for b in gpu_blocks if b >= 0]
    if g != sorted(set(g)):
        return False, False, 0
    bt = t // p.block_size
    lo, hi = p.n_init, bt - p.n_local
    fixed = set(range(min(p.n_init, bt + 1))) | set(range(max(0, bt - p.n_local + 1), bt + 1))
    if not fixed.issubset(g):
        return False, False, 0
    cands = info["cands"]
    if len(cands) <= p.n_topk:
        return sorted(g) == sorted(oracle_blocks), False, 0
    k = p.n_topk
    if k == 0:                       # no top-k: exactly the init and local blocks
        return set(g) == fixed and sorted(g) == sorted(oracle_blocks), False, 0
    scores = info["scores"]          # oracle candidate scores in oracle order (desc, idx asc)
    order = info["order"]
    sk, sk1 = scores[k - 1], scores[k]
    exempt = (sk - sk1) < rel * sk
    gsel = set(g) - fixed
    if len(gsel) != k or not gsel.issubset(set(cands)):
        return False, exempt, 0
    score_of = dict(zip(order, scores))
    upper, lower = sk * (1 + rel), sk * (1 - rel)
    n_band = 0
    for b in cands:
        sc = score_of[b]
        if sc > upper and b not in gsel:
            return False, exempt, n_band
        if sc < lower and b in gsel:
            return False, exempt, n_band
        if lower <= sc <= upper:
            n_band += 1
    if not exempt and sorted(g) != sorted(oracle_blocks):
        return False, exempt, n_band
    return True, exempt, n_band


def attn_errors(gpu, ref):
    """max-abs error and relative RMS of gpu (float) against ref (float64)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = gpu - ref
    max_abs = float(np.abs(err).max()) if err.size else 0.0
    rms = float(np.sqrt((err ** 2).mean())) if err.size else 0.0
    ref_rms = float(np.sqrt((ref ** 2).mean())) if ref.size else 1.0
    return max_abs, rms / max(ref_rms, 1e-30)


def sample_positions(n, count, seed=0, must=()):
    """Spread sample of positions in [0, n): ends, block edges and random ones."""
    rng = np.random.Generator(np.random.PCG64(seed))
    base = {0, n - 1, n // 2, min(n - 1, 64), min(n - 1, 63)}
    base |= {x for x in must if 0 <= x < n}
    extra = rng.choice(n, size=min(n, max(0, count - len(base))), replace=False)
    return sorted(base | set(int(x) for x in extra))

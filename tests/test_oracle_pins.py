"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function checks one part of the oracle against the pages'
printed numbers, a closed form, a library routine (numpy convolution,
scipy logsumexp / softmax, torch scaled_dot_product_attention in float64) or
brute force on tiny inputs, and returns True when it holds.  The tests assert
every pin holds, and ``test_planted_mistakes_are_caught`` plants plausible
mistakes in the oracle (on the CPU) and asserts that some pin fails for each.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle.reference as R

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _tiny(seed=0, n=333, h_q=4, h_kv=2, d=8):
    g = _rng(seed)
    return (g.standard_normal((n, h_q, d)), g.standard_normal((n, h_kv, d)),
            g.standard_normal((n, h_kv, d)))


def _close(a, b, tol=1e-10):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        return False
    fin = np.isfinite(b)
    if not np.array_equal(np.isfinite(a), fin):
        return False
    return bool(np.all(np.abs(a[fin] - b[fin]) <= tol * (1 + np.abs(b[fin]))))


# ---------------------------------------------------------------- pins ----

def pin_worked_example():
    """Token 20000 lies in block 313 (1-based); with 1 init + 32 local + 63
    top-k blocks it sees 96 blocks (the 6144-token budget); the tail block is
    partial, so 95*64 + 32 = 6112 keys."""
    f = FACTS["worked_example"]
    p = R.Params(block_size=f["block_size"], n_init=f["init_blocks"], n_local=f["local_blocks"],
                 n_topk=f["visible_blocks"] - f["init_blocks"] - f["local_blocks"])
    t = f["token_1based"] - 1
    if t // p.block_size + 1 != f["block_1based"]:
        return False
    if p.n_sel * p.block_size != f["visible_tokens_budget"]:
        return False
    scores = _rng(1).random(t // p.block_size + 1)
    blocks, _ = R.select_from_scores(t, scores, p)
    bt = f["block_1based"] - 1
    ok = len(blocks) == f["visible_blocks"] and 0 in blocks
    ok &= all(b in blocks for b in range(bt - f["local_blocks"] + 1, bt + 1))
    nkeys = sum(min(p.block_size, t + 1 - b * p.block_size) for b in blocks)
    return bool(ok and nkeys == 95 * 64 + (t % 64) + 1 == 6112)


def pin_stage_parameters():
    """l_C1 = B/2, s_C1 = B/4, pool (5, 4); l_C2 = 4 l_C1, s_C2 = 4 s_C1."""
    p = R.Params()
    f3, f4 = FACTS["three_stage_compression"], FACTS["lse_approximation"]
    return (p.c1_kernel == f3["c1_kernel_over_block"] * p.block_size
            and p.c1_stride == f3["c1_stride_over_block"] * p.block_size
            and (p.pool_kernel, p.pool_stride) == (f3["pool_kernel"], f3["pool_stride"])
            and p.c2_kernel == f4["c2_kernel_over_c1_kernel"] * p.c1_kernel
            and p.c2_stride == f4["c2_stride_over_c1_stride"] * p.c1_stride)


def pin_window_counts():
    """Window counts by brute-force enumeration of window starts."""
    for n in (0, 31, 32, 47, 48, 4096, 32768, 131072):
        for (l, s) in ((32, 16), (128, 64)):
            brute = sum(1 for st in range(0, n, s) if st + l <= n)
            if R.n_windows(n, l, s) != brute:
                return False
    return (R.n_windows(4096, 32, 16), R.n_windows(32768, 32, 16), R.n_windows(131072, 32, 16),
            R.n_windows(131072, 128, 64)) == (255, 2047, 8191, 2047)


def pin_compress_by_convolution():
    """Compressed keys equal a full sliding mean (numpy.convolve) sampled at the stride."""
    _, K, _ = _tiny(2)
    for (l, s) in ((32, 16), (128, 64), (5, 3)):
        KC = R.compress_keys(K, l, s)
        for g in range(K.shape[1]):
            for dd in range(K.shape[2]):
                c = np.convolve(K[:, g, dd], np.ones(l) / l, mode="valid")[::s]
                if not _close(KC[g, :, dd], c, 1e-12):
                    return False
    return True


def pin_compress_constant():
    K = np.full((200, 2, 8), 0.375)
    return bool(np.all(R.compress_keys(K, 32, 16) == 0.375))


def pin_compress_bf16_rounding():
    """round_to_bf16 against exact enumeration of the neighbouring bf16 values."""
    vals = _rng(3).standard_normal(2000) * np.exp2(_rng(4).integers(-20, 20, 2000))
    vals = np.concatenate([vals, [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)]])
    r = R.round_to_bf16(vals)
    for x, y in zip(vals, r):
        e = math.floor(math.log2(abs(x)))
        ulp = 2.0 ** (e - 7)
        lo = math.floor(x / ulp) * ulp
        hi = lo + ulp
        if x - lo < hi - x:
            want = lo
        elif x - lo > hi - x:
            want = hi
        else:  # tie: even significand
            want = lo if int(round(lo / ulp)) % 2 == 0 else hi
        if y != want:
            return False
    return True


def _brute_logits(q, KC, G, scale, h, nv):
    return np.array([scale * sum(q[h, i] * KC[h // G, j, i] for i in range(q.shape[1]))
                     for j in range(nv)])


def pin_lse_exact_scipy():
    """Exact LSE equals scipy's logsumexp over brute-force logits of the
    windows whose last token is <= t."""
    Q, K, _ = _tiny(5)
    p = R.Params()
    KC1 = R.compress_keys(K, 32, 16)
    G = Q.shape[1] // K.shape[1]
    scale = 1 / math.sqrt(Q.shape[2])
    for t in (0, 30, 31, 46, 47, 48, 63, 150, 332):
        nv = sum(1 for j in range(KC1.shape[1]) if 16 * j + 31 <= t)
        L = R.lse_exact(Q[t], t, KC1, G, p)
        for h in range(Q.shape[1]):
            want = logsumexp(_brute_logits(Q[t], KC1, G, scale, h, nv)) if nv else -np.inf
            if not _close([L[h]], [want], 1e-11):
                return False
    return True


def pin_lse_approx_scipy():
    Q, K, _ = _tiny(6, n=400)
    p = R.Params(lse_mode="approx")
    KC2 = R.compress_keys(K, 128, 64)
    G = Q.shape[1] // K.shape[1]
    scale = 1 / math.sqrt(Q.shape[2])
    for t in (127, 128, 190, 191, 255, 399):
        nv = sum(1 for j in range(KC2.shape[1]) if 64 * j + 127 <= t)
        L = R.lse_approx(Q[t], t, KC2, G, p)
        for h in range(Q.shape[1]):
            want = logsumexp(_brute_logits(Q[t], KC2, G, scale, h, nv)) if nv else -np.inf
            if not _close([L[h]], [want], 1e-11):
                return False
    return True


def pin_group_sum_softmax():
    """G = 1: S_shared is scipy's softmax of the visible logits; in general
    the visible entries of each group sum to G and the rest are 0; permuting
    heads inside a group leaves S_shared unchanged."""
    p = R.Params()
    Q, K, _ = _tiny(7, h_q=2, h_kv=2)
    KC1 = R.compress_keys(K, 32, 16)
    scale = 1 / math.sqrt(Q.shape[2])
    for t in (47, 100, 332):
        nv = sum(1 for j in range(KC1.shape[1]) if 16 * j + 31 <= t)
        L = R.lse_exact(Q[t], t, KC1, 1, p)
        S = R.shared_scores(Q[t], t, KC1, L, 1, p)
        for h in range(2):
            want = np.zeros(KC1.shape[1])
            want[:nv] = softmax(_brute_logits(Q[t], KC1, 1, scale, h, nv))
            if not _close(S[h], want, 1e-11):
                return False
    Q, K, _ = _tiny(8, h_q=8, h_kv=2)
    KC1 = R.compress_keys(K, 32, 16)
    for t in (63, 200, 332):
        L = R.lse_exact(Q[t], t, KC1, 4, p)
        S = R.shared_scores(Q[t], t, KC1, L, 4, p)
        if not _close(S.sum(axis=1), [4.0, 4.0], 1e-12):
            return False
        perm = np.array([2, 0, 3, 1, 5, 7, 6, 4])
        Sp = R.shared_scores(Q[t][perm], t, KC1, L[perm], 4, p)
        if not _close(S, Sp, 1e-12):
            return False
    return True


def pin_constant_keys():
    """All keys equal: every visible window gets probability 1/|visible|, so
    S_shared = G/|visible|; approx LSE differs from exact by ln(|V1|/|V2|)."""
    p = R.Params()
    g = _rng(9)
    Q = g.standard_normal((400, 4, 8))
    K = np.tile(g.standard_normal((1, 2, 8)), (400, 1, 1))
    KC1 = R.compress_keys(K, 32, 16)
    KC2 = R.compress_keys(K, 128, 64)
    for t in (40, 131, 399):
        nv1 = R.n_visible(t, 32, 16, KC1.shape[1])
        L = R.lse_exact(Q[t], t, KC1, 2, p)
        S = R.shared_scores(Q[t], t, KC1, L, 2, p)
        if not _close(S[:, :nv1], np.full((2, nv1), 2.0 / nv1), 1e-12):
            return False
        if t >= 127:
            nv2 = R.n_visible(t, 128, 64, KC2.shape[1])
            La = R.lse_approx(Q[t], t, KC2, 2, p)
            if not _close(L - La, np.full(4, math.log(nv1 / nv2)), 1e-12):
                return False
    return True


def pin_approx_bound():
    """Mean-pooled coarse keys give L_approx <= L_exact - ln 2 for every
    query and head (convexity of exp; each coarse window is tiled by four
    fine windows and each fine window is reused by at most two coarse ones)."""
    p = R.Params()
    for seed in (10, 11):
        Q, K, _ = _tiny(seed, n=700, d=16)
        KC1 = R.compress_keys(K, 32, 16)
        KC2 = R.compress_keys(K, 128, 64)
        for t in range(127, 700, 37):
            L = R.lse_exact(Q[t], t, KC1, 2, p)
            La = R.lse_approx(Q[t], t, KC2, 2, p)
            if not np.all(La <= L - math.log(2) + 1e-12):
                return False
    return True


def pin_pool_by_token_overlap():
    """Block score = max of S_shared over the stage-1 windows whose tokens
    overlap the block's tokens (enumerated directly)."""
    p = R.Params()
    S = _rng(12).random((2, 60))
    nb = 17
    bs = R.block_scores(S, nb, p)
    for b in range(nb):
        js = [j for j in range(S.shape[1])
              if 16 * j < 64 * (b + 1) and 16 * j + 32 > 64 * b]
        want = S[:, js].max(axis=1) if js else np.zeros(2)
        if not _close(bs[:, b], want, 0):
            return False
        if b > 0 and 4 * b + 3 < S.shape[1] and len(js) != 5:
            return False
    return True


def pin_topk_full_sort():
    """Top-k against a full lexicographic sort (score desc, index asc), with
    planted exact ties; union with init and local; k >= |C| keeps all."""
    p = R.Params(n_init=1, n_local=4, n_topk=11)
    g = _rng(13)
    for t in range(0, 4096, 61):
        nb = t // 64 + 1
        sc = np.round(g.random(nb), 2)  # many exact ties
        blocks, _ = R.select_from_scores(t, sc, p)
        bt = nb - 1
        cands = np.arange(1, bt - 4 + 1)
        if len(cands) > 11:
            order = np.lexsort((cands, -sc[cands]))
            top = set(cands[order[:11]].tolist())
        else:
            top = set(cands.tolist())
        want = sorted(set(range(min(1, nb))) | set(range(max(0, bt - 3), bt + 1)) | top)
        if blocks != want or len(blocks) != min(nb, 16):
            return False
    return True


def _sdpa(q, k, v, mask):
    """torch SDPA in float64 with an explicit boolean mask [h_q, n, n]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    G = q.shape[1] // k.shape[1]
    kt = kt.repeat_interleave(G, dim=1)
    vt = vt.repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask)[None])
    return o[0].permute(1, 0, 2).numpy()


def pin_attention_sdpa():
    """Dense attention and sparse attention over all causal blocks equal torch
    SDPA (causal); sparse attention over arbitrary block lists equals SDPA
    with the corresponding block mask."""
    p = R.Params(block_size=16)
    Q, K, V = _tiny(14, n=90, h_q=4, h_kv=2, d=8)
    n = Q.shape[0]
    causal = np.tril(np.ones((n, n), dtype=bool))
    ref = _sdpa(Q, K, V, np.broadcast_to(causal, (4, n, n)).copy())
    g = _rng(15)
    mask = np.zeros((4, n, n), dtype=bool)
    sels = []
    for t in range(n):
        bt = t // 16
        o_d, _ = R.dense_token(Q[t], t, K, V, 2, 1 / math.sqrt(8))
        o_s, _ = R.attend_token(Q[t], t, K, V, [list(range(bt + 1))] * 2, 2, p)
        if not (_close(o_d, ref[t], 1e-10) and _close(o_s, ref[t], 1e-10)):
            return False
        sel = []
        for gg in range(2):
            bl = sorted(set([bt]) | set(g.choice(bt + 1, size=min(bt + 1, 2), replace=False).tolist()))
            sel.append(bl)
            for h in range(2 * gg, 2 * gg + 2):
                for b in bl:
                    mask[h, t, b * 16:min((b + 1) * 16, t + 1)] = True
        sels.append(sel)
    sel_ref = _sdpa(Q, K, V, mask)
    for t in range(n):
        o_b, _ = R.attend_token(Q[t], t, K, V, sels[t], 2, p)
        if not _close(o_b, sel_ref[t], 1e-10):
            return False
    return True


def pin_attention_special_cases():
    """V constant -> output constant; a single visible key -> output = v_0."""
    Q, K, V = _tiny(16, n=130)
    V[:] = 0.625
    p = R.Params()
    o, _ = R.attend_token(Q[100], 100, K, V, [[0, 1], [1]], 2, p)
    if not np.allclose(o, 0.625, atol=1e-14):
        return False
    Q, K, V = _tiny(17, n=10)
    o, lse = R.dense_token(Q[0], 0, K, V, 2, 0.3)
    want = np.stack([V[0, h // 2] for h in range(4)])
    return bool(np.allclose(o, want, atol=1e-14))


def pin_cost_identities():
    """Logit evaluations over a 128K prefill: approx pass 1 sees a quarter of
    the windows, so two passes (2x) become about 1.25x of one pass; the fused
    group-sum write is h_q n^2 / (s_C1 G) against h_q n^2 / s_C1 unfused."""
    n, h_q, G = 131072, 32, 16
    N1, N2 = R.n_windows(n, 32, 16), R.n_windows(n, 128, 64)
    ts = np.arange(n)
    v1 = np.minimum(N1, np.maximum(0, (ts - 31) // 16 + 1))
    v2 = np.minimum(N2, np.maximum(0, (ts - 127) // 64 + 1))
    one_pass = v1.sum()
    exact, approx = 2 * one_pass, one_pass + v2.sum()
    if abs(exact / one_pass - 2.0) > 1e-12 or abs(approx / one_pass - 1.25) > 5e-3:
        return False
    unfused, fused = h_q * n * N1, (h_q // G) * n * N1
    return abs(unfused / (h_q * n * n / 16) - 1) < 1e-3 and unfused / fused == G


def _grad_case(seed=31, n=150, h_q=4, h_kv=2, d=8, B=16, with_sets=True):
    """Tiny sequence with random per-token block sets (own block always in)."""
    Q, K, V = _tiny(seed, n=n, h_q=h_q, h_kv=h_kv, d=d)
    dO = _rng(seed + 1).standard_normal((n, h_q, d))
    p = R.Params(block_size=B)
    g = _rng(seed + 2)
    idx = {}
    for t in range(n):
        bt = t // B
        idx[t] = [sorted({bt} | {b for b in range(bt) if g.random() < 0.5}) for _ in range(h_kv)]
    return Q, K, V, dO, p, idx


def _loss(Q, K, V, dO, G, p, idx):
    """sum(dO * O) through the forward oracle (attend_token)."""
    tot = 0.0
    for t, blocks in idx.items():
        o, _ = R.attend_token(Q[t], t, K, V, blocks, G, p)
        tot += float((dO[t] * o).sum())
    return tot


def pin_grad_finite_differences():
    """Analytic gradients of the sparse attention against central differences
    of the forward oracle, at 12 random coordinates of each of Q, K, V."""
    Q, K, V, dO, p, idx = _grad_case()
    G = Q.shape[1] // K.shape[1]
    dQ, dK, dV = R.attention_grad(Q, K, V, dO, G, p, idx)
    g = _rng(40)
    eps = 1e-5
    for X, dX in ((Q, dQ), (K, dK), (V, dV)):
        for _ in range(12):
            at = tuple(int(g.integers(0, m)) for m in X.shape)
            old = X[at]
            X[at] = old + eps
            lp = _loss(Q, K, V, dO, G, p, idx)
            X[at] = old - eps
            lm = _loss(Q, K, V, dO, G, p, idx)
            X[at] = old
            fd = (lp - lm) / (2 * eps)
            if abs(fd - dX[at]) > 1e-7 * (1 + abs(fd)):
                return False
    return True


def pin_grad_identities():
    """Exact identities: the key gradients of a group sum to zero (each row of
    dl/dz sums to zero); the value gradients sum to the group's upstream
    gradient (each row of P sums to one); values equal along the keys leave
    dQ and dK at zero; a query that sees one key gets dq = 0."""
    Q, K, V, dO, p, idx = _grad_case(seed=33)
    h_kv = K.shape[1]
    G = Q.shape[1] // h_kv
    dQ, dK, dV = R.attention_grad(Q, K, V, dO, G, p, idx)
    for g in range(h_kv):
        if not np.allclose(dK[:, g].sum(axis=0), 0.0, atol=1e-11):
            return False
        want = dO[:, g * G:(g + 1) * G].sum(axis=(0, 1))
        if not np.allclose(dV[:, g].sum(axis=0), want, atol=1e-11):
            return False
    Vc = np.broadcast_to(_rng(34).standard_normal((1, h_kv, K.shape[2])), K.shape).copy()
    dQc, dKc, _ = R.attention_grad(Q, K, Vc, dO, G, p, idx)
    if not (np.allclose(dQc, 0.0, atol=1e-12) and np.allclose(dKc, 0.0, atol=1e-12)):
        return False
    dq, parts = R.attend_token_grad(Q[0], dO[0], 0, K, V, [[0]] * h_kv, G, p)
    return bool(np.allclose(dq, 0.0, atol=1e-14) and all(len(u) == 1 for u, _, _ in parts))


def pin_grad_dense_torch():
    """Dense causal gradients against torch autograd of
    scaled_dot_product_attention in float64 (K, V repeated per group)."""
    Q, K, V = _tiny(35, n=96, h_q=4, h_kv=2, d=8)
    dO = _rng(36).standard_normal(Q.shape)
    G = 2
    p = R.Params(block_size=16)
    dQ, dK, dV = R.attention_grad(Q, K, V, dO, G, p, dense=True)
    q = torch.tensor(Q).permute(1, 0, 2).requires_grad_(True)
    k = torch.tensor(K).permute(1, 0, 2).requires_grad_(True)
    v = torch.tensor(V).permute(1, 0, 2).requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(G, 0), v.repeat_interleave(G, 0), is_causal=True)
    o.backward(torch.tensor(dO).permute(1, 0, 2))
    return (_close(dQ, q.grad.permute(1, 0, 2).numpy(), 1e-11)
            and _close(dK, k.grad.permute(1, 0, 2).numpy(), 1e-11)
            and _close(dV, v.grad.permute(1, 0, 2).numpy(), 1e-11))



def _brute_select(Q, K, t, G, p: R.Params, scale):
    """Selection of query t written out without the oracle's helpers:
    compressed keys from a running sum, logits by einsum, the exact LSE as
    scipy's softmax normaliser (or scipy's logsumexp over the coarse keys),
    the group sum, the pool over windows enumerated by token overlap, and the
    top-k by numpy's lexsort.  Returns (blocks per group, block scores or
    None when no row score is needed)."""
    n, h_kv, d = K.shape
    csum = np.concatenate([np.zeros((1, h_kv, d)), np.cumsum(K, axis=0)])

    def windows(l, s):
        starts = [j for j in range(0, n) if j * s + l <= n]
        return np.stack([(csum[j * s + l] - csum[j * s]) / l for j in starts], axis=1) if starts \
            else np.zeros((h_kv, 0, d))

    B = p.block_size
    bt = t // B
    init = set(range(min(p.n_init, bt + 1)))
    local = set(range(max(0, bt - p.n_local + 1), bt + 1))
    cands = [b for b in range(bt + 1) if p.n_init <= b <= bt - p.n_local]
    if len(cands) <= p.n_topk:
        return [sorted(init | local | set(cands))] * h_kv, None
    KC1 = windows(p.c1_kernel, p.c1_stride)
    vis1 = [j for j in range(KC1.shape[1]) if p.c1_stride * j + p.c1_kernel - 1 <= t]
    z = scale * np.einsum("hd,hjd->hj", Q[t], KC1[np.arange(Q.shape[1]) // G][:, vis1])
    if p.lse_mode == "exact":
        P = softmax(z, axis=1)
    else:
        KC2 = windows(p.c2_kernel, p.c2_stride)
        vis2 = [j for j in range(KC2.shape[1]) if p.c2_stride * j + p.c2_kernel - 1 <= t]
        z2 = scale * np.einsum("hd,hjd->hj", Q[t], KC2[np.arange(Q.shape[1]) // G][:, vis2])
        P = np.exp(z - logsumexp(z2, axis=1)[:, None])
    S = P.reshape(h_kv, G, -1).sum(axis=1)
    scores = np.zeros((h_kv, bt + 1))
    out = []
    for g in range(h_kv):
        for b in range(bt + 1):
            over = [i for i, j in enumerate(vis1)
                    if p.c1_stride * j < B * (b + 1) and p.c1_stride * j + p.c1_kernel > B * b]
            scores[g, b] = S[g, over].max() if over else 0.0
        c = np.array(cands)
        order = np.lexsort((c, -scores[g, c]))
        out.append(sorted(init | local | set(c[order[:p.n_topk]].tolist())))
    return out, scores


def pin_select_token_brute():
    """select_token (the whole selection of one query: LSE in the configured
    mode, group-summed probabilities, max pool, top-k union) against the
    brute-force pipeline above, in both LSE modes, for G = 2 and 4, on rows
    before and after the first row that needs scores; the LSE is reported
    exactly for the rows that need scores."""
    for seed, (h_q, h_kv) in ((19, (4, 2)), (20, (8, 2))):
        Q, K, _ = _tiny(seed, n=900, h_q=h_q, h_kv=h_kv, d=8)
        G = h_q // h_kv
        scale = 1 / math.sqrt(8)
        for mode in ("exact", "approx"):
            p = R.Params(n_init=1, n_local=2, n_topk=3, lse_mode=mode)
            KC1 = R.compress_keys(K, 32, 16)
            KC2 = R.compress_keys(K, 128, 64)
            for t in (0, 63, 64, 383, 384, 447, 448, 500, 640, 767, 899):
                idx, diag = R.select_token(Q[t], t, KC1, KC2, G, p)
                want, scores = _brute_select(Q, K, t, G, p, scale)
                if idx != want or diag["scored"] != (scores is not None):
                    return False
                if scores is None:
                    if diag["L"] is not None:
                        return False
                    continue
                bt = t // 64
                cand = np.arange(p.n_init, bt - p.n_local + 1)
                if not _close(diag["block_scores"][:, cand], scores[:, cand], 1e-11):
                    return False
                Lw = (R.lse_exact(Q[t], t, KC1, G, p) if mode == "exact"
                      else R.lse_approx(Q[t], t, KC2, G, p))
                nv = (len([j for j in range(KC1.shape[1]) if 16 * j + 31 <= t]) if mode == "exact"
                      else len([j for j in range(KC2.shape[1]) if 64 * j + 127 <= t]))
                kc = KC1 if mode == "exact" else KC2
                Lb = [logsumexp(_brute_logits(Q[t], kc, G, scale, h, nv)) for h in range(h_q)]
                if not (_close(diag["L"], Lb, 1e-11) and _close(Lw, Lb, 1e-11)):
                    return False
    return True


def pin_bf16_decoding():
    """as_f64 on bf16 bit patterns equals torch's bfloat16 -> float64
    conversion for all 65536 patterns (signed zeros, subnormals, infinities
    and NaNs included)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):          # signalling NaN patterns
        got = R.as_f64(bits)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    if got.dtype != np.float64 or got.shape != want.shape:
        return False
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    return bool(same.all() and np.array_equal(np.signbit(got), np.signbit(want))
                and R.as_f64(np.array([0x3F80], dtype=np.uint16))[0] == 1.0)


ALL_PINS = [pin_worked_example, pin_stage_parameters, pin_window_counts,
            pin_compress_by_convolution, pin_compress_constant, pin_compress_bf16_rounding,
            pin_lse_exact_scipy, pin_lse_approx_scipy, pin_group_sum_softmax,
            pin_constant_keys, pin_approx_bound, pin_pool_by_token_overlap,
            pin_topk_full_sort, pin_attention_sdpa, pin_attention_special_cases,
            pin_cost_identities, pin_grad_finite_differences, pin_grad_identities,
            pin_grad_dense_torch, pin_select_token_brute, pin_bf16_decoding]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    assert pin()


def test_decode_row_equals_prefill_row_and_incremental_compress():
    """A decode step at position t selects and attends exactly like prefill
    row t; appending windows one token at a time equals full compression."""
    Q, K, V = _tiny(18, n=1500, h_q=4, h_kv=2, d=16)
    p = R.Params(n_init=1, n_local=4, n_topk=6)
    KC1 = R.compress_keys(K[:1200], 32, 16)
    for t in range(1200, 1500):
        KC1 = R.compress_keys_incremental(K[:t + 1], KC1, 32, 16)
    if not np.array_equal(KC1, R.compress_keys(K, 32, 16)):
        raise AssertionError("incremental compression differs")
    full = R.prefill_select(Q, K, 2, p, positions=[1499, 1333])
    for t in (1499, 1333):
        dec = R.prefill_select(Q[t:t + 1], K[:t + 1], 2, p)
        assert dec[t][0] == full[t][0]
        o1 = R.prefill_attend(Q, K, V, 2, p, {t: full[t][0]})[t][0]
        o2 = R.prefill_attend(Q[t:t + 1], K[:t + 1], V[:t + 1], 2, p, {t: dec[t][0]})[t][0]
        assert np.array_equal(o1, o2)


# ------------------------------------------------ planted mistakes --------

def _wrong_n_visible(t, kernel, stride, n_total):          # one window too many
    if t < kernel - 2:
        return 0
    return min(n_total, (t - (kernel - 2)) // stride + 1)


def _wrong_shared_scores(q, t, KC1, L, G, p):               # sums logits, not probabilities
    d = KC1.shape[2]
    nv = R.n_visible(t, p.c1_kernel, p.c1_stride, KC1.shape[1])
    S = np.zeros((KC1.shape[0], KC1.shape[1]))
    z = R.logits(q, KC1[:, :nv], G, 1 / math.sqrt(d))
    for g in range(KC1.shape[0]):
        S[g, :nv] = (z[g * G:(g + 1) * G] - L[g * G:(g + 1) * G, None]).sum(axis=0)
    return S


def _wrong_logits(q, KC, G, scale):                          # head -> KV head transposed
    q = R.as_f64(q)
    h_kv = KC.shape[0]
    return np.stack([scale * (KC[h % h_kv] @ q[h]) for h in range(q.shape[0])])


def _wrong_compress(K, kernel, stride, round_bf16=False):   # window starts one token late
    K = R.as_f64(K)
    N = R.n_windows(K.shape[0] - 1, kernel, stride)
    out = np.empty((K.shape[1], N, K.shape[2]))
    for j in range(N):
        out[:, j, :] = K[stride * j + 1: stride * j + 1 + kernel].mean(axis=0)
    return out


def _wrong_attend(q, t, K, V, blocks, G, p):                # excludes the query itself
    B = p.block_size
    keys = [np.array([x for b in bl for x in range(b * B, min((b + 1) * B, t))] or [0])
            for bl in blocks]
    return R._attend(q, t, K, V, keys, G, 1 / math.sqrt(K.shape[2]))


def _wrong_select(t, score_row, p):                          # ties toward the higher index
    bt = t // p.block_size
    lo, hi = R.candidate_range(t, p)
    cands = list(range(lo, hi + 1)) if hi >= lo else []
    top = sorted(cands, key=lambda b: (-score_row[b], -b))[:p.n_topk]
    blocks = sorted(set(range(min(p.n_init, bt + 1))) | set(range(max(0, bt - p.n_local + 1), bt + 1)) | set(top))
    return blocks, {}


def _wrong_attend_grad_no_delta(q, dout, K, V, keys_per_group, G, scale):   # drops the dO . o term
    q, dout = R.as_f64(q), R.as_f64(dout)
    h_q, d = q.shape
    dq = np.zeros((h_q, d))
    dk = [np.zeros((len(u), d)) for u in keys_per_group]
    dv = [np.zeros((len(u), d)) for u in keys_per_group]
    for h in range(h_q):
        g = h // G
        u = keys_per_group[g]
        z = scale * (K[u, g] @ q[h])
        P = np.exp(z - z.max())
        P /= P.sum()
        dz = P * (V[u, g] @ dout[h])
        dq[h] = scale * (dz @ K[u, g])
        dk[g] += scale * np.outer(dz, q[h])
        dv[g] += np.outer(P, dout[h])
    return dq, dk, dv


def _wrong_attend_grad_unscaled_dk(q, dout, K, V, keys_per_group, G, scale):  # dk without the scale
    dq, dk, dv = _ORIG_ATTEND_GRAD(q, dout, K, V, keys_per_group, G, scale)
    return dq, [x / scale for x in dk], dv


def _wrong_attend_grad_dv_transposed(q, dout, K, V, keys_per_group, G, scale):  # dv from dz, not P
    q, dout = R.as_f64(q), R.as_f64(dout)
    dq, dk, dv = _ORIG_ATTEND_GRAD(q, dout, K, V, keys_per_group, G, scale)
    for h in range(q.shape[0]):
        g = h // G
        u = keys_per_group[g]
        z = scale * (K[u, g] @ q[h])
        P = np.exp(z - z.max())
        P /= P.sum()
        dv[g] += np.outer(P[::-1], dout[h]) - np.outer(P, dout[h])
    return dq, dk, dv



def _wrong_as_f64(x):                                        # bits read as float16
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return a.view(np.float16).astype(np.float64)
    return a.astype(np.float64)


def _select_token_variant(dispatch_swapped=False, gate=">"):
    """select_token with its LSE dispatch swapped or its scoring gate changed."""
    def fn(q, t, KC1, KC2, G, p):
        h_kv = KC1.shape[0]
        n_blocks = t // p.block_size + 1
        lo, hi = R.candidate_range(t, p)
        ncand = hi - lo + 1
        need = {">": ncand > p.n_topk, ">=": ncand >= p.n_topk, "never": False}[gate]
        if need:
            exact = (p.lse_mode == "exact") != dispatch_swapped
            L = R.lse_exact(q, t, KC1, G, p) if exact else R.lse_approx(q, t, KC2, G, p)
            S = R.shared_scores(q, t, KC1, L, G, p)
            bs = R.block_scores(S, n_blocks, p)
        else:
            L, bs = None, np.zeros((h_kv, n_blocks))
        idx, infos = [], []
        for g in range(h_kv):
            blocks, info = R.select_from_scores(t, bs[g], p)
            idx.append(blocks)
            infos.append(info)
        return idx, {"L": L, "block_scores": bs, "info": infos, "scored": need}
    return fn

_ORIG_ATTEND_GRAD = R._attend_grad


def _params_pad0(**kw):
    kw.setdefault("pool_pad", 0)
    return _ORIG_PARAMS(**kw)


_ORIG_PARAMS = R.Params

MUTATIONS = {
    "visibility_off_by_one": ("n_visible", _wrong_n_visible),
    "group_sum_of_logits": ("shared_scores", _wrong_shared_scores),
    "head_to_kv_transposed": ("logits", _wrong_logits),
    "window_start_shifted": ("compress_keys", _wrong_compress),
    "causal_excludes_self": ("attend_token", _wrong_attend),
    "ties_toward_higher_index": ("select_from_scores", _wrong_select),
    "grad_without_delta_term": ("_attend_grad", _wrong_attend_grad_no_delta),
    "grad_dk_unscaled": ("_attend_grad", _wrong_attend_grad_unscaled_dk),
    "grad_dv_keys_reversed": ("_attend_grad", _wrong_attend_grad_dv_transposed),
    "bf16_bits_read_as_fp16": ("as_f64", _wrong_as_f64),
    "select_lse_dispatch_swapped": ("select_token", _select_token_variant(dispatch_swapped=True)),
    "select_scores_gate_inclusive": ("select_token", _select_token_variant(gate=">=")),
    "select_scores_never": ("select_token", _select_token_variant(gate="never")),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(R, attr, fn)
    failed = []
    for pin in ALL_PINS:
        try:
            ok = pin()
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"


def test_planted_pool_padding_is_caught(monkeypatch):
    from dataclasses import replace
    orig = R.block_scores
    monkeypatch.setattr(R, "block_scores", lambda S, nb, p: orig(S, nb, replace(p, pool_pad=0)))
    assert not pin_pool_by_token_overlap()

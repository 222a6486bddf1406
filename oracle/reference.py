"""Plain, slow fp64 oracle of the InfLLM-V2 sparse-attention path.

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library or its Python binding.

Sources (the pages' own titles and sections):
  [R]  "论文阅读：InfLLM-V2" reading notes (xiaohongrsx.github.io): sections
       "先看一个具体例子" (worked example: token 20000 in block 313, 96 blocks of
       64 tokens), "对齐计算图" (one output branch), "Dense-Sparse Switchable
       Attention" (switch pseudocode).
  [T3] top168.com article, section 三 "块表示的三阶段压缩" (three-stage
       compression: mean pooling with l_C1 = B/2, s_C1 = B/4; group sum; max
       pooling with l = 5, s = 4).
  [T4] same article, section 四 "高效实现的技术突破" (two-pass LSE; LSE
       approximation with s_C2 = 4 s_C1, l_C2 = 4 l_C1).
  [T7] same article, section 七 "技术实现的创新细节" (init ∪ local ∪ top-k; local
       blocks cover the sliding window; GQA group size 16).

Everything is float64 except where a decision must be taken in the kernel's
precision: ``compress_keys(..., round_bf16=True)`` rounds the compressed keys
to bfloat16 exactly as the kernel stores them, so that block selection on both
sides starts from the same compressed keys.

Readings of points the pages leave open (each is stated where it is used):
  * a compressed window exists only when complete, and is visible to query t
    only when its last token is <= t;
  * the group sum adds softmax probabilities (not logits);
  * the max pool over block b covers stage-1 windows 4b-1 .. 4b+3 (kernel 5,
    stride 4, one window of left padding): exactly the windows that overlap
    the block's tokens;
  * top-k ties break toward the lower block index;
  * the approximate LSE is the plain log-sum-exp over visible coarse windows;
  * gradients (training, [R] "训练是怎么做的": the sparse attention is trained
    with the plain next-token objective) treat the block sets as constants:
    selection is a top-k, piecewise constant in q and k, and its scores
    reach no output.

Positions are per sequence and 0-based; with ``len_q`` queries and ``len_k``
keys, query i sits at position ``len_k - len_q + i`` (bottom-right causal).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Params", "as_f64", "round_to_bf16", "n_windows", "n_visible", "compress_keys",
    "compress_keys_incremental", "logits", "lse_exact", "lse_approx", "shared_scores",
    "block_scores", "select_from_scores", "select_token", "attend_token", "dense_token",
    "prefill_select", "prefill_attend", "dense_prefill", "candidate_range",
    "attend_token_grad", "attention_grad",
]


@dataclass(frozen=True)
class Params:
    """Method parameters.  Defaults are the pages' training setting."""
    block_size: int = 64      # B = 64 tokens  [R] worked example
    n_init: int = 1           # init blocks
    n_local: int = 32         # local blocks (include the query's own block)
    n_topk: int = 63          # |I| = 1 + 32 + 63 = 96  [R]
    c1_kernel: int = 32       # l_C1 = B/2  [T3]
    c1_stride: int = 16       # s_C1 = B/4  [T3]
    c2_kernel: int = 128      # l_C2 = 4 l_C1  [T4]
    c2_stride: int = 64       # s_C2 = 4 s_C1  [T4]
    pool_kernel: int = 5      # stage-3 max pool l = 5  [T3]
    pool_stride: int = 4      # s = 4  [T3]
    pool_pad: int = 1         # reading: one window of left padding
    lse_mode: str = "exact"   # "exact" (two-pass) or "approx" (coarse keys)  [T4]
    scale: float | None = None  # softmax scale; None -> 1/sqrt(d)
    round_kc: bool = False    # compressed keys rounded to bf16 (kernel storage)

    @property
    def n_sel(self) -> int:
        return self.n_init + self.n_local + self.n_topk

    def with_(self, **kw) -> "Params":
        return replace(self, **kw)


# --------------------------------------------------------------------------
# bf16 handling (own code; inputs arrive as bf16 bit patterns)
# --------------------------------------------------------------------------

def as_f64(x) -> np.ndarray:
    """bf16 bit patterns (uint16) or floats -> float64, exactly."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even),
    directly from float64 (no intermediate float32 rounding).  Returns float64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    m, e = np.frexp(x[nz])              # x = m * 2**e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits; the quantum is 2**(e-8), but never below
    # the smallest bf16 subnormal step 2**-133.
    q_exp = np.maximum(e - 8, -133)
    scaled = np.ldexp(x[nz], -q_exp)    # exact (power-of-two scaling)
    out[nz] = np.ldexp(np.rint(scaled), q_exp)   # rint: ties to even
    return out


# --------------------------------------------------------------------------
# Stage 1: mean-pooled compressed keys  [T3]
# --------------------------------------------------------------------------

def n_windows(n: int, kernel: int, stride: int) -> int:
    """Number of complete windows of length ``kernel`` at ``stride`` in n tokens."""
    if n < kernel:
        return 0
    return (n - kernel) // stride + 1


def n_visible(t: int, kernel: int, stride: int, n_total: int) -> int:
    """Windows j whose last token stride*j + kernel - 1 is <= t (a prefix)."""
    if t < kernel - 1:
        return 0
    return min(n_total, (t - (kernel - 1)) // stride + 1)


def compress_keys(K, kernel: int, stride: int, round_bf16: bool = False) -> np.ndarray:
    """K [n, h_kv, d] -> K_C [h_kv, N, d]: K_C[g, j] = mean of K[stride*j : stride*j + kernel, g]."""
    K = as_f64(K)
    n, h_kv, d = K.shape
    N = n_windows(n, kernel, stride)
    out = np.empty((h_kv, N, d), dtype=np.float64)
    for j in range(N):
        out[:, j, :] = K[stride * j: stride * j + kernel].sum(axis=0) / kernel
    return round_to_bf16(out) if round_bf16 else out


def compress_keys_incremental(K, prev: np.ndarray, kernel: int, stride: int,
                              round_bf16: bool = False) -> np.ndarray:
    """Append the windows completed since ``prev`` was computed (decode).
    Only the key rows of the new windows are read."""
    K = np.asarray(K)
    N = n_windows(K.shape[0], kernel, stride)
    have = prev.shape[1]
    new = np.empty((K.shape[1], N - have, K.shape[2]))
    for j in range(have, N):
        new[:, j - have, :] = as_f64(K[stride * j: stride * j + kernel]).sum(axis=0) / kernel
    if round_bf16:
        new = round_to_bf16(new)
    return np.concatenate([prev, new], axis=1)


# --------------------------------------------------------------------------
# Stage 2: compressed attention scores, LSE, group sum  [T3], [T4]
# --------------------------------------------------------------------------

def _scale(p: Params, d: int) -> float:
    return p.scale if p.scale is not None else 1.0 / math.sqrt(d)


def logits(q, KC: np.ndarray, G: int, scale: float) -> np.ndarray:
    """q [h_q, d], KC [h_kv, N, d] -> z [h_q, N] with z[h, j] = scale * q[h] . KC[h // G, j]."""
    q = as_f64(q)
    return np.stack([scale * (KC[h // G] @ q[h]) for h in range(q.shape[0])])


def _logsumexp(z: np.ndarray) -> np.ndarray:
    """Row-wise log-sum-exp of z [h, m]; -inf for an empty row."""
    if z.shape[1] == 0:
        return np.full(z.shape[0], -np.inf)
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def lse_exact(q, t: int, KC1: np.ndarray, G: int, p: Params) -> np.ndarray:
    """Exact normaliser of the stage-1 softmax of query t over its visible
    windows (the first pass of the two-pass scheme)  [T4]."""
    d = KC1.shape[2]
    nv = n_visible(t, p.c1_kernel, p.c1_stride, KC1.shape[1])
    return _logsumexp(logits(q, KC1[:, :nv], G, _scale(p, d)))


def lse_approx(q, t: int, KC2: np.ndarray, G: int, p: Params) -> np.ndarray:
    """LSE approximation: the same log-sum-exp taken over the coarse
    compressed keys (kernel l_C2, stride s_C2) visible to t  [T4]."""
    d = KC2.shape[2]
    nv = n_visible(t, p.c2_kernel, p.c2_stride, KC2.shape[1])
    return _logsumexp(logits(q, KC2[:, :nv], G, _scale(p, d)))


def shared_scores(q, t: int, KC1: np.ndarray, L: np.ndarray, G: int, p: Params) -> np.ndarray:
    """S_shared [h_kv, N1]: per KV group, the sum over the group's heads of
    the stage-1 softmax probabilities exp(z - L); zero for windows not visible
    to t  [T3] (group sum), [T4] (second pass)."""
    d = KC1.shape[2]
    h_q = np.asarray(q).shape[0]
    h_kv, N1 = KC1.shape[0], KC1.shape[1]
    nv = n_visible(t, p.c1_kernel, p.c1_stride, N1)
    S = np.zeros((h_kv, N1))
    if nv == 0:
        return S
    z = logits(q, KC1[:, :nv], G, _scale(p, d))
    prob = np.exp(z - L[:, None])
    for g in range(h_kv):
        S[g, :nv] = prob[g * G:(g + 1) * G].sum(axis=0)
    assert h_q == h_kv * G
    return S


# --------------------------------------------------------------------------
# Stage 3: max pooling to block scores  [T3]
# --------------------------------------------------------------------------

def block_scores(S: np.ndarray, n_blocks: int, p: Params) -> np.ndarray:
    """score[g, b] = max of S[g, j] over the pool window of block b:
    j in [pool_stride*b - pool_pad, pool_stride*b - pool_pad + pool_kernel),
    clipped to existing windows; 0 when the clipped window is empty."""
    h_kv, N1 = S.shape
    out = np.zeros((h_kv, n_blocks))
    for b in range(n_blocks):
        lo = max(0, p.pool_stride * b - p.pool_pad)
        hi = min(N1, p.pool_stride * b - p.pool_pad + p.pool_kernel)
        if hi > lo:
            out[:, b] = S[:, lo:hi].max(axis=1)
    return out


# --------------------------------------------------------------------------
# Selection: init ∪ local ∪ top-k  [T7], [R]
# --------------------------------------------------------------------------

def candidate_range(t: int, p: Params):
    """Top-k candidates of query t: blocks n_init .. b_t - n_local (inclusive)."""
    bt = t // p.block_size
    return p.n_init, bt - p.n_local


def select_from_scores(t: int, score_row: np.ndarray, p: Params):
    """Selected block set of query t for one KV group, ascending.

    Init = {0 .. n_init-1}; local = {b_t-n_local+1 .. b_t} (the query's own
    block and the blocks right before it); top-k over the remaining causal
    blocks, largest score first, ties toward the lower block index.  Returns
    (blocks, info) where info holds the sorted candidate scores for the
    acceptance rule.
    """
    bt = t // p.block_size
    init = set(range(0, min(p.n_init, bt + 1)))
    local = set(range(max(0, bt - p.n_local + 1), bt + 1))
    lo, hi = candidate_range(t, p)
    cands = list(range(lo, hi + 1)) if hi >= lo else []
    if len(cands) <= p.n_topk:
        top = cands
        order = cands
    else:
        # sort by (score desc, index asc)
        order = sorted(cands, key=lambda b: (-score_row[b], b))
        top = order[:p.n_topk]
    blocks = sorted(init | local | set(top))
    info = {"cands": cands, "order": order,
            "scores": np.array([score_row[b] for b in order])}
    return blocks, info


def select_token(q, t: int, KC1: np.ndarray, KC2, G: int, p: Params):
    """Full selection for query t: LSE (exact or approx), group-summed
    scores, max pool, top-k union.  Returns (idx [h_kv][list], diag)."""
    h_kv = KC1.shape[0]
    n_blocks = t // p.block_size + 1
    lo, hi = candidate_range(t, p)
    need_scores = (hi - lo + 1) > p.n_topk
    if need_scores:
        L = lse_exact(q, t, KC1, G, p) if p.lse_mode == "exact" else lse_approx(q, t, KC2, G, p)
        S = shared_scores(q, t, KC1, L, G, p)
        bs = block_scores(S, n_blocks, p)
    else:
        L = None
        bs = np.zeros((h_kv, n_blocks))
    idx, infos = [], []
    for g in range(h_kv):
        blocks, info = select_from_scores(t, bs[g], p)
        idx.append(blocks)
        infos.append(info)
    return idx, {"L": L, "block_scores": bs, "info": infos, "scored": need_scores}


# --------------------------------------------------------------------------
# Attention  [R] (switch pseudocode), [T7] (single unified sparse branch)
# --------------------------------------------------------------------------

def _attend(q, t: int, K, V, keys_per_group, G: int, scale: float):
    q = as_f64(q)
    h_q, d = q.shape
    o = np.zeros((h_q, d))
    lse = np.zeros(h_q)
    for g, u in enumerate(keys_per_group):
        Ku, Vu = K[u, g], V[u, g]          # the group's keys and values, gathered once
        for h in range(g * G, (g + 1) * G):
            z = scale * (Ku @ q[h])
            m = z.max()
            w = np.exp(z - m)
            o[h] = (w @ Vu) / w.sum()
            lse[h] = m + math.log(w.sum())
    return o, lse


def attend_token(q, t: int, K, V, blocks, G: int, p: Params):
    """Sparse attention of query t: softmax over keys u <= t whose block
    floor(u / B) is in the group's selected set, applied to V.  K, V are
    float64 [n, h_kv, d]; ``blocks`` is one ascending list per KV group."""
    B = p.block_size
    keys = []
    for blist in blocks:
        u = [x for b in blist if b >= 0 for x in range(b * B, min((b + 1) * B, t + 1))]
        keys.append(np.array(u, dtype=np.int64))
    return _attend(q, t, K, V, keys, G, _scale(p, K.shape[2]))


def dense_token(q, t: int, K, V, G: int, scale: float):
    """Dense causal attention of query t over keys 0..t."""
    h_kv = K.shape[1]
    keys = [np.arange(t + 1)] * h_kv
    return _attend(q, t, K, V, keys, G, scale)


# --------------------------------------------------------------------------
# Per-sequence drivers (small sizes, or sampled rows of large ones)
# --------------------------------------------------------------------------

def _compressed(K, p: Params):
    KC1 = compress_keys(K, p.c1_kernel, p.c1_stride, p.round_kc)
    KC2 = compress_keys(K, p.c2_kernel, p.c2_stride, p.round_kc) if p.lse_mode == "approx" else None
    return KC1, KC2


def prefill_select(Q, K, G: int, p: Params, positions=None, KC1=None, KC2=None):
    """Selection for the given positions of one sequence (all by default).
    Q: [len_q, h_q, d] bits or floats, queries at the last len_q positions."""
    Q = np.asarray(Q)
    n_k = np.asarray(K).shape[0]
    n_q = Q.shape[0]
    if KC1 is None:
        KC1, KC2 = _compressed(K, p)
    if positions is None:
        positions = range(n_k - n_q, n_k)
    out = {}
    for t in positions:
        out[t] = select_token(Q[t - (n_k - n_q)], t, KC1, KC2, G, p)
    return out


def prefill_attend(Q, K, V, G: int, p: Params, idx_by_pos: dict):
    """Sparse attention outputs for the positions in ``idx_by_pos``."""
    Kf, Vf = as_f64(K), as_f64(V)
    n_k, n_q = Kf.shape[0], np.asarray(Q).shape[0]
    res = {}
    for t, blocks in idx_by_pos.items():
        res[t] = attend_token(np.asarray(Q)[t - (n_k - n_q)], t, Kf, Vf, blocks, G, p)
    return res


def dense_prefill(Q, K, V, G: int, scale: float, positions=None):
    Kf, Vf = as_f64(K), as_f64(V)
    n_k, n_q = Kf.shape[0], np.asarray(Q).shape[0]
    if positions is None:
        positions = range(n_k - n_q, n_k)
    return {t: dense_token(np.asarray(Q)[t - (n_k - n_q)], t, Kf, Vf, G, scale) for t in positions}


# --------------------------------------------------------------------------
# Gradients of the sparse attention, block sets held fixed  [R] (training:
# "训练是怎么做的", long-context fine-tuning through the sparse attention)
# --------------------------------------------------------------------------
#
# For one query and head with logits z_u = scale * q . k_u over its key set
# T, probabilities P_u = exp(z_u) / sum_w exp(z_w) and output o = sum_u P_u v_u,
# an upstream gradient dO = dl/do gives, by the chain rule through the
# softmax Jacobian dP_u/dz_w = P_u (delta_uw - P_w):
#   dl/dv_u = P_u dO
#   dl/dz_u = P_u (dO . v_u - dO . o)
#   dl/dq   = scale * sum_u dl/dz_u k_u,   dl/dk_u = scale * dl/dz_u q.
# Query heads of one group add their dk, dv into the group's shared K, V.

def _attend_grad(q, dout, K, V, keys_per_group, G: int, scale: float):
    q, dout = as_f64(q), as_f64(dout)
    h_q, d = q.shape
    dq = np.zeros((h_q, d))
    dk = [np.zeros((len(u), d)) for u in keys_per_group]
    dv = [np.zeros((len(u), d)) for u in keys_per_group]
    for h in range(h_q):
        g = h // G
        u = keys_per_group[g]
        if len(u) == 0:
            continue
        Ku, Vu = K[u, g], V[u, g]
        z = scale * (Ku @ q[h])
        w = np.exp(z - z.max())
        P = w / w.sum()
        o = P @ Vu
        dz = P * (Vu @ dout[h] - dout[h] @ o)
        dq[h] = scale * (dz @ Ku)
        dk[g] += scale * np.outer(dz, q[h])
        dv[g] += np.outer(P, dout[h])
    return dq, dk, dv


def _keys_of(blocks, t: int, B: int):
    """Keys u <= t of the given blocks, read as a set (-1 and repeats skipped)."""
    bs = sorted({b for b in blocks if 0 <= b <= t // B})
    return np.array([x for b in bs for x in range(b * B, min((b + 1) * B, t + 1))], dtype=np.int64)


def attend_token_grad(q, dout, t: int, K, V, blocks, G: int, p: Params):
    """Gradients of sum(dout * o) for the sparse attention of query t (see
    attend_token).  Returns dq [h_q, d] and, per KV group, (keys, dk rows,
    dv rows) of its contribution to the key gradients."""
    B = p.block_size
    keys = [_keys_of(bl, t, B) for bl in blocks]
    dq, dk, dv = _attend_grad(q, dout, K, V, keys, G, _scale(p, K.shape[2]))
    return dq, [(keys[g], dk[g], dv[g]) for g in range(len(keys))]


def attention_grad(Q, K, V, dO, G: int, p: Params, idx_by_pos=None, dense: bool = False):
    """Whole-sequence gradients (dQ, dK, dV) of sum(dO * O) for one sequence:
    queries are the last len_q positions of the len_k keys; ``idx_by_pos``
    maps each position to its per-group block lists (the selection, held
    fixed); ``dense`` uses every causal key instead."""
    Kf, Vf = as_f64(K), as_f64(V)
    Qa, dOa = np.asarray(Q), np.asarray(dO)
    n_k, n_q = Kf.shape[0], Qa.shape[0]
    h_kv = Kf.shape[1]
    dQ = np.zeros(Qa.shape, dtype=np.float64)
    dK = np.zeros(Kf.shape)
    dV = np.zeros(Vf.shape)
    nblk = (n_k + p.block_size - 1) // p.block_size
    for i in range(n_q):
        t = n_k - n_q + i
        blocks = [list(range(nblk))] * h_kv if dense else idx_by_pos[t]
        dq, parts = attend_token_grad(Qa[i], dOa[i], t, Kf, Vf, blocks, G, p)
        dQ[i] = dq
        for g, (u, dk, dv) in enumerate(parts):
            dK[u, g] += dk
            dV[u, g] += dv
    return dQ, dK, dV

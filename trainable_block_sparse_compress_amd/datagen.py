"""Seeded synthetic inputs for the InfLLM-V2 sparse-attention path.

This module only draws and rounds numbers; it holds none of the method's
arithmetic (no compression, scoring, selection or attention).  Both the HIP
path (through the binding) and the CPU oracle consume what it returns, so the
two sides always see bit-identical bf16 inputs.

Shapes follow the 8B GQA layer the pages describe (32 query heads, 2 KV heads,
head_dim 128: top168.com article, section 5 "experiments"), blocks of 64 tokens
and a visible budget of 96 blocks (xiaohongrsx.github.io reading notes,
"a concrete example").  Values are i.i.d. N(0, 1), drawn in float32 from
``numpy.random.Generator(PCG64(seed))`` and rounded to bfloat16 with
round-to-nearest-even.

Needle blocks give top-k something to find.  The literal recipe "shift the
needle keys by 0.5 * mean(Q)" is inert for i.i.d. queries (the mean is ~1e-3
per element), so a needle block's keys (every key of the block, one KV head at
a time) are shifted by ``needle_scale * sqrt(d) * u_g`` where ``u_g`` is the
unit vector along the mean query of that KV head's query-head group.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "PrefillInputs",
    "make_prefill",
    "varlen_lengths",
    "DecodeInputs",
    "make_decode",
    "make_grad",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as uint16.  NaN is not expected in the inputs
    and is not special-cased.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _unit_group_mean(q_bits: np.ndarray, h_kv: int) -> np.ndarray:
    """Unit vector along the mean query of each KV head's group: [h_kv, d]."""
    n, h_q, d = q_bits.shape
    g = h_q // h_kv
    dirs = np.zeros((h_kv, d), dtype=np.float64)
    chunk = 8192
    for s in range(0, n, chunk):
        qf = bf16_bits_to_f32(q_bits[s:s + chunk]).astype(np.float64)
        dirs += qf.reshape(-1, h_kv, g, d).sum(axis=(0, 2))
    norms = np.linalg.norm(dirs, axis=1, keepdims=True)
    norms[norms == 0] = 1.0
    return dirs / norms


@dataclass
class PrefillInputs:
    q: np.ndarray            # uint16 bf16 bits [total, h_q, d]
    k: np.ndarray            # uint16 bf16 bits [total, h_kv, d]
    v: np.ndarray            # uint16 bf16 bits [total, h_kv, d]
    cu_seqlens: np.ndarray   # int32 [batch + 1]
    needles: list = field(default_factory=list)  # per sequence: needle block ids
    seed: int = 0
    needle_scale: float = 0.0


def _draw_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def make_prefill(seed: int, lengths, h_q: int, h_kv: int, d: int = 128,
                 n_needles: int = 0, needle_scale: float = 0.5,
                 block_size: int = 64, needle_lo: int = 1,
                 needle_hi_margin: int = 33) -> PrefillInputs:
    """Packed (varlen) prefill inputs.

    Draw order: Q, K, V for the whole packed batch, then for each sequence the
    needle block ids (without replacement, from ``[needle_lo, nblocks -
    needle_hi_margin)``), then the needle shift.  ``lengths`` may be an int
    (one sequence).
    """
    if isinstance(lengths, (int, np.integer)):
        lengths = [int(lengths)]
    lengths = [int(x) for x in lengths]
    total = int(sum(lengths))
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _draw_bf16(rng, (total, h_q, d))
    k = _draw_bf16(rng, (total, h_kv, d))
    v = _draw_bf16(rng, (total, h_kv, d))
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    needles = []
    if n_needles > 0:
        for s, n in enumerate(lengths):
            nblk = (n + block_size - 1) // block_size
            hi = nblk - needle_hi_margin
            if hi - needle_lo < n_needles:
                needles.append([])
                continue
            ids = np.sort(rng.choice(np.arange(needle_lo, hi), size=n_needles, replace=False))
            needles.append([int(i) for i in ids])
            start = int(cu[s])
            dirs = _unit_group_mean(q[start:start + n], h_kv)  # [h_kv, d]
            shift = (needle_scale * math.sqrt(d) * dirs).astype(np.float32)
            for b in ids:
                lo = start + int(b) * block_size
                hi_t = min(start + n, lo + block_size)
                kf = bf16_bits_to_f32(k[lo:hi_t]) + shift[None, :, :]
                k[lo:hi_t] = f32_to_bf16_bits(kf)
    return PrefillInputs(q=q, k=k, v=v, cu_seqlens=cu, needles=needles, seed=seed,
                         needle_scale=needle_scale if n_needles else 0.0)


_BUCKETS = ((1, 4096), (4097, 12288), (12289, 24576), (24577, 32768))


def varlen_lengths(seed: int, total: int = 65536, buckets=_BUCKETS) -> list:
    """Sequence lengths for a packed batch of exactly ``total`` tokens.

    A bucket is picked uniformly, then a length uniformly inside it; the last
    sequence is truncated so the lengths sum to ``total``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    left = total
    while left > 0:
        lo, hi = buckets[int(rng.integers(0, len(buckets)))]
        n = int(rng.integers(lo, hi + 1))
        n = min(n, left)
        out.append(n)
        left -= n
    return out


@dataclass
class DecodeInputs:
    k_cache: np.ndarray   # uint16 [batch, cap, h_kv, d]; first len0 rows filled
    v_cache: np.ndarray   # uint16 [batch, cap, h_kv, d]
    q_steps: np.ndarray   # uint16 [steps, batch, h_q, d]
    k_steps: np.ndarray   # uint16 [steps, batch, h_kv, d]
    v_steps: np.ndarray   # uint16 [steps, batch, h_kv, d]
    len0: int
    needles: list
    seed: int
    needle_scale: float


def make_decode(seed: int, batch: int, len0: int, steps: int, h_q: int, h_kv: int,
                d: int = 128, n_needles: int = 0, needle_scale: float = 0.5,
                block_size: int = 64, needle_hi_margin: int = 33,
                threads: int = 8) -> DecodeInputs:
    """Decode inputs: a KV cache of ``len0`` tokens per sequence plus ``steps``
    new (q, k, v) tokens per sequence.  Cache capacity is ``len0 + steps``.

    Streams: ``SeedSequence(seed)`` is split into batch + 1 child streams.
    Child s draws sequence s's cache K, then its cache V (so the sequences
    can be drawn in parallel threads with the same result); the last child
    draws the step Q, K, V, then the needle ids and shifts of each sequence.
    The needle direction is the unit mean of that sequence's step queries over
    the group's heads.
    """
    from concurrent.futures import ThreadPoolExecutor

    children = np.random.SeedSequence(seed).spawn(batch + 1)
    cap = len0 + steps
    k_cache = np.zeros((batch, cap, h_kv, d), dtype=np.uint16)
    v_cache = np.zeros((batch, cap, h_kv, d), dtype=np.uint16)

    def draw_cache(s):
        r = np.random.Generator(np.random.PCG64(children[s]))
        k_cache[s, :len0] = _draw_bf16(r, (len0, h_kv, d))
        v_cache[s, :len0] = _draw_bf16(r, (len0, h_kv, d))

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(draw_cache, range(batch)))
    rng = np.random.Generator(np.random.PCG64(children[batch]))
    q_steps = _draw_bf16(rng, (steps, batch, h_q, d))
    k_steps = _draw_bf16(rng, (steps, batch, h_kv, d))
    v_steps = _draw_bf16(rng, (steps, batch, h_kv, d))
    needles = []
    if n_needles > 0:
        nblk = len0 // block_size
        for s in range(batch):
            ids = np.sort(rng.choice(np.arange(1, nblk - needle_hi_margin), size=n_needles,
                                     replace=False))
            needles.append([int(i) for i in ids])
            dirs = _unit_group_mean(q_steps[:, s], h_kv)
            shift = (needle_scale * math.sqrt(d) * dirs).astype(np.float32)
            for b in ids:
                lo = int(b) * block_size
                kf = bf16_bits_to_f32(k_cache[s, lo:lo + block_size]) + shift[None, :, :]
                k_cache[s, lo:lo + block_size] = f32_to_bf16_bits(kf)
    return DecodeInputs(k_cache=k_cache, v_cache=v_cache, q_steps=q_steps, k_steps=k_steps,
                        v_steps=v_steps, len0=len0, needles=needles, seed=seed,
                        needle_scale=needle_scale if n_needles else 0.0)


def make_grad(seed: int, rows: int, h_q: int, d: int = 128) -> np.ndarray:
    """Upstream gradient of the attention output for the backward: i.i.d.
    N(0, 1) bf16 bits [rows, h_q, d] from its own seeded stream."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _draw_bf16(rng, (int(rows), h_q, d))

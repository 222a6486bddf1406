"""InfLLM-V2 attention over packed batches: the dense/sparse switch and
preallocated execution plans, on top of the C ABI.

The switch follows the reading notes "论文阅读：InfLLM-V2", section
"Dense-Sparse Switchable Attention": a sequence no longer than ``threshold``
tokens takes dense attention, a longer one the sparse path (compressed keys
-> block selection -> sparse attention).  Only one path runs per sequence.
The switch is host logic over host-known lengths; every numeric step runs in
the library's kernels.  PyTorch supplies device memory and the stream.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import binding as B

__all__ = ["SparseConfig", "n_windows", "SparsePlan", "DensePlan", "SwitchPlan", "attention",
           "DecodeState", "DecodeGraph", "attention_trainable"]


@dataclass(frozen=True)
class SparseConfig:
    block_size: int = 64       # B (reading notes, worked example)
    n_init: int = 1
    n_local: int = 32
    n_topk: int = 63           # 1 + 32 + 63 = 96 visible blocks
    c1: tuple = (32, 16)       # (l_C1, s_C1) = (B/2, B/4)
    c2: tuple = (128, 64)      # (4 l_C1, 4 s_C1), LSE approximation
    pool: tuple = (5, 4, 1)    # max pool kernel, stride, left pad
    lse_mode: str = "exact"    # "exact" (two-pass) or "approx"
    threshold: int = 8192      # sequences <= threshold take the dense path
    softmax_scale: float | None = None

    @property
    def n_sel(self) -> int:
        return self.n_init + self.n_local + self.n_topk

    def scale(self, d: int) -> float:
        return self.softmax_scale if self.softmax_scale is not None else 1.0 / math.sqrt(d)


def n_windows(n: int, kernel: int, stride: int) -> int:
    return 0 if n < kernel else (n - kernel) // stride + 1


def _i32(x, device):
    return torch.tensor(list(x), dtype=torch.int32, device=device)


class SparsePlan:
    """Buffers of the sparse path for sequences given by host-side
    (q start, q length, k start, k length) lists.  ``run`` enqueues
    compress_k (stage 1, plus the coarse keys in approx mode),
    select_blocks and sparse_attn on the current stream; nothing is
    allocated inside ``run``."""

    def __init__(self, q_starts, q_lens, k_starts, k_lens, rows_q, h_q, h_kv, cfg: SparseConfig,
                 device="cuda", d=128, unfused_select=False):
        self.cfg = cfg
        self.unfused_select = unfused_select   # the fusion-ablation baseline of the selection
        self.batch = len(q_lens)
        self.max_q = max(q_lens) if q_lens else 0
        self.max_k = max(k_lens) if k_lens else 0
        self.rows_q, self.h_q, self.h_kv, self.d = rows_q, h_q, h_kv, d
        self.cu_q = _i32(q_starts, device)
        self.used_q = _i32(q_lens, device)
        self.cu_k = _i32(k_starts, device)
        self.used_k = _i32(k_lens, device)
        n1 = [n_windows(n, *cfg.c1) for n in k_lens]
        off1 = [0]
        for x in n1[:-1]:
            off1.append(off1[-1] + x)
        self.cu_c1 = _i32(off1, device)
        self.kc1 = torch.empty((h_kv, max(1, sum(n1)), d), dtype=torch.bfloat16, device=device)
        self.approx = cfg.lse_mode == "approx"
        if self.approx:
            n2 = [n_windows(n, *cfg.c2) for n in k_lens]
            off2 = [0]
            for x in n2[:-1]:
                off2.append(off2[-1] + x)
            self.cu_c2 = _i32(off2, device)
            self.kc2 = torch.empty((h_kv, max(1, sum(n2)), d), dtype=torch.bfloat16, device=device)
        else:
            self.cu_c2, self.kc2 = None, None
        self.block_idx = torch.empty((h_kv, rows_q, cfg.n_sel), dtype=torch.int32, device=device)
        ws1 = B.select_blocks_workspace(rows_q, h_q, h_kv, self.max_q, self.max_k, cfg.n_init,
                                        cfg.n_local, cfg.n_topk, self.approx, batch=self.batch,
                                        unfused=unfused_select)
        ws2 = B.attn_workspace(h_q, h_kv, self.batch, self.max_q, self.max_k, rows_q,
                               n_sel=cfg.n_sel, n_init=cfg.n_init, n_local=cfg.n_local)
        self.ws_select = torch.empty(ws1, dtype=torch.uint8, device=device)
        self.ws_attn = torch.empty(max(1, ws2), dtype=torch.uint8, device=device)

    def compress(self, k):
        c = self.cfg
        B.compress_k(k, self.cu_k, self.used_k, self.batch, self.max_k, c.c1[0], c.c1[1],
                     self.cu_c1, self.kc1)
        if self.approx:
            B.compress_k(k, self.cu_k, self.used_k, self.batch, self.max_k, c.c2[0], c.c2[1],
                         self.cu_c2, self.kc2)

    def select(self, q):
        c = self.cfg
        fn = B.select_blocks_unfused if self.unfused_select else B.select_blocks
        fn(q, self.kc1, self.kc2, self.cu_q, self.used_q, self.cu_k, self.used_k,
                        self.cu_c1, self.cu_c2, self.batch, self.max_q, self.max_k, c.n_init,
                        c.n_local, c.n_topk, c.scale(self.d), self.block_idx, self.ws_select,
                        block_size=c.block_size, c1=c.c1, c2=c.c2, pool=c.pool)

    def attend(self, q, k, v, out, lse=None):
        c = self.cfg
        B.sparse_attn(q, k, v, self.cu_q, self.used_q, self.cu_k, self.used_k, self.batch,
                      self.max_q, self.max_k, self.block_idx, c.n_init, c.n_local,
                      c.scale(self.d), out, lse, self.ws_attn, block_size=c.block_size)

    def run(self, q, k, v, out, lse=None):
        if self.batch == 0:
            return
        self.compress(k)
        self.select(q)
        self.attend(q, k, v, out, lse)

    def backward(self, q, k, v, out, lse, dout, dq, dk, dv, block_idx=None):
        """Gradients into dq, dk, dv (rows of these sequences) with the block
        lists held fixed: ``block_idx`` (the lists of the forward being
        differentiated), by default the lists the last ``run`` left in the
        plan.  The workspace is allocated on first use and kept."""
        if self.batch == 0:
            return
        c = self.cfg
        idx = self.block_idx if block_idx is None else block_idx
        if getattr(self, "ws_bwd", None) is None:
            size = B.attn_bwd_workspace(q.shape[1], k.shape[1], self.batch, self.max_q, self.max_k,
                                        q.shape[0], k.shape[0], n_sel=c.n_sel, n_init=c.n_init,
                                        n_local=c.n_local)
            self.ws_bwd = torch.empty(max(1, size), dtype=torch.uint8, device=q.device)
        B.sparse_attn_bwd(q, k, v, out, lse, dout, self.cu_q, self.used_q, self.cu_k, self.used_k,
                          self.batch, self.max_q, self.max_k, idx, c.n_init, c.n_local,
                          c.scale(self.d), dq, dk, dv, self.ws_bwd, block_size=c.block_size)


class DensePlan:
    """Dense causal attention for the given sequences."""

    def __init__(self, q_starts, q_lens, k_starts, k_lens, rows_q, h_q, h_kv, cfg: SparseConfig,
                 device="cuda", d=128):
        self.cfg, self.d = cfg, d
        self.batch = len(q_lens)
        self.max_q = max(q_lens) if q_lens else 0
        self.max_k = max(k_lens) if k_lens else 0
        self.cu_q = _i32(q_starts, device)
        self.used_q = _i32(q_lens, device)
        self.cu_k = _i32(k_starts, device)
        self.used_k = _i32(k_lens, device)
        ws = B.attn_workspace(h_q, h_kv, self.batch, self.max_q, self.max_k, rows_q)
        self.ws = torch.empty(max(1, ws), dtype=torch.uint8, device=device)

    def run(self, q, k, v, out, lse=None):
        if self.batch == 0:
            return
        B.dense_attn(q, k, v, self.cu_q, self.used_q, self.cu_k, self.used_k, self.batch,
                     self.max_q, self.max_k, self.cfg.scale(self.d), out, lse, self.ws)

    def backward(self, q, k, v, out, lse, dout, dq, dk, dv):
        """Gradients of the dense causal attention of these sequences."""
        if self.batch == 0:
            return
        if getattr(self, "ws_bwd", None) is None:
            size = B.attn_bwd_workspace(q.shape[1], k.shape[1], self.batch, self.max_q, self.max_k,
                                        q.shape[0], k.shape[0])
            self.ws_bwd = torch.empty(max(1, size), dtype=torch.uint8, device=q.device)
        B.sparse_attn_bwd(q, k, v, out, lse, dout, self.cu_q, self.used_q, self.cu_k, self.used_k,
                          self.batch, self.max_q, self.max_k, None, 0, 0, self.cfg.scale(self.d),
                          dq, dk, dv, self.ws_bwd)


class SwitchPlan:
    """The dense/sparse switch over one packed prefill batch (queries and keys
    share rows).  Sequences of length <= threshold go to a DensePlan, the rest
    to a SparsePlan; both write into the same packed output."""

    def __init__(self, seqlens, h_q, h_kv, cfg: SparseConfig, device="cuda", d=128):
        seqlens = [int(n) for n in seqlens]
        starts = [0]
        for n in seqlens[:-1]:
            starts.append(starts[-1] + n)
        self.rows = sum(seqlens)
        self.dense_ids = [i for i, n in enumerate(seqlens) if n <= cfg.threshold]
        self.sparse_ids = [i for i, n in enumerate(seqlens) if n > cfg.threshold]
        ds = [starts[i] for i in self.dense_ids]
        dl = [seqlens[i] for i in self.dense_ids]
        ss = [starts[i] for i in self.sparse_ids]
        sl = [seqlens[i] for i in self.sparse_ids]
        self.dense = DensePlan(ds, dl, ds, dl, self.rows, h_q, h_kv, cfg, device, d)
        self.sparse = SparsePlan(ss, sl, ss, sl, self.rows, h_q, h_kv, cfg, device, d)

    def run(self, q, k, v, out, lse=None):
        self.dense.run(q, k, v, out, lse)
        self.sparse.run(q, k, v, out, lse)

    def backward(self, q, k, v, out, lse, dout, dq, dk, dv, block_idx=None):
        """Gradients of a forward of this plan (``block_idx``: the sparse
        sequences' lists of that forward, by default those of the last
        ``run``); dense and sparse sequences write disjoint rows of dq, dk,
        dv."""
        self.dense.backward(q, k, v, out, lse, dout, dq, dk, dv)
        self.sparse.backward(q, k, v, out, lse, dout, dq, dk, dv, block_idx)


def attention(q, k, v, seqlens, cfg: SparseConfig | None = None, lse=None):
    """InfLLM-V2 attention of a packed prefill batch; returns the output."""
    cfg = cfg or SparseConfig()
    plan = SwitchPlan(seqlens, q.shape[1], k.shape[1], cfg, q.device, q.shape[2])
    out = torch.empty_like(q)
    plan.run(q, k, v, out, lse)
    return out


class _SwitchAttention(torch.autograd.Function):
    """Forward through the switch's kernels (the sparse sequences' block lists
    from select_blocks), backward through infllmv2_sparse_attn_bwd on the same
    lists: the selection is held fixed, so no gradient reaches the scoring.
    The forward keeps its own copy of the lists, so a plan that serves
    several forwards before their backwards (layers of equal lengths) gives
    each backward the lists of its own forward."""

    @staticmethod
    def forward(ctx, q, k, v, plan):
        out = torch.empty_like(q)
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
        plan.run(q, k, v, out, lse)
        idx = plan.sparse.block_idx.clone() if plan.sparse.batch > 0 else None
        ctx.save_for_backward(q, k, v, out, lse, idx)
        ctx.plan = plan
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse, idx = ctx.saved_tensors
        dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
        ctx.plan.backward(q, k, v, out, lse, dout.to(torch.bfloat16).contiguous(), dq, dk, dv, idx)
        return dq, dk, dv, None


def attention_trainable(q, k, v, seqlens, cfg: SparseConfig | None = None, plan=None):
    """``attention`` with gradients (packed prefill batch, q/k/v bf16 with
    requires_grad).  Pass a SwitchPlan built for these lengths to reuse its
    buffers and workspaces across steps."""
    cfg = cfg or SparseConfig()
    plan = plan or SwitchPlan(seqlens, q.shape[1], k.shape[1], cfg, q.device, q.shape[2])
    return _SwitchAttention.apply(q, k, v, plan)


class DecodeState:
    """Decode over a batch of KV caches with capacity ``cap`` tokens each.

    K lives in ``k_cache`` [batch * cap, h_kv, d] (sequence s at rows
    s * cap ...); V lives transposed in ``vt_cache`` [h_kv, d, batch, cap] so
    that the attention kernel reads 8 consecutive keys of one dim per load.
    Compressed keys are kept per sequence at capacity offsets and updated
    incrementally: a step writes only the windows the new token completes.
    """

    def __init__(self, batch, cap, h_q, h_kv, cfg: SparseConfig, device="cuda", d=128):
        assert cap % 64 == 0
        self.batch, self.cap, self.h_q, self.h_kv, self.cfg, self.d = batch, cap, h_q, h_kv, cfg, d
        self.k_cache = torch.zeros((batch * cap, h_kv, d), dtype=torch.bfloat16, device=device)
        self.vt_cache = torch.zeros((h_kv, d, batch, cap), dtype=torch.bfloat16, device=device)
        self.cap1 = n_windows(cap, *cfg.c1)
        self.kc1 = torch.zeros((h_kv, batch * self.cap1, d), dtype=torch.bfloat16, device=device)
        self.cu_k = _i32([s * cap for s in range(batch)], device)
        self.cu_c1 = _i32([s * self.cap1 for s in range(batch)], device)
        self.approx = cfg.lse_mode == "approx"
        if self.approx:
            self.cap2 = n_windows(cap, *cfg.c2)
            self.kc2 = torch.zeros((h_kv, batch * self.cap2, d), dtype=torch.bfloat16, device=device)
            self.cu_c2 = _i32([s * self.cap2 for s in range(batch)], device)
        else:
            self.kc2, self.cu_c2 = None, None
        self.cu_q = _i32(range(batch), device)
        self.used_q = _i32([1] * batch, device)
        self.lens = [0] * batch
        self.used_k = torch.zeros(batch, dtype=torch.int32, device=device)
        self.begin1 = torch.zeros(batch, dtype=torch.int32, device=device)
        self.begin2 = torch.zeros(batch, dtype=torch.int32, device=device)
        self.block_idx = torch.empty((h_kv, batch, cfg.n_sel), dtype=torch.int32, device=device)
        ws = B.select_blocks_workspace(batch, h_q, h_kv, 1, cap, cfg.n_init, cfg.n_local,
                                       cfg.n_topk, self.approx, batch=batch)
        self.ws_select = torch.empty(ws, dtype=torch.uint8, device=device)
        ws = B.attn_workspace(h_q, h_kv, batch, 1, cap, batch, v_seq_stride=cap, n_sel=cfg.n_sel,
                              n_init=cfg.n_init, n_local=cfg.n_local)
        self.ws_attn = torch.empty(max(1, ws), dtype=torch.uint8, device=device)

    def fill(self, k_rows, v_rows, lens):
        """Load prefix K/V (lists of [len, h_kv, d] bf16 tensors) and compress."""
        for s, (kk, vv) in enumerate(zip(k_rows, v_rows)):
            self.fill_one(s, kk, vv)
        self.compress_all()

    def fill_one(self, s, k_rows, v_rows):
        """Load sequence s's prefix K/V ([len, h_kv, d] bf16); compress_all
        must follow once every sequence is loaded."""
        n = k_rows.shape[0]
        self.k_cache[s * self.cap: s * self.cap + n] = k_rows
        self.vt_cache[:, :, s, :n] = v_rows.permute(1, 2, 0)
        self.lens[s] = n

    def compress_all(self):
        """Compressed keys of the loaded prefixes."""
        self.used_k.copy_(torch.tensor(self.lens, dtype=torch.int32))
        c = self.cfg
        mx = max(self.lens)
        B.compress_k(self.k_cache, self.cu_k, self.used_k, self.batch, mx, c.c1[0], c.c1[1],
                     self.cu_c1, self.kc1)
        if self.approx:
            B.compress_k(self.k_cache, self.cu_k, self.used_k, self.batch, mx, c.c2[0], c.c2[1],
                         self.cu_c2, self.kc2)

    def append(self, k_new, v_new):
        """Caller-side cache write of one token per sequence ([batch, h_kv, d])."""
        rows = torch.tensor([s * self.cap + self.lens[s] for s in range(self.batch)],
                            device=k_new.device)
        self.k_cache.index_copy_(0, rows, k_new)
        for s in range(self.batch):
            self.vt_cache[:, :, s, self.lens[s]] = v_new[s]
        old = list(self.lens)
        self.lens = [n + 1 for n in self.lens]
        return old

    def step_prepare(self, old_lens):
        """Host-side metadata of a step: key lengths and first new windows."""
        c = self.cfg
        self.used_k.copy_(torch.tensor(self.lens, dtype=torch.int32), non_blocking=True)
        self.begin1.copy_(torch.tensor([n_windows(n, *c.c1) for n in old_lens], dtype=torch.int32),
                          non_blocking=True)
        if self.approx:
            self.begin2.copy_(torch.tensor([n_windows(n, *c.c2) for n in old_lens],
                                           dtype=torch.int32), non_blocking=True)

    def step(self, q_new, out, max_len):
        """One decode step after ``append``/``step_prepare``: incremental
        compression, selection for the new token, sparse attention."""
        c = self.cfg
        B.compress_k(self.k_cache, self.cu_k, self.used_k, self.batch, max_len, c.c1[0], c.c1[1],
                     self.cu_c1, self.kc1, cmp_begin=self.begin1, max_new=1)
        if self.approx:
            B.compress_k(self.k_cache, self.cu_k, self.used_k, self.batch, max_len, c.c2[0],
                         c.c2[1], self.cu_c2, self.kc2, cmp_begin=self.begin2, max_new=1)
        B.select_blocks(q_new, self.kc1, self.kc2, self.cu_q, self.used_q, self.cu_k, self.used_k,
                        self.cu_c1, self.cu_c2, self.batch, 1, max_len, c.n_init, c.n_local,
                        c.n_topk, c.scale(self.d), self.block_idx, self.ws_select)
        B.sparse_attn(q_new, self.k_cache, self.vt_cache, self.cu_q, self.used_q, self.cu_k,
                      self.used_k, self.batch, 1, max_len, self.block_idx, c.n_init, c.n_local,
                      c.scale(self.d), out, None, self.ws_attn, v_seq_stride=self.cap)


class DecodeGraph:
    """One decode step of a ``DecodeState`` captured as a HIP graph.

    The step is kernel launches only (the library allocates, frees and
    synchronises nothing), so it captures as is.  It is captured with the
    cache capacity as the maximum key length: grids cover the capacity and
    every kernel takes the actual lengths from the device metadata that
    ``append`` / ``step_prepare`` update, so one capture serves every step.
    ``step`` copies the new queries into the captured input buffer and
    replays; the result is in ``out``.
    """

    def __init__(self, dec: DecodeState):
        self.dec = dec
        dev = dec.k_cache.device
        self.q = torch.zeros((dec.batch, dec.h_q, dec.d), dtype=torch.bfloat16, device=dev)
        self.out = torch.zeros_like(self.q)
        self.graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(self.graph):
            dec.step(self.q, self.out, dec.cap)

    def step(self, q_new):
        self.q.copy_(q_new)
        self.graph.replay()
        return self.out

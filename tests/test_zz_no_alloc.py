"""infllmv2_sparse_attn_noalloc (scratch in the library's static per-GPU
array) against infllmv2_sparse_attn (caller workspace), through the C ABI:
the two run the same kernels on the same inputs, so their outputs and LSEs
must be bit-identical.  Two calls in a row on each path, the second with a
smaller input (the scratch keeps the first call's contents): decode (the
split-K path, partials in the scratch, transposed V cache) and prefill
with V in its natural layout (transposed into the scratch)."""
import numpy as np
import pytest
import torch

from trainable_block_sparse_compress_amd import binding as B
from trainable_block_sparse_compress_amd import datagen as D
from tests.gpu_util import i32, say, to_dev

pytestmark = pytest.mark.gpu


def _lists(rows_bt, h_kv, n_sel, seed):
    """Random block lists (sets with -1 pads) for rows with last blocks rows_bt."""
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = np.full((h_kv, len(rows_bt), n_sel), -1, dtype=np.int32)
    for r, bt in enumerate(rows_bt):
        for g in range(h_kv):
            k = min(bt + 1, n_sel)
            idx[g, r, :k] = np.sort(rng.choice(bt + 1, size=k, replace=False))
    return torch.from_numpy(idx).cuda()


def _both(q, k, v, cu_q, used_q, cu_k, used_k, batch, mq, mk, idx, v_stride):
    h_q, h_kv = q.shape[1], k.shape[1]
    outs = []
    for noalloc in (False, True):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((h_q, q.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            B.sparse_attn_noalloc(q, k, v, cu_q, used_q, cu_k, used_k, batch, mq, mk, idx, 1, 4, 0.088,
                                  out, lse, v_seq_stride=v_stride)
        else:
            ws = torch.empty(max(1, B.attn_workspace(h_q, h_kv, batch, mq, mk, q.shape[0],
                                                     v_seq_stride=v_stride, n_sel=idx.shape[-1],
                                                     n_init=1, n_local=4)),
                             dtype=torch.uint8, device="cuda")
            B.sparse_attn(q, k, v, cu_q, used_q, cu_k, used_k, batch, mq, mk, idx, 1, 4, 0.088, out,
                          lse, ws, v_seq_stride=v_stride)
        torch.cuda.synchronize()
        outs.append((out, lse))
    return outs


def test_noalloc_decode_two_calls(lib):
    """Decode: one new token per sequence over transposed V caches."""
    for batch, lens, seed in ((16, [20000 + 777 * s for s in range(16)], 1), (5, [3000 + 99 * s for s in range(5)], 2)):
        say(f"noalloc decode batch {batch}")
        cap = (max(lens) + 63) // 64 * 64
        h_q, h_kv = 32, 2
        inp = D.make_decode(seed, batch, cap, 1, h_q, h_kv)
        k = to_dev(np.ascontiguousarray(inp.k_cache[:, :cap]).reshape(batch * cap, h_kv, 128))
        vt = to_dev(np.ascontiguousarray(inp.v_cache[:, :cap].transpose(2, 3, 0, 1)))   # [h_kv, d, batch, cap]
        q = to_dev(np.ascontiguousarray(inp.q_steps[0]))
        idx = _lists([(n - 1) // 64 for n in lens], h_kv, 24, seed)
        cu_q, used_q = i32(range(batch)), i32([1] * batch)
        cu_k, used_k = i32([s * cap for s in range(batch)]), i32(lens)
        (o1, l1), (o2, l2) = _both(q, k, vt, cu_q, used_q, cu_k, used_k, batch, 1, max(lens), idx, cap)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)


def test_noalloc_prefill_two_calls(lib):
    """Prefill with V in its natural layout (transposed into the scratch)."""
    for lengths, seed in (([9000, 4100], 3), ([2000], 4)):
        say(f"noalloc prefill lengths {lengths}")
        h_q, h_kv = 32, 2
        inp = D.make_prefill(seed, lengths, h_q, h_kv)
        q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
        st = [0] + list(np.cumsum(lengths)[:-1])
        bts = [t // 64 for n in lengths for t in range(n)]
        idx = _lists(bts, h_kv, 12, seed)
        cu, used = i32(st), i32(lengths)
        (o1, l1), (o2, l2) = _both(q, k, v, cu, used, cu, used, len(lengths), max(lengths),
                                   max(lengths), idx, 0)
        assert not torch.isnan(o1.float()).any()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)

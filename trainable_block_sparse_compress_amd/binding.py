"""Thin ctypes binding of ``libinfllmv2.so`` (the C ABI in include/infllmv2.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers and shapes to the entry point of
the same name, and raises ``InfLLMv2Error`` on a non-zero return code.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  PyTorch provides device memory and the current stream.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "InfLLMv2Error", "load", "library_path", "version", "compress_k", "select_blocks",
    "select_blocks_workspace", "select_blocks_unfused", "sparse_attn", "sparse_attn_noalloc",
    "dense_attn", "attn_workspace",
    "sparse_attn_bwd", "attn_bwd_workspace",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "lib", "libinfllmv2.so")
_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZP = ctypes.POINTER(ctypes.c_size_t)

_SIGS = {
    "infllmv2_compress_k": [_P, _P, _P, _I32, _I32, _I64, _I32, _I32, _I32, _I32, _P, _P, _I32,
                            _I64, _P, _P],
    "infllmv2_select_blocks": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I64,
                               _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                               _I32, _I32, _I32, _I32, _F, _P, _SZP, _P, _P],
    "infllmv2_select_blocks_unfused": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64,
                                       _I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                       _I32, _I32, _I32, _I32, _I32, _I32, _F, _P, _SZP, _P, _P],
    "infllmv2_sparse_attn": [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I64, _I32, _I32,
                             _I32, _I32, _P, _I32, _I32, _I32, _F, _I64, _P, _P, _P, _SZP, _P],
    "infllmv2_sparse_attn_noalloc": [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I64, _I32,
                                     _I32, _I32, _I32, _P, _I32, _I32, _I32, _F, _I64, _P, _P, _P],
    "infllmv2_dense_attn": [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I64, _I32, _I32,
                            _I32, _F, _I64, _P, _P, _P, _SZP, _P],
    "infllmv2_sparse_attn_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64,
                                 _I64, _I32, _I32, _I32, _I32, _P, _I32, _I32, _I32, _F, _P, _P,
                                 _P, _P, _SZP, _P],
}


class InfLLMv2Error(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load the library (once).  Fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise InfLLMv2Error(f"{_LIB_PATH} is missing: build it first (python "
                                "trainable_block_sparse_compress_amd/build.py)")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        for name in ("infllmv2_strerror",):
            getattr(lib, name).argtypes = [ctypes.c_int]
            getattr(lib, name).restype = ctypes.c_char_p
        for name in ("infllmv2_last_error", "infllmv2_version"):
            getattr(lib, name).argtypes = []
            getattr(lib, name).restype = ctypes.c_char_p
        _lib = lib
    return _lib


def version() -> str:
    return load().infllmv2_version().decode()


def _check(rc: int):
    if rc != 0:
        lib = load()
        raise InfLLMv2Error(f"{lib.infllmv2_strerror(rc).decode()} ({rc}): "
                            f"{lib.infllmv2_last_error().decode()}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise InfLLMv2Error("tensors passed to the library must be on the GPU")
    if not t.is_contiguous():
        raise InfLLMv2Error("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _i32(t, name):
    if t is not None and t.dtype != torch.int32:
        raise InfLLMv2Error(f"{name} must be int32")
    return _ptr(t)


def _bf16(t, name):
    if t is not None and t.dtype != torch.bfloat16:
        raise InfLLMv2Error(f"{name} must be bfloat16")
    return _ptr(t)


def _shape(t, name, shape, dtype=None):
    """A tensor argument must have exactly ``shape`` (and ``dtype``)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise InfLLMv2Error(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise InfLLMv2Error(f"{name} must be {dtype}")


def _meta(t, name, count):
    """Per-sequence metadata: int32 with at least ``count`` entries."""
    if t is None:
        return
    if t.dtype != torch.int32 or t.dim() != 1 or t.numel() < count:
        raise InfLLMv2Error(f"{name} must be a 1-D int32 tensor of at least {count} entries")


def _seq_meta(batch, cu_q, used_q, cu_k, used_k):
    _meta(cu_q, "cu_seqlens_q", batch + (0 if used_q is not None else 1))
    _meta(used_q, "seqused_q", batch)
    _meta(cu_k, "cu_seqlens_k", batch + (0 if used_k is not None else 1))
    _meta(used_k, "seqused_k", batch)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ws(workspace):
    """(pointer, size pointer) for a caller workspace.  Without one, both are
    NULL: a NULL workspace with a non-NULL size pointer would be a size query."""
    if workspace is None:
        return None, None
    return _ptr(workspace), ctypes.byref(ctypes.c_size_t(workspace.numel() * workspace.element_size()))


def compress_k(k, cu_seqlens_k, seqused_k, batch, max_seqlen_k, kernel_size, stride, cu_cmp,
               k_cmp, cmp_begin=None, max_new=0):
    """k [rows_k, h_kv, d] bf16 -> k_cmp [h_kv, c_rows, d] bf16 (in place)."""
    rows_k, h_kv, d = k.shape
    _shape(k_cmp, "k_cmp", (h_kv, k_cmp.shape[1], d))
    _meta(cu_seqlens_k, "cu_seqlens_k", batch + (0 if seqused_k is not None else 1))
    _meta(seqused_k, "seqused_k", batch)
    _meta(cu_cmp, "cu_cmp", batch)
    _meta(cmp_begin, "cmp_begin", batch)
    _check(load().infllmv2_compress_k(
        _bf16(k, "k"), _i32(cu_seqlens_k, "cu_seqlens_k"), _i32(seqused_k, "seqused_k"), batch,
        max_seqlen_k, rows_k, h_kv, d, kernel_size, stride, _i32(cu_cmp, "cu_cmp"),
        _i32(cmp_begin, "cmp_begin"), max_new, k_cmp.shape[1], _bf16(k_cmp, "k_cmp"), _stream()))


def select_blocks_workspace(rows_q, h_q, h_kv, max_seqlen_q, max_seqlen_k, n_init, n_local,
                            n_topk, approx=False, batch=1, unfused=False) -> int:
    size = ctypes.c_size_t(0)
    fn = load().infllmv2_select_blocks_unfused if unfused else load().infllmv2_select_blocks
    _check(fn(
        None, None, _P(1) if approx else None, None, None, None, None, None, None, batch,
        max_seqlen_q, max_seqlen_k, rows_q, 0, 0, h_q, h_kv, 128, 64, n_init, n_local, n_topk,
        32, 16, 128, 64, 5, 4, 1, 1.0, None, ctypes.byref(size), None, None))
    return size.value


def select_blocks(q, k_c1, k_c2, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k, cu_c1, cu_c2,
                  batch, max_seqlen_q, max_seqlen_k, n_init, n_local, n_topk, softmax_scale,
                  block_idx, workspace, block_size=64, c1=(32, 16), c2=(128, 64), pool=(5, 4, 1),
                  _entry="infllmv2_select_blocks"):
    """Writes block_idx [h_kv, rows_q, n_init + n_local + n_topk] int32."""
    rows_q, h_q, d = q.shape
    h_kv, c1_rows, _ = k_c1.shape
    c2_rows = k_c2.shape[1] if k_c2 is not None else 0
    _shape(k_c1, "k_c1", (h_kv, c1_rows, d))
    _shape(k_c2, "k_c2", (h_kv, c2_rows, d))
    _shape(block_idx, "block_idx", (h_kv, rows_q, n_init + n_local + n_topk), torch.int32)
    _seq_meta(batch, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k)
    _meta(cu_c1, "cu_c1", batch)
    _meta(cu_c2, "cu_c2", batch if k_c2 is not None else 0)
    ws, ws_bytes = _ws(workspace)
    _check(getattr(load(), _entry)(
        _bf16(q, "q"), _bf16(k_c1, "k_c1"), _bf16(k_c2, "k_c2"), _i32(cu_seqlens_q, "cu_seqlens_q"),
        _i32(seqused_q, "seqused_q"), _i32(cu_seqlens_k, "cu_seqlens_k"),
        _i32(seqused_k, "seqused_k"), _i32(cu_c1, "cu_c1"), _i32(cu_c2, "cu_c2"), batch,
        max_seqlen_q, max_seqlen_k, rows_q, c1_rows, c2_rows, h_q, h_kv, d, block_size, n_init,
        n_local, n_topk, c1[0], c1[1], c2[0], c2[1], pool[0], pool[1], pool[2], softmax_scale,
        ws, ws_bytes, _i32(block_idx, "block_idx"), _stream()))


def select_blocks_unfused(*args, **kw):
    """select_blocks through infllmv2_select_blocks_unfused (the unfused
    group-sum baseline; its workspace size comes from
    select_blocks_workspace(..., unfused=True))."""
    return select_blocks(*args, **kw, _entry="infllmv2_select_blocks_unfused")


def attn_workspace(h_q, h_kv, batch, max_seqlen_q, max_seqlen_k, rows_q, v_seq_stride=0,
                   n_sel=0, n_init=0, n_local=0) -> int:
    """Workspace bytes of sparse_attn (n_sel > 0) or dense_attn (n_sel == 0)
    for these sizes: the V transposition (v_seq_stride == 0) and, for
    launches with few query tiles, the split-K partials."""
    size = ctypes.c_size_t(0)
    if n_sel > 0:
        _check(load().infllmv2_sparse_attn(
            None, None, None, None, None, None, None, batch, max_seqlen_q, max_seqlen_k, rows_q, 0,
            h_q, h_kv, 128, 64, None, n_sel, n_init, n_local, 1.0, v_seq_stride, None, None, None,
            ctypes.byref(size), None))
    else:
        _check(load().infllmv2_dense_attn(
            None, None, None, None, None, None, None, batch, max_seqlen_q, max_seqlen_k, rows_q, 0,
            h_q, h_kv, 128, 1.0, v_seq_stride, None, None, None, ctypes.byref(size), None))
    return size.value


def _attn_shapes(q, k, v, out, lse, v_seq_stride, batch):
    rows_q, h_q, d = q.shape
    rows_k, h_kv, _ = k.shape
    _shape(k, "k", (rows_k, h_kv, d))
    _shape(out, "out", (rows_q, h_q, d))
    _shape(lse, "lse", (h_q, rows_q), torch.float32)
    if v_seq_stride == 0:
        _shape(v, "v", (rows_k, h_kv, d))
    else:
        _shape(v, "v (transposed)", (h_kv, d, batch, v_seq_stride))


def sparse_attn(q, k, v, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k, batch, max_seqlen_q,
                max_seqlen_k, block_idx, n_init, n_local, softmax_scale, out, lse=None,
                workspace=None, v_seq_stride=0, block_size=64):
    rows_q, h_q, d = q.shape
    rows_k, h_kv, _ = k.shape
    n_sel = block_idx.shape[-1]
    _attn_shapes(q, k, v, out, lse, v_seq_stride, batch)
    _shape(block_idx, "block_idx", (h_kv, rows_q, n_sel), torch.int32)
    _seq_meta(batch, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k)
    ws, ws_bytes = _ws(workspace)
    _check(load().infllmv2_sparse_attn(
        _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), _i32(cu_seqlens_q, "cu_seqlens_q"),
        _i32(seqused_q, "seqused_q"), _i32(cu_seqlens_k, "cu_seqlens_k"),
        _i32(seqused_k, "seqused_k"), batch, max_seqlen_q, max_seqlen_k, rows_q, rows_k, h_q,
        h_kv, d, block_size, _i32(block_idx, "block_idx"), n_sel, n_init, n_local, softmax_scale,
        v_seq_stride, _bf16(out, "out"), _ptr(lse), ws, ws_bytes, _stream()))


def sparse_attn_noalloc(q, k, v, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k, batch,
                        max_seqlen_q, max_seqlen_k, block_idx, n_init, n_local, softmax_scale, out,
                        lse=None, v_seq_stride=0, block_size=64):
    """sparse_attn through infllmv2_sparse_attn_noalloc: no workspace, the
    library's static per-GPU scratch instead (at most 64 MiB)."""
    rows_q, h_q, d = q.shape
    rows_k, h_kv, _ = k.shape
    n_sel = block_idx.shape[-1]
    _attn_shapes(q, k, v, out, lse, v_seq_stride, batch)
    _shape(block_idx, "block_idx", (h_kv, rows_q, n_sel), torch.int32)
    _seq_meta(batch, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k)
    _check(load().infllmv2_sparse_attn_noalloc(
        _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), _i32(cu_seqlens_q, "cu_seqlens_q"),
        _i32(seqused_q, "seqused_q"), _i32(cu_seqlens_k, "cu_seqlens_k"),
        _i32(seqused_k, "seqused_k"), batch, max_seqlen_q, max_seqlen_k, rows_q, rows_k, h_q,
        h_kv, d, block_size, _i32(block_idx, "block_idx"), n_sel, n_init, n_local, softmax_scale,
        v_seq_stride, _bf16(out, "out"), _ptr(lse), _stream()))


def dense_attn(q, k, v, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k, batch, max_seqlen_q,
               max_seqlen_k, softmax_scale, out, lse=None, workspace=None, v_seq_stride=0):
    rows_q, h_q, d = q.shape
    rows_k, h_kv, _ = k.shape
    _attn_shapes(q, k, v, out, lse, v_seq_stride, batch)
    _seq_meta(batch, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k)
    ws, ws_bytes = _ws(workspace)
    _check(load().infllmv2_dense_attn(
        _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), _i32(cu_seqlens_q, "cu_seqlens_q"),
        _i32(seqused_q, "seqused_q"), _i32(cu_seqlens_k, "cu_seqlens_k"),
        _i32(seqused_k, "seqused_k"), batch, max_seqlen_q, max_seqlen_k, rows_q, rows_k, h_q,
        h_kv, d, softmax_scale, v_seq_stride, _bf16(out, "out"), _ptr(lse), ws, ws_bytes,
        _stream()))


def attn_bwd_workspace(h_q, h_kv, batch, max_seqlen_q, max_seqlen_k, rows_q, rows_k, n_sel=0,
                       n_init=0, n_local=0) -> int:
    """Workspace bytes of sparse_attn_bwd for these sizes (n_sel == 0: the
    dense backward)."""
    size = ctypes.c_size_t(0)
    _check(load().infllmv2_sparse_attn_bwd(
        None, None, None, None, None, None, None, None, None, None, batch, max_seqlen_q,
        max_seqlen_k, rows_q, rows_k, h_q, h_kv, 128, 64, _P(1) if n_sel > 0 else None, n_sel,
        n_init, n_local, 1.0, None, None, None, None, ctypes.byref(size), None))
    return size.value


def sparse_attn_bwd(q, k, v, out, lse, dout, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k,
                    batch, max_seqlen_q, max_seqlen_k, block_idx, n_init, n_local, softmax_scale,
                    dq, dk, dv, workspace, block_size=64):
    """Gradients dq, dk, dv (bf16, written in place) of the sparse attention
    (block_idx given) or the dense causal attention (block_idx None), from the
    forward's out and lse and the upstream gradient dout."""
    rows_q, h_q, d = q.shape
    rows_k, h_kv, _ = k.shape
    n_sel = block_idx.shape[-1] if block_idx is not None else 0
    if lse is None:
        raise InfLLMv2Error("lse must be the forward's float32 [h_q, rows_q] LSE")
    _shape(lse, "lse", (h_q, rows_q), torch.float32)
    for name, t in (("out", out), ("dout", dout), ("dq", dq)):
        _shape(t, name, (rows_q, h_q, d))
    for name, t in (("v", v), ("dk", dk), ("dv", dv)):
        _shape(t, name, (rows_k, h_kv, d))
    _shape(block_idx, "block_idx", (h_kv, rows_q, n_sel), torch.int32)
    _seq_meta(batch, cu_seqlens_q, seqused_q, cu_seqlens_k, seqused_k)
    ws, ws_bytes = _ws(workspace)
    _check(load().infllmv2_sparse_attn_bwd(
        _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), _bf16(out, "out"), _ptr(lse),
        _bf16(dout, "dout"), _i32(cu_seqlens_q, "cu_seqlens_q"), _i32(seqused_q, "seqused_q"),
        _i32(cu_seqlens_k, "cu_seqlens_k"), _i32(seqused_k, "seqused_k"), batch, max_seqlen_q,
        max_seqlen_k, rows_q, rows_k, h_q, h_kv, d, block_size, _i32(block_idx, "block_idx"),
        n_sel, n_init, n_local, softmax_scale, _bf16(dq, "dq"), _bf16(dk, "dk"), _bf16(dv, "dv"),
        ws, ws_bytes, _stream()))

"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, validates arguments before any HIP call and answers
workspace-size queries without touching a GPU.  No compute call is made."""
import ctypes
import os
import re

import pytest

from trainable_block_sparse_compress_amd import binding as B
from trainable_block_sparse_compress_amd import pipeline as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "infllmv2.h")

OK, EINVAL, EUNSUP, EWS = 0, -1, -2, -3
# floats of one split-K partial: O[16][128], l[16], m[16]
PART_FLOATS = 16 * 128 + 32


def align(x):
    return (x + 255) // 256 * 256


@pytest.fixture(scope="module")
def lib():
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(infllmv2_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("infllmv2_compress_k", "infllmv2_select_blocks", "infllmv2_sparse_attn",
              "infllmv2_dense_attn"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror_and_version(lib):
    assert B.version().startswith("infllmv2-gfx950")
    for code in (OK, EINVAL, EUNSUP, EWS, -4):
        assert lib.infllmv2_strerror(code)
    assert lib.infllmv2_strerror(7) == b"unknown error"


def _select(lib, **kw):
    a = dict(q=None, k_c1=None, k_c2=None, cu_q=None, used_q=None, cu_k=None, used_k=None,
             cu_c1=None, cu_c2=None, batch=1, max_q=4096, max_k=4096, rows_q=4096, c1_rows=255,
             c2_rows=0, h_q=32, h_kv=2, d=128, B=64, n_init=1, n_local=32, n_topk=63, c1k=32,
             c1s=16, c2k=128, c2s=64, pk=5, ps=4, pp=1, scale=0.088, ws=None, query=True, idx=None)
    a.update(kw)
    size = ctypes.c_size_t(0)
    rc = lib.infllmv2_select_blocks(
        a["q"], a["k_c1"], a["k_c2"], a["cu_q"], a["used_q"], a["cu_k"], a["used_k"], a["cu_c1"],
        a["cu_c2"], a["batch"], a["max_q"], a["max_k"], a["rows_q"], a["c1_rows"], a["c2_rows"],
        a["h_q"], a["h_kv"], a["d"], a["B"], a["n_init"], a["n_local"], a["n_topk"], a["c1k"],
        a["c1s"], a["c2k"], a["c2s"], a["pk"], a["ps"], a["pp"], a["scale"], a["ws"],
        ctypes.byref(size) if a["query"] else None, a["idx"], None)
    return rc, size.value


@pytest.mark.parametrize("kw,code", [
    (dict(d=64), EUNSUP),
    (dict(B=128), EUNSUP),
    (dict(h_q=31), EINVAL),
    (dict(h_q=64, h_kv=2), EUNSUP),           # G = 32
    (dict(c1k=64), EUNSUP),
    (dict(pp=0), EUNSUP),
    (dict(n_init=0, n_local=0, n_topk=0), EINVAL),
    (dict(n_topk=-1), EINVAL),
    (dict(scale=0.0), EINVAL),
    (dict(scale=float("nan")), EINVAL),
    (dict(batch=-1), EINVAL),
    (dict(max_q=5000), EINVAL),               # queries longer than keys
    (dict(max_k=64 * 8193, max_q=64), EUNSUP),  # more than 8192 blocks
    (dict(k_c2=ctypes.c_void_p(16), n_init=1, n_local=0, n_topk=0), EINVAL),  # approx, |I|*64 < 128
    (dict(k_c2=ctypes.c_void_p(16), c2k=256), EUNSUP),
])
def test_select_blocks_validation(lib, kw, code):
    rc, _ = _select(lib, **kw)
    assert rc == code
    assert lib.infllmv2_last_error()


def test_select_blocks_workspace_size(lib):
    rows, h_q, h_kv, n = 131072, 32, 2, 131072
    rc, size = _select(lib, max_q=n, max_k=n, rows_q=rows, h_q=h_q, h_kv=h_kv)
    assert rc == OK
    lse = h_q * rows * 4
    bs_ld = ((n // 64 + 3) // 4) * 4
    bs = h_kv * rows * bs_ld * 4
    assert size == align(lse) + align(bs)


def test_select_blocks_missing_workspace(lib):
    rc, _ = _select(lib, query=False, q=ctypes.c_void_p(16))
    assert rc == EWS


def test_attention_validation_and_workspace(lib):
    size = ctypes.c_size_t(0)
    rc = lib.infllmv2_dense_attn(None, None, None, None, None, None, None, 2, 100, 100, 200, 200,
                                 32, 2, 128, 0.088, 0, None, None, None, ctypes.byref(size), None)
    assert rc == OK and size.value == 2 * 128 * 2 * 128 * 2
    rc = lib.infllmv2_dense_attn(None, None, None, None, None, None, None, 1, 10, 10, 10, 10,
                                 32, 2, 96, 0.088, 0, None, None, None, ctypes.byref(size), None)
    assert rc == EUNSUP
    rc = lib.infllmv2_dense_attn(None, None, None, None, None, None, None, 1, 10, 10, 10, 10,
                                 32, 2, 128, 0.088, 100, None, None, None, ctypes.byref(size), None)
    assert rc == EINVAL  # v_seq_stride not a multiple of 64
    # one tiny sequence: split-K partials only (V given transposed), one split
    rc = lib.infllmv2_dense_attn(None, None, None, None, None, None, None, 1, 10, 10, 10, 10,
                                 32, 2, 128, 0.088, 64, None, None, None, ctypes.byref(size), None)
    assert rc == OK and size.value == align(10 * 2 * 1 * PART_FLOATS * 4)
    # decode-like: 16 sequences x 1 query over 128K keys, 96 + 33 blocks -> 8 splits
    rc = lib.infllmv2_sparse_attn(None, None, None, None, None, None, None, 16, 1, 131072, 16, 0,
                                  32, 2, 128, 64, None, 96, 1, 32, 0.088, 131072, None, None, None,
                                  ctypes.byref(size), None)
    assert rc == OK and size.value == align(16 * 2 * 8 * PART_FLOATS * 4)
    # many query tiles: the tile kernel, no partials
    rc = lib.infllmv2_sparse_attn(None, None, None, None, None, None, None, 1, 131072, 131072,
                                  131072, 0, 32, 2, 128, 64, None, 96, 1, 32, 0.088, 131072, None,
                                  None, None, ctypes.byref(size), None)
    assert rc == OK and size.value == 0
    rc = lib.infllmv2_sparse_attn(None, None, None, None, None, None, None, 1, 10, 10, 10, 10,
                                  32, 2, 128, 64, None, 0, 1, 32, 0.088, 0, None, None, None,
                                  ctypes.byref(size), None)
    assert rc == EINVAL  # n_sel = 0
    rc = lib.infllmv2_sparse_attn(None, None, None, None, None, None, None, 1, 10, 10, 10, 10,
                                  32, 2, 128, 32, None, 96, 1, 32, 0.088, 0, None, None, None,
                                  ctypes.byref(size), None)
    assert rc == EUNSUP  # block size 32
    # transposed-V rows of batch x columns at the 2^27 limit (the kernel's
    # 32-bit offsets over 16 such rows) are refused; one column less is not
    for stride, code in ((1 << 20, EUNSUP), ((1 << 20) - 64, OK)):
        rc = lib.infllmv2_sparse_attn(None, None, None, None, None, None, None, 128, 1, 64, 128, 0,
                                      32, 2, 128, 64, None, 96, 1, 32, 0.088, stride, None, None,
                                      None, ctypes.byref(size), None)
        assert rc == code, (stride, rc)


def test_compress_validation(lib):
    rc = lib.infllmv2_compress_k(None, None, None, 1, 100, 100, 2, 64, 32, 16, None, None, 0, 10,
                                 None, None)
    assert rc == EUNSUP
    rc = lib.infllmv2_compress_k(None, None, None, 1, 100, 100, 2, 128, 0, 16, None, None, 0, 10,
                                 None, None)
    assert rc == EINVAL
    rc = lib.infllmv2_compress_k(None, None, None, 1, 100, 100, 2, 128, 32, 16, None,
                                 ctypes.c_void_p(16), 0, 10, None, None)
    assert rc == EINVAL  # cmp_begin without max_new
    rc = lib.infllmv2_compress_k(None, None, None, 1, 100, 100, 2, 128, 32, 16, None, None, 0, 10,
                                 None, None)
    assert rc == EINVAL  # null pointers with work to do
    rc = lib.infllmv2_compress_k(None, None, None, 1, 20, 20, 2, 128, 32, 16, None, None, 0, 0,
                                 None, None)
    assert rc == OK  # no complete window: nothing to do


def test_switch_partition_and_window_counts():
    import oracle.reference as R
    cfg = P.SparseConfig()
    for n in (0, 31, 32, 100, 4096, 131072):
        assert P.n_windows(n, *cfg.c1) == R.n_windows(n, 32, 16)
        assert P.n_windows(n, *cfg.c2) == R.n_windows(n, 128, 64)
    assert cfg.n_sel == 96


def test_no_workspace_is_not_a_size_query(lib):
    """A NULL workspace with a NULL size pointer must take the launch path
    (here: rejected for NULL tensors), never the size-query path."""
    # (enough query tiles for the tile kernel, V given transposed: no workspace needed)
    rc = lib.infllmv2_dense_attn(None, None, None, None, None, None, None, 1, 8192, 8192, 8192,
                                 8192, 32, 2, 128, 0.088, 8192, None, None, None, None, None)
    assert rc == EINVAL
    assert B._ws(None) == (None, None)


def _bwd(lib, **kw):
    a = dict(batch=1, max_q=4096, max_k=4096, rows_q=4096, rows_k=4096, h_q=32, h_kv=2, d=128,
             B=64, idx=None, n_sel=0, n_init=0, n_local=0, scale=0.088)
    a.update(kw)
    size = ctypes.c_size_t(0)
    rc = lib.infllmv2_sparse_attn_bwd(
        None, None, None, None, None, None, None, None, None, None, a["batch"], a["max_q"],
        a["max_k"], a["rows_q"], a["rows_k"], a["h_q"], a["h_kv"], a["d"], a["B"], a["idx"],
        a["n_sel"], a["n_init"], a["n_local"], a["scale"], None, None, None, None,
        ctypes.byref(size), None)
    return rc, size.value


def test_backward_workspace_layout(lib):
    """Workspace of the backward: statistics (2 x 64 B) and the re-laid-out
    Q, dO (2 x 4 KB) per (query row, group); 64 KB of fp32 dK / dV partial
    sums per work item; two 16-bit mask tables; per-block item counts and
    offsets; the work list."""
    rows, n, h_kv = 4096, 4096, 2
    for dense, n_sel, n_init, n_local in ((True, 0, 0, 0), (False, 63, 1, 32)):
        rc, size = _bwd(lib, idx=None if dense else ctypes.c_void_p(16), n_sel=n_sel,
                        n_init=n_init, n_local=n_local)
        assert rc == OK
        ntiles, nblk = n // 16, n // 64
        nb = h_kv * nblk
        per_row = nblk if dense else min(nblk, n_sel + n_init + n_local)
        wmax = -(-h_kv * rows * per_row // 1024) + nb + 1
        want = (2 * align(rows * h_kv * 16 * 4) + 2 * align(rows * h_kv * 128 * 16 * 2)
                + align(wmax * 16384 * 4) + 2 * align(nb * ntiles * 2) + 2 * align(nb * 4)
                + align(wmax * 8) + align(4))
        assert size == want, (dense, size, want)


@pytest.mark.parametrize("kw,code", [
    (dict(max_k=64 * 8193, max_q=64, rows_k=64 * 8193), EUNSUP),   # > 8192 blocks
    (dict(d=64), EUNSUP),
    (dict(B=32), EUNSUP),
    (dict(h_q=24, h_kv=2), EUNSUP),         # G = 12
    (dict(h_q=31), EINVAL),
    (dict(scale=0.0), EINVAL),
    (dict(idx=ctypes.c_void_p(16), n_sel=0), EINVAL),
    (dict(max_q=5000), EINVAL),
])
def test_backward_validation(lib, kw, code):
    rc, _ = _bwd(lib, **kw)
    assert rc == code
    assert lib.infllmv2_last_error()


def test_binding_rejects_mismatched_shapes():
    """The Python binding checks every tensor's shape and dtype against the
    sizes it passes to the C ABI before any pointer is taken (so this runs
    on CPU tensors): a mismatch raises instead of reaching the kernels."""
    import torch

    from trainable_block_sparse_compress_amd import binding as B
    bf, i32 = torch.bfloat16, torch.int32
    q = torch.zeros((100, 4, 128), dtype=bf)
    k = torch.zeros((100, 2, 128), dtype=bf)
    cu = torch.zeros(2, dtype=i32)
    idx = torch.zeros((2, 100, 8), dtype=i32)
    bad = [
        dict(out=torch.zeros((99, 4, 128), dtype=bf)),
        dict(lse=torch.zeros((4, 99), dtype=torch.float32)),
        dict(lse=torch.zeros((4, 100), dtype=torch.float16)),
        dict(v=torch.zeros((100, 1, 128), dtype=bf)),
        dict(v=torch.zeros((2, 128, 1, 64), dtype=bf), v_seq_stride=128),
        dict(block_idx=torch.zeros((2, 99, 8), dtype=i32)),
        dict(block_idx=torch.zeros((2, 100, 8), dtype=torch.int64)),
        dict(cu_seqlens_q=torch.zeros(1, dtype=i32)),
    ]
    for kw in bad:
        a = dict(q=q, k=k, v=k, cu_seqlens_q=cu, seqused_q=None, cu_seqlens_k=cu, seqused_k=None,
                 batch=1, max_seqlen_q=100, max_seqlen_k=100, block_idx=idx, n_init=1, n_local=2,
                 softmax_scale=0.1, out=torch.zeros_like(q), lse=None)
        a.update(kw)
        with pytest.raises(B.InfLLMv2Error):
            B.sparse_attn(**a)
    kc = torch.zeros((2, 5, 128), dtype=bf)
    with pytest.raises(B.InfLLMv2Error):
        B.select_blocks(q, kc, None, cu, None, cu, None, torch.zeros(1, dtype=i32), None, 1, 100, 100,
                        1, 2, 5, 0.1, torch.zeros((2, 100, 7), dtype=i32), None)
    with pytest.raises(B.InfLLMv2Error):
        B.compress_k(k, cu, None, 1, 100, 32, 16, torch.zeros(1, dtype=i32),
                     torch.zeros((2, 5, 64), dtype=bf))
    with pytest.raises(B.InfLLMv2Error):
        B.sparse_attn_bwd(q, k, k, q, torch.zeros((4, 100)), q, cu, None, cu, None, 1, 100, 100, idx,
                          1, 2, 0.1, q, k, torch.zeros((100, 2, 64), dtype=bf), None)


def test_noalloc_attention_rejects_scratch_above_its_maximum(lib):
    """infllmv2_sparse_attn_noalloc refuses, before any HIP call, a call
    whose scratch (here the transposed V of 200000 keys x 2 KV heads, 97.7 MB)
    exceeds its 64 MiB static array; without a GPU, a call that fits goes on
    to the pointer checks (EINVAL for the NULL tensors)."""
    fn = lib.infllmv2_sparse_attn_noalloc
    args = [None] * 7
    rc = fn(*args, 1, 200000, 200000, 200000, 200000, 32, 2, 128, 64, None, 8, 1, 2, 0.1, 0, None, None, None)
    assert rc == EUNSUP and b"static maximum" in lib.infllmv2_last_error()
    rc = fn(*args, 1, 1000, 1000, 1000, 1000, 32, 2, 128, 64, None, 8, 1, 2, 0.1, 0, None, None, None)
    assert rc == EINVAL

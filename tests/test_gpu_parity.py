"""Parity of the HIP path (called through the C ABI) with the fp64 oracle.

Bars: compressed keys bit-exact; block selection per the acceptance rule
(exact match except inside the 1e-3 relative tie band around the k-th
score); attention max-abs <= 2e-2 and relative RMS <= 1e-2 on bf16 outputs.
Inputs come from the seeded generator; both sides see the same bf16 values.
"""
import math

import numpy as np
import pytest
import torch

import oracle.reference as R
from trainable_block_sparse_compress_amd import binding as B
from trainable_block_sparse_compress_amd import datagen as D
from trainable_block_sparse_compress_amd import pipeline as P
from tests.gpu_util import f64_to_bits, i32, say, to_bits, to_dev, to_f64
from tests.helpers import (ATT_MAX_ABS, ATT_REL_RMS, attn_errors, check_block_scores, check_selection,
                           extreme_inputs, sample_positions)

pytestmark = pytest.mark.gpu


def _starts(lengths):
    st = [0]
    for n in lengths[:-1]:
        st.append(st[-1] + n)
    return st


def _cfg(p: R.Params, **kw):
    return P.SparseConfig(n_init=p.n_init, n_local=p.n_local, n_topk=p.n_topk,
                          lse_mode=p.lse_mode, **kw)


# ----------------------------------------------------------------------------
# compress_k
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("lengths,h_kv,kl", [
    ([4096], 1, (32, 16)),
    ([3000, 77, 31, 1000], 2, (32, 16)),
    ([3000, 77, 130, 1000], 2, (128, 64)),
    ([131072], 2, (32, 16)),
])
def test_compress_bit_exact(lib, lengths, h_kv, kl):
    say(f"compress_k lengths={lengths} h_kv={h_kv} kernel/stride={kl}")
    inp = D.make_prefill(21, lengths, h_q=h_kv, h_kv=h_kv)
    k = to_dev(inp.k)
    nw = [P.n_windows(n, *kl) for n in lengths]
    offs = _starts(nw)
    kc = torch.zeros((h_kv, max(1, sum(nw)), 128), dtype=torch.bfloat16, device="cuda")
    B.compress_k(k, i32(_starts(lengths)), i32(lengths), len(lengths), max(lengths), kl[0], kl[1],
                 i32(offs), kc)
    torch.cuda.synchronize()
    got = to_bits(kc)
    st = _starts(lengths)
    for s, n in enumerate(lengths):
        ref = R.compress_keys(inp.k[st[s]:st[s] + n], kl[0], kl[1], round_bf16=True)
        assert np.array_equal(got[:, offs[s]:offs[s] + nw[s]], f64_to_bits(ref)), f"sequence {s}"


def test_compress_incremental(lib):
    """Decode-style updates: windows completed by each new token are appended
    in place and equal a full compression of the final cache."""
    say("compress_k incremental")
    cap, h_kv, lens0 = 1024, 2, [700, 129, 31]
    inp = D.make_prefill(22, [cap] * 3, h_q=h_kv, h_kv=h_kv)
    k = to_dev(inp.k)
    cap1 = P.n_windows(cap, 32, 16)
    kc = torch.zeros((h_kv, 3 * cap1, 128), dtype=torch.bfloat16, device="cuda")
    cu_k, cu_c = i32([0, cap, 2 * cap]), i32([0, cap1, 2 * cap1])
    lens = list(lens0)
    B.compress_k(k, cu_k, i32(lens), 3, max(lens), 32, 16, cu_c, kc)
    for _ in range(40):
        begin = [P.n_windows(n, 32, 16) for n in lens]
        lens = [n + 1 for n in lens]
        B.compress_k(k, cu_k, i32(lens), 3, max(lens), 32, 16, cu_c, kc, cmp_begin=i32(begin),
                     max_new=1)
    torch.cuda.synchronize()
    got = to_bits(kc)
    for s, n in enumerate(lens):
        ref = R.compress_keys(inp.k[s * cap:s * cap + n], 32, 16, round_bf16=True)
        N = ref.shape[1]
        assert np.array_equal(got[:, s * cap1:s * cap1 + N], f64_to_bits(ref))


# ----------------------------------------------------------------------------
# dense attention
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("lengths,h_q,h_kv", [
    ([1, 64, 65, 200, 1000], 32, 2),
    ([777, 300], 2, 1),
    ([513], 8, 1),
])
def test_dense_attention(lib, lengths, h_q, h_kv):
    say(f"dense_attn lengths={lengths} h_q={h_q} h_kv={h_kv}")
    inp = D.make_prefill(23, lengths, h_q, h_kv)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    st = _starts(lengths)
    cfg = P.SparseConfig()
    out = torch.empty_like(q)
    lse = torch.empty((h_q, q.shape[0]), dtype=torch.float32, device="cuda")
    P.DensePlan(st, lengths, st, lengths, sum(lengths), h_q, h_kv, cfg).run(q, k, v, out, lse)
    torch.cuda.synchronize()
    of, lf = to_f64(out), lse.cpu().numpy()
    G, scale = h_q // h_kv, 1 / math.sqrt(128)
    worst = 0.0
    for s, n in enumerate(lengths):
        Qs, Ks, Vs = R.as_f64(inp.q[st[s]:st[s] + n]), R.as_f64(inp.k[st[s]:st[s] + n]), R.as_f64(inp.v[st[s]:st[s] + n])
        ref = R.dense_prefill(Qs, Ks, Vs, G, scale)
        o_ref = np.stack([ref[t][0] for t in range(n)])
        l_ref = np.stack([ref[t][1] for t in range(n)])
        ma, rr = attn_errors(of[st[s]:st[s] + n], o_ref)
        worst = max(worst, ma)
        assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS, (s, ma, rr)
        assert np.abs(lf[:, st[s]:st[s] + n].T - l_ref).max() < 1e-3
    say(f"  max abs err {worst:.3e}")


@pytest.mark.parametrize("lengths", [[32768], [8192] * 3 + [777]])
def test_dense_attention_long(lib, lengths):
    """Dense causal attention of the 32q/2kv layer over one 32K sequence
    (its tiles are spread over the XCDs in chunks, heaviest first) and over
    several 8K sequences plus a ragged one (contiguous ranges, heaviest
    first): sampled rows of every sequence, including the ends of tiles and
    of the launch order, against the oracle."""
    say(f"dense long lengths={lengths}")
    h_q, h_kv = 32, 2
    inp = D.make_prefill(29, lengths, h_q, h_kv)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    st = _starts(lengths)
    out = torch.empty_like(q)
    lse = torch.empty((h_q, q.shape[0]), dtype=torch.float32, device="cuda")
    P.DensePlan(st, lengths, st, lengths, sum(lengths), h_q, h_kv, P.SparseConfig()).run(q, k, v, out, lse)
    torch.cuda.synchronize()
    of, lf = to_f64(out), lse.cpu().numpy()
    worst = 0.0
    for s, n in enumerate(lengths):
        Ks, Vs = R.as_f64(inp.k[st[s]:st[s] + n]), R.as_f64(inp.v[st[s]:st[s] + n])
        pos = sample_positions(n, 40, seed=s, must=(15, 16, 511, 512, n - 17, n - 16))
        ref = R.dense_prefill(inp.q[st[s]:st[s] + n], Ks, Vs, h_q // h_kv, 1 / math.sqrt(128), positions=pos)
        for t in pos:
            ma, rr = attn_errors(of[st[s] + t], ref[t][0])
            worst = max(worst, ma)
            assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS, (s, t, ma, rr)
            assert np.abs(lf[:, st[s] + t] - ref[t][1]).max() < 1e-3, (s, t)
    say(f"  max abs err {worst:.3e}")


@pytest.mark.parametrize("lengths,stride", [([5000, 3000], 131072 + 64), ([131072 + 2048 + 37], 0)])
def test_dense_attention_multi_window(lib, lengths, stride):
    """The dense instance that walks the keys in windows of 2048 blocks, taken
    when the transposed V's rows are longer than 131072 columns: short
    sequences with V passed transposed at a longer stride (one window each),
    and one sequence past 128K keys (two windows).  Sampled rows, including
    both sides of the window boundary, against the oracle."""
    say(f"dense multi-window lengths={lengths} stride={stride}")
    h_q, h_kv = 32, 2
    inp = D.make_prefill(31, lengths, h_q, h_kv)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    st = _starts(lengths)
    out = torch.empty_like(q)
    lse = torch.empty((h_q, q.shape[0]), dtype=torch.float32, device="cuda")
    if stride:
        vt = torch.zeros((h_kv, 128, len(lengths), stride), dtype=torch.bfloat16, device="cuda")
        for s, n in enumerate(lengths):
            vt[:, :, s, :n] = v[st[s]:st[s] + n].permute(1, 2, 0)
        cu = torch.tensor(st + [sum(lengths)], dtype=torch.int32, device="cuda")
        B.dense_attn(q, k, vt, cu, None, cu, None, len(lengths), max(lengths), max(lengths),
                     1 / math.sqrt(128), out, lse, v_seq_stride=stride)
    else:
        P.DensePlan(st, lengths, st, lengths, sum(lengths), h_q, h_kv, P.SparseConfig()).run(q, k, v, out, lse)
    torch.cuda.synchronize()
    of, lf = to_f64(out), lse.cpu().numpy()
    worst = 0.0
    for s, n in enumerate(lengths):
        Ks, Vs = R.as_f64(inp.k[st[s]:st[s] + n]), R.as_f64(inp.v[st[s]:st[s] + n])
        must = (15, 16, n - 1) if n <= 131072 else (131071, 131072, 131072 + 100, n - 1)
        pos = sample_positions(n, 16 if n <= 131072 else 3, seed=40 + s, must=must)
        ref = R.dense_prefill(inp.q[st[s]:st[s] + n], Ks, Vs, h_q // h_kv, 1 / math.sqrt(128), positions=pos)
        for t in pos:
            ma, rr = attn_errors(of[st[s] + t], ref[t][0])
            worst = max(worst, ma)
            assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS, (s, t, ma, rr)
            assert np.abs(lf[:, st[s] + t] - ref[t][1]).max() < 1e-3, (s, t)
    say(f"  max abs err {worst:.3e}")


# ----------------------------------------------------------------------------
# sparse attention on given block lists (selection noise excluded)
# ----------------------------------------------------------------------------

def _random_lists(lengths, h_kv, p: R.Params, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = sum(lengths)
    idx = np.full((h_kv, rows, p.n_sel), -1, dtype=np.int32)
    lists = {}
    st = _starts(lengths)
    for s, n in enumerate(lengths):
        for t in range(n):
            bt = t // 64
            for g in range(h_kv):
                fixed = set(range(min(p.n_init, bt + 1))) | set(range(max(0, bt - p.n_local + 1), bt + 1))
                rest = [b for b in range(bt + 1) if b not in fixed]
                kk = min(len(rest), p.n_topk)
                pick = set(rng.choice(rest, size=kk, replace=False).tolist()) if kk else set()
                bl = sorted(fixed | pick)
                idx[g, st[s] + t, :len(bl)] = bl
                lists[(s, t, g)] = bl
    return idx, lists


@pytest.mark.parametrize("lengths,h_q,h_kv,sel", [
    ([4096], 2, 1, (1, 4, 11)),
    ([3000, 700], 32, 2, (1, 4, 11)),
    ([2500], 32, 2, (0, 0, 9)),       # generic lists: the query's own block may or may not appear
    ([1000, 37], 16, 2, (2, 3, 5)),
    ([1700], 8, 2, (1, 2, 6)),        # G = 4
])
def test_sparse_attention_given_lists(lib, lengths, h_q, h_kv, sel):
    say(f"sparse_attn lists lengths={lengths} h_q={h_q} h_kv={h_kv} sel={sel}")
    p = R.Params(n_init=sel[0], n_local=sel[1], n_topk=sel[2])
    inp = D.make_prefill(24, lengths, h_q, h_kv)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    idx_np, lists = _random_lists(lengths, h_kv, p, seed=5)
    idx = torch.from_numpy(idx_np).cuda()
    st = _starts(lengths)
    out = torch.empty_like(q)
    lse = torch.empty((h_q, q.shape[0]), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, B.attn_workspace(h_q, h_kv, len(lengths), max(lengths), max(lengths),
                                             sum(lengths), n_sel=idx.shape[-1], n_init=p.n_init,
                                             n_local=p.n_local)),
                     dtype=torch.uint8, device="cuda")
    B.sparse_attn(q, k, v, i32(st), i32(lengths), i32(st), i32(lengths), len(lengths),
                  max(lengths), max(lengths), idx, p.n_init, p.n_local, 1 / math.sqrt(128), out,
                  lse, ws)
    torch.cuda.synchronize()
    of, lf = to_f64(out), lse.cpu().numpy()
    G = h_q // h_kv
    worst = 0.0
    for s, n in enumerate(lengths):
        Ks, Vs = R.as_f64(inp.k[st[s]:st[s] + n]), R.as_f64(inp.v[st[s]:st[s] + n])
        pos = range(n) if n * h_q <= 8192 * 8 else sample_positions(n, 160, seed=s)
        for t in pos:
            o_ref, l_ref = R.attend_token(inp.q[st[s] + t], t, Ks, Vs,
                                          [lists[(s, t, g)] for g in range(h_kv)], G, p)
            ma, rr = attn_errors(of[st[s] + t], o_ref)
            worst = max(worst, ma)
            assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS, (s, t, ma, rr)
            assert np.abs(lf[:, st[s] + t] - l_ref).max() < 1e-3, (s, t)
    say(f"  max abs err {worst:.3e}")


@pytest.mark.parametrize("h_q,h_kv", [(32, 2), (8, 1)])
def test_split_path_short_queries(lib, h_q, h_kv):
    """Few query tiles (decode-like: 5, 1 and 3 queries at the end of 3000,
    4100 and 700 keys) take the split-K kernels.  Lists carry repeats, -1
    pads and blocks after the query's own, in scrambled order; both the
    sparse and the dense entry point are checked against the oracle."""
    say(f"split path h_q={h_q} h_kv={h_kv}")
    klens, qlens = [3000, 4100, 700], [5, 1, 3]
    inp = D.make_prefill(31, klens, h_q, h_kv)
    kst = _starts(klens)
    qrows = [kst[s] + klens[s] - qlens[s] + i for s in range(3) for i in range(qlens[s])]
    qst = _starts(qlens)
    q = to_dev(np.ascontiguousarray(inp.q[qrows]))
    k, v = to_dev(inp.k), to_dev(inp.v)
    rng = np.random.Generator(np.random.PCG64(7))
    n_sel = 40
    idx = np.full((h_kv, len(qrows), n_sel), -1, dtype=np.int32)
    want = {}
    for s in range(3):
        for i in range(qlens[s]):
            t = klens[s] - qlens[s] + i
            bt = t // 64
            for g in range(h_kv):
                pick = rng.choice(bt + 1, size=min(bt + 1, 20), replace=False).tolist()
                extra = pick[:5] + [-1, -1, bt + 1 + int(rng.integers(0, 3))]
                entries = pick + extra
                rng.shuffle(entries)
                idx[g, qst[s] + i, :len(entries)] = entries
                want[(s, i, g)] = sorted(set(b for b in pick if 0 <= b <= bt))
    idx_t = torch.from_numpy(idx).cuda()
    scale = 1 / math.sqrt(128)
    args = (i32(qst), i32(qlens), i32(kst), i32(klens), 3, max(qlens), max(klens))
    for dense in (False, True):
        ws_bytes = B.attn_workspace(h_q, h_kv, 3, max(qlens), max(klens), len(qrows),
                                    n_sel=0 if dense else n_sel)
        ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda")
        out = torch.full_like(q, float("nan"))
        lse = torch.empty((h_q, len(qrows)), dtype=torch.float32, device="cuda")
        if dense:
            B.dense_attn(q, k, v, *args, scale, out, lse, ws)
        else:
            B.sparse_attn(q, k, v, *args, idx_t, 0, 0, scale, out, lse, ws)
        torch.cuda.synchronize()
        of, lf = to_f64(out), lse.cpu().numpy()
        p = R.Params()
        for s in range(3):
            Ks = R.as_f64(inp.k[kst[s]:kst[s] + klens[s]])
            Vs = R.as_f64(inp.v[kst[s]:kst[s] + klens[s]])
            for i in range(qlens[s]):
                t = klens[s] - qlens[s] + i
                qv = inp.q[kst[s] + t]
                if dense:
                    o_ref, l_ref = R.dense_token(qv, t, Ks, Vs, h_q // h_kv, scale)
                else:
                    o_ref, l_ref = R.attend_token(qv, t, Ks, Vs, [want[(s, i, g)] for g in range(h_kv)],
                                                  h_q // h_kv, p)
                ma, rr = attn_errors(of[qst[s] + i], o_ref)
                assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS, (dense, s, i, ma, rr)
                assert np.abs(lf[:, qst[s] + i] - l_ref).max() < 1e-3, (dense, s, i)


@pytest.mark.parametrize("klens,qlens", [
    ([40, 700], [50, 3]),          # few query tiles: the split-K kernels
    ([100, 3000], [300, 3000]),    # the tile kernel
])
def test_rows_before_first_key(lib, klens, qlens):
    """A sequence with more query rows than keys places its first rows
    before the first key (position t = len_k - len_q + i < 0): such a row
    attends no key, so the entry points give out = 0 and lse = -inf (the
    contract of infllmv2.h); the other rows match the oracle.  Sparse (local
    blocks only, empty lists) and dense, on both kernel paths."""
    h_q, h_kv = 32, 2
    say(f"rows before the first key klens={klens} qlens={qlens}")
    iq = D.make_prefill(41, qlens, h_q, h_kv)
    ik = D.make_prefill(42, klens, h_q, h_kv)
    q, k, v = to_dev(iq.q), to_dev(ik.k), to_dev(ik.v)
    qst, kst = _starts(qlens), _starts(klens)
    rows = sum(qlens)
    p = R.Params(n_init=0, n_local=2, n_topk=1)
    idx = torch.full((h_kv, rows, 1), -1, dtype=torch.int32, device="cuda")
    scale = 1 / math.sqrt(128)
    args = (i32(qst), i32(qlens), i32(kst), i32(klens), 2, max(qlens), max(klens))
    for dense in (False, True):
        ws = torch.empty(max(1, B.attn_workspace(h_q, h_kv, 2, max(qlens), max(klens), rows,
                                                 n_sel=0 if dense else 1, n_init=0, n_local=2)),
                         dtype=torch.uint8, device="cuda")
        out = torch.full_like(q, float("nan"))
        lse = torch.full((h_q, rows), float("nan"), dtype=torch.float32, device="cuda")
        if dense:
            B.dense_attn(q, k, v, *args, scale, out, lse, ws)
        else:
            B.sparse_attn(q, k, v, *args, idx, 0, 2, scale, out, lse, ws)
        torch.cuda.synchronize()
        of, lf = to_f64(out), lse.cpu().numpy()
        n_empty = 0
        for s in range(2):
            Ks = R.as_f64(ik.k[kst[s]:kst[s] + klens[s]])
            Vs = R.as_f64(ik.v[kst[s]:kst[s] + klens[s]])
            rows_s = range(qlens[s]) if qlens[s] <= 64 else sample_positions(qlens[s], 96, seed=s)
            edge = {0, qlens[s] - klens[s] - 1, qlens[s] - klens[s]}   # the last row before / first after
            rows_s = sorted(set(rows_s) | {i for i in edge if 0 <= i < qlens[s]})
            for i in rows_s:
                t = klens[s] - qlens[s] + i
                r = qst[s] + i
                if t < 0:
                    n_empty += 1
                    assert np.all(of[r] == 0.0), (dense, s, i)
                    assert np.all(np.isneginf(lf[:, r])), (dense, s, i)
                    continue
                qv = iq.q[r]
                if dense:
                    o_ref, l_ref = R.dense_token(qv, t, Ks, Vs, h_q // h_kv, scale)
                else:
                    bt = t // 64
                    o_ref, l_ref = R.attend_token(qv, t, Ks, Vs, [[b for b in (bt - 1, bt) if b >= 0]] * h_kv,
                                                  h_q // h_kv, p)
                ma, rr = attn_errors(of[r], o_ref)
                assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS, (dense, s, i, ma, rr)
                assert np.abs(lf[:, r] - l_ref).max() < 1e-3, (dense, s, i)
        assert n_empty > 0


# ----------------------------------------------------------------------------
# selection
# ----------------------------------------------------------------------------

def _block_scores(plan, h_q, rows_q, rows):
    """Block scores of the given global query rows from the select
    workspace: fp32 [h_kv, rows_q, bs_ld] after the fp32 LSE [h_q, rows_q]
    (256-byte aligned), bs_ld = ceil(max_k / 64) rounded up to 4."""
    lse_bytes = (h_q * rows_q * 4 + 255) // 256 * 256
    bs_ld = ((plan.max_k + 63) // 64 + 3) // 4 * 4
    n = plan.h_kv * rows_q * bs_ld
    bs = plan.ws_select[lse_bytes:lse_bytes + 4 * n].view(torch.float32).view(plan.h_kv, rows_q, bs_ld)
    sel = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=bs.device)
    return dict(zip([int(r) for r in rows], bs.index_select(1, sel).permute(1, 0, 2).cpu().numpy()))


def _run_select(inp, lengths, h_q, h_kv, p: R.Params):
    st = _starts(lengths)
    plan = P.SparsePlan(st, lengths, st, lengths, sum(lengths), h_q, h_kv, _cfg(p))
    q, k = to_dev(inp.q), to_dev(inp.k)
    plan.compress(k)
    plan.select(q)
    torch.cuda.synchronize()
    lse = plan.ws_select[:h_q * sum(lengths) * 4].view(torch.float32).view(h_q, sum(lengths))
    return plan, plan.block_idx.cpu().numpy(), lse.cpu().numpy()


def _check_rows(inp, lengths, h_q, h_kv, p, idx, lse, positions_by_seq, plan=None):
    """Selection (and the LSE of scored rows) of the given positions against
    the oracle; with ``plan``, also the block scores element-wise."""
    pr = p.with_(round_kc=True)
    st = _starts(lengths)
    G = h_q // h_kv
    stats = {"rows": 0, "scored": 0, "exempt": 0, "band": 0, "scores": 0}
    bsd = {}
    if plan is not None:
        bsd = _block_scores(plan, h_q, sum(lengths),
                            [st[s] + t for s in range(len(lengths)) for t in positions_by_seq[s]])
    for s, n in enumerate(lengths):
        Ks = inp.k[st[s]:st[s] + n]
        KC1 = R.compress_keys(Ks, 32, 16, True)
        KC2 = R.compress_keys(Ks, 128, 64, True) if p.lse_mode == "approx" else None
        for t in positions_by_seq[s]:
            sel, diag = R.select_token(inp.q[st[s] + t], t, KC1, KC2, G, pr)
            if diag["scored"]:
                stats["scored"] += 1
                L_gpu = lse[:, st[s] + t]
                assert np.abs(L_gpu - diag["L"]).max() < 1e-3, (s, t, "lse")
            for g in range(h_kv):
                gl = [int(b) for b in idx[g, st[s] + t] if b >= 0]
                ok, exempt, band = check_selection(gl, sel[g], diag["info"][g], t, pr)
                assert ok, (s, t, g, gl, sel[g])
                stats["exempt"] += int(exempt)
                stats["band"] += band
                stats["rows"] += 1
                if bsd and diag["scored"]:
                    stats["scores"] += check_block_scores(bsd[st[s] + t][g], diag["block_scores"][g], t, pr)
    return stats


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_select_tiny_all_rows(lib, mode):
    """Tiny case, one KV head, G = 2, n = 4096, |I| = 1 + 4 + 11; every row."""
    say(f"select tiny {mode}")
    lengths, h_q, h_kv = [4096], 2, 1
    p = R.Params(n_init=1, n_local=4, n_topk=11, lse_mode=mode)
    inp = D.make_prefill(1, lengths, h_q, h_kv)
    plan, idx, lse = _run_select(inp, lengths, h_q, h_kv, p)
    stats = _check_rows(inp, lengths, h_q, h_kv, p, idx, lse, [range(4096)], plan)
    say(f"  {stats}")


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_select_group16_ragged(lib, mode):
    """32q/2kv, |I| = 96, two ragged sequences; sampled rows incl. every
    boundary where rows start needing scores."""
    say(f"select G=16 ragged {mode}")
    lengths, h_q, h_kv = [9001, 6300], 32, 2
    p = R.Params(lse_mode=mode)
    inp = D.make_prefill(6, lengths, h_q, h_kv, n_needles=4)
    plan, idx, lse = _run_select(inp, lengths, h_q, h_kv, p)
    pos = [sample_positions(n, 40, seed=s, must=(6143, 6144, 6145, 6207, 6208)) for s, n in enumerate(lengths)]
    stats = _check_rows(inp, lengths, h_q, h_kv, p, idx, lse, pos, plan)
    say(f"  {stats}")


def test_select_extreme_scores(lib):
    """Exact LSE through scores far above the first windows' (pass 1's
    overflowed-tile redo and its power-of-two renormalisation), G = 16,
    |I| = 1 + 4 + 16; LSE and selection on rows across the jump."""
    say("select extreme scores")
    n, h_q, h_kv = 6000, 16, 1
    lengths = [n, n]
    p = R.Params(n_init=1, n_local=4, n_topk=16, lse_mode="exact")
    inp = extreme_inputs(77, n, h_q)
    plan, idx, lse = _run_select(inp, lengths, h_q, h_kv, p)
    # From token 1800 on every scored row has at least 20 candidate blocks past
    # block 4, so its n_topk-th score is far from fp32 underflow.
    pos = [sorted(set(range(1800, 2720, 11)) | {t for t in sample_positions(n, 30, seed=30 + s) if t >= 1800})
           for s in range(2)]
    stats = _check_rows(inp, lengths, h_q, h_kv, p, idx, lse, pos, plan)
    assert stats["scored"] > 100
    assert float(lse[:, 2500].max()) > 100.0     # the jump reached the LSE of a scored row
    say(f"  {stats}")


@pytest.mark.parametrize("sel", [(0, 2, 9), (2, 0, 7), (1, 3, 0), (1, 2, 80), (0, 0, 64), (40, 4, 20)])
def test_select_budgets(lib, sel):
    """Unusual budgets: no init, no local or no top-k blocks, top-k counts at
    and above 64 (the top-k kernel's lane-maximum bound applies only up to
    64), and 40 init blocks (pass 2 then starts at window 128, one scoring
    tile in), 8q/2kv, two ragged sequences, sampled rows."""
    say(f"select budgets {sel}")
    lengths, h_q, h_kv = [12000, 7001], 8, 2
    p = R.Params(n_init=sel[0], n_local=sel[1], n_topk=sel[2], lse_mode="exact")
    inp = D.make_prefill(8, lengths, h_q, h_kv, n_needles=3)
    plan, idx, lse = _run_select(inp, lengths, h_q, h_kv, p)
    pos = [sample_positions(n, 40, seed=10 + s) for s, n in enumerate(lengths)]
    stats = _check_rows(inp, lengths, h_q, h_kv, p, idx, lse, pos, plan)
    say(f"  {stats}")


# ----------------------------------------------------------------------------
# end-to-end sparse path
# ----------------------------------------------------------------------------

def _e2e(inp, lengths, h_q, h_kv, p: R.Params, positions_by_seq, check_sel=True):
    st = _starts(lengths)
    plan = P.SparsePlan(st, lengths, st, lengths, sum(lengths), h_q, h_kv, _cfg(p))
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    out = torch.empty_like(q)
    lse_o = torch.empty((h_q, q.shape[0]), dtype=torch.float32, device="cuda")
    plan.run(q, k, v, out, lse_o)
    torch.cuda.synchronize()
    idx = plan.block_idx.cpu().numpy()
    lse_s = plan.ws_select[:h_q * sum(lengths) * 4].view(torch.float32).view(h_q, sum(lengths)).cpu().numpy()
    if check_sel:
        stats = _check_rows(inp, lengths, h_q, h_kv, p, idx, lse_s, positions_by_seq, plan)
        say(f"  selection {stats}")
    of, lf = to_f64(out), lse_o.cpu().numpy()
    G = h_q // h_kv
    worst = 0.0
    for s, n in enumerate(lengths):
        Ks, Vs = R.as_f64(inp.k[st[s]:st[s] + n]), R.as_f64(inp.v[st[s]:st[s] + n])
        for t in positions_by_seq[s]:
            gl = [[int(b) for b in idx[g, st[s] + t] if b >= 0] for g in range(h_kv)]
            o_ref, l_ref = R.attend_token(inp.q[st[s] + t], t, Ks, Vs, gl, G, p)
            ma, rr = attn_errors(of[st[s] + t], o_ref)
            worst = max(worst, ma)
            assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS, (s, t, ma, rr)
            assert np.abs(lf[:, st[s] + t] - l_ref).max() < 1e-3
    say(f"  attention max abs err {worst:.3e}")
    return plan, out


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_select_flat_scores_lowest_index(lib, mode):
    """Zero queries make every block score of a row equal, so the top-k is
    the n_topk lowest candidate blocks (ties go to the lower block index).
    At n = 40960 rows have up to 607 candidates, more than the top-k kernel
    keeps in its compacted LDS list, so both of its paths run."""
    say(f"select flat scores {mode}")
    n, h_q, h_kv = 40960, 32, 2
    p = R.Params(n_init=1, n_local=32, n_topk=63, lse_mode=mode)
    inp = D.make_prefill(5, [n], h_q, h_kv)
    inp.q[...] = 0
    _, idx, _ = _run_select(inp, [n], h_q, h_kv, p)
    n_sel = p.n_init + p.n_local + p.n_topk
    bt = np.arange(n) // 64
    want = np.full((n, n_sel), -1, dtype=np.int64)
    e = np.arange(n_sel)
    few = bt - p.n_local - p.n_init + 1 <= p.n_topk        # every causal block
    want[few] = np.where(e[None, :] <= bt[few, None], e[None, :], -1)
    many = ~few
    want[many, :p.n_init + p.n_topk] = np.arange(p.n_init + p.n_topk)[None, :]
    want[many, p.n_init + p.n_topk:] = bt[many, None] - p.n_local + 1 + np.arange(p.n_local)[None, :]
    for g in range(h_kv):
        bad = np.nonzero((idx[g].astype(np.int64) != want).any(axis=1))[0]
        assert bad.size == 0, (g, bad[:5], idx[g, bad[:1]], want[bad[:1]])


def test_tiny_full_budget_equals_dense(lib):
    """|I| = 64 covers all 64 blocks of n = 4096: the sparse path must equal
    dense causal attention (oracle dense and the GPU dense kernel)."""
    say("tiny |I|=64 == dense")
    lengths, h_q, h_kv = [4096], 2, 1
    p = R.Params(n_init=1, n_local=4, n_topk=59)
    inp = D.make_prefill(1, lengths, h_q, h_kv)
    plan, out = _e2e(inp, lengths, h_q, h_kv, p, [range(0, 4096, 7)], check_sel=False)
    idx = plan.block_idx.cpu().numpy()
    for t in range(4096):
        assert list(idx[0, t][:t // 64 + 1]) == list(range(t // 64 + 1))
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    dense = torch.empty_like(q)
    P.DensePlan([0], [4096], [0], [4096], 4096, h_q, h_kv, P.SparseConfig()).run(q, k, v, dense)
    Qf, Kf, Vf = R.as_f64(inp.q), R.as_f64(inp.k), R.as_f64(inp.v)
    ref = R.dense_prefill(Qf, Kf, Vf, 2, 1 / math.sqrt(128), positions=range(0, 4096, 5))
    o_ref = np.stack([ref[t][0] for t in ref])
    of = to_f64(out)[list(ref)]
    ma, rr = attn_errors(of, o_ref)
    assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS
    assert (out.float() - dense.float()).abs().max().item() <= 2 * 2.0 ** -8


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_end_to_end_with_empty_sequences(lib, mode):
    """A packed batch with empty sequences between real ones (8q/2kv,
    |I| = 1 + 4 + 11): selection and attention of the real sequences match
    the oracle; the empty ones own no rows."""
    say(f"end-to-end with empty sequences {mode}")
    lengths, h_q, h_kv = [0, 4100, 0, 1500, 0], 8, 2
    p = R.Params(n_init=1, n_local=4, n_topk=11, lse_mode=mode)
    inp = D.make_prefill(9, lengths, h_q, h_kv)
    pos = [[] if n == 0 else sample_positions(n, 30, seed=20 + s) for s, n in enumerate(lengths)]
    _e2e(inp, lengths, h_q, h_kv, p, pos)


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_tiny_end_to_end(lib, mode):
    say(f"tiny end-to-end {mode}")
    p = R.Params(n_init=1, n_local=4, n_topk=11, lse_mode=mode)
    inp = D.make_prefill(1, [4096], 2, 1)
    _e2e(inp, [4096], 2, 1, p, [range(0, 4096, 3)])


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_32k_sampled(lib, mode):
    """Single layer of the 8B shape at n = 32768 with 8 needle blocks."""
    say(f"32K end-to-end {mode}")
    n = 32768
    p = R.Params(lse_mode=mode)
    inp = D.make_prefill(2, n, 32, 2, n_needles=8)
    pos = sample_positions(n, 256, seed=2, must=(6143, 6144, 20000 - 1))
    _e2e(inp, [n], 32, 2, p, [pos])


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_128k_sampled(lib, mode):
    """n = 131072 (2048 blocks) with 32 needle blocks, the benchmark's
    prefill: 544 rows per mode, namely all 16 rows of 24 query tiles spread
    over the sequence (every row slot of the scoring, top-k and attention
    tiles) and 160 spread rows, both KV groups of each; selection, LSE, block
    scores and attention against the oracle."""
    say(f"128K end-to-end {mode}")
    n = 131072
    p = R.Params(lse_mode=mode)
    inp = D.make_prefill(3, n, 32, 2, n_needles=32)
    rng = np.random.Generator(np.random.PCG64(3))
    tiles = rng.choice(np.arange(6144 // 16, n // 16), size=24, replace=False)
    tile_rows = {int(16 * t + r) for t in tiles for r in range(16)}
    pos = sorted(tile_rows | set(sample_positions(n, 160, seed=3, must=(6144, 131071))))
    assert len(pos) >= 512
    _e2e(inp, [n], 32, 2, p, [pos])


def test_beyond_128k_two_windows(lib):
    """n = 133157 (2081 blocks): keys past 128K take the attention kernel
    that walks the block lists in two windows of 2048 blocks."""
    say("beyond-128K two-window end-to-end exact")
    n = 131072 + 2048 + 37
    p = R.Params(lse_mode="exact")
    inp = D.make_prefill(11, n, 32, 2, n_needles=32)
    pos = sample_positions(n, 6, seed=11, must=(131071, 131072 + 100, n - 1))
    _e2e(inp, [n], 32, 2, p, [pos])


def test_varlen_switch(lib):
    """Packed batch of 65536 tokens, lengths from the four buckets; <= 8192
    takes the dense path, longer sequences the sparse path."""
    lengths = D.varlen_lengths(5)
    say(f"varlen switch lengths={lengths}")
    h_q, h_kv = 32, 2
    inp = D.make_prefill(5, lengths, h_q, h_kv)
    cfg = P.SparseConfig()
    plan = P.SwitchPlan(lengths, h_q, h_kv, cfg)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    out = torch.empty_like(q)
    plan.run(q, k, v, out)
    torch.cuda.synchronize()
    of = to_f64(out)
    idx = plan.sparse.block_idx.cpu().numpy()
    st = _starts(lengths)
    p = R.Params()
    pr = p.with_(round_kc=True)
    for s, n in enumerate(lengths):
        Qs, Ks, Vs = inp.q[st[s]:st[s] + n], R.as_f64(inp.k[st[s]:st[s] + n]), R.as_f64(inp.v[st[s]:st[s] + n])
        pos = sample_positions(n, 6, seed=s)
        if n <= cfg.threshold:
            ref = R.dense_prefill(Qs, Ks, Vs, 16, 1 / math.sqrt(128), positions=pos)
            for t in pos:
                ma, rr = attn_errors(of[st[s] + t], ref[t][0])
                assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS, ("dense", s, t, ma)
        else:
            KC1 = R.compress_keys(inp.k[st[s]:st[s] + n], 32, 16, True)
            for t in pos:
                sel, diag = R.select_token(Qs[t], t, KC1, None, 16, pr)
                gl = [[int(b) for b in idx[g, st[s] + t] if b >= 0] for g in range(h_kv)]
                for g in range(h_kv):
                    ok, _, _ = check_selection(gl[g], sel[g], diag["info"][g], t, pr)
                    assert ok, ("sparse select", s, t, g)
                o_ref, _ = R.attend_token(Qs[t], t, Ks, Vs, gl, 16, p)
                ma, rr = attn_errors(of[st[s] + t], o_ref)
                assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS, ("sparse", s, t, ma)


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_split_select_short_queries(lib, mode):
    """Few query tiles (5, 1 and 3 queries at the end of 6000, 9001 and 4500
    keys) take the split-K scoring kernels; every row's selection is checked
    against the oracle's."""
    say(f"split select {mode}")
    h_q, h_kv = 32, 2
    klens, qlens = [6000, 9001, 4500], [5, 1, 3]
    p = R.Params(lse_mode=mode)
    pr = p.with_(round_kc=True)
    inp = D.make_prefill(33, klens, h_q, h_kv, n_needles=4)
    kst = _starts(klens)
    qrows = [kst[s] + klens[s] - qlens[s] + i for s in range(3) for i in range(qlens[s])]
    qst = _starts(qlens)
    plan = P.SparsePlan(qst, qlens, kst, klens, len(qrows), h_q, h_kv, _cfg(p))
    plan.compress(to_dev(inp.k))
    plan.select(to_dev(np.ascontiguousarray(inp.q[qrows])))
    torch.cuda.synchronize()
    idx = plan.block_idx.cpu().numpy()
    for s in range(3):
        Ks = inp.k[kst[s]:kst[s] + klens[s]]
        KC1 = R.compress_keys(Ks, 32, 16, True)
        KC2 = R.compress_keys(Ks, 128, 64, True) if mode == "approx" else None
        for i in range(qlens[s]):
            t = klens[s] - qlens[s] + i
            sel, diag = R.select_token(inp.q[kst[s] + t], t, KC1, KC2, h_q // h_kv, pr)
            for g in range(h_kv):
                gl = [int(b) for b in idx[g, qst[s] + i] if b >= 0]
                ok, _, _ = check_selection(gl, sel[g], diag["info"][g], t, pr)
                assert ok, (s, i, g)


def test_split_path_many_sequences(lib):
    """More than 64 sequences on the split-K kernels (one query at the end of
    each of 80 sequences of 300-6000 keys): the kernels find a row's sequence
    by binary search instead of the one-round ballot of smaller batches.
    Selection (exact LSE) and attention over the selected lists are checked
    against the oracle on a spread of rows, including the first and last
    sequence."""
    say("split path, 80 sequences")
    h_q, h_kv = 32, 2
    rng = np.random.Generator(np.random.PCG64(81))
    klens = [int(x) for x in rng.integers(300, 6000, size=80)]
    qlens = [1] * len(klens)
    p = R.Params(n_init=1, n_local=4, n_topk=11, lse_mode="exact")
    pr = p.with_(round_kc=True)
    inp = D.make_prefill(34, klens, h_q, h_kv, n_needles=2)
    kst = _starts(klens)
    qrows = [kst[s] + klens[s] - 1 for s in range(len(klens))]
    qst = _starts(qlens)
    plan = P.SparsePlan(qst, qlens, kst, klens, len(qrows), h_q, h_kv, _cfg(p))
    q = to_dev(np.ascontiguousarray(inp.q[qrows]))
    k, v = to_dev(inp.k), to_dev(inp.v)
    out = torch.empty_like(q)
    plan.run(q, k, v, out)
    torch.cuda.synchronize()
    idx = plan.block_idx.cpu().numpy()
    of = to_f64(out)
    check = sorted({0, 1, 63, 64, 65, len(klens) - 1} | set(int(x) for x in rng.choice(len(klens), 10, replace=False)))
    for s in check:
        t = klens[s] - 1
        Ks = inp.k[kst[s]:kst[s] + klens[s]]
        KC1 = R.compress_keys(Ks, 32, 16, True)
        sel, diag = R.select_token(inp.q[kst[s] + t], t, KC1, None, h_q // h_kv, pr)
        lists = []
        for g in range(h_kv):
            gl = [int(b) for b in idx[g, s] if b >= 0]
            ok, _, _ = check_selection(gl, sel[g], diag["info"][g], t, pr)
            assert ok, (s, g)
            lists.append(gl)
        o_ref, _ = R.attend_token(inp.q[kst[s] + t], t, R.as_f64(Ks), R.as_f64(inp.v[kst[s]:kst[s] + klens[s]]),
                                  lists, h_q // h_kv, p)
        ma, rr = attn_errors(of[s], o_ref)
        assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS, (s, ma, rr)


def test_end_to_end_extreme_scores(lib):
    """Selection and attention on the extreme-score inputs: the attention
    kernel's running max jumps by up to ~175 log2 units between blocks (its
    rescale path), sampled rows from token 1800 on."""
    say("end to end extreme scores")
    n, h_q, h_kv = 6000, 16, 1
    p = R.Params(n_init=1, n_local=4, n_topk=16, lse_mode="exact")
    inp = extreme_inputs(77, n, h_q)
    pos = [sorted({t for t in sample_positions(n, 40, seed=50 + s) if t >= 1800} | {1800, 2047, 2048, 2111, 5999})
           for s in range(2)]
    _e2e(inp, [n, n], h_q, h_kv, p, pos)


def test_split_select_extreme_scores(lib):
    """The split-K scoring kernels (4 and 2 queries at the end of the two
    sequences of the extreme-score inputs) against the oracle's selection."""
    say("split select extreme scores")
    n, h_q, h_kv = 6000, 16, 1
    klens, qlens = [n, n], [4, 2]
    p = R.Params(n_init=1, n_local=4, n_topk=16, lse_mode="exact")
    pr = p.with_(round_kc=True)
    inp = extreme_inputs(77, n, h_q)
    kst = _starts(klens)
    qrows = [kst[s] + klens[s] - qlens[s] + i for s in range(2) for i in range(qlens[s])]
    qst = _starts(qlens)
    plan = P.SparsePlan(qst, qlens, kst, klens, len(qrows), h_q, h_kv, _cfg(p))
    plan.compress(to_dev(inp.k))
    plan.select(to_dev(np.ascontiguousarray(inp.q[qrows])))
    torch.cuda.synchronize()
    idx = plan.block_idx.cpu().numpy()
    for s in range(2):
        KC1 = R.compress_keys(inp.k[kst[s]:kst[s] + klens[s]], 32, 16, True)
        for i in range(qlens[s]):
            t = klens[s] - qlens[s] + i
            sel, diag = R.select_token(inp.q[kst[s] + t], t, KC1, None, h_q // h_kv, pr)
            gl = [int(b) for b in idx[0, qst[s] + i] if b >= 0]
            ok, _, _ = check_selection(gl, sel[0], diag["info"][0], t, pr)
            assert ok, (s, i, gl, sel[0])


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_decode_steps(lib, mode):
    """Decode: incremental compression, selection for one new token per
    sequence and sparse attention over a transposed V cache, checked at
    every step against the oracle's row for that position (split-K scoring
    and attention)."""
    say(f"decode steps {mode}")
    batch, h_q, h_kv, steps = 3, 32, 2, 6
    lens0 = [7000, 9001, 6400]
    cap = 9088
    p = R.Params(lse_mode=mode)
    pr = p.with_(round_kc=True)
    inp = D.make_prefill(4, [cap] * batch, h_q, h_kv, n_needles=4)
    st = _starts([cap] * batch)
    cfg = _cfg(p)
    dec = P.DecodeState(batch, cap, h_q, h_kv, cfg)
    kt, vt = to_dev(inp.k), to_dev(inp.v)
    dec.fill([kt[st[s]:st[s] + lens0[s]] for s in range(batch)],
             [vt[st[s]:st[s] + lens0[s]] for s in range(batch)], lens0)
    qt = to_dev(inp.q)
    out = torch.empty((batch, h_q, 128), dtype=torch.bfloat16, device="cuda")
    for step in range(steps):
        pos = [dec.lens[s] for s in range(batch)]          # position of the new token
        k_new = torch.stack([kt[st[s] + pos[s]] for s in range(batch)])
        v_new = torch.stack([vt[st[s] + pos[s]] for s in range(batch)])
        q_new = torch.stack([qt[st[s] + pos[s]] for s in range(batch)]).contiguous()
        old = dec.append(k_new, v_new)
        dec.step_prepare(old)
        dec.step(q_new, out, max(dec.lens))
        torch.cuda.synchronize()
        idx = dec.block_idx.cpu().numpy()
        of = to_f64(out)
        for s in range(batch):
            t = pos[s]
            Ks = inp.k[st[s]:st[s] + t + 1]
            KC1 = R.compress_keys(Ks, 32, 16, True)
            KC2 = R.compress_keys(Ks, 128, 64, True) if mode == "approx" else None
            sel, diag = R.select_token(inp.q[st[s] + t], t, KC1, KC2, 16, pr)
            gl = [[int(b) for b in idx[g, s] if b >= 0] for g in range(h_kv)]
            for g in range(h_kv):
                ok, _, _ = check_selection(gl[g], sel[g], diag["info"][g], t, pr)
                assert ok, (step, s, g)
            o_ref, _ = R.attend_token(inp.q[st[s] + t], t, R.as_f64(Ks), R.as_f64(inp.v[st[s]:st[s] + t + 1]), gl, 16, p)
            ma, rr = attn_errors(of[s], o_ref)
            assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS, (step, s, ma, rr)


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_decode_graph_replays_match_eager(lib, mode):
    """The decode step captured once as a HIP graph and replayed for several
    steps, with the caller's eager cache appends between replays, gives
    bit-identical block lists and outputs to the eager step."""
    say(f"decode graph {mode}")
    batch, h_q, h_kv, steps = 3, 32, 2, 5
    lens0 = [7000, 9001, 6400]
    cap = 9088
    cfg = _cfg(R.Params(lse_mode=mode))
    inp = D.make_prefill(4, [cap] * batch, h_q, h_kv, n_needles=4)
    st = _starts([cap] * batch)
    kt, vt, qt = to_dev(inp.k), to_dev(inp.v), to_dev(inp.q)
    decs = [P.DecodeState(batch, cap, h_q, h_kv, cfg) for _ in range(2)]
    for dec in decs:
        dec.fill([kt[st[s]:st[s] + lens0[s]] for s in range(batch)],
                 [vt[st[s]:st[s] + lens0[s]] for s in range(batch)], lens0)
    graph = P.DecodeGraph(decs[1])
    out = torch.empty((batch, h_q, 128), dtype=torch.bfloat16, device="cuda")
    for step in range(steps):
        pos = [decs[0].lens[s] for s in range(batch)]
        k_new = torch.stack([kt[st[s] + pos[s]] for s in range(batch)])
        v_new = torch.stack([vt[st[s] + pos[s]] for s in range(batch)])
        q_new = torch.stack([qt[st[s] + pos[s]] for s in range(batch)]).contiguous()
        for dec in decs:
            dec.step_prepare(dec.append(k_new, v_new))
        decs[0].step(q_new, out, max(decs[0].lens))
        got = graph.step(q_new)
        torch.cuda.synchronize()
        assert torch.equal(decs[0].block_idx, decs[1].block_idx), step
        assert torch.equal(out.view(torch.int16), got.view(torch.int16)), step


def test_deterministic(lib):
    say("determinism")
    n = 8192
    inp = D.make_prefill(9, n, 32, 2, n_needles=4)
    plan = P.SparsePlan([0], [n], [0], [n], n, 32, 2, P.SparseConfig())
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    outs, idxs = [], []
    for _ in range(2):
        out = torch.empty_like(q)
        plan.run(q, k, v, out)
        torch.cuda.synchronize()
        outs.append(out.clone())
        idxs.append(plan.block_idx.clone())
    assert torch.equal(idxs[0], idxs[1])
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))

"""Decode at the benchmark's configuration: batch 16, a KV cache of about
131072 tokens per sequence, 32q/2kv, |I| = 1 + 32 + 63, one new token per
sequence per step, in both LSE modes.

72 consecutive steps per sequence, with starting lengths staggered by 0, 5,
10 and 15 tokens, so that every sequence passes positions t = 15 (mod 16)
(a stage-1 window completes), t = 63 (mod 64) (a coarse window completes)
and a block start, and the caches grow past 2048 blocks (the cache capacity
the step is captured with is 2049 blocks: the top-k and scoring instances of
the benchmark's decode run).  Every step is run eagerly and as a replay of
the captured HIP graph; the replay must equal the eager step bit for bit,
and every row of every step is checked against the oracle (selection by the
acceptance rule, attention at max-abs 2e-2 and relative RMS 1e-2, and the
block scores of the select workspace element-wise).
"""
import numpy as np
import pytest
import torch

import oracle.reference as R
from trainable_block_sparse_compress_amd import datagen as D
from trainable_block_sparse_compress_amd import pipeline as P
from tests.gpu_util import say, to_dev, to_f64
from tests.helpers import ATT_MAX_ABS, ATT_REL_RMS, attn_errors, check_selection, check_block_scores

pytestmark = pytest.mark.gpu

BATCH, H_Q, H_KV, STEPS = 16, 32, 2, 72
L0 = 131072 - 16           # cache rows drawn per sequence before the steps
STAGGER = (0, 5, 10, 15)   # sequence s starts at L0 - STAGGER[s % 4]


@pytest.fixture(scope="module")
def decode_inputs():
    """The seeded decode workload (drawn once for both LSE modes): sequence s
    holds tokens 0 .. L0 + STEPS - 1, the drawn cache followed by the drawn
    step tokens."""
    say("drawing the decode inputs (batch 16 x 128K)")
    inp = D.make_decode(4, BATCH, L0, STEPS, H_Q, H_KV, n_needles=32)
    k_all = [np.concatenate([inp.k_cache[s, :L0], inp.k_steps[:, s]]) for s in range(BATCH)]
    v_all = [np.concatenate([inp.v_cache[s, :L0], inp.v_steps[:, s]]) for s in range(BATCH)]
    return inp, k_all, v_all


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_decode_128k_batch16_every_row(lib, decode_inputs, mode):
    say(f"decode batch 16 x 128K, {STEPS} steps, {mode}")
    inp, k_all, v_all = decode_inputs
    cap = (L0 + STEPS + 63) // 64 * 64
    assert cap // 64 > 2048
    p = R.Params(lse_mode=mode)
    pr = p.with_(round_kc=True)
    cfg = P.SparseConfig(lse_mode=mode)
    # Sequence s starts at len0[s] tokens and appends one token a step.
    len0 = [L0 - STAGGER[s % 4] for s in range(BATCH)]
    eager = P.DecodeState(BATCH, cap, H_Q, H_KV, cfg)
    replay = P.DecodeState(BATCH, cap, H_Q, H_KV, cfg)
    for dec in (eager, replay):
        dec.fill([to_dev(k_all[s][:len0[s]]) for s in range(BATCH)],
                 [to_dev(v_all[s][:len0[s]]) for s in range(BATCH)], len0)
    graph = P.DecodeGraph(replay)
    out = torch.empty((BATCH, H_Q, 128), dtype=torch.bfloat16, device="cuda")
    idx_steps, out_steps, bs_steps, pos_steps = [], [], [], []
    bs_ld = (cap + 63) // 64
    bs_ld = (bs_ld + 3) // 4 * 4
    lse_bytes = (H_Q * BATCH * 4 + 255) // 256 * 256
    for i in range(STEPS):
        pos = list(eager.lens)
        k_new = to_dev(np.stack([k_all[s][pos[s]] for s in range(BATCH)]))
        v_new = to_dev(np.stack([v_all[s][pos[s]] for s in range(BATCH)]))
        q_new = to_dev(np.ascontiguousarray(inp.q_steps[i]))
        for dec in (eager, replay):
            dec.step_prepare(dec.append(k_new, v_new))
        eager.step(q_new, out, max(eager.lens))
        got = graph.step(q_new)
        torch.cuda.synchronize()
        assert torch.equal(eager.block_idx, replay.block_idx), ("graph lists", i)
        assert torch.equal(out.view(torch.int16), got.view(torch.int16)), ("graph output", i)
        idx_steps.append(eager.block_idx.cpu().numpy())
        out_steps.append(to_f64(out))
        # Block scores in the replayed step's select workspace (captured with
        # max_seqlen_k = cap): fp32 [h_kv, batch, bs_ld] after the fp32 LSE.
        ws = replay.ws_select[lse_bytes:lse_bytes + H_KV * BATCH * bs_ld * 4]
        bs_steps.append(ws.view(torch.float32).view(H_KV, BATCH, bs_ld).cpu().numpy())
        pos_steps.append(pos)
    say(f"  GPU steps done (graph replays bit-exact); checking {BATCH * STEPS} rows")
    residues = set()
    stats = {"rows": 0, "exempt": 0, "band": 0, "scores": 0}
    worst = 0.0
    for s in range(BATCH):
        say(f"  oracle rows of sequence {s}")
        K = k_all[s]
        Kf, Vf = R.as_f64(K), R.as_f64(v_all[s])
        KC1 = R.compress_keys(K[:len0[s]], 32, 16, True)
        KC2 = R.compress_keys(K[:len0[s]], 128, 64, True) if mode == "approx" else None
        for i in range(STEPS):
            t = pos_steps[i][s]
            assert t == len0[s] + i
            residues |= {("w1", t % 16 == 15), ("w2", t % 64 == 63), ("blk", t % 64 == 0)}
            KC1 = R.compress_keys_incremental(K[:t + 1], KC1, 32, 16, True)
            if KC2 is not None:
                KC2 = R.compress_keys_incremental(K[:t + 1], KC2, 128, 64, True)
            sel, diag = R.select_token(inp.q_steps[i, s], t, KC1, KC2, H_Q // H_KV, pr)
            gl = [[int(b) for b in idx_steps[i][g, s] if b >= 0] for g in range(H_KV)]
            for g in range(H_KV):
                ok, exempt, band = check_selection(gl[g], sel[g], diag["info"][g], t, pr)
                assert ok, (mode, s, i, t, g)
                stats["exempt"] += int(exempt)
                stats["band"] += band
                stats["rows"] += 1
                if diag["scored"]:
                    stats["scores"] += check_block_scores(bs_steps[i][g, s], diag["block_scores"][g], t, pr)
            o_ref, _ = R.attend_token(inp.q_steps[i, s], t, Kf, Vf, gl, H_Q // H_KV, p)
            ma, rr = attn_errors(out_steps[i][s], o_ref)
            worst = max(worst, ma)
            assert ma <= ATT_MAX_ABS and rr <= ATT_REL_RMS, (mode, s, i, t, ma, rr)
    assert {("w1", True), ("w2", True), ("blk", True)} <= residues
    say(f"  {stats}; attention max abs err {worst:.3e}")

"""The unfused selection baseline (infllmv2_select_blocks_unfused: every
head's stage-1 probabilities written to HBM, then summed per group and
max-pooled by a second kernel) against the oracle, with the same bars as
the fused path: selection by the acceptance rule, the LSE, and the block
scores element-wise; and against the fused kernels' block scores."""
import numpy as np
import pytest
import torch

import oracle.reference as R
from trainable_block_sparse_compress_amd import datagen as D
from trainable_block_sparse_compress_amd import pipeline as P
from tests.gpu_util import say, to_dev
from tests.helpers import sample_positions
from tests.test_gpu_parity import _block_scores, _cfg, _check_rows, _starts

pytestmark = pytest.mark.gpu


def _select(inp, lengths, h_q, h_kv, p, unfused):
    st = _starts(lengths)
    plan = P.SparsePlan(st, lengths, st, lengths, sum(lengths), h_q, h_kv, _cfg(p),
                        unfused_select=unfused)
    plan.compress(to_dev(inp.k))
    plan.select(to_dev(inp.q))
    torch.cuda.synchronize()
    lse = plan.ws_select[:h_q * sum(lengths) * 4].view(torch.float32).view(h_q, sum(lengths))
    return plan, plan.block_idx.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_unfused_select_tiny_all_rows(lib, mode):
    say(f"unfused select tiny {mode}")
    lengths, h_q, h_kv = [4096], 2, 1
    p = R.Params(n_init=1, n_local=4, n_topk=11, lse_mode=mode)
    inp = D.make_prefill(1, lengths, h_q, h_kv)
    plan, idx, lse = _select(inp, lengths, h_q, h_kv, p, True)
    say(f"  {_check_rows(inp, lengths, h_q, h_kv, p, idx, lse, [range(4096)], plan)}")


@pytest.mark.parametrize("mode", ["exact", "approx"])
def test_unfused_select_group16_ragged(lib, mode):
    say(f"unfused select G=16 ragged {mode}")
    lengths, h_q, h_kv = [9001, 6300], 32, 2
    p = R.Params(lse_mode=mode)
    inp = D.make_prefill(6, lengths, h_q, h_kv, n_needles=4)
    plan, idx, lse = _select(inp, lengths, h_q, h_kv, p, True)
    pos = [sample_positions(n, 40, seed=s, must=(6143, 6144, 6145, 6207, 6208)) for s, n in enumerate(lengths)]
    say(f"  {_check_rows(inp, lengths, h_q, h_kv, p, idx, lse, pos, plan)}")


def test_unfused_select_32k_against_oracle_and_fused(lib):
    """n = 32768 (two chunks of query rows): sampled rows against the oracle,
    and every scored row's block scores against the fused kernels' (the two
    differ only in the order of the fp32 group sum)."""
    say("unfused select 32K")
    n, h_q, h_kv = 32768, 32, 2
    p = R.Params()
    inp = D.make_prefill(2, n, h_q, h_kv, n_needles=8)
    plan_u, idx_u, lse_u = _select(inp, [n], h_q, h_kv, p, True)
    pos = sample_positions(n, 64, seed=2, must=(6143, 6144, 16383, 16384, 20000 - 1))
    say(f"  {_check_rows(inp, [n], h_q, h_kv, p, idx_u, lse_u, [pos], plan_u)}")
    plan_f, idx_f, lse_f = _select(inp, [n], h_q, h_kv, p, False)
    assert np.array_equal(lse_u[:, 96 * 64:], lse_f[:, 96 * 64:])   # pass 1 is shared (rows with scores)
    rows = list(range(96 * 64, n, 7))
    bu, bf = _block_scores(plan_u, h_q, n, rows), _block_scores(plan_f, h_q, n, rows)
    worst = 0.0
    for t in rows:
        c = np.arange(p.n_init, t // 64 - p.n_local + 1)
        a, b = bu[t][:, c].astype(np.float64), bf[t][:, c].astype(np.float64)
        rel = np.abs(a - b) / np.maximum(np.abs(b), 1e-30)
        worst = max(worst, float(rel[b > 1e-6 * b.max()].max()))
    say(f"  block scores unfused vs fused: max relative difference {worst:.2e}; "
        f"identical lists {np.mean(np.all(idx_u == idx_f, axis=2)):.4f}")
    assert worst <= 1e-5

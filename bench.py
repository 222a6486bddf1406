#!/usr/bin/env python3
"""Benchmark of the InfLLM-V2 sparse-attention prefill path on one MI355X.

One step = the whole sparse path for one attention layer over one 131072-token
sequence (32 query heads, 2 KV heads, head_dim 128, |I| = 1 + 32 + 63 = 96
blocks of 64 tokens, 32 needle blocks): compress_k (stage-1 keys, plus the
coarse keys in approx mode) -> select_blocks (LSE pass, fused group-sum /
max-pool pass, top-k) -> sparse_attn.  Inputs are resident in HBM before the
timed region.  V is supplied in the transposed layout [h_kv, d, batch, n]
that the attention kernel reads (the V projection can emit it directly).

Prints one JSON line (see the keys below), with a roofline entry for the
dominant kernel (sparse attention) measured with HIP events on the stream it
runs on, and the fp64 oracle timed on a bounded sample as CPU baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn prefill tokens/s @128K (32q/2kv,d128,|I|=96); % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def visible_keys(t, n_sel, B=64):
    bt = t // B
    return np.where(bt < n_sel, t + 1, (n_sel - 1) * B + (t % B) + 1)


def algorithmic_work(n, h_q, h_kv, d=128, n_init=1, n_local=32, n_topk=63):
    """Algorithmic flops / bytes of each stage for one prefill of length n
    (no masked or padded work counted)."""
    n_sel = n_init + n_local + n_topk
    t = np.arange(n, dtype=np.int64)
    bt = t // 64
    scored = bt >= n_sel                      # rows with more candidates than n_topk
    nv1 = np.clip((t - 31) // 16 + 1, 0, None)
    nv2 = np.clip((t - 127) // 64 + 1, 0, None)
    cand_windows = np.clip(4 * (bt - n_local) + 4 - max(0, 4 * n_init - 1), 0, None)
    ncand = np.clip(bt - n_local - n_init + 1, 0, None)
    w = {}
    w["attn_flops"] = float(4 * d * h_q * visible_keys(t, n_sel).sum())
    w["lse_exact_flops"] = float(2 * d * h_q * nv1[scored].sum())
    w["lse_approx_flops"] = float(2 * d * h_q * nv2[scored].sum())
    w["blocks_flops"] = float(2 * d * h_q * cand_windows[scored].sum())
    w["topk_bytes"] = float(4 * h_kv * ncand[scored].sum() + 4 * h_kv * n * n_sel)
    n1, n2 = (n - 32) // 16 + 1, (n - 128) // 64 + 1
    w["compress_bytes"] = float(2 * h_kv * d * (n + n1))
    w["compress2_bytes"] = float(2 * h_kv * d * (n + n2))
    return w


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_from_profile(kernel_src):
    """Bytes per launch between the L2 and the memory side (FETCH_SIZE +
    WRITE_SIZE, scaled by a plain copy of known size) from the committed PMC
    summary, if it was taken on the current kernel source; None otherwise.
    The memory side is HBM or the Infinity Cache in front of it (the
    counters do not separate them), so this bounds the HBM bytes from above.
    The summary covers the default workload (n = 131072, exact LSE) only."""
    f = os.path.join(ROOT, "profiles", "attn_kernel_128k_pmc.json")
    if not os.path.exists(f):
        return None
    try:
        rec = json.load(open(f))
    except Exception:
        return None
    if rec.get("source_sha256_16") != source_hash(kernel_src):
        return None
    return rec.get("memory_side_bytes_per_launch")


def host_cores():
    """Worker processes for the oracle baseline: the cores this process may
    run on, capped by OMP_NUM_THREADS when it is set (the host's CPU share)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Oracle state shared with the forked baseline workers (copy-on-write).
_ORACLE = {}


def _oracle_rows(args):
    """Worker: whole oracle rows (selection + attention) at the given
    positions until the time budget is spent; returns the per-row times."""
    positions, budget = args
    from threadpoolctl import threadpool_limits

    import oracle.reference as R
    c = _ORACLE
    times = []
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        for t in positions:
            ts = time.perf_counter()
            sel, _ = R.select_token(c["q"][t], t, c["KC1"], c["KC2"], c["G"], c["p"])
            R.attend_token(c["q"][t], t, c["Kf"], c["Vf"], sel, c["G"], c["p"])
            times.append(time.perf_counter() - ts)
            if time.perf_counter() - t0 > budget:
                break
    return times


def cpu_baseline(inp, n, h_q, h_kv, lse_mode, budget_s=15.0):
    """The fp64 oracle on the host's cores, on a bounded sample of the same
    workload: the stage-1 (and coarse) compression of all n tokens once, then
    whole rows (selection + attention) at spread positions in worker
    processes (one BLAS thread each) for about ``budget_s`` seconds of wall
    time; the measured parallel row rate is extrapolated to all n rows.  Runs
    before the GPU is touched (the workers are forked)."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    import oracle.reference as R
    cores = host_cores()
    p = R.Params(lse_mode=lse_mode, round_kc=True)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        KC1 = R.compress_keys(inp.k, 32, 16, True)
        KC2 = R.compress_keys(inp.k, 128, 64, True) if lse_mode == "approx" else None
        t_pre = time.perf_counter() - t0
    _ORACLE.update(q=inp.q, KC1=KC1, KC2=KC2, Kf=R.as_f64(inp.k), Vf=R.as_f64(inp.v),
                   G=h_q // h_kv, p=p)
    positions = np.random.Generator(np.random.PCG64(0)).permutation(
        np.linspace(0, n - 1, 1024 * cores).astype(int))
    jobs = [([int(t) for t in positions[w::cores]], budget_s) for w in range(cores)]
    t1 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as pool:
        per_worker = pool.map(_oracle_rows, jobs)
    wall = time.perf_counter() - t1
    _ORACLE.clear()
    times = [x for w in per_worker for x in w]
    rows = len(times)
    rate = rows / wall                         # rows per second on `cores` processes
    value = n / (t_pre + n / rate)
    one_core = n / (t_pre + n * float(np.mean(times)))
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "value_1core": one_core,
            "sample": f"fp64 oracle: stage-1{' and coarse' if KC2 is not None else ''} compression "
                      f"of all {n} tokens ({t_pre:.1f} s, one process), then {rows} whole rows "
                      f"(selection + attention) at spread positions on {cores} worker processes "
                      f"(1 BLAS thread each) in {wall:.1f} s, extrapolated to {n} rows"}


# L2 -> CU read bandwidth of MI355X: 16 L2 channels of 128 B/clk per XCD
# (2048 B/clk), 8 XCDs, 2.4 GHz.  The gather roof of the attention kernel.
PEAK_L2_GBS = 2048 * 8 * 2.4

DECODE_BATCH, DECODE_CACHE, DECODE_STEPS = 16, 131072, 256


def staged_bytes(idx):
    """Bytes the tile attention kernel stages per launch: every 16-row query
    tile stages each distinct block of its rows' block sets once (K and V,
    64 x 128 bf16 each).  idx: int32 [h_kv, rows, n_sel], -1 padded."""
    h_kv, rows, n_sel = idx.shape
    nt = (rows + 15) // 16
    total = 0
    for g in range(h_kv):
        x = np.full((nt * 16, n_sel), -1, dtype=np.int32)
        x[:rows] = idx[g]
        x = np.sort(x.reshape(nt, 16 * n_sel), axis=1)
        distinct = (np.diff(x, axis=1) != 0).sum(axis=1) + 1 - (x[:, 0] < 0)
        total += int(distinct.sum())
    return total * 2 * 64 * 128 * 2


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seq", type=int, default=131072)
    ap.add_argument("--lse", choices=["exact", "approx"], default="exact")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-extras", action="store_true",
                    help="prefill: skip the extra keys (approximate-LSE step, 256-step decode)")
    ap.add_argument("--decode-steps", type=int, default=DECODE_STEPS,
                    help="decode steps timed (the extra decode key and --workload decode)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB 3 times (a plain copy "
                         "kernel of known size, to calibrate HBM byte counters)")
    ap.add_argument("--dense-steps", type=int, default=0,
                    help="also time the dense causal kernel at the same length (context)")
    ap.add_argument("--workload", choices=["prefill", "decode", "varlen", "dense", "sweep", "backward",
                                           "layer", "layer_decode", "unfused"],
                    default="prefill",
                    help="prefill (default): one 128K sequence; decode: 16 sequences x 128K "
                         "cache, one token each per step; varlen: 65536 packed tokens of mixed "
                         "lengths through the dense/sparse switch; dense: the switch's short path "
                         "alone (8 x 8192 packed tokens); sweep: the prefill at several "
                         "selection sizes |I| against the dense kernel at the same length; "
                         "backward: the gradients of the 128K sparse attention (selection "
                         "held fixed); layer: one attention layer of the 8B shape (hidden 4096) "
                         "with its Q/K/V/O projections, sparse against dense (prefill, time to "
                         "first token); layer_decode: the same layer in decode (time per output "
                         "token); unfused: block selection with and without the fused group sum")
    ap.add_argument("--no-graph", action="store_true",
                    help="decode: launch the step's kernels one by one instead of replaying "
                         "the captured HIP graph of the step")
    ap.add_argument("--sel", type=str, default="16,32,64,96",
                    help="sweep: selection sizes |I| (1 init block, |I|//3 local, rest top-k)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 "
                                   "(sharding across GPUs is not implemented)"}))
        sys.exit(2)

    if args.workload == "decode":
        return bench_decode(args)
    if args.workload == "varlen":
        return bench_varlen(args)
    if args.workload == "dense":
        return bench_dense(args)
    if args.workload == "sweep":
        return bench_sweep(args)
    if args.workload == "backward":
        return bench_backward(args)
    if args.workload == "layer":
        return bench_layer(args)
    if args.workload == "layer_decode":
        return bench_layer_decode(args)
    if args.workload == "unfused":
        return bench_unfused(args)
    return bench_prefill(args)


def time_prefill(plan, q, k, vt, n, cfg, d, steps, warmup, out):
    """Warmup, then `steps` timed steps of compress_k + select_blocks +
    sparse_attn on the current stream: (ms per step, ms per stage)."""
    import torch

    from trainable_block_sparse_compress_amd import binding as B
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        plan.compress(k)
        if ev is not None:
            ev[1].record(stream)
        plan.select(q)
        if ev is not None:
            ev[2].record(stream)
        B.sparse_attn(q, k, vt, plan.cu_q, plan.used_q, plan.cu_k, plan.used_k, 1, n, n,
                      plan.block_idx, cfg.n_init, cfg.n_local, cfg.scale(d), out, None, None,
                      v_seq_stride=n)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        step(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    stages = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j in range(3)]
    return ms, stages


def bench_prefill(args):
    from trainable_block_sparse_compress_amd import datagen as D

    n, h_q, h_kv, d = args.seq, 32, 2, 128
    extras = not args.no_extras and n == 131072
    print(f"[bench] generating inputs n={n}", file=sys.stderr, flush=True)
    inp = D.make_prefill(3, n, h_q, h_kv, d, n_needles=32)
    cpu = None
    if not args.no_cpu:
        # The oracle runs first, in forked workers, before the GPU is touched.
        print(f"[bench] cpu baseline (oracle, {host_cores()} processes)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, n, h_q, h_kv, args.lse, args.cpu_budget)
    dec_inp = None
    if extras:
        print("[bench] decode inputs", file=sys.stderr, flush=True)
        dec_inp = D.make_decode(4, DECODE_BATCH, DECODE_CACHE, 8 + args.decode_steps, h_q, h_kv, d,
                                n_needles=32)

    import torch

    from trainable_block_sparse_compress_amd import binding as B
    from trainable_block_sparse_compress_amd import pipeline as P

    dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    vt = v.permute(1, 2, 0).contiguous().view(h_kv, d, 1, n)   # caller-side layout, outside the timed region
    out = torch.empty_like(q)
    cfg = P.SparseConfig(lse_mode=args.lse)
    plan = P.SparsePlan([0], [n], [0], [n], n, h_q, h_kv, cfg)
    print("[bench] timed steps", file=sys.stderr, flush=True)
    ms, (ms_compress, ms_select, ms_attn) = time_prefill(plan, q, k, vt, n, cfg, d, args.steps,
                                                         args.warmup, out)

    w = algorithmic_work(n, h_q, h_kv, d)
    lse_flops = w["lse_exact_flops"] if args.lse == "exact" else w["lse_approx_flops"]
    mfma_flops = w["attn_flops"] + lse_flops + w["blocks_flops"]
    attn_tflops = w["attn_flops"] / (ms_attn * 1e-3) / 1e12
    staged = staged_bytes(plan.block_idx.cpu().numpy())
    gather_gbs = staged / (ms_attn * 1e-3) / 1e9
    kernel_src = os.path.join(ROOT, "trainable_block_sparse_compress_amd", "csrc", "attention.hip")
    traffic = traffic_from_profile(kernel_src) if (n == 131072 and args.lse == "exact") else None
    res = {
        "metric": METRIC,
        "value": n / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) bf16 Q/K/V with 32 planted needle blocks",
        "config": {"workload": f"sparse prefill, one layer, n={n}", "seq_len": n, "h_q": h_q,
                   "h_kv": h_kv, "head_dim": d, "block_size": 64, "n_init": 1, "n_local": 32,
                   "n_topk": 63, "lse": args.lse,
                   "v_layout": "transposed [h_kv, d, batch, n] (the attention kernel's; formed "
                               "outside the timed region)"},
        "mfma_frac_of_peak": mfma_flops / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "ms_compress_k": ms_compress,
        "ms_select_blocks": ms_select,
        "ms_sparse_attn": ms_attn,
        "roofline": {"bound": "mfma", "kernel": "attn_kernel (infllmv2_sparse_attn)",
                     "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "gather": {"bytes_per_launch": staged, "achieved": gather_gbs,
                                "peak": PEAK_L2_GBS, "unit": "GB/s", "frac": gather_gbs / PEAK_L2_GBS,
                                "basis": "K and V of every distinct block of each 16-row query "
                                         "tile, staged once per tile, over the kernel's time; "
                                         "peak = L2->CU reads, 2048 B/clk per XCD x 8 x 2.4 GHz"}},
    }
    if extras and args.lse == "exact":
        print("[bench] approximate LSE", file=sys.stderr, flush=True)
        cfg2 = P.SparseConfig(lse_mode="approx")
        plan2 = P.SparsePlan([0], [n], [0], [n], n, h_q, h_kv, cfg2)
        ms2, (c2, s2, a2) = time_prefill(plan2, q, k, vt, n, cfg2, d, args.steps, args.warmup, out)
        f2 = w["attn_flops"] + w["lse_approx_flops"] + w["blocks_flops"]
        res["approx_lse"] = {"value": n / (ms2 * 1e-3), "unit": "tokens/s", "ms_per_step": ms2,
                             "steps": args.steps, "ms_compress_k": c2, "ms_select_blocks": s2,
                             "ms_sparse_attn": a2,
                             "mfma_frac_of_peak": f2 / (ms2 * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)}
        del plan2
    if dec_inp is not None:
        del plan
        torch.cuda.empty_cache()
        print(f"[bench] decode, {args.decode_steps} steps", file=sys.stderr, flush=True)
        r = run_decode(dec_inp, DECODE_BATCH, DECODE_CACHE, args.decode_steps, 8, args.lse,
                       graph=True)
        res["decode"] = {"value": r["value"], "unit": "tokens/s", "ms_per_step": r["ms_per_step"],
                         "steps": args.decode_steps, "workload": r["workload"],
                         "launch": r["launch"], "hbm_frac": r["roofline"]["frac"],
                         "hbm_gbs": r["roofline"]["achieved"]}
    if args.dense_steps > 0:
        print("[bench] dense kernel", file=sys.stderr, flush=True)
        stream = torch.cuda.current_stream()
        dplan = P.DensePlan([0], [n], [0], [n], n, h_q, h_kv, cfg)
        dout = torch.empty_like(q)
        run_dense = lambda: B.dense_attn(q, k, vt, dplan.cu_q, dplan.used_q, dplan.cu_k,
                                         dplan.used_k, 1, n, n, cfg.scale(d), dout, None, None,
                                         v_seq_stride=n)
        run_dense()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.dense_steps):
            run_dense()
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / args.dense_steps
        dflops = 4.0 * d * h_q * (n * (n + 1) / 2)
        res["dense_attn_ms"] = dms
        res["dense_attn_tflops"] = dflops / (dms * 1e-3) / 1e12
        res["sparse_vs_dense_kernel_speedup"] = dms / ms_attn
    if args.copy_calib_mb > 0:
        nb = args.copy_calib_mb << 20
        src = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calib_bytes"] = nb
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


def decode_step_bytes(batch, len0, h_kv, n_sel, d=128):
    """Algorithmic HBM bytes of one decode step: the stage-1 keys read once
    (scoring), the selected K and V blocks of every sequence and KV group,
    the block scores written and read, and the block lists."""
    n1 = (len0 - 32) // 16 + 1
    nblk = (len0 + 63) // 64
    kc1_bytes = batch * h_kv * n1 * d * 2
    kv_bytes = batch * h_kv * n_sel * 64 * d * 2 * 2
    bs_bytes = 2 * batch * h_kv * nblk * 4 + batch * h_kv * n_sel * 4
    return kc1_bytes + kv_bytes + bs_bytes


def run_decode(inp, batch, len0, steps, warmup, lse_mode, graph=True):
    """Decode over `warmup + steps` consecutive tokens per sequence of a
    batch of `len0`-token caches (incremental compress_k, select_blocks,
    sparse_attn: the split-K path), replayed as the captured HIP graph of
    the step (graph=False: the library calls one by one).  Each step is
    timed with HIP events around the replay (or the calls); the caller's
    cache append and query placement are outside the timed region."""
    import torch

    from trainable_block_sparse_compress_amd import binding as B
    from trainable_block_sparse_compress_amd import pipeline as P

    h_q, h_kv, d = inp.q_steps.shape[2], inp.k_steps.shape[2], inp.q_steps.shape[3]
    nsteps = warmup + steps
    cap = (len0 + nsteps + 63) // 64 * 64
    cfg = P.SparseConfig(lse_mode=lse_mode)
    dec = P.DecodeState(batch, cap, h_q, h_kv, cfg)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    for s in range(batch):
        kc, vc = dev(inp.k_cache[s, :len0]), dev(inp.v_cache[s, :len0])
        dec.fill_one(s, kc, vc)
    dec.compress_all()
    qs, ks, vs = dev(inp.q_steps), dev(inp.k_steps), dev(inp.v_steps)
    out = torch.empty((batch, h_q, d), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    t_step, t_sel, t_attn = [], [], []
    g = P.DecodeGraph(dec) if graph else None
    for i in range(nsteps):
        old = dec.append(ks[i], vs[i])
        dec.step_prepare(old)
        q_new = qs[i].contiguous()
        if g is not None:
            g.q.copy_(q_new)          # the caller's input placement, outside the timed region
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= warmup:
                t_step.append(e0.elapsed_time(e1))
            continue
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        c, mx = cfg, max(dec.lens)
        ev[0].record(stream)
        B.compress_k(dec.k_cache, dec.cu_k, dec.used_k, batch, mx, c.c1[0], c.c1[1], dec.cu_c1,
                     dec.kc1, cmp_begin=dec.begin1, max_new=1)
        if dec.approx:
            B.compress_k(dec.k_cache, dec.cu_k, dec.used_k, batch, mx, c.c2[0], c.c2[1], dec.cu_c2,
                         dec.kc2, cmp_begin=dec.begin2, max_new=1)
        ev[1].record(stream)
        B.select_blocks(q_new, dec.kc1, dec.kc2, dec.cu_q, dec.used_q, dec.cu_k, dec.used_k,
                        dec.cu_c1, dec.cu_c2, batch, 1, mx, c.n_init, c.n_local, c.n_topk,
                        c.scale(d), dec.block_idx, dec.ws_select)
        ev[2].record(stream)
        B.sparse_attn(q_new, dec.k_cache, dec.vt_cache, dec.cu_q, dec.used_q, dec.cu_k, dec.used_k,
                      batch, 1, mx, dec.block_idx, c.n_init, c.n_local, c.scale(d), out, None,
                      dec.ws_attn, v_seq_stride=cap)
        ev[3].record(stream)
        torch.cuda.synchronize()
        if i >= warmup:
            t_step.append(ev[0].elapsed_time(ev[3]))
            t_sel.append(ev[1].elapsed_time(ev[2]))
            t_attn.append(ev[2].elapsed_time(ev[3]))
    ms = float(np.mean(t_step))
    step_bytes = decode_step_bytes(batch, len0, h_kv, cfg.n_sel, d)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    return {
        "value": batch / (ms * 1e-3), "ms_per_step": ms,
        "workload": f"decode, batch {batch}, cache {len0} per sequence, {steps} consecutive "
                    "tokens per sequence",
        "launch": "eager" if g is None else "HIP graph replay of the captured step",
        "ms_per_step_median": float(np.median(t_step)),
        "ms_select_blocks": float(np.mean(t_sel)) if t_sel else None,
        "ms_sparse_attn": float(np.mean(t_attn)) if t_attn else None,
        "ms_select_blocks_median": float(np.median(t_sel)) if t_sel else None,
        "ms_sparse_attn_median": float(np.median(t_attn)) if t_attn else None,
        "roofline": {"bound": "hbm", "kernel": "whole decode step (compress_k + select_blocks + "
                                                "sparse_attn)",
                     "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                     "bytes_per_step": step_bytes, "traffic": None},
    }


def bench_decode(args):
    """Decode: batch 16, a 128K-token cache per sequence, one new token per
    sequence per step, `--decode-steps` consecutive steps (see run_decode)."""
    from trainable_block_sparse_compress_amd import datagen as D

    batch, len0, h_q, h_kv, d = DECODE_BATCH, args.seq, 32, 2, 128
    print(f"[bench] decode inputs batch={batch} cache={len0}", file=sys.stderr, flush=True)
    inp = D.make_decode(4, batch, len0, 8 + args.decode_steps, h_q, h_kv, d, n_needles=32)
    cpu = None
    if not args.no_cpu:
        print(f"[bench] cpu baseline (oracle, {host_cores()} processes)", file=sys.stderr, flush=True)
        cpu = cpu_baseline_decode(inp, batch, len0, h_q, h_kv, args.lse)
    print(f"[bench] decode steps ({'eager' if args.no_graph else 'graph replay'})", file=sys.stderr,
          flush=True)
    r = run_decode(inp, batch, len0, args.decode_steps, 8, args.lse, graph=not args.no_graph)
    res = {
        "metric": "sparse-attn decode tokens/s (batch 16, 128K cache, 32q/2kv, d128, |I|=96)",
        "value": r["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.decode_steps,
        "warmup": 8, "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) bf16 cache and step tokens, 32 needle blocks/seq",
        "config": {"workload": r["workload"], "h_q": h_q, "h_kv": h_kv, "head_dim": d,
                   "n_init": 1, "n_local": 32, "n_topk": 63, "lse": args.lse},
        "launch": r["launch"], "ms_per_step_median": r["ms_per_step_median"],
        "ms_select_blocks": r["ms_select_blocks"], "ms_sparse_attn": r["ms_sparse_attn"],
        "ms_select_blocks_median": r["ms_select_blocks_median"],
        "ms_sparse_attn_median": r["ms_sparse_attn_median"], "roofline": r["roofline"],
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


def _oracle_decode_row(s):
    """Worker: selection + attention of sequence s's first new token."""
    from threadpoolctl import threadpool_limits

    import oracle.reference as R
    c = _ORACLE
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        sel, _ = R.select_token(c["q"][s], c["t"], c["KC1"][s], c["KC2"][s], c["G"], c["p"])
        R.attend_token(c["q"][s], c["t"], c["Kf"][s], c["Vf"][s], sel, c["G"], c["p"])
        return time.perf_counter() - t0


def cpu_baseline_decode(inp, batch, len0, h_q, h_kv, lse_mode):
    """The fp64 oracle on the first decode step: the caches' compressed keys
    are built first (a one-time cost, not counted), then the selection and
    attention of every sequence's new token run in forked worker processes
    (one BLAS thread each), timed as wall time for the whole batch."""
    import multiprocessing as mp

    import oracle.reference as R
    cores = host_cores()
    p = R.Params(lse_mode=lse_mode, round_kc=True)
    K = [np.concatenate([inp.k_cache[s, :len0], inp.k_steps[0, s][None]]) for s in range(batch)]
    V = [np.concatenate([inp.v_cache[s, :len0], inp.v_steps[0, s][None]]) for s in range(batch)]
    _ORACLE.update(q=inp.q_steps[0], t=len0, G=h_q // h_kv, p=p,
                   KC1=[R.compress_keys(x, 32, 16, True) for x in K],
                   KC2=[R.compress_keys(x, 128, 64, True) if lse_mode == "approx" else None for x in K],
                   Kf=[R.as_f64(x) for x in K], Vf=[R.as_f64(x) for x in V])
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(min(cores, batch)) as pool:
        times = pool.map(_oracle_decode_row, range(batch))
    wall = time.perf_counter() - t0
    _ORACLE.clear()
    return {"value": batch / wall, "unit": "tokens/s", "cores": min(cores, batch), "kind": "oracle",
            "cpu_model": cpu_model(), "value_1core": batch / float(np.sum(times)),
            "sample": f"fp64 oracle: selection + attention of the new token of all {batch} sequences "
                      f"at position {len0} on {min(cores, batch)} worker processes (1 BLAS thread "
                      f"each), {wall:.2f} s wall including the pool start; cache compression not "
                      f"counted"}


def bench_varlen(args):
    """Varlen prefill: 65536 packed tokens, lengths drawn from the 0-4K, 4-12K,
    12-24K and 24-32K buckets; sequences <= 8192 take dense attention, the
    rest the sparse path (one SwitchPlan call per step)."""
    import torch

    from trainable_block_sparse_compress_amd import datagen as D
    from trainable_block_sparse_compress_amd import pipeline as P

    h_q, h_kv, d = 32, 2, 128
    lengths = D.varlen_lengths(5)
    print(f"[bench] varlen inputs: {len(lengths)} sequences", file=sys.stderr, flush=True)
    inp = D.make_prefill(5, lengths, h_q, h_kv, d)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    cfg = P.SparseConfig(lse_mode=args.lse)
    plan = P.SwitchPlan(lengths, h_q, h_kv, cfg)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        plan.run(q, k, v, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        plan.run(q, k, v, out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    total = sum(lengths)
    flops = 0.0
    for n in lengths:
        if n <= cfg.threshold:
            flops += 4.0 * d * h_q * n * (n + 1) / 2
        else:
            w = algorithmic_work(n, h_q, h_kv, d)
            flops += w["attn_flops"] + w["blocks_flops"] + (
                w["lse_exact_flops"] if args.lse == "exact" else w["lse_approx_flops"])
    tf = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": "varlen prefill tokens/s (65536 packed tokens, 0-32K mix, 32q/2kv, d128)",
        "value": total / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic: seeded i.i.d. N(0,1) bf16 Q/K/V",
        "config": {"workload": f"varlen prefill, {len(lengths)} sequences, {total} tokens "
                               "(<= 8192 dense, longer sparse |I| = 96)",
                   "lengths": lengths, "lse": args.lse},
        "roofline": {"bound": "mfma", "kernel": "whole step (all kernels)", "achieved": tf,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                     "traffic": None},
    }
    print(json.dumps(res), flush=True)


def bench_dense(args):
    """The switch's short path alone: a packed batch of sequences at the
    dense threshold (8192 tokens each unless --seq is lowered; 65536 tokens
    in all) through dense causal attention (the library transposes V into
    its workspace on every call, as the switch does)."""
    import torch

    from trainable_block_sparse_compress_amd import datagen as D
    from trainable_block_sparse_compress_amd import pipeline as P

    h_q, h_kv, d = 32, 2, 128
    cfg = P.SparseConfig()
    n = min(args.seq, cfg.threshold)
    lengths = [n] * max(1, 65536 // n)
    print(f"[bench] dense inputs: {len(lengths)} x {n}", file=sys.stderr, flush=True)
    inp = D.make_prefill(6, lengths, h_q, h_kv, d)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    starts = [i * n for i in range(len(lengths))]
    plan = P.DensePlan(starts, lengths, starts, lengths, q.shape[0], h_q, h_kv, cfg)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        plan.run(q, k, v, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        plan.run(q, k, v, out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    total = sum(lengths)
    flops = sum(4.0 * d * h_q * m * (m + 1) / 2 for m in lengths)
    tf = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": f"dense causal prefill tokens/s ({len(lengths)} x {n} packed tokens, 32q/2kv, d128)",
        "value": total / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic: seeded i.i.d. N(0,1) bf16 Q/K/V",
        "config": {"workload": f"dense causal attention (the switch's short path), {len(lengths)} "
                               f"sequences of {n} tokens", "lengths": lengths},
        "roofline": {"bound": "mfma", "kernel": "infllmv2_dense_attn (V transposition + attn_kernel)",
                     "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "traffic": None},
    }
    print(json.dumps(res), flush=True)


def sweep_split(n_sel):
    """Selection size |I| -> (n_init, n_local, n_topk): one init block, a
    third of |I| as the local window (32 of 96 at the headline size), the
    rest top-k."""
    n_local = n_sel // 3
    return 1, n_local, n_sel - 1 - n_local


def bench_sweep(args):
    """The prefill path at several selection sizes |I| (the pages compare the
    kernel against dense attention at 16 selected blocks), each against the
    dense causal kernel at the same length.  Per |I|: compress_k +
    select_blocks + sparse_attn timed with HIP events, algorithmic flops of
    the attention kernel, and its speedup over the dense kernel."""
    import torch

    from trainable_block_sparse_compress_amd import binding as B
    from trainable_block_sparse_compress_amd import datagen as D
    from trainable_block_sparse_compress_amd import pipeline as P

    n, h_q, h_kv, d = args.seq, 32, 2, 128
    sizes = [int(x) for x in args.sel.split(",") if x.strip()]
    print(f"[bench] sweep inputs n={n} |I| in {sizes}", file=sys.stderr, flush=True)
    inp = D.make_prefill(3, n, h_q, h_kv, d, n_needles=32)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    vt = v.permute(1, 2, 0).contiguous().view(h_kv, d, 1, n)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    base = P.SparseConfig(lse_mode=args.lse)
    dplan = P.DensePlan([0], [n], [0], [n], n, h_q, h_kv, base, "cuda", d)
    print("[bench] dense kernel", file=sys.stderr, flush=True)
    dms = timed(lambda: B.dense_attn(q, k, vt, dplan.cu_q, dplan.used_q, dplan.cu_k,
                                     dplan.used_k, 1, n, n, base.scale(d), out, None, None,
                                     v_seq_stride=n), max(1, args.dense_steps or 2))
    dflops = 4.0 * d * h_q * (n * (n + 1) / 2)
    rows = []
    for n_sel in sizes:
        ni, nl, nt = sweep_split(n_sel)
        cfg = P.SparseConfig(n_init=ni, n_local=nl, n_topk=nt, lse_mode=args.lse)
        plan = P.SparsePlan([0], [n], [0], [n], n, h_q, h_kv, cfg)
        print(f"[bench] |I| = {n_sel} ({ni} + {nl} + {nt})", file=sys.stderr, flush=True)
        for _ in range(args.warmup):
            plan.compress(k)
            plan.select(q)
        run_attn = lambda: B.sparse_attn(q, k, vt, plan.cu_q, plan.used_q, plan.cu_k,
                                         plan.used_k, 1, n, n, plan.block_idx, cfg.n_init,
                                         cfg.n_local, cfg.scale(d), out, None, None,
                                         v_seq_stride=n)
        ms_c = timed(lambda: plan.compress(k), args.steps)
        ms_s = timed(lambda: plan.select(q), args.steps)
        ms_a = timed(run_attn, args.steps)
        w = algorithmic_work(n, h_q, h_kv, d, ni, nl, nt)
        lse = w["lse_exact_flops"] if args.lse == "exact" else w["lse_approx_flops"]
        ms = ms_c + ms_s + ms_a
        rows.append({"n_sel": n_sel, "split": [ni, nl, nt], "ms_step": ms,
                     "tokens_per_s": n / (ms * 1e-3), "ms_compress_k": ms_c,
                     "ms_select_blocks": ms_s, "ms_sparse_attn": ms_a,
                     "attn_tflops": w["attn_flops"] / (ms_a * 1e-3) / 1e12,
                     "step_mfma_frac": (w["attn_flops"] + lse + w["blocks_flops"])
                     / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
                     "attn_speedup_vs_dense_kernel": dms / ms_a,
                     "step_speedup_vs_dense_kernel": dms / ms})
        del plan
    head = next((r for r in rows if r["n_sel"] == 96), rows[-1])
    res = {
        "metric": f"sparse-attn prefill tokens/s by selection size |I| at n={n} "
                  "(32q/2kv, d128) vs the dense kernel",
        "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) bf16 Q/K/V with 32 planted needle blocks",
        "config": {"workload": f"sparse prefill at |I| in {sizes}, one layer, n={n}",
                   "seq_len": n, "lse": args.lse, "value_is": f"|I| = {head['n_sel']}"},
        "dense_attn_ms": dms, "dense_attn_tflops": dflops / (dms * 1e-3) / 1e12,
        "sweep": rows,
        "roofline": {"bound": "mfma", "kernel": f"attn_kernel at |I| = {head['n_sel']}",
                     "achieved": head["attn_tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": head["attn_tflops"] / PEAK_BF16_TFLOPS,
                     "traffic": None},
    }
    print(json.dumps(res), flush=True)


def bench_backward(args):
    """Backward of the sparse attention at n = 131072 (32q/2kv, |I| = 96):
    the block lists come from select_blocks and the forward's output and LSE
    from sparse_attn, both outside the timed region; one step is one
    infllmv2_sparse_attn_bwd call (dq, dk, dv from a seeded upstream
    gradient).  Algorithmic flops: five products of 2*d per (row, head,
    visible key): S, dP, dV, dK, dQ (the dQ pass recomputing S and dP is not
    counted)."""
    import torch

    from trainable_block_sparse_compress_amd import binding as B
    from trainable_block_sparse_compress_amd import datagen as D
    from trainable_block_sparse_compress_amd import pipeline as P

    n, h_q, h_kv, d = args.seq, 32, 2, 128
    print(f"[bench] backward inputs n={n}", file=sys.stderr, flush=True)
    inp = D.make_prefill(3, n, h_q, h_kv, d, n_needles=32)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    dout = dev(D.make_grad(46, n, h_q, d))
    vt = v.permute(1, 2, 0).contiguous().view(h_kv, d, 1, n)
    cfg = P.SparseConfig(lse_mode=args.lse)
    plan = P.SparsePlan([0], [n], [0], [n], n, h_q, h_kv, cfg)
    plan.compress(k)
    plan.select(q)
    out = torch.empty_like(q)
    lse = torch.empty((h_q, n), dtype=torch.float32, device="cuda")
    B.sparse_attn(q, k, vt, plan.cu_q, plan.used_q, plan.cu_k, plan.used_k, 1, n, n,
                  plan.block_idx, cfg.n_init, cfg.n_local, cfg.scale(d), out, lse, None,
                  v_seq_stride=n)
    ws = torch.empty(B.attn_bwd_workspace(h_q, h_kv, 1, n, n, n, n, n_sel=plan.block_idx.shape[-1],
                                          n_init=cfg.n_init, n_local=cfg.n_local),
                     dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream()
    step = lambda: B.sparse_attn_bwd(q, k, v, out, lse, dout, plan.cu_q, plan.used_q, plan.cu_k,
                                     plan.used_k, 1, n, n, plan.block_idx, cfg.n_init,
                                     cfg.n_local, cfg.scale(d), dq, dk, dv, ws)
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    print("[bench] timed steps", file=sys.stderr, flush=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = 2.5 * algorithmic_work(n, h_q, h_kv, d)["attn_flops"]
    tf = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": "sparse-attn backward tokens/s @128K (32q/2kv, d128, |I|=96; dq, dk, dv)",
        "value": n / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) bf16 Q/K/V (32 needle blocks) and upstream "
                "gradient",
        "config": {"workload": f"sparse attention backward, one layer, n={n}", "seq_len": n,
                   "h_q": h_q, "h_kv": h_kv, "head_dim": d, "n_init": cfg.n_init,
                   "n_local": cfg.n_local, "n_topk": cfg.n_topk},
        "roofline": {"bound": "mfma", "kernel": "whole backward (infllmv2_sparse_attn_bwd)",
                     "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "traffic": None},
    }
    print(json.dumps(res), flush=True)


def bench_layer(args):
    """One attention layer of the 8B GQA shape the pages evaluate (hidden
    4096, 32 query heads, 2 KV heads, head_dim 128) at prefill length n:
    Q/K/V projections of a seeded hidden state (random weights; library
    GEMMs), then either the sparse path (compress_k, select_blocks,
    sparse_attn) or the dense kernel, then the output projection.  Time to
    first token of one layer, sparse against dense (the pages' end-to-end
    prefill comparison measures whole models; FFN and norms are not part of
    the attention path and are left out)."""
    import torch

    from trainable_block_sparse_compress_amd import binding as B
    from trainable_block_sparse_compress_amd import pipeline as P

    n, hidden, h_q, h_kv, d = args.seq, 4096, 32, 2, 128
    print(f"[bench] layer inputs n={n}", file=sys.stderr, flush=True)
    gen = torch.Generator(device="cuda").manual_seed(11)
    bf = torch.bfloat16
    x = torch.randn((n, hidden), generator=gen, device="cuda", dtype=torch.float32).to(bf)
    w = lambda o: (torch.randn((hidden, o), generator=gen, device="cuda", dtype=torch.float32)
                   / math.sqrt(hidden)).to(bf)
    wq, wk, wv = w(h_q * d), w(h_kv * d), w(h_kv * d)    # stored [in, out]: no transposed operand
    wo = (torch.randn((h_q * d, hidden), generator=gen, device="cuda", dtype=torch.float32)
          / math.sqrt(h_q * d)).to(bf)
    cfg = P.SparseConfig(lse_mode=args.lse)
    plan = P.SparsePlan([0], [n], [0], [n], n, h_q, h_kv, cfg)
    dplan = P.DensePlan([0], [n], [0], [n], n, h_q, h_kv, cfg, "cuda", d)
    ws = torch.empty(max(1, B.attn_workspace(h_q, h_kv, 1, n, n, n, n_sel=cfg.n_sel,
                                             n_init=cfg.n_init, n_local=cfg.n_local)),
                     dtype=torch.uint8, device="cuda")
    wsd = torch.empty(max(1, B.attn_workspace(h_q, h_kv, 1, n, n, n)), dtype=torch.uint8,
                      device="cuda")
    out = torch.empty((n, h_q, d), dtype=bf, device="cuda")
    stream = torch.cuda.current_stream()

    def layer(sparse):
        q = (x @ wq).view(n, h_q, d)
        k = (x @ wk).view(n, h_kv, d)
        v = (x @ wv).view(n, h_kv, d)
        if sparse:
            plan.compress(k)
            plan.select(q)
            B.sparse_attn(q, k, v, plan.cu_q, plan.used_q, plan.cu_k, plan.used_k, 1, n, n,
                          plan.block_idx, cfg.n_init, cfg.n_local, cfg.scale(d), out, None, ws)
        else:
            B.dense_attn(q, k, v, dplan.cu_q, dplan.used_q, dplan.cu_k, dplan.used_k, 1, n, n,
                         cfg.scale(d), out, None, wsd)
        return out.view(n, h_q * d) @ wo

    def timed(sparse, reps):
        layer(sparse)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            layer(sparse)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    print("[bench] sparse layer", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        layer(True)
    ms_sparse = timed(True, args.steps)
    print("[bench] dense layer", file=sys.stderr, flush=True)
    ms_dense = timed(False, max(1, args.dense_steps or 2))
    proj_flops = 2.0 * n * hidden * (h_q * d + 2 * h_kv * d) + 2.0 * n * h_q * d * hidden
    res = {
        "metric": f"attention-layer prefill tokens/s at n={n} (hidden 4096, 32q/2kv, d128, "
                  "|I|=96, with Q/K/V/O projections)",
        "value": n / (ms_sparse * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_sparse, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) hidden state, random projection weights",
        "config": {"workload": f"one attention layer (projections + sparse path), n={n}",
                   "seq_len": n, "hidden": hidden, "h_q": h_q, "h_kv": h_kv, "head_dim": d,
                   "lse": args.lse},
        "ms_dense_layer": ms_dense, "layer_speedup_vs_dense": ms_dense / ms_sparse,
        "projection_flops": proj_flops,
        "roofline": None,
    }
    print(json.dumps(res), flush=True)



def bench_layer_decode(args):
    """One attention layer of the 8B GQA shape (hidden 4096, 32q/2kv, d128)
    in decode, time per output token: batch 16, a 128K-token cache per
    sequence; per step the Q/K/V projections of a seeded hidden state
    (random weights, library GEMMs), the cache append of the new K and V
    (one scatter each, positions from the device lengths), the sparse decode
    step (incremental compress_k, select_blocks, sparse_attn) or our dense
    kernel over the whole cache, then the output projection.  Every step is
    timed with HIP events, launched eagerly."""
    import torch

    from trainable_block_sparse_compress_amd import binding as B
    from trainable_block_sparse_compress_amd import datagen as D
    from trainable_block_sparse_compress_amd import pipeline as P

    batch, len0, hidden, h_q, h_kv, d = DECODE_BATCH, args.seq, 4096, 32, 2, 128
    steps, warmup = args.decode_steps, 8
    print(f"[bench] layer decode inputs batch={batch} cache={len0}", file=sys.stderr, flush=True)
    inp = D.make_decode(4, batch, len0, 1, h_q, h_kv, d, n_needles=32)
    cap = (len0 + warmup + steps + 63) // 64 * 64
    cfg = P.SparseConfig(lse_mode=args.lse)
    gen = torch.Generator(device="cuda").manual_seed(12)
    bf = torch.bfloat16
    w = lambda i, o: (torch.randn((i, o), generator=gen, device="cuda", dtype=torch.float32)
                      / math.sqrt(i)).to(bf)
    wq, wk, wv, wo = w(hidden, h_q * d), w(hidden, h_kv * d), w(hidden, h_kv * d), w(h_q * d, hidden)
    xs = torch.randn((warmup + steps, batch, hidden), generator=gen, device="cuda",
                     dtype=torch.float32).to(bf)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    stream = torch.cuda.current_stream()
    seq = torch.arange(batch, device="cuda")
    out = torch.empty((batch, h_q, d), dtype=bf, device="cuda")

    def run(sparse):
        dec = P.DecodeState(batch, cap, h_q, h_kv, cfg)
        for s in range(batch):
            dec.fill_one(s, dev(inp.k_cache[s, :len0]), dev(inp.v_cache[s, :len0]))
        dec.compress_all()
        dcu = dec.cu_k
        dws = None
        if not sparse:
            dws = torch.empty(max(1, B.attn_workspace(h_q, h_kv, batch, 1, cap, batch,
                                                      v_seq_stride=cap)), dtype=torch.uint8,
                              device="cuda")
        times = []
        for i in range(warmup + steps):
            old = list(dec.lens)
            dec.lens = [x + 1 for x in dec.lens]
            pos = dec.used_k.clone()                 # device lengths before the append
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            x = xs[i]
            q = (x @ wq).view(batch, h_q, d)
            k_new = (x @ wk).view(batch, h_kv, d)
            v_new = (x @ wv).view(batch, h_kv, d)
            dec.k_cache.index_copy_(0, dcu.long() + pos.long(), k_new)
            dec.vt_cache[:, :, seq, pos.long()] = v_new.permute(1, 2, 0)
            dec.step_prepare(old)
            if sparse:
                dec.step(q, out, max(dec.lens))
            else:
                B.dense_attn(q, dec.k_cache, dec.vt_cache, dec.cu_q, dec.used_q, dec.cu_k,
                             dec.used_k, batch, 1, max(dec.lens), cfg.scale(d), out, None, dws,
                             v_seq_stride=cap)
            y = out.view(batch, h_q * d) @ wo
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= warmup:
                times.append(e0.elapsed_time(e1))
        del dec
        torch.cuda.empty_cache()
        return float(np.mean(times)), y

    print("[bench] sparse layer decode", file=sys.stderr, flush=True)
    ms_sparse, _ = run(True)
    print("[bench] dense layer decode", file=sys.stderr, flush=True)
    ms_dense, _ = run(False)
    res = {
        "metric": f"attention-layer decode tokens/s (time per output token; batch {batch}, "
                  f"{len0}-token cache, hidden 4096, 32q/2kv, d128, |I|=96, with Q/K/V/O projections)",
        "value": batch / (ms_sparse * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_sparse, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) cache and hidden states, random projection weights",
        "config": {"workload": f"one attention layer in decode (projections, cache append, sparse "
                               f"step, output projection), batch {batch}, cache {len0}",
                   "hidden": hidden, "h_q": h_q, "h_kv": h_kv, "head_dim": d, "lse": args.lse,
                   "launch": "eager"},
        "ms_dense_layer": ms_dense, "layer_speedup_vs_dense": ms_dense / ms_sparse,
        "roofline": None,
    }
    print(json.dumps(res), flush=True)



def bench_unfused(args):
    """The fusion ablation of the selection: select_blocks (group sum fused
    into the score kernel, block scores only reach HBM) against
    select_blocks_unfused (every head's stage-1 probabilities written to HBM
    and read back for the group sum and max pool), at n = 32768 and at
    --seq, exact LSE, 32q/2kv, |I| = 96.  HIP-event times per call, the
    S_C1 bytes the unfused path writes and reads, and the share of
    (row, group) lists the two produce identically."""
    import torch

    from trainable_block_sparse_compress_amd import datagen as D
    from trainable_block_sparse_compress_amd import pipeline as P

    h_q, h_kv, d = 32, 2, 128
    stream = torch.cuda.current_stream()
    rows = []
    for n in sorted({32768, args.seq}):
        print(f"[bench] unfused ablation n={n}", file=sys.stderr, flush=True)
        inp = D.make_prefill(3 if n == 131072 else 2, n, h_q, h_kv, d,
                             n_needles=32 if n == 131072 else 8)
        dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
        q, k = dev(inp.q), dev(inp.k)
        cfg = P.SparseConfig(lse_mode=args.lse)
        res = {}
        idx = {}
        for unfused in (False, True):
            plan = P.SparsePlan([0], [n], [0], [n], n, h_q, h_kv, cfg, unfused_select=unfused)
            plan.compress(k)
            for _ in range(args.warmup):
                plan.select(q)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                plan.select(q)
            e1.record(stream)
            torch.cuda.synchronize()
            res[unfused] = e0.elapsed_time(e1) / args.steps
            idx[unfused] = plan.block_idx.cpu().numpy()
            del plan
            torch.cuda.empty_cache()
        t = np.arange(n)
        bt = t // 64
        scored = bt - 32 - 1 + 1 > 63
        nv = np.clip((t - 31) // 16 + 1, 0, None)
        sc1 = float(4 * h_q * nv[scored].sum())
        rows.append({"n": n, "ms_select_fused": res[False], "ms_select_unfused": res[True],
                     "unfused_over_fused": res[True] / res[False],
                     "fused_time_cut": 1.0 - res[False] / res[True],
                     "s_c1_bytes_written": sc1, "s_c1_bytes_read": sc1,
                     "s_c1_gbs": 2 * sc1 / (res[True] * 1e-3) / 1e9,
                     "identical_lists": float(np.mean(np.all(idx[False] == idx[True], axis=2)))})
    head = rows[-1]
    print(json.dumps({
        "metric": "block selection ms per call, group sum fused into the score kernel vs unfused",
        "value": head["ms_select_fused"], "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_select_fused"], "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) bf16 Q/K with planted needle blocks",
        "config": {"workload": f"select_blocks fused vs unfused, n in {[r['n'] for r in rows]}",
                   "h_q": h_q, "h_kv": h_kv, "lse": args.lse}, "ablation": rows, "roofline": None,
    }), flush=True)


if __name__ == "__main__":
    main()

"""Decode-attention benchmark of the JSSA sparse path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole sparse hot path over one batch: subspace
scores -> per-KV-head top-k -> gather-free indexed split-K attention ->
log-sum-exp combine, for all B sequences of one layer, inputs resident in HBM.
The same run times the in-library dense full-KV step and the gather ablation
on the same inputs, and the fp64 CPU oracle on a bounded sample of the same
workload. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_128k_b16",
                    choices=["gqa_128k_b16", "gqa_128k_b4", "llama3.1-8b_layer_32k", "qwen3-14b_paged_ragged",
                             "deepseek-v3_mla_128k"])
    ap.add_argument("--k", type=int, default=0, help="override the budget (paged workload sweep)")
    ap.add_argument("--splits", type=int, default=0, help="splits of the selected set (0: by k)")
    ap.add_argument("--dense-splits", type=int, default=64)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-compare", action="store_true", help="skip the dense and gather comparisons")
    ap.add_argument("--no-calib", action="store_true", help="skip the subspace-calibration leg")
    ap.add_argument("--no-topdelta", action="store_true", help="skip the top-delta leg")
    ap.add_argument("--no-screen", action="store_true", help="skip the lossless-screening leg")
    ap.add_argument("--graph", action="store_true", help="time HIP graph replays of the step instead of eager launches")
    return ap.parse_args()


def workload(name: str):
    from dataclasses import replace
    from token_level_sparse_amd import synth
    if name == "gqa_128k_b16":
        return synth.BATCHED_128K
    if name == "gqa_128k_b4":
        return replace(synth.BATCHED_128K, B=4, name="gqa_128k_b4")
    if name == "llama3.1-8b_layer_32k":
        return synth.LLAMA8B_32K
    if name == "qwen3-14b_paged_ragged":
        return synth.PAGED_QWEN14B
    return synth.MLA_DSV3


FLUSH_BYTES = 512 << 20          # > 2x the 256 MB MALL: evicts every cache level


class Flush:
    """Reads a 512 MiB buffer on the launch stream (a sum over it): run before
    a timed step, outside its events, so that the step finds nothing of its
    working set in the L2 caches or the MALL (as in a decode loop, where other
    layers run between two steps of one layer). A read leaves the caches
    clean, so no write-back of the flush itself overlaps the step."""

    def __init__(self, torch):
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.torch = torch

    def __call__(self):
        self.sink = self.torch.sum(self.buf)


def _pct(xs, q):
    return float(np.percentile(np.asarray(xs, np.float64), q))


def summary(us):
    """median / p10 / p90 / mean of a list of microsecond timings."""
    return {"median_us": round(_pct(us, 50), 2), "p10_us": round(_pct(us, 10), 2),
            "p90_us": round(_pct(us, 90), 2), "mean_us": round(float(np.mean(us)), 2), "n": len(us)}


def time_steps(fns, steps, warmup, torch, stream, flush=None, graph=None):
    """The step protocol. warmup untimed steps, then `steps` timed ones; each
    timed step is preceded by a cache flush (outside its timing) and bracketed
    by one HIP event pair on the launch stream. Returns (per-step
    microseconds, wall seconds of the timed region, which includes the
    flushes). The region is bracketed by device synchronisation. When
    `graph` (a captured torch CUDAGraph of the same stages) is given, each
    step is one replay of it."""
    run = graph.replay if graph is not None else (lambda: [f() for f in fns])
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        if flush is not None:
            flush()
        ev[s][0].record(stream)
        run()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) * 1e3 for a, b in ev], wall


def time_stages(fns, steps, torch, stream, flush=None):
    """Per-stage microseconds: like time_steps, with an event pair around
    every stage (a separate pass, so that the extra events do not touch the
    step timing). Returns one list of per-step times per stage."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    for s in range(steps):
        if flush is not None:
            flush()
        ev[s][0].record(stream)
        for i, f in enumerate(fns):
            f()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    return [[ev[s][i].elapsed_time(ev[s][i + 1]) * 1e3 for s in range(steps)] for i in range(len(fns))]


def time_warm(fns, steps, torch):
    """Back-to-back steps with nothing between them (caches stay warm):
    wall seconds for `steps` steps, bracketed by device synchronisation."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def time_loop(fns, steps, warmup, torch, stream, graph=None, flush=None):
    """(seconds per step x steps, per-stage median microseconds) of the
    flushed protocol, for the comparison legs."""
    us, _ = time_steps(fns, steps, warmup, torch, stream, flush=flush, graph=graph)
    st = time_stages(fns, steps, torch, stream, flush=flush)
    return float(np.median(us)) * 1e-6 * steps, [float(np.median(x)) for x in st]


def time_launches(fn, n, torch, stream):
    """Mean microseconds per launch of `fn` over n back-to-back launches,
    from one HIP event pair on the launch stream."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle, untuned, timed on the host's cores. Runs
# before the GPU is touched: the worker processes are forked and inherit the
# generated inputs.
# ---------------------------------------------------------------------------
_CPU = {}


def _host_cores() -> int:
    """Cores this process may use, capped by JSSA_CPU_WORKERS (the GPU machine's
    share of its host is 16 cores)."""
    n = len(os.sched_getaffinity(0))
    return max(1, min(n, int(os.environ.get("JSSA_CPU_WORKERS", "16"))))


def _oracle_worker(args):
    """Time the oracle on `units` in one process with one BLAS thread. Every
    worker first builds its units' projected keys (set-up, not timed), then
    waits at the barrier, so that all workers time the same interval."""
    kind, units, reps = args
    from threadpoolctl import threadpool_limits
    from oracle import jssa_oracle as O
    inp, k = _CPU["inp"], _CPU["k"]
    cfg = inp.cfg
    scale = 1.0 / math.sqrt(cfg.d)
    with threadpool_limits(limits=1):
        prep = []
        for b, j in units:
            n = int(inp.seq_lens[b])
            K, V = inp.K[b, j, :n], inp.V[b, j, :n]
            hs = list(O.group_heads(j, cfg.G))
            Kp = O.project_keys(K, inp.P[j]) if kind == "sparse" else None
            prep.append((b, j, hs, K, V, Kp))
        if _CPU.get("barrier") is not None:
            _CPU["barrier"].wait()
        times, res = [], []
        for rep in range(reps):
            t0 = time.perf_counter()
            out = []
            for b, j, hs, K, V, Kp in prep:
                if kind == "sparse":
                    out.append(O.sparse_unit(inp.q[b, hs], inp.P[j], Kp, K, V, k, scale))
                else:
                    out.append(O.dense_unit(inp.q[b, hs], K, V, scale))
            times.append(time.perf_counter() - t0)
            if rep == 0:
                res = out
    return times, res


def _oracle_parallel(kind, units, workers, reps):
    """Wall seconds per pass (max over the workers, which start together) of
    the oracle over `units` split statically over `workers` processes, and
    the results in unit order."""
    import multiprocessing as mp
    slices = [units[i::workers] for i in range(workers)]
    ctx = mp.get_context("fork")
    _CPU["barrier"] = ctx.Barrier(workers)
    with ctx.Pool(workers) as pool:
        outs = pool.map(_oracle_worker, [(kind, sl, reps) for sl in slices], chunksize=1)
    _CPU["barrier"] = None
    per_pass = [max(o[0][r] for o in outs) for r in range(reps)]
    res = {}
    for sl, (_, r) in zip(slices, outs):
        res.update(dict(zip(sl, r)))
    return per_pass, [res[u] for u in units]


def cpu_baseline(inp, k, min_single_s=10.0):
    """The oracle's sparse step (score, top-k and attention from the
    projected key cache, for every (sequence, KV head) unit) on one thread
    and on all host cores, and its dense full-KV step on all cores over a
    sample of units."""
    cfg = inp.cfg
    _CPU["inp"], _CPU["k"] = inp, k
    units = [(b, j) for b in range(cfg.B) for j in range(cfg.Hkv)]
    cores = min(_host_cores(), len(units))
    # all cores, the whole step, three passes
    passes, res = _oracle_parallel("sparse", units, cores, 3)
    allc = float(np.median(passes))
    # one thread: a sample of units repeated until min_single_s, scaled to the step
    _CPU["barrier"] = None
    n1 = max(1, min(len(units), 16))
    t1, _ = _oracle_worker(("sparse", units[:n1], 1))
    reps = max(1, int(math.ceil(min_single_s / max(t1[0], 1e-3))))
    t1r, _ = _oracle_worker(("sparse", units[:n1], reps)) if reps > 1 else (t1, None)
    single = float(np.median(t1r)) * len(units) / n1
    # dense full-KV step on all cores, a sample of two units per core, scaled
    nd = min(len(units), 2 * cores)
    dsamp = units[:: max(1, len(units) // nd)][:nd]
    dpass, _ = _oracle_parallel("dense", dsamp, min(cores, nd), 1)
    dense = dpass[0] * len(units) / len(dsamp)
    return {
        "value": round(1.0 / allc, 4), "unit": "steps/s", "cores": cores, "kind": "oracle",
        "sample": f"the whole step ({len(units)} (sequence, KV-head) units, score + top-k + attention from the "
                  f"projected cache, fp64 numpy), split over {cores} processes with one BLAS thread each; "
                  f"median of 3 passes ({allc:.2f} s per step)",
        "single_thread": {"value": round(1.0 / single, 5), "unit": "steps/s", "cores": 1,
                          "sample": f"{n1} of {len(units)} units x {len(t1r)} passes on one thread, "
                                    f"{float(np.median(t1r)):.2f} s per pass, scaled to the step"},
        "dense_step": {"value": round(1.0 / dense, 5), "unit": "steps/s", "cores": min(cores, nd),
                       "sample": f"{len(dsamp)} of {len(units)} units of the full-KV step on "
                                 f"{min(cores, nd)} processes ({dpass[0]:.1f} s), scaled to the step"},
        "cpu": _cpu_model(), "host_cores_visible": len(os.sched_getaffinity(0)),
    }, res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the per-(sequence, KV-head) work would shard over batch or KV heads with no "
              "communication).", file=sys.stderr)
        sys.exit(2)
    from token_level_sparse_amd import synth
    cfg = workload(args.workload)
    if args.workload == "deepseek-v3_mla_128k":
        import torch
        from token_level_sparse_amd import pipeline
        torch.cuda.set_device(0)
        return bench_mla(args, cfg, torch, pipeline, synth, torch.cuda.current_stream())
    if args.k:
        from dataclasses import replace
        cfg = replace(cfg, k=args.k)
    t_gen = time.perf_counter()
    inp = synth.make_gqa(cfg)
    print(f"[bench] generated {cfg.name} in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    k = cfg.k
    cpu = None
    if not args.no_cpu and not cfg.paged:
        # before the GPU is touched: the oracle's worker processes are forked
        t_cpu = time.perf_counter()
        cpu = cpu_baseline(inp, k)
        print(f"[bench] cpu oracle leg done in {time.perf_counter() - t_cpu:.1f}s", file=sys.stderr, flush=True)

    import torch
    from token_level_sparse_amd import jssa, pipeline  # noqa: F401  (loads libjssa.so)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    c = pipeline.GqaCache(inp)
    c.project()
    torch.cuda.synchronize()
    print("[bench] projected keys on GPU", file=sys.stderr, flush=True)
    flush = Flush(torch)
    B, Hkv, Hq, d, r, T = cfg.B, cfg.Hkv, cfg.Hq, cfg.d, cfg.r, cfg.T
    tot_tok = int(np.sum(inp.seq_lens)) * Hkv            # (token, KV head) pairs scanned
    nsel = int(np.sum(np.minimum(k, inp.seq_lens))) * Hkv
    # the headline step: fused score -> top-k, then gather-free indexed attention
    sp = pipeline.SparseStep(c, k=k, S=args.splits or None, fused=True, keep_scores=False)
    S = sp.S
    graph = sp.capture() if args.graph else None
    step_us, wall = time_steps(sp.stages(), args.steps, args.warmup, torch, stream, flush=flush, graph=graph)
    med_us = float(np.median(step_us))
    steps_s = 1e6 / med_us
    print(f"[bench] sparse step (flushed caches) median {med_us:.1f} us", file=sys.stderr, flush=True)
    st_us = time_stages(sp.stages(), args.steps, torch, stream, flush=flush)
    warm_s = time_warm(sp.stages(), args.steps, torch)
    # the same step through the separate jssa_score / jssa_topk / jssa_indexed_decode entry points,
    # with the split count that fills the CUs when the attention runs as its own launch
    sp2 = pipeline.SparseStep(c, k=k, S=args.splits or None, fused=False)
    S2 = sp2.S
    sep_step, _ = time_steps(sp2.stages(), args.steps, args.warmup, torch, stream, flush=flush)
    st2_us = time_stages(sp2.stages(), args.steps, torch, stream, flush=flush)
    print(f"[bench] sparse (separate score, top-k) median {np.median(sep_step):.1f} us", file=sys.stderr,
          flush=True)

    kp_bytes = tot_tok * 2 * r
    q_bytes = B * Hq * d * 2
    p_bytes = Hkv * d * r * 4
    fused_bytes = kp_bytes + q_bytes + p_bytes            # the fused pass writes no score row
    score_bytes = kp_bytes + q_bytes + p_bytes + B * Hkv * T * 4
    topk_bytes = B * Hkv * T * 4 + B * Hkv * k * 4
    idx_bytes = nsel * 4 * d + B * Hkv * k * 4 + q_bytes + B * Hq * S * (d + 1) * 4
    comb_bytes = B * Hq * S * (d + 1) * 4 + B * Hq * (d + 1) * 4 if S > 1 else 0
    idx_bytes2 = idx_bytes + B * Hq * (S2 - S) * (d + 1) * 4
    comb_bytes2 = B * Hq * S2 * (d + 1) * 4 + B * Hq * (d + 1) * 4 if S2 > 1 else 0
    cand_bytes = B * Hkv * -(-T // 8192) * 8 * (k + 1)     # about k kept (key, index) pairs per 8192-token chunk

    def stage(us_list, nbytes):
        us = float(np.median(us_list))
        gbs = nbytes / (us * 1e-6) / 1e9 if us > 0 else None
        out = {"us": round(us, 2), "p10_us": round(_pct(us_list, 10), 2), "p90_us": round(_pct(us_list, 90), 2),
               "bytes": int(nbytes), "GB_s": round(gbs, 1) if gbs else None,
               "frac_hbm": round(gbs / HBM_PEAK_GBS, 3) if gbs else None}
        return out

    if S == 1:
        stages = {"score_topk_chunks": stage(st_us[0], fused_bytes),
                  "select_final_attend": stage(st_us[1], cand_bytes + idx_bytes)}
    else:
        stages = {"score_topk_chunks": stage(st_us[0], fused_bytes),
                  "select_final": stage(st_us[1], cand_bytes + B * Hkv * k * 4),
                  "indexed": stage(st_us[2], idx_bytes), "combine": stage(st_us[3], comb_bytes)}
    stages_split = {"S": S2, "score": stage(st2_us[0], score_bytes), "topk": stage(st2_us[1], topk_bytes),
                    "indexed": stage(st2_us[2], idx_bytes2),
                    "combine": stage(st2_us[3] if S2 > 1 else [0.0], comb_bytes2),
                    "step": summary(sep_step), "steps_per_s": round(1e6 / float(np.median(sep_step)), 2)}
    # the final stage warm (back-to-back launches over the same candidates), beside its cold time above
    if S == 1:
        warm_final = time_launches(sp.final_attend, args.steps, torch, stream)
        stages["select_final_attend"]["warm_back_to_back_us"] = round(warm_final, 2)
    warm_idx = time_launches(sp2.attend, args.steps, torch, stream)
    stages_split["indexed"]["warm_back_to_back_us"] = round(warm_idx, 2)
    # the dominant kernel: the chunk pass, its duration from the timed region's per-stage events
    kern_us = float(np.median(st_us[0]))
    achieved = fused_bytes / (kern_us * 1e-6) / 1e9
    kern_b2b = time_launches(sp.score_chunks, args.steps, torch, stream)
    # measured HBM bytes per launch of the chunk-pass kernel (rocprofv3 FETCH_SIZE + WRITE_SIZE,
    # calibrated on a plain copy), reported only while the kernel sources match the measurement
    traffic = None
    if cfg.name == "gqa_128k_b16" and not args.k:
        from token_level_sparse_amd.prof_summary import read_traffic
        t = read_traffic(os.path.join(ROOT, "profiles", "score_kernel_fused_gqa_128k_b16_hbm_traffic.txt"),
                         f"score_kernel<{r},0,true,false>")
        if t is not None:
            traffic = t["bytes"]
    # A1: one appended token per sequence (rewrites each sequence's last token with its own
    # values, so the cache is unchanged)
    pos = (c.seq_lens - 1).clamp(min=0).to(torch.int32).contiguous()
    if not c.paged:
        knew = c.K[torch.arange(B, device="cuda")[:, None], torch.arange(Hkv, device="cuda")[None, :],
                   pos.long()[:, None]].unsqueeze(2).contiguous()
        vnew = c.V[torch.arange(B, device="cuda")[:, None], torch.arange(Hkv, device="cuda")[None, :],
                   pos.long()[:, None]].unsqueeze(2).contiguous()
        app = lambda: jssa.jssa_append_kv(c.desc, c.K, c.V, c.Kp, knew, vnew, c.P, pos, 1)   # noqa: E731
        app_us, _ = time_steps([app], args.steps, 2, torch, stream, flush=flush)
        app_bytes = B * Hkv * (2 * d * 2 * 2 + r * 2) + Hkv * d * r * 4
        append = {"entry_point": "jssa_append_kv (n_new = 1)", **summary(app_us), "bytes": app_bytes,
                  "note": "A1, reported beside the step (outside it); flushed caches"}
    else:
        append = None

    result = {
        "metric": "sparse decode-attn steps/s at 128K,B=16 (Hkv=8,d=128,k=256); HBM GB/s vs peak",
        "value": round(steps_s, 2), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(med_us / 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "storage_dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "Hq": Hq, "Hkv": Hkv, "d": d, "T": T, "r": r, "k": k,
                   "S": S, "paged": bool(cfg.paged)},
        "timed_as": ("median of per-step HIP event times, each step after a 512 MiB cache flush outside its "
                     "events" + ("; each step one HIP graph replay" if graph is not None else "; eager launches")),
        "step_us": summary(step_us),
        "timed_region_wall_s": round(wall, 4),
        "warm_back_to_back": {"ms_per_step": round(warm_s / args.steps * 1e3, 4),
                              "steps_per_s": round(args.steps / warm_s, 2),
                              "note": "the same steps back to back, no flush (caches warm)"},
        "tokens_per_s": round(B * steps_s, 1),
        "context_tokens_scanned_per_s": round(tot_tok * steps_s, 1),
        "roofline": {"bound": "hbm", "kernel": "score_kernel (fused score + top-k chunk stage)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(fused_bytes), "duration_us": round(kern_us, 2),
                     "duration_source": "median of the chunk-pass HIP event pairs of the timed (flushed) steps, "
                                        "on its launch stream",
                     "duration_back_to_back_us": round(kern_b2b, 2)},
        "stages": stages,
        "separate_entry_points": stages_split,
        "append_kv": append,
    }

    if not args.no_compare:
        dn = pipeline.DenseStep(c, S=args.dense_splits)
        dsteps = max(3, args.steps // 5)
        d_step, _ = time_steps([dn.attend, dn.combine], dsteps, 2, torch, stream, flush=flush)
        dst_us = [float(np.median(x)) for x in time_stages([dn.attend, dn.combine], dsteps, torch, stream, flush)]
        dense_bytes = tot_tok * 4 * d + B * Hq * d * 2
        dmed = float(np.median(d_step))
        result["dense"] = {"ms_per_step": round(dmed / 1e3, 4), "steps_per_s": round(1e6 / dmed, 2),
                           "attend_us": round(dst_us[0], 2), "combine_us": round(dst_us[1], 2),
                           "GB_s": round(dense_bytes / (dst_us[0] * 1e-6) / 1e9, 1),
                           "frac_hbm": round(dense_bytes / (dst_us[0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 3)}
        result["speedup_vs_dense"] = round(dmed / med_us, 3)
        ga = pipeline.GatherStep(sp, S=max(S, 4))
        gsteps = max(3, args.steps // 5)
        g_step, _ = time_steps([sp.score_topk, ga.gather, ga.attend, ga.combine], gsteps, 2, torch, stream,
                               flush=flush)
        gst_us = [float(np.median(x)) for x in
                  time_stages([sp.score_topk, ga.gather, ga.attend, ga.combine], gsteps, torch, stream, flush)]
        sparse_attn_us = float(np.median(st2_us[2])) + (float(np.median(st2_us[3])) if S2 > 1 else 0.0)
        gather_attn_us = gst_us[1] + gst_us[2] + gst_us[3]
        dense_attn_us = dst_us[0] + dst_us[1]
        result["gather_ablation"] = {
            "ms_per_step": round(float(np.median(g_step)) / 1e3, 4), "gather_us": round(gst_us[1], 2),
            "dense_on_gathered_us": round(gst_us[2], 2), "combine_us": round(gst_us[3], 2),
            "attention_stage_us": {"gather_free": round(sparse_attn_us, 2), "gather": round(gather_attn_us, 2),
                                   "dense_full_kv": round(dense_attn_us, 2)},
            "attention_stage_speedup_vs_dense": {"gather_free": round(dense_attn_us / sparse_attn_us, 2),
                                                 "gather": round(dense_attn_us / gather_attn_us, 2)}}
        print("[bench] dense and gather comparisons done", file=sys.stderr, flush=True)

    if not args.no_topdelta:
        td = {}
        for delta in (1.0, 2.0, 3.0):
            tds = pipeline.TopDeltaStep(c, k, delta, 4, 64)
            tsteps = max(5, args.steps // 2)
            t_us, _ = time_steps([tds.run], tsteps, 2, torch, stream, flush=flush)
            cnt = tds.counts.cpu().numpy()
            td[f"delta_{delta:g}"] = {"ms_per_step": round(float(np.median(t_us)) / 1e3, 4),
                                      "steps_per_s": round(1e6 / float(np.median(t_us)), 2),
                                      "mean_kept": round(float(cnt.mean()), 1), "min_kept": int(cnt.min()),
                                      "max_kept": int(cnt.max())}
        result["topdelta"] = {"k_max": k, "n_sink": 4, "n_local": 64, "entry_point": "jssa_score_topdelta_attend",
                              "topk_step_ms": round(med_us / 1e3, 4), "by_delta": td}
        print("[bench] top-delta leg done", file=sys.stderr, flush=True)

    if not args.no_screen and not cfg.paged:
        from dataclasses import replace as _replace
        scr = {"seeds": "the previous step's selection (top-k under the query plus N(0, 0.1^2) noise)"}
        scr[cfg.name] = bench_screening(args, cfg, inp, c, torch, pipeline, synth, stream, flush)
        del_cfg = _replace(cfg, B=min(cfg.B, 4), key_model="clustered", name=cfg.name + "_clustered")
        inp_c = synth.make_gqa(del_cfg)
        c_c = pipeline.GqaCache(inp_c)
        c_c.project()
        scr[del_cfg.name] = bench_screening(args, del_cfg, inp_c, c_c, torch, pipeline, synth, stream, flush)
        del c_c, inp_c
        torch.cuda.empty_cache()
        result["screening"] = scr
        print("[bench] screening leg done", file=sys.stderr, flush=True)

    if not args.no_calib and not cfg.paged:
        result["calibration"] = bench_calibration(args, cfg, inp, c, sp, torch, pipeline, synth, jssa, stream)
        print("[bench] calibration leg done", file=sys.stderr, flush=True)

    if cpu is not None:
        cpu_info, res = cpu
        result["cpu_baseline"] = cpu_info
        result["oracle_check"] = oracle_check(inp, cfg, sp, res, k)
        print("[bench] oracle check done", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


def oracle_check(inp, cfg, sp, res, k):
    """Index and output parity of the timed step's result against the
    oracle, on every (sequence, KV head) unit: the index sets equal up to
    swaps within 1e-4 (relative) of the k-th score, and the outputs within
    2e-3 of the oracle's attention over the GPU's own set."""
    from oracle import jssa_oracle as O
    idx, out, lse = sp.idx.cpu().numpy(), sp.out.cpu().numpy(), sp.lse.cpu().numpy()
    units = [(b, j) for b in range(cfg.B) for j in range(cfg.Hkv)]
    swaps, max_err = 0, 0.0
    scale = 1.0 / math.sqrt(cfg.d)
    for (b, j), (s, oidx, o, ol) in zip(units, res):
        n = min(k, int(inp.seq_lens[b]))
        g = idx[b, j, :n]
        assert np.all(idx[b, j, n:] == -1) and np.all(np.diff(g) > 0), "index layout"
        diff = np.setxor1d(g, oidx[:n])
        if diff.size:
            sk = O.kth_score(s, k)
            assert np.all(np.abs(s[diff] - sk) <= 1e-4 * abs(sk)), f"index parity failed in bench at {(b, j)}"
            hs = list(O.group_heads(j, cfg.G))
            o, ol = O.attend(inp.q[b, hs], inp.K[b, j, g], inp.V[b, j, g], scale)
        hs = list(O.group_heads(j, cfg.G))
        err = np.abs(out[b, hs] - o) / np.maximum(1.0, np.abs(o))
        errl = np.abs(lse[b, hs] - ol) / np.maximum(1.0, np.abs(ol))
        assert err.max() <= 2e-3 and errl.max() <= 2e-3, f"output parity failed in bench at {(b, j)}"
        max_err = max(max_err, float(err.max()), float(errl.max()))
        swaps += diff.size // 2
    return {"units": len(units), "index_parity": "ok", "tie_swaps": int(swaps), "output_parity": "ok",
            "max_rel_err": max_err}


def bench_screening(args, cfg, inp, c, torch, pipeline, synth, stream, flush=None):
    """Lossless tile screening on one cache: the screened step (screen +
    chunk pass over the kept tiles + final select/attend) against the plain
    step, with the seeds taken from the previous step's selection."""
    k = cfg.k
    rng = np.random.default_rng(11)
    q_prev = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(inp.q) + 0.1 * rng.standard_normal(inp.q.shape))
    q_keep = c.q
    c.q = torch.from_numpy(q_prev.view(np.int16)).cuda()
    prev = pipeline.SparseStep(c, k=k, fused=True)
    prev.score_topk()
    torch.cuda.synchronize()
    c.q = q_keep
    seeds = prev.idx.clone()
    sc = pipeline.ScreenedStep(c, k, seeds)
    b_us = time_launches(sc.build_bounds, 3, torch, stream)
    # one appended token per sequence (its last): only its tile is rebuilt
    last_pos = (c.seq_lens - 1).clamp(min=0).to(torch.int32).contiguous()
    u_us = time_launches(lambda: sc.update_bounds(last_pos, 1), 20, torch, stream)
    plain = pipeline.SparseStep(c, k=k, S=1, fused=True, keep_scores=False)
    steps = max(5, args.steps // 2)
    p_total, _ = time_loop(plain.stages(), steps, 2, torch, stream, flush=flush)
    s_total, s_us = time_loop([sc.chunks, sc.final_attend], steps, 2, torch, stream, flush=flush)
    torch.cuda.synchronize()
    same = bool(torch.equal(sc.idx, plain.idx))
    kept = sc.kept_tiles.cpu().numpy().astype(np.int64)
    tiles = int(np.sum((inp.seq_lens.astype(np.int64) + 63) // 64)) * cfg.Hkv
    kept_frac = float(kept.sum()) / tiles
    read_bytes = int(kept.sum()) * 64 * 2 * cfg.r + tiles * 2 * cfg.r * 2 + seeds.numel() * (4 + 2 * cfg.r)
    return {"B": cfg.B, "plain_ms_per_step": round(p_total / steps * 1e3, 4),
            "screened_ms_per_step": round(s_total / steps * 1e3, 4),
            "screen_plus_chunks_us": round(s_us[0], 2), "final_attend_us": round(s_us[1], 2),
            "kept_tile_fraction": round(kept_frac, 4),
            "chunk_pass_bytes": {"plain": int(tiles * 64 * 2 * cfg.r), "screened": read_bytes},
            "bounds_build_us": round(b_us, 1), "bounds_update_one_token_us": round(u_us, 2),
            "indices_equal_plain": same}


def bench_calibration(args, cfg, inp, c, sp, torch, pipeline, synth, jssa, stream, n_queries=4096):
    """Offline subspace calibration on the benchmark's own cache: key second
    moments over every cached key (MFMA Gram kernel, HBM-bound), query second
    moments over n_queries synthetic decode queries, the host spectral step,
    then the recall of the exact (full-width) top-k by the calibrated basis
    against the random orthonormal one the timed step uses."""
    B, Hkv, Hq, d, r, k = cfg.B, cfg.Hkv, cfg.Hq, cfg.d, cfg.r, cfg.k
    ws = torch.empty(jssa.jssa_calib_workspace_size(c.desc), dtype=torch.uint8, device="cuda")
    Sk = torch.empty((Hkv, d, d), dtype=torch.float32, device="cuda")
    km = lambda: jssa.jssa_calib_key_moments(c.desc, c.K, Sk, ws)   # noqa: E731
    km_us = time_launches(km, max(5, args.steps // 5), torch, stream)
    k_bytes = int(np.sum(inp.seq_lens)) * Hkv * d * 2
    qs = torch.from_numpy(synth.gen_calib_queries(cfg, n_queries).view(np.int16)).cuda()
    Sq = torch.empty((Hkv, d, d), dtype=torch.float32, device="cuda")
    qws = torch.empty(jssa.jssa_calib_query_workspace_size(Hkv), dtype=torch.uint8, device="cuda")
    qm_us = time_launches(lambda: jssa.jssa_calib_query_moments(n_queries, Hq, Hkv, qs, Sq, qws), 5, torch, stream)
    torch.cuda.synchronize()
    Skh, Sqh = Sk.cpu().numpy(), Sq.cpu().numpy()
    t0 = time.perf_counter()
    P = np.stack([jssa.jssa_calib_projection(Sqh[j], Skh[j], r)[0] for j in range(Hkv)])
    host_ms = (time.perf_counter() - t0) * 1e3
    # selection with the calibrated basis (a second projected cache)
    cc = pipeline.GqaCache.__new__(pipeline.GqaCache)
    cc.__dict__.update(c.__dict__)
    cc.P = torch.from_numpy(P).cuda()
    cc.Kp = torch.empty_like(c.Kp)
    cc.project()
    cal = pipeline.SparseStep(cc, k=k, fused=True)
    cal.score_topk()
    # exact top-k: full-width scores (rank 128, P = I, K itself as the projected cache)
    eye = torch.eye(d, dtype=torch.float32, device="cuda").repeat(Hkv, 1, 1).contiguous()
    dx = jssa.gqa_desc(B, Hq, Hkv, d, cfg.T, seq_lens=c.seq_lens)
    idx_x = torch.empty((B, Hkv, k), dtype=torch.int32, device="cuda")
    wx = torch.empty(jssa.jssa_score_topk_workspace_size(dx, k), dtype=torch.uint8, device="cuda")
    jssa.jssa_score_topk(dx, c.q, eye, c.K, k, None, idx_x, wx)
    rnd = pipeline.SparseStep(c, k=k, fused=True)
    rnd.score_topk()
    torch.cuda.synchronize()
    gi, gx, gr = cal.idx.cpu().numpy(), idx_x.cpu().numpy(), rnd.idx.cpu().numpy()

    def recall(a, x):
        vals = []
        for b in range(B):
            for j in range(Hkv):
                ref = x[b, j][x[b, j] >= 0]
                vals.append(np.intersect1d(a[b, j], ref).size / max(1, ref.size))
        return float(np.mean(vals))
    del cc, cal
    gbs = k_bytes / (km_us * 1e-6) / 1e9
    return {"key_moments": {"us": round(km_us, 2), "bytes": k_bytes, "GB_s": round(gbs, 1),
                            "frac_hbm": round(gbs / HBM_PEAK_GBS, 3), "bound": "hbm",
                            "kernels": "gram_kernel + gram_reduce_kernel (one jssa_calib_key_moments call)"},
            "query_moments_us": round(qm_us, 2), "query_samples": n_queries,
            "host_spectral_ms": round(host_ms, 1), "rank": r,
            "recall_of_exact_topk": {"calibrated": round(recall(gi, gx), 4), "random": round(recall(gr, gx), 4),
                                     "k": k, "units": B * Hkv}}


def bench_mla(args, cfg, torch, pipeline, synth, stream):
    inp = synth.make_mla(cfg)
    S = args.splits or 16
    st = pipeline.MlaStep(inp, S=S)
    st.project()
    torch.cuda.synchronize()
    from token_level_sparse_amd import jssa
    c = cfg

    def absorb():
        jssa.jssa_mla_absorb_q(st.desc, st.q_nope, st.q_rope, st.W_uk, st.P, st.U, st.q_abs, st.q_sel, stream)

    def score_topk():
        jssa.jssa_mla_score_topk(st.desc, st.q_sel, st.Kp, st.k, st.scores, st.idx, st.ws, None, stream)

    def attend():
        jssa.jssa_mla_indexed_decode(st.desc, st.q_abs, st.latent, st.idx, st.k, st.S, st.scale, st.part_o,
                                     st.part_lse, stream)

    def combine_up():
        jssa.jssa_mla_combine_up_v(st.desc, st.S, st.part_o, st.part_lse, st.W_uv, st.out, st.lse, stream)

    flush = Flush(torch)
    fns = [absorb, score_topk, attend, combine_up]
    step_us, _ = time_steps(fns, args.steps, args.warmup, torch, stream, flush=flush)
    us = [float(np.median(x)) for x in time_stages(fns, args.steps, torch, stream, flush=flush)]
    names = ["absorb", "score_topk", "indexed_mfma", "combine_up_v"]
    total = float(np.median(step_us)) * 1e-6 * args.steps
    steps_s = args.steps / total
    core_flops = 2 * c.B * c.H * c.k * (2 * c.d_c + c.d_latent)       # QK^T (hi+lo) + PV
    res = {"metric": "MLA sparse decode steps/s (DeepSeek-V3-shaped, 128K, k=2048)", "value": round(steps_s, 2),
           "unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(total / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16-mfma/f32", "data": "synthetic",
           "config": {"workload": c.name, "B": c.B, "H": c.H, "T": c.T, "r": c.r, "k": c.k, "S": S},
           "step_us": summary(step_us), "timed_as": "median of flushed per-step HIP event times",
           "stages_us": {n: round(u, 2) for n, u in zip(names, us)},
           "indexed_mfma_TFLOP_s": round(core_flops / (us[2] * 1e-6) / 1e12, 2)}
    print(json.dumps(res), flush=True)


def _cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it, with its family / model /
    stepping numbers (a virtualised host may give only a generic name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break                                   # the first processor's block
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


if __name__ == "__main__":
    main()

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


def time_loop(fns, steps, warmup, torch, stream, graph=None):
    """Run `fns` (a list of stage callables) warmup + steps times. Returns
    (seconds of the timed steps, per-stage mean microseconds).

    The timed steps run back to back with nothing between them (bracketed by
    device synchronisation); when `graph` (a captured torch CUDAGraph of the
    same stages) is given, each step is one replay of it. The per-stage times
    come from a second pass of eager steps with an event pair around every
    stage on the launch stream."""
    run = graph.replay if graph is not None else (lambda: [f() for f in fns])
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    for s in range(steps):
        ev[s][0].record(stream)
        for i, f in enumerate(fns):
            f()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    stage_us = [float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)]) * 1e3)
                for i in range(len(fns))]
    return total, stage_us


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


def cpu_oracle_gqa(inp, k, units, min_seconds=10.0):
    """fp64 oracle sparse step (score, top-k, attention from the projected
    key cache) on a sample of (b, j) units, repeated until at least
    min_seconds of single-thread CPU time; returns (seconds, passes, the
    first pass's results)."""
    from threadpoolctl import threadpool_limits
    from oracle import jssa_oracle as O
    cfg = inp.cfg
    prepared = []
    for b, j in units:
        n = int(inp.seq_lens[b])
        K, V = inp.K[b, j, :n], inp.V[b, j, :n]
        prepared.append((b, j, K, V, O.project_keys(K, inp.P[j])))
    with threadpool_limits(limits=1):
        res, passes = None, 0
        t0 = time.perf_counter()
        while passes == 0 or time.perf_counter() - t0 < min_seconds:     # repeat the sample for a stable time
            out = []
            for b, j, K, V, Kp in prepared:
                hs = list(O.group_heads(j, cfg.G))
                out.append(O.sparse_unit(inp.q[b, hs], inp.P[j], Kp, K, V, k, 1 / math.sqrt(cfg.d)))
            res = res or out
            passes += 1
        dt = time.perf_counter() - t0
    return dt, passes, res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the per-(sequence, KV-head) work would shard over batch or KV heads with no "
              "communication).", file=sys.stderr)
        sys.exit(2)
    import torch
    from token_level_sparse_amd import jssa, pipeline, synth  # noqa: F401  (loads libjssa.so)

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    cfg = workload(args.workload)
    t_gen = time.perf_counter()
    if args.workload == "deepseek-v3_mla_128k":
        return bench_mla(args, cfg, torch, pipeline, synth, stream)
    if args.k:
        from dataclasses import replace
        cfg = replace(cfg, k=args.k)
    inp = synth.make_gqa(cfg)
    gen_s = time.perf_counter() - t_gen
    print(f"[bench] generated {cfg.name} in {gen_s:.1f}s", file=sys.stderr, flush=True)
    c = pipeline.GqaCache(inp)
    c.project()
    torch.cuda.synchronize()
    print("[bench] projected keys on GPU", file=sys.stderr, flush=True)
    k = cfg.k
    B, Hkv, Hq, d, r, T = cfg.B, cfg.Hkv, cfg.Hq, cfg.d, cfg.r, cfg.T
    tot_tok = int(np.sum(inp.seq_lens)) * Hkv            # (token, KV head) pairs scanned
    nsel = int(np.sum(np.minimum(k, inp.seq_lens))) * Hkv
    # the headline step: fused score -> top-k, then gather-free indexed attention
    sp = pipeline.SparseStep(c, k=k, S=args.splits or None, fused=True, keep_scores=False)
    S = sp.S
    # timed steps: eager launches (measured faster here than replaying a HIP graph of the same
    # launches, which --graph times instead; the eager time is then reported beside it)
    graph = sp.capture() if args.graph else None
    total, st_us = time_loop(sp.stages(), args.steps, args.warmup, torch, stream, graph=graph)
    total_eager = time_loop(sp.stages(), args.steps, args.warmup, torch, stream)[0] if graph is not None else total
    ms = total / args.steps * 1e3
    steps_s = args.steps / total
    print(f"[bench] sparse (fused score+top-k) {ms:.3f} ms/step", file=sys.stderr, flush=True)
    # the same step through the separate jssa_score / jssa_topk entry points
    sp2 = pipeline.SparseStep(c, k=k, S=S, fused=False)
    total2, st2_us = time_loop(sp2.stages(), args.steps, args.warmup, torch, stream)
    print(f"[bench] sparse (separate score, top-k) {total2 / args.steps * 1e3:.3f} ms/step", file=sys.stderr,
          flush=True)
    # fused stages: S == 1: [chunk pass (score stream + chunk select), final select + attention];
    # S > 1: [chunk pass, final select, indexed split attention, combine]
    chunk_us = st_us[0]
    if S == 1:
        final_attend_us = st_us[1]
    else:
        final_us, attn_us, comb_us = st_us[1], st_us[2], st_us[3]
    # the separate entry points: [jssa_score, jssa_topk, jssa_indexed_decode, (jssa_combine)]
    sep_attn_us = st2_us[2] + (st2_us[3] if S > 1 else 0.0)

    kp_bytes = tot_tok * 2 * r
    q_bytes = B * Hq * d * 2
    p_bytes = Hkv * d * r * 4
    fused_bytes = kp_bytes + q_bytes + p_bytes            # the fused pass writes no score row
    score_bytes = kp_bytes + q_bytes + p_bytes + B * Hkv * T * 4
    topk_bytes = B * Hkv * T * 4 + B * Hkv * k * 4
    idx_bytes = nsel * 4 * d + B * Hkv * k * 4 + q_bytes + B * Hq * S * (d + 1) * 4
    comb_bytes = B * Hq * S * (d + 1) * 4 + B * Hq * (d + 1) * 4 if S > 1 else 0

    def stage(us, nbytes):
        gbs = nbytes / (us * 1e-6) / 1e9 if us > 0 else None
        return {"us": round(us, 2), "bytes": int(nbytes), "GB_s": round(gbs, 1) if gbs else None,
                "frac_hbm": round(gbs / HBM_PEAK_GBS, 3) if gbs else None}

    cand_bytes = B * Hkv * -(-T // 8192) * 8 * (k + 1)     # about k kept (key, index) pairs per 8192-token chunk
    stages = {"score_topk_chunks": stage(chunk_us, fused_bytes)}
    if S == 1:
        stages["select_final_attend"] = stage(final_attend_us, cand_bytes + idx_bytes)
    else:
        stages["select_final"] = stage(final_us, cand_bytes + B * Hkv * k * 4)
        stages["indexed"] = stage(attn_us, idx_bytes)
        stages["combine"] = stage(comb_us, comb_bytes)
    stages_split = {"score": stage(st2_us[0], score_bytes), "topk": stage(st2_us[1], topk_bytes),
                    "indexed": stage(st2_us[2], idx_bytes),
                    "combine": stage(st2_us[3] if S > 1 else 0.0, comb_bytes),
                    "ms_per_step": round(total2 / args.steps * 1e3, 4),
                    "steps_per_s": round(args.steps / total2, 2)}
    # the dominant kernel's launch duration: back-to-back launches of the chunk pass
    kern_us = time_launches(sp.score_chunks, args.steps, torch, stream)
    achieved = fused_bytes / (kern_us * 1e-6) / 1e9
    # measured HBM bytes per launch of the chunk-pass kernel (rocprofv3 FETCH_SIZE + WRITE_SIZE,
    # calibrated on a plain copy), reported only while the kernel sources match the measurement
    traffic = None
    if cfg.name == "gqa_128k_b16" and not args.k:
        from token_level_sparse_amd.prof_summary import read_traffic
        t = read_traffic(os.path.join(ROOT, "profiles", "score_kernel_fused_gqa_128k_b16_hbm_traffic.txt"),
                         f"score_kernel<{r},0,true,false>")
        if t is not None:
            traffic = t["bytes"]

    result = {
        "metric": "sparse decode-attn steps/s at 128K,B=16 (Hkv=8,d=128,k=256); HBM GB/s vs peak",
        "value": round(steps_s, 2), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "storage_dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "Hq": Hq, "Hkv": Hkv, "d": d, "T": T, "r": r, "k": k,
                   "S": S, "paged": bool(cfg.paged)},
        "timed_as": "HIP graph replay of the step" if graph is not None else "eager launches",
        "eager_ms_per_step": round(total_eager / args.steps * 1e3, 4),
        "tokens_per_s": round(B * steps_s, 1),
        "context_tokens_scanned_per_s": round(tot_tok * steps_s, 1),
        "roofline": {"bound": "hbm", "kernel": "score_kernel (fused score + top-k chunk stage)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(fused_bytes), "duration_us": round(kern_us, 2),
                     "duration_source": f"HIP event pair around {args.steps} back-to-back jssa_score_topk_chunks "
                                        "launches on their stream"},
        "stages": stages,
        "separate_entry_points": stages_split,
    }

    if not args.no_compare:
        dn = pipeline.DenseStep(c, S=args.dense_splits)
        dsteps = max(3, args.steps // 5)
        dtotal, dst_us = time_loop([dn.attend, dn.combine], dsteps, 2, torch, stream)
        dense_bytes = tot_tok * 4 * d + B * Hq * d * 2
        result["dense"] = {"ms_per_step": round(dtotal / dsteps * 1e3, 4), "steps_per_s": round(dsteps / dtotal, 2),
                           "attend_us": round(dst_us[0], 2), "combine_us": round(dst_us[1], 2),
                           "GB_s": round(dense_bytes / (dst_us[0] * 1e-6) / 1e9, 1),
                           "frac_hbm": round(dense_bytes / (dst_us[0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 3)}
        result["speedup_vs_dense"] = round((dtotal / dsteps) / (total / args.steps), 3)
        ga = pipeline.GatherStep(sp, S=max(S, 4))
        gsteps = max(3, args.steps // 5)
        gtotal, gst_us = time_loop([sp.score_topk, ga.gather, ga.attend, ga.combine], gsteps, 2, torch, stream)
        sparse_attn_us = sep_attn_us                    # jssa_indexed_decode (+ combine) alone
        gather_attn_us = gst_us[1] + gst_us[2] + gst_us[3]
        dense_attn_us = dst_us[0] + dst_us[1]
        result["gather_ablation"] = {
            "ms_per_step": round(gtotal / gsteps * 1e3, 4), "gather_us": round(gst_us[1], 2),
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
            ttotal, _ = time_loop([tds.run], tsteps, 2, torch, stream)
            cnt = tds.counts.cpu().numpy()
            td[f"delta_{delta:g}"] = {"ms_per_step": round(ttotal / tsteps * 1e3, 4),
                                      "steps_per_s": round(tsteps / ttotal, 2),
                                      "mean_kept": round(float(cnt.mean()), 1), "min_kept": int(cnt.min()),
                                      "max_kept": int(cnt.max())}
        result["topdelta"] = {"k_max": k, "n_sink": 4, "n_local": 64, "entry_point": "jssa_score_topdelta_attend",
                              "topk_step_ms": round(ms, 4), "by_delta": td}
        print("[bench] top-delta leg done", file=sys.stderr, flush=True)

    if not args.no_screen and not cfg.paged:
        from dataclasses import replace as _replace
        scr = {"seeds": "the previous step's selection (top-k under the query plus N(0, 0.1^2) noise)"}
        scr[cfg.name] = bench_screening(args, cfg, inp, c, torch, pipeline, synth, stream)
        del_cfg = _replace(cfg, B=min(cfg.B, 4), key_model="clustered", name=cfg.name + "_clustered")
        inp_c = synth.make_gqa(del_cfg)
        c_c = pipeline.GqaCache(inp_c)
        c_c.project()
        scr[del_cfg.name] = bench_screening(args, del_cfg, inp_c, c_c, torch, pipeline, synth, stream)
        del c_c, inp_c
        torch.cuda.empty_cache()
        result["screening"] = scr
        print("[bench] screening leg done", file=sys.stderr, flush=True)

    if not args.no_calib and not cfg.paged:
        result["calibration"] = bench_calibration(args, cfg, inp, c, sp, torch, pipeline, synth, jssa, stream)
        print("[bench] calibration leg done", file=sys.stderr, flush=True)

    if not args.no_cpu:
        units = [(b, j) for b in range(min(2, B)) for j in range(Hkv)]
        dt, passes, res = cpu_oracle_gqa(inp, k, units)
        per_step = dt / passes * (B * Hkv) / len(units)
        result["cpu_baseline"] = {"value": round(1.0 / per_step, 5), "unit": "steps/s", "cores": 1, "kind": "oracle",
                                  "sample": f"{len(units)} of {B * Hkv} (sequence, KV-head) units of one step, "
                                            f"{passes} passes in {dt:.1f}s on one thread, scaled to a whole step",
                                  "cpu": _cpu_model()}
        idx = sp.idx.cpu().numpy()
        swaps = 0
        from oracle import jssa_oracle as O
        for (b, j), (s, oidx, o, lse) in zip(units, res):
            n = min(k, int(inp.seq_lens[b]))
            g = idx[b, j, :n]
            diff = np.setxor1d(g, oidx[:n])
            if diff.size:
                sk = O.kth_score(s, k)
                assert np.all(np.abs(s[diff] - sk) <= 1e-4 * abs(sk)), "index parity failed in bench"
            swaps += diff.size // 2
        result["oracle_check"] = {"units": len(units), "index_parity": "ok", "tie_swaps": int(swaps)}
        print("[bench] cpu oracle leg done", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


def bench_screening(args, cfg, inp, c, torch, pipeline, synth, stream):
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
    p_total, _ = time_loop(plain.stages(), steps, 2, torch, stream)
    s_total, s_us = time_loop([sc.chunks, sc.final_attend], steps, 2, torch, stream)
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
        jssa.jssa_mla_absorb_q(st.desc, st.q_nope, st.q_rope, st.W_uk, st.P, st.q_abs, st.q_sel, stream)

    def score():
        jssa.jssa_mla_score(st.desc, st.q_sel, st.Kp, st.scores, stream)

    def topk():
        jssa.jssa_topk(c.B, 1, c.T, st.seq_lens, st.scores, st.k, st.idx, st.ws, None, stream)

    def attend():
        jssa.jssa_mla_indexed_decode(st.desc, st.q_abs, st.latent, st.idx, st.k, st.S, st.scale, st.part_o,
                                     st.part_lse, stream)

    def combine():
        jssa.jssa_combine(c.B, c.H, st.S, c.d_latent, st.part_o, st.part_lse, st.o_lat, 0, st.lse, stream)

    def up():
        jssa.jssa_mla_up_v(st.desc, st.o_lat, st.W_uv, st.out, stream)

    total, us = time_loop([absorb, score, topk, attend, combine, up], args.steps, args.warmup, torch, stream)
    names = ["absorb", "score", "topk", "indexed_mfma", "combine", "up_v"]
    steps_s = args.steps / total
    core_flops = 2 * c.B * c.H * c.k * (2 * c.d_c + c.d_latent)       # QK^T (hi+lo) + PV
    res = {"metric": "MLA sparse decode steps/s (DeepSeek-V3-shaped, 128K, k=2048)", "value": round(steps_s, 2),
           "unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(total / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16-mfma/f32", "data": "synthetic",
           "config": {"workload": c.name, "B": c.B, "H": c.H, "T": c.T, "r": c.r, "k": c.k, "S": S},
           "stages_us": {n: round(u, 2) for n, u in zip(names, us)},
           "indexed_mfma_TFLOP_s": round(core_flops / (us[3] * 1e-6) / 1e12, 2)}
    print(json.dumps(res), flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()

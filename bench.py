"""Benchmark of the block-sparse cross-scale attention hot path on one MI355X.

One step = one pass of the CSLA hot path over the batch of the 2B-shaped last
scale: build the block mask and its kept-tile lists (varsparse_build_mask),
then block-sparse attention of the 64 x 64 query scale over the 10521-token
multi-scale cache (varsparse_attn_fwd), B = 2 (CFG pair), H = 16, d = 128,
bf16.  Inputs are synthetic (seeded spatial fields), resident in HBM before the
timed region.

value = effective TFLOP/s: 4 d |Q| |K| summed over the kept (query tile, key
tile) pairs with real token counts, per step, divided by the step time.  The
dense kernel written with the same tile engine is timed on the same tensors
for the speedup; the CS4A path (decision-scale scoring + selection + mapping +
attention at sides 40/48/64) is timed as a second line item.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch of the sparse attention kernel on this workload, from
# rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs scaled by a 256 MiB copy
# (x2.000 and x1.000), and its MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES
# over GRBM_GUI_ACTIVE / 8 x 1024 SIMDs), recorded with the SHA-256 of the
# kernel sources they were taken on; reported only while those sources are
# unchanged.
TRAFFIC = {"bytes": 469.7e6, "mfma_busy": 0.369, "sources_sha256": "26e5adec3ecd9226f3eed2be011dd45f12edb22b56727feabb445d4f3f8ea4a4"}
KERNEL_SOURCES = ("block_sparse_cross_csla_amd/csrc/attn_bf16.hip", "block_sparse_cross_csla_amd/csrc/common.h",
                  "block_sparse_cross_csla_amd/csrc/kernel_args.h")


def kernel_sources_sha256():
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # defaults: ~50 ms of warm-up brings the GPU to its steady clocks (a few
    # warm-up steps measure it still ramping, ~8% slower), ~35 ms timed
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-cs4a", action="store_true")
    p.add_argument("--no-high-res", action="store_true")
    p.add_argument("--no-sweep", action="store_true", help="skip the 8B-shaped budget sweep")
    # the GPU reaches steady clocks only after some hundreds of milliseconds of
    # load: steps are run for this long before the --warmup count, whatever
    # --warmup says, so that the timed steps and the per-kernel timings do not
    # measure the clock ramp
    p.add_argument("--settle-ms", type=float, default=400.0)
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-single", action="store_true",
                   help="skip the single-launch warm/cold timings (keeps counter runs to back-to-back launches)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    return p.parse_args()


def tile_sizes(sides, q_scale, t):
    """Token count of every key tile of scales 0..q_scale (id order)."""
    out = []
    for s in range(q_scale + 1):
        h = sides[s]
        nb = -(-h // t)
        for a in range(nb):
            for b in range(nb):
                out.append(min(t, h - a * t) * min(t, h - b * t))
    return np.array(out, np.int64)


def kept_flops(cnt, idx, sizes, q_tile_tokens, d, heads):
    """4 d |Q| |K| over the kept pairs of shared (heads > 0) or per-head lists."""
    cnt = cnt.reshape(-1, cnt.shape[-1]) if cnt.ndim > 1 else cnt[None]
    idx = idx.reshape(-1, *idx.shape[-2:]) if idx.ndim > 2 else idx[None]
    total = 0
    for c, ix in zip(cnt, idx):
        for r in range(c.shape[0]):
            total += int(sizes[ix[r, : c[r]]].sum())
    mult = heads if cnt.shape[0] == 1 else 1
    return 4.0 * d * q_tile_tokens * total * mult


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py runs on one GPU: the kernels use one device; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import block_sparse_cross_csla_amd as vs
    from varsparse_inputs import SpatialField, bf16_bits, round_bf16, workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(bf16_bits(x)).view(np.int16)).view(torch.bfloat16).to(dev)

    w = W.LAST_SCALE_2B
    f = SpatialField(w.seed, w.wid, w.B, w.H, w.d)
    k_np, v_np = f.keys_values(w.sides[: w.q_scale + 1], w.n_sink, largest_side=w.sides[w.q_scale])
    q_np = f.queries(w.sides[w.q_scale])
    q, k, v = to_dev(q_np), to_dev(k_np), to_dev(v_np)
    nqb, nkb, nq, nk = vs.geom_counts(w.sides, w.tile, w.q_scale)
    kv_cnt = torch.empty(nqb, dtype=torch.int32, device=dev)
    kv_idx = torch.empty(nqb, nkb, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, nq, dtype=torch.float32, device=dev)
    od = torch.empty_like(q)
    lsed = torch.empty_like(lse)
    scale = 1.0 / math.sqrt(w.d)
    stream = torch.cuda.current_stream()

    def step():
        vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, radius=w.radii, out=(kv_cnt, kv_idx, None), stream=stream)
        vs.attn_fwd(q, k, v, w.sides, w.tile, w.q_scale, kv_cnt, kv_idx, softmax_scale=scale, out=o, lse=lse,
                    stream=stream)

    # clock settling (time-based), then the --warmup count
    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        settle_steps += 20
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] clocks settled ({settle_steps} steps, {settle_ms:.0f} ms); warmup done ({args.warmup} steps)",
          file=sys.stderr, flush=True)

    # Mean launch duration of one kernel: reps back-to-back launches on the
    # launch stream, HIP events around the whole run (an event between two
    # launches would put a timing packet, and its cache flush, between them).
    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # timed region: K whole steps (mask + attention) bracketed by device
    # synchronisations; HIP events only at its two ends
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for _ in range(args.steps):
        step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    gpu_ms_step = e_start.elapsed_time(e_end) / args.steps
    print(f"[bench] sparse steps done: {ms_step:.4f} ms/step (events {gpu_ms_step:.4f})", file=sys.stderr, flush=True)

    # each kernel of the step alone, same lists and tensors
    # (at least 200 launches whatever --steps says: the roofline is taken from this)
    n_alone = max(args.steps, 200)
    attn_ms = timed(lambda: vs.attn_fwd(q, k, v, w.sides, w.tile, w.q_scale, kv_cnt, kv_idx, softmax_scale=scale,
                                        out=o, lse=lse, stream=stream), n_alone)
    mask_ms = timed(lambda: vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, radius=w.radii,
                                          out=(kv_cnt, kv_idx, None), stream=stream), n_alone)
    print(f"[bench] kernels alone: attn {attn_ms:.4f} ms, mask {mask_ms:.4f} ms", file=sys.stderr, flush=True)

    # single launches, warm and cold: HIP events around one attention launch,
    # median over runs; cold = a 512 MiB scrub buffer written before each launch
    # (more than the L2s and the MALL hold, so K, V and Q come from HBM)
    def single_launch_median(runs, scrub=None):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(runs)]
        for i, e in enumerate(evs):
            if scrub is not None:
                scrub.fill_(i & 0xff)
            e[0].record(stream)
            vs.attn_fwd(q, k, v, w.sides, w.tile, w.q_scale, kv_cnt, kv_idx, softmax_scale=scale, out=o, lse=lse,
                        stream=stream)
            e[1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([e[0].elapsed_time(e[1]) for e in evs]))

    single = None
    if not args.no_single:
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        n_single = max(10, min(100, args.steps))
        warm_single_ms = single_launch_median(n_single)
        cold_single_ms = single_launch_median(max(10, n_single // 3), scrub)
        del scrub
        single = {"warm_median_ms": warm_single_ms, "cold_median_ms": cold_single_ms,
                  "cold_tflops": None, "runs": [n_single, max(10, n_single // 3)],
                  "what": "HIP events around one launch, median; cold: 512 MiB scrub written before each"}
        print(f"[bench] single launches: warm {warm_single_ms:.4f} ms, cold {cold_single_ms:.4f} ms",
              file=sys.stderr, flush=True)

    sizes = tile_sizes(w.sides, w.q_scale, w.tile)
    cnt_h, idx_h = kv_cnt.cpu().numpy(), kv_idx.cpu().numpy()
    flops = kept_flops(cnt_h, idx_h, sizes, w.tile * w.tile, w.d, w.B * w.H)
    dense_flops = 4.0 * w.d * nq * nk * w.B * w.H
    count_sparsity = 1.0 - cnt_h.sum() / (nqb * nkb)
    flop_sparsity = 1.0 - flops / dense_flops

    # dense comparator on the same tensors
    nd = max(3, args.steps // 5)
    dense_ms = timed(lambda: vs.dense_attn_fwd(q, k, v, softmax_scale=scale, out=od, lse=lsed, stream=stream), nd)
    print(f"[bench] dense done: {dense_ms:.4f} ms", file=sys.stderr, flush=True)

    # token-level CSLA on the same tensors: the token-masked dense baseline
    # (every key tile, the token rule applied) and token-exact block-sparse
    # attention (the CSLA tiles, the token rule inside them)
    tok_dense_ms = timed(lambda: vs.attn_fwd_token(q, k, v, w.sides, w.tile, w.q_scale, w.n_sink, w.radii,
                                                   softmax_scale=scale, out=od, lse=lsed, stream=stream), nd)
    tok_sparse_ms = timed(lambda: vs.attn_fwd_token(q, k, v, w.sides, w.tile, w.q_scale, w.n_sink, w.radii, kv_cnt, kv_idx,
                                                    softmax_scale=scale, out=od, lse=lsed, stream=stream),
                          args.steps)
    print(f"[bench] token-wise done: dense {tok_dense_ms:.4f} ms, exact sparse {tok_sparse_ms:.4f} ms",
          file=sys.stderr, flush=True)

    # the block-128 variant: 128-query workgroups over pairs of query tiles,
    # same tensors and lists
    # (both kernels timed the same way: back-to-back launches on the stream)
    ref64_ms = timed(lambda: vs.attn_fwd(q, k, v, w.sides, w.tile, w.q_scale, kv_cnt, kv_idx, softmax_scale=scale,
                                         out=od, lse=lsed, stream=stream), args.steps)
    pair_ms = timed(lambda: vs.attn_fwd_pair(q, k, v, w.sides, w.tile, w.q_scale, kv_cnt, kv_idx, softmax_scale=scale,
                                             out=od, lse=lsed, stream=stream), args.steps)
    print(f"[bench] paired-tile kernel done: {pair_ms:.4f} ms", file=sys.stderr, flush=True)

    result = {
        "metric": "last-scale sparse-attn effective TFLOP/s + speedup vs dense attn, 1 MI355X",
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"steps": settle_steps, "ms": settle_ms,
                   "what": "steps run before the --warmup count until this much wall time passed (clock ramp)"},
        "ms_per_step": ms_step,
        "gpu_ms_per_step": gpu_ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "last_scale_2b", "B": w.B, "H": w.H, "head_dim": w.d, "query_side": w.sides[w.q_scale],
                   "query_tokens": nq, "cached_tokens": nk, "scales": list(w.sides), "tile": w.tile,
                   "n_sink": w.n_sink, "radius": w.radius, "mask": "csla"},
        "speedup_vs_dense": dense_ms / ms_step,
        "kernel_speedup_vs_dense": dense_ms / attn_ms,
        "attn_kernel_ms": attn_ms,
        "mask_kernel_ms": mask_ms,
        "dense_kernel_ms": dense_ms,
        "dense_tflops": dense_flops / (dense_ms * 1e-3) / 1e12,
        "block_sparsity": {"count": float(count_sparsity), "flop": float(flop_sparsity)},
        "token_wise": {"token_masked_dense_ms": tok_dense_ms, "token_exact_sparse_ms": tok_sparse_ms,
                       "block_sparse_ms": attn_ms, "block_vs_token_masked_dense": tok_dense_ms / attn_ms,
                       "token_exact_vs_token_masked_dense": tok_dense_ms / tok_sparse_ms,
                       "pages_block_vs_token_wise": 15.26},
        "block128_pair": {"ms": pair_ms, "ms_64_query_kernel": ref64_ms, "flop_per_launch": flops,
                          "tflops": flops / (pair_ms * 1e-3) / 1e12, "vs_64_query_kernel": ref64_ms / pair_ms,
                          "what": "128-query workgroups over pairs of 8x8 query tiles, union chunk walk"},
        "single_launch": single,
        "attn_kernel_launches_timed": n_alone,
        "roofline": {"bound": "mfma", "achieved": flops / (attn_ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "traffic": TRAFFIC["bytes"] if kernel_sources_sha256() == TRAFFIC["sources_sha256"] else None,
                     "traffic_unit": "bytes per launch",
                     "traffic_tb_per_s": (TRAFFIC["bytes"] / (attn_ms * 1e-3) / 1e12
                                          if kernel_sources_sha256() == TRAFFIC["sources_sha256"] else None),
                     "mfma_busy": (TRAFFIC["mfma_busy"]
                                   if kernel_sources_sha256() == TRAFFIC["sources_sha256"] else None),
                     "kernel": "attn_fwd_bf16_kernel<128,false,false>",
                     "flop_per_launch": flops},
    }

    if single is not None:
        single["cold_tflops"] = flops / (single["cold_median_ms"] * 1e-3) / 1e12
    if args.copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    if not args.no_cs4a:
        result["cs4a"] = bench_cs4a(vs, torch, W, SpatialField, to_dev, args, stream, dev)
        print("[bench] cs4a done", file=sys.stderr, flush=True)

    if not args.no_cs4a:
        result["scale_loop"] = bench_scale_loop(vs, torch, W, SpatialField, to_dev, args, stream, dev)
        print("[bench] scale loop done", file=sys.stderr, flush=True)

    if not args.no_high_res:
        result["high_res"] = bench_high_res(vs, torch, W, SpatialField, to_dev, args, stream, dev)
        print("[bench] high-res done", file=sys.stderr, flush=True)

    if not args.no_sweep:
        result["budget_sweep"] = bench_budget_sweep(vs, torch, W, SpatialField, to_dev, args, stream, dev)
        print("[bench] budget sweep done", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, q_np, k_np, v_np, cnt_h, idx_h, sizes, round_bf16, args.cpu_seconds)
        print("[bench] cpu baseline done", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


def bench_cs4a(vs, torch, W, SpatialField, to_dev, args, stream, dev):
    """Score at side 32, select top-p 0.9, map to sides 40/48/64, attend at each."""
    w = W.CS4A
    D = W.CS4A_DECISION
    f = SpatialField(w.seed, w.wid, w.B, w.H, w.d)
    k_np, v_np = f.keys_values(w.sides[: w.q_scale + 1], w.n_sink, largest_side=w.sides[w.q_scale])
    k, v = to_dev(k_np), to_dev(v_np)
    q_d = to_dev(f.queries(w.sides[D]))
    qs = {T: to_dev(f.queries(w.sides[T])) for T in W.CS4A_TARGETS}
    scores = torch.empty(w.B, w.H, *vs.geom_counts(w.sides, w.tile, D)[:2], dtype=torch.float32, device=dev)
    lists, outs, nks = {}, {}, {}
    for T in W.CS4A_TARGETS:
        nqb, nkb, nq, nk = vs.geom_counts(w.sides, w.tile, T)
        lists[T] = (torch.empty(w.B, w.H, nqb, dtype=torch.int32, device=dev),
                    torch.empty(w.B, w.H, nqb, nkb, dtype=torch.int32, device=dev))
        outs[T] = torch.empty_like(qs[T])
        nks[T] = nk
    scale = 1.0 / math.sqrt(w.d)

    target_lists = [lists[T] for T in W.CS4A_TARGETS]
    by_size = W.CS4A_TARGETS[::-1]   # largest target first: its longer walks start first

    def step(one_launch=True):
        # scores at the decision scale, then the lists of the three targets in one launch
        vs.map_indices_multi(w.sides, w.tile, D, W.CS4A_TARGETS, w.n_sink, W.CS4A_TOP_P, q_d=q_d, k=k,
                             scores=scores, out=target_lists, stream=stream)
        if one_launch:   # the three target attentions in one launch
            vs.attn_fwd_multi([qs[T] for T in by_size], k, v, w.sides, w.tile, by_size,
                              [lists[T] for T in by_size], softmax_scale=scale, outs=[outs[T] for T in by_size],
                              want_lse=False, stream=stream)
            return
        for T in W.CS4A_TARGETS:
            vs.attn_fwd(qs[T], k[:, :, : nks[T]], v[:, :, : nks[T]], w.sides, w.tile, T, *lists[T],
                        softmax_scale=scale, out=outs[T], want_lse=False, stream=stream)

    def dense_step():
        for T in W.CS4A_TARGETS:
            vs.dense_attn_fwd(qs[T], k[:, :, : nks[T]], v[:, :, : nks[T]], softmax_scale=scale, out=outs[T],
                              want_lse=False, stream=stream)

    n = max(5, args.steps // 2)
    res = {}
    for name, fn in (("sparse", step), ("sparse_three_launches", lambda: step(False)), ("dense", dense_step)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / n
    # O_cache: the decision scale's residual (full minus block-sparse output
    # over its own selection) upsampled onto each target output.  The full
    # attention at the decision scale is the model's own and is timed apart.
    nqb_d, nkb_d, _, nk_d = vs.geom_counts(w.sides, w.tile, D)
    lists_d = (torch.empty(w.B, w.H, nqb_d, dtype=torch.int32, device=dev),
               torch.empty(w.B, w.H, nqb_d, nkb_d, dtype=torch.int32, device=dev))
    o_full_d, o_sparse_d = torch.empty_like(q_d), torch.empty_like(q_d)

    def full_d():
        vs.dense_attn_fwd(q_d, k[:, :, :nk_d], v[:, :, :nk_d], softmax_scale=scale, out=o_full_d,
                          want_lse=False, stream=stream)

    def ocache_step():
        vs.map_indices(w.sides, w.tile, D, D, w.n_sink, W.CS4A_TOP_P, scores=scores, out=lists_d, stream=stream)
        vs.attn_fwd(q_d, k[:, :, :nk_d], v[:, :, :nk_d], w.sides, w.tile, D, *lists_d, softmax_scale=scale,
                    out=o_sparse_d, want_lse=False, stream=stream)
        for T in W.CS4A_TARGETS:
            vs.ocache_correct(o_full_d, o_sparse_d, outs[T], w.sides[D], w.sides[T], stream=stream)

    T_last = W.CS4A_TARGETS[-1]

    def correct_last():
        vs.ocache_correct(o_full_d, o_sparse_d, outs[T_last], w.sides[D], w.sides[T_last], stream=stream)

    step()
    for name, fn in (("full_d", full_d), ("ocache", ocache_step), ("correct_last", correct_last)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / n
    corr_bytes = 2 * 2 * w.B * w.H * w.d * (w.sides[T_last] ** 2 + w.sides[D] ** 2)
    flops = 0.0
    for T in W.CS4A_TARGETS:
        sizes = tile_sizes(w.sides, T, w.tile)
        flops += kept_flops(lists[T][0].cpu().numpy(), lists[T][1].cpu().numpy(), sizes, w.tile * w.tile, w.d, 0)
    nqb_D, nkb_D = scores.shape[2:]
    return {"workload": "cs4a_2b", "B": w.B, "H": w.H, "decision_side": w.sides[D],
            "target_sides": [w.sides[T] for T in W.CS4A_TARGETS], "top_p": W.CS4A_TOP_P,
            "ms_per_step": res["sparse"], "dense_ms_per_step": res["dense"],
            "speedup_vs_dense": res["dense"] / res["sparse"],
            "attention_tflop_per_step": flops / 1e12,
            "effective_tflops": flops / (res["sparse"] * 1e-3) / 1e12,
            "ms_per_step_three_attention_launches": res["sparse_three_launches"],
            "timed": "score + one select/map launch for the 3 targets + the 3 block-sparse attentions in one "
                     "launch; dense: 3 dense attentions",
            "ocache": {"ms_per_step": res["ocache"],
                       "timed": "map D->D + block-sparse attention at D + 3 corrections",
                       "decision_full_attention_ms": res["full_d"],
                       "correct_side64_ms": res["correct_last"],
                       "correct_side64_bytes": corr_bytes,
                       "correct_side64_gbps": corr_bytes / (res["correct_last"] * 1e-3) / 1e9,
                       "hbm_peak_gbps": 8000.0}}


def bench_high_res(vs, torch, W, SpatialField, to_dev, args, stream, dev):
    """The side-128 query scale over the 16-scale cache (42521 tokens), B = 1,
    H = 16, CSLA radius 2: mask + block-sparse attention steps, the attention
    alone, and the dense kernel on the same tensors."""
    w = W.HIGH_RES
    f = SpatialField(w.seed, w.wid, w.B, w.H, w.d)
    k_np, v_np = f.keys_values(w.sides[: w.q_scale + 1], w.n_sink, largest_side=w.sides[w.q_scale])
    q, k, v = to_dev(f.queries(w.sides[w.q_scale])), to_dev(k_np), to_dev(v_np)
    del k_np, v_np
    nqb, nkb, nq, nk = vs.geom_counts(w.sides, w.tile, w.q_scale)
    cnt = torch.empty(nqb, dtype=torch.int32, device=dev)
    idx = torch.empty(nqb, nkb, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    scale = 1.0 / math.sqrt(w.d)

    def mask():
        vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, radius=w.radii, out=(cnt, idx, None), stream=stream)

    def attn():
        vs.attn_fwd(q, k, v, w.sides, w.tile, w.q_scale, cnt, idx, softmax_scale=scale, out=o, want_lse=False,
                    stream=stream)

    def step():
        mask()
        attn()

    def run(fn, warm, reps):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = max(5, args.steps // 4)
    step_ms = run(step, 50, reps)
    attn_ms = run(attn, 2, reps)
    dense_ms = run(lambda: vs.dense_attn_fwd(q, k, v, softmax_scale=scale, out=o, want_lse=False, stream=stream),
                   2, max(3, args.steps // 40))
    mask()
    torch.cuda.synchronize()
    cnt_h, idx_h = cnt.cpu().numpy(), idx.cpu().numpy()
    sizes = tile_sizes(w.sides, w.q_scale, w.tile)
    flops = kept_flops(cnt_h, idx_h, sizes, w.tile * w.tile, w.d, w.B * w.H)
    dense_flops = 4.0 * w.d * nq * nk * w.B * w.H
    return {"workload": "high_res_128", "B": w.B, "H": w.H, "head_dim": w.d, "query_side": w.sides[w.q_scale],
            "cached_tokens": nk, "radius": w.radius, "ms_per_step": step_ms, "attn_kernel_ms": attn_ms,
            "dense_kernel_ms": dense_ms, "effective_tflops": flops / (step_ms * 1e-3) / 1e12,
            "attn_tflops": flops / (attn_ms * 1e-3) / 1e12, "speedup_vs_dense": dense_ms / step_ms,
            "kernel_speedup_vs_dense": dense_ms / attn_ms,
            "count_sparsity": float(1.0 - cnt_h.sum() / (nqb * nkb)), "flop_sparsity": float(1.0 - flops / dense_flops),
            "timed": "mask + attention steps; the attention alone; the dense kernel, HIP events around back-to-back runs"}


def bench_budget_sweep(vs, torch, W, SpatialField, to_dev, args, stream, dev):
    """The 8B-shaped last two scales (B = 2, H = 28, d = 128): queries at side
    48 (2304 tokens over 6425) and side 64 (4096 over 10521), the CSLA budget
    mode keeping 75 / 85 / 90 / 95% of the key tiles out of each row.  Per
    point: the budget mask + attention step, the attention alone, effective
    TFLOP/s, fraction of the bf16 peak and speedup against the dense kernel on
    the same tensors (HIP events around back-to-back launches)."""
    out = []
    for w in (W.LAST_TWO_8B_48, W.LAST_TWO_8B_64):
        f = SpatialField(w.seed, w.wid, w.B, w.H, w.d)
        k_np, v_np = f.keys_values(w.sides[: w.q_scale + 1], w.n_sink, largest_side=w.sides[w.q_scale])
        q, k, v = to_dev(f.queries(w.sides[w.q_scale])), to_dev(k_np), to_dev(v_np)
        del k_np, v_np
        nqb, nkb, nq, nk = vs.geom_counts(w.sides, w.tile, w.q_scale)
        cnt = torch.empty(nqb, dtype=torch.int32, device=dev)
        idx = torch.empty(nqb, nkb, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        scale = 1.0 / math.sqrt(w.d)
        sizes = tile_sizes(w.sides, w.q_scale, w.tile)
        dense_flops = 4.0 * w.d * nq * nk * w.B * w.H

        def run(fn, warm, reps):
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        dense_ms = run(lambda: vs.dense_attn_fwd(q, k, v, softmax_scale=scale, out=o, want_lse=False, stream=stream),
                       2, 20)
        for budget in w.budgets:
            def mask():
                vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, budget=budget, out=(cnt, idx, None),
                              stream=stream)

            def attn():
                vs.attn_fwd(q, k, v, w.sides, w.tile, w.q_scale, cnt, idx, softmax_scale=scale, out=o,
                            want_lse=False, stream=stream)

            def step():
                mask()
                attn()

            step_ms = run(step, 20, 100)
            attn_ms = run(attn, 2, 100)
            mask()
            torch.cuda.synchronize()
            cnt_h, idx_h = cnt.cpu().numpy(), idx.cpu().numpy()
            flops = kept_flops(cnt_h, idx_h, sizes, w.tile * w.tile, w.d, w.B * w.H)
            tf = flops / (attn_ms * 1e-3) / 1e12
            out.append({"query_side": w.sides[w.q_scale], "cached_tokens": nk, "budget_tiles": budget,
                        "count_sparsity": float(1.0 - cnt_h.sum() / (nqb * nkb)),
                        "flop_sparsity": float(1.0 - flops / dense_flops),
                        "ms_per_step": step_ms, "attn_kernel_ms": attn_ms, "dense_kernel_ms": dense_ms,
                        "effective_tflops": flops / (step_ms * 1e-3) / 1e12, "attn_tflops": tf,
                        "frac_of_peak": tf / PEAK_BF16_TFLOPS, "speedup_vs_dense": dense_ms / step_ms,
                        "kernel_speedup_vs_dense": dense_ms / attn_ms})
        del q, k, v, o
    return {"workload": "last_two_8b (B=2, H=28, d=128, sides 48 and 64, budget mode 75/85/90/95%)", "points": out,
            "timed": "budget mask + attention steps; the attention alone; the dense kernel, HIP events around "
                     "back-to-back runs", "both_scales": bench_last_two_joint(vs, torch, W, SpatialField, to_dev,
                                                                               stream, dev)}


def bench_last_two_joint(vs, torch, W, SpatialField, to_dev, stream, dev):
    """The last two scales of the 8B shape as one step over one cache (the
    side-64 workload's 13-scale cache; side 48 attends to its first 6425
    tokens): both budget masks, then both attentions in one launch
    (varsparse_attn_fwd_multi), against the same two attentions as two
    launches and against dense attention at both sides; the budgets paired
    by sparsity (75/85/90/95%)."""
    w48, w64 = W.LAST_TWO_8B_48, W.LAST_TWO_8B_64
    f = SpatialField(w64.seed, w64.wid, w64.B, w64.H, w64.d)
    k_np, v_np = f.keys_values(w64.sides[: w64.q_scale + 1], w64.n_sink, largest_side=w64.sides[w64.q_scale])
    k, v = to_dev(k_np), to_dev(v_np)
    del k_np, v_np
    ws = (w64, w48)   # largest first in the one launch
    qs = [to_dev(f.queries(w.sides[w.q_scale])) for w in ws]
    outs = [torch.empty_like(q) for q in qs]
    scale = 1.0 / math.sqrt(w64.d)
    geo = [vs.geom_counts(w.sides, w.tile, w.q_scale) for w in ws]
    lists = [(torch.empty(g[0], dtype=torch.int32, device=dev), torch.empty(g[0], g[1], dtype=torch.int32, device=dev))
             for g in geo]

    def run(fn, warm, reps):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def dense():
        for w, q, o, g in zip(ws, qs, outs, geo):
            vs.dense_attn_fwd(q, k[:, :, : g[3]], v[:, :, : g[3]], softmax_scale=scale, out=o, want_lse=False,
                              stream=stream)

    dense_ms = run(dense, 2, 10)
    dense_flops = sum(4.0 * w.d * g[2] * g[3] * w.B * w.H for w, g in zip(ws, geo))
    points = []
    for b64, b48 in zip(w64.budgets, w48.budgets):
        def masks():
            for w, budget, (c, i) in zip(ws, (b64, b48), lists):
                vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, budget=budget, out=(c, i, None), stream=stream)

        def step(one_launch=True):
            masks()
            if one_launch:
                vs.attn_fwd_multi(qs, k, v, w64.sides, w64.tile, [w.q_scale for w in ws], lists,
                                  softmax_scale=scale, outs=outs, want_lse=False, stream=stream)
                return
            for w, q, o, (c, i) in zip(ws, qs, outs, lists):
                vs.attn_fwd(q, k, v, w.sides, w.tile, w.q_scale, c, i, softmax_scale=scale, out=o, want_lse=False,
                            stream=stream)

        one = run(step, 10, 50)
        two = run(lambda: step(False), 10, 50)
        masks()
        torch.cuda.synchronize()
        flops = 0.0
        for w, (c, i) in zip(ws, lists):
            flops += kept_flops(c.cpu().numpy(), i.cpu().numpy(), tile_sizes(w.sides, w.q_scale, w.tile),
                                w.tile * w.tile, w.d, w.B * w.H)
        points.append({"budget_tiles": {"64": b64, "48": b48}, "flop_sparsity": float(1.0 - flops / dense_flops),
                       "ms_per_step": one, "ms_per_step_two_attention_launches": two, "dense_ms": dense_ms,
                       "effective_tflops": flops / (one * 1e-3) / 1e12, "speedup_vs_dense": dense_ms / one})
    del k, v, qs, outs
    return {"workload": "last_two_8b sides 64 and 48 in one step over one cache",
            "timed": "two budget masks + both attentions in one launch (or two); dense: both sides, two launches",
            "points": points}


def bench_scale_loop(vs, torch, W, SpatialField, to_dev, args, stream, dev):
    """One generation step of attention over all 13 query scales of the 2B
    schedule: dense below the decision scale (side 32); at it, full attention,
    scores + selection and block-sparse attention over its own selection; at
    sides 40/48/64, CS4A mapping joined (union) with the CSLA window lists of
    windows 3/5/7, then block-sparse attention with the O_cache correction in
    its epilogue (one launch; the two-launch form, attention then correction,
    is timed beside it).  Compared with dense attention at every scale."""
    w = W.CS4A
    D = W.CS4A_DECISION
    windows = (3, 5, 7)
    n = len(w.sides)
    f = SpatialField(w.seed, w.wid, w.B, w.H, w.d)
    k_np, v_np = f.keys_values(w.sides, w.n_sink)
    k, v = to_dev(k_np), to_dev(v_np)
    qs = [to_dev(f.queries(s)) for s in w.sides]
    outs = [torch.empty_like(x) for x in qs]
    nks = [vs.geom_counts(w.sides, w.tile, s)[3] for s in range(n)]
    scale = 1.0 / math.sqrt(w.d)
    nqb_d, nkb_d = vs.geom_counts(w.sides, w.tile, D)[:2]
    scores = torch.empty(w.B, w.H, nqb_d, nkb_d, dtype=torch.float32, device=dev)
    lists_d = (torch.empty(w.B, w.H, nqb_d, dtype=torch.int32, device=dev),
               torch.empty(w.B, w.H, nqb_d, nkb_d, dtype=torch.int32, device=dev))
    o_sparse_d = torch.empty_like(qs[D])
    bufs = {}
    for T in W.CS4A_TARGETS:
        nqb, nkb = vs.geom_counts(w.sides, w.tile, T)[:2]
        mk = lambda *lead: (torch.empty(*lead, nqb, dtype=torch.int32, device=dev),
                            torch.empty(*lead, nqb, nkb, dtype=torch.int32, device=dev))
        bufs[T] = (mk(w.B, w.H), mk(), mk(w.B, w.H), vs.window_radius(n, T, windows))

    def dense_at(s):
        vs.dense_attn_fwd(qs[s], k[:, :, : nks[s]], v[:, :, : nks[s]], softmax_scale=scale, out=outs[s],
                          want_lse=False, stream=stream)

    small = list(range(D))[::-1]   # the scales below the decision scale, largest first

    def dense_small(one_launch=True):
        if one_launch:   # sides 1 ... 24 in one launch, each over the cache up to its own scale
            vs.dense_attn_fwd_multi([qs[s] for s in small], k, v, [nks[s] for s in small], softmax_scale=scale,
                                    outs=[outs[s] for s in small], want_lse=False, stream=stream)
        else:
            for s in small:
                dense_at(s)

    multi_out = [lists_d] + [bufs[T][0] for T in W.CS4A_TARGETS]

    def loop_step(fused=True):
        dense_small()
        dense_at(D)
        # the decision scale's scores and the lists of itself and every later scale, in one launch
        vs.map_indices_multi(w.sides, w.tile, D, [D, *W.CS4A_TARGETS], w.n_sink, W.CS4A_TOP_P, q_d=qs[D], k=k,
                             scores=scores, out=multi_out, stream=stream)
        vs.attn_fwd(qs[D], k[:, :, : nks[D]], v[:, :, : nks[D]], w.sides, w.tile, D, *lists_d, softmax_scale=scale,
                    out=o_sparse_d, want_lse=False, stream=stream)
        for T in W.CS4A_TARGETS:
            mapped, window, joined, radius = bufs[T]
            vs.build_mask(w.sides, w.tile, T, w.n_sink, radius=radius, out=(*window, None), stream=stream)
            vs.join_lists(*mapped, *window, join="union", out=joined, stream=stream)
            if fused == "multi":
                continue
            if fused:
                vs.attn_fwd_ocache(qs[T], k[:, :, : nks[T]], v[:, :, : nks[T]], w.sides, w.tile, T, *joined, D,
                                   outs[D], o_sparse_d, softmax_scale=scale, out=outs[T], want_lse=False,
                                   stream=stream)
            else:
                vs.attn_fwd(qs[T], k[:, :, : nks[T]], v[:, :, : nks[T]], w.sides, w.tile, T, *joined,
                            softmax_scale=scale, out=outs[T], want_lse=False, stream=stream)
                vs.ocache_correct(outs[D], o_sparse_d, outs[T], w.sides[D], w.sides[T], stream=stream)
        if fused == "multi":   # the three corrected target attentions in one launch, largest first
            by_size = W.CS4A_TARGETS[::-1]
            vs.attn_fwd_multi([qs[T] for T in by_size], k, v, w.sides, w.tile, by_size,
                              [bufs[T][2] for T in by_size], softmax_scale=scale, outs=[outs[T] for T in by_size],
                              want_lse=False, d_scale=D, o_full_d=outs[D], o_sparse_d=o_sparse_d, stream=stream)

    def dense_step():
        dense_small()
        for s in range(D, n):
            dense_at(s)

    def below_d():
        dense_small()

    # the four forms timed in turn, three rounds, median per form (slow clock
    # drift then affects every form alike)
    reps = max(5, args.steps // 2)
    forms = (("loop", lambda: loop_step(fused="multi")), ("loop_per_target", loop_step),
             ("loop_two_launch", lambda: loop_step(fused=False)),
             ("dense", dense_step), ("below_d", below_d), ("below_d_per_scale", lambda: dense_small(False)))
    runs = {name: [] for name, _ in forms}
    for _ in range(3):
        for name, fn in forms:
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            runs[name].append(e0.elapsed_time(e1) / reps)
    res = {name: float(np.median(v)) for name, v in runs.items()}
    loop_step(fused="multi")
    torch.cuda.synchronize()
    sparsity = {}
    for T in W.CS4A_TARGETS:
        nqb, nkb = vs.geom_counts(w.sides, w.tile, T)[:2]
        mapped, window, joined, _ = bufs[T]
        sparsity[str(w.sides[T])] = {
            "cs4a": 1.0 - float(mapped[0].sum()) / (w.B * w.H * nqb * nkb),
            "csla_window": 1.0 - float(window[0].sum()) / (nqb * nkb),
            "union": 1.0 - float(joined[0].sum()) / (w.B * w.H * nqb * nkb)}
    return {"workload": "cs4a_2b all 13 query scales", "B": w.B, "H": w.H, "decision_side": w.sides[D],
            "windows": list(windows), "join": "union", "top_p": W.CS4A_TOP_P,
            "ms_per_step": res["loop"], "dense_ms_per_step": res["dense"],
            "speedup_vs_dense": res["dense"] / res["loop"],
            "ms_per_step_one_launch_per_target": res["loop_per_target"],
            "ms_per_step_two_launch_ocache": res["loop_two_launch"],
            "dense_below_decision_ms": res["below_d"],
            "dense_below_decision_ms_one_launch_per_scale": res["below_d_per_scale"],
            "count_sparsity": sparsity,
            "timed": "dense attention at sides 1..24 in one launch; at 32 dense + scores + one select/map launch for 32/40/48/64 + "
                     "block-sparse over its own selection; at 40/48/64 CSLA window mask + union, then one "
                     "block-sparse attention launch over the three with the O_cache correction in its epilogue; "
                     "dense: all 13 scales (sides 1..24 in one launch, as in the loop)"}


def cpu_baseline(w, q_np, k_np, v_np, cnt_h, idx_h, sizes, round_bf16, seconds):
    """The oracle (numpy float64 masked dense softmax attention) on a bounded
    sample of the same workload: (query tile, head) pairs in order until about
    ``seconds`` of CPU work, scaled to effective TFLOP/s."""
    from threadpoolctl import threadpool_info
    from oracle import attention as OA
    done, flops = 0, 0.0
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    t0 = time.perf_counter()
    for (b, h) in heads:
        q = round_bf16(q_np[b:b + 1, h:h + 1]).astype(np.float64)
        k = round_bf16(k_np[b:b + 1, h:h + 1]).astype(np.float64)
        v = round_bf16(v_np[b:b + 1, h:h + 1]).astype(np.float64)
        for tile in range(cnt_h.shape[0]):
            if time.perf_counter() - t0 >= seconds:
                break
            OA.block_sparse_attention(q, k, v, w.sides, w.q_scale, w.tile, cnt_h, idx_h, 1 / math.sqrt(w.d),
                                      q_tiles=[tile])
            flops += 4.0 * w.d * w.tile * w.tile * int(sizes[idx_h[tile, : cnt_h[tile]]].sum())
            done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {cnt_h.shape[0] * len(heads)} (query tile, head) pairs in order, {el:.1f} s, "
                      f"numpy float64, host of {os.cpu_count()} logical CPUs"}


if __name__ == "__main__":
    main()

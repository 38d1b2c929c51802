#!/usr/bin/env python3
"""Benchmark of the RocketKV hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input of
the Llama-3.1-8B-shaped single-layer workload (batch 1, 32K prompt, 32 query /
8 KV heads, d 128, bf16, c = 16): the adaptive split, SnapKV eviction of the
layer (window scoring, pooling, top-k, compaction), the Kmax/Kmin build and
the 64 HSA decode steps of the workload.  Inputs are resident in HBM before
timing; steps rotate over several prompt replicas so the eviction does not
re-read a cache-resident K.  Each step is replayed from two HIP graphs (evict +
aux, then the 64 decode calls) with HIP events between them.

Reported: `value` = HSA decode time per decode step (us), `ms_per_step` = one
whole pass, plus SnapKV eviction ms/layer, decode HBM GB/s and the roofline of
the dominant kernel (per-kernel durations from the library's own HIP-event
timing over an eager pass of the same steps), and the CPU oracle timed on a
bounded sample on the host.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b-layer-s32k-c16")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-graph", action="store_true", help="issue every call eagerly instead of graph replay")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (the hot path shards over (batch, KV head) "
              f"units with no exchange; multi-GPU runs are not part of it); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_decode_attention_amd import rocketkv as rk
    from sparse_decode_attention_amd import workloads as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WL.WORKLOADS[args.workload]
    assert w.layers == 1 and w.mt_turns == 0, "bench runs a single-layer RocketKV workload"
    sp = rk.rk_split(w.c, w.seq, w.window, w.block, w.d)
    S, W, B, Hq, Hkv, d = w.seq, w.window, w.batch, w.n_q, w.n_kv, w.d
    n_keep, k2, blk, k1 = sp["n_keep"], sp["k2_blocks"], w.block, w.k1
    nblk = -(-n_keep // blk)
    nsel = min(k2, nblk)
    R = max(1, args.replicas)
    steps_dec = w.decode_steps
    esize = 2 if w.dtype == "bf16" else 4
    log(f"workload {w.name}: S={S} n_keep={n_keep} pages={nblk} k1={k1} k2={k2} replicas={R}")

    # ---- inputs, resident in HBM ----
    reps = []
    for r in range(R):
        k, v, _ = WL.layer_kv(w, r, device=dev)
        qw = WL.window_queries(w, r, device=dev)
        qs = torch.stack([WL.decode_query(w, r, s, device=dev) for s in range(steps_dec)])
        reps.append((k, v, qw, qs))
    kept = torch.empty(B, Hkv, n_keep, dtype=torch.int32, device=dev)
    kc = torch.empty(B, Hkv, n_keep, d, dtype=w.torch_dtype, device=dev)
    vc = torch.empty_like(kc)
    kmax = torch.empty(B, Hkv, d, rk.aux_capacity(n_keep, blk), dtype=w.torch_dtype, device=dev)
    kmin = torch.empty_like(kmax)
    out = torch.empty(steps_dec, B, Hq, d, dtype=torch.float32, device=dev)
    shape = rk.shape_of(B, Hq, Hkv, d, w.torch_dtype)
    ws_e = torch.empty(rk.rk_snapkv_workspace_bytes(shape, S, W), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(rk.rk_hsa_workspace_bytes(shape, n_keep, blk, k1, k2), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def evict_part(r):
        k, v, qw, _ = reps[r]
        rk.rk_snapkv_evict(qw, k, v, S, W, w.pool, n_keep, kept, kc, vc, None, ws=ws_e)
        rk.rk_hsa_build_aux(kc, n_keep, 0, blk, kmax, kmin, n_q_heads=Hq)

    def decode_part(r):
        qs = reps[r][3]
        for s in range(steps_dec):
            rk.rk_hsa_decode(qs[s], kc, vc, kmax, kmin, n_keep, blk, k1, k2, out[s], ws=ws_d)

    # eager warm-up (also before capture)
    for i in range(max(1, args.warmup)):
        evict_part(i % R)
        decode_part(i % R)
    torch.cuda.synchronize()

    use_graph = not args.no_graph
    graphs = []
    if use_graph:
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for r in range(R):
                ge, gd = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
                with torch.cuda.graph(ge, stream=stream):
                    evict_part(r)
                with torch.cuda.graph(gd, stream=stream):
                    decode_part(r)
                graphs.append((ge, gd))
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()

    def run_step(i, ev):
        r = i % R
        ev[0].record()
        if use_graph:
            graphs[r][0].replay()
        else:
            evict_part(r)
        ev[1].record()
        if use_graph:
            graphs[r][1].replay()
        else:
            decode_part(r)
        ev[2].record()

    for i in range(args.warmup):
        run_step(i, [torch.cuda.Event(enable_timing=True) for _ in range(3)])
    torch.cuda.synchronize()

    # ---- timed region ----
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    evict_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    evict_ms_layer = sum(evict_ms) / len(evict_ms)
    dec_us_step = sum(dec_ms) / len(dec_ms) * 1e3 / steps_dec
    log(f"wall {ms_per_step:.3f} ms/step; evict+aux {evict_ms_layer:.3f} ms/layer; "
        f"decode {dec_us_step:.2f} us/step")

    # ---- per-kernel durations: library HIP-event timing over an eager pass ----
    rk.rk_profile_begin()
    for i in range(args.steps):
        evict_part(i % R)
        decode_part(i % R)
    prof = rk.rk_profile_end()
    torch.cuda.synchronize()
    per_step = {n: (c / args.steps, t / args.steps, t / c) for n, (c, t) in prof.items()}
    for n, (cps, tps, avg) in per_step.items():
        log(f"kernel {n:14s} {cps:6.1f} launches/step {tps:8.4f} ms/step avg {avg * 1e3:8.2f} us")

    # algorithmic bytes per launch (what the method must move)
    units = B * Hkv
    alg = {
        "hsa_attn": units * nsel * blk * 2 * d * esize + B * Hq * d * (esize + 4),
        "hsa_select": units * k1 * nblk * esize + B * Hq * d * esize,
        "aux_build": units * n_keep * d * esize + 2 * units * d * nblk * esize,
        "gather_kv": 2 * 2 * units * n_keep * d * esize,
        "ws_pass1": units * S * d * esize + B * Hq * W * d * esize,
        "ws_pass2": units * (S - W) * d * esize + B * Hq * W * d * esize,
    }
    dominant = max(per_step, key=lambda n: per_step[n][1])
    avg_ms = per_step[dominant][2]
    roof = None
    if dominant in alg:
        achieved = alg[dominant] / (avg_ms * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                "bytes_per_launch": alg[dominant], "avg_launch_us": round(avg_ms * 1e3, 3)}
    attn_avg = per_step.get("hsa_attn", (0, 0, float("nan")))[2]
    dec_bytes = alg["hsa_attn"] + alg["hsa_select"]
    dec_gbps = dec_bytes / (dec_us_step * 1e-6) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, reps[0], n_keep, k1, k2, args.cpu_seconds)

    line = {
        "metric": "HSA decode us/step + HBM GB/s (% peak); SnapKV evict ms/layer",
        "value": round(dec_us_step, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seq_len": S, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": d, "kv_dtype": w.dtype, "compression": w.c, "n_keep": n_keep,
                   "k1": k1, "k2_pages": k2, "page": blk, "decode_steps": steps_dec,
                   "replicas": R, "graph_replay": use_graph},
        "snapkv_evict_ms_per_layer": round(evict_ms_layer, 4),
        "hsa_decode_GBps": round(dec_gbps, 1),
        "hsa_decode_hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "hsa_attn_avg_us": round(attn_avg * 1e3, 3),
        "kernels_ms_per_step": {n: round(v[1], 5) for n, v in per_step.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(w, rep, n_keep, k1, k2, budget_s):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np

    import oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    k, v, qw, qs = rep
    G = w.group
    # stage 1 on one unit, extrapolated to the layer
    t0 = time.perf_counter()
    kn = k[0, 0].float().cpu().numpy()
    vn = v[0, 0].float().cpu().numpy()
    qn = qw[0, :G].float().cpu().numpy()
    sc = O.window_scores(qn, kn)
    pl = O.pool_sum(sc, w.pool)
    kept = O.snapkv_select(pl, w.seq, w.window, n_keep)
    kc, vc = kn[kept], vn[kept]
    kmax, kmin = O.build_aux(kc, n_keep, w.block)
    evict_unit_ms = (time.perf_counter() - t0) * 1e3
    # decode: all units of the batch, as many steps as the budget allows
    units = [(0, h) for h in range(w.n_kv)]
    caches = {}
    for b, h in units:
        if (b, h) == (0, 0):
            caches[(b, h)] = (kc, vc, kmax, kmin)
            continue
        kk = k[b, h].float().cpu().numpy()
        vv = v[b, h].float().cpu().numpy()
        pl2 = O.pool_sum(O.window_scores(qw[b, h * G:(h + 1) * G].float().cpu().numpy(), kk), w.pool)
        kp = O.snapkv_select(pl2, w.seq, w.window, n_keep)
        ka, kb = O.build_aux(kk[kp], n_keep, w.block)
        caches[(b, h)] = (kk[kp], vv[kp], ka, kb)
    qn_all = qs.float().cpu().numpy()
    t0 = time.perf_counter()
    done = 0
    while done < qn_all.shape[0] and time.perf_counter() - t0 < budget_s:
        for b, h in units:
            c = caches[(b, h)]
            O.hsa_unit(qn_all[done, b, h * G:(h + 1) * G], c[0], c[1], c[2], c[3], n_keep, w.block, k1, k2)
        done += 1
    dec_us = (time.perf_counter() - t0) * 1e6 / max(done, 1)
    return {"value": round(dec_us, 1), "unit": "us/step", "cores": threads, "kind": "oracle",
            "sample": f"HSA decode of all {len(units)} units for {done} of {w.decode_steps} steps "
                      f"(aux built once); stage 1 of one unit {evict_unit_ms:.0f} ms, "
                      f"x{w.batch * w.n_kv} units = {evict_unit_ms * w.batch * w.n_kv:.0f} ms/layer (extrapolated)",
            "evict_ms_per_layer_extrapolated": round(evict_unit_ms * w.batch * w.n_kv, 1)}


if __name__ == "__main__":
    main()

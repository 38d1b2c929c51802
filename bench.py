#!/usr/bin/env python3
"""Benchmark of the RocketKV hot path on one MI355X.

Default workload: RocketKV-MT on the MHA shape (batch 8, 32 heads, d 128,
bf16, c 32), its last turn: a 32K prompt plus 4 x 1024 appended tokens kept
whole in HBM, index-only SnapKV eviction over all 36864 tokens, Kmax/Kmin
over the candidates and 64 MT decode steps.  It is the largest workload that
fits one GPU and one of the two whose decode is HBM-bound.  The other
HBM-bound workload, one layer of the batch-32 Llama-8B stack (c 64, per-step
appends), is measured in the same run and reported under "also".

A step is one pass of the whole hot path over R layers of the workload (each
layer its own synthetic inputs and caches): per layer the adaptive split,
SnapKV eviction and the Kmax/Kmin build; then the decode steps, interleaved
across the layers (step s of layer 0, of layer 1, ..., then step s + 1), as a
stack of layers runs them.  R is chosen so that the decode traffic of the
other layers between two visits to one layer exceeds twice the 256 MB MALL:
every decode step then reads its pages from HBM, as it would between the
other layers (and weights) of a real model.  Per-layer figures are the step's
totals divided by R.

Inputs are resident in HBM before timing.  Each step replays two HIP graphs
(eviction + aux of the R layers; the interleaved decode calls) with HIP
events between them.  Reported: `value` = HSA decode time per layer per
decode step (median over steps, us), `ms_per_step` = one whole step (wall
clock, mean over the K timed steps), SnapKV eviction ms/layer, decode HBM
GB/s, window-scoring TFLOP/s (the once-counted 2*G*W*S*d over pass 1 +
statistics + pass 2), the roofline of the dominant kernel (per-kernel
durations from the library's HIP-event timing over an eager step) and the
CPU oracle timed on a bounded sample on the host.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256e6
MODEL_LAYERS = 32            # the stacks the large workloads stand for


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mt-mha-b8-s32k-c32")
    ap.add_argument("--also", default="llama8b-stack-b32-s32k-c64",
                    help="a second workload measured in the same run ('' for none)")
    ap.add_argument("--layers", type=int, default=0,
                    help="layers per step (0: enough that other layers' decode traffic exceeds 2x MALL)")
    ap.add_argument("--no-graph", action="store_true", help="issue every call eagerly instead of graph replay")
    ap.add_argument("--paged", type=int, default=0, metavar="P",
                    help="decode from a paged pool of P-token physical pages (block tables, pages in random "
                         "order; the compact cache is copied into it after eviction); not for RocketKV-MT")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--selection-recall", action="store_true",
                    help="only compare the selection methods (HSA, Quest, SparQ, Exact-TopK, two-stage "
                         "RocketKV) on the Llama-8B layer and the 109K needle: recall of the exact top "
                         "tokens, attention mass, output error, needle hits, us per decode step")
    ap.add_argument("--recall-steps", type=int, default=8)
    ap.add_argument("--evict-compare", default="", metavar="WORKLOADS",
                    help="only time stage 1 on the given comma-separated workloads, per-head SnapKV "
                         "against Ada-KV's shared budget (both with compaction and Kmax/Kmin): ms per "
                         "layer and per-kernel us, one JSON line per workload")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (scales the HBM byte "
                         "counters FETCH_SIZE / WRITE_SIZE of a profiler run)")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain copy kernel of known size: reads and writes mib MiB per launch."""
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 3}),
          flush=True)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Layer:
    """Inputs, caches and outputs of one layer of a workload."""


class Path:
    """Buffers and calls of R layers of a workload."""

    def __init__(self, rk, WL, w, dev, n_layers, paged=0):
        import torch

        self.rk, self.w = rk, w
        self.mt = w.mt_turns > 0
        self.paged = paged if not self.mt else 0
        self.S = w.seq + (w.mt_turns * w.mt_append if self.mt else 0)   # MT: the last turn
        sp = rk.rk_split(w.c, self.S, w.window, w.block, w.d)
        self.n_keep, self.k2 = sp["n_keep"], WL.stage2_pages(w, sp)
        self.steps = w.decode_steps
        B, Hq, Hkv, d = w.batch, w.n_q, w.n_kv, w.d
        G = w.group
        self.cap_c = self.n_keep + (self.steps if w.appends else 0)
        self.nblk = -(-self.cap_c // w.block)
        esize = 2 if w.dtype == "bf16" else 4
        units = B * Hkv
        nb0 = -(-self.n_keep // w.block)
        nsel = min(self.k2, self.nblk)
        # algorithmic bytes per launch (what the method must move), per kernel
        self.alg = {
            "hsa_attn": units * nsel * w.block * 2 * d * esize + B * Hq * d * esize,
            "hsa_attn_mt": units * nsel * w.block * (2 * d * esize + 4) + B * Hq * d * esize,
            "hsa_score": units * w.k1 * nb0 * esize + B * Hq * d * esize,
            "hsa_fused": units * w.k1 * nb0 * esize + units * nsel * w.block * 2 * d * esize
            + B * Hq * d * esize,
            "hsa_fused_mt": units * w.k1 * nb0 * esize + units * nsel * w.block * (2 * d * esize + 4)
            + B * Hq * d * esize,
            "aux_build": units * self.n_keep * d * esize + 2 * units * d * nb0 * esize
            + (units * self.n_keep * 4 if self.mt else 0),
            "gather_kv": 2 * 2 * units * self.n_keep * d * esize + 2 * units * d * nb0 * esize,
            "ws_pass1": units * self.S * d * esize + B * Hq * w.window * d * esize,
            "ws_pass2": units * (self.S - w.window) * d * esize + B * Hq * w.window * d * esize,
            "append_kv": units * d * esize * 5,
        }
        # the one-launch decode step with its append: the fused bytes plus the append's
        self.alg["hsa_fused_append"] = self.alg["hsa_fused"] + self.alg["append_kv"]
        self.flops_ws = 2.0 * units * G * w.window * self.S * d
        if self.mt:
            self.dec_bytes = self.alg["hsa_fused_mt"]
        elif w.appends:
            self.dec_bytes = self.alg["hsa_fused"] + self.alg["append_kv"]
        else:
            self.dec_bytes = self.alg["hsa_fused"]
        # layers: enough that the other layers' decode traffic between two
        # visits of one layer's data exceeds twice the MALL
        aux_bytes = 2 * units * d * nb0 * esize
        self.R = n_layers or max(2, math.ceil(2 * MALL_BYTES / (self.dec_bytes + aux_bytes)) + 1)
        self.R = min(self.R, 16)
        # prompt K/V of the plain workloads is only read by the eviction
        # (> MALL on its own for the large ones): two copies rotate; MT keeps
        # each layer's full cache
        kv_bytes = 2 * B * Hkv * self.S * d * esize
        n_prompts = self.R if self.mt else max(1, min(self.R, math.ceil(2 * MALL_BYTES / kv_bytes)))
        prompts = []
        for r in range(n_prompts):
            if self.mt:
                k = torch.empty(B, Hkv, self.S, d, dtype=w.torch_dtype, device=dev)
                v = torch.empty_like(k)
                k0, v0, _ = WL.layer_kv(w, r, device=dev)
                k[:, :, :w.seq], v[:, :, :w.seq] = k0, v0
                del k0, v0
                s0 = w.seq
                for t in range(w.mt_turns):
                    kt, vt = WL.turn_kv(w, r, t, device=dev)
                    k[:, :, s0:s0 + w.mt_append], v[:, :, s0:s0 + w.mt_append] = kt, vt
                    s0 += w.mt_append
            else:
                k, v, _ = WL.layer_kv(w, r, device=dev)
            prompts.append((k, v))
        shape = rk.shape_of(B, Hq, Hkv, d, w.torch_dtype)
        self.ws_e = torch.empty(rk.rk_snapkv_workspace_bytes(shape, self.S, w.window), dtype=torch.uint8,
                                device=dev)
        self.ws_d = torch.empty(rk.rk_hsa_workspace_bytes(shape, self.cap_c, w.block, w.k1, self.k2),
                                dtype=torch.uint8, device=dev)
        self.layers = []
        for r in range(self.R):
            L = Layer()
            L.k, L.v = prompts[r % n_prompts]
            turn = w.mt_turns - 1 if self.mt else -1
            L.qw = WL.window_queries(w, r, device=dev, turn=turn)
            s_off = (w.mt_turns - 1) * self.steps if self.mt else 0
            L.qs = torch.stack([WL.decode_query(w, r, s_off + s, device=dev) for s in range(self.steps)])
            L.app = [WL.append_kv(w, r, s, device=dev) for s in range(self.steps)] if w.appends else None
            L.kept = torch.empty(B, Hkv, self.n_keep, dtype=torch.int32, device=dev)
            L.kc = L.vc = None
            if not self.mt:
                L.kc = torch.empty(B, Hkv, self.cap_c, d, dtype=w.torch_dtype, device=dev)
                L.vc = torch.empty_like(L.kc)
            L.kmax = torch.empty(B, Hkv, d, rk.aux_capacity(self.cap_c, w.block), dtype=w.torch_dtype, device=dev)
            L.kmin = torch.empty_like(L.kmax)
            if self.paged:
                per_seq = -(-self.cap_c // self.paged)
                n_pages = B * per_seq
                g = torch.Generator().manual_seed(77 + r)
                L.table = torch.randperm(n_pages, generator=g).view(B, per_seq).to(torch.int32).to(dev)
                L.kp = torch.empty(n_pages, Hkv, self.paged, d, dtype=w.torch_dtype, device=dev)
                L.vp = torch.empty_like(L.kp)
                L.pages = rk.paged_kv(L.table, n_pages, self.paged)
            L.out = torch.empty(self.steps, B, Hq, d, dtype=torch.float32, device=dev)
            self.layers.append(L)

    def evict_part(self):
        rk, w = self.rk, self.w
        for L in self.layers:
            if self.mt:
                rk.rk_snapkv_evict(L.qw, L.k, L.v, self.S, w.window, w.pool, self.n_keep, L.kept, None, None,
                                   None, ws=self.ws_e)
                rk.rk_hsa_build_aux(L.k, self.n_keep, 0, w.block, L.kmax, L.kmin, n_q_heads=w.n_q, idx=L.kept)
            else:
                # the compaction builds Kmax/Kmin of the compact cache on the way
                rk.rk_snapkv_evict(L.qw, L.k, L.v, self.S, w.window, w.pool, self.n_keep, L.kept, L.kc, L.vc,
                                   None, ws=self.ws_e, kmax=L.kmax, kmin=L.kmin, block=w.block)
                if self.paged:
                    rk.rk_paged_write_kv(L.kc, L.vc, 0, self.n_keep, L.kp, L.vp, L.pages, n_q_heads=w.n_q)

    def decode_part(self):
        rk, w = self.rk, self.w
        for s in range(self.steps):
            for L in self.layers:
                if self.mt:
                    rk.rk_hsa_decode_mt(L.qs[s], L.k, L.v, L.kept, self.n_keep, L.kmax, L.kmin, w.block, w.k1,
                                        self.k2, L.out[s], ws=self.ws_d)
                elif self.paged and L.app is not None:
                    rk.rk_paged_hsa_append_decode(L.qs[s], L.app[s][0], L.app[s][1], L.kp, L.vp, L.pages,
                                                  self.n_keep + s, L.kmax, L.kmin, w.block, w.k1, self.k2,
                                                  L.out[s], ws=self.ws_d)
                elif self.paged:
                    rk.rk_paged_hsa_decode(L.qs[s], L.kp, L.vp, L.pages, L.kmax, L.kmin, self.n_keep, w.block,
                                           w.k1, self.k2, L.out[s], ws=self.ws_d)
                elif L.app is not None:   # the step appends its token, then decodes (one call)
                    rk.rk_hsa_append_decode(L.qs[s], L.app[s][0], L.app[s][1], L.kc, L.vc, self.n_keep + s,
                                            L.kmax, L.kmin, w.block, w.k1, self.k2, L.out[s], ws=self.ws_d)
                else:
                    rk.rk_hsa_decode(L.qs[s], L.kc, L.vc, L.kmax, L.kmin, self.n_keep, w.block, w.k1,
                                     self.k2, L.out[s], ws=self.ws_d)


def measure(rk, WL, name, args, dev, with_cpu):
    """Time `args.steps` steps of R layers of workload `name`; returns the
    figures of the JSON line (and the per-kernel table)."""
    import torch

    w = WL.WORKLOADS[name]
    p = Path(rk, WL, w, dev, args.layers, getattr(args, "paged", 0))
    R = p.R
    log(f"workload {w.name}: {R} layers per step, S={p.S} n_keep={p.n_keep} k1={w.k1} k2={p.k2} "
        f"decode steps={p.steps}")
    torch.cuda.synchronize()
    for _ in range(max(1, args.warmup)):           # eager warm-up (also before capture)
        p.evict_part()
        p.decode_part()
    torch.cuda.synchronize()

    use_graph = not args.no_graph
    if use_graph:
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            ge, gd = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(ge, stream=stream):
                p.evict_part()
            with torch.cuda.graph(gd, stream=stream):
                p.decode_part()
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()

    def run_step(ev):
        ev[0].record()
        ge.replay() if use_graph else p.evict_part()
        ev[1].record()
        gd.replay() if use_graph else p.decode_part()
        ev[2].record()

    for _ in range(args.warmup):
        run_step([torch.cuda.Event(enable_timing=True) for _ in range(3)])
    torch.cuda.synchronize()

    # ---- timed region ----
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    evict_ms = [e[0].elapsed_time(e[1]) / R for e in evs]                       # per layer
    dec_us = [e[1].elapsed_time(e[2]) * 1e3 / (R * p.steps) for e in evs]      # per layer-step
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    evict_ms_layer = statistics.median(evict_ms)
    dec_us_step = statistics.median(dec_us)
    log(f"wall {ms_per_step:.3f} ms/step ({R} layers); evict+aux {evict_ms_layer:.3f} ms/layer; "
        f"decode {dec_us_step:.2f} us per layer-step (medians)")

    # ---- per-kernel durations: library HIP-event timing over eager steps ----
    prof_steps = min(args.steps, 3)
    rk.rk_profile_begin()
    for _ in range(prof_steps):
        p.evict_part()
        p.decode_part()
    prof = rk.rk_profile_end()
    torch.cuda.synchronize()
    # per layer (launches and ms), and the average launch (ms)
    per_layer = {n: (c / (prof_steps * R), t / (prof_steps * R), t / c) for n, (c, t) in prof.items()}
    for n, (cpl, tpl, avg) in per_layer.items():
        log(f"kernel {n:16s} {cpl:6.1f} launches/layer {tpl:8.4f} ms/layer avg {avg * 1e3:8.2f} us")

    dominant = max(per_layer, key=lambda n: per_layer[n][1])
    roof = None
    if dominant in p.alg:
        avg_ms = per_layer[dominant][2]
        achieved = p.alg[dominant] / (avg_ms * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(dominant, w.name),
                "bytes_per_launch": p.alg[dominant], "avg_launch_us": round(avg_ms * 1e3, 3)}
    attn_name = next((n for n in ("hsa_fused_mt", "hsa_fused_append", "hsa_fused", "hsa_attn_mt", "hsa_attn")
                      if n in per_layer), "hsa_attn")
    attn_avg = per_layer.get(attn_name, (0, 0, float("nan")))[2]
    attn_gbps = p.alg[attn_name] / (attn_avg * 1e-3) / 1e9 if attn_avg == attn_avg else None
    ws_ms = sum(per_layer.get(n, (0, 0, 0))[1] for n in ("ws_pass1", "ws_stats", "ws_pass2"))
    ws1 = per_layer.get("ws_pass1", (0, 0, float("nan")))[2]
    dec_gbps = p.dec_bytes / (dec_us_step * 1e-6) / 1e9
    ws_tflops = p.flops_ws / (ws_ms * 1e-3) / 1e12 if ws_ms > 0 else None

    res = {
        "workload": w.name,
        "layers_per_step": R,
        "evict_ms_per_layer": round(evict_ms_layer, 4),
        "decode_us_per_layer_step": round(dec_us_step, 3),
        "decode_us_per_32_layer_step": round(dec_us_step * MODEL_LAYERS, 1),
        "evict_ms_per_32_layers": round(evict_ms_layer * MODEL_LAYERS, 2),
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median_events": round(statistics.median(step_ms), 4),
        "hsa_decode_GBps": round(dec_gbps, 1),
        "hsa_decode_hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "hsa_decode_bytes_per_layer_step": p.dec_bytes,
        "hsa_attn_kernel": attn_name,
        "hsa_attn_avg_us": round(attn_avg * 1e3, 3),
        "hsa_attn_GBps": round(attn_gbps, 1) if attn_gbps else None,
        "hsa_attn_hbm_frac": round(attn_gbps / HBM_PEAK_GBPS, 4) if attn_gbps else None,
        "window_scoring_us_per_layer": round(ws_ms * 1e3, 2),
        "window_scoring_TFLOPs": round(ws_tflops, 2) if ws_tflops else None,
        "window_scoring_bf16_frac": round(ws_tflops / BF16_PEAK_TFLOPS, 4) if ws_tflops else None,
        "ws_pass1_TFLOPs": round(p.flops_ws / (ws1 * 1e-3) / 1e12, 2) if ws1 == ws1 else None,
        "kernels_ms_per_layer": {n: round(v[1], 5) for n, v in per_layer.items()},
        "kernels_avg_us": {n: round(v[2] * 1e3, 3) for n, v in per_layer.items()},
        "roofline": roof,
        "config": {"workload": w.name, "layers_timed": R, "batch": w.batch, "seq_len": p.S, "n_q_heads": w.n_q,
                   "n_kv_heads": w.n_kv, "head_dim": w.d, "kv_dtype": w.dtype, "compression": round(w.c, 3),
                   "n_keep": p.n_keep, "k1": w.k1, "k2_pages": p.k2, "page": w.block, "decode_steps": p.steps,
                   "appends": w.appends, "rocketkv_mt": p.mt, "graph_replay": use_graph,
                   "paged_tokens_per_page": p.paged or None},
    }
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(w, p, args.cpu_seconds)
    del p
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def evict_compare(args):
    """Stage 1 alone: rk_snapkv_evict against rk_adakv_evict on one layer of
    each workload, both compacting and building Kmax/Kmin, the same workspace;
    medians over args.steps calls after args.warmup, plus the library's
    per-kernel times of one call."""
    import statistics

    import torch

    from sparse_decode_attention_amd import rocketkv as rk
    from sparse_decode_attention_amd import workloads as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for wname in args.evict_compare.split(","):
        w = WL.WORKLOADS[wname]
        S, W = w.seq, w.window
        n_keep = rk.rk_split(w.c, S, W, w.block, w.d)["n_keep"]
        k, v, _ = WL.layer_kv(w, 0, device=dev)
        qw = WL.window_queries(w, 0, device=dev)
        B, Hkv, d = w.batch, w.n_kv, w.d
        cap = rk.adakv_capacity(Hkv, S, W, n_keep)
        ws = torch.empty(rk.rk_snapkv_workspace_bytes(rk.shape_of(B, w.n_q, Hkv, d, k.dtype), S, W),
                         dtype=torch.uint8, device=dev)
        res = {"evict_compare": wname, "n_keep": n_keep, "ada_out_cap": cap}
        for mode in ("snapkv", "adakv"):
            oc = cap if mode == "adakv" else n_keep
            kept = torch.empty(B, Hkv, oc, dtype=torch.int32, device=dev)
            cnt = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
            kk = torch.empty(B, Hkv, oc, d, dtype=k.dtype, device=dev)
            vv = torch.empty_like(kk)
            kmax = torch.empty(B, Hkv, d, rk.aux_capacity(oc, w.block), dtype=k.dtype, device=dev)
            kmin = torch.empty_like(kmax)

            def run():
                if mode == "adakv":
                    rk.rk_adakv_evict(qw, k, v, S, W, w.pool, n_keep, kept, cnt, kk, vv, ws=ws, kmax=kmax,
                                      kmin=kmin, block=w.block)
                else:
                    rk.rk_snapkv_evict(qw, k, v, S, W, w.pool, n_keep, kept, kk, vv, None, ws=ws, kmax=kmax,
                                       kmin=kmin, block=w.block)

            for _ in range(args.warmup):
                run()
            torch.cuda.synchronize()
            times = []
            for _ in range(args.steps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                run()
                b.record()
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b))
            rk.rk_profile_begin()
            run()
            prof = rk.rk_profile_end()
            res[mode + "_ms_per_layer"] = round(statistics.median(times), 4)
            res[mode + "_kernels_us"] = {n: round(t[1] * 1e3, 1) for n, t in prof.items()}
            del kept, cnt, kk, vv, kmax, kmin
        print(json.dumps(res), flush=True)
        del k, v, qw, ws
        torch.cuda.empty_cache()


def selection_recall(args):
    """Selection quality of each method at its planned budget split (one layer,
    full prompt; RocketKV adds SnapKV eviction first), against exact attention
    over the whole prompt, on the GPU through rk_select_decode / the RocketKV
    calls.  Per (unit, step), averaged: recall = |T & E| / |T| with E the |T|
    tokens of largest accumulated logit q_bar . k; mass = the group's mean
    attention probability on T; err = rel-L2 of the output against dense
    attention; needle = the planted key is in T (the needle workload)."""
    import torch

    from sparse_decode_attention_amd import rocketkv as rk
    from sparse_decode_attention_amd import workloads as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rows = []
    for name in ("llama8b-layer-s32k-c16", "needle-s109k-c428"):
        w = WL.WORKLOADS[name]
        B, Hq, Hkv, d, G, S = w.batch, w.n_q, w.n_kv, w.d, w.group, w.seq
        k, v, pos = WL.layer_kv(w, 0, device=dev)
        qw = WL.window_queries(w, 0, device=dev)
        kf = k.float()
        qs = [WL.decode_query(w, 0, s, device=dev) for s in range(args.recall_steps)]
        # dense reference and exact scores, float32
        ref = []
        for q in qs:
            qf = q.float().view(B, Hkv, G, d)
            logits = torch.matmul(qf, kf.transpose(2, 3).contiguous()) / math.sqrt(d)   # [B,Hkv,G,S]
            p = torch.softmax(logits, dim=-1)
            o = torch.matmul(p, v.float())                                                # [B,Hkv,G,d]
            ref.append((p.mean(dim=2), o, torch.matmul(kf, qf.sum(dim=2).unsqueeze(-1)).squeeze(-1)))
        methods = []
        for m in ("exact", "hsa", "quest", "sparq"):
            methods.append((m, rk.rk_select_plan(m, w.c, S, d)))
        sp = rk.rk_split(w.c, S, w.window, w.block, d)
        methods.append(("rocketkv", dict(page=sp["paper_page"], channels=sp["paper_k1_channels"],
                                         k2=sp["paper_k2_blocks"], n_keep=sp["n_keep"])))
        methods.append(("rocketkv-w", dict(page=w.block, channels=w.k1, k2=sp["k2_blocks"], n_keep=sp["n_keep"])))
        methods.append(("rocketkv-ada", dict(page=sp["paper_page"], channels=sp["paper_k1_channels"],
                                             k2=sp["paper_k2_blocks"], n_keep=sp["n_keep"])))
        for m, p in methods:
            page, ch, k2 = p["page"], p["channels"], p["k2"]
            kmax = kmin = None
            kept = None
            kk, vv, n = k, v, S
            lens = None
            if m == "rocketkv-ada":       # shared stage-1 budget, decode per unit length
                n = rk.adakv_capacity(Hkv, S, w.window, p["n_keep"])
                kept = torch.empty(B, Hkv, n, dtype=torch.int32, device=dev)
                lens = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
                kk = torch.empty(B, Hkv, n, d, dtype=k.dtype, device=dev)
                vv = torch.empty_like(kk)
                rk.rk_adakv_evict(qw, k, v, S, w.window, w.pool, p["n_keep"], kept, lens, kk, vv)
            elif m.startswith("rocketkv"):
                n = p["n_keep"]
                kept = torch.empty(B, Hkv, n, dtype=torch.int32, device=dev)
                kk = torch.empty(B, Hkv, n, d, dtype=k.dtype, device=dev)
                vv = torch.empty_like(kk)
                rk.rk_snapkv_evict(qw, k, v, S, w.window, w.pool, n, kept, kk, vv, None)
            if m != "exact":
                kmax = torch.empty(B, Hkv, d, rk.aux_capacity(n, page), dtype=k.dtype, device=dev)
                kmin = None if m == "sparq" else torch.empty_like(kmax)
                rk.rk_hsa_build_aux(kk, n, 0, page, kmax, kmin, n_q_heads=Hq)   # (ada: past a unit's rows unused)
            nblk = -(-n // page)
            nsel = min(k2, nblk)
            sel = torch.empty(B, Hkv, nsel, dtype=torch.int32, device=dev)
            out = torch.empty(B, Hq, d, device=dev)
            method = "hsa" if m.startswith("rocketkv") else m

            def call(q, ws=None):
                if lens is not None:
                    return rk.rk_hsa_decode_ragged(q, kk, vv, kmax, kmin, lens, n, page, ch, k2, out, sel, ws=ws)
                return rk.rk_select_decode(method, q, kk, vv, kmax, kmin, n, page, ch, k2, out, sel, ws=ws)

            ws = call(qs[0])
            rec = mass = err = hit = 0.0
            cnt = 0
            tok_total = 0
            for si, q in enumerate(qs):
                call(q, ws)
                torch.cuda.synchronize()
                pbar, o_ref, sc = ref[si]
                toks = (sel.long().unsqueeze(-1) * page + torch.arange(page, device=dev)).view(B, Hkv, -1)
                lim = lens.long().unsqueeze(-1) if lens is not None else n
                valid = (toks < lim) & (sel.long().unsqueeze(-1) >= 0).expand(-1, -1, -1, page).reshape(B, Hkv, -1)
                toks = torch.where(valid, toks, torch.zeros_like(toks))
                if kept is not None:
                    toks = torch.gather(kept.long(), 2, toks)
                for b in range(B):
                    for h in range(Hkv):
                        T = torch.unique(toks[b, h][valid[b, h]])
                        nt = T.numel()
                        E = torch.topk(sc[b, h], nt).indices
                        rec += float(torch.isin(T, E).float().mean())
                        mass += float(pbar[b, h, T].sum())
                        og = out.view(B, Hkv, G, d)[b, h]
                        err += float((og - o_ref[b, h]).norm() / o_ref[b, h].norm())
                        if w.n_plant == 1:
                            hit += float(bool(torch.isin(pos[b, h, 0], T)))
                        tok_total += nt
                        cnt += 1
            # decode time per step (eager, events)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for q in qs:
                call(q, ws)
            e1.record()
            torch.cuda.synchronize()
            # estimation traffic over the pages each unit actually has
            nb_eff = float(((lens.float() + page - 1) // page).mean()) if lens is not None else nblk
            est = ch * nb_eff / (2.0 * d)
            rows.append(dict(workload=name, method=m, page=page, channels=ch, k2_pages=k2,
                             tokens_attended=round(tok_total / cnt, 1), est_pairs=round(est, 1),
                             recall=round(rec / cnt, 4), mass=round(mass / cnt, 4), out_rel_l2=round(err / cnt, 5),
                             needle_hit=round(hit / cnt, 4) if w.n_plant == 1 else None,
                             us_per_step=round(e0.elapsed_time(e1) * 1e3 / len(qs), 2)))
            log(json.dumps(rows[-1]))
            del kmax, kmin, kept, ws
        del k, v, kf, ref
        torch.cuda.empty_cache()
    print("| workload | method | page | channels | pages | tokens attended | estimation (KV pairs) | "
          "recall of exact top tokens | attention mass | output rel-L2 | needle found | us/step |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['workload']} | {r['method']} | {r['page']} | {r['channels']} | {r['k2_pages']} | "
              f"{r['tokens_attended']} | {r['est_pairs']} | {r['recall']} | {r['mass']} | {r['out_rel_l2']} | "
              f"{'' if r['needle_hit'] is None else r['needle_hit']} | {r['us_per_step']} |")
    print(json.dumps({"selection_recall": rows}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.selection_recall:
        selection_recall(args)
        return
    if args.evict_compare:
        evict_compare(args)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (the hot path shards over (batch, KV head) units "
              f"with no exchange; multi-GPU runs are not measured here); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_decode_attention_amd import rocketkv as rk
    from sparse_decode_attention_amd import workloads as WL

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    main_res = measure(rk, WL, args.workload, args, dev, not args.no_cpu_baseline)
    also = None
    if args.also and args.also != args.workload:
        a = measure(rk, WL, args.also, args, dev, False)
        also = {k: a[k] for k in ("workload", "layers_per_step", "decode_us_per_layer_step",
                                  "decode_us_per_32_layer_step", "evict_ms_per_layer", "evict_ms_per_32_layers",
                                  "hsa_decode_GBps", "hsa_decode_hbm_frac", "hsa_attn_kernel", "hsa_attn_avg_us",
                                  "hsa_attn_GBps", "hsa_attn_hbm_frac", "window_scoring_us_per_layer",
                                  "window_scoring_TFLOPs", "window_scoring_bf16_frac", "kernels_avg_us",
                                  "roofline", "config")}

    line = {
        "metric": "HSA decode us/step + HBM GB/s (% peak); SnapKV evict ms/layer",
        "value": main_res["decode_us_per_layer_step"],
        "unit": "us/step (one layer)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        # storage type of q, K and V; products accumulate in float32 either way
        "dtype": main_res["config"]["kv_dtype"],
        "data": "synthetic",
        "config": main_res["config"],
    }
    for k, v in main_res.items():
        if k not in ("config", "ms_per_step", "workload"):
            line[k] = v
    line["also"] = also
    print(json.dumps(line), flush=True)


def code_only(src):
    """C/C++ source without comments and whitespace (edits to comments keep the hash)."""
    import re

    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return re.sub(r"\s+", "", src)


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    summary (profiles/hbm_traffic_counters.md), or None when there is no row or
    the kernel's sources (comments and whitespace aside) have changed since the
    counters were taken."""
    import hashlib

    # timing-hook names -> kernel function names (the MT variants share the function)
    kernel = {"hsa_attn_mt": "hsa_attn", "hsa_fused_mt": "hsa_fused", "hsa_fused_append": "hsa_fused",
              "select_tokens": "select",
              "gather_kv": "gather"}.get(kernel, kernel)
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "hbm_traffic_counters.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) != 8 or cells[0] != kernel or cells[1] != workload:
            continue
        h = hashlib.sha256()
        for n in ("rk_device.hpp", "rk_internal.hpp", cells[6]):
            with open(os.path.join(root, "sparse_decode_attention_amd", "csrc", n)) as f:
                h.update(code_only(f.read()).encode())
        return round(float(cells[5]) * 1e6) if h.hexdigest()[:12] == cells[7] else None
    return None


def cpu_baseline(w, p, budget_s):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import oracle as O

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    L = p.layers[0]
    k, v, qw, qs = L.k, L.v, L.qw, L.qs
    G = w.group
    S, W = p.S, w.window
    units_all = [(b, h) for b in range(w.batch) for h in range(w.n_kv)]

    def stage1(b, h):
        kn = k[b, h, :S].float().cpu().numpy()
        vn = v[b, h, :S].float().cpu().numpy()
        pl = O.pool_sum(O.window_scores(qw[b, h * G:(h + 1) * G].float().cpu().numpy(), kn), w.pool)
        kept = O.snapkv_select(pl, S, W, p.n_keep)
        kc, vc = kn[kept], vn[kept]
        kmax, kmin = O.build_aux(kc, p.n_keep, w.block)
        return kc, vc, kmax, kmin

    t0 = time.perf_counter()
    caches = {units_all[0]: stage1(*units_all[0])}
    evict_unit_ms = (time.perf_counter() - t0) * 1e3
    # decode over the units of batch 0 (all of them for single-sequence workloads)
    units = [u for u in units_all if u[0] == 0]
    for u in units[1:]:
        caches[u] = stage1(*u)
    qn = qs.float().cpu().numpy()
    t0 = time.perf_counter()
    done = 0
    while done < p.steps and time.perf_counter() - t0 < budget_s:
        for b, h in units:
            c = caches[(b, h)]
            O.hsa_unit(qn[done, b, h * G:(h + 1) * G], c[0], c[1], c[2], c[3], p.n_keep, w.block, w.k1, p.k2)
        done += 1
    per_step_us = (time.perf_counter() - t0) * 1e6 / max(done, 1) * (len(units_all) / len(units))
    return {"value": round(per_step_us, 1), "unit": "us/step (one layer)", "cores": cores,
            "blas_threads": blas_threads, "kind": "oracle",
            "sample": f"HSA decode of {len(units)} of {len(units_all)} units for {done} of {p.steps} steps "
                      f"of one layer, scaled to all units (aux built once; for RocketKV-MT over the "
                      f"compacted candidate rows, which is the same arithmetic); stage 1 of one unit "
                      f"{evict_unit_ms:.0f} ms, x{len(units_all)} units = "
                      f"{evict_unit_ms * len(units_all):.0f} ms/layer (extrapolated)",
            "evict_ms_per_layer_extrapolated": round(evict_unit_ms * len(units_all), 1)}


if __name__ == "__main__":
    main()

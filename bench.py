#!/usr/bin/env python3
"""Benchmark of the RocketKV hot path on one MI355X.

Default workload: the Llama-3.1-8B-shaped single layer (batch 1, 32K prompt,
32 query / 8 KV heads, d 128, bf16, c = 16).  A step is one pass of the whole
hot path over one batch of synthetic input: the adaptive split, SnapKV
eviction of the layer (window scoring, pooling, top-k, compaction), the
Kmax/Kmin build and the workload's HSA decode steps.  `--workload` runs one
layer of another workload instead (the batch-32 stack: append + decode per
step; the 109K needle; the last RocketKV-MT turn: index-only eviction of the
resident full cache, aux over the candidates, MT decode).

Inputs are resident in HBM before timing; steps rotate over enough prompt
replicas that eviction does not re-read a cache-resident K.  Each step is
replayed from two HIP graphs (eviction + aux, then the decode calls) with HIP
events between them.  Reported: `value` = HSA decode time per decode step
(us), `ms_per_step` = one whole pass, SnapKV eviction ms/layer, decode HBM
GB/s, the roofline of the dominant kernel (per-kernel durations from the
library's HIP-event timing over an eager pass of the same steps) and the CPU
oracle timed on a bounded sample on the host.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import json
import math
import sys
import time

HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b-layer-s32k-c16")
    ap.add_argument("--replicas", type=int, default=0, help="prompt replicas (0: enough to exceed 512 MB)")
    ap.add_argument("--no-graph", action="store_true", help="issue every call eagerly instead of graph replay")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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


class Path:
    """Buffers and calls of one layer of a workload (one replica per prompt)."""

    def __init__(self, rk, WL, w, dev, replicas):
        import torch

        self.rk, self.w = rk, w
        self.mt = w.mt_turns > 0
        self.S = w.seq + (w.mt_turns * w.mt_append if self.mt else 0)   # MT: the last turn
        sp = rk.rk_split(w.c, self.S, w.window, w.block, w.d)
        self.n_keep, self.k2 = sp["n_keep"], WL.stage2_pages(w, sp)
        self.steps = w.decode_steps
        B, Hq, Hkv, d = w.batch, w.n_q, w.n_kv, w.d
        cap_c = self.n_keep + (self.steps if w.appends else 0)
        self.nblk = -(-cap_c // w.block)
        esize = 2 if w.dtype == "bf16" else 4
        kv_bytes = 2 * B * Hkv * self.S * d * esize
        R = replicas or max(1, min(4, math.ceil(512e6 / kv_bytes)))
        self.R = R
        self.reps = []
        for r in range(R):
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
                qw = WL.window_queries(w, r, device=dev, turn=w.mt_turns - 1)
                qs = torch.stack([WL.decode_query(w, r, (w.mt_turns - 1) * self.steps + s, device=dev)
                                  for s in range(self.steps)])
            else:
                k, v, _ = WL.layer_kv(w, r, device=dev)
                qw = WL.window_queries(w, r, device=dev)
                qs = torch.stack([WL.decode_query(w, r, s, device=dev) for s in range(self.steps)])
            app = None
            if w.appends:
                app = [WL.append_kv(w, r, s, device=dev) for s in range(self.steps)]
            self.reps.append((k, v, qw, qs, app))
        self.kept = torch.empty(B, Hkv, self.n_keep, dtype=torch.int32, device=dev)
        self.kc = self.vc = None
        if not self.mt:
            self.kc = torch.empty(B, Hkv, cap_c, d, dtype=w.torch_dtype, device=dev)
            self.vc = torch.empty_like(self.kc)
        self.kmax = torch.empty(B, Hkv, d, rk.aux_capacity(cap_c, w.block), dtype=w.torch_dtype, device=dev)
        self.kmin = torch.empty_like(self.kmax)
        self.out = torch.empty(self.steps, B, Hq, d, dtype=torch.float32, device=dev)
        shape = rk.shape_of(B, Hq, Hkv, d, w.torch_dtype)
        self.ws_e = torch.empty(rk.rk_snapkv_workspace_bytes(shape, self.S, w.window), dtype=torch.uint8, device=dev)
        self.ws_d = torch.empty(rk.rk_hsa_workspace_bytes(shape, cap_c, w.block, w.k1, self.k2),
                                dtype=torch.uint8, device=dev)
        # algorithmic bytes per launch (what the method must move)
        units = B * Hkv
        nb0 = -(-self.n_keep // w.block)
        nsel = min(self.k2, self.nblk)
        G = w.group
        self.alg = {
            "hsa_attn": units * nsel * w.block * 2 * d * esize + B * Hq * d * esize,
            "hsa_attn_mt": units * nsel * w.block * (2 * d * esize + 4) + B * Hq * d * esize,
            "hsa_score": units * w.k1 * nb0 * esize + B * Hq * d * esize,
            "hsa_fused": units * w.k1 * nb0 * esize + units * nsel * w.block * 2 * d * esize
            + B * Hq * d * esize,
            "hsa_fused_mt": units * w.k1 * nb0 * esize + units * nsel * w.block * (2 * d * esize + 4)
            + B * Hq * d * esize,
            "aux_build": units * self.n_keep * d * esize + 2 * units * d * nb0 * esize,
            "gather_kv": 2 * 2 * units * self.n_keep * d * esize + 2 * units * d * nb0 * esize,
            "ws_pass1": units * self.S * d * esize + B * Hq * w.window * d * esize,
            "ws_pass2": units * (self.S - w.window) * d * esize + B * Hq * w.window * d * esize,
            "append_kv": units * d * esize * 5,
        }
        # the one-launch decode step with its append: the fused bytes plus the append's
        self.alg["hsa_fused_append"] = self.alg["hsa_fused"] + self.alg["append_kv"]
        self.flops_ws = 2.0 * units * G * w.window * self.S * d
        self.dec_bytes = self.alg["hsa_attn_mt" if self.mt else "hsa_attn"] + self.alg["hsa_score"]

    def evict_part(self, r):
        rk, w = self.rk, self.w
        k, v, qw = self.reps[r][:3]
        if self.mt:
            rk.rk_snapkv_evict(qw, k, v, self.S, w.window, w.pool, self.n_keep, self.kept, None, None, None,
                               ws=self.ws_e)
            rk.rk_hsa_build_aux(k, self.n_keep, 0, w.block, self.kmax, self.kmin, n_q_heads=w.n_q, idx=self.kept)
        else:
            # the compaction builds Kmax/Kmin of the compact cache on the way
            rk.rk_snapkv_evict(qw, k, v, self.S, w.window, w.pool, self.n_keep, self.kept, self.kc, self.vc,
                               None, ws=self.ws_e, kmax=self.kmax, kmin=self.kmin, block=w.block)

    def decode_part(self, r):
        rk, w = self.rk, self.w
        k, v, _, qs, app = self.reps[r]
        for s in range(self.steps):
            if self.mt:
                rk.rk_hsa_decode_mt(qs[s], k, v, self.kept, self.n_keep, self.kmax, self.kmin, w.block, w.k1,
                                    self.k2, self.out[s], ws=self.ws_d)
            else:
                if app is not None:   # the step appends its token, then decodes (one call)
                    rk.rk_hsa_append_decode(qs[s], app[s][0], app[s][1], self.kc, self.vc, self.n_keep + s,
                                            self.kmax, self.kmin, w.block, w.k1, self.k2, self.out[s],
                                            ws=self.ws_d)
                else:
                    rk.rk_hsa_decode(qs[s], self.kc, self.vc, self.kmax, self.kmin, self.n_keep, w.block, w.k1,
                                     self.k2, self.out[s], ws=self.ws_d)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
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
    w = WL.WORKLOADS[args.workload]
    p = Path(rk, WL, w, dev, args.replicas)
    R = p.R
    log(f"workload {w.name} (one layer): S={p.S} n_keep={p.n_keep} k1={w.k1} k2={p.k2} "
        f"decode steps={p.steps} replicas={R}")
    torch.cuda.synchronize()

    for i in range(max(1, args.warmup)):           # eager warm-up (also before capture)
        p.evict_part(i % R)
        p.decode_part(i % R)
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
                    p.evict_part(r)
                with torch.cuda.graph(gd, stream=stream):
                    p.decode_part(r)
                graphs.append((ge, gd))
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()

    def run_step(i, ev):
        r = i % R
        ev[0].record()
        graphs[r][0].replay() if use_graph else p.evict_part(r)
        ev[1].record()
        graphs[r][1].replay() if use_graph else p.decode_part(r)
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
    evict_ms_layer = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    dec_us_step = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps * 1e3 / p.steps
    log(f"wall {ms_per_step:.3f} ms/step; evict+aux {evict_ms_layer:.3f} ms/layer; decode {dec_us_step:.2f} us/step")

    # ---- per-kernel durations: library HIP-event timing over an eager pass ----
    rk.rk_profile_begin()
    for i in range(args.steps):
        p.evict_part(i % R)
        p.decode_part(i % R)
    prof = rk.rk_profile_end()
    torch.cuda.synchronize()
    per_step = {n: (c / args.steps, t / args.steps, t / c) for n, (c, t) in prof.items()}
    for n, (cps, tps, avg) in per_step.items():
        log(f"kernel {n:14s} {cps:6.1f} launches/step {tps:8.4f} ms/step avg {avg * 1e3:8.2f} us")

    dominant = max(per_step, key=lambda n: per_step[n][1])
    avg_ms = per_step[dominant][2]
    roof = None
    if dominant in p.alg:
        achieved = p.alg[dominant] / (avg_ms * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(dominant, w.name),
                "bytes_per_launch": p.alg[dominant], "avg_launch_us": round(avg_ms * 1e3, 3)}
    attn_name = next((n for n in ("hsa_fused_mt", "hsa_fused_append", "hsa_fused", "hsa_attn_mt", "hsa_attn")
                      if n in per_step),
                     "hsa_attn")
    attn_avg = per_step.get(attn_name, (0, 0, float("nan")))[2]
    attn_gbps = p.alg[attn_name] / (attn_avg * 1e-3) / 1e9 if attn_avg == attn_avg else None
    ws1 = per_step.get("ws_pass1", (0, 0, float("nan")))[2]
    dec_gbps = p.dec_bytes / (dec_us_step * 1e-6) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, p, args.cpu_seconds)

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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers_timed": 1, "batch": w.batch, "seq_len": p.S, "n_q_heads": w.n_q,
                   "n_kv_heads": w.n_kv, "head_dim": w.d, "kv_dtype": w.dtype, "compression": round(w.c, 3),
                   "n_keep": p.n_keep, "k1": w.k1, "k2_pages": p.k2, "page": w.block, "decode_steps": p.steps,
                   "appends": w.appends, "rocketkv_mt": p.mt, "replicas": R, "graph_replay": use_graph},
        "snapkv_evict_ms_per_layer": round(evict_ms_layer, 4),
        "hsa_decode_GBps": round(dec_gbps, 1),
        "hsa_decode_hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "hsa_attn_avg_us": round(attn_avg * 1e3, 3),
        "hsa_attn_GBps": round(attn_gbps, 1) if attn_gbps else None,
        "window_scoring_TFLOPs": round(p.flops_ws / (ws1 * 1e-3) / 1e12, 2) if ws1 == ws1 else None,
        "kernels_ms_per_step": {n: round(v[1], 5) for n, v in per_step.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
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
    import os

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
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    k, v, qw, qs, _ = p.reps[0]
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
    return {"value": round(per_step_us, 1), "unit": "us/step", "cores": threads, "kind": "oracle",
            "sample": f"HSA decode of {len(units)} of {len(units_all)} units for {done} of {p.steps} steps, "
                      f"scaled to all units (aux built once); stage 1 of one unit {evict_unit_ms:.0f} ms, "
                      f"x{len(units_all)} units = {evict_unit_ms * len(units_all):.0f} ms/layer (extrapolated)",
            "evict_ms_per_layer_extrapolated": round(evict_unit_ms * len(units_all), 1)}


if __name__ == "__main__":
    main()

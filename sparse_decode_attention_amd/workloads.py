"""Seeded synthetic workloads for the RocketKV hot path.

This module only draws inputs: it holds none of the method's arithmetic (no
scoring, pooling, selection, aux build or attention).  Both the HIP path and
the CPU oracle are fed from it; neither is imported here.

Recipe (the same for every workload, sizes per workload below):
  * q_hat = sqrt(d) * u, u a seeded random unit vector: unit per-coordinate RMS,
    the same scale as the N(0, 1) key rows ("unit direction" read as unit RMS;
    ``qhat_scale="unit"`` gives |q_hat| = 1 instead).
  * K, V ~ N(0, 1) (standard deviation 1).  A seeded set of outlier channels
    of K is scaled after the draw.
  * Planted keys: distinct positions drawn uniformly from the prefix
    [0, S - W) per (layer, batch, kv-head); each planted K row is overwritten
    with a * q_hat + N(0, sigma); V is left as drawn.
  * Window queries (last W positions, every query head) and decode queries:
    q_hat + N(0, 0.5), independent per head, row and step.
  * Values are drawn in float32, then rounded to bf16 (round to nearest even)
    for bf16 workloads.
Every tensor has its own generator stream keyed by (workload, layer, tensor,
step), so any slice can be regenerated on its own.
"""

from __future__ import annotations

import dataclasses
import math
import zlib

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    seq: int
    n_q: int
    n_kv: int
    d: int
    dtype: str              # "f32" | "bf16"
    window: int
    pool: int
    c: float                # total compression ratio S / t
    block: int
    k1: int
    decode_steps: int
    n_plant: int
    plant_scale: float
    plant_sigma: float
    n_outlier: int
    outlier_scale: float
    appends: bool = False   # one new K/V row per decode step (incremental aux)
    mt_turns: int = 0       # RocketKV-MT turns (0: plain RocketKV)
    mt_append: int = 0      # tokens appended to the full cache per turn
    qhat_scale: str = "sqrt_d"
    paper_split: bool = False  # page, k1 and k2 from the notes' own decomposition

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def units(self) -> int:
        return self.batch * self.n_kv


WORKLOADS = {
    w.name: w
    for w in [
        # tiny GQA, fp32, one layer: the case the oracle finishes in seconds
        Workload("tiny-gqa-s2048-d64-fp32", 1, 1, 2048, 8, 2, 64, "f32", 16, 7, 8.0, 16, 16, 8,
                 16, 3.0, 0.3, 4, 8.0),
        # Llama-3.1-8B-shaped single layer, 32K prompt, budget 2048
        Workload("llama8b-layer-s32k-c16", 1, 1, 32768, 32, 8, 128, "bf16", 32, 63, 16.0, 16, 64, 64,
                 256, 3.0, 0.3, 8, 6.0),
        # the same layer with the notes' own decomposition: pages of ceil(c^((1-r)/2)) = 3
        # tokens, k1 = round(d * page / c^(1-r)) = 81, half the budget (342 pages) to step 3
        Workload("llama8b-layer-s32k-c16-paper", 1, 1, 32768, 32, 8, 128, "bf16", 32, 63, 16.0, 3, 81,
                 64, 256, 3.0, 0.3, 8, 6.0, paper_split=True),
        # Llama-3.1-8B-shaped full stack, batch 32, budget 512, per-step appends
        Workload("llama8b-stack-b32-s32k-c64", 32, 32, 32768, 32, 8, 128, "bf16", 32, 63, 64.0, 16, 32,
                 32, 256, 3.0, 0.3, 8, 6.0, appends=True),
        # 109K-token needle, budget 256 (c = 428)
        Workload("needle-s109k-c428", 32, 1, 109568, 32, 8, 128, "bf16", 32, 63, 109568 / 256, 16, 16,
                 128, 1, 4.0, 0.0, 0, 1.0),
        # RocketKV-MT on an MHA shape, batch 8, 4 turns of 64 steps, +1024 tokens per turn
        Workload("mt-mha-b8-s32k-c32", 32, 8, 32768, 32, 32, 128, "bf16", 32, 63, 32.0, 16, 32,
                 64, 256, 3.0, 0.3, 8, 6.0, mt_turns=4, mt_append=1024),
    ]
}

def stage2_pages(w: Workload, split: dict) -> int:
    """k2 of the workload, taken from a split result: the whole budget in pages
    of w.block tokens, or the notes' step-3 half when w.paper_split."""
    return split["paper_k2_blocks"] if w.paper_split else split["k2_blocks"]


_TENSOR_IDS = {"qhat": 1, "outliers": 2, "k": 3, "v": 4, "plant_pos": 5, "plant_noise": 6,
               "q_win": 7, "q_dec": 8, "k_app": 9, "v_app": 10, "k_turn": 11, "v_turn": 12,
               "q_turn_win": 13}


def _gen(w: Workload, tensor: str, layer: int = 0, step: int = 0, device="cpu", seed: int = 0):
    key = f"{seed}|{w.name}|{_TENSOR_IDS[tensor]}|{layer}|{step}".encode()
    g = torch.Generator(device=device)
    g.manual_seed(zlib.crc32(key) * 2654435761 % (1 << 62))
    return g


def qhat(w: Workload, device="cpu", seed: int = 0) -> torch.Tensor:
    """The workload's fixed query direction, float32 [d]."""
    u = torch.randn(w.d, generator=_gen(w, "qhat", device=device, seed=seed), device=device)
    u = u / u.norm()
    return u * (math.sqrt(w.d) if w.qhat_scale == "sqrt_d" else 1.0)


def outlier_channels(w: Workload, device="cpu", seed: int = 0) -> torch.Tensor:
    perm = torch.randperm(w.d, generator=_gen(w, "outliers", device=device, seed=seed), device=device)
    return perm[: w.n_outlier]


def _background_k(w: Workload, shape, tensor: str, layer: int, step: int, device, seed) -> torch.Tensor:
    k = torch.randn(*shape, generator=_gen(w, tensor, layer, step, device, seed), device=device)
    if w.n_outlier:
        ch = outlier_channels(w, device, seed)
        k[..., ch] *= w.outlier_scale
    return k


def layer_kv(w: Workload, layer: int, device="cpu", seed: int = 0, seq: int | None = None):
    """Prompt K, V [B, H_kv, S, d] in the workload dtype, plus planted positions
    [B, H_kv, n_plant] (int64) of the planted keys."""
    S = w.seq if seq is None else seq
    shape = (w.batch, w.n_kv, S, w.d)
    k = _background_k(w, shape, "k", layer, 0, device, seed)
    v = torch.randn(*shape, generator=_gen(w, "v", layer, 0, device, seed), device=device)
    units = w.batch * w.n_kv
    pos = torch.empty(units, 0, dtype=torch.long, device=device)
    if w.n_plant:
        r = torch.rand(units, S - w.window, generator=_gen(w, "plant_pos", layer, 0, device, seed),
                       device=device)
        pos = r.topk(w.n_plant, dim=1).indices                      # distinct per unit
        rows = w.plant_scale * qhat(w, device, seed).expand(units, w.n_plant, w.d).clone()
        if w.plant_sigma > 0:
            rows += w.plant_sigma * torch.randn(units, w.n_plant, w.d,
                                                generator=_gen(w, "plant_noise", layer, 0, device, seed),
                                                device=device)
        kf = k.view(units, S, w.d)
        kf.scatter_(1, pos[..., None].expand(-1, -1, w.d), rows)
    return (k.to(w.torch_dtype), v.to(w.torch_dtype),
            pos.view(w.batch, w.n_kv, w.n_plant))


def window_queries(w: Workload, layer: int, device="cpu", seed: int = 0, turn: int = -1) -> torch.Tensor:
    """Observation-window queries [B, H_q, W, d] (turn >= 0: that MT turn's window)."""
    tensor, step = ("q_win", 0) if turn < 0 else ("q_turn_win", turn)
    noise = torch.randn(w.batch, w.n_q, w.window, w.d, generator=_gen(w, tensor, layer, step, device, seed),
                        device=device)
    return (qhat(w, device, seed) + 0.5 * noise).to(w.torch_dtype)


def decode_query(w: Workload, layer: int, step: int, device="cpu", seed: int = 0) -> torch.Tensor:
    """Decode query of one step [B, H_q, d]."""
    noise = torch.randn(w.batch, w.n_q, w.d, generator=_gen(w, "q_dec", layer, step, device, seed),
                        device=device)
    return (qhat(w, device, seed) + 0.5 * noise).to(w.torch_dtype)


def append_kv(w: Workload, layer: int, step: int, device="cpu", seed: int = 0):
    """The K, V row appended at a decode step, each [B, H_kv, d]."""
    shape = (w.batch, w.n_kv, w.d)
    k = _background_k(w, shape, "k_app", layer, step, device, seed)
    v = torch.randn(*shape, generator=_gen(w, "v_app", layer, step, device, seed), device=device)
    return k.to(w.torch_dtype), v.to(w.torch_dtype)


def turn_kv(w: Workload, layer: int, turn: int, device="cpu", seed: int = 0):
    """The mt_append new plain N(0, 1) K, V tokens of an MT turn, [B, H_kv, n, d]."""
    shape = (w.batch, w.n_kv, w.mt_append, w.d)
    k = torch.randn(*shape, generator=_gen(w, "k_turn", layer, turn, device, seed), device=device)
    v = torch.randn(*shape, generator=_gen(w, "v_turn", layer, turn, device, seed), device=device)
    return k.to(w.torch_dtype), v.to(w.torch_dtype)


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(w, **changes)

"""Seeded workload generators (CPU) and the oracle on the tiny GQA workload."""

import numpy as np
import torch

import oracle as O
from sparse_decode_attention_amd import workloads as WL

TINY = WL.WORKLOADS["tiny-gqa-s2048-d64-fp32"]


def test_generators_are_deterministic_and_shaped():
    k1, v1, p1 = WL.layer_kv(TINY, 0)
    k2, v2, p2 = WL.layer_kv(TINY, 0)
    assert torch.equal(k1, k2) and torch.equal(v1, v2) and torch.equal(p1, p2)
    assert k1.shape == (1, 2, 2048, 64) and k1.dtype == torch.float32
    assert p1.shape == (1, 2, 16)
    for h in range(2):
        pos = p1[0, h]
        assert len(set(pos.tolist())) == 16 and int(pos.max()) < 2048 - TINY.window
    k3, _, _ = WL.layer_kv(TINY, 1)
    assert not torch.equal(k1, k3)
    q = WL.window_queries(TINY, 0)
    assert q.shape == (1, 8, 16, 64)
    assert WL.decode_query(TINY, 0, 3).shape == (1, 8, 64)
    assert abs(float(WL.qhat(TINY).norm()) - 8.0) < 1e-4          # sqrt(d) * unit vector


def test_bf16_cast_is_round_to_nearest_even():
    w = WL.scaled(WL.WORKLOADS["llama8b-layer-s32k-c16"], seq=256, n_plant=4)
    k, v, _ = WL.layer_kv(w, 0)
    assert k.dtype == torch.bfloat16 and k.shape == (1, 8, 256, 128)


def test_oracle_keeps_and_selects_planted_keys_tiny():
    """On the tiny workload the planted high-affinity keys survive stage 1 and
    their pages win stage 2 (a property of the workload under the oracle)."""
    s = O.split(TINY.c, TINY.seq, TINY.window, TINY.block, TINY.d)
    assert s["n_keep"] == 930 and s["k2_blocks"] == 16
    k, v, pos = WL.layer_kv(TINY, 0)
    qw = WL.window_queries(TINY, 0)
    ev = O.snapkv_evict(qw.numpy(), k.numpy(), v.numpy(), TINY.window, TINY.pool, s["n_keep"])
    for h in range(TINY.n_kv):
        assert set(pos[0, h].tolist()) <= set(ev["kept"][0, h].tolist())
    q = WL.decode_query(TINY, 0, 0).numpy()
    res = O.hsa_decode(q, ev["k"], ev["v"], s["n_keep"], TINY.block, TINY.k1, s["k2_blocks"])
    for h in range(TINY.n_kv):
        kept = ev["kept"][0, h]
        compact_pos = np.searchsorted(kept, pos[0, h].numpy())
        assert set((compact_pos // TINY.block).tolist()) <= set(res["sel"][h].tolist())

"""GPU parity of Ada-KV stage 1 (a sequence's budget shared by its KV heads)
and of the decode over units of different lengths, against the oracle."""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import rk_testutil as U
from sparse_decode_attention_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda"
LLAMA = WL.WORKLOADS["llama8b-layer-s32k-c16"]
TINY = WL.WORKLOADS["tiny-gqa-s2048-d64-fp32"]


@pytest.fixture(scope="module")
def rk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_decode_attention_amd import rocketkv
    return rocketkv


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def ada_evict_and_check(rk, w, n_keep, block=16, aux=True, kvq=None, pool_op="sum"):
    """rk_adakv_evict on layer 0 of w (or on the given K, V and window
    queries), checked against the oracle; returns the GPU's kept counts,
    compact cache and aux."""
    if kvq is None:
        k, v, _ = WL.layer_kv(w, 0, device=DEV)
        qw = WL.window_queries(w, 0, device=DEV)
    else:
        k, v, qw = kvq
    B, Hkv, S, d = k.shape
    W = w.window
    G = w.group
    cap = rk.adakv_capacity(Hkv, S, W, n_keep)
    kept = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(B, Hkv, dtype=torch.int32, device=DEV)
    ko = torch.empty(B, Hkv, cap, d, dtype=k.dtype, device=DEV)
    vo = torch.empty_like(ko)
    pooled = torch.empty(B, Hkv, S - W, device=DEV)
    kmax = kmin = None
    if aux:
        kmax = torch.full((B, Hkv, d, rk.aux_capacity(cap, block)), 7.0, dtype=k.dtype, device=DEV)
        kmin = torch.full_like(kmax, 7.0)
    rk.rk_adakv_evict(qw, k, v, S, W, w.pool, n_keep, kept, cnt, ko, vo, pooled, kmax=kmax, kmin=kmin, block=block,
                      pool_op=pool_op)
    torch.cuda.synchronize()
    counts = cnt.cpu().numpy()
    assert (counts.sum(axis=1) == Hkv * n_keep).all()
    swaps = 0
    for b in range(B):
        g_pl = U.np32(pooled[b])
        o_pl = np.stack([O.pool(O.window_scores(U.np32(qw[b, h * G:(h + 1) * G]), U.np32(k[b, h])), w.pool,
                                pool_op) for h in range(Hkv)])
        np.testing.assert_allclose(g_pl, o_pl, rtol=1e-4, atol=1e-6 * float(np.abs(o_pl).max()))
        mine = O.adakv_select(g_pl, S, W, n_keep)       # exact on the GPU's own pooled scores
        want = O.adakv_select(o_pl, S, W, n_keep)       # the oracle's: near-tie swaps only
        P = S - W
        got_flat, want_flat = [], []
        for h in range(Hkv):
            c = int(counts[b, h])
            g = kept[b, h, :c].cpu().numpy()
            assert g.tolist() == mine[h].tolist(), (b, h)
            got_flat += (h * P + g[:-W]).tolist()
            want_flat += (h * P + want[h][:-W]).tolist()
            idx = torch.as_tensor(g, dtype=torch.long, device=DEV)
            assert torch.equal(ko[b, h, :c], k[b, h, idx]) and torch.equal(vo[b, h, :c], v[b, h, idx])
            if aux:
                nb = -(-c // block)
                wmax, wmin = O.build_aux(U.np32(ko[b, h, :c]), c, block)
                assert np.array_equal(U.np32(kmax[b, h, :, :nb]), wmax), (b, h)
                assert np.array_equal(U.np32(kmin[b, h, :, :nb]), wmin), (b, h)
        swaps += U.compare_sets(np.array(got_flat), np.array(want_flat), o_pl.reshape(-1))
    say("  counts per head", counts.tolist()[:2], "swaps", swaps)
    return cnt, ko, vo, kmax, kmin, cap


@pytest.mark.parametrize("w,n_keep", [
    (WL.scaled(TINY, batch=2), 930),                                       # fp32 d 64, pool 7
    (WL.scaled(LLAMA, batch=2, seq=3000, n_plant=32), 900),                # bf16, 16K keys per sequence: staged
    (WL.scaled(LLAMA, batch=1, seq=9000, n_plant=64), 2000),               # 72K keys per sequence: read from L2
])
def test_adakv_evict(rk, w, n_keep):
    say("adakv evict", w.name, w.batch, w.n_kv, w.seq, n_keep)
    ada_evict_and_check(rk, w, n_keep, block=w.block)


@pytest.mark.parametrize("B,seq,n_keep", [
    (2, 5000, 1200),     # 40K keys per sequence, two sequences: the many-workgroup cut
    (1, 9000, 9000),     # budget covers every key
    (1, 9000, 32),       # budget is the window alone
])
def test_adakv_evict_many_workgroup_select(rk, B, seq, n_keep):
    """Sequences with more pooled keys than one workgroup's LDS holds: the
    shared cut comes from the radix select spread over many workgroups."""
    w = WL.scaled(LLAMA, batch=B, seq=seq, n_plant=32)
    assert n_keep in (w.window, seq) or w.n_kv * (seq - w.window) * 4 > 140 * 1024
    say("adakv evict, many-workgroup select", B, seq, n_keep)
    ada_evict_and_check(rk, w, n_keep, block=w.block)


def test_adakv_tied_heads_many_workgroup_select(rk):
    """The even heads hold one head's keys and queries and the odd heads
    another's, so every pooled value appears four times and the cut falls
    inside a run of equal keys spread over heads: the lower heads take
    theirs first."""
    w = WL.scaled(LLAMA, batch=2, seq=6000, n_plant=16)
    say("adakv evict, tied heads", w.batch, w.seq)
    k, v, _ = WL.layer_kv(w, 0, device=DEV)
    qw = WL.window_queries(w, 0, device=DEV)
    G = w.group
    k = k[:, :2].repeat(1, 4, 1, 1).contiguous()
    v = v[:, :2].repeat(1, 4, 1, 1).contiguous()
    qw = qw[:, :2 * G].repeat(1, 4, 1, 1).contiguous()
    cnt = ada_evict_and_check(rk, w, 1500, block=w.block, kvq=(k, v, qw))[0].cpu().numpy()
    # heads with the same data: the lower one never keeps fewer
    assert (cnt[:, :2] >= cnt[:, 6:]).all()


@pytest.mark.parametrize("B,seq,n_keep", [(2, 3000, 900), (1, 9000, 2000)])
def test_adakv_evict_max_pooling(rk, B, seq, n_keep):
    """The max reading of the pooling under the shared budget: one workgroup
    per sequence (16K keys) and the many-workgroup select (72K keys)."""
    w = WL.scaled(LLAMA, batch=B, seq=seq, n_plant=32)
    say("adakv evict, max pooling", B, seq, n_keep)
    ada_evict_and_check(rk, w, n_keep, block=w.block, pool_op="max")


def test_adakv_all_keys_equal_many_workgroup_select(rk):
    """Every key row the same vector and every head the same queries: each
    window row spreads its probability evenly, and every head computes the
    same values, so with pool kernel 1 every pooled score of the sequence is
    one value and the whole budget goes in flattened order: head 0 takes its
    whole prefix, head 1 the rest of the budget, later heads nothing.  (With
    different queries per head the heads' even scores differ in the last
    bits, through the rounding of their logits, and the cut follows those.)"""
    w = WL.scaled(LLAMA, batch=1, seq=9000, n_plant=0, pool=1)
    say("adakv evict, all keys equal", w.batch, w.seq)
    k, v, _ = WL.layer_kv(w, 0, device=DEV)
    qw = WL.window_queries(w, 0, device=DEV)
    k = k[:, :1, :1].expand(-1, w.n_kv, k.shape[2], -1).contiguous()
    qw = qw[:, :w.group].repeat(1, w.n_kv, 1, 1).contiguous()
    P = w.seq - w.window
    n_keep = w.window + (3 * P) // (2 * w.n_kv)         # budget: 1.5 heads' prefixes
    cnt = ada_evict_and_check(rk, w, n_keep, block=w.block, kvq=(k, v, qw))[0].cpu().numpy()
    budget = w.n_kv * (n_keep - w.window)
    want = [min(P, max(0, budget - h * P)) + w.window for h in range(w.n_kv)]
    assert cnt[0].tolist() == want, (cnt[0].tolist(), want)


def test_adakv_equal_heads_is_snapkv(rk):
    """Every head with the same keys and queries: the shared budget splits
    evenly and the result is rk_snapkv_evict's.  Pool kernel 1, so the cut
    has no tie: with wide pooling, runs of equal pooled values around a
    planted key often straddle the cut in every head, and those ties go to
    the lower head (as the oracle's rule says), so the split is then uneven."""
    say("adakv, equal heads")
    w = WL.scaled(LLAMA, batch=1, n_kv=4, n_q=16, seq=1500, n_plant=8, pool=1)
    k, v, _ = WL.layer_kv(w, 0, device=DEV)
    qw = WL.window_queries(w, 0, device=DEV)
    k = k[:, :1].expand(-1, 4, -1, -1).contiguous()
    v = v[:, :1].expand(-1, 4, -1, -1).contiguous()
    qw = qw[:, :4].repeat(1, 4, 1, 1).contiguous()
    n_keep = 500
    cap = rk.adakv_capacity(4, 1500, w.window, n_keep)
    kept = torch.empty(1, 4, cap, dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, 4, dtype=torch.int32, device=DEV)
    rk.rk_adakv_evict(qw, k, v, 1500, w.window, w.pool, n_keep, kept, cnt)
    ref = torch.empty(1, 4, n_keep, dtype=torch.int32, device=DEV)
    rk.rk_snapkv_evict(qw, k, v, 1500, w.window, w.pool, n_keep, ref)
    torch.cuda.synchronize()
    assert cnt.cpu().tolist() == [[n_keep] * 4]
    assert torch.equal(kept[..., :n_keep], ref)


@pytest.mark.parametrize("B,n_keep", [(2, 900), (20, 400)])
def test_ragged_decode_after_adakv(rk, B, n_keep):
    """Decode over the Ada-KV compact cache, each unit its own length: split
    path (16 units) and fused path (160 units)."""
    say("ragged decode", B, n_keep)
    w = WL.scaled(LLAMA, batch=B, seq=3000, n_plant=32)
    cnt, kc, vc, kmax, kmin, cap = ada_evict_and_check(rk, w, n_keep)
    k1, k2, block = 32, 24, 16
    q = WL.decode_query(w, 0, 0, device=DEV)
    Hkv, G, d = w.n_kv, w.group, w.d
    nblk = -(-cap // block)
    nsel = min(k2, nblk)
    out = torch.empty(B, w.n_q, d, device=DEV)
    sel = torch.empty(B, Hkv, nsel, dtype=torch.int32, device=DEV)
    chan = torch.empty(B, Hkv, k1, dtype=torch.int32, device=DEV)
    s1 = torch.empty(B, Hkv, nblk, device=DEV)
    rk.rk_profile_begin()
    rk.rk_hsa_decode_ragged(q, kc, vc, kmax, kmin, cnt, cap, block, k1, k2, out, sel, chan, s1)
    launched = set(rk.rk_profile_end())
    assert launched == ({"hsa_fused"} if B * Hkv >= 160 else {"hsa_score", "hsa_attn", "hsa_combine"}), launched
    torch.cuda.synchronize()
    counts = cnt.cpu().numpy()
    for b, h in [(0, 0), (B - 1, Hkv - 1), (B // 2, 3)]:
        n = int(counts[b, h])
        nb = -(-n // block)
        qg = U.np32(q[b, h * G:(h + 1) * G])
        wmax, wmin = O.build_aux(U.np32(kc[b, h, :n]), n, block)
        i1, qbar = O.channel_select(qg, k1)
        assert np.array_equal(chan[b, h].cpu().numpy(), i1)
        ws1 = O.block_scores(qbar, i1, wmax, wmin)
        assert np.array_equal(U.np32(s1[b, h, :nb]), ws1), (b, h)
        want = O.block_select(ws1, k2)
        gs = sel[b, h].cpu().numpy()
        assert gs[:len(want)].tolist() == want.tolist() and (gs[len(want):] == -1).all(), (b, h)
        toks = O.selected_tokens(want, n, block)
        ridx = torch.as_tensor(toks, dtype=torch.long, device=DEV)
        U.check_output(U.np32(out[b, h * G:(h + 1) * G]),
                       O.attention(qg, U.np32(kc[b, h, ridx]), U.np32(vc[b, h, ridx])))


def test_ragged_decode_uniform_lengths_equal_decode(rk):
    """Every unit at the same length: bit-identical to rk_hsa_decode."""
    say("ragged decode, uniform lengths")
    w = WL.scaled(LLAMA, batch=2, seq=2000, n_plant=8)
    kc, vc, _ = WL.layer_kv(w, 0, device=DEV)
    n = 1997
    kmax = torch.empty(2, 8, 128, rk.aux_capacity(n, 16), dtype=kc.dtype, device=DEV)
    kmin = torch.empty_like(kmax)
    rk.rk_hsa_build_aux(kc, n, 0, 16, kmax, kmin)
    q = WL.decode_query(w, 0, 0, device=DEV)
    lens = torch.full((2, 8), n, dtype=torch.int32, device=DEV)
    a = torch.empty(2, 32, 128, device=DEV)
    b = torch.empty_like(a)
    rk.rk_hsa_decode(q, kc, vc, kmax, kmin, n, 16, 32, 40, a)
    rk.rk_hsa_decode_ragged(q, kc, vc, kmax, kmin, lens, n, 16, 32, 40, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)

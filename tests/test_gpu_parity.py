"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Every test prints the case it runs before launching, so a failure names it.
Inputs are the seeded synthetic workloads; sizes are chosen so the oracle
finishes in seconds while still spanning several tiles and a ragged tail.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import rk_testutil as U
from sparse_decode_attention_amd import workloads as WL

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def rk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_decode_attention_amd import rocketkv
    return rocketkv


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _pipeline(rk, w, layer=0, steps=None, seed=0, fused_aux=True):
    """Stage 1 + aux + decode steps of one layer of workload w, checked stage-wise."""
    s = rk.rk_split(w.c, w.seq, w.window, w.block, w.d)
    k, v, pos = WL.layer_kv(w, layer, device=DEV, seed=seed)
    qw = WL.window_queries(w, layer, device=DEV, seed=seed)
    n_keep, k2 = s["n_keep"], WL.stage2_pages(w, s)
    if fused_aux:   # the compaction builds Kmax/Kmin on the way
        kept, kc, vc, pooled, sw1, kmax, kmin = U.evict_and_check(rk, qw, k, v, w.seq, w.window, w.pool,
                                                                  n_keep, aux_block=w.block)
    else:
        kept, kc, vc, pooled, sw1 = U.evict_and_check(rk, qw, k, v, w.seq, w.window, w.pool, n_keep)
        kmax, kmin = U.aux_and_check(rk, kc, n_keep, w.block, w.n_q)
    swaps = 0
    for step in range(w.decode_steps if steps is None else steps):
        q = WL.decode_query(w, layer, step, device=DEV, seed=seed)
        _, _, sw = U.decode_and_check(rk, q, kc, vc, kmax, kmin, n_keep, w.block, w.k1, k2)
        swaps += sw
    return dict(kept=kept, pos=pos, swaps_evict=sw1, swaps_decode=swaps)


def test_tiny_gqa_fp32_full_pipeline(rk):
    w = WL.WORKLOADS["tiny-gqa-s2048-d64-fp32"]
    say(w.name, "all 8 decode steps")
    res = _pipeline(rk, w, fused_aux=False)     # separate aux build
    # the planted keys survive stage 1
    kept = res["kept"].cpu().numpy()
    for h in range(w.n_kv):
        assert set(res["pos"][0, h].tolist()) <= set(kept[0, h].tolist())
    say("swaps", res["swaps_evict"], res["swaps_decode"])


def test_llama8b_layer_full_pipeline(rk):
    w = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    say(w.name, "64 decode steps")
    res = _pipeline(rk, w)
    say("swaps", res["swaps_evict"], res["swaps_decode"])


def test_paper_decomposition_pipeline(rk):
    """The notes' own HSA decomposition: 3-token pages, k1 = 81, 342 pages."""
    w = WL.scaled(WL.WORKLOADS["llama8b-layer-s32k-c16-paper"], decode_steps=8)
    s = rk.rk_split(w.c, w.seq, w.window, w.block, w.d)
    assert (w.block, w.k1, WL.stage2_pages(w, s)) == (s["paper_page"], s["paper_k1_channels"], 342)
    say(w.name, "8 decode steps")
    res = _pipeline(rk, w)
    say("swaps", res["swaps_evict"], res["swaps_decode"])


@pytest.mark.parametrize("block", [1, 3, 5, 24])
def test_short_and_odd_pages(rk, block):
    """Pages of 1, 3, 5 and 24 tokens on both decode paths (the attention takes
    a wave's pages as one token sequence when they are shorter than a step)."""
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    say("pages of", block, "split path")
    w = WL.scaled(base, batch=2, seq=900, n_plant=8, block=block)
    _decode_only(rk, w, 877, 32, max(17, 200 // block))     # > 16 pages: split path
    say("pages of", block, "fused path")
    w = WL.scaled(base, batch=20, seq=500, n_plant=4, block=block)
    _decode_only(rk, w, 487, 32, max(1, 120 // block), units_to_check=[(0, 0), (7, 3), (19, 7)], steps=1)


@pytest.mark.parametrize("dtype,d,G,S,W,pool", [
    ("bf16", 128, 4, 1000, 32, 63),     # ragged S (tile 64), pool larger than gaps
    ("bf16", 64, 2, 777, 16, 7),
    ("f32", 128, 1, 513, 8, 3),
    ("f32", 64, 8, 300, 4, 1),
    ("bf16", 128, 8, 2100, 32, 63),
    # pool 1: the pooled output is the per-key window score itself, so the
    # matrix-core scorer is compared with the oracle key by key (G*W = 128, 32, 32)
    ("bf16", 128, 4, 1000, 32, 1),
    ("bf16", 128, 1, 1000, 32, 1),
    ("bf16", 64, 2, 777, 16, 1),
])
def test_shapes_and_ragged_tails(rk, dtype, d, G, S, W, pool):
    say("shape", dtype, d, G, S, W, pool)
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=2, n_kv=2, n_q=2 * G, d=d, dtype=dtype, seq=S, window=W, pool=pool,
                  n_plant=8, n_outlier=4, c=6.0, k1=min(16, d), decode_steps=3)
    res = _pipeline(rk, w)
    say("swaps", res["swaps_evict"], res["swaps_decode"])


@pytest.mark.parametrize("B,n_kv,d,dtype,S,W,pool,n_keep", [
    (1, 8, 128, "bf16", 3000, 32, 63, 900),     # kernel 63, pooled in its own launch
    (20, 8, 128, "bf16", 1500, 32, 63, 400),    # 160 units: pooled inside the select launch
    (2, 2, 64, "f32", 777, 16, 7, 300),         # other kernel widths
    (1, 2, 64, "bf16", 300, 4, 1, 100),         # kernel 1: the scores themselves
])
def test_evict_max_pooling(rk, B, n_kv, d, dtype, S, W, pool, n_keep):
    """The max reading of the pooling (rk_snapkv_evict_pool, RK_POOL_MAX)
    against the oracle's pool_max on every pooling path."""
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=B, n_kv=n_kv, n_q=4 * n_kv, d=d, dtype=dtype, seq=S, window=W, pool=pool,
                  n_plant=8)
    say("evict, max pooling", B, n_kv, d, dtype, S, W, pool, n_keep)
    k, v, _ = WL.layer_kv(w, 0, device=DEV)
    qw = WL.window_queries(w, 0, device=DEV)
    units = [(0, 0), (B - 1, n_kv - 1), (B // 2, n_kv // 2)]
    swaps = U.evict_and_check(rk, qw, k, v, S, W, pool, n_keep, units_to_check=units, aux_block=16,
                              pool_op="max")[4]
    say("  swaps", swaps)


@pytest.mark.parametrize("B,S,pool,op,n_keep", [
    (1, 3000, 1, "sum", 900),      # keys staged in LDS, pooling in its own launch
    (20, 1500, 63, "max", 400),    # 160 units: pooling inside the select launch
    (1, 45000, 1, "sum", 5000),    # more keys than LDS holds: chunked select
])
def test_stage1_select_all_ties(rk, B, S, pool, op, n_keep):
    """Every key row of a unit the same vector: each window row spreads its
    probability evenly over the prefix, so every pooled score of a unit is
    one value (with kernel 1, or the maximum over any kernel) and the lower
    positions win every tie: the unit keeps its first n_keep - W positions."""
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=B, seq=S, pool=pool, n_plant=0)
    say("stage 1, all ties", B, S, pool, op, n_keep)
    k, v, _ = WL.layer_kv(w, 0, device=DEV)
    qw = WL.window_queries(w, 0, device=DEV)
    k = k[:, :, :1].expand(-1, -1, S, -1).contiguous()
    units = [(0, 0), (B - 1, w.n_kv - 1)]
    kept = U.evict_and_check(rk, qw, k, v, S, w.window, pool, n_keep, units_to_check=units, pool_op=op)[0]
    want = torch.cat([torch.arange(n_keep - w.window), torch.arange(S - w.window, S)]).to(torch.int32)
    for b in range(B):
        for h in range(w.n_kv):
            assert torch.equal(kept[b, h].cpu(), want), (b, h)


@pytest.mark.parametrize("n_keep,out_cap", [(700, 700), (705, 760)])
def test_compaction_aux_many_pages(rk, n_keep, out_cap):
    """Batch 32 x 8 KV heads: the compaction with Kmax/Kmin takes its wide
    (32 pages per workgroup) form; ragged last page, spare capacity."""
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=32, seq=1500, n_plant=8)
    say("compaction + aux", w.batch, "x", w.n_kv, "units, n_keep", n_keep, "cap", out_cap)
    k, v, _ = WL.layer_kv(w, 0, device=DEV)
    qw = WL.window_queries(w, 0, device=DEV)
    U.evict_and_check(rk, qw, k, v, w.seq, w.window, w.pool, n_keep, out_cap=out_cap,
                      aux_block=w.block, units_to_check=[(0, 0), (13, 5), (31, 7)])


def test_keep_all_and_window_only_many_units(rk):
    """64 units with kernel 63 (pooling inside the select launch): keep all,
    window only, and one prefix key."""
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=8, seq=600, n_plant=4)
    k, v, _ = WL.layer_kv(w, 0, device=DEV)
    qw = WL.window_queries(w, 0, device=DEV)
    units = [(0, 0), (3, 5), (7, 7)]
    say("64 units, keep all")
    kept, kc, vc, _, _ = U.evict_and_check(rk, qw, k, v, 600, w.window, w.pool, 600, units_to_check=units)
    assert (kept.cpu().numpy() == np.arange(600)).all()
    assert torch.equal(kc, k) and torch.equal(vc, v)
    say("64 units, window only")
    kept, _, _, _, _ = U.evict_and_check(rk, qw, k, v, 600, w.window, w.pool, w.window, units_to_check=units)
    assert (kept.cpu().numpy() == np.arange(600 - w.window, 600)).all()
    say("64 units, one prefix key")
    U.evict_and_check(rk, qw, k, v, 600, w.window, w.pool, w.window + 1, units_to_check=units)


def test_keep_all_and_window_only(rk):
    base = WL.WORKLOADS["tiny-gqa-s2048-d64-fp32"]
    w = WL.scaled(base, seq=600, batch=2)
    k, v, _ = WL.layer_kv(w, 0, device=DEV)
    qw = WL.window_queries(w, 0, device=DEV)
    say("keep all S=600")
    kept, kc, vc, _, _ = U.evict_and_check(rk, qw, k, v, 600, w.window, w.pool, 600)
    assert (kept.cpu().numpy() == np.arange(600)).all()
    assert torch.equal(kc, k) and torch.equal(vc, v)
    say("window only")
    kept, _, _, _, _ = U.evict_and_check(rk, qw, k, v, 600, w.window, w.pool, w.window)
    assert (kept.cpu().numpy() == np.arange(600 - w.window, 600)).all()
    say("S == W")
    w2 = WL.scaled(base, seq=16, window=16, batch=1)
    k2, v2, _ = WL.layer_kv(WL.scaled(w2, n_plant=0), 0, device=DEV)
    qw2 = WL.window_queries(w2, 0, device=DEV)
    kept, _, _, _, _ = U.evict_and_check(rk, qw2, k2, v2, 16, 16, 7, 16)
    assert (kept.cpu().numpy() == np.arange(16)).all()


def test_decode_all_pages_is_dense_attention(rk):
    """k2 >= pages: the output equals dense attention over the whole cache."""
    say("dense special case")
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=2, seq=1000, n_plant=4)
    kc, vc, _ = WL.layer_kv(w, 0, device=DEV)
    n = 997                                              # ragged last page
    kmax, kmin = U.aux_and_check(rk, kc, n, 16, w.n_q)
    q = WL.decode_query(w, 0, 0, device=DEV)
    out, sel, _ = U.decode_and_check(rk, q, kc, vc, kmax, kmin, n, 16, 128, 10 ** 6)
    assert (sel.cpu().numpy() == np.arange(-(-n // 16))).all()
    G = w.group
    for b in range(2):
        for h in range(w.n_kv):
            want = O.attention(U.np32(q[b, h * G:(h + 1) * G]), U.np32(kc[b, h, :n]), U.np32(vc[b, h, :n]))
            U.check_output(U.np32(out[b, h * G:(h + 1) * G]), want)


def test_incremental_aux_equals_rebuild(rk):
    say("incremental aux")
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=2, seq=700, n_plant=0)
    kc, _, _ = WL.layer_kv(w, 0, device=DEV)
    nblk = -(-700 // 16)
    full_max = torch.empty(2, w.n_kv, 128, nblk + 4, dtype=kc.dtype, device=DEV)
    full_min = torch.empty_like(full_max)
    inc_max = torch.zeros_like(full_max)
    inc_min = torch.zeros_like(full_max)
    rk.rk_hsa_build_aux(kc, 700, 0, 16, full_max, full_min, n_q_heads=w.n_q)
    rk.rk_hsa_build_aux(kc, 650, 0, 16, inc_max, inc_min, n_q_heads=w.n_q)
    for n_old in range(650, 700, 7):
        rk.rk_hsa_build_aux(kc, min(n_old + 7, 700), n_old, 16, inc_max, inc_min, n_q_heads=w.n_q)
    torch.cuda.synchronize()
    assert torch.equal(full_max[..., :nblk], inc_max[..., :nblk])
    assert torch.equal(full_min[..., :nblk], inc_min[..., :nblk])


def test_mt_decode_over_candidates(rk):
    """RocketKV-MT: full cache kept, stage 2 restricted to the stage-1 candidates."""
    base = WL.WORKLOADS["mt-mha-b8-s32k-c32"]
    w = WL.scaled(base, batch=2, n_q=4, n_kv=4, seq=3000, n_plant=16, decode_steps=3)
    s = rk.rk_split(w.c, w.seq, w.window, w.block, w.d)
    cap = 3500                                          # full cache with spare capacity
    k = torch.zeros(2, 4, cap, 128, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    k0, v0, _ = WL.layer_kv(w, 0, device=DEV)
    k[:, :, :3000] = k0
    v[:, :, :3000] = v0
    qw = WL.window_queries(w, 0, device=DEV)
    say("MT evict indices only")
    kept, _, _, _, _ = U.evict_and_check(rk, qw, k, v, 3000, w.window, w.pool, s["n_keep"], compact=False)
    say("MT aux over candidates")
    kmax, kmin = U.aux_and_check(rk, k, s["n_keep"], 16, w.n_q, idx=kept)
    for step in range(3):
        say("MT decode step", step)
        q = WL.decode_query(w, 0, step, device=DEV)
        U.decode_and_check(rk, q, k, v, kmax, kmin, s["n_keep"], 16, w.k1, s["k2_blocks"], cand=kept)


def test_deterministic(rk):
    say("run twice, bit-identical")
    w = WL.scaled(WL.WORKLOADS["llama8b-layer-s32k-c16"], seq=4096, batch=1)
    k, v, _ = WL.layer_kv(w, 0, device=DEV)
    qw = WL.window_queries(w, 0, device=DEV)
    q = WL.decode_query(w, 0, 0, device=DEV)
    outs = []
    for _ in range(2):
        kept = torch.empty(1, 8, 1500, dtype=torch.int32, device=DEV)
        kc = torch.empty(1, 8, 1500, 128, dtype=k.dtype, device=DEV)
        vc = torch.empty_like(kc)
        pooled = torch.empty(1, 8, 4096 - 32, device=DEV)
        rk.rk_snapkv_evict(qw, k, v, 4096, 32, 63, 1500, kept, kc, vc, pooled)
        kmax = torch.empty(1, 8, 128, 96, dtype=k.dtype, device=DEV)
        kmin = torch.empty_like(kmax)
        rk.rk_hsa_build_aux(kc, 1500, 0, 16, kmax, kmin, n_q_heads=32)
        out = torch.empty(1, 32, 128, device=DEV)
        rk.rk_hsa_decode(q, kc, vc, kmax, kmin, 1500, 16, 64, 32, out)
        torch.cuda.synchronize()
        outs.append((kept.clone(), pooled.clone(), out.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_graph_replay_matches_eager(rk):
    """Decode calls captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager result bit for bit."""
    say("graph capture / replay")
    w = WL.scaled(WL.WORKLOADS["llama8b-layer-s32k-c16"], seq=4096, batch=2)
    s = rk.rk_split(w.c, w.seq, w.window, w.block, w.d)
    n_keep, k2 = s["n_keep"], s["k2_blocks"]
    k, v, _ = WL.layer_kv(w, 0, device=DEV)
    qw = WL.window_queries(w, 0, device=DEV)
    kept = torch.empty(2, 8, n_keep, dtype=torch.int32, device=DEV)
    kc = torch.empty(2, 8, n_keep, 128, dtype=k.dtype, device=DEV)
    vc = torch.empty_like(kc)
    nblk = -(-n_keep // 16)
    kmax = torch.empty(2, 8, 128, rk.aux_capacity(n_keep, 16), dtype=k.dtype, device=DEV)
    kmin = torch.empty_like(kmax)
    shape = rk.shape_of(2, 32, 8, 128, k.dtype)
    ws_e = torch.empty(rk.rk_snapkv_workspace_bytes(shape, w.seq, w.window), dtype=torch.uint8, device=DEV)
    ws_d = torch.empty(rk.rk_hsa_workspace_bytes(shape, n_keep, 16, w.k1, k2), dtype=torch.uint8, device=DEV)
    qs = torch.stack([WL.decode_query(w, 0, i, device=DEV) for i in range(4)])
    out = torch.empty(4, 2, 32, 128, device=DEV)

    def body():
        rk.rk_snapkv_evict(qw, k, v, w.seq, w.window, w.pool, n_keep, kept, kc, vc, None, ws=ws_e)
        rk.rk_hsa_build_aux(kc, n_keep, 0, 16, kmax, kmin, n_q_heads=32)
        for i in range(4):
            rk.rk_hsa_decode(qs[i], kc, vc, kmax, kmin, n_keep, 16, w.k1, k2, out[i], ws=ws_d)

    body()
    torch.cuda.synchronize()
    ref = (kept.clone(), kc.clone(), kmax[..., :nblk].clone(), out.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        kept.zero_()
        out.zero_()
        kmax.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (kept, kc, kmax[..., :nblk], out)):
            assert torch.equal(a, b), rep
        body()                                               # eager work between replays
        torch.cuda.synchronize()


def test_kernel_timing_hooks(rk):
    say("rk_profile_begin/end")
    w = WL.scaled(WL.WORKLOADS["tiny-gqa-s2048-d64-fp32"], seq=512)
    kc, vc, _ = WL.layer_kv(w, 0, device=DEV)
    kmax = torch.empty(1, 2, 64, 32, device=DEV)
    kmin = torch.empty_like(kmax)
    rk.rk_profile_begin()
    for _ in range(3):
        rk.rk_hsa_build_aux(kc, 512, 0, 16, kmax, kmin, n_q_heads=8)
    q = WL.decode_query(w, 0, 0, device=DEV)
    out = torch.empty(1, 8, 64, device=DEV)
    rk.rk_hsa_decode(q, kc, vc, kmax, kmin, 512, 16, 16, 20, out)   # > 16 pages: split path
    prof = rk.rk_profile_end()
    assert prof["aux_build"][0] == 3 and prof["aux_build"][1] > 0
    assert set(prof) == {"aux_build", "hsa_score", "hsa_attn", "hsa_combine"}
    assert rk.rk_profile_end() == {}


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_append_equals_rebuild(rk, dtype, d):
    """rk_append_kv writes the rows and leaves Kmax/Kmin equal to a full rebuild."""
    say("append", dtype, d)
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=3, n_kv=2, n_q=4, d=d, dtype=dtype, seq=200, n_plant=0)
    kc0, vc0, _ = WL.layer_kv(w, 0, device=DEV)
    cap = 240
    kc = torch.zeros(3, 2, cap, d, dtype=kc0.dtype, device=DEV)
    vc = torch.zeros_like(kc)
    kc[:, :, :200] = kc0
    vc[:, :, :200] = vc0
    kmax = torch.empty(3, 2, d, rk.aux_capacity(cap, 16), dtype=kc.dtype, device=DEV)
    kmin = torch.empty_like(kmax)
    rk.rk_hsa_build_aux(kc, 200, 0, 16, kmax, kmin)
    for step in range(40):                       # crosses page boundaries at 208, 224
        ka, va = WL.append_kv(w, 0, step, device=DEV)
        rk.rk_append_kv(ka, va, kc, vc, 200 + step, kmax, kmin, 16)
        torch.cuda.synchronize()
        assert torch.equal(kc[:, :, 200 + step], ka) and torch.equal(vc[:, :, 200 + step], va)
        U.check_aux_units(kmax, kmin, kc, 201 + step, 16, [(b, h) for b in range(3) for h in range(2)])


@pytest.mark.parametrize("dtype,d,G,B,Hkv,n0,k2,big", [
    ("bf16", 128, 4, 20, 8, 997, 16, False),   # 160 units: one launch; new token mid-page
    ("bf16", 128, 4, 20, 8, 992, 16, True),    # new token opens a page that gets chosen
    ("bf16", 128, 4, 20, 8, 1001, 64, True),   # mid-page, its page chosen
    ("f32", 64, 2, 40, 4, 500, 8, True),
    # 8 units choosing more pages than the fused kernel's 16 waves: the split
    # path, which appends with a launch of its own first
    ("bf16", 128, 4, 1, 8, 997, 32, True),
    ("bf16", 128, 4, 1, 8, 992, 32, False),
    ("bf16", 128, 8, 1, 4, 1001, 32, True),    # group of 8 (always the split path)
    ("f32", 64, 2, 2, 4, 500, 24, True),
])
def test_append_decode_equals_append_then_decode(rk, dtype, d, G, B, Hkv, n0, k2, big):
    """rk_hsa_append_decode leaves the cache and Kmax/Kmin exactly as rk_append_kv
    does, selects exactly what rk_hsa_decode selects on that state, and its output
    agrees with it to float32 rounding and with the oracle over the chosen pages."""
    say("append+decode", dtype, d, G, B, Hkv, n0, k2, big)
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=B, n_kv=Hkv, n_q=Hkv * G, d=d, dtype=dtype, seq=n0, n_plant=4)
    kc0, vc0, _ = WL.layer_kv(w, 0, device=DEV)
    cap, k1, block = n0 + 24, 32 if d == 128 else 16, 16
    kc = torch.zeros(B, Hkv, cap, d, dtype=kc0.dtype, device=DEV)
    vc = torch.zeros_like(kc)
    kc[:, :, :n0] = kc0
    vc[:, :, :n0] = vc0
    kmax = torch.empty(B, Hkv, d, rk.aux_capacity(cap, block), dtype=kc.dtype, device=DEV)
    kmin = torch.empty_like(kmax)
    rk.rk_hsa_build_aux(kc, n0, 0, block, kmax, kmin)
    ka, va = WL.append_kv(w, 0, 0, device=DEV)
    if big:   # a strong new key makes its page a likely pick
        ka = (ka.float() * 6).to(ka.dtype).contiguous()
    q = WL.decode_query(w, 0, 0, device=DEV)
    n = n0 + 1
    nsel = min(k2, -(-n // block))
    outs = []
    for fused in (False, True):
        kcx, vcx, kxx, knx = kc.clone(), vc.clone(), kmax.clone(), kmin.clone()
        out = torch.empty(B, Hkv * G, d, device=DEV)
        sel = torch.empty(B, Hkv, nsel, dtype=torch.int32, device=DEV)
        chan = torch.empty(B, Hkv, k1, dtype=torch.int32, device=DEV)
        s1 = torch.empty(B, Hkv, -(-n // block), device=DEV)
        if fused:
            rk.rk_hsa_append_decode(q, ka, va, kcx, vcx, n0, kxx, knx, block, k1, k2, out, sel, chan, s1)
        else:
            rk.rk_append_kv(ka, va, kcx, vcx, n0, kxx, knx, block)
            rk.rk_hsa_decode(q, kcx, vcx, kxx, knx, n, block, k1, k2, out, sel, chan, s1)
        torch.cuda.synchronize()
        outs.append((kcx, vcx, kxx, knx, out, sel, chan, s1))
    a, b = outs
    for x, y in zip(a[:4], b[:4]):   # bitwise: spare aux pages hold whatever torch.empty left (NaN included)
        assert torch.equal(x.view(torch.int16 if x.element_size() == 2 else torch.int32),
                           y.view(torch.int16 if y.element_size() == 2 else torch.int32))
    for x, y in zip(a[5:], b[5:]):
        assert torch.equal(x, y)
    assert (a[4] - b[4]).abs().max().item() <= 1e-5
    last = (n - 1) // block
    picked = int((b[5][..., -1] == last).sum())
    say("  last page chosen in", picked, "of", B * Hkv, "units")
    if big:
        assert picked > 0
    for bb, h in [(0, 0), (B - 1, Hkv - 1), (B // 2, Hkv // 2)]:
        toks = O.selected_tokens(b[5][bb, h].cpu().numpy(), n, block)
        ridx = torch.as_tensor(toks, dtype=torch.long, device=DEV)
        want = O.attention(U.np32(q[bb, h * G:(h + 1) * G]), U.np32(b[0][bb, h, ridx]),
                           U.np32(b[1][bb, h, ridx]))
        U.check_output(U.np32(b[4][bb, h * G:(h + 1) * G]), want)
    rk.rk_profile_begin()
    rk.rk_hsa_append_decode(q, ka, va, kc, vc, n0, kmax, kmin, block, k1, k2,
                            torch.empty(B, Hkv * G, d, device=DEV))
    launched = set(rk.rk_profile_end())
    if B * Hkv >= 160:
        assert launched == {"hsa_fused_append"}
    else:
        assert launched == {"append_kv", "hsa_score", "hsa_attn", "hsa_combine"}, launched


def _decode_only(rk, w, n, k1, k2, units_to_check=None, cand_total=None, steps=2):
    """Aux + decode over a synthetic cache (no stage 1), checked stage-wise."""
    kc, vc, _ = WL.layer_kv(w, 0, device=DEV)
    cand = None
    if cand_total is not None:                       # MT: candidates = a strided subset of the cache
        B, H = kc.shape[:2]
        base = torch.arange(n, device=DEV, dtype=torch.int32) * (cand_total // n)
        cand = base.repeat(B, H, 1).contiguous()
        kmax, kmin = U.aux_and_check(rk, kc, n, w.block, w.n_q, idx=cand, units_to_check=units_to_check)
    else:
        kmax, kmin = U.aux_and_check(rk, kc, n, w.block, w.n_q, units_to_check=units_to_check)
    for step in range(steps):
        q = WL.decode_query(w, 0, step, device=DEV)
        U.decode_and_check(rk, q, kc, vc, kmax, kmin, n, w.block, k1, k2, cand=cand,
                           units_to_check=units_to_check)


@pytest.mark.parametrize("dtype,d,G,B,Hkv,n,k1,k2", [
    ("bf16", 128, 4, 20, 8, 997, 32, 16),      # 160 units: one fused workgroup per unit
    ("f32", 64, 2, 40, 4, 500, 16, 8),
    ("bf16", 128, 1, 6, 32, 1200, 32, 20),     # MHA group of one, 192 units
])
def test_fused_large_batch_decode(rk, dtype, d, G, B, Hkv, n, k1, k2):
    say("fused decode", dtype, d, G, B, Hkv, n, k1, k2)
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=B, n_kv=Hkv, n_q=Hkv * G, d=d, dtype=dtype, seq=n + 40, n_plant=4)
    _decode_only(rk, w, n, k1, k2)
    kc, vc, _ = WL.layer_kv(w, 0, device=DEV)
    kmax = torch.empty(B, Hkv, d, rk.aux_capacity(n, 16), dtype=kc.dtype, device=DEV)
    kmin = torch.empty_like(kmax)
    rk.rk_hsa_build_aux(kc, n, 0, 16, kmax, kmin)
    out = torch.empty(B, Hkv * G, d, device=DEV)
    rk.rk_profile_begin()
    rk.rk_hsa_decode(WL.decode_query(w, 0, 0, device=DEV), kc, vc, kmax, kmin, n, 16, k1, k2, out)
    assert set(rk.rk_profile_end()) == {"hsa_fused"}


@pytest.mark.parametrize("k2", [16, 5])
def test_fused_few_pages_batch1(rk, k2):
    """Batch 1 with at most 16 chosen pages (one per wave): one workgroup per
    unit, checked against the oracle, and the launch is the fused kernel."""
    say("fused decode, batch 1, k2", k2)
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=1, seq=1040, n_plant=4)
    _decode_only(rk, w, 997, 32, k2)
    kc, vc, _ = WL.layer_kv(w, 0, device=DEV)
    kmax = torch.empty(1, 8, 128, rk.aux_capacity(997, 16), dtype=kc.dtype, device=DEV)
    kmin = torch.empty_like(kmax)
    rk.rk_hsa_build_aux(kc, 997, 0, 16, kmax, kmin)
    rk.rk_profile_begin()
    rk.rk_hsa_decode(WL.decode_query(w, 0, 0, device=DEV), kc, vc, kmax, kmin, 997, 16, 32, k2,
                     torch.empty(1, 32, 128, device=DEV))
    assert set(rk.rk_profile_end()) == {"hsa_fused"}


def test_fused_mt_decode(rk):
    say("fused MT decode, 160 units")
    base = WL.WORKLOADS["mt-mha-b8-s32k-c32"]
    w = WL.scaled(base, batch=5, n_q=32, n_kv=32, seq=3000, n_plant=4)
    _decode_only(rk, w, 700, 32, 12, cand_total=2900, units_to_check=[(0, 0), (2, 17), (4, 31)])


@pytest.mark.parametrize("dtype,B,k2,mt", [
    ("bf16", 1, 32, False),    # split path
    ("bf16", 20, 16, False),   # one fused workgroup per unit
    ("f32", 1, 32, False),
    ("bf16", 40, 16, True),    # MT, fused (160 units of 4 query heads... here 320)
])
def test_decode_wide_score_range(rk, dtype, B, k2, mt):
    """Scores spread over hundreds of log2 units, with the largest keys planted
    late in the pages a wave walks: the online softmax's reference must move
    (and l, o be rescaled) in the middle of the stream, not just at its start;
    every unit checked against the oracle."""
    say("wide score range", dtype, B, k2, mt)
    Hkv, G, d, n, block, k1 = 8, 4, 128, 997, 16, 32
    gen = torch.Generator(device="cpu").manual_seed(7)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.randn(B, Hkv, n + 40, d, generator=gen).to(tdt)
    vc = torch.randn(B, Hkv, n + 40, d, generator=gen).to(tdt)
    q = (torch.randn(B, Hkv * G, d, generator=gen) * 6).to(tdt)
    qbar = q.float().view(B, Hkv, G, d).sum(2)
    # keys aligned with the group's mean query, ever stronger towards the end
    # of the cache: token j of the planted set scores about 40 * (j + 1) above
    # the rest (scaled by 1/sqrt(d) and log2 e, hundreds of log2 units)
    plant = torch.tensor([100, 300, 520, 700, 900, 990])
    for j, t in enumerate(plant.tolist()):
        kc[:, :, t] = (qbar / qbar.norm(dim=-1, keepdim=True) * (3.0 * (j + 1))).to(tdt)
    kc, vc, q = kc.to(DEV), vc.to(DEV), q.to(DEV)
    cand = None
    if mt:
        cand = torch.arange(n, dtype=torch.int32, device=DEV).repeat(B, Hkv, 1).contiguous()
    kmax, kmin = U.aux_and_check(rk, kc, n, block, Hkv * G, idx=cand)
    U.decode_and_check(rk, q, kc, vc, kmax, kmin, n, block, k1, k2, cand=cand)


def test_mt_decode_long_candidate_list_many_units(rk):
    """160 units whose candidate lists (40 000 indices, 160 KB) do not fit the
    fused workgroup's LDS: the split path, which reads them from memory."""
    say("MT decode, 160 units, 40000 candidates")
    base = WL.WORKLOADS["mt-mha-b8-s32k-c32"]
    w = WL.scaled(base, batch=5, n_q=32, n_kv=32, seq=41000, n_plant=4)
    _decode_only(rk, w, 40000, 32, 12, cand_total=41000, units_to_check=[(0, 0), (4, 31)], steps=1)
    kc, vc, _ = WL.layer_kv(w, 0, device=DEV)
    cand = torch.arange(40000, device=DEV, dtype=torch.int32).repeat(5, 32, 1).contiguous()
    kmax = torch.empty(5, 32, 128, rk.aux_capacity(40000, 16), dtype=kc.dtype, device=DEV)
    kmin = torch.empty_like(kmax)
    rk.rk_hsa_build_aux(kc, 40000, 0, 16, kmax, kmin, idx=cand)
    rk.rk_profile_begin()
    rk.rk_hsa_decode_mt(WL.decode_query(w, 0, 0, device=DEV), kc, vc, cand, 40000, kmax, kmin, 16, 32, 12,
                        torch.empty(5, 32, 128, device=DEV))
    assert set(rk.rk_profile_end()) == {"hsa_score", "hsa_attn_mt", "hsa_combine"}


def test_split_decode_many_workgroups(rk):
    """96 units on the split-K path with 768 attention workgroups (more than one
    per CU: the two-tokens-per-slot variant), next to the batch-1 tests that run
    the one-workgroup-per-CU variant."""
    say("split decode, 96 units")
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=12, n_kv=8, n_q=32, seq=1040, n_plant=4)
    _decode_only(rk, w, 997, 32, 32, units_to_check=[(0, 0), (5, 3), (11, 7)])
    kc, vc, _ = WL.layer_kv(w, 0, device=DEV)
    kmax = torch.empty(12, 8, 128, rk.aux_capacity(997, 16), dtype=kc.dtype, device=DEV)
    kmin = torch.empty_like(kmax)
    rk.rk_hsa_build_aux(kc, 997, 0, 16, kmax, kmin)
    rk.rk_profile_begin()
    rk.rk_hsa_decode(WL.decode_query(w, 0, 0, device=DEV), kc, vc, kmax, kmin, 997, 16, 32, 32,
                     torch.empty(12, 32, 128, device=DEV))
    assert set(rk.rk_profile_end()) == {"hsa_score", "hsa_attn", "hsa_combine"}


@pytest.mark.parametrize("B,Hkv,n,k2", [
    (1, 2, 20000, 200),      # 1250 pages: split path, workgroup page top-k
    (20, 8, 17000, 64),      # 160 units with 1063 pages: fused path, workgroup page top-k
])
def test_many_pages_decode(rk, B, Hkv, n, k2):
    say("many pages", B, Hkv, n, k2)
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=B, n_kv=Hkv, n_q=4 * Hkv, seq=n, n_plant=8)
    units = [(0, 0), (B - 1, Hkv - 1)]
    _decode_only(rk, w, n, 64, k2, units_to_check=units, steps=1)


@pytest.mark.parametrize("n", [12288 * 16, 12288 * 16 - 5])
def test_max_pages_decode(rk, n):
    """The largest page count a decode call takes (12288 pages of 16; the
    second case with a ragged last page): workgroup page top-k over every
    page key held in LDS at its full size."""
    say("max pages", n)
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=1, n_kv=2, n_q=8, seq=n, n_plant=8)
    _decode_only(rk, w, n, 64, 256, steps=1)


@pytest.mark.parametrize("B,spread", [(1, 2), (1, 200), (20, 2), (20, 200)])
def test_page_topk_exact_ties(rk, B, spread):
    """Integer-valued q and Kmax/Kmin make many channel sums and page scores
    exactly equal (spread 2: a few distinct scores; 200: scattered ties): the
    channel and page choices must follow the lower-index tie rule exactly, on
    the split path (8 units) and the fused path (160 units)."""
    say("exact ties", B, spread)
    Hkv, G, d, n, block, k1, k2 = 8, 4, 128, 605 * 16 - 7, 16, 64, 128
    g = torch.Generator().manual_seed(1000 + spread + B)
    q = torch.randint(-2, 3, (B, Hkv * G, d), generator=g).to(torch.bfloat16).to(DEV)
    cap = rk.aux_capacity(n, block)
    kmax = torch.randint(0, spread + 1, (B, Hkv, d, cap), generator=g)
    kmin = kmax - torch.randint(0, spread + 1, (B, Hkv, d, cap), generator=g)
    kmax = kmax.to(torch.bfloat16).to(DEV)
    kmin = kmin.to(torch.bfloat16).to(DEV)
    kc = torch.randn(B, Hkv, n, d, generator=g).to(torch.bfloat16).to(DEV)
    vc = torch.randn(B, Hkv, n, d, generator=g).to(torch.bfloat16).to(DEV)
    units = None if B == 1 else [(0, 0), (7, 3), (13, 5), (B - 1, Hkv - 1)]
    U.decode_and_check(rk, q, kc, vc, kmax, kmin, n, block, k1, k2, units_to_check=units)


@pytest.mark.parametrize("n_keep", [3000, 15000])
def test_long_prompt_select(rk, n_keep):
    """More prompt keys than LDS holds (80000): the chunked two-launch select
    (3000 kept) and the global-key select (15000 kept, too many candidates)."""
    say("long prompt select, keep", n_keep)
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=1, n_kv=2, n_q=4, seq=80000, n_plant=16)
    k, v, _ = WL.layer_kv(w, 0, device=DEV)
    qw = WL.window_queries(w, 0, device=DEV)
    U.evict_and_check(rk, qw, k, v, w.seq, w.window, w.pool, n_keep)

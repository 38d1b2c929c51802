"""GPU parity of the paged K/V pool (block tables) against the contiguous cache.

A contiguous cache is scattered into a pool of physical pages through a block
table that maps every sequence's logical pages to random distinct physical
pages (the pool also holds spare pages filled with noise).  Every paged call
must then equal the contiguous call on the same tokens bit for bit: the
kernels are the same and only the row addresses differ.  One case is also
checked against the oracle directly."""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import rk_testutil as U
from sparse_decode_attention_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda"
BASE = WL.WORKLOADS["llama8b-layer-s32k-c16"]


@pytest.fixture(scope="module")
def rk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_decode_attention_amd import rocketkv
    return rocketkv


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def make_pool(rk, kc, vc, n, P, cap_tokens, seed=0):
    """Scatter tokens [0, n) of kc, vc [B,Hkv,cap,d] into a noise-filled pool."""
    B, Hkv, _, d = kc.shape
    per_seq = -(-cap_tokens // P)
    n_pages = B * per_seq + 7
    g = torch.Generator().manual_seed(1234 + seed)
    table = torch.randperm(n_pages, generator=g)[: B * per_seq].view(B, per_seq).to(torch.int32).to(DEV)
    kp = torch.randn(n_pages, Hkv, P, d, generator=g).to(kc.dtype).to(DEV)
    vp = torch.randn(n_pages, Hkv, P, d, generator=g).to(kc.dtype).to(DEV)
    pages = rk.paged_kv(table, n_pages, P)
    rk.rk_paged_write_kv(kc, vc, 0, n, kp, vp, pages)
    torch.cuda.synchronize()
    tab = table.cpu()
    for b in range(B):
        for j in range(-(-n // P)):
            m = min(P, n - j * P)
            pg = int(tab[b, j])
            assert torch.equal(bits(kp[pg, :, :m]), bits(kc[b, :, j * P:j * P + m]))
            assert torch.equal(bits(vp[pg, :, :m]), bits(vc[b, :, j * P:j * P + m]))
    return kp, vp, pages, table


def dense_and_paged_decode(rk, w, n, P, block, k1, k2, seed=0, same_path=True):
    kc, vc, _ = WL.layer_kv(w, 0, device=DEV)
    kc, vc = kc.contiguous(), vc.contiguous()
    B, Hkv, _, d = kc.shape
    kp, vp, pages, _ = make_pool(rk, kc, vc, n, P, n, seed)
    cap = rk.aux_capacity(n, block)
    kx = torch.empty(B, Hkv, d, cap, dtype=kc.dtype, device=DEV)
    kn = torch.empty_like(kx)
    px, pn = torch.empty_like(kx), torch.empty_like(kx)
    rk.rk_hsa_build_aux(kc, n, 0, block, kx, kn, n_q_heads=w.n_q)
    rk.rk_paged_build_aux(kp, pages, B, n, 0, block, px, pn, n_q_heads=w.n_q)
    torch.cuda.synchronize()
    nblk = -(-n // block)
    assert torch.equal(bits(kx[..., :nblk]), bits(px[..., :nblk]))
    assert torch.equal(bits(kn[..., :nblk]), bits(pn[..., :nblk]))
    q = WL.decode_query(w, 0, seed, device=DEV)
    nsel = min(k2, nblk)
    res = []
    for paged in (False, True):
        out = torch.empty(B, w.n_q, d, device=DEV)
        sel = torch.empty(B, Hkv, nsel, dtype=torch.int32, device=DEV)
        chan = torch.empty(B, Hkv, k1, dtype=torch.int32, device=DEV)
        s1 = torch.empty(B, Hkv, nblk, device=DEV)
        if paged:
            rk.rk_paged_hsa_decode(q, kp, vp, pages, px, pn, n, block, k1, k2, out, sel, chan, s1)
        else:
            rk.rk_hsa_decode(q, kc, vc, kx, kn, n, block, k1, k2, out, sel, chan, s1)
        torch.cuda.synchronize()
        res.append((out, sel, chan, s1))
    (o0, *idx0), (o1, *idx1) = res
    for a, b in zip(idx0, idx1):
        assert torch.equal(bits(a), bits(b))
    if same_path:
        assert torch.equal(bits(o0), bits(o1))
    else:   # one side merges split-K partials: the same sums in another order
        assert torch.allclose(o0, o1, rtol=1e-5, atol=1e-6), (o0 - o1).abs().max().item()
    return kc, vc, q, res[1]


@pytest.mark.parametrize("B,Hkv,G,d,n,P,block,k1,k2", [
    (2, 8, 4, 128, 3001, 64, 16, 32, 40),        # split path, 64-token physical pages
    (20, 8, 4, 128, 997, 16, 16, 32, 16),        # 160 units: fused path
    (1, 4, 8, 128, 2500, 64, 16, 32, 40),        # group of 8 (split path)
    (6, 32, 1, 128, 1200, 32, 16, 32, 20),       # MHA, 192 units: fused path
    (2, 2, 2, 64, 1500, 128, 16, 16, 30),        # d 64
    (1, 8, 4, 128, 9675, 64, 3, 81, 342),        # the notes' 3-token pages over 64-token physical pages
    (20, 8, 4, 128, 997, 1, 16, 32, 16),         # fused path, one-token physical pages (997 row bases)
    # 40000 row bases do not fit the fused kernel's LDS: the paged call takes
    # the split path while the contiguous one stays fused, so their outputs
    # agree to float32 rounding rather than bit for bit
    (20, 8, 4, 128, 40000, 1, 16, 32, 16),
])
def test_paged_decode_equals_contiguous(rk, B, Hkv, G, d, n, P, block, k1, k2):
    say("paged decode", B, Hkv, G, d, n, P, block, k1, k2)
    w = WL.scaled(BASE, batch=B, n_kv=Hkv, n_q=Hkv * G, d=d, seq=n + 8, n_plant=8)
    kc, vc, q, (out, sel, chan, s1) = dense_and_paged_decode(rk, w, n, P, block, k1, k2,
                                                             same_path=(n, P) != (40000, 1))
    # and the oracle on one unit
    b, h = B - 1, Hkv - 1
    qg = U.np32(q[b, h * G:(h + 1) * G])
    kmax, kmin = O.build_aux(U.np32(kc[b, h, :n]), n, block)
    i1, qbar = O.channel_select(qg, k1)
    assert np.array_equal(chan[b, h].cpu().numpy(), i1)
    ws1 = O.block_scores(qbar, i1, kmax, kmin)
    assert np.array_equal(U.np32(s1[b, h]), ws1)
    assert np.array_equal(sel[b, h].cpu().numpy(), O.block_select(ws1, k2))
    toks = O.selected_tokens(sel[b, h].cpu().numpy(), n, block)
    ridx = torch.as_tensor(toks, dtype=torch.long, device=DEV)
    U.check_output(U.np32(out[b, h * G:(h + 1) * G]), O.attention(qg, U.np32(kc[b, h, ridx]), U.np32(vc[b, h, ridx])))


def test_paged_decode_many_pages(rk):
    """More than 12288 HSA pages: the separate page-choice launch over a pool."""
    say("paged decode, 13000 pages")
    w = WL.scaled(BASE, batch=1, n_kv=2, n_q=8, seq=13000 * 16, n_plant=8)
    dense_and_paged_decode(rk, w, 13000 * 16 - 3, 64, 16, 64, 64)


@pytest.mark.parametrize("B,Hkv,G,P", [(20, 8, 4, 16), (1, 8, 4, 16), (2, 4, 8, 32)])
def test_paged_append_and_append_decode(rk, B, Hkv, G, P):
    """40 appended tokens crossing physical pages: rk_paged_append_kv and the
    one-call rk_paged_hsa_append_decode leave the pool and Kmax/Kmin exactly
    as the contiguous calls leave the cache, and decode identically (fused path
    at 160 units, split path otherwise)."""
    say("paged append", B, Hkv, G, P)
    d, n0, steps, block, k1, k2 = 128, 997, 40, 16, 32, 24
    w = WL.scaled(BASE, batch=B, n_kv=Hkv, n_q=Hkv * G, d=d, seq=n0, n_plant=4)
    k0, v0, _ = WL.layer_kv(w, 0, device=DEV)
    cap = n0 + steps
    kc = torch.zeros(B, Hkv, cap, d, dtype=k0.dtype, device=DEV)
    vc = torch.zeros_like(kc)
    kc[:, :, :n0] = k0
    vc[:, :, :n0] = v0
    kp, vp, pages, table = make_pool(rk, kc, vc, n0, P, cap)
    acap = rk.aux_capacity(cap, block)
    kx = torch.empty(B, Hkv, d, acap, dtype=kc.dtype, device=DEV)
    kn = torch.empty_like(kx)
    rk.rk_hsa_build_aux(kc, n0, 0, block, kx, kn)
    px, pn = kx.clone(), kn.clone()
    for step in range(steps):
        pos = n0 + step
        ka, va = WL.append_kv(w, 0, step, device=DEV)
        q = WL.decode_query(w, 0, step, device=DEV)
        nblk = -(-(pos + 1) // block)
        outs = []
        for paged in (False, True):
            out = torch.empty(B, w.n_q, d, device=DEV)
            sel = torch.empty(B, Hkv, min(k2, nblk), dtype=torch.int32, device=DEV)
            if step % 2 == 0:      # append + decode in one call
                if paged:
                    rk.rk_paged_hsa_append_decode(q, ka, va, kp, vp, pages, pos, px, pn, block, k1, k2, out, sel)
                else:
                    rk.rk_hsa_append_decode(q, ka, va, kc, vc, pos, kx, kn, block, k1, k2, out, sel)
            else:                  # append, then decode
                if paged:
                    rk.rk_paged_append_kv(ka, va, kp, vp, pages, pos, px, pn, block)
                    rk.rk_paged_hsa_decode(q, kp, vp, pages, px, pn, pos + 1, block, k1, k2, out, sel)
                else:
                    rk.rk_append_kv(ka, va, kc, vc, pos, kx, kn, block)
                    rk.rk_hsa_decode(q, kc, vc, kx, kn, pos + 1, block, k1, k2, out, sel)
            torch.cuda.synchronize()
            outs.append((out, sel))
        assert torch.equal(bits(outs[0][0]), bits(outs[1][0])), step
        assert torch.equal(outs[0][1], outs[1][1]), step
        assert torch.equal(bits(kx[..., :nblk]), bits(px[..., :nblk])), step
        assert torch.equal(bits(kn[..., :nblk]), bits(pn[..., :nblk])), step
        tab = table.cpu()
        for b in (0, B - 1):
            pg = int(tab[b, pos // P])
            assert torch.equal(bits(kp[pg, :, pos % P]), bits(kc[b, :, pos])), (step, b)
            assert torch.equal(bits(vp[pg, :, pos % P]), bits(vc[b, :, pos])), (step, b)

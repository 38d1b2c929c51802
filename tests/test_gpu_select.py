"""GPU parity of the dynamic-selection methods (HSA, Quest, SparQ, Exact-TopK)
through rk_select_decode against the oracle's own formulas for each method.

The scores are float32 sums in one fixed order on both sides, so they must
match bit for bit, and with them the chosen pages (ties to the lower page);
the output is compared with the oracle's attention over the chosen tokens.
Cases span the in-workgroup page choice (<= 12288 pages) and the separate
page-choice launch (token-level methods, and more pages than that), with its
keys staged in LDS or read from memory."""

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


def _oracle_scores(method, qg, rows, page, channels):
    if method == "exact":
        return O.exact_topk_scores(qg, rows)
    if method == "sparq":
        return O.sparq_scores(qg, rows, channels)
    kmax, kmin = O.build_aux(rows, rows.shape[0], page)
    if method == "quest":
        return O.quest_page_scores(qg, kmax, kmin)
    i1, qbar = O.channel_select(qg, channels)
    return O.block_scores(qbar, i1, kmax, kmin)


def run_method(rk, method, w, n, page, channels, k2, units_to_check=None, steps=1):
    kc, vc, _ = WL.layer_kv(w, 0, device=DEV)
    B, Hkv, _, d = kc.shape
    G = w.group
    kmax = kmin = None
    if method in ("hsa", "quest"):
        kmax = torch.empty(B, Hkv, d, rk.aux_capacity(n, page), dtype=kc.dtype, device=DEV)
        kmin = torch.empty_like(kmax)
        rk.rk_hsa_build_aux(kc, n, 0, page, kmax, kmin, n_q_heads=w.n_q)
    elif method == "sparq":
        kmax = torch.empty(B, Hkv, d, rk.aux_capacity(n, 1), dtype=kc.dtype, device=DEV)
        rk.rk_hsa_build_aux(kc, n, 0, 1, kmax, None, n_q_heads=w.n_q)     # Kmax only: the keys, channel-major
    nblk = -(-n // page)
    nsel = min(k2, nblk)
    units = units_to_check or [(b, h) for b in range(B) for h in range(Hkv)]
    for step in range(steps):
        q = WL.decode_query(w, 0, step, device=DEV)
        out = torch.full((B, w.n_q, d), float("nan"), device=DEV)
        sel = torch.full((B, Hkv, nsel), -1, dtype=torch.int32, device=DEV)
        sc = torch.empty(B, Hkv, nblk, device=DEV)
        rk.rk_select_decode(method, q, kc, vc, kmax, kmin, n, page, channels, k2, out, sel, sc)
        torch.cuda.synchronize()
        for b, h in units:
            qg = U.np32(q[b, h * G:(h + 1) * G])
            rows = U.np32(kc[b, h, :n])
            want = _oracle_scores(method, qg, rows, page, channels)
            got = U.np32(sc[b, h])
            assert np.array_equal(got, want), (method, b, h, np.abs(got - want).max())
            gsel = sel[b, h].cpu().numpy()
            assert np.array_equal(gsel, O.block_select(want, k2)), (method, b, h)
            toks = O.selected_tokens(gsel, n, page)
            ridx = torch.as_tensor(toks, dtype=torch.long, device=DEV)
            ref = O.attention(qg, U.np32(kc[b, h, ridx]), U.np32(vc[b, h, ridx]))
            U.check_output(U.np32(out[b, h * G:(h + 1) * G]), ref)
    return kc


BASE = WL.WORKLOADS["llama8b-layer-s32k-c16"]


@pytest.mark.parametrize("method", ["hsa", "quest", "sparq", "exact"])
def test_methods_at_their_plans(rk, method):
    """Each method at its planned page / channels / k2 for c = 16 on a 3000-token
    cache (GQA group of 4, bf16, ragged last page)."""
    n = 2999
    p = rk.rk_select_plan(method, 16.0, n, 128)
    want = O.select_plan(method, 16.0, n, 128)
    assert (p["page"], p["channels"], p["k2"]) == (want["page"], want["channels"], want["k2"])
    say(method, "plan", p)
    w = WL.scaled(BASE, batch=2, seq=n + 16, n_plant=16)
    run_method(rk, method, w, n, p["page"], p["channels"], p["k2"], steps=2)


@pytest.mark.parametrize("method,dtype,d,G", [("exact", "f32", 64, 2), ("sparq", "f32", 64, 8),
                                              ("quest", "f32", 64, 1), ("exact", "bf16", 128, 1),
                                              ("sparq", "bf16", 128, 2)])
def test_methods_other_shapes(rk, method, dtype, d, G):
    say(method, dtype, d, G)
    w = WL.scaled(BASE, batch=3, n_kv=2, n_q=2 * G, d=d, dtype=dtype, seq=1300, n_plant=8)
    n = 1283
    p = rk.rk_select_plan(method, 8.0, n, d)
    run_method(rk, method, w, n, p["page"], p["channels"], p["k2"])


@pytest.mark.parametrize("method,n,page,channels,k2", [
    ("sparq", 20000, 1, 8, 1000),        # 20000 one-token pages: separate choice, keys staged in LDS
    ("exact", 40000, 1, 128, 600),       # 40000 pages: the choice reads its keys from memory
    ("hsa", 15000, 1, 32, 300),          # HSA with one-token pages past the LDS limit
    ("hsa", 13000 * 16 - 3, 16, 32, 64), # 13000 pages of 16 tokens (ragged last page)
])
def test_many_pages_separate_choice(rk, method, n, page, channels, k2):
    say("separate page choice", method, n, page, channels, k2)
    w = WL.scaled(BASE, batch=1, n_kv=2, n_q=8, seq=n + 8, n_plant=16)
    rk.rk_profile_begin()
    run_method(rk, method, w, n, page, channels, k2)
    prof = rk.rk_profile_end()
    assert "page_select" in prof, prof


def test_exact_on_the_llama8b_layer(rk):
    """Exact-TopK over the full 32K prompt of the Llama-8B layer, budget 2048."""
    say("exact, 32K prompt, 8 KV heads")
    w = BASE
    run_method(rk, "exact", w, w.seq, 1, 128, 2048, units_to_check=[(0, 0), (0, 5)])


def test_aux_kmax_only_block1_is_the_transposed_keys(rk):
    say("aux, block 1, Kmax only")
    w = WL.scaled(BASE, batch=2, seq=500, n_plant=0)
    kc, _, _ = WL.layer_kv(w, 0, device=DEV)
    kmax = torch.empty(2, 8, 128, rk.aux_capacity(500, 1), dtype=kc.dtype, device=DEV)
    rk.rk_hsa_build_aux(kc, 500, 0, 1, kmax, None)
    torch.cuda.synchronize()
    assert torch.equal(kmax[..., :500], kc.transpose(2, 3).contiguous())

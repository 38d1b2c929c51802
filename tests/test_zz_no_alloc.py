"""rk_hsa_decode_noalloc (static scratch, no allocation) against rk_hsa_decode.

Two calls in a row on the split-K path (the path that uses scratch), the second
with a smaller input, each compared bit for bit with rk_hsa_decode on the same
inputs (same kernels, same order of operations) and against the oracle; then a
request larger than the scratch is refused with RK_EWORKSPACE before any
launch, and a call after it still works.
"""

import sys

import numpy as np
import pytest
import torch

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


def _case(rk, B, n, k1, k2, seed_step):
    base = WL.WORKLOADS["llama8b-layer-s32k-c16"]
    w = WL.scaled(base, batch=B, seq=n + 16, n_plant=8)
    kc, vc, _ = WL.layer_kv(w, 0, device=DEV)
    kmax = torch.empty(B, w.n_kv, w.d, rk.aux_capacity(n, w.block), dtype=kc.dtype, device=DEV)
    kmin = torch.empty_like(kmax)
    rk.rk_hsa_build_aux(kc, n, 0, w.block, kmax, kmin, n_q_heads=w.n_q)
    q = WL.decode_query(w, 0, seed_step, device=DEV)
    nsel = min(k2, -(-n // w.block))
    outs = []
    for noalloc in (True, False):
        out = torch.full((B, w.n_q, w.d), float("nan"), device=DEV)
        sel = torch.full((B, w.n_kv, nsel), -1, dtype=torch.int32, device=DEV)
        chan = torch.full((B, w.n_kv, k1), -1, dtype=torch.int32, device=DEV)
        if noalloc:
            rk.rk_hsa_decode_noalloc(q, kc, vc, kmax, kmin, n, w.block, k1, k2, out, sel, chan)
        else:
            rk.rk_hsa_decode(q, kc, vc, kmax, kmin, n, w.block, k1, k2, out, sel, chan)
        torch.cuda.synchronize()
        outs.append((out, sel, chan))
    (a_out, a_sel, a_ch), (b_out, b_sel, b_ch) = outs
    assert torch.equal(a_sel, b_sel) and torch.equal(a_ch, b_ch)
    assert torch.equal(a_out, b_out)
    # and the oracle's bar, on two units
    G = w.group
    for b, h in [(0, 0), (B - 1, w.n_kv - 1)]:
        toks = U.O.selected_tokens(a_sel[b, h].cpu().numpy(), n, w.block)
        ridx = torch.as_tensor(toks, dtype=torch.long, device=DEV)
        want = U.O.attention(U.np32(q[b, h * G:(h + 1) * G]), U.np32(kc[b, h, ridx]), U.np32(vc[b, h, ridx]))
        U.check_output(U.np32(a_out[b, h * G:(h + 1) * G]), want)


def test_noalloc_matches_workspace_decode_twice(rk):
    say("noalloc decode: batch 2, 9675 tokens, k2 128")
    _case(rk, 2, 9675, 64, 128, 0)
    say("noalloc decode again, smaller: batch 1, 3001 tokens, k2 40")
    _case(rk, 1, 3001, 32, 40, 1)


def test_noalloc_refuses_more_than_scratch(rk):
    cap = rk.rk_hsa_decode_noalloc_max_bytes()
    assert cap == 16 << 20
    B, Hkv, d = 64, 8, 128
    n = 12000 * 16                      # 12000 pages x 512 units of keys alone exceed the scratch
    shape = rk.shape_of(B, 4 * Hkv, Hkv, d, torch.bfloat16)
    assert rk.rk_hsa_workspace_bytes(shape, n, 16, 32, 256) > cap
    say("noalloc refusal")
    t = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    lib = rk.raw_library()
    import ctypes
    st = lib.rk_hsa_decode_noalloc(ctypes.byref(shape), rk._ptr(t), rk._ptr(t), rk._ptr(t), n, rk._ptr(t),
                                   rk._ptr(t), 12000, n, 16, 32, 256, rk._ptr(t), None, None, None, None)
    assert st == rk.RK_EWORKSPACE
    assert b"static scratch" in lib.rk_last_error()
    say("noalloc after a refusal")
    _case(rk, 1, 2000, 32, 24, 2)

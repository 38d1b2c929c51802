"""Shared helpers of the GPU parity tests: stage-wise comparison of the HIP
path (through the C ABI binding) with the CPU oracle on the same inputs.

Comparison rules:
  * Kmax/Kmin, channel sets, compaction rows: bit-exact.
  * Kept-token and page sets: the GPU set P and the oracle set O (same size)
    may differ only by swaps between elements whose oracle scores are within
    1e-4 relative of each other (near ties); the number of swaps is returned.
  * Attention outputs: compared with the oracle's attention over the pages the
    GPU selected, at max-abs 1e-2 and rel-L2 5e-3.
Each stage is fed the GPU's own upstream output, so an accepted near-tie swap
cannot cascade.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle as O

SWAP_REL = 1e-4
OUT_MAX_ABS = 1e-2
OUT_REL_L2 = 5e-3


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def compare_sets(gpu_idx, oracle_idx, scores, rel=SWAP_REL) -> int:
    """Accept GPU vs oracle index sets that differ only by near-tie swaps."""
    P = set(int(x) for x in np.asarray(gpu_idx).ravel())
    Oset = set(int(x) for x in np.asarray(oracle_idx).ravel())
    assert len(P) == len(np.asarray(gpu_idx).ravel()), "duplicate indices in the GPU set"
    assert len(P) == len(Oset), "set sizes differ"
    only_p = np.array(sorted(P - Oset), dtype=np.int64)
    only_o = np.array(sorted(Oset - P), dtype=np.int64)
    if only_p.size == 0:
        return 0
    s = np.asarray(scores, dtype=np.float64)
    sx = s[only_p][:, None]
    sy = s[only_o][None, :]
    ok = np.abs(sx - sy) <= rel * np.maximum(np.abs(sx), np.abs(sy))
    assert ok.all(), (f"{only_p.size} swaps, worst pair not a near tie: "
                      f"gpu-only {only_p[:8]} scores {s[only_p][:8]}, oracle-only {only_o[:8]} "
                      f"scores {s[only_o][:8]}")
    return int(only_p.size)


def check_output(got: np.ndarray, want: np.ndarray):
    err = np.abs(got - want).max()
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    assert err <= OUT_MAX_ABS and rel <= OUT_REL_L2, (err, rel)
    return float(err), float(rel)


def ascending(x) -> bool:
    x = np.asarray(x)
    return bool(np.all(np.diff(x) > 0))


# --------------------------------------------------------------------------
def evict_and_check(rk, qw, k, v, S, W, pool, n_keep, units_to_check=None, compact=True, out_cap=None,
                    aux_block=None, pool_op="sum"):
    """Run rk_snapkv_evict and check every (or the given) unit against the oracle;
    with aux_block, the call also builds Kmax/Kmin of the compact cache, checked
    bit-exactly.  Returns (kept, k_out, v_out, pooled, swaps), plus (kmax, kmin)
    with aux_block."""
    B, Hq, _, d = qw.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    dev = k.device
    kept = torch.full((B, Hkv, n_keep), -1, dtype=torch.int32, device=dev)
    pooled = torch.empty(B, Hkv, S - W, dtype=torch.float32, device=dev)
    ko = vo = None
    kmax = kmin = None
    if compact:
        ko = torch.empty(B, Hkv, out_cap or n_keep, d, dtype=k.dtype, device=dev)
        vo = torch.empty_like(ko)
        if aux_block:
            kmax = torch.full((B, Hkv, d, rk.aux_capacity(out_cap or n_keep, aux_block)), 7.0,
                              dtype=k.dtype, device=dev)
            kmin = torch.full_like(kmax, 7.0)
    rk.rk_snapkv_evict(qw, k, v, S, W, pool, n_keep, kept, ko, vo, pooled, kmax=kmax, kmin=kmin,
                       block=aux_block or 16, pool_op=pool_op)
    torch.cuda.synchronize()
    swaps = 0
    units = units_to_check or [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in units:
        q_np = np32(qw[b, h * G:(h + 1) * G])
        k_np = np32(k[b, h, :S])
        sc = O.window_scores(q_np, k_np)
        pl = O.pool(sc, pool, pool_op)
        if S > W:
            g_pl = np32(pooled[b, h])
            scale = float(np.abs(pl).max())
            np.testing.assert_allclose(g_pl, pl, rtol=1e-4, atol=1e-6 * scale)
        want = O.snapkv_select(pl, S, W, n_keep)
        got = kept[b, h].cpu().numpy()
        assert ascending(got[: n_keep - W]) or n_keep - W <= 1
        assert (got[n_keep - W:] == np.arange(S - W, S)).all()
        assert got.min() >= 0 and got[: n_keep - W].max(initial=-1) < S - W
        swaps += compare_sets(got[: n_keep - W], want[: n_keep - W], pl)
        if S > W:   # on the GPU's own pooled scores the choice is exact (ties to the lower position)
            assert np.array_equal(got, O.snapkv_select(g_pl, S, W, n_keep)), (b, h)
        if compact:
            idx = torch.as_tensor(got, dtype=torch.long, device=dev)
            assert torch.equal(ko[b, h, :n_keep], k[b, h, idx]) and torch.equal(vo[b, h, :n_keep], v[b, h, idx])
        if kmax is not None:
            nblk = -(-n_keep // aux_block)
            wmax, wmin = O.build_aux(np32(ko[b, h, :n_keep]), n_keep, aux_block)
            assert np.array_equal(np32(kmax[b, h, :, :nblk]), wmax), (b, h)
            assert np.array_equal(np32(kmin[b, h, :, :nblk]), wmin), (b, h)
            # pages beyond the compact cache are left untouched
            assert bool((kmax[b, h, :, nblk:] == 7.0).all()) and bool((kmin[b, h, :, nblk:] == 7.0).all())
    if aux_block:
        return kept, ko, vo, pooled, swaps, kmax, kmin
    return kept, ko, vo, pooled, swaps


def aux_and_check(rk, kc, n_tokens, block, n_q_heads, idx=None, units_to_check=None):
    """Run rk_hsa_build_aux over kc (or the rows idx of kc) and check bit-exactly."""
    B, Hkv, _, d = kc.shape
    nblk = -(-n_tokens // block)
    kmax = torch.empty(B, Hkv, d, rk.aux_capacity(n_tokens, block), dtype=kc.dtype, device=kc.device)
    kmin = torch.empty_like(kmax)
    rk.rk_hsa_build_aux(kc, n_tokens, 0, block, kmax, kmin, n_q_heads=n_q_heads, idx=idx)
    torch.cuda.synchronize()
    units = units_to_check or [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in units:
        rows = kc[b, h] if idx is None else kc[b, h, idx[b, h, :n_tokens].long()]
        wmax, wmin = O.build_aux(rows[:n_tokens].cpu().float().numpy(), n_tokens, block)
        assert np.array_equal(np32(kmax[b, h, :, :nblk]), wmax), (b, h)
        assert np.array_equal(np32(kmin[b, h, :, :nblk]), wmin), (b, h)
    return kmax, kmin


def decode_and_check(rk, q, kc, vc, kmax, kmin, n_tokens, block, k1, k2, cand=None,
                     units_to_check=None):
    """Run one rk_hsa_decode (or _mt when cand is given) and check against the
    oracle stage by stage.  Returns (out, sel, swaps)."""
    B, Hq, d = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    dev = q.device
    nblk = -(-n_tokens // block)
    nsel = min(k2, nblk)
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    sel = torch.empty(B, Hkv, nsel, dtype=torch.int32, device=dev)
    chan = torch.empty(B, Hkv, k1, dtype=torch.int32, device=dev)
    s1 = torch.empty(B, Hkv, nblk, dtype=torch.float32, device=dev)
    # twice: the checked call gets a workspace holding all-ones bytes (the
    # result must not depend on what the workspace held before the call)
    ws = None
    for _ in range(2):
        if ws is not None:
            ws.fill_(255)
            out.fill_(float("nan"))
        if cand is None:
            ws = rk.rk_hsa_decode(q, kc, vc, kmax, kmin, n_tokens, block, k1, k2, out, sel, chan,
                                  s1, ws=ws)
        else:
            ws = rk.rk_hsa_decode_mt(q, kc, vc, cand, n_tokens, kmax, kmin, block, k1, k2, out,
                                     sel, chan, s1, ws=ws)
    torch.cuda.synchronize()
    swaps = 0
    units = units_to_check or [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in units:
        qg = np32(q[b, h * G:(h + 1) * G])
        i1, qbar = O.channel_select(qg, k1)
        assert np.array_equal(chan[b, h].cpu().numpy(), i1), (b, h)
        ws1 = O.block_scores(qbar, i1, np32(kmax[b, h, :, :nblk]), np32(kmin[b, h, :, :nblk]))
        assert np.array_equal(np32(s1[b, h]), ws1), (b, h)           # same float32 ops, same order
        gsel = sel[b, h].cpu().numpy()
        assert ascending(gsel) or nsel == 1
        # the scores are bit-exact, so the page choice (ties to the lower page) is too
        assert np.array_equal(gsel, O.block_select(ws1, k2)), (b, h)
        toks = O.selected_tokens(gsel, n_tokens, block)
        if cand is None:
            rows = toks
        else:
            rows = cand[b, h, :n_tokens].cpu().numpy()[toks]
        ridx = torch.as_tensor(rows, dtype=torch.long, device=dev)
        want = O.attention(qg, np32(kc[b, h, ridx]), np32(vc[b, h, ridx]))
        check_output(np32(out[b, h * G:(h + 1) * G]), want)
    return out, sel, swaps


def check_aux_units(kmax, kmin, kc, n_tokens, block, units, idx=None):
    """Bit-exact Kmax/Kmin of the given units against the oracle rebuilt from scratch."""
    nblk = -(-n_tokens // block)
    for b, h in units:
        rows = kc[b, h, :n_tokens] if idx is None else kc[b, h, idx[b, h, :n_tokens].long()]
        wmax, wmin = O.build_aux(rows.cpu().float().numpy(), n_tokens, block)
        assert np.array_equal(np32(kmax[b, h, :, :nblk]), wmax), (b, h)
        assert np.array_equal(np32(kmin[b, h, :, :nblk]), wmin), (b, h)


def append_decode_and_check(rk, q, ka, va, kc, vc, kmax, kmin, pos, block, k1, k2, units_to_check,
                            ws=None):
    """One rk_hsa_append_decode step (append row `pos`, then decode over pos + 1
    tokens), checked on the given units: the appended rows, Kmax/Kmin against a
    rebuild from the cache rows (bit-exact), the channel set and page scores
    against the oracle on the post-append state (bit-exact), the page choice
    (exact on those scores) and the output against the oracle's attention over
    the chosen pages.  Returns (out, sel, ws)."""
    B, Hq, d = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    dev = q.device
    n = pos + 1
    nblk = -(-n // block)
    nsel = min(k2, nblk)
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    sel = torch.empty(B, Hkv, nsel, dtype=torch.int32, device=dev)
    chan = torch.empty(B, Hkv, k1, dtype=torch.int32, device=dev)
    s1 = torch.empty(B, Hkv, nblk, dtype=torch.float32, device=dev)
    ws = rk.rk_hsa_append_decode(q, ka, va, kc, vc, pos, kmax, kmin, block, k1, k2, out, sel, chan, s1,
                                 ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(kc[:, :, pos], ka) and torch.equal(vc[:, :, pos], va)
    check_aux_units(kmax, kmin, kc, n, block, units_to_check)
    for b, h in units_to_check:
        qg = np32(q[b, h * G:(h + 1) * G])
        i1, qbar = O.channel_select(qg, k1)
        assert np.array_equal(chan[b, h].cpu().numpy(), i1), (b, h)
        ws1 = O.block_scores(qbar, i1, np32(kmax[b, h, :, :nblk]), np32(kmin[b, h, :, :nblk]))
        assert np.array_equal(np32(s1[b, h]), ws1), (b, h)
        gsel = sel[b, h].cpu().numpy()
        assert np.array_equal(gsel, O.block_select(ws1, k2)), (b, h)
        toks = O.selected_tokens(gsel, n, block)
        ridx = torch.as_tensor(toks, dtype=torch.long, device=dev)
        want = O.attention(qg, np32(kc[b, h, ridx]), np32(vc[b, h, ridx]))
        check_output(np32(out[b, h * G:(h + 1) * G]), want)
    return out, sel, ws

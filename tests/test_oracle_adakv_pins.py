"""Pins of the oracle's Ada-KV stage-1 selection (reading R27: one prefix
budget per sequence shared by its KV heads, the largest pooled scores over
all heads together).  The pages name Ada-KV without its rule, so the rule is
parity-unpinned against them; these pins fix its consistency."""

import numpy as np
import pytest

import oracle as O


def test_worked_example_concentrated_head_keeps_fewer():
    """Hand-worked: head 0 puts its mass on one token, head 1 spreads it.  With
    a per-head budget of 3 prefix tokens (6 shared), head 0 keeps 1 and head 1
    keeps 5 (its equal scores taken lowest position first)."""
    S, W, n_keep = 8, 2, 5
    pooled = np.array([[10, 0, 0, 0, 0, 0], [2, 2, 2, 2, 2, 2]], np.float32)
    kept = O.adakv_select(pooled, S, W, n_keep)
    assert kept[0].tolist() == [0, 6, 7]
    assert kept[1].tolist() == [0, 1, 2, 3, 4, 6, 7]


@pytest.mark.parametrize("seed", range(6))
def test_equal_heads_reduce_to_per_head_snapkv(seed):
    """When every head has the same pooled scores, and no value at the cut is
    repeated within a head, the shared budget splits evenly (the cut value's
    copies span the heads), so each head keeps exactly its SnapKV selection.
    (A value repeated within a head at the cut goes to the lower heads first.)"""
    rng = np.random.default_rng(seed)
    S, W, n_keep, H = 200, 8, 57, 4
    row = rng.standard_normal(S - W).astype(np.float32)
    kept = O.adakv_select(np.tile(row, (H, 1)), S, W, n_keep)
    want = O.snapkv_select(row, S, W, n_keep)
    for h in range(H):
        assert kept[h].tolist() == want.tolist()


@pytest.mark.parametrize("seed", range(8))
def test_brute_force_and_budget(seed):
    """Counting definition over (head, position) pairs, ties to the lower pair;
    the shared budget is spent exactly; window positions always kept."""
    rng = np.random.default_rng(100 + seed)
    H, S, W = 3, 40, 4
    n_keep = int(rng.integers(W, S + 1))
    pooled = rng.integers(0, 6, (H, S - W)).astype(np.float32)      # many exact ties
    kept = O.adakv_select(pooled, S, W, n_keep)
    K = H * (n_keep - W)
    assert sum(len(x) - W for x in kept) == K
    flat = pooled.reshape(-1)
    for h in range(H):
        assert kept[h][-W:].tolist() == list(range(S - W, S))
        got = set(kept[h][:-W].tolist())
        for j in range(S - W):
            i = h * (S - W) + j
            ahead = int(np.sum(flat > flat[i]) + np.sum((flat == flat[i]) & (np.arange(flat.size) < i)))
            assert (j in got) == (ahead < K), (h, j)


def test_adakv_evict_on_a_small_prompt_conserves_the_budget():
    rng = np.random.default_rng(5)
    B, Hkv, G, S, W, d = 2, 4, 2, 300, 8, 16
    q = rng.standard_normal((B, Hkv * G, W, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    k[0, 1, 17] = 4 * q[0, 2:4].mean(axis=(0, 1))       # head 1 of batch 0 gets a strong key
    res = O.adakv_evict(q, k, W, 7, 60)
    assert (res["counts"].sum(axis=1) == Hkv * 60).all()
    assert 17 in res["kept"][0][1].tolist()


def test_equal_heads_with_a_tied_cut_favour_the_lower_heads():
    """Equal heads whose cut value repeats within a head: the tied copies are
    taken head by head, lowest head first (the flattened order)."""
    S, W, n_keep = 10, 2, 5                     # 3 prefix slots per head, 6 shared
    row = np.array([5, 3, 3, 3, 3, 0, 0, 0], np.float32)
    kept = O.adakv_select(np.tile(row, (2, 1)), S, W, n_keep)
    # 5 in both heads (2 slots), then four 3s of head 0 (4 slots)
    assert kept[0].tolist() == [0, 1, 2, 3, 4, 8, 9]
    assert kept[1].tolist() == [0, 8, 9]

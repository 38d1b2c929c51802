"""Pins of the oracle's selection baselines (Exact-TopK, Quest, SparQ) and
their budget plan against what the pages and the mathematics fix.

Sources: papercache notes on RocketKV -- background (Exact-TopK), method
details (Quest's per-page min/max, SparQ's head-dimension sparsity, the token
budget and its even split between HSA steps 2 and 3, Table 1's storage
column) and appendix A.3 (budget split evenly between estimation and
attention for Quest and SparQ; group-level Quest)."""

import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle as O


def _data(seed, N, d, G):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((G, d)).astype(np.float32), rng.standard_normal((N, d)).astype(np.float32),
            rng.standard_normal((N, d)).astype(np.float32))


# ---------------------------------------------------------------- Exact-TopK
@pytest.mark.parametrize("seed,G", [(1, 1), (2, 2), (3, 4)])
def test_exact_topk_is_brute_force_top_k_of_summed_logits(seed, G):
    """Reading R23: the group's score of token n is sum_g q_g . k_n.  Brute
    force in float64 (sum of per-head dot products, no q_bar) picks the same
    tokens whenever the cut has no near tie; for one head it is also the top-k
    by attention weight.  A max over heads, or |q| in place of q, fails."""
    q, k, _ = _data(seed, 500, 32, G)
    kk = 40
    s = O.exact_topk_scores(q, k)
    got = O.topk_lower_index(s, kk)
    exact = (q.astype(np.float64) @ k.T.astype(np.float64)).sum(axis=0)
    order = np.argsort(-exact)
    assert exact[order[kk - 1]] - exact[order[kk]] > 1e-4
    assert got.tolist() == sorted(order[:kk].tolist())
    np.testing.assert_allclose(s, exact, rtol=1e-5, atol=1e-4)
    if G == 1:
        w = softmax(q[0].astype(np.float64) @ k.T.astype(np.float64) / math.sqrt(32))
        assert got.tolist() == sorted(np.argsort(-w)[:kk].tolist())
    # the other group aggregations choose differently on these inputs
    by_max = (q.astype(np.float64) @ k.T.astype(np.float64)).max(axis=0)
    if G > 1:
        assert sorted(np.argsort(-by_max)[:kk].tolist()) != got.tolist()


def test_exact_topk_worked_example():
    """Hand-computed: q = (1, -2), rows (3, 1) -> 1, (0, -1) -> 2, (-1, -1) ->
    1, (2, 2) -> -2; top-2 are rows 0 and 1 ... with the tie between rows 0 and
    2 (both 1) going to the lower row."""
    q = np.array([[1.0, -2.0]], np.float32)
    k = np.array([[3, 1], [0, -1], [-1, -1], [2, 2]], np.float32)
    s = O.exact_topk_scores(q, k)
    assert s.tolist() == [1.0, 2.0, 1.0, -2.0]
    assert O.topk_lower_index(s, 2).tolist() == [0, 1]


# ---------------------------------------------------------------- Quest
@pytest.mark.parametrize("G,page", [(1, 16), (2, 7), (4, 33)])
def test_quest_page_score_bounds_every_token(G, page):
    """Reading R24 (and invariant I3): the page score bounds the accumulated
    score of every token of the page -- exactly in float32, since both sides
    add term by term in the same channel order and each Quest term is at
    least the token's term.  Taking min for max, or always Kmax, breaks it."""
    q, k, _ = _data(10 + G, 300, 24, G)
    kmax, kmin = O.build_aux(k, 300, page)
    s = O.quest_page_scores(q, kmax, kmin)
    tok = O.exact_topk_scores(q, k)
    for b in range(kmax.shape[1]):
        assert (s[b] >= tok[b * page:(b + 1) * page]).all(), b
    # a plausible slip (Kmax on every channel) is not a bound
    qbar = q[0].copy()
    for g in range(1, G):
        qbar = (qbar + q[g]).astype(np.float32)
    slip = np.zeros(kmax.shape[1], np.float32)
    for i in range(24):
        slip = (slip + (qbar[i] * kmax[i]).astype(np.float32)).astype(np.float32)
    assert not all((slip[b] >= tok[b * page:(b + 1) * page]).all() for b in range(kmax.shape[1]))


def test_quest_pages_of_one_token_are_exact():
    q, k, _ = _data(31, 200, 16, 2)
    kmax, kmin = O.build_aux(k, 200, 1)
    np.testing.assert_array_equal(O.quest_page_scores(q, kmax, kmin), O.exact_topk_scores(q, k))


def test_quest_equals_hsa_with_every_channel():
    """Quest's max form and HSA's sign-selected form (Algorithm 1 with k1 = d)
    are two ways of writing one bound: bit-identical in float32."""
    q, k, _ = _data(5, 400, 32, 4)
    kmax, kmin = O.build_aux(k, 400, 16)
    i1, qbar = O.channel_select(q, 32)
    np.testing.assert_array_equal(O.quest_page_scores(q, kmax, kmin), O.block_scores(qbar, i1, kmax, kmin))


# ---------------------------------------------------------------- SparQ
def test_sparq_with_every_channel_is_exact_topk():
    """Invariant I5: with r = d SparQ's score is the exact accumulated logit."""
    q, k, _ = _data(6, 256, 16, 4)
    np.testing.assert_array_equal(O.sparq_scores(q, k, 16), O.exact_topk_scores(q, k))


def test_sparq_channel_choice_sums_magnitudes_over_the_group():
    """Channels are ranked by sum_g |q_g| (not |sum_g q_g|): two heads with
    opposite large values on channel 0 make it the first choice although
    q_bar_0 = 0, which then contributes nothing to the score."""
    q = np.array([[5.0, 0.5, -1.0, 0.0], [-5.0, 0.5, 0.2, 0.1]], np.float32)
    assert O.sparq_channels(q, 1).tolist() == [0]
    assert O.sparq_channels(q, 2).tolist() == [0, 2]
    k = np.array([[9.0, 1.0, 1.0, 1.0], [-9.0, 2.0, 0.0, 0.0]], np.float32)
    # r = 2: channels 0 (q_bar 0) and 2 (q_bar -0.8): scores -0.8 and 0
    np.testing.assert_allclose(O.sparq_scores(q, k, 2), [-0.8, 0.0], rtol=0, atol=1e-7)


def test_sparq_one_head_takes_largest_magnitude_query_channels():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 64)).astype(np.float32)
    want = sorted(np.argsort(-np.abs(q[0]))[:7].tolist())
    assert O.sparq_channels(q, 7).tolist() == want


# ---------------------------------------------------------------- plan
@pytest.mark.parametrize("c,S,d", [(16, 32768, 128), (64, 65536, 128), (4, 4096, 64)])
def test_plan_splits_the_budget_evenly(c, S, d):
    """[RKV] token budget paragraph and A.3: estimation and attention each get
    t/2 KV pairs (exactly, where the sizes divide)."""
    t = S / c
    for m in ("hsa", "quest", "sparq"):
        p = O.select_plan(m, c, S, d)
        assert p["est_pairs"] == pytest.approx(t / 2), m
        assert p["k2"] * p["page"] == pytest.approx(t / 2), m
    e = O.select_plan("exact", c, S, d)
    assert (e["page"], e["channels"], e["k2"]) == (1, d, t)


def test_plan_values_on_the_workloads():
    """The Llama-8B layer (c 16) and the 109K needle (c 428)."""
    assert [O.select_plan(m, 16, 32768, 128)[x] for m in ("hsa", "quest", "sparq")
            for x in ("page", "channels", "k2")] == [4, 32, 256, 16, 128, 64, 1, 8, 1024]
    n = O.select_plan("quest", 109568 / 256, 109568, 128)
    assert (n["page"], n["k2"], n["attn_tokens"]) == (428, 1, 428)       # one page exceeds t/2
    s = O.select_plan("sparq", 109568 / 256, 109568, 128)
    assert (s["channels"], s["k2"]) == (1, 128) and s["est_pairs"] > 128  # one channel exceeds t/2
    h = O.select_plan("hsa", 109568 / 256, 109568, 128)
    assert (h["page"], h["channels"], h["k2"]) == (21, 6, 7)


def test_quest_storage_matches_table1():
    """Table 1: Quest stores 1 + 1/c of the full cache (Kmax and Kmin, d values
    each, per page of c tokens, against 2d values per KV pair)."""
    for c in (4, 16, 64):
        S, d = 4096 * c, 128
        p = O.select_plan("quest", c, S, d)
        aux_values = 2 * d * (S // p["page"])
        assert 1 + aux_values / (2 * d * S) == pytest.approx(1 + 1 / c)


# ---------------------------------------------------------------- decode
@pytest.mark.parametrize("method,page,ch", [("hsa", 4, 8), ("quest", 16, 32), ("sparq", 1, 4), ("exact", 1, 32)])
def test_select_decode_all_pages_is_dense_attention(method, page, ch):
    q, k, v = _data(12, 150, 32, 2)
    res = O.select_decode_unit(method, q, k, v, 150, page, ch, 10 ** 6)
    want = softmax(q.astype(np.float64) @ k.T.astype(np.float64) / math.sqrt(32), axis=1) @ v
    np.testing.assert_allclose(res["out"], want, rtol=1e-10, atol=1e-12)
    assert len(res["tokens"]) == 150


def test_select_decode_exact_attends_the_top_tokens():
    q, k, v = _data(13, 300, 32, 1)
    res = O.select_decode_unit("exact", q, k, v, 300, 1, 32, 25)
    dots = k.astype(np.float64) @ q[0].astype(np.float64)
    assert res["tokens"].tolist() == sorted(np.argsort(-dots)[:25].tolist())

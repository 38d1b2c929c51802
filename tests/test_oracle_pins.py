"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  Each one is chosen so that a plausible slip in
the oracle (a dropped term, a flipped sign or mask, a wrong index or a
transposed operand) fails it.  Sources are the papercache notes on RocketKV
([RKV]) and the aifetchly RocketKV guide ([GUIDE]).
"""

import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kv_line(line):
    return {k: float(v) for k, v in (t.split("=") for t in line.split()[(1 if line.startswith("tol") else 0):])}


# ---------------------------------------------------------------- split
def test_split_worked_example():
    """[RKV] method details, the printed c = 64 example."""
    lines = [ln for ln in open(os.path.join(GOLDEN, "split_worked_example.txt")) if not ln.startswith("#")]
    want, tol = _kv_line(lines[0]), _kv_line(lines[1])
    s = O.split(want["c"], 65536, 32, 16, 128)
    assert abs(s["r"] - want["r"]) <= tol["r"]
    assert abs(s["c1"] - want["stage1"]) <= tol["stage1"]
    assert abs(s["c2"] - want["stage2"]) <= tol["stage2"]
    assert s["paper_page"] == int(want["page"])
    assert abs(s["c2"] / s["paper_page"] - want["headdim"]) <= tol["headdim"]
    # the two stages multiply back to the total ratio
    assert math.isclose(s["c1"] * s["c2"], want["c"], rel_tol=1e-12)


def test_split_paper_decomposition_halves_budget():
    """[RKV] token budget paragraph: the budget t is shared evenly between HSA
    steps 2 and 3; split inside HSA: pages of ceil(c^((1-r)/2)) tokens and
    k1 = d / (c^(1-r)/page) channels.  Step 3 then fetches about t/2 KV
    pairs, and step 2 (k1 sign-selected aux values for each of the N1/page
    pages, d-element KV rows counted in pairs of two) about t/2 as well."""
    # the printed c = 64 example: page 3, head-dim share 6.2 / 3 ~ 2.1, so about 62 of 128 channels
    s = O.split(64.0, 65536, 32, 16, 128)
    assert s["paper_page"] == 3 and s["paper_k1_channels"] == 62
    for c, S, d in [(16, 32768, 128), (64, 32768, 128), (428, 109568, 128), (32, 36864, 128), (8, 2048, 64)]:
        s = O.split(c, S, 32, 16, d)
        page, t = s["paper_page"], s["budget_t"]
        # step 3: the smallest page count covering half the budget
        assert s["paper_k2_blocks"] * page >= t / 2 > (s["paper_k2_blocks"] - 1) * page
        # step 2: k1 aux values per page over the stage-1 pages, in KV-pair units
        step2_pairs = s["paper_k1"] * (S / s["c1"] / page) / (2 * d)
        assert step2_pairs == pytest.approx(t / 2, rel=1e-9)
        assert abs(s["paper_k1_channels"] - s["paper_k1"]) <= 0.5


def test_split_clamp_bounds():
    """[RKV] prose after the r equation: r is restricted to [0.2, 0.8]."""
    assert O.split(1.0, 4096, 16, 16, 64)["r"] == pytest.approx(0.2)
    assert O.split(2.0 ** 10, 1 << 20, 16, 16, 64)["r"] == pytest.approx(0.8)
    assert O.split(2.0 ** 30, 1 << 31, 16, 16, 64)["r"] == pytest.approx(0.8)
    # monotone in c between the bounds
    rs = [O.split(c, 1 << 20, 16, 16, 64)["r"] for c in (1, 2, 4, 8, 16, 64, 256, 1024, 4096)]
    assert all(a <= b for a, b in zip(rs, rs[1:]))
    with pytest.raises(ValueError):
        O.split(0.5, 1024, 16, 16, 64)


def test_split_budget_covers_stages():
    """[RKV] token budget paragraph: t = S / c; the stage-1 keep count covers
    S / c^r (rounded up, never below the window, never above S)."""
    for c, S, W in [(8, 2048, 16), (16, 32768, 32), (64, 32768, 32), (428, 109568, 32), (32, 33792, 32)]:
        s = O.split(c, S, W, 16, 128)
        assert s["budget_t"] == pytest.approx(S / c)
        assert s["n_keep"] >= S / s["c1"] - 1e-9 and s["n_keep"] - 1 < S / s["c1"]
        assert s["k2_blocks"] * 16 >= s["budget_t"] > (s["k2_blocks"] - 1) * 16
    assert O.split(1.0, 100, 10, 16, 64)["n_keep"] == 100
    assert O.split(1e6, 100, 10, 16, 64)["n_keep"] == 10


def test_table1_closed_forms():
    """[RKV] Table 1: the derivation in the oracle (stage-1 share times per-page
    aux overhead, two tensors) equals the table's closed forms."""
    rows = {}
    for ln in open(os.path.join(GOLDEN, "table1_closed_forms.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        name, storage, traffic = (p.strip() for p in ln.split("|"))
        rows[name] = (storage, traffic)
    for c in (2.0, 8.0, 16.0, 64.0, 428.0, 5000.0):
        r = O.split(c, 1 << 20, 1, 1, 1)["r"]
        got = O.table1_storage_traffic(c)
        env = {"c": c, "r": r}
        assert got["rocketkv_storage"] == pytest.approx(eval(rows["RocketKV"][0], {}, env), rel=1e-12)
        assert got["mt_storage"] == pytest.approx(eval(rows["RocketKV-MT"][0], {}, env), rel=1e-12)
        assert got["traffic"] == pytest.approx(eval(rows["RocketKV"][1], {}, env), rel=1e-12)


# ---------------------------------------------------------------- top-k
def _brute_topk(v, k):
    n = len(v)
    return sorted(j for j in range(n)
                  if sum(1 for i in range(n) if v[i] > v[j] or (v[i] == v[j] and i < j)) < k)


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force(seed):
    """Counting definition of top-k with the lower-index tie rule."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    v = rng.integers(-4, 5, n).astype(np.float32)          # many exact ties
    if seed % 3 == 0:
        v = rng.standard_normal(n).astype(np.float32)
    for k in {0, 1, n // 2, n - 1 if n > 1 else 1, n}:
        assert list(O.topk_lower_index(v, k)) == _brute_topk(v, k)


def test_topk_signed_zero_is_a_tie():
    v = np.array([0.0, -0.0, 0.0, -1.0], np.float32)
    v[1] = -0.0
    assert list(O.topk_lower_index(v, 2)) == [0, 1]


# ---------------------------------------------------------------- pooling
@pytest.mark.parametrize("k", [1, 3, 7, 63])
def test_pool_is_box_filter(k):
    """[RKV] pooling paragraph: zero-padded windowed sum.  Integer-valued input
    makes every order exact, so it must equal numpy's full convolution with a
    box, cropped to 'same'."""
    rng = np.random.default_rng(k)
    s = rng.integers(0, 50, 200).astype(np.float32)
    want = np.convolve(s, np.ones(k), mode="same")
    np.testing.assert_array_equal(O.pool_sum(s, k), want.astype(np.float32))
    delta = np.zeros(101, np.float32)
    delta[50] = 1.0
    out = O.pool_sum(delta, k)
    assert out.sum() == k and np.all(out[50 - k // 2:51 + k // 2] == 1)
    with pytest.raises(ValueError):
        O.pool_sum(s, 4)


def test_pool_left_to_right_order():
    """The sum is taken left to right: 1 + 2^-24 + 2^-24 stays 1 in float32
    (each small term is lost), while the right-to-left order would keep them."""
    s = np.array([1.0, 2.0 ** -24, 2.0 ** -24], np.float32)
    assert O.pool_sum(s, 3)[1] == np.float32(1.0)


def test_pool_max_hand_worked():
    """Max pooling (the other reading of the pooling paragraph), worked by hand:
    windows are cut at the ends, never padded into the result."""
    s = np.array([1, 5, 2, 0, 3], np.float32)
    assert O.pool_max(s, 1).tolist() == [1, 5, 2, 0, 3]
    assert O.pool_max(s, 3).tolist() == [5, 5, 5, 3, 3]
    assert O.pool_max(s, 5).tolist() == [5, 5, 5, 5, 3]
    assert O.pool_max(s, 63).tolist() == [5] * 5
    with pytest.raises(ValueError):
        O.pool_max(s, 2)
    with pytest.raises(ValueError):
        O.pool(s, 3, "mean")


@pytest.mark.parametrize("k", [1, 7, 63])
def test_pool_max_is_a_maximum_filter(k):
    """Equal to scipy's one-dimensional maximum filter with out-of-range
    samples ignored, and a spike spreads to exactly k positions."""
    from scipy.ndimage import maximum_filter1d
    rng = np.random.default_rng(k)
    s = rng.random(300).astype(np.float32)
    want = maximum_filter1d(s, size=k, mode="constant", cval=-np.inf)
    np.testing.assert_array_equal(O.pool_max(s, k), want)
    delta = np.zeros(101, np.float32)
    delta[50] = 2.0
    out = O.pool_max(delta, k)
    assert (out == 2.0).sum() == k and np.all(out[50 - k // 2:51 + k // 2] == 2.0)


def test_pool_max_kernel_one_is_sum_kernel_one():
    """With kernel 1 both readings leave the scores as they are, so stage 1
    keeps the same tokens under either."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 4, 8, 16)).astype(np.float32)
    k = rng.standard_normal((1, 2, 120, 16)).astype(np.float32)
    a = O.snapkv_evict(q, k, None, 8, 1, 40)
    b = O.snapkv_evict(q, k, None, 8, 1, 40, pool_op="max")
    assert np.array_equal(a["kept"], b["kept"]) and np.array_equal(a["pooled"], b["pooled"])
    c = O.snapkv_evict(q, k, None, 8, 7, 40, pool_op="max")
    for h in range(2):
        sc = O.window_scores(q[0, 2 * h:2 * h + 2], k[0, h])
        np.testing.assert_array_equal(c["pooled"][0, h], O.pool_max(sc, 7))


# ---------------------------------------------------------------- window scores
def _window_scores_loop(q, k):
    """Pure-Python per-row softmax on a tiny case (brute force)."""
    G, W, d = q.shape
    S = k.shape[0]
    out = [0.0] * (S - W)
    for g in range(G):
        for r in range(W):
            vis = S - W + r
            logits = [sum(float(q[g, r, c]) * float(k[j, c]) for c in range(d)) / math.sqrt(d)
                      for j in range(vis + 1)]
            m = max(logits)
            z = sum(math.exp(x - m) for x in logits)
            for j in range(S - W):
                out[j] += math.exp(logits[j] - m) / z
    return np.array(out)


@pytest.mark.parametrize("G,W,S,d", [(1, 1, 9, 4), (2, 3, 17, 8), (4, 4, 23, 8)])
def test_window_scores_brute_force(G, W, S, d):
    rng = np.random.default_rng(S)
    q = rng.standard_normal((G, W, d)).astype(np.float32)
    k = rng.standard_normal((S, d)).astype(np.float32)
    np.testing.assert_allclose(O.window_scores(q, k), _window_scores_loop(q, k), rtol=2e-5, atol=1e-7)


def test_window_scores_mass_and_causality():
    """Total probability of each row is 1: with the window keys pushed far away
    the prefix holds G*W of mass.  With the LAST window key made dominant, only
    the last row may see it (causal), so the prefix keeps G*(W-1) of mass."""
    rng = np.random.default_rng(1)
    G, W, S, d = 4, 8, 300, 16
    q = rng.standard_normal((G, W, d)).astype(np.float32)
    qdir = q.reshape(-1, d).mean(0)
    qdir /= np.linalg.norm(qdir)
    k = rng.standard_normal((S, d)).astype(np.float32)
    k_far = k.copy()
    k_far[S - W:] = -30.0 * qdir                               # window keys unattractive
    q_al = (qdir[None, None, :] * 2.0 + 0.1 * q).astype(np.float32)
    assert O.window_scores(q_al, k_far).sum() == pytest.approx(G * W, rel=1e-4)
    k_hot = k_far.copy()
    k_hot[S - 1] = 60.0 * qdir                                 # only row W-1 can see this key
    tot = O.window_scores(q_al, k_hot).sum()
    assert tot == pytest.approx(G * (W - 1), rel=1e-4)


def test_snapkv_w1_g1_k1_is_exact_topk():
    """W = 1, G = 1, pool 1: softmax is monotone, so the kept prefix is the
    exact top of q.k (float64 brute force, no near ties in the data)."""
    rng = np.random.default_rng(7)
    S, d, n_keep = 400, 32, 61
    q = rng.standard_normal((1, 1, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, S, d)).astype(np.float32)
    dots = k[0, 0].astype(np.float64) @ q[0, 0, 0].astype(np.float64)
    pre = dots[: S - 1]
    order = np.argsort(-pre)
    assert pre[order[n_keep - 2]] - pre[order[n_keep - 1]] > 1e-3   # no near tie at the cut
    res = O.snapkv_evict(q, k, k, 1, 1, n_keep)
    want = sorted(order[: n_keep - 1].tolist()) + [S - 1]
    assert res["kept"][0, 0].tolist() == want


def test_snapkv_keep_all_and_window_only():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, S, W, d = 2, 4, 2, 64, 8, 16
    q = rng.standard_normal((B, Hq, W, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    all_ = O.snapkv_evict(q, k, v, W, 7, S)
    assert (all_["kept"] == np.arange(S)).all()
    np.testing.assert_array_equal(all_["k"], k)
    np.testing.assert_array_equal(all_["v"], v)
    win = O.snapkv_evict(q, k, v, W, 7, W)
    assert (win["kept"] == np.arange(S - W, S)).all()
    with pytest.raises(ValueError):
        O.snapkv_evict(q, k, v, W, 7, W - 1)


def test_snapkv_group_shares_selection_and_pools_neighbours():
    """[RKV] GQA paragraph: the group's heads share one selection.  [RKV]
    pooling paragraph: a key token is kept with its neighbours -- a single
    dominant key pulls in the (kernel-1)/2 tokens on each side."""
    rng = np.random.default_rng(5)
    G, W, S, d, kern = 4, 4, 512, 32, 7
    qdir = rng.standard_normal(d).astype(np.float32)
    qdir *= math.sqrt(d) / np.linalg.norm(qdir)
    q = (qdir + 0.3 * rng.standard_normal((1, G, W, d))).astype(np.float32)
    k = (0.3 * rng.standard_normal((1, 1, S, d))).astype(np.float32)
    k[0, 0, 200] = 3 * qdir
    res = O.snapkv_evict(q, k, None, W, kern, W + kern)
    assert res["kept"][0, 0].tolist() == list(range(197, 204)) + list(range(S - W, S))


# ---------------------------------------------------------------- aux
def test_build_aux_bounds_and_attained():
    """[RKV] HSA step 1: element-wise page max/min, last page partial."""
    rng = np.random.default_rng(11)
    N, d, B = 83, 12, 16
    kc = rng.standard_normal((N + 5, d)).astype(np.float32)
    kc[N:] = 1e9                                                   # rows past n_tokens ignored
    kmax, kmin = O.build_aux(kc, N, B)
    assert kmax.shape == (d, -(-N // B))
    for b in range(kmax.shape[1]):
        rows = kc[b * B:min((b + 1) * B, N)]
        for c in range(d):
            assert np.all(rows[:, c] <= kmax[c, b]) and kmax[c, b] in rows[:, c]
            assert np.all(rows[:, c] >= kmin[c, b]) and kmin[c, b] in rows[:, c]


# ---------------------------------------------------------------- HSA step 2
def test_channel_select_g1_is_top_abs_q_and_sign_zero():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 40)).astype(np.float32)
    i1, qbar = O.channel_select(q, 9)
    assert i1.tolist() == _brute_topk(np.abs(q[0]), 9)
    np.testing.assert_array_equal(qbar, q[0])
    # two heads that cancel: q_bar = 0 everywhere -> Kmax side (sign >= 0)
    q2 = np.stack([q[0], -q[0]])
    i1b, qb = O.channel_select(q2, 9)
    assert i1b.tolist() == i1.tolist() and np.all(qb == 0)
    kmax = rng.standard_normal((40, 6)).astype(np.float32)
    kmin = kmax - 1
    assert np.all(O.block_scores(qb, i1b, kmax, kmin) == 0)


@pytest.mark.parametrize("G", [1, 2, 4])
def test_block_score_upper_bound_with_all_channels(G):
    """k1 = d: the sign-selected Kmax/Kmin score bounds q_bar.k of every token
    of its page, in float32 with the same (ascending channel) order."""
    rng = np.random.default_rng(G)
    N, d, B = 203, 16, 16
    kc = rng.standard_normal((N, d)).astype(np.float32)
    q = rng.standard_normal((G, d)).astype(np.float32)
    kmax, kmin = O.build_aux(kc, N, B)
    i1, qbar = O.channel_select(q, d)
    s1 = O.block_scores(qbar, i1, kmax, kmin)
    for n in range(N):
        dot = np.float32(0)
        for i in range(d):
            dot = np.float32(dot + np.float32(qbar[i] * kc[n, i]))
        assert s1[n // B] >= dot
    # and a wrong sign choice breaks the bound on this data
    bad = np.zeros_like(s1)
    for i in range(d):
        bad = (bad + qbar[i] * (kmin[i] if qbar[i] >= 0 else kmax[i])).astype(np.float32)
    assert np.any(bad < s1)


def test_hsa_block1_all_channels_is_exact_topk():
    """Page size 1, k1 = d, G = 1: s1 = q.k exactly, so the pages chosen are the
    exact top-k2 tokens by q.k (float64 brute force, no near ties)."""
    rng = np.random.default_rng(9)
    N, d, k2 = 300, 24, 37
    kc = rng.standard_normal((N, d)).astype(np.float32)
    vc = rng.standard_normal((N, d)).astype(np.float32)
    q = rng.standard_normal((1, d)).astype(np.float32)
    kmax, kmin = O.build_aux(kc, N, 1)
    res = O.hsa_unit(q, kc, vc, kmax, kmin, N, 1, d, k2)
    dots = kc.astype(np.float64) @ q[0].astype(np.float64)
    srt = np.sort(dots)[::-1]
    assert srt[k2 - 1] - srt[k2] > 1e-4                     # no near tie at the cut
    assert res["sel"].tolist() == sorted(np.argsort(-dots)[:k2].tolist())


@pytest.mark.parametrize("G,N,B", [(1, 64, 16), (4, 203, 16), (2, 50, 7)])
def test_hsa_all_pages_is_dense_attention(G, N, B):
    """k2 >= number of pages: HSA is dense attention (textbook softmax)."""
    rng = np.random.default_rng(N)
    d = 32
    kc = rng.standard_normal((N, d)).astype(np.float32)
    vc = rng.standard_normal((N, d)).astype(np.float32)
    q = rng.standard_normal((G, d)).astype(np.float32)
    kmax, kmin = O.build_aux(kc, N, B)
    res = O.hsa_unit(q, kc, vc, kmax, kmin, N, B, 5, 10 ** 6)
    assert res["sel"].tolist() == list(range(kmax.shape[1]))
    want = softmax(q.astype(np.float64) @ kc.T.astype(np.float64) / math.sqrt(d), axis=1) @ vc
    np.testing.assert_allclose(res["out"], want, rtol=1e-10, atol=1e-12)


def test_hsa_decode_batch_heads_grouping():
    """Query head j uses KV head j // G: permuting KV heads permutes outputs in
    whole groups."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, N, d = 2, 8, 2, 96, 16
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    kc = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    vc = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    a = O.hsa_decode(q, kc, vc, N, 16, 8, 3)
    b = O.hsa_decode(q[:, [4, 5, 6, 7, 0, 1, 2, 3]], kc[:, ::-1], vc[:, ::-1], N, 16, 8, 3)
    np.testing.assert_allclose(a["out"][:, :4], b["out"][:, 4:])
    np.testing.assert_allclose(a["out"][:, 4:], b["out"][:, :4])


# ---------------------------------------------------------------- MT
def test_mt_ignores_non_candidates():
    """[RKV] RocketKV-MT: stage 2 chooses only among the stage-1 subset.  Tokens
    outside it never contribute, however attractive."""
    rng = np.random.default_rng(8)
    M, d, G, B = 400, 32, 2, 16
    kf = rng.standard_normal((M, d)).astype(np.float32)
    vf = rng.standard_normal((M, d)).astype(np.float32)
    q = rng.standard_normal((G, d)).astype(np.float32)
    cand = np.sort(rng.choice(M, 120, replace=False))
    out_set = np.setdiff1d(np.arange(M), cand)
    kf_hot = kf.copy()
    kf_hot[out_set] = 50.0 * q.sum(0) / np.linalg.norm(q.sum(0))
    a = O.hsa_decode_mt_unit(q, kf, vf, cand, B, 8, 4)
    b = O.hsa_decode_mt_unit(q, kf_hot, vf, cand, B, 8, 4)
    assert a["sel"].tolist() == b["sel"].tolist()
    np.testing.assert_array_equal(a["out"], b["out"])
    # with every page chosen, MT equals dense attention over the candidates
    c = O.hsa_decode_mt_unit(q, kf, vf, cand, B, 8, 10 ** 6)
    want = softmax(q.astype(np.float64) @ kf[cand].T.astype(np.float64) / math.sqrt(d), axis=1) @ vf[cand]
    np.testing.assert_allclose(c["out"], want, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- attention (closed forms)
def test_attention_zero_query_is_mean_of_values():
    """[RKV] HSA step 3 / Algorithm 1, y = attn(q, K[i2], V[i2]): with q = 0
    every logit is 0, so each weight is 1/n and the output is the plain mean
    of the value rows (worked by hand, no softmax call)."""
    rng = np.random.default_rng(21)
    for n, d, G in [(1, 8, 1), (5, 16, 2), (37, 32, 4)]:
        k = rng.standard_normal((n, d))
        v = rng.standard_normal((n, d))
        out = O.attention(np.zeros((G, d)), k, v)
        want = v.sum(axis=0) / n
        for g in range(G):
            np.testing.assert_allclose(out[g], want, rtol=0, atol=1e-14)


def test_attention_two_keys_log3_apart_weigh_three_to_one():
    """Two keys whose scaled logits differ by ln 3 get weights exactly 3/4 and
    1/4: e^(ln 3) / (e^(ln 3) + 1) = 3/4.  d = 4, so the 1/sqrt(d) scale is
    1/2 and q carries 2 ln 3 on channel 0; a transposed operand, a missing or
    doubled scale, or a swapped K/V each move the result."""
    d = 4
    q = np.array([[2.0 * math.log(3.0), 0.0, 0.0, 0.0]])
    k = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]])   # logits ln 3 and 0
    v = np.array([[4.0, 0.0, -8.0, 1.0], [0.0, 8.0, 4.0, 1.0]])
    out = O.attention(q, k, v)
    np.testing.assert_allclose(out[0], [3.0, 2.0, -5.0, 1.0], rtol=0, atol=1e-13)
    # a second head with the logits swapped (ln 3 on the second key) takes the mirror weights
    q2 = np.array([[2.0 * math.log(3.0), 0.0, 0.0, 0.0], [0.0, 2.0 * math.log(3.0), 0.0, 0.0]])
    out2 = O.attention(q2, k, v)
    np.testing.assert_allclose(out2[1], [1.0, 6.0, 1.0, 1.0], rtol=0, atol=1e-13)
    # a shift common to every logit changes nothing (softmax is shift invariant):
    # a third key with logit ln 3 as well splits the weight 3/7, 1/7, 3/7
    k3 = np.vstack([k, [[1.0, 0.0, 0.0, 0.0]]])
    v3 = np.vstack([v, [[0.0, 0.0, 0.0, 8.0]]])
    out3 = O.attention(q, k3, v3)
    np.testing.assert_allclose(out3[0], [12.0 / 7, 8.0 / 7, -20.0 / 7, 4.0], rtol=0, atol=1e-13)


def test_attention_single_key_returns_its_value():
    """With one key the softmax weight is 1 whatever the logit (here a large
    one, which a missing max subtraction would overflow)."""
    v = np.array([[0.5, -2.0, 3.25]])
    out = O.attention(np.array([[900.0, 0.0, 0.0]]), np.array([[1.0, 0.0, 0.0]]), v)
    np.testing.assert_allclose(out[0], v[0], rtol=0, atol=0)


def test_block_select_and_selected_tokens_hand_worked():
    """Page choice and the tokens it covers, worked by hand: ties go to the
    lower page, the choice is ascending, k2 past the page count takes every
    page, and a ragged last page covers only its valid tokens."""
    s1 = np.array([0.5, 2.0, 2.0, -1.0, 3.0], np.float32)
    assert O.block_select(s1, 1).tolist() == [4]
    assert O.block_select(s1, 2).tolist() == [1, 4]          # 2.0 at pages 1 and 2: the lower wins
    assert O.block_select(s1, 3).tolist() == [1, 2, 4]
    assert O.block_select(s1, 99).tolist() == [0, 1, 2, 3, 4]
    assert O.selected_tokens(np.array([0, 2]), 8, 3).tolist() == [0, 1, 2, 6, 7]
    assert O.selected_tokens(np.array([1]), 8, 3).tolist() == [3, 4, 5]
    assert O.selected_tokens(np.array([], np.int64), 8, 3).tolist() == []

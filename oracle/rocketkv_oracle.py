"""Plain CPU oracle for RocketKV's two-stage KV-cache compression hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library and imports nothing but numpy and the standard
library.  It is written to be read against the pages, not to be fast.

Sources (cited by key in every docstring below):

[RKV]   papercache.org deep notes "RocketKV: Accelerating Long-Context LLM
        Inference via Two-Stage KV Cache Compression" (arXiv 2502.14051,
        ICML'25).  Sections used: quick read ("how it works"), method details
        (SnapKV stage, GQA group-level selection, pooling kernel size, HSA
        steps 1-3, Algorithm 1, RocketKV-MT, token budget, adaptive split
        equation for r, split inside HSA and its worked c=64 example,
        storage/traffic analysis and Table 1).
[GUIDE] aifetchly blog "RocketKV Guide: Two-Stage KV Cache Compression for
        LLMs", section "Stage 1: Coarse-Grain Permanent Eviction via SnapKV"
        (observation window and softmax(Q K^T / sqrt(D)) scoring).

Precision.  Every quantity that decides an index set (window scores, pooled
scores, channel magnitudes, approximate block scores) is computed in float32,
the precision both sides must take such decisions in; reductions whose order
could change a float32 result that decides an index are written in an
explicit order (stated per function).  The attention output, which decides
nothing, is computed in float64.  bf16 inputs are up-cast exactly by the
caller (every bf16 value is an exact float32).

Readings where the pages are silent or ambiguous:
  R1  r is clamped to [0.2, 0.8] (the prose bound), c >= 1 is required.
  R2  the stage-1 keep count is ceil(S / c^r), at least the window W and at
      most S.
  R3  k2 (in blocks) = ceil(t / block) with t = S / c the token budget.
  R5  softmax scale 1/sqrt(d) for both window scoring and decode attention.
  R6  window rows attend causally (row r at position S-W+r sees keys <= it).
  R7  candidates for eviction are the prefix [0, S-W); the window is kept.
  R8  group aggregation is a sum over the G heads and the W window rows.
  R9  pooling is an average pool evaluated as a zero-padded windowed SUM of
      width k (same ranking as the average); parity of this choice with the
      pages is unpinned.  Max pooling, the other plain reading, is kept as
      the option pool_op="max" (pool_max).
  R11 ties in every top-k go to the lower index.
  R12 kept tokens are stored in ascending original position.
  R14 sign 0 selects Kmax (q_bar >= 0).
  R15 the approximate block score is sum over i in i1 of q_bar_i * P_i[b].
  R16 no block is forced into the selection.
  R17 RocketKV-MT builds blocks over the sorted candidate list.
  R23-R26 (the Exact-TopK, Quest and SparQ baselines and their budgets) and
      R27 (Ada-KV's shared budget; parity unpinned against the pages, which
      name Ada-KV but not its rule) are stated with their functions at the
      end of this module.
"""

from __future__ import annotations

import math

import numpy as np

F32 = np.float32


# --------------------------------------------------------------------------
# Adaptive compression split
# --------------------------------------------------------------------------
def split(c: float, seq_len: int, window: int, block: int, head_dim: int) -> dict:
    """Adaptive split of the total compression ratio c.

    [RKV] method details, adaptive split equation: r = min(0.2 + 0.06*log2 c,
    0.8), and the prose right after it restricting r to [0.2, 0.8]; stage 1
    takes c^r, stage 2 takes c^(1-r).  [RKV] token budget paragraph: t = S/c
    (KV pairs fetched per attention op, per GQA group).  [RKV] split inside
    HSA: page = ceil(c^((1-r)/2)) on the sequence axis, the head-dim axis gets
    c^(1-r)/page, hence k1 = d / (c^(1-r)/page).

    Returns float64 scalars r, c1, c2, t and the integer sizes n_keep (stage-1
    kept tokens, reading R2), k2_blocks (reading R3), paper_page and the
    paper's (real-valued) k1.  The notes' own decomposition also shares the
    budget t evenly between HSA steps 2 and 3 ([RKV] token budget paragraph):
    paper_k2_blocks = ceil((t/2) / paper_page) pages for step 3 and
    paper_k1_channels = paper_k1 rounded to the nearest integer in [1, d]
    (reading R22).
    """
    if not (c >= 1.0):
        raise ValueError("compression ratio must be >= 1")
    if not (0 < window <= seq_len) or block < 1 or head_dim < 1:
        raise ValueError("bad sizes")
    r = min(max(0.2 + 0.06 * math.log2(c), 0.2), 0.8)
    c1 = c ** r
    c2 = c ** (1.0 - r)
    t = seq_len / c
    n_keep = min(seq_len, max(window, math.ceil(seq_len / c1)))
    k2 = max(1, math.ceil(t / block))
    page = math.ceil(c ** ((1.0 - r) / 2.0))
    paper_k1 = head_dim / (c2 / page)
    paper_k1_channels = min(head_dim, max(1, math.floor(paper_k1 + 0.5)))
    paper_k2 = max(1, math.ceil(t / 2.0 / page))
    return dict(r=r, c1=c1, c2=c2, budget_t=t, n_keep=n_keep, k2_blocks=k2,
                paper_page=page, paper_k1=paper_k1, paper_k1_channels=paper_k1_channels,
                paper_k2_blocks=paper_k2)


def table1_storage_traffic(c: float) -> dict:
    """Normalised KV storage (including aux data) and traffic at ratio c.

    [RKV] storage/traffic analysis and Table 1: after stage 1 the relative KV
    storage is 1/c^r; the element-wise max and min tensors each add
    1/c^((1-r)/2) of that (one value per page of size c^((1-r)/2), rounding
    ignored), giving 2/c^((1+r)/2).  RocketKV-MT keeps the full cache (1).
    Traffic is 1/c for both.
    """
    r = split(c, 1 << 20, 1, 1, 1)["r"]
    after_stage1 = 1.0 / c ** r
    per_tensor = 1.0 / c ** ((1.0 - r) / 2.0)
    aux = after_stage1 * per_tensor * 2.0
    return dict(rocketkv_storage=after_stage1 + aux, mt_storage=1.0 + aux,
                traffic=1.0 / c)


# --------------------------------------------------------------------------
# Top-k with the lower-index tie rule
# --------------------------------------------------------------------------
def topk_lower_index(values: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest values, ties to the lower index, ascending.

    [RKV] Algorithm 1 (argtopk) and the stage-1 top-k; tie rule is reading
    R11.  Defined by a stable sort on the negated values: among equal values
    the original (ascending) index order survives, so the first k entries are
    exactly {j : #{i : v_i > v_j or (v_i == v_j and i < j)} < k}.  -0.0 and
    +0.0 compare equal here.  Returned sorted ascending (reading R12).
    """
    values = np.asarray(values)
    n = values.shape[0]
    if not (0 <= k <= n):
        raise ValueError("k out of range")
    order = np.argsort(-values, kind="stable")
    return np.sort(order[:k]).astype(np.int64)


# --------------------------------------------------------------------------
# Stage 1: SnapKV window scoring, pooling, selection, compaction
# --------------------------------------------------------------------------
def window_scores(q_win_group: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Group-aggregated observation-window attention over the prefix.

    [RKV] method details, SnapKV paragraph (aggregate attention between the
    input context and the observation window at the prompt tail) and the GQA
    paragraph (selection on group-level aggregated scores, shared by the
    group); [GUIDE] stage 1, softmax(Q_obs K^T / sqrt(D)) summed over the
    window.

    q_win_group: [G, W, d] float32, the window queries of the G query heads
    that share this KV head (window row r sits at position S-W+r).
    k: [S, d] float32.
    Returns score[j] for j in [0, S-W), float32:
        score[j] = sum_g sum_r softmax_row(L[g, r, :])[j],
        L[g, r, j] = q[g, r] . k[j] / sqrt(d), masked to -inf for j > S-W+r.
    Readings R5, R6, R7, R8.  Summation order is numpy's (no index decision
    depends on it beyond the stated tolerance).
    """
    q = np.asarray(q_win_group, dtype=F32)
    k = np.asarray(k, dtype=F32)
    G, W, d = q.shape
    S = k.shape[0]
    if W > S:
        raise ValueError("window longer than sequence")
    logits = (np.matmul(q, k.T) / F32(math.sqrt(d))).astype(F32)   # [G, W, S]
    pos = np.arange(S)[None, :]
    row_pos = (S - W + np.arange(W))[:, None]
    logits = np.where((pos > row_pos)[None, :, :], F32(-np.inf), logits)
    m = logits.max(axis=2, keepdims=True)
    e = np.exp(logits - m).astype(F32)
    z = e.sum(axis=2, keepdims=True, dtype=F32)
    p = (e / z).astype(F32)
    return p[:, :, : S - W].sum(axis=(0, 1), dtype=F32)


def pool_sum(scores: np.ndarray, kernel: int) -> np.ndarray:
    """Sequence pooling of the window scores (reading R9).

    [RKV] quick read ("how it works", stage 1) and method details, pooling
    paragraph: SnapKV pools along the sequence so that a key token is kept
    together with its neighbours; kernel 63 in all RocketKV experiments.

    out[j] = sum_{i=j-h}^{j+h} scores[i], h = (kernel-1)/2, terms outside
    [0, n) are zero.  Added strictly left to right (i ascending) in float32,
    starting from the first term.  kernel must be odd.
    """
    s = np.asarray(scores, dtype=F32)
    if kernel < 1 or kernel % 2 == 0:
        raise ValueError("pool kernel must be odd and positive")
    n = s.shape[0]
    h = (kernel - 1) // 2
    out = np.zeros(n, dtype=F32)
    for off in range(-h, h + 1):
        lo = max(0, -off)
        hi = min(n, n - off)
        if lo < hi:
            out[lo:hi] = (out[lo:hi] + s[lo + off:hi + off]).astype(F32)
    return out


def pool_max(scores: np.ndarray, kernel: int) -> np.ndarray:
    """The other reading of the sequence pooling (R9): max pooling.

    [RKV] quick read and method details, pooling paragraph: the notes name
    the pooling and its kernel size but not its kind.  out[j] = the largest
    of scores[i] for i in [j-h, j+h] within [0, n), h = (kernel-1)/2.  A
    maximum involves no rounding.  kernel must be odd.
    """
    s = np.asarray(scores, dtype=F32)
    if kernel < 1 or kernel % 2 == 0:
        raise ValueError("pool kernel must be odd and positive")
    n = s.shape[0]
    h = (kernel - 1) // 2
    out = np.empty(n, dtype=F32)
    for j in range(n):
        out[j] = s[max(0, j - h):min(n, j + h + 1)].max()
    return out


def pool(scores: np.ndarray, kernel: int, op: str = "sum") -> np.ndarray:
    """Sequence pooling by reading: "sum" (R9, built by default) or "max"."""
    if op == "sum":
        return pool_sum(scores, kernel)
    if op == "max":
        return pool_max(scores, kernel)
    raise ValueError("pool op must be 'sum' or 'max'")


def snapkv_select(pooled: np.ndarray, seq_len: int, window: int, n_keep: int) -> np.ndarray:
    """Kept token positions of one KV head (readings R7, R11, R12).

    [RKV] method details, SnapKV paragraph (keep the most relevant prompt
    tokens, permanently drop the rest) and quick read (stage 1).  The top
    (n_keep - W) prefix positions by pooled score, ascending, followed by the
    W window positions [S-W, S).
    """
    if not (window <= n_keep <= seq_len):
        raise ValueError("n_keep outside [W, S]")
    sel = topk_lower_index(pooled, n_keep - window)
    return np.concatenate([sel, np.arange(seq_len - window, seq_len)]).astype(np.int64)


def snapkv_evict(q_win: np.ndarray, k: np.ndarray, v: np.ndarray | None,
                 window: int, pool_kernel: int, n_keep: int, pool_op: str = "sum") -> dict:
    """Stage 1 for a whole [B, H_kv] cache.

    q_win: [B, H_q, W, d]; k, v: [B, H_kv, S, d] (v may be None for the
    RocketKV-MT form, which returns indices only).  Query head j uses KV head
    j // G (contiguous groups).  Returns kept [B, H_kv, n_keep] int64, pooled
    [B, H_kv, S-W] float32, and compact k/v [B, H_kv, n_keep, d] (gathered
    rows, [RKV] quick read: permanent eviction into a smaller cache).
    """
    q_win = np.asarray(q_win, dtype=F32)
    k = np.asarray(k, dtype=F32)
    B, Hq, W, d = q_win.shape
    _, Hkv, S, _ = k.shape
    if W != window or Hq % Hkv:
        raise ValueError("shape mismatch")
    G = Hq // Hkv
    kept = np.zeros((B, Hkv, n_keep), np.int64)
    pooled = np.zeros((B, Hkv, S - W), F32)
    for b in range(B):
        for h in range(Hkv):
            sc = window_scores(q_win[b, h * G:(h + 1) * G], k[b, h])
            pooled[b, h] = pool(sc, pool_kernel, pool_op)
            kept[b, h] = snapkv_select(pooled[b, h], S, W, n_keep)
    out = dict(kept=kept, pooled=pooled)
    out["k"] = np.take_along_axis(k, kept[..., None], axis=2)
    if v is not None:
        out["v"] = np.take_along_axis(np.asarray(v, dtype=F32), kept[..., None], axis=2)
    return out


# --------------------------------------------------------------------------
# Stage 2: HSA
# --------------------------------------------------------------------------
def build_aux(kc: np.ndarray, n_tokens: int, block: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-page element-wise key max/min (HSA step 1).

    [RKV] method details, HSA step 1: keys grouped into consecutive pages
    along the sequence; the element-wise max (Kmax) and min (Kmin) of each
    page are kept as auxiliary storage, laid out along the head dimension for
    the step-2 gather.  kc: [N, d] (rows >= n_tokens ignored).  Returns
    (kmax, kmin), each [d, nblk] with nblk = ceil(n_tokens / block); the last
    page covers only its valid tokens.  Exact (no rounding).
    """
    kc = np.asarray(kc)
    nblk = -(-n_tokens // block)
    d = kc.shape[1]
    kmax = np.empty((d, nblk), kc.dtype)
    kmin = np.empty((d, nblk), kc.dtype)
    for b in range(nblk):
        rows = kc[b * block:min((b + 1) * block, n_tokens)]
        kmax[:, b] = rows.max(axis=0)
        kmin[:, b] = rows.min(axis=0)
    return kmax, kmin


def channel_select(q_group: np.ndarray, k1: int) -> tuple[np.ndarray, np.ndarray]:
    """HSA step 2, channel part, for one GQA group.

    [RKV] method details, HSA step 2 and the GQA paragraph of Algorithm 1:
    i1 = argtopk(sum over the group of |q|, k1); the sign comes from the sum
    over the group of q.  q_group: [G, d] float32.  Both group sums are taken
    in float32 with g ascending.  Returns (i1 ascending, q_bar [d]).
    """
    q = np.asarray(q_group, dtype=F32)
    G, d = q.shape
    if not (1 <= k1 <= d):
        raise ValueError("k1 outside [1, d]")
    a = np.zeros(d, F32)
    qbar = np.zeros(d, F32)
    for g in range(G):
        a = (a + np.abs(q[g])).astype(F32)
        qbar = (qbar + q[g]).astype(F32)
    return topk_lower_index(a, k1), qbar


def block_scores(qbar: np.ndarray, i1: np.ndarray, kmax: np.ndarray, kmin: np.ndarray) -> np.ndarray:
    """HSA step 2, approximate page scores.

    [RKV] Algorithm 1: P takes row i of Kmax where the group-summed q is >= 0
    and of Kmin otherwise (reading R14); s1 = score(q[i1], P).  [RKV] HSA
    step 2: the element-wise max(q*Kmax, q*Kmin) over the k1 channels
    approximates the best attention score inside the page; for each channel
    that max is q_bar_i * P_i[b], so s1[b] = sum_{i in i1} q_bar_i * P_i[b]
    (reading R15), accumulated in float32 over i1 in ascending channel order,
    one multiply then one add per term.
    """
    qbar = np.asarray(qbar, F32)
    kmax = np.asarray(kmax, F32)
    kmin = np.asarray(kmin, F32)
    s1 = np.zeros(kmax.shape[1], F32)
    for i in np.sort(i1):
        row = kmax[i] if qbar[i] >= 0 else kmin[i]
        s1 = (s1 + (qbar[i] * row).astype(F32)).astype(F32)
    return s1


def block_select(s1: np.ndarray, k2: int) -> np.ndarray:
    """HSA step 2, page choice: i2 = argtopk(s1, k2) ([RKV] Algorithm 1).

    min(k2, nblk) pages, ties to the lower page, ascending (R11, R16).
    """
    return topk_lower_index(s1, min(k2, s1.shape[0]))


def selected_tokens(sel_blocks: np.ndarray, n_tokens: int, block: int) -> np.ndarray:
    """Token positions covered by the chosen pages (valid tokens only)."""
    toks = (np.asarray(sel_blocks)[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return toks[toks < n_tokens]


def attention(q_group: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray) -> np.ndarray:
    """Exact attention of the G group heads over the given rows (HSA step 3).

    [RKV] method details, HSA step 3 and Algorithm 1 (y = attn(q, K[i2],
    V[i2])): o_g = softmax(q_g K^T / sqrt(d)) V, reading R5.  Float64.
    """
    q = np.asarray(q_group, np.float64)
    kr = np.asarray(k_rows, np.float64)
    vr = np.asarray(v_rows, np.float64)
    d = q.shape[1]
    logits = q @ kr.T / math.sqrt(d)
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p @ vr


def hsa_unit(q_group, kc, vc, kmax, kmin, n_tokens, block, k1, k2, sel_override=None) -> dict:
    """Algorithm 1 of [RKV] for one GQA group over a compact cache.

    q_group [G, d]; kc, vc [N, d] (rows >= n_tokens ignored); kmax/kmin
    [d, nblk].  ``sel_override`` replaces the chosen pages when the caller
    wants the attention over a given page set (used to compare outputs over
    another implementation's selection).  Returns i1, qbar, s1, sel, out
    [G, d] float64.
    """
    i1, qbar = channel_select(q_group, k1)
    s1 = block_scores(qbar, i1, kmax, kmin)
    sel = block_select(s1, k2)
    use = sel if sel_override is None else np.sort(np.asarray(sel_override))
    toks = selected_tokens(use, n_tokens, block)
    out = attention(q_group, np.asarray(kc)[toks], np.asarray(vc)[toks])
    return dict(i1=i1, qbar=qbar, s1=s1, sel=sel, out=out)


def hsa_decode(q: np.ndarray, kc: np.ndarray, vc: np.ndarray, n_tokens: int,
               block: int, k1: int, k2: int) -> dict:
    """HSA decode for a whole [B, H_kv] compact cache (aux built here).

    q: [B, H_q, d]; kc, vc: [B, H_kv, N, d].  Returns stacked i1, s1, sel
    and out [B, H_q, d] float64.
    """
    q = np.asarray(q, F32)
    B, Hq, d = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    res = dict(i1=[], s1=[], sel=[], out=np.zeros((B, Hq, d)))
    for b in range(B):
        for h in range(Hkv):
            kmax, kmin = build_aux(kc[b, h], n_tokens, block)
            u = hsa_unit(q[b, h * G:(h + 1) * G], kc[b, h], vc[b, h], kmax, kmin,
                         n_tokens, block, k1, k2)
            res["i1"].append(u["i1"])
            res["s1"].append(u["s1"])
            res["sel"].append(u["sel"])
            res["out"][b, h * G:(h + 1) * G] = u["out"]
    return res


def hsa_decode_mt_unit(q_group, k_full, v_full, cand, block, k1, k2, sel_override=None) -> dict:
    """RocketKV-MT decode for one group (reading R17).

    [RKV] method details, RocketKV-MT: all M tokens stay in memory, but stage
    2 chooses only among the N tokens stage 1 kept (plus newly generated
    ones).  Pages are formed over the ascending candidate list, so this is
    HSA over the candidate rows K[cand], V[cand].
    """
    cand = np.asarray(cand)
    kc = np.asarray(k_full)[cand]
    vc = np.asarray(v_full)[cand]
    kmax, kmin = build_aux(kc, len(cand), block)
    return hsa_unit(q_group, kc, vc, kmax, kmin, len(cand), block, k1, k2, sel_override)


# --------------------------------------------------------------------------
# Dynamic-selection baselines compared with HSA: Exact-TopK, Quest, SparQ
# --------------------------------------------------------------------------
# [RKV] background (Exact-TopK as the ideal top-k attention, Figs. 1-2),
# method details ("limits of existing dynamic selection": Quest keeps per-page
# element-wise min/max along the sequence, SparQ uses head-dimension
# sparsity), appendix A.3 (for Quest and SparQ the token budget is shared
# evenly between the approximate scoring that finds the top-k indices and the
# sparse attention; Quest is made GQA-aware by choosing per attention group
# on the accumulated scores) and B.1.1 (standalone HSA against Quest and
# SparQ, Fig. 8).  Table 1: Quest stores 1 + 1/c, SparQ 2.
#
# Readings (R23-R26):
#   R23 the "attention score" a group accumulates for token n is the sum over
#       its heads of the logits, sum_g q_g . k_n = q_bar . k_n, the quantity
#       HSA step 2 approximates; Exact-TopK takes the top-k tokens by it (for
#       one head this is the top-k by attention weight, softmax being
#       monotone).  Float32, q_bar summed over g ascending, then channels in
#       ascending order, one rounded multiply and one rounded add per term.
#   R24 Quest: pages of `page` tokens with element-wise Kmax/Kmin; the page
#       score is the per-channel bound max(q_bar_i Kmax_i, q_bar_i Kmin_i)
#       summed over all d channels (the bound of the accumulated score
#       q_bar . k of every token in the page); it reads one of the two values
#       per channel (the sign of q_bar picks it), d values per page.
#   R25 SparQ: the r channels of largest sum_g |q_g| (ties to the lower
#       channel), token score q_bar[i1] . k[i1] over those channels only, the
#       top tokens by it; attention is then exact over the chosen tokens (the
#       pages do not describe SparQ's value-mean correction; every method is
#       compared by the tokens it attends).
#   R26 budgets at total compression c, t = S / c KV pairs, estimation and
#       attention t/2 each: Quest page = ceil(c) (d of 2d values per page of
#       c tokens), SparQ r = d / c channels (rounded, in [1, d]), standalone
#       HSA page = ceil(sqrt(c)) and k1 = d * page / c (the split inside HSA
#       with all of c in stage 2); each attends ceil((t/2) / page) pages.
#       Exact-TopK spends nothing on estimation in this accounting (it is the
#       ideal) and attends ceil(t) tokens.
SELECT_METHODS = ("hsa", "quest", "sparq", "exact")


def select_plan(method: str, c: float, seq_len: int, head_dim: int) -> dict:
    """Page size, channels per page and attended pages of a selection method
    at total compression c (readings R24-R26), plus its estimation traffic
    in KV pairs (channels values per page over ceil(S/page) pages, 2d values
    per pair)."""
    if not (c >= 1.0) or seq_len < 1 or head_dim < 1:
        raise ValueError("bad plan arguments")
    t = seq_len / c
    d = head_dim
    if method == "hsa":
        page = math.ceil(math.sqrt(c))
        channels = min(d, max(1, math.floor(d * page / c + 0.5)))
        k2 = max(1, math.ceil(t / 2 / page))
    elif method == "quest":
        page = math.ceil(c)
        channels = d
        k2 = max(1, math.ceil(t / 2 / page))
    elif method == "sparq":
        page = 1
        channels = min(d, max(1, math.floor(d / c + 0.5)))
        k2 = max(1, math.ceil(t / 2))
    elif method == "exact":
        page = 1
        channels = d
        k2 = max(1, math.ceil(t))
    else:
        raise ValueError(f"unknown method {method}")
    n_pages = -(-seq_len // page)
    return dict(page=page, channels=channels, k2=k2, attn_tokens=min(seq_len, k2 * page), budget_t=t,
                est_pairs=channels * n_pages / (2.0 * d))


def _group_sums(q_group):
    """(sum_g |q_g|, q_bar = sum_g q_g) in float32, g ascending."""
    q = np.asarray(q_group, dtype=F32)
    a = np.zeros(q.shape[1], F32)
    qbar = np.zeros(q.shape[1], F32)
    for g in range(q.shape[0]):
        a = (a + np.abs(q[g])).astype(F32)
        qbar = (qbar + q[g]).astype(F32)
    return a, qbar


def exact_topk_scores(q_group: np.ndarray, k_rows: np.ndarray) -> np.ndarray:
    """Accumulated group logit of every token (reading R23): score[n] =
    q_bar . k_n, float32, channels ascending, one rounded product and one
    rounded add per term.  q_group [G, d], k_rows [N, d]."""
    _, qbar = _group_sums(q_group)
    k = np.asarray(k_rows, dtype=F32)
    s = np.zeros(k.shape[0], F32)
    for i in range(k.shape[1]):
        s = (s + (qbar[i] * k[:, i]).astype(F32)).astype(F32)
    return s


def quest_page_scores(q_group: np.ndarray, kmax: np.ndarray, kmin: np.ndarray) -> np.ndarray:
    """Quest's page bound of the accumulated score (reading R24): s[b] = sum
    over channels i ascending of max(q_bar_i Kmax_i[b], q_bar_i Kmin_i[b]),
    float32, each term the larger of two rounded products, one rounded add.
    kmax, kmin [d, nblk]."""
    _, qbar = _group_sums(q_group)
    kmax = np.asarray(kmax, F32)
    kmin = np.asarray(kmin, F32)
    s = np.zeros(kmax.shape[1], F32)
    for i in range(kmax.shape[0]):
        hi = (qbar[i] * kmax[i]).astype(F32)
        lo = (qbar[i] * kmin[i]).astype(F32)
        s = (s + np.maximum(hi, lo)).astype(F32)
    return s


def sparq_channels(q_group: np.ndarray, r: int) -> np.ndarray:
    """SparQ's r channels of largest sum_g |q_g| (ties to the lower channel),
    ascending (reading R25)."""
    a, _ = _group_sums(q_group)
    return topk_lower_index(a, r)


def sparq_scores(q_group: np.ndarray, k_rows: np.ndarray, r: int) -> np.ndarray:
    """SparQ's approximate accumulated logit (reading R25): score[n] = sum over
    the r chosen channels, ascending, of q_bar_i k_n,i (float32, rounded
    product then rounded add)."""
    _, qbar = _group_sums(q_group)
    k = np.asarray(k_rows, dtype=F32)
    s = np.zeros(k.shape[0], F32)
    for i in sparq_channels(q_group, r):
        s = (s + (qbar[i] * k[:, i]).astype(F32)).astype(F32)
    return s


def select_decode_unit(method: str, q_group, kc, vc, n_tokens: int, page: int, channels: int,
                       k2: int, sel_override=None) -> dict:
    """One decode step of a selection method for one GQA group over the first
    n_tokens rows of kc / vc: page scores, the min(k2, pages) best pages (ties
    to the lower page, ascending) and exact attention over their tokens.
    hsa: Algorithm 1 (channel_select, build_aux, block_scores); quest: R24
    over build_aux pages; sparq (page 1): R25; exact (page 1): R23."""
    kc = np.asarray(kc)[:n_tokens]
    vc = np.asarray(vc)[:n_tokens]
    if method == "hsa":
        kmax, kmin = build_aux(kc, n_tokens, page)
        i1, qbar = channel_select(q_group, channels)
        s = block_scores(qbar, i1, kmax, kmin)
    elif method == "quest":
        if channels != kc.shape[1]:
            raise ValueError("Quest reads every channel")
        kmax, kmin = build_aux(kc, n_tokens, page)
        s = quest_page_scores(q_group, kmax, kmin)
    elif method == "sparq":
        if page != 1:
            raise ValueError("SparQ selects tokens (page 1)")
        s = sparq_scores(q_group, kc, channels)
    elif method == "exact":
        if page != 1 or channels != kc.shape[1]:
            raise ValueError("Exact-TopK selects tokens over every channel")
        s = exact_topk_scores(q_group, kc)
    else:
        raise ValueError(f"unknown method {method}")
    sel = block_select(s, k2)
    use = sel if sel_override is None else np.sort(np.asarray(sel_override))
    toks = selected_tokens(use, n_tokens, page)
    out = attention(q_group, kc[toks], vc[toks])
    return dict(scores=s, sel=sel, tokens=toks, out=out)


# --------------------------------------------------------------------------
# Ada-KV adaptive per-head budgets in stage 1
# --------------------------------------------------------------------------
# [RKV] method details ("the second stage and the framework's generality":
# SnapKV or Ada-KV can serve as stage 1; GQA group-level selection follows
# Ada-KV).  The notes name Ada-KV's adaptive budget allocation but not its
# rule.  Reading R27: the budget of a sequence in a layer is shared by its
# KV heads (groups) instead of being fixed per head: the Hkv * (n_keep - W)
# prefix slots go to the largest pooled group scores over all of the
# sequence's heads taken together (flattened [head, position], ties to the
# lower head, then the lower position), so a head whose group attends to few
# tokens keeps few and a head whose attention is spread keeps more; each head
# also keeps its W window tokens.  The scores are comparable across heads:
# every window row of every group is one softmax (total mass G * W per head).
# The rule itself is parity-unpinned against the pages; the pins fix its
# internal consistency (equal heads reduce to per-head SnapKV, the budget is
# conserved, brute force on tiny inputs).
def adakv_select(pooled_heads: np.ndarray, seq_len: int, window: int, n_keep: int) -> list:
    """Kept positions of each KV head of one sequence under the shared budget
    (reading R27).  pooled_heads [Hkv, S-W] (pooled group scores).  Returns a
    list of Hkv int64 arrays: the head's chosen prefix positions ascending,
    then the W window positions [S-W, S)."""
    pooled_heads = np.asarray(pooled_heads)
    Hkv, P = pooled_heads.shape
    if P != seq_len - window or not (window <= n_keep <= seq_len):
        raise ValueError("bad sizes")
    flat = pooled_heads.reshape(-1)           # index h * P + j: (head, position) order
    chosen = topk_lower_index(flat, Hkv * (n_keep - window))
    out = []
    for h in range(Hkv):
        mine = chosen[(chosen >= h * P) & (chosen < (h + 1) * P)] - h * P
        out.append(np.concatenate([np.sort(mine), np.arange(seq_len - window, seq_len)]).astype(np.int64))
    return out


def adakv_evict(q_win: np.ndarray, k: np.ndarray, window: int, pool_kernel: int, n_keep: int,
                pool_op: str = "sum") -> dict:
    """Stage 1 with Ada-KV budgets for a whole [B, H_kv] cache: window scores
    and pooling per head as SnapKV (R5-R10), then adakv_select per sequence.
    Returns kept (list per batch of per-head arrays), counts [B, H_kv] and
    pooled [B, H_kv, S-W]."""
    q_win = np.asarray(q_win, dtype=F32)
    k = np.asarray(k, dtype=F32)
    B, Hq, W, d = q_win.shape
    _, Hkv, S, _ = k.shape
    G = Hq // Hkv
    pooled = np.zeros((B, Hkv, S - W), F32)
    kept, counts = [], np.zeros((B, Hkv), np.int64)
    for b in range(B):
        for h in range(Hkv):
            pooled[b, h] = pool(window_scores(q_win[b, h * G:(h + 1) * G], k[b, h]), pool_kernel, pool_op)
        kb = adakv_select(pooled[b], S, W, n_keep)
        kept.append(kb)
        counts[b] = [len(x) for x in kb]
    return dict(kept=kept, counts=counts, pooled=pooled)

// rk_decode.hip -- HSA steps 2 and 3 (decode), plain and RocketKV-MT.
//
// Source: papercache notes "RocketKV: Accelerating Long-Context LLM Inference
// via Two-Stage KV Cache Compression", method details: HSA step 2 (top-k1
// channels of |q|, sign-selected Kmax/Kmin, approximate page scores, top-k2
// pages), HSA step 3 (exact attention over the chosen pages), the GQA
// paragraph with Algorithm 1 (group sums of |q| and q so a whole group makes
// one choice) and RocketKV-MT (pages over the stage-1 candidates of a full
// cache).
//
// Small batches, three launches per call:
//   hsa_score   one workgroup per (page range, unit): channel sums and top-k1;
//               the range's k1 sign-selected aux rows are staged into LDS with
//               16-byte loads (one memory round trip) and its pages scored
//   hsa_attn    top-k2 of the unit's page scores (radix select, in every
//               workgroup), then split-K over the selected pages: a wave streams
//               whole pages with 16-byte K/V loads, online softmax in the exp2
//               domain, one partial (m, l, o[d]) per head per workgroup
//   hsa_combine one wave per (unit, head) merges the partials
// Large batches (kFusedMinUnits units or more), one launch:
//   hsa_fused   one 1024-thread workgroup per unit runs all of the above and
//               writes the normalised output
// HBM-bound: bytes per unit = q + k1*nblk aux elements + 2*d*|T| K/V elements.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "rk_device.hpp"
#include "rk_internal.hpp"

namespace rk {
namespace {

// ---- step 2 building blocks --------------------------------------------------
// Staging: thread (channel j, vector slot) of NT fetches 16-byte runs of the
// sign-selected aux row of i1[j] (EPV consecutive pages; xu/nu point at the
// first page of the range, a multiple of 8, and nblk_cap is a multiple of 8,
// so runs stay aligned and inside the row) and scatters them transposed into
// LDS as stage[page][channel] with row pitch k1p (16-channel blocks plus one
// vector of padding).  All of a thread's loads are in flight together.
template <typename T>
__device__ __forceinline__ int staged_pitch(int k1) {
  return (k1 + 15) / 16 * 16 + int(16 / sizeof(T));
}
template <typename T, int NT>
__device__ __forceinline__ void stage_rows(const T* xu, const T* nu, int64_t nblk_cap, int np,
                                           int k1, const int* i1_off, T* stage) {
  constexpr int EPV = 16 / sizeof(T);
  const int t = threadIdx.x;
  const int k1p = staged_pitch<T>(k1);
  const int groups = NT / k1;  // vector slots per channel (k1 <= 128 <= NT / 2)
  const int nv = (np + EPV - 1) / EPV;
  if (t >= groups * k1) return;
  const int j = t % k1;
  const int off = i1_off[j];
  const T* row = off >= 0 ? xu + size_t(off) * nblk_cap : nu + size_t(-1 - off) * nblk_cap;
  constexpr int NB = 4;
  for (int v0 = t / k1; v0 < nv; v0 += groups * NB) {
    Vec16<T> buf[NB];
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      const int vi = v0 + x * groups;
      if (vi < nv) buf[x] = load16(row + vi * EPV);
    }
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      const int vi = v0 + x * groups;
      if (vi < nv) {
        const T* src = reinterpret_cast<const T*>(&buf[x].raw);
#pragma unroll
        for (int e = 0; e < EPV; ++e) stage[size_t(vi * EPV + e) * k1p + j] = src[e];
      }
    }
  }
}

// Scoring of staged pages: s1[b] = sum over i1 (ascending) of q_bar_i * P_i[b],
// thread t taking pages b = t, t + NT, ...  Channels go in blocks of 16: the
// block's q_bar values come from LDS as float4 broadcasts and the page's 16
// staged values as 16-byte reads, then the ordered terms, each one rounded
// multiply and one rounded add (no fused multiply-add).  Writes order keys to
// keys[b] and, when s1 is given, the scores to s1[b].
template <typename T, int NT>
__device__ __forceinline__ void score_staged(const T* stage, int np, int k1, const float* i1_q,
                                             uint32_t* keys, float* s1) {
#pragma clang fp contract(off)
  constexpr int EPV = 16 / sizeof(T);
  const int k1p = staged_pitch<T>(k1);
  for (int b = threadIdx.x; b < np; b += NT) {
    const T* sp = stage + size_t(b) * k1p;
    float acc = 0.f;
    // whole 16-channel blocks unmasked, then the masked tail block
    auto block16 = [&](int j0, int lim) {
      float qv[16], sv[16];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float4 q4 = *reinterpret_cast<const float4*>(i1_q + j0 + 4 * x);
        qv[4 * x] = q4.x;
        qv[4 * x + 1] = q4.y;
        qv[4 * x + 2] = q4.z;
        qv[4 * x + 3] = q4.w;
      }
#pragma unroll
      for (int x = 0; x < 16 / EPV; ++x) {
        const Vec16<T> vv = load16(sp + j0 + x * EPV);
#pragma unroll
        for (int e = 0; e < EPV; ++e) sv[x * EPV + e] = vv.get(e);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (e < lim) acc = acc + qv[e] * sv[e];
    };
    const int kfull = k1 & ~15;
#pragma unroll 2
    for (int j0 = 0; j0 < kfull; j0 += 16) block16(j0, 16);
    if (kfull < k1) block16(kfull, k1 - kfull);
    keys[b] = order_key(acc);
    if (s1) s1[b] = acc;
  }
}

// Channel choice of HSA step 2 by one wave (wave 0 of the caller): group sums
// of |q| and q per channel (g ascending, float32), top-k1 channels with ties
// toward the lower channel, in ascending channel order.  Writes i1_q[rank] =
// q_bar of the channel, i1_off[rank] = ch if q_bar >= 0 (Kmax row) else
// -1 - ch (Kmin row), and chan_out[rank] = ch when chan_out is given.
template <typename T, int D, int G>
__device__ __forceinline__ void wave_choose_channels(const float (&qx)[D / kWave][G], int k1,
                                                     float* i1_q, int* i1_off, int32_t* chan_out,
                                                     uint32_t* hist) {
  constexpr int R = D / kWave;
  float qb[R];
  uint32_t kr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float a = 0.f, s = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      a = __fadd_rn(a, fabsf(qx[r][g]));
      s = __fadd_rn(s, qx[r][g]);
    }
    kr[r] = order_key(a);
    qb[r] = s;
  }
  wave_topk<R>(kr, D, k1, [&](int rank, int ch) {
    float qv = qb[0];  // the emitting lane holds the channel's q_bar
#pragma unroll
    for (int r = 1; r < R; ++r)
      if ((ch >> 6) == r) qv = qb[r];
    i1_q[rank] = qv;
    i1_off[rank] = qv >= 0.f ? ch : -1 - ch;
    if (chan_out) chan_out[rank] = ch;
  }, hist);
}

// Step 2a: one workgroup per (page range, unit).  Every workgroup of a unit
// makes the same channel choice (group sums of |q| in g order, top-k1 with
// ties toward the lower channel), then stages its pages' sign-selected aux
// rows into LDS with all 16-byte loads in flight and scores them.  Spreading
// a unit's pages over many workgroups keeps the aux fetch of a small batch
// from queueing behind one CU's outstanding-load limit.  ALL (small launches,
// where latency rules and bytes are cheap): the range's Kmax and Kmin rows of
// every channel are fetched together with q, so the channel choice no longer
// sits between two memory round trips.
template <typename T, int D, int G, bool ALL>
__global__ __launch_bounds__(256) void hsa_score_kernel(
    const T* __restrict__ q, const T* __restrict__ kmax, const T* __restrict__ kmin,
    int64_t nblk_cap, int nblk, int k1, int ppw, int units, uint32_t* __restrict__ keys,
    int keys_pitch, int32_t* __restrict__ chan_opt, float* __restrict__ s1_opt,
    const int32_t* __restrict__ lens, int n_max, int block) {
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  extern __shared__ __align__(16) unsigned char dyn_lds[];
  T* stage = reinterpret_cast<T*>(dyn_lds);  // [ppw][k1p]
  __shared__ __align__(16) float i1_q[D + 16];
  __shared__ __align__(16) int i1_off[D + 16];  // sign-selected row of i1[j]: ch (Kmax) or -1-ch (Kmin)
  __shared__ __align__(16) uint32_t hist[1024];

  constexpr int R = D / kWave;  // channels per lane of wave 0
  constexpr int NBA = 8;        // 16-byte vectors per thread in ALL mode (one round)
  // work items (unit, page range), unit-major, XCD-local: the ranges of a unit
  // read neighbouring 16-byte runs of the same aux rows
  const int n_ranges = (nblk + ppw - 1) / ppw;
  const int item = xcd_local_item(n_ranges * units);
  if (item >= n_ranges * units) return;
  const int u = item / n_ranges;
  const int p0 = (item % n_ranges) * ppw;
  // per-unit token counts (ragged units): ranges past the unit's pages idle
  const int nblk_u = lens ? (max(1, min(lens[u], n_max)) + block - 1) / block : nblk;
  if (p0 >= nblk_u) return;
  const int np = min(ppw, nblk_u - p0);
  const int t = threadIdx.x;
  const int wave = t / kWave, lane = lane_id();
  const T* xu = kmax + size_t(u) * D * size_t(nblk_cap) + p0;
  const T* nu = kmin + size_t(u) * D * size_t(nblk_cap) + p0;
  const int nv = (np + EPV - 1) / EPV;  // 16-byte vectors per row slice
  float qx[R][G];
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int g = 0; g < G; ++g) qx[r][g] = to_f32(q[(size_t(u) * G + g) * D + r * kWave + lane]);
  }
  // ALL: rows r < D are Kmax channel r, rows r >= D Kmin channel r - D;
  // stage[r][page] with pitch ppw (2*D*nv <= 256*NBA, set by the launcher)
  Vec16<T> buf[NBA];
  if (ALL) {
#pragma unroll
    for (int x = 0; x < NBA; ++x) {
      const int id = x * 256 + t;
      if (id < 2 * D * nv) {
        const int r = id / nv, vi = id % nv;
        buf[x] = load16((r < D ? xu + size_t(r) * nblk_cap : nu + size_t(r - D) * nblk_cap) + vi * EPV);
      }
    }
  }
  if (wave == 0)
    wave_choose_channels<T, D, G>(qx, k1, i1_q, i1_off,
                                  chan_opt && p0 == 0 ? chan_opt + size_t(u) * k1 : nullptr,
                                  hist);
  if (ALL) {
#pragma unroll
    for (int x = 0; x < NBA; ++x) {
      const int id = x * 256 + t;
      if (id < 2 * D * nv) {
        const int r = id / nv, vi = id % nv;
        *reinterpret_cast<decltype(buf[x].raw)*>(stage + size_t(r) * ppw + vi * EPV) = buf[x].raw;
      }
    }
  }
  __syncthreads();
  uint32_t* ku = keys + size_t(u) * keys_pitch + p0;
  if (ALL) {
    // s1[b] = sum over i1 (ascending) of q_bar_i * P_i[b], P_i read from the
    // Kmax or Kmin row the sign picked.  All threads first form the rounded
    // products q_bar_i * P_i[b] (np * k1 of them) into LDS; then the thread
    // of page b adds its row of products in channel order (one rounded
    // multiply and one rounded add per term, as in a sequential sum).
#pragma clang fp contract(off)
    float* prod = reinterpret_cast<float*>(stage + size_t(2) * D * ppw);  // [np][pp]
    const int pp = (k1 + 15) / 16 * 16 + 4;  // whole 16-channel blocks, padded row
    for (int idx = t; idx < np * k1; idx += 256) {
      const int b = idx / k1, j = idx - b * k1;
      const int o = i1_off[j];
      const int r = o >= 0 ? o : D + (-1 - o);
      prod[b * pp + j] = i1_q[j] * to_f32(stage[size_t(r) * ppw + b]);
    }
    __syncthreads();
    for (int b = t; b < np; b += 256) {
      const float* pb = prod + b * pp;
      float acc = 0.f;
      // whole 16-channel blocks unmasked, then the masked tail block
      const int kfull = k1 & ~15;
      auto block16 = [&](int j0, int lim) {
        float pv[16];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float4 f = *reinterpret_cast<const float4*>(pb + j0 + 4 * x);
          pv[4 * x] = f.x;
          pv[4 * x + 1] = f.y;
          pv[4 * x + 2] = f.z;
          pv[4 * x + 3] = f.w;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (e < lim) acc = acc + pv[e];
      };
#pragma unroll 4
      for (int j0 = 0; j0 < kfull; j0 += 16) block16(j0, 16);
      if (kfull < k1) block16(kfull, k1 - kfull);
      ku[b] = order_key(acc);
      if (s1_opt) s1_opt[size_t(u) * nblk + p0 + b] = acc;
    }
    return;
  }

  stage_rows<T, 256>(xu, nu, nblk_cap, np, k1, i1_off, stage);
  __syncthreads();
  score_staged<T, 256>(stage, np, k1, i1_q, ku, s1_opt ? s1_opt + size_t(u) * nblk + p0 : nullptr);
}

// Exact-TopK scoring: the group's accumulated logit of every token, over the
// key rows themselves (pages of one token, all channels): s[n] = sum over
// channels i ascending of q_bar_i * k_n,i, one rounded multiply and one
// rounded add per term (float32), q_bar = sum_g q_g with g ascending.  One
// thread per token reads its row with 16-byte loads; q_bar is formed once per
// workgroup in LDS.  Writes order keys (and, when asked, the scores).
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void exact_score_kernel(const T* __restrict__ q,
                                                          const T* __restrict__ k, int64_t kv_cap,
                                                          int n_tokens, uint32_t* __restrict__ keys,
                                                          int keys_pitch, float* __restrict__ s_opt) {
#pragma clang fp contract(off)
  constexpr int EPL = Vec16<T>::N;
  __shared__ float qb[D];
  const int u = blockIdx.y;
  for (int ch = threadIdx.x; ch < D; ch += 256) {
    float a = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) a = __fadd_rn(a, to_f32(q[(size_t(u) * G + g) * D + ch]));
    qb[ch] = a;
  }
  __syncthreads();
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= n_tokens) return;
  const T* row = k + (size_t(u) * size_t(kv_cap) + size_t(n)) * D;
  Vec16<T> r[D / EPL];
#pragma unroll
  for (int c = 0; c < D / EPL; ++c) r[c] = load16(row + c * EPL);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / EPL; ++c)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = acc + qb[c * EPL + e] * r[c].get(e);
  keys[size_t(u) * keys_pitch + n] = order_key(acc);
  if (s_opt) s_opt[size_t(u) * n_tokens + n] = acc;
}

// out[i] = i % period (the channel list 0..D-1 of every unit).
__global__ __launch_bounds__(256) void fill_iota_kernel(int32_t* __restrict__ out, int period, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = i % period;
}

// Page choice in a launch of its own (more pages than the attention
// workgroups hold in LDS, or token-level scoring): one workgroup per unit
// takes the top-nsel of the unit's page keys (ties to the lower page) and
// writes the chosen pages, ascending, to sel (and sel_opt).  staged: the keys
// fit in LDS (with the key range taken while staging, and spare LDS for the
// radix candidates); otherwise every pass reads them from memory (L2).
__global__ __launch_bounds__(1024) void page_select_kernel(const uint32_t* __restrict__ keys,
                                                           int keys_pitch, int nblk, int nsel,
                                                           int staged, int cand_cap,
                                                           int32_t* __restrict__ sel,
                                                           int32_t* __restrict__ sel_opt) {
  extern __shared__ uint32_t pk[];
  __shared__ TopkSmem<1024, 2048, 1> sm;
  const int u = blockIdx.x;
  const uint32_t* kg = keys + size_t(u) * keys_pitch;
  int32_t* su = sel + size_t(u) * nsel;
  // without sel_opt the second store repeats the first (a branch-free emit
  // keeps the one-wave emission loop unrollable)
  int32_t* so = sel_opt ? sel_opt + size_t(u) * nsel : su;
  auto emit = [=](int r, int i) {
    su[r] = i;
    so[r] = i;
  };
  if (staged) {
    uint32_t lo = 0xffffffffu, hi = 0u;
    for (int i = threadIdx.x; i < nblk; i += 1024) {
      const uint32_t kk = kg[i];
      pk[i] = kk;
      lo = min(lo, kk);
      hi = max(hi, kk);
    }
    __syncthreads();
    wg_topk<1024, 2048>([&](int i) { return pk[i]; }, nblk, nsel, emit, sm, true, lo, hi, pk + nblk,
                        cand_cap);
  } else {
    wg_topk<1024, 2048>([&](int i) { return kg[i]; }, nblk, nsel, emit, sm);
  }
}

// ---- step 3 building blocks -------------------------------------------------
// A wave streams whole pages.  Lanes split a row into LPR 16-byte chunks, so
// SLOTS tokens are in flight per wave and each slot takes TPS tokens per chunk.
// Per lane: a reference m (at most kLazyRescale below the running maximum),
// the sum l and o over its channel chunk of exp2(score - m) weights, per
// head of the group, in the exp2 domain.
constexpr float kLazyRescale = 8.0f;
template <typename T, int D, int G, int TPS_ = (G >= 4 ? 2 : 4)>
struct AttnShape {
  static constexpr int EPL = Vec16<T>::N;
  static constexpr int LPR = D / EPL;
  static constexpr int SLOTS = kWave / LPR;
  // tokens per slot per step; the split-K kernel takes fewer for wide groups
  // (registers at four waves per SIMD)
  static constexpr int TPS = TPS_;
  static constexpr int CHUNK = SLOTS * TPS;
  static_assert(kWave % LPR == 0, "row chunks must tile a wave");
};

// One unit's view of a paged pool (PagedArgs, resolved for the unit).
struct UnitPages {
  const int32_t* table;
  int64_t n_phys;
  int shift, hkv, h;
  // when set: the first pool row of each of the sequence's pages for this
  // unit's head, already clamped (the fused kernel keeps them in LDS)
  const int32_t* base = nullptr;
};

// PAGED: ku / vu are the pool base (plus the lane's channel offset) and token
// n of the unit is pool row paged_row(n); otherwise the unit's base, with
// row n (or, MT, its candidate row cu[n]).
template <typename T, int D, int G, bool MT, int TPS_ = AttnShape<T, D, G>::TPS, bool PAGED = false>
__device__ __forceinline__ void attend_pages(
    const float (&qf)[G][Vec16<T>::N], const T* ku, const T* vu, const int32_t* cu,
    int64_t kv_cap, const int* pages, int e_begin, int e_end, int e_step, int block,
    int n_tokens, float scale_log2, float (&m)[G], float (&l)[G],
    float (&o)[G][Vec16<T>::N], UnitPages up = {}) {
  static_assert(!(MT && PAGED), "candidate lists over a paged pool are not built");
  using S = AttnShape<T, D, G, TPS_>;
  constexpr int EPL = S::EPL, LPR = S::LPR, SLOTS = S::SLOTS, TPS = S::TPS, CHUNK = S::CHUNK;
  const int slot = lane_id() / LPR;
  // bf16: q's values (bf16 to begin with, so exact) as packed pairs
  uint32_t qp[G][4];
  if constexpr (std::is_same_v<T, bf16_t>) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
        qp[g][e2] = (__float_as_uint(qf[g][2 * e2]) >> 16) | (__float_as_uint(qf[g][2 * e2 + 1]) & 0xffff0000u);
  }
  // One step: TPS tokens per slot (rows[i], valid when ok[i]): K and V rows
  // with 16-byte loads, scores, one online-softmax rescale, V accumulation.
  auto step = [&](const int (&rows)[TPS], const bool (&ok)[TPS]) {
    Vec16<T> kr[TPS], vr[TPS];
    // every load unconditional (a masked token reads row 0, which exists)
    // and non-temporal: read once per decode step (6-9 % faster at batch
    // 8-32 than cached loads); masked tokens' values are zeroed after
#pragma unroll
    for (int i = 0; i < TPS; ++i) {
      kr[i] = load16_nt(ku + size_t(rows[i]) * D);
      vr[i] = load16_nt(vu + size_t(rows[i]) * D);
    }
#pragma unroll
    for (int i = 0; i < TPS; ++i)
      if (!ok[i]) {
        kr[i].raw = {};
        vr[i].raw = {};
      }
    float x[G][TPS];
    if constexpr (std::is_same_v<T, bf16_t>) {
      // bf16: the key's packed pairs straight into two-term dot products
      // with q's pairs (no unpacking of the key)
#pragma unroll
      for (int i = 0; i < TPS; ++i) {
        const uint32_t kw[4] = {kr[i].raw.x, kr[i].raw.y, kr[i].raw.z, kr[i].raw.w};
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float s = 0.f;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) s = dot2_bf16(qp[g][e2], kw[e2], s);
          x[g][i] = group_sum<LPR>(s) * scale_log2;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < TPS; ++i) {
        float kf[EPL];
        unpack16(kr[i], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float s = 0.f;
#pragma unroll
          for (int ee = 0; ee < EPL; ++ee) s += qf[g][ee] * kf[ee];
          x[g][i] = group_sum<LPR>(s) * scale_log2;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float cm = kNegBig;
#pragma unroll
      for (int i = 0; i < TPS; ++i)
        if (ok[i]) cm = fmaxf(cm, x[g][i]);
      // the reference m moves (and l, o are rescaled) only when a score
      // passes it by more than kLazyRescale, which after the first step is
      // rare; the weights exp2(x - m) then stay below 2^kLazyRescale
      const bool up = cm > m[g] + kLazyRescale;
      if (ballot(up)) {
        const float mn = up ? cm : m[g];
        const float corr = fast_exp2(m[g] - mn);
        l[g] = l[g] * corr;
#pragma unroll
        for (int ee = 0; ee < EPL; ++ee) o[g][ee] = o[g][ee] * corr;
        m[g] = mn;
      }
      float p[TPS];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < TPS; ++i) {
        p[i] = ok[i] ? fast_exp2(x[g][i] - m[g]) : 0.f;
        ps += p[i];
      }
      l[g] = l[g] + ps;
#pragma unroll
      for (int ee = 0; ee < EPL; ++ee) {
        float acc = o[g][ee];
#pragma unroll
        for (int i = 0; i < TPS; ++i) acc += p[i] * vr[i].get(ee);
        o[g][ee] = acc;
      }
    }
  };
  // The wave's pages (e_begin, e_begin + e_step, ... < e_end) are taken as one
  // token sequence, tau = (page rank) * block + offset, so pages shorter than
  // a step still fill every slot; tokens past n_tokens (a ragged last page)
  // are skipped.
  const int npw = e_end > e_begin ? (e_end - e_begin + e_step - 1) / e_step : 0;
  const int ntok = npw * block;
  // token tau of the sequence is offset off of the wave's page pr; both move
  // by a fixed amount per step (no division inside the loop)
  int pr[TPS], off[TPS];
#pragma unroll
  for (int i = 0; i < TPS; ++i) {
    const int tau = slot + SLOTS * i;
    pr[i] = tau / block;
    off[i] = tau - pr[i] * block;
  }
  const int dpr = CHUNK / block, doff = CHUNK - dpr * block;
  for (int tc = 0; tc < ntok; tc += CHUNK) {
    int rows[TPS], tok[TPS];
    bool ok[TPS];
    // every token's page entry, then every token's row lookup (MT candidate
    // index, paged table entry), with no branch between them, so the reads
    // of a step are in flight together; masked tokens read token 0's entry
#pragma unroll
    for (int i = 0; i < TPS; ++i) {
      const int prc = pr[i] < npw ? pr[i] : npw - 1;  // past the wave's pages: its last one
      const int t0 = pages[e_begin + prc * e_step] * block + off[i];
      ok[i] = pr[i] < npw && t0 < n_tokens;
      tok[i] = ok[i] ? t0 : 0;
      pr[i] += dpr;
      off[i] += doff;
      if (off[i] >= block) {
        off[i] -= block;
        ++pr[i];
      }
    }
#pragma unroll
    for (int i = 0; i < TPS; ++i) {
      int r;
      if constexpr (PAGED)
        r = up.base ? up.base[tok[i] >> up.shift] + (tok[i] & ((1 << up.shift) - 1))
                    : paged_row(up.table, tok[i], up.n_phys, up.shift, up.hkv, up.h);
      else if constexpr (MT)
        r = clamp_row(cu[tok[i]], kv_cap);
      else
        r = tok[i];
      rows[i] = ok[i] ? r : 0;
    }
    step(rows, ok);
  }
}

// Merge the SLOTS token slots of a wave (lanes sharing a channel chunk), then
// slot 0 stores the wave's (m, l, o) at wm[wave*G + g], wl[..], wo[(wave*G + g)*D + ch].
template <typename T, int D, int G>
__device__ __forceinline__ void wave_state_to_lds(float (&m)[G], float (&l)[G],
                                                  float (&o)[G][Vec16<T>::N],
                                                  int wave, float* wm, float* wl, float* wo) {
  using S = AttnShape<T, D, G>;
  constexpr int EPL = S::EPL, LPR = S::LPR;
  const int lane = lane_id();
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float a = fast_exp2(m[g] - mn), b = fast_exp2(mo - mn);
      l[g] = l[g] * a + lo * b;
#pragma unroll
      for (int ee = 0; ee < EPL; ++ee) {
        const float oo = __shfl_xor(o[g][ee], off);
        o[g][ee] = o[g][ee] * a + oo * b;
      }
      m[g] = mn;
    }
  }
  if (lane < LPR) {
    const int c = lane;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (c == 0) {
        wm[wave * G + g] = m[g];
        wl[wave * G + g] = l[g];
      }
#pragma unroll
      for (int ee = 0; ee < EPL; ++ee) wo[size_t(wave * G + g) * D + c * EPL + ee] = o[g][ee];
    }
  }
}

// Merge NW waves' states (in wave order) for element idx = g*D + ch.
template <int D, int G, int NW>
__device__ __forceinline__ void merge_waves(int idx, const float* wm, const float* wl,
                                            const float* wo, float* mm_out, float* ll_out,
                                            float* oo_out) {
  const int g = idx / D, ch = idx % D;
  float mm = kNegBig;
  for (int w = 0; w < NW; ++w) mm = fmaxf(mm, wm[w * G + g]);
  float ll = 0.f, oo = 0.f;
  for (int w = 0; w < NW; ++w) {
    const float a = fast_exp2(wm[w * G + g] - mm);
    ll += wl[w * G + g] * a;
    oo += wo[size_t(w * G + g) * D + ch] * a;
  }
  *mm_out = mm;
  *ll_out = ll;
  *oo_out = oo;
}

// Step 2b + step 3, split-K form.  Every workgroup of a unit first takes the
// top-k2 of the unit's page scores itself (the same radix select in each, so
// all agree; ties toward the lower page, pages in ascending order) and keeps
// the pages of its own split: this saves a launch and a memory round trip
// between the choice and the K/V fetch.  Then 4 waves stream the pages and the
// workgroup writes one partial (m, l, o[d]) per head.  TPS_: tokens per slot
// per step (more loads in flight per wave, more registers).
//
// PRESEL: the pages were chosen by page_select_kernel (written to presel,
// ascending, nsel per unit); the workgroup copies its split's run of them.
template <typename T, int D, int G, bool MT, int TPS_ = AttnShape<T, D, G>::TPS, bool PRESEL = false,
          bool PAGED = false>
__global__ __launch_bounds__(256) void hsa_attn_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t kv_cap,
    const int32_t* __restrict__ cand, int64_t cand_stride, const uint32_t* __restrict__ keys,
    int keys_pitch, int nblk, int nsel, int pages_per_split, int n_split, int units, int n_tokens,
    int block, float scale_log2, float* __restrict__ partials, int32_t* __restrict__ sel_opt,
    const int32_t* __restrict__ presel, PagedArgs pga, const int32_t* __restrict__ lens) {
  using S = AttnShape<T, D, G>;
  constexpr int EPL = S::EPL, LPR = S::LPR;
  constexpr int NW = 4;
  constexpr int PF = D + 4;  // floats per head partial: m, l, pad, pad, o[D]
  __shared__ float wm[NW * G], wl[NW * G];
  __shared__ __align__(16) float wo[NW * G * D];
  __shared__ TopkSmem<256, 1024, 1> tsm;
  extern __shared__ __align__(16) uint32_t attn_lds[];  // the split's pages, then (many pages) the keys

  // work items (unit, split), unit-major, XCD-local: the splits of a unit read
  // the same page keys
  const int item = xcd_local_item(n_split * units);
  if (item >= n_split * units) return;
  const int u = item / n_split;
  const int split = item % n_split;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int c = lane % LPR;

  float qf[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) unpack16(load16(q + (size_t(u) * G + g) * D + c * EPL), qf[g]);
  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegBig;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = 0.f;
  }

  // ragged units: this unit's tokens, pages and chosen pages
  const int n_u = lens ? max(1, min(lens[u], n_tokens)) : n_tokens;
  const int nblk_u = lens ? (n_u + block - 1) / block : nblk;
  const int nsel_u = min(nsel, nblk_u);
  int* pages = reinterpret_cast<int*>(attn_lds);  // [pages_per_split]
  const int e0 = split * pages_per_split;
  const int np = max(0, min(e0 + pages_per_split, nsel_u) - e0);
  int32_t* so = sel_opt && split == 0 ? sel_opt + size_t(u) * nsel : nullptr;
  const uint32_t* kg = keys + size_t(u) * keys_pitch;
  [[maybe_unused]] auto emit = [=](int r, int i) {  // by value: no local needs an address
    if (r >= e0 && r < e0 + np) pages[r - e0] = i;
    if (so) so[r] = i;
  };
  static_assert(kWaveTopkPages <= 16 * kWave, "one-wave top-k holds at most 16 rows");
  if constexpr (PRESEL) {
    const int32_t* pg = presel + size_t(u) * nsel + e0;
    for (int i = threadIdx.x; i < np; i += 256) pages[i] = pg[i];
  } else if (nblk <= kWaveTopkPages) {
    // one wave selects from keys held in registers (no barrier inside) and
    // emits only the ranks this split needs (all of them for the sel output)
    if (wave == 0)
      wave_topk_rows([=](int i) { return kg[i]; }, nblk_u, nsel_u, emit, tsm.hist[0], so ? 0 : e0,
                     so ? nsel_u : e0 + np);
  } else {
    uint32_t* kl = attn_lds + pages_per_split;  // [keys_pitch]
    for (int i = threadIdx.x; i < keys_pitch / 4; i += 256)
      reinterpret_cast<uint4*>(kl)[i] = reinterpret_cast<const uint4*>(kg)[i];
    __syncthreads();
    wg_topk<256, 1024>([&](int i) { return kl[i]; }, nblk_u, nsel_u, emit, tsm);
  }
  if (so)  // ranks past a ragged unit's choice
    for (int r = nsel_u + threadIdx.x; r < nsel; r += 256) so[r] = -1;
  __syncthreads();

  const size_t ubase = PAGED ? 0 : size_t(u) * size_t(kv_cap) * D;
  const T* ku = k + ubase + c * EPL;
  const T* vu = v + ubase + c * EPL;
  const int32_t* cu = MT ? cand + size_t(u) * size_t(cand_stride) : nullptr;
  const UnitPages up = PAGED ? UnitPages{pga.table + size_t(u / pga.hkv) * pga.table_stride, pga.n_phys,
                                         pga.shift, pga.hkv, u % pga.hkv}
                             : UnitPages{};
  attend_pages<T, D, G, MT, TPS_, PAGED>(qf, ku, vu, cu, kv_cap, pages, wave, np, NW, block, n_u,
                                         scale_log2, m, l, o, up);
  wave_state_to_lds<T, D, G>(m, l, o, wave, wm, wl, wo);
  __syncthreads();
  // merge the 4 waves in order and write this split's partial per head
  float* pw = partials + (size_t(u) * n_split + split) * G * PF;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    float mm, ll, oo;
    merge_waves<D, G, NW>(idx, wm, wl, wo, &mm, &ll, &oo);
    float* pg = pw + size_t(idx / D) * PF;
    pg[4 + idx % D] = oo;
    if (idx % D == 0) {
      pg[0] = mm;
      pg[1] = ll;
    }
  }
}

// Typed form of AppendArgs for the fused kernel.
template <typename T>
struct AppendPtrs {
  const T* k_new;
  const T* v_new;
  T* k;
  T* v;
  T* kmax;
  T* kmin;
};

// Steps 2 and 3 in one workgroup per unit, for large batches (the units alone
// fill the chip, so no split-K, no partials and no combine).  NT_ threads:
// wave 0 makes the channel choice; all threads stage and score the unit's
// pages chunk by chunk (npc pages per chunk); one wave (or, for many pages,
// the workgroup) takes the top-k2 pages; all waves stream them and the
// workgroup writes the normalised output.  Gathers of scattered rows on this
// chip gain bandwidth with resident waves per CU more than with loads in
// flight per wave, hence 1024 threads (4 waves per SIMD) by default; groups
// of four heads, whose per-token state leaves 1024-thread waves room for
// only 8 rows in flight, measured faster at 512 threads with 16 rows per wave.
//
// APP (a decode step that first appends token n_tokens - 1, as rk_append_kv
// would): the workgroup reads the last page's Kmax/Kmin column up front,
// patches the new key into its own staged copy of that column, lets the new
// token into the attention from LDS, and writes the new K/V row and the
// refreshed column at the very end (stores issued while the pages stream
// slow the stream), never reading back what it wrote.
//
// Dynamic LDS: page keys [roundup4(nblk)] | chosen pages [roundup4(nsel)] |
// a region holding first the staged chunk [npc][k1p], then the waves' merge
// state (m, l per wave and head, o per wave, head and channel).
// The cache and aux inputs are not restrict-qualified in the append form,
// which writes them through the AppendPtrs (same buffers) in the same launch.
template <typename T, bool APP>
using CacheIn = std::conditional_t<APP, const T*, const T* __restrict__>;

//
// PAGED: the K/V rows live in a paged pool (PagedArgs); the append writes its
// row there too.
template <typename T, int D, int G, bool MT, bool APP = false, bool PAGED = false, int NT_ = kFusedThreads>
__global__ __launch_bounds__(NT_) void hsa_fused_kernel(
    const T* __restrict__ q, CacheIn<T, APP> k, CacheIn<T, APP> v, int64_t kv_cap,
    const int32_t* __restrict__ cand, int64_t cand_stride, CacheIn<T, APP> kmax,
    CacheIn<T, APP> kmin, int64_t nblk_cap, int nblk, int k1, int nsel, int npc,
    int n_tokens, int block, float scale_log2, float* __restrict__ out,
    int32_t* __restrict__ sel_opt, int32_t* __restrict__ chan_opt, float* __restrict__ s1_opt,
    AppendPtrs<T> app, PagedArgs pga, const int32_t* __restrict__ lens) {
  // tokens per slot per step: MT 2 (with its candidate indices in LDS, 1, 3,
  // 4, 8 and 10 measured 0.6-3.5 us per step slower at batch 8 x 32 heads);
  // the 512-thread form for groups of four holds 4 (registers are twice as
  // plentiful per wave, so each wave keeps twice the rows in flight)
  constexpr int TPS = MT ? 2 : NT_ == kFusedThreadsWide ? 4 : AttnShape<T, D, G>::TPS;
  using S = AttnShape<T, D, G, TPS>;
  constexpr int EPL = S::EPL, LPR = S::LPR;
  constexpr int NT = NT_, NW = NT / kWave;
  constexpr int R = D / kWave;
  extern __shared__ __align__(16) unsigned char dyn_lds[];
  uint32_t* pkeys = reinterpret_cast<uint32_t*>(dyn_lds);
  int* pages = reinterpret_cast<int*>(pkeys + ((nblk + 3) & ~3));
  // MT: the unit's candidate indices [roundup4(n_tokens)]; PAGED: the first
  // pool row of each of its pages [roundup4(n_tokens / P)]
  int32_t* cand_l = reinterpret_cast<int32_t*>(pages + ((nsel + 3) & ~3));
  const int n_rows_l = MT ? n_tokens : PAGED ? ((n_tokens - 1) >> pga.shift) + 1 : 0;
  unsigned char* region = reinterpret_cast<unsigned char*>(cand_l + ((n_rows_l + 3) & ~3));
  T* stage = reinterpret_cast<T*>(region);
  float* wm = reinterpret_cast<float*>(region);
  float* wl = wm + NW * G;
  float* wo = wl + NW * G;
  __shared__ __align__(16) float i1_q[D + 16];
  __shared__ __align__(16) int i1_off[D + 16];
  __shared__ TopkSmem<NT, 1024, 1> tsm;

  const int u = blockIdx.x;
  const int t = threadIdx.x;
  const int wave = t / kWave, lane = lane_id();
  const int c = lane % LPR;

  float qf[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) unpack16(load16(q + (size_t(u) * G + g) * D + c * EPL), qf[g]);
  // ragged units (not with APP): this unit's tokens, pages and chosen pages;
  // the LDS layout keeps the launch-wide nblk and nsel
  const int n_unit = lens ? max(1, min(lens[u], n_tokens)) : n_tokens;
  const int nblk_u = lens ? (n_unit + block - 1) / block : nblk;
  const int nsel_u = min(nsel, nblk_u);
  const int n_cached = APP ? n_tokens - 1 : n_unit;  // tokens read from the cache
  const int app_page = (n_tokens - 1) / block;
  const UnitPages up = PAGED ? UnitPages{pga.table + size_t(u / pga.hkv) * pga.table_stride, pga.n_phys,
                                         pga.shift, pga.hkv, u % pga.hkv}
                             : UnitPages{};
  // first element of the appended token's row (APP only: row n_cached exists
  // only when a token is appended)
  size_t app_row = 0;
  if constexpr (APP)
    app_row = PAGED ? size_t(paged_row(up.table, n_cached, up.n_phys, up.shift, up.hkv, up.h)) * D
                    : (size_t(u) * size_t(kv_cap) + size_t(n_cached)) * D;
  // APP: the new key (as T, for the patch) and the new K/V rows (as float,
  // for the attention) go to LDS; the page's old Kmax/Kmin column is fetched
  // now and folded and written back at the end, after the stream.
  // The last waves do this work: wave 0's loads for the channel choice must
  // not queue behind the scattered column reads.
  __shared__ T app_knt[APP ? D : 1];
  __shared__ float app_kf[APP ? D : 1], app_vf[APP ? D : 1];
  T app_kn{}, app_vn{}, app_ox{}, app_on{};
  const bool app_fold = n_cached % block != 0;  // the page already holds tokens
  const int ta = t - (NT - D);                   // channel of this thread in the append work
  if constexpr (APP) {
    if (ta >= 0) {
      const size_t a = (size_t(u) * D + ta) * size_t(nblk_cap) + app_page;
      app_kn = app.k_new[size_t(u) * D + ta];
      app_vn = app.v_new[size_t(u) * D + ta];
      if (app_fold) {
        app_ox = app.kmax[a];
        app_on = app.kmin[a];
      }
    }
  }
  if (wave == 0) {
    float qx[R][G];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int g = 0; g < G; ++g) qx[r][g] = to_f32(q[(size_t(u) * G + g) * D + r * kWave + lane]);
    wave_choose_channels<T, D, G>(qx, k1, i1_q, i1_off, chan_opt ? chan_opt + size_t(u) * k1 : nullptr,
                                  tsm.hist[0]);
  } else if (MT) {
    // RocketKV-MT: the unit's candidate indices do not depend on the page
    // choice, so waves 1.. fetch all of them into LDS while wave 0 chooses
    // the channels (8 loads per thread in flight per round); the streaming
    // then finds each chosen token's row without a memory round trip
    const int32_t* cg = cand + size_t(u) * size_t(cand_stride);
    constexpr int NC = 8, NTC = NT - kWave;
    for (int i0 = t - kWave; i0 < n_unit; i0 += NTC * NC) {
      int32_t cb[NC];
#pragma unroll
      for (int x = 0; x < NC; ++x) cb[x] = i0 + x * NTC < n_unit ? cg[i0 + x * NTC] : 0;
#pragma unroll
      for (int x = 0; x < NC; ++x)
        if (i0 + x * NTC < n_unit) cand_l[i0 + x * NTC] = cb[x];
    }
  } else if (PAGED) {
    // paged pool: the same for the unit's block-table row, as pool row bases
    const int n_pg = ((n_unit - 1) >> pga.shift) + 1;
    for (int i = t - kWave; i < n_pg; i += NT - kWave)
      cand_l[i] = (clamp_row(up.table[i], up.n_phys) * up.hkv + up.h) << up.shift;
  }
  __syncthreads();

  const T* xu = kmax + size_t(u) * D * size_t(nblk_cap);
  const T* nu = kmin + size_t(u) * D * size_t(nblk_cap);
  for (int p0 = 0; p0 < nblk_u; p0 += npc) {
    const int np = min(npc, nblk_u - p0);
    stage_rows<T, NT>(xu + p0, nu + p0, nblk_cap, np, k1, i1_off, stage);
    if (APP && p0 == 0 && ta >= 0) {
      app_knt[ta] = app_kn;
      app_kf[ta] = to_f32(app_kn);
      app_vf[ta] = to_f32(app_vn);
    }
    __syncthreads();
    if (APP && app_page >= p0 && app_page < p0 + np) {
      // the staged (old) value of each chosen row of the last page takes the
      // new key in: max for a Kmax row, min for a Kmin row, the key itself
      // when the page starts with it
      if (t < k1) {
        const int o = i1_off[t];
        T* sv = stage + size_t(app_page - p0) * staged_pitch<T>(k1) + t;
        const T kn = app_knt[o >= 0 ? o : -1 - o];
        const float x = to_f32(kn), old = to_f32(*sv);
        if (!app_fold || (o >= 0 ? x > old : x < old)) *sv = kn;
      }
      __syncthreads();
    }
    score_staged<T, NT>(stage, np, k1, i1_q, pkeys + p0,
                        s1_opt ? s1_opt + size_t(u) * nblk + p0 : nullptr);
    __syncthreads();
  }

  int32_t* so = sel_opt ? sel_opt + size_t(u) * nsel : nullptr;
  auto emit = [=](int r, int i) {
    pages[r] = i;
    if (so) so[r] = i;
  };
  if (nblk <= kWaveTopkPages) {
    if (wave == 0)
      wave_topk_rows([=](int i) { return pkeys[i]; }, nblk_u, nsel_u, emit, tsm.hist[0], 0, nsel_u);
  } else {
    wg_topk<NT, 1024>([&](int i) { return pkeys[i]; }, nblk_u, nsel_u, emit, tsm);
  }
  if (so)  // ranks past a ragged unit's choice
    for (int r = nsel_u + t; r < nsel; r += NT) so[r] = -1;
  __syncthreads();

  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegBig;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = 0.f;
  }
  const size_t ubase = PAGED ? 0 : size_t(u) * size_t(kv_cap) * D;
  const T* ku = k + ubase + c * EPL;
  const T* vu = v + ubase + c * EPL;
  const int32_t* cu = MT ? cand_l : nullptr;
  UnitPages upl = up;
  if constexpr (PAGED) upl.base = cand_l;
  attend_pages<T, D, G, MT, TPS, PAGED>(qf, ku, vu, cu, kv_cap, pages, wave, nsel_u, NW, block, n_cached,
                                        scale_log2, m, l, o, upl);
  if constexpr (APP) {
    // the new token, when its page was chosen (the last page, so the last
    // entry of the ascending list), goes to wave 0's token slot 0
    if (wave == 0 && pages[nsel - 1] == app_page) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float sdot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) sdot += qf[g][e] * app_kf[c * EPL + e];
        const float x = group_sum<LPR>(sdot) * scale_log2;
        if (lane < LPR) {
          const float mn = fmaxf(m[g], x);
          const float corr = fast_exp2(m[g] - mn), pn = fast_exp2(x - mn);
          l[g] = l[g] * corr + pn;
          m[g] = mn;
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[g][e] = o[g][e] * corr + pn * app_vf[c * EPL + e];
        }
      }
    }
  }
  wave_state_to_lds<T, D, G>(m, l, o, wave, wm, wl, wo);  // the staged chunk is no longer read
  __syncthreads();
  for (int idx = t; idx < G * D; idx += NT) {
    float mm, ll, oo;
    merge_waves<D, G, NW>(idx, wm, wl, wo, &mm, &ll, &oo);
    out[size_t(u) * G * D + idx] = oo / ll;
  }
  if (APP && ta >= 0) {  // the refreshed column of the last page, for later steps
    T mx = app_kn, mn = app_kn;
    if (app_fold) {
      const float x = to_f32(app_kn);
      mx = x > to_f32(app_ox) ? app_kn : app_ox;
      mn = x < to_f32(app_on) ? app_kn : app_on;
    }
    const size_t a = (size_t(u) * D + ta) * size_t(nblk_cap) + app_page;
    app.kmax[a] = mx;
    app.kmin[a] = mn;
    app.k[app_row + ta] = app_kn;
    app.v[app_row + ta] = app_vn;
  }
}

// Dynamic LDS of the fused kernel for a chunk of npc pages.
inline size_t fused_lds_bytes(int nblk, int nsel, int npc, int k1p, size_t esize, int D, int G,
                              int64_t n_cand, int NW) {
  const size_t stage = size_t(npc) * k1p * esize;
  const size_t merge = (size_t(2) * NW * G + size_t(NW) * G * D) * sizeof(float);
  return size_t((nblk + 3) & ~3) * 4 + size_t((nsel + 3) & ~3) * 4 + size_t((n_cand + 3) & ~3) * 4 +
         (stage > merge ? stage : merge);
}

// One wave per (unit, head) merges the split partials.  Lane s (< n_split)
// holds split s's (m, l); the o rows are read as float4, each lane covering
// one 4-channel slice for one residue class of splits, all loads issued
// before any use.  Classes are then merged with a fixed butterfly.
template <int D, int G>
__global__ __launch_bounds__(256) void hsa_combine_kernel(const float* __restrict__ partials,
                                                          int n_split, int units,
                                                          float* __restrict__ out) {
  constexpr int PF = D + 4;
  constexpr int C4 = D / 4;               // float4 slices per head row
  constexpr int CLASSES = kWave / C4;     // split residue classes per wave
  constexpr int PER = kMaxSplits / CLASSES;
  static_assert(kWave % C4 == 0, "head row must tile a wave");
  const int wi = blockIdx.x * 4 + threadIdx.x / kWave;
  if (wi >= units * G) return;
  const int lane = lane_id();
  const int u = wi / G, g = wi % G;
  const float* pu = partials + size_t(u) * n_split * G * PF + size_t(g) * PF;
  const size_t stride = size_t(G) * PF;
  const int c4 = lane % C4, cls = lane / C4;
  float4 ov[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = cls + i * CLASSES;
    ov[i] = s < n_split ? reinterpret_cast<const float4*>(pu + s * stride + 4)[c4]
                        : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float2 ml = lane < n_split ? *reinterpret_cast<const float2*>(pu + lane * stride)
                                   : make_float2(kNegBig, 0.f);
  const float mm = wave_max(ml.x);
  const float a = lane < n_split ? fast_exp2(ml.x - mm) : 0.f;
  const float ll = wave_sum(ml.y * a);
  // every split's weight first (the lane permutes issue together), then the sums
  float wv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = cls + i * CLASSES;
    wv[i] = __shfl(a, s < kWave ? s : 0);
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = cls + i * CLASSES;
    const float w = wv[i];
    if (s < n_split) {
      acc.x += ov[i].x * w;
      acc.y += ov[i].y * w;
      acc.z += ov[i].z * w;
      acc.w += ov[i].w * w;
    }
  }
#pragma unroll
  for (int off = C4; off < kWave; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }
  if (cls == 0) {
    const float inv = 1.0f / ll;
    reinterpret_cast<float4*>(out + (size_t(u) * G + g) * D)[c4] =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
}

template <typename T, int D, int G>
hipError_t launch_decode_t(const Dims& d, const void* q, const void* k, const void* v,
                           int64_t kv_cap, const int32_t* cand, int64_t cand_stride,
                           const void* kmax, const void* kmin, int64_t nblk_cap,
                           int64_t n_tokens, int block, int k1, int k2, float* out,
                           int32_t* sel_opt, int32_t* chan_opt, float* s1_opt, void* ws,
                           hipStream_t s, const AppendArgs* app, bool exact_rows,
                           const PagedArgs* paged, const int32_t* lens) {
  const int nblk = int((n_tokens + block - 1) / block);
  const DecodeWs lay = decode_ws_layout(d, nblk, k2);
  // paged pools are built for bf16 only (the API refuses the rest)
  constexpr bool kPagedBuilt = std::is_same_v<T, bf16_t>;
  if (paged && !kPagedBuilt) return hipErrorInvalidValue;
  const PagedArgs pg = paged ? *paged : PagedArgs{};
  char* wsb = static_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(wsb + lay.partials);
  const int units = d.units();
  // the page choice gets a launch of its own when the attention workgroups
  // could not hold the page keys in LDS, and for token-level exact scoring
  const bool presel = exact_rows || nblk > kMaxPages;

  const float scale_log2 = float(1.4426950408889634 / sqrt(double(D)));
  // one workgroup per unit when the units fill the chip, or when each of its
  // 16 waves streams at most one page (the 109K needle: 16 pages per unit),
  // where the split path's three launches cost more than one CU per unit
  if constexpr (G <= 4) if (!presel && (units >= kFusedMinUnits || lay.nsel <= kFusedThreads / kWave)) {
    // one workgroup per unit: chunk of npc pages within the LDS budget
    const int k1pf = (k1 + 15) / 16 * 16 + int(16 / sizeof(T));
    // MT: the candidate indices go to LDS, paged pools the page table's row
    // bases; a list that leaves no room for a staged chunk of 64 pages takes
    // the split path
    const int64_t n_cand = cand ? n_tokens : paged ? ((n_tokens - 1) >> pg.shift) + 1 : 0;
    const bool cand_fits = size_t((nblk + 3) & ~3) * 4 + size_t((lay.nsel + 3) & ~3) * 4 +
                               size_t((n_cand + 3) & ~3) * 4 + size_t(64) * k1pf * sizeof(T) <=
                           kFusedLdsBudget;
    // groups of four at large batch: 512-thread workgroups (8 waves with up
    // to 256 registers each, 4 tokens per slot per step) measured 1.1 us per
    // step faster than 1024 threads at batch 32; MT and the few-pages batch-1
    // case keep 1024 (16 waves)
    const bool wide = G == 4 && !cand && units >= kFusedMinUnits;
    const int nw = (wide ? kFusedThreadsWide : kFusedThreads) / kWave;
    const size_t fixed = fused_lds_bytes(nblk, lay.nsel, 0, k1pf, sizeof(T), D, G, n_cand, nw);
    const size_t keys_sel = size_t((nblk + 3) & ~3) * 4 + size_t((lay.nsel + 3) & ~3) * 4 +
                            size_t((n_cand + 3) & ~3) * 4;
    int npc = kFusedLdsBudget > keys_sel
                  ? int((kFusedLdsBudget - keys_sel) / (size_t(k1pf) * sizeof(T))) / 8 * 8
                  : 0;
    const int nblk8 = (nblk + 7) / 8 * 8;
    npc = npc > nblk8 ? nblk8 : npc;
    if (npc >= 8 && fixed <= kFusedLdsBudget && cand_fits) {
      const size_t lds = fused_lds_bytes(nblk, lay.nsel, npc, k1pf, sizeof(T), D, G, n_cand, nw);
      // the wide form is built for groups of four only
      constexpr int kWideNT = G == 4 ? kFusedThreadsWide : kFusedThreads;
      static bool fattr = false;  // once per template instantiation
      if (!fattr) {
        for (const void* f :
             {reinterpret_cast<const void*>(&hsa_fused_kernel<T, D, G, true>),
              reinterpret_cast<const void*>(&hsa_fused_kernel<T, D, G, false>),
              reinterpret_cast<const void*>(&hsa_fused_kernel<T, D, G, false, true>),
              reinterpret_cast<const void*>(&hsa_fused_kernel<T, D, G, false, false, kPagedBuilt>),
              reinterpret_cast<const void*>(&hsa_fused_kernel<T, D, G, false, true, kPagedBuilt>),
              reinterpret_cast<const void*>(&hsa_fused_kernel<T, D, G, false, false, false, kWideNT>),
              reinterpret_cast<const void*>(&hsa_fused_kernel<T, D, G, false, true, false, kWideNT>),
              reinterpret_cast<const void*>(&hsa_fused_kernel<T, D, G, false, false, kPagedBuilt, kWideNT>),
              reinterpret_cast<const void*>(&hsa_fused_kernel<T, D, G, false, true, kPagedBuilt, kWideNT>)}) {
          hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             int(kFusedLdsBudget));
          if (e != hipSuccess) return e;
        }
        fattr = true;
      }
      const AppendPtrs<T> ap =
          app ? AppendPtrs<T>{static_cast<const T*>(app->k_new), static_cast<const T*>(app->v_new),
                              static_cast<T*>(app->k), static_cast<T*>(app->v),
                              static_cast<T*>(app->kmax), static_cast<T*>(app->kmin)}
              : AppendPtrs<T>{};
#define RK_FUSED(NAME, MTV, APPV, PGV, NTV)                                                       \
  RK_LAUNCH(NAME, (hsa_fused_kernel<T, D, G, MTV, APPV, PGV, NTV>), dim3(units), dim3(NTV), lds,    \
            s, static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), kv_cap, \
            cand, cand_stride, static_cast<const T*>(kmax), static_cast<const T*>(kmin), nblk_cap,  \
            nblk, k1, lay.nsel, npc, int(n_tokens), block, scale_log2, out, sel_opt, chan_opt,      \
            s1_opt, ap, pg, lens)
#define RK_FUSED_NT(NAME, APPV, PGV)                  \
  do {                                                \
    if (wide)                                         \
      RK_FUSED(NAME, false, APPV, PGV, kWideNT);      \
    else                                              \
      RK_FUSED(NAME, false, APPV, PGV, kFusedThreads); \
  } while (0)
      if (cand)
        RK_FUSED("hsa_fused_mt", true, false, false, kFusedThreads);
      else if (paged && app)
        RK_FUSED_NT("hsa_fused_append", true, kPagedBuilt);
      else if (paged)
        RK_FUSED_NT("hsa_fused", false, kPagedBuilt);
      else if (app)
        RK_FUSED_NT("hsa_fused_append", true, false);
      else
        RK_FUSED_NT("hsa_fused", false, false);
#undef RK_FUSED_NT
#undef RK_FUSED
      return hipGetLastError();
    }
  }

  // the split-K path appends with its own launch first
  if (app) {
    const hipError_t e = launch_append_kv(d, app->k_new, app->v_new, app->k, app->v, kv_cap,
                                          n_tokens - 1, app->kmax, app->kmin, nblk_cap, block, s,
                                          paged);
    if (e != hipSuccess) return e;
  }

  // Step 2a grid: page ranges of ppw pages (a multiple of 8, the staged
  // slice within the LDS budget) so the launch has about 1024 workgroups, at
  // least 8 pages each (at batch 1, 8-page ranges measured 0.2 us per step
  // faster than 16-page ones and 32-page ones 0.6 us slower).  Launches whose
  // full aux slices come to at most kScoreAllBytes fetch every channel's rows
  // up front (ALL).
  constexpr int EPV = 16 / sizeof(T);
  const int k1p = (k1 + 15) / 16 * 16 + EPV;
  const int ppw_max = int(kSelectLdsBudget / (size_t(k1p) * sizeof(T))) / 8 * 8;
  if (ppw_max < 8) return hipErrorInvalidValue;
  int ppw = int((int64_t(nblk) * units + 1023) / 1024);
  ppw = ppw < 8 ? 8 : ppw;
  ppw = (ppw + 7) / 8 * 8;
  ppw = ppw > ppw_max ? ppw_max : ppw;
  // ALL also needs the range to come in one round of 8 vectors per thread
  const bool all = size_t(2) * D * nblk * units * sizeof(T) <= kScoreAllBytes &&
                   2 * D * (ppw / EPV) <= 256 * 8;
  const int n_ranges = (nblk + ppw - 1) / ppw;
  const int score_wgs = (n_ranges * units + kXcds - 1) / kXcds * kXcds;
  uint32_t* keys = reinterpret_cast<uint32_t*>(wsb + lay.keys);
  // ALL: every channel's two rows, then the products [ppw][roundup16(k1) + 4] fp32
  const size_t lds = all ? size_t(2) * D * sizeof(T) * ppw + size_t(ppw) * ((k1 + 15) / 16 * 16 + 4) * 4
                         : size_t(k1p) * sizeof(T) * ppw;
  static bool attr_set = false;  // once per template instantiation
  if (!attr_set) {
    for (const void* f : {reinterpret_cast<const void*>(&hsa_score_kernel<T, D, G, true>),
                          reinterpret_cast<const void*>(&hsa_score_kernel<T, D, G, false>)}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         int(kSelectLdsBudget));
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  if (exact_rows)
    RK_LAUNCH("exact_score", (exact_score_kernel<T, D, G>),
              dim3(unsigned((n_tokens + 255) / 256), unsigned(units)), dim3(256), 0, s,
              static_cast<const T*>(q), static_cast<const T*>(k), kv_cap, int(n_tokens), keys,
              lay.keys_pitch, s1_opt);
  else if (all)
    RK_LAUNCH("hsa_score", (hsa_score_kernel<T, D, G, true>), dim3(score_wgs), dim3(256), lds, s,
              static_cast<const T*>(q), static_cast<const T*>(kmax), static_cast<const T*>(kmin),
              nblk_cap, nblk, k1, ppw, units, keys, lay.keys_pitch, chan_opt, s1_opt, lens,
              int(n_tokens), block);
  else
    RK_LAUNCH("hsa_score", (hsa_score_kernel<T, D, G, false>), dim3(score_wgs), dim3(256), lds, s,
              static_cast<const T*>(q), static_cast<const T*>(kmax), static_cast<const T*>(kmin),
              nblk_cap, nblk, k1, ppw, units, keys, lay.keys_pitch, chan_opt, s1_opt, lens,
              int(n_tokens), block);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // the page choice in a launch of its own (keys in LDS when they fit, with
  // up to 4096 words of radix candidates after them)
  int32_t* presel_pages = reinterpret_cast<int32_t*>(wsb + lay.sel);
  if (presel) {
    const size_t staged_words = size_t(lay.keys_pitch) + 4096;
    const bool staged = staged_words * 4 <= kSelectKeysLds;
    static bool sel_attr_set = false;  // once per template instantiation
    if (!sel_attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&page_select_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         int(kSelectKeysLds));
      if (e != hipSuccess) return e;
      sel_attr_set = true;
    }
    RK_LAUNCH("page_select", page_select_kernel, dim3(units), dim3(1024),
              staged ? staged_words * 4 : size_t(0), s, keys, lay.keys_pitch, nblk, lay.nsel,
              staged ? 1 : 0, staged ? 4096 : 0, presel_pages, sel_opt);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (exact_rows && chan_opt) {
      // every channel takes part, in ascending order
      RK_LAUNCH("exact_channels", fill_iota_kernel, dim3((units * D + 255) / 256), dim3(256), 0, s,
                chan_opt, D, units * D);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }

  // split-K sizing: aim for ~2048 workgroups over the whole launch, at least
  // kMinPagesPerSplit pages (one per wave; with a separate page choice, at
  // least 64 tokens: 16 per wave) and at most kMaxSplits splits per unit
  const int64_t total_pages = int64_t(units) * lay.nsel;
  int pps = int((total_pages + 2047) / 2048);
  const int pps_min = presel ? std::max(kMinPagesPerSplit, (64 + block - 1) / block) : kMinPagesPerSplit;
  pps = pps < pps_min ? pps_min : pps;
  const int pps_cap = (lay.nsel + kMaxSplits - 1) / kMaxSplits;
  pps = pps < pps_cap ? pps_cap : pps;
  pps = (pps + 3) / 4 * 4;
  const int nsel4 = (lay.nsel + 3) / 4 * 4;
  pps = pps > nsel4 ? nsel4 : pps;
  const int n_split = (lay.nsel + pps - 1) / pps;
  const size_t attn_lds =
      size_t(pps + (!presel && nblk > kWaveTopkPages ? lay.keys_pitch : 0)) * sizeof(uint32_t);  // <= 96 KB
  static bool attn_attr_set = false;  // once per template instantiation
  if (!attn_attr_set) {
    for (const void* f : {reinterpret_cast<const void*>(&hsa_attn_kernel<T, D, G, true>),
                          reinterpret_cast<const void*>(&hsa_attn_kernel<T, D, G, false>),
                          reinterpret_cast<const void*>(&hsa_attn_kernel<T, D, G, true, 4>),
                          reinterpret_cast<const void*>(&hsa_attn_kernel<T, D, G, false, 4>)}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         int(kAttnDynLds));
      if (e != hipSuccess) return e;
    }
    attn_attr_set = true;
  }
  if (attn_lds > kAttnDynLds) return hipErrorInvalidValue;
  const int attn_wgs = (n_split * units + kXcds - 1) / kXcds * kXcds;
  // at most one workgroup per CU: registers cannot limit occupancy, so each
  // wave takes 4 tokens per slot per step (fewer dependent load rounds)
  const bool one_per_cu = attn_wgs <= kComputeUnits;
#define RK_ATTN_P(NAME, MTV, TPSV, PRE, PGV)                                                      \
  RK_LAUNCH(NAME, (hsa_attn_kernel<T, D, G, MTV, TPSV, PRE, PGV>), dim3(attn_wgs), dim3(256),     \
            attn_lds, s, static_cast<const T*>(q), static_cast<const T*>(k),                      \
            static_cast<const T*>(v), kv_cap, cand, cand_stride, keys, lay.keys_pitch, nblk,       \
            lay.nsel, pps, n_split, units, int(n_tokens), block, scale_log2, part, sel_opt,        \
            presel_pages, pg, lens)
#define RK_ATTN(NAME, MTV, TPSV, PRE) RK_ATTN_P(NAME, MTV, TPSV, PRE, false)
  if (paged) {
    static bool pg_attr_set = false;  // once per template instantiation
    if (!pg_attr_set) {
      for (const void* f :
           {reinterpret_cast<const void*>(&hsa_attn_kernel<T, D, G, false, AttnShape<T, D, G>::TPS, false, kPagedBuilt>),
            reinterpret_cast<const void*>(&hsa_attn_kernel<T, D, G, false, 4, false, kPagedBuilt>),
            reinterpret_cast<const void*>(&hsa_attn_kernel<T, D, G, false, AttnShape<T, D, G>::TPS, true, kPagedBuilt>)}) {
        hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           int(kAttnDynLds));
        if (e != hipSuccess) return e;
      }
      pg_attr_set = true;
    }
    if (presel)
      RK_ATTN_P("hsa_attn", false, (AttnShape<T, D, G>::TPS), true, kPagedBuilt);
    else if (one_per_cu)
      RK_ATTN_P("hsa_attn", false, 4, false, kPagedBuilt);
    else
      RK_ATTN_P("hsa_attn", false, (AttnShape<T, D, G>::TPS), false, kPagedBuilt);
  } else if (presel) {
    static bool pre_attr_set = false;  // once per template instantiation
    if (!pre_attr_set) {
      for (const void* f :
           {reinterpret_cast<const void*>(&hsa_attn_kernel<T, D, G, true, AttnShape<T, D, G>::TPS, true>),
            reinterpret_cast<const void*>(&hsa_attn_kernel<T, D, G, false, AttnShape<T, D, G>::TPS, true>)}) {
        hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           int(kAttnDynLds));
        if (e != hipSuccess) return e;
      }
      pre_attr_set = true;
    }
    if (cand)
      RK_ATTN("hsa_attn_mt", true, (AttnShape<T, D, G>::TPS), true);
    else
      RK_ATTN("hsa_attn", false, (AttnShape<T, D, G>::TPS), true);
  } else if (cand) {
    if (one_per_cu)
      RK_ATTN("hsa_attn_mt", true, 4, false);
    else
      RK_ATTN("hsa_attn_mt", true, (AttnShape<T, D, G>::TPS), false);
  } else {
    if (one_per_cu)
      RK_ATTN("hsa_attn", false, 4, false);
    else
      RK_ATTN("hsa_attn", false, (AttnShape<T, D, G>::TPS), false);
  }
#undef RK_ATTN
#undef RK_ATTN_P
  if ((err = hipGetLastError()) != hipSuccess) return err;
  RK_LAUNCH("hsa_combine", (hsa_combine_kernel<D, G>), dim3((units * G + 3) / 4), dim3(256), 0, s,
            part, n_split, units, out);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_d(const Dims& d, const void* q, const void* k, const void* v,
                           int64_t kv_cap, const int32_t* cand, int64_t cand_stride,
                           const void* kmax, const void* kmin, int64_t nblk_cap,
                           int64_t n_tokens, int block, int k1, int k2, float* out,
                           int32_t* sel_opt, int32_t* chan_opt, float* s1_opt, void* ws,
                           hipStream_t s, const AppendArgs* app, bool exact_rows,
                           const PagedArgs* paged, const int32_t* lens) {
#define RK_DECODE_G(GG)                                                                        \
  case GG:                                                                                     \
    return launch_decode_t<T, D, GG>(d, q, k, v, kv_cap, cand, cand_stride, kmax, kmin,       \
                                     nblk_cap, n_tokens, block, k1, k2, out, sel_opt,         \
                                     chan_opt, s1_opt, ws, s, app, exact_rows, paged, lens);
  switch (d.G) {
    RK_DECODE_G(1)
    RK_DECODE_G(2)
    RK_DECODE_G(4)
    RK_DECODE_G(8)
    default:
      return hipErrorInvalidValue;
  }
#undef RK_DECODE_G
}

}  // namespace

hipError_t launch_hsa_decode(const Dims& d, const void* q, const void* k, const void* v,
                             int64_t kv_cap, const int32_t* cand, int64_t cand_stride,
                             const void* kmax, const void* kmin, int64_t nblk_cap,
                             int64_t n_tokens, int block, int k1, int k2, float* out,
                             int32_t* sel_opt, int32_t* chan_opt, float* s1_opt, void* ws,
                             hipStream_t s, const AppendArgs* app, bool exact_rows,
                             const PagedArgs* paged, const int32_t* lens) {
  if (d.bf16) {
    if (d.D == 128)
      return launch_decode_d<bf16_t, 128>(d, q, k, v, kv_cap, cand, cand_stride, kmax, kmin,
                                          nblk_cap, n_tokens, block, k1, k2, out, sel_opt,
                                          chan_opt, s1_opt, ws, s, app, exact_rows, paged, lens);
    return launch_decode_d<bf16_t, 64>(d, q, k, v, kv_cap, cand, cand_stride, kmax, kmin,
                                       nblk_cap, n_tokens, block, k1, k2, out, sel_opt,
                                       chan_opt, s1_opt, ws, s, app, exact_rows, paged, lens);
  }
  if (d.D == 128)
    return launch_decode_d<float, 128>(d, q, k, v, kv_cap, cand, cand_stride, kmax, kmin,
                                       nblk_cap, n_tokens, block, k1, k2, out, sel_opt,
                                       chan_opt, s1_opt, ws, s, app, exact_rows, paged, lens);
  return launch_decode_d<float, 64>(d, q, k, v, kv_cap, cand, cand_stride, kmax, kmin,
                                    nblk_cap, n_tokens, block, k1, k2, out, sel_opt, chan_opt,
                                    s1_opt, ws, s, app, exact_rows, paged, lens);
}

}  // namespace rk

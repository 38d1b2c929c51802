// rk_evict.hip -- stage 1: SnapKV-style permanent eviction.
//
// Sources: papercache notes "RocketKV: Accelerating Long-Context LLM Inference
// via Two-Stage KV Cache Compression" -- quick read (stage 1 keeps tokens by
// observation-window attention and pools with kernel 63) and method details
// (SnapKV paragraph, GQA group-level selection shared by the group, pooling
// kernel size); aifetchly "RocketKV Guide", stage 1 (observation window,
// softmax(Q K^T / sqrt(D)) summed over the window).
//
// Launch sequence per call (one stream, no host synchronisation):
//   ws_pass1   logits of the group's G*W window rows against K tiles (bf16 on
//              the matrix cores), causal on the window keys; per row, each
//              workgroup's max and sum of exp2 (log2 domain) -> partials
//   ws_stats   merge the partials of each row in tile order -> (m, 1/Z)
//   ws_pass2   recompute the prefix logits, p = exp2(x - m) / Z, sum over the
//              G*W rows in a fixed order -> score[j], j < S-W
//   pool       windowed sum of width pool_kernel -> pooled (for kernel 63 with
//              many units, done inside the select launch instead)
//   select     workgroup radix top-k (ties to the lower position) + window
//   gather     compaction of K and V rows, with the compact cache's Kmax/Kmin
//              when asked for (skipped for the RocketKV-MT form)
#include <math.h>

#include <algorithm>

#include "rk_device.hpp"
#include "rk_internal.hpp"

namespace rk {
namespace {

constexpr int TN = kWsTile;  // keys per tile
constexpr int RC = 32;       // window rows per chunk

// Loads RC rows (starting at r0) of the group's window queries into Qs and the
// key tile [j0, j0+TN) into Ks, then writes the scaled logits of the chunk to
// Ls[row][col].  Out-of-range rows/columns produce zeros (masked by callers).
template <typename T, int D>
__device__ __forceinline__ void ws_logits_chunk(const T* __restrict__ qg, const T* __restrict__ ku,
                                                int M, int r0, int j0, int S, bool load_k,
                                                float (*Qs)[D + 1], float (*Ks)[D + 1],
                                                float (*Ls)[TN + 1], float scale_log2) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int CPR = D / EPL;
  const int t = threadIdx.x;
  if (load_k) {
    for (int e = t; e < TN * CPR; e += 256) {
      const int col = e / CPR, ch = e % CPR;
      float x[EPL];
      if (j0 + col < S) {
        unpack16(load16(ku + size_t(j0 + col) * D + ch * EPL), x);
      } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) x[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i) Ks[col][ch * EPL + i] = x[i];
    }
  }
  for (int e = t; e < RC * CPR; e += 256) {
    const int row = e / CPR, ch = e % CPR;
    float x[EPL];
    if (r0 + row < M) {
      unpack16(load16(qg + size_t(r0 + row) * D + ch * EPL), x);
    } else {
#pragma unroll
      for (int i = 0; i < EPL; ++i) x[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) Qs[row][ch * EPL + i] = x[i];
  }
  __syncthreads();
  // thread -> (row, 8 consecutive columns)
  const int row = t % RC;
  const int cb = (t / RC) * (TN / 8);
  float acc[TN / 8];
#pragma unroll
  for (int i = 0; i < TN / 8; ++i) acc[i] = 0.f;
  for (int kk = 0; kk < D; ++kk) {
    const float qv = Qs[row][kk];
#pragma unroll
    for (int i = 0; i < TN / 8; ++i) acc[i] += qv * Ks[cb + i][kk];
  }
#pragma unroll
  for (int i = 0; i < TN / 8; ++i) Ls[row][cb + i] = acc[i] * scale_log2;
  __syncthreads();
}

// Pass 1: per (unit, key tile), per window row: tile max and sum of exp2.
template <typename T, int D>
__global__ __launch_bounds__(256) void ws_pass1_kernel(const T* __restrict__ q_win,
                                                       const T* __restrict__ k, int64_t kv_cap,
                                                       int S, int W, int G, int n_tiles,
                                                       float scale_log2,
                                                       float2* __restrict__ partials) {
  __shared__ float Qs[RC][D + 1];
  __shared__ float Ks[TN][D + 1];
  __shared__ float Ls[RC][TN + 1];
  const int u = blockIdx.y;
  const int tile = blockIdx.x;
  const int j0 = tile * TN;
  const int M = G * W;
  const T* qg = q_win + size_t(u) * M * D;  // the group's G heads x W rows are contiguous
  const T* ku = k + size_t(u) * size_t(kv_cap) * D;
  const int t = threadIdx.x;
  for (int r0 = 0; r0 < M; r0 += RC) {
    ws_logits_chunk<T, D>(qg, ku, M, r0, j0, S, r0 == 0, Qs, Ks, Ls, scale_log2);
    // thread -> (row, 8 columns); 8 lanes per row
    const int row = t / 8;
    const int part = t % 8;
    const int r_all = r0 + row;
    const int lim = S - W + (r_all % W);  // last key this row may see
    float mx = kNegBig;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int col = part * 8 + i;
      const int j = j0 + col;
      if (j < S && j <= lim) mx = fmaxf(mx, Ls[row][col]);
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int col = part * 8 + i;
      const int j = j0 + col;
      if (j < S && j <= lim) z += fast_exp2(Ls[row][col] - mx);
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) z += __shfl_xor(z, off);
    if (part == 0 && r_all < M) partials[(size_t(u) * n_tiles + tile) * M + r_all] = make_float2(mx, z);
    __syncthreads();
  }
}

// Merge the tile partials of every row: (m, 1/Z).  Partials are laid out
// [unit][tile][row] (each pass-1 workgroup writes one contiguous run, no
// partial-line writes).  A workgroup takes 64 rows; its 16 waves split the
// tiles in groups of 8 consecutive ones (wave s: groups s, s+16, ...), each
// thread one row, so a wave's reads of one tile are consecutive and a
// group's loads are in flight together.  The 16 split results are then
// merged in split order.
__global__ __launch_bounds__(1024) void ws_stats_kernel(const float2* __restrict__ partials,
                                                        int M, int n_tiles, int units,
                                                        float2* __restrict__ stats) {
  constexpr int RPW = 64, SPL = 16, GRP = 8;
  __shared__ float2 part[SPL][RPW];
  const int rl = threadIdx.x % RPW, sp = threadIdx.x / RPW;
  const int i = blockIdx.x * RPW + rl;  // row of all units: u * M + r
  float mm = kNegBig, z = 0.f;
  if (i < units * M) {
    const int u = i / M, r = i % M;
    const float2* pr = partials + size_t(u) * n_tiles * M + r;
    for (int t0 = sp * GRP; t0 < n_tiles; t0 += SPL * GRP) {
      float2 p[GRP];
#pragma unroll
      for (int g = 0; g < GRP; ++g)
        p[g] = t0 + g < n_tiles ? pr[size_t(t0 + g) * M] : make_float2(kNegBig, 0.f);
      float mn = mm;
#pragma unroll
      for (int g = 0; g < GRP; ++g) mn = fmaxf(mn, p[g].x);
      float zz = z * fast_exp2(mm - mn);
#pragma unroll
      for (int g = 0; g < GRP; ++g) zz += p[g].y * fast_exp2(p[g].x - mn);
      z = zz;
      mm = mn;
    }
  }
  part[sp][rl] = make_float2(mm, z);
  __syncthreads();
  if (sp == 0 && i < units * M) {
#pragma unroll
    for (int s2 = 1; s2 < SPL; ++s2) {
      const float2 q = part[s2][rl];
      const float mn = fmaxf(mm, q.x);
      z = z * fast_exp2(mm - mn) + q.y * fast_exp2(q.x - mn);
      mm = mn;
    }
    stats[i] = make_float2(mm, 1.0f / z);
  }
}

// Pass 2: score[j] = sum over the G*W rows of exp2(x - m) / Z, prefix keys only.
template <typename T, int D>
__global__ __launch_bounds__(256) void ws_pass2_kernel(const T* __restrict__ q_win,
                                                       const T* __restrict__ k, int64_t kv_cap,
                                                       int S, int W, int G, float scale_log2,
                                                       const float2* __restrict__ stats,
                                                       float* __restrict__ scores) {
  __shared__ float Qs[RC][D + 1];
  __shared__ float Ks[TN][D + 1];
  __shared__ float Ls[RC][TN + 1];
  __shared__ float red[4][TN];
  const int u = blockIdx.y;
  const int j0 = blockIdx.x * TN;
  const int M = G * W;
  const int P = S - W;
  const T* qg = q_win + size_t(u) * M * D;
  const T* ku = k + size_t(u) * size_t(kv_cap) * D;
  const float2* st = stats + size_t(u) * M;
  const int t = threadIdx.x;
  const int col = t % TN;
  const int part = t / TN;  // 4 parts x 8 rows of a 32-row chunk
  float total = 0.f;
  for (int r0 = 0; r0 < M; r0 += RC) {
    // keys at or past P (window keys) are never scored; they load as zero here
    ws_logits_chunk<T, D>(qg, ku, M, r0, j0, P, r0 == 0, Qs, Ks, Ls, scale_log2);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r_all = r0 + part * 8 + i;
      if (r_all < M) {
        const float2 mz = st[r_all];
        s += fast_exp2(Ls[part * 8 + i][col] - mz.x) * mz.y;
      }
    }
    red[part][col] = s;
    __syncthreads();
    if (part == 0) total += ((red[0][col] + red[1][col]) + red[2][col]) + red[3][col];
    __syncthreads();
  }
  if (part == 0 && j0 + col < P) scores[size_t(u) * P + j0 + col] = total;
}

// Pooling for a kernel 2*H+1 wide (H >= 4): a workgroup makes 2048 outputs,
// PT = 8 consecutive ones per thread, from a zero-padded LDS tile read back as
// 16-byte vectors.  The thread's outputs j0..j0+7 share the 2H-6 terms
// j0+7-H .. j0+H; that middle is summed once (left to right) and each output
// adds its own left run (summed right to left, so the runs nest) and right
// run (left to right): about 10 adds per output instead of 2H, which made
// the old one-sum-per-output form arithmetic-bound.  All terms are
// non-negative, so the regrouping changes a sum by a few ulp at most; zeros
// past either end add nothing.  Results go through LDS so the stores are
// coalesced whatever the row alignment.
// The pooling's combining operation: a rounded add, or (the max reading of
// the pooling) a maximum, which is exact, so any grouping gives the same
// value.  Window scores are never negative, so the zeros past either end of
// the prefix leave a maximum unchanged as they leave a sum.
template <bool MX>
__device__ __forceinline__ float pool_comb(float a, float b) {
  return MX ? fmaxf(a, b) : __fadd_rn(a, b);
}

template <int H, bool MX = false>
__global__ __launch_bounds__(256) void pool_sum_reg_kernel(const float* __restrict__ scores,
                                                           int P, float* __restrict__ pooled) {
  constexpr int PT = 8;
  constexpr int OUT = 256 * PT;
  constexpr int NVAL = PT + 2 * H;        // scores a thread reads
  constexpr int NV = (NVAL + 3) / 4;      // as 16-byte vectors
  constexpr int TW = OUT - PT + 4 * NV;   // tile width (a multiple of 4)
  static_assert(2 * H + 1 >= PT, "the outputs of a thread must share a middle");
  __shared__ __align__(16) float tile[TW];
  __shared__ float res[OUT];
  const int u = blockIdx.y;
  const int j0 = blockIdx.x * OUT;
  const float* su = scores + size_t(u) * P;
  for (int e = threadIdx.x; e < TW; e += 256) {
    const int j = j0 - H + e;
    tile[e] = (j >= 0 && j < P) ? su[j] : 0.f;
  }
  __syncthreads();
  const int t = threadIdx.x;
  float v[NV * 4];
#pragma unroll
  for (int x = 0; x < NV; ++x) {
    const float4 f = *reinterpret_cast<const float4*>(tile + PT * t + 4 * x);
    v[4 * x] = f.x;
    v[4 * x + 1] = f.y;
    v[4 * x + 2] = f.z;
    v[4 * x + 3] = f.w;
  }
  // output e (0 <= e < PT) sums v[e .. e + 2H]
  float mid = v[PT - 1];
#pragma unroll
  for (int i = PT; i <= 2 * H; ++i) mid = pool_comb<MX>(mid, v[i]);
  float left[PT];  // left[e] = v[e] + ... + v[PT - 2]
  left[PT - 1] = 0.f;
#pragma unroll
  for (int e = PT - 2; e >= 0; --e) left[e] = e == PT - 2 ? v[e] : pool_comb<MX>(v[e], left[e + 1]);
  float right = 0.f;  // v[2H + 1] + ... + v[2H + e]
#pragma unroll
  for (int e = 0; e < PT; ++e) {
    if (e > 0) right = e == 1 ? v[2 * H + 1] : pool_comb<MX>(right, v[2 * H + e]);
    float acc = e < PT - 1 ? pool_comb<MX>(left[e], mid) : mid;
    if (e > 0) acc = pool_comb<MX>(acc, right);
    res[PT * t + e] = acc;
  }
  __syncthreads();
  float* pu = pooled + size_t(u) * P;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int j = j0 + i * 256 + t;
    if (j < P) pu[j] = res[i * 256 + t];
  }
}

// pooled[j] = sum_{i=j-h}^{j+h} score[i] (zero outside [0, P)), left to right;
// MX: the maximum of the same terms.
template <bool MX = false>
__global__ __launch_bounds__(256) void pool_sum_kernel(const float* __restrict__ scores, int P, int h,
                                                   float* __restrict__ pooled) {
  extern __shared__ float tile[];  // 256 + 2h
  const int u = blockIdx.y;
  const int j0 = blockIdx.x * 256;
  const float* su = scores + size_t(u) * P;
  for (int e = threadIdx.x; e < 256 + 2 * h; e += 256) {
    const int j = j0 - h + e;
    tile[e] = (j >= 0 && j < P) ? su[j] : 0.f;
  }
  __syncthreads();
  const int j = j0 + threadIdx.x;
  if (j >= P) return;
  float acc = 0.f;
  for (int i = 0; i <= 2 * h; ++i) {
    const int src = j - h + i;
    if (src >= 0 && src < P) acc = pool_comb<MX>(acc, tile[threadIdx.x + i]);
  }
  pooled[size_t(u) * P + j] = acc;
}

// Top (n_keep - W) prefix positions by pooled score, ascending, then the window.
// When the P = S - W keys fit, they are converted to order keys once and held
// in LDS (dynamic, P words) for all radix passes and the compaction.
__global__ __launch_bounds__(1024) void select_kernel(const float* __restrict__ pooled, int S,
                                                      int W, int n_keep, int staged, int cand_cap,
                                                      int32_t* __restrict__ kept) {
  extern __shared__ uint32_t skeys[];
  __shared__ TopkSmem<1024, 2048, 1> sm;
  const int u = blockIdx.x;
  const int P = S - W;
  const float* pu = pooled + size_t(u) * P;
  int32_t* ku = kept + size_t(u) * n_keep;
  auto emit = [&](int r, int i) { ku[r] = i; };
  if (staged) {
    // 16-byte loads where the row allows it, all of a thread's loads in flight
    // (the key range comes along: no separate pass for it)
    const bool vec = (reinterpret_cast<uintptr_t>(pu) & 15u) == 0;
    const int P4 = vec ? P / 4 : 0;
    uint32_t lo = 0xffffffffu, hi = 0u;
    auto put = [&](int i, float x) {
      const uint32_t kk = order_key(x);
      skeys[i] = kk;
      lo = min(lo, kk);
      hi = max(hi, kk);
    };
    for (int i0 = threadIdx.x; i0 < P4; i0 += 1024 * 16) {
      float4 buf[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int i = i0 + x * 1024;
        if (i < P4) buf[x] = reinterpret_cast<const float4*>(pu)[i];
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int i = i0 + x * 1024;
        if (i < P4) {
          put(4 * i, buf[x].x);
          put(4 * i + 1, buf[x].y);
          put(4 * i + 2, buf[x].z);
          put(4 * i + 3, buf[x].w);
        }
      }
    }
    for (int i = 4 * P4 + threadIdx.x; i < P; i += 1024) put(i, pu[i]);
    __syncthreads();
    // the LDS after the keys (cand_cap words) takes the later passes' candidates
    wg_topk<1024, 2048>([&](int i) { return skeys[i]; }, P, n_keep - W, emit, sm, true, lo, hi,
                        skeys + P, cand_cap);
  } else {
    wg_topk<1024, 2048>([&](int i) { return order_key(pu[i]); }, P, n_keep - W, emit, sm);
  }
  for (int r = threadIdx.x; r < W; r += 1024) ku[n_keep - W + r] = P + r;
}

// Pooling and selection in one launch (pool kernel 2H+1, the prefix keys
// held in LDS): the workgroup stages the unit's window scores with a zero
// halo of H on either side, pools them eight outputs per thread at a time as
// pool_sum_reg_kernel does (same grouping, so the same values), turns them
// into order keys in place once every thread has read its window, and selects
// as select_kernel does.  Saves the pooled scores' round trip through memory
// and a launch; the pooled scores are still written when asked for.
template <int H, bool MX = false>
__global__ __launch_bounds__(1024) void select_pool_kernel(const float* __restrict__ scores,
                                                           int S, int W, int n_keep, int cand_cap,
                                                           float* __restrict__ pooled_opt,
                                                           int32_t* __restrict__ kept) {
  constexpr int PT = 8;                       // outputs per thread chunk
  constexpr int NVAL = PT + 2 * H;            // window of a chunk
  constexpr int NV = (NVAL + 3) / 4;          // as 16-byte vectors
  constexpr int MAXC = 5;                     // chunks per thread: P <= 5 * 8 * 1024
  static_assert(2 * H + 1 >= PT, "the outputs of a chunk must share a middle");
  extern __shared__ __align__(16) uint32_t skeys[];  // raw scores (haloed), then keys
  __shared__ TopkSmem<1024, 2048, 1> sm;
  float* raw = reinterpret_cast<float*>(skeys);   // raw[H + i] = score[i]
  const int u = blockIdx.x;
  const int t = threadIdx.x;
  const int P = S - W;
  const float* su = scores + size_t(u) * P;
  int32_t* ku = kept + size_t(u) * n_keep;
  auto emit = [&](int r, int i) { ku[r] = i; };
  const int nchunk = (P + PT - 1) / PT;
  const int tw = nchunk * PT + 4 * NV - PT;       // raw words any chunk reads
  for (int e = t; e < H; e += 1024) raw[e] = 0.f;
  for (int e = H + P + t; e < tw; e += 1024) raw[e] = 0.f;
  {
    // 16-byte loads where the row allows it, all of a thread's loads in flight
    const bool vec = (reinterpret_cast<uintptr_t>(su) & 15u) == 0;
    const int P4 = vec ? P / 4 : 0;
    for (int i0 = t; i0 < P4; i0 += 1024 * 16) {
      float4 buf[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int i = i0 + x * 1024;
        if (i < P4) buf[x] = reinterpret_cast<const float4*>(su)[i];
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int i = i0 + x * 1024;
        if (i < P4) {
          raw[H + 4 * i] = buf[x].x;
          raw[H + 4 * i + 1] = buf[x].y;
          raw[H + 4 * i + 2] = buf[x].z;
          raw[H + 4 * i + 3] = buf[x].w;
        }
      }
    }
    for (int i = 4 * P4 + t; i < P; i += 1024) raw[H + i] = su[i];
  }
  __syncthreads();
  float out[MAXC][PT];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int ch = t + c * 1024;
    if (ch < nchunk) {
      float v[NV * 4];
#pragma unroll
      for (int x = 0; x < NV; ++x) {
        const float4 f = *reinterpret_cast<const float4*>(raw + PT * ch + 4 * x);
        v[4 * x] = f.x;
        v[4 * x + 1] = f.y;
        v[4 * x + 2] = f.z;
        v[4 * x + 3] = f.w;
      }
      float mid = v[PT - 1];
#pragma unroll
      for (int i = PT; i <= 2 * H; ++i) mid = pool_comb<MX>(mid, v[i]);
      float left[PT];
      left[PT - 1] = 0.f;
#pragma unroll
      for (int e = PT - 2; e >= 0; --e) left[e] = e == PT - 2 ? v[e] : pool_comb<MX>(v[e], left[e + 1]);
      float right = 0.f;
#pragma unroll
      for (int e = 0; e < PT; ++e) {
        if (e > 0) right = e == 1 ? v[2 * H + 1] : pool_comb<MX>(right, v[2 * H + e]);
        float acc = e < PT - 1 ? pool_comb<MX>(left[e], mid) : mid;
        if (e > 0) acc = pool_comb<MX>(acc, right);
        out[c][e] = acc;
      }
    }
  }
  __syncthreads();  // every window is read: the keys go over the raw scores
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int ch = t + c * 1024;
    if (ch < nchunk) {
#pragma unroll
      for (int e = 0; e < PT; ++e) {
        const int i = PT * ch + e;
        if (i < P) {
          const uint32_t kk = order_key(out[c][e]);
          skeys[i] = kk;
          lo = min(lo, kk);
          hi = max(hi, kk);
          if (pooled_opt) pooled_opt[size_t(u) * P + i] = out[c][e];
        }
      }
    }
  }
  __syncthreads();
  wg_topk<1024, 2048>([&](int i) { return skeys[i]; }, P, n_keep - W, emit, sm, true, lo, hi,
                      skeys + P, cand_cap);
  for (int r = t; r < W; r += 1024) ku[n_keep - W + r] = P + r;
}

// Top-k over more keys than LDS holds, in two launches.  select_chunk: one
// workgroup per (chunk of C keys, unit) takes the chunk's own top-min(k, len)
// and writes their positions, ascending, over the chunk's (spent) score
// entries.  select_final: one workgroup per unit takes the top-k of the union
// of the candidates, which are in ascending position order.  Exact: a key in
// the overall top-k has fewer than k keys ahead of it (greater, or equal at a
// lower position) overall, so also within its chunk.
__global__ __launch_bounds__(1024) void select_chunk_kernel(const float* __restrict__ pooled,
                                                            int P, int C, int k,
                                                            int32_t* __restrict__ cand) {
  extern __shared__ uint32_t skeys[];
  __shared__ TopkSmem<1024, 2048, 1> sm;
  const int u = blockIdx.y;
  const int j0 = blockIdx.x * C;
  const int len = min(C, P - j0);
  const float* pu = pooled + size_t(u) * P + j0;
  for (int i = threadIdx.x; i < len; i += 1024) skeys[i] = order_key(pu[i]);
  __syncthreads();
  int32_t* cu = cand + size_t(u) * P + j0;
  wg_topk<1024, 2048>([&](int i) { return skeys[i]; }, len, min(k, len),
                      [&](int r, int i) { cu[r] = j0 + i; }, sm);
}

__global__ __launch_bounds__(1024) void select_final_kernel(const float* __restrict__ pooled, int S,
                                                            int W, int C, int n_keep,
                                                            const int32_t* __restrict__ cand,
                                                            int32_t* __restrict__ kept) {
  extern __shared__ uint32_t fl[];  // keys [n_cand], then positions [n_cand]
  __shared__ TopkSmem<1024, 2048, 1> sm;
  const int u = blockIdx.x;
  const int P = S - W;
  const int k = n_keep - W;
  const int n_chunks = (P + C - 1) / C;
  const int kc = min(k, C);
  int n_cand = 0;
  for (int c = 0; c < n_chunks; ++c) n_cand += min(kc, P - c * C);
  uint32_t* keys = fl;
  int32_t* pos = reinterpret_cast<int32_t*>(fl + n_cand);
  const float* pu = pooled + size_t(u) * P;
  const int32_t* cu = cand + size_t(u) * P;
  for (int i = threadIdx.x; i < n_cand; i += 1024) {
    const int c = min(i / kc, n_chunks - 1);  // every chunk but the last holds kc candidates
    const int p = cu[c * C + (i - c * kc)];
    pos[i] = p;
    keys[i] = order_key(pu[p]);
  }
  __syncthreads();
  int32_t* ku = kept + size_t(u) * n_keep;
  wg_topk<1024, 2048>([&](int i) { return keys[i]; }, n_cand, k,
                      [&](int r, int i) { ku[r] = pos[i]; }, sm);
  for (int r = threadIdx.x; r < W; r += 1024) ku[k + r] = P + r;
}

// Compact cache rows: out[n] = in[kept[n]] for K and V.
// Ada-KV shared budget: one workgroup per sequence takes the K = Hkv * kper
// largest pooled scores over all of its heads together (flattened [head,
// position], ties to the lower head, then position), staged in LDS when they
// fit (`staged`, with spare LDS for radix candidates) or read from memory each
// pass.  The chosen flattened indices come out ascending into tmp, so each
// head's run is contiguous: its bounds are found by binary search, its
// positions written to kept[unit][0 ..) and followed by the W window
// positions, and counts[unit] = its prefix count + W.
constexpr int kAdaMaxHeads = 64;

// ---- Ada-KV shared budget over many workgroups ------------------------------
// For a sequence whose Hkv * P pooled keys do not fit one workgroup's LDS,
// the cut is found by a most-significant-digit radix select in three passes
// (key bits 31-21, 20-10, 9-0), one launch each: every workgroup adds the
// LDS histogram of kAdaChunk keys into the sequence's global 2048-bin
// histogram of that pass.  A pass needs the prefix fixed by the earlier
// ones: each of its workgroups finds it again from the earlier passes'
// histograms (8 KB each, read from L2), so no launch does only that and no
// workgroup waits for another.  The count launch finds the cut T the same
// way and counts, per unit and kAdaEmitChunk chunk, the keys above and equal
// to T; the emit launch writes each unit's kept positions: keys above T, and
// keys equal to it in flattened (head-major, then position) order, so a lower
// head takes its equal keys first.
constexpr int kAdaChunk = 8192;      // keys per histogram workgroup (1024 threads x 8)
constexpr int kAdaBins = 2048;
constexpr int kAdaEmitChunk = 4096;  // positions per emit workgroup (256 threads x 16)
constexpr int kAdaCountChunks = 4;   // emit chunks per count workgroup (1024 threads)
struct AdaCut {
  uint32_t T;  // the cut: the K-th largest key of the sequence
  int need;    // keys equal to T that are taken
};

// zeroes the three passes' histograms (a fill kernel, so the sequence of
// launches stays capturable)
__global__ __launch_bounds__(256) void ada_clear_kernel(uint32_t* __restrict__ hist, int words) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < words) hist[i] = 0u;
}

// hist: [3][B][kAdaBins]
__global__ __launch_bounds__(1024) void ada_hist_kernel(const float* __restrict__ pooled, int B, int n, int pass,
                                                       int K, uint32_t* __restrict__ hist) {
  __shared__ __align__(16) uint32_t h[kAdaBins];
  __shared__ __align__(16) uint32_t hp[2 * kAdaBins];
  __shared__ int res[2];
  const int b = blockIdx.y;
  for (int i = threadIdx.x; i < kAdaBins; i += 1024) h[i] = 0u;
  uint32_t prefix = 0u;
  if (pass > 0) {
    // the earlier passes' histograms of this sequence, one after another
    const uint32_t* hb0 = hist + size_t(b) * kAdaBins;
    for (int i = threadIdx.x; i < pass * kAdaBins / 4; i += 1024) {
      const int p = i / (kAdaBins / 4), j = i % (kAdaBins / 4);
      reinterpret_cast<uint4*>(hp)[i] =
          reinterpret_cast<const uint4*>(hb0 + size_t(p) * B * kAdaBins)[j];
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      uint32_t pre = 0u;
      int need = K;
      for (int p = 0; p < pass; ++p) {
        const int3 f = wave_find_bin<kAdaBins>(hp + p * kAdaBins, need);
        pre = (pre << 11) | uint32_t(f.x);
        need = f.y;
      }
      if (threadIdx.x == 0) res[0] = int(pre);
    }
    __syncthreads();
    prefix = uint32_t(res[0]);
  } else {
    __syncthreads();
  }
  const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
  const uint32_t mask = pass == 2 ? 1023u : 2047u;
  const int fixed = pass == 0 ? 32 : pass == 1 ? 21 : 10;  // key bits [fixed, 32) equal the prefix
  const float* pb = pooled + size_t(b) * n;
  const int i0 = blockIdx.x * kAdaChunk;
  const int i1 = min(i0 + kAdaChunk, n);
  for (int i = i0 + int(threadIdx.x); i < i1; i += 1024) {
    const uint32_t kk = order_key(pb[i]);
    if (fixed == 32 || (kk >> fixed) == prefix) atomicAdd(&h[(kk >> shift) & mask], 1u);
  }
  __syncthreads();
  uint32_t* hb = hist + (size_t(pass) * B + b) * kAdaBins;
  for (int i = threadIdx.x; i < kAdaBins; i += 1024)
    if (h[i]) atomicAdd(&hb[i], h[i]);
}

// The cut from the three histograms, then the keys above and equal to it in
// each kAdaEmitChunk chunk of each unit: cnt[u * nchunk + c].  Workgroup
// (0, unit 0 of b) stores the cut of sequence b.
__global__ __launch_bounds__(1024) void ada_count_kernel(const float* __restrict__ pooled, int B, int Hkv, int P,
                                                        int nchunk, int K, const uint32_t* __restrict__ hist,
                                                        AdaCut* __restrict__ cut, int2* __restrict__ cnt) {
  __shared__ __align__(16) uint32_t hp[3 * kAdaBins];
  __shared__ int res[2];
  __shared__ int red[2][1024 / kWave];
  const int cc = blockIdx.x, u = blockIdx.y;
  const int b = u / Hkv;
  const uint32_t* hb0 = hist + size_t(b) * kAdaBins;
  for (int i = threadIdx.x; i < 3 * kAdaBins / 4; i += 1024) {
    const int p = i / (kAdaBins / 4), j = i % (kAdaBins / 4);
    reinterpret_cast<uint4*>(hp)[i] = reinterpret_cast<const uint4*>(hb0 + size_t(p) * B * kAdaBins)[j];
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    uint32_t pre = 0u;
    int need = K;
    for (int p = 0; p < 3; ++p) {
      const int3 f = wave_find_bin<kAdaBins>(hp + p * kAdaBins, need);
      pre = (pre << (p == 2 ? 10 : 11)) | uint32_t(f.x);
      need = f.y;
    }
    if (threadIdx.x == 0) {
      res[0] = int(pre);
      res[1] = need;
      if (cc == 0 && u % Hkv == 0) cut[b] = AdaCut{pre, need};
    }
  }
  __syncthreads();
  const uint32_t T = uint32_t(res[0]);
  // thread t counts sub-chunk t / 256 of this workgroup's kAdaCountChunks
  const int sc = threadIdx.x / 256;
  const int c = cc * kAdaCountChunks + sc;
  const float* pu = pooled + size_t(u) * P;
  const int i1 = min((c + 1) * kAdaEmitChunk, P);
  int gt = 0, eq = 0;
  for (int i = c * kAdaEmitChunk + int(threadIdx.x % 256); i < i1; i += 256) {
    const uint32_t kk = order_key(pu[i]);
    gt += kk > T ? 1 : 0;
    eq += kk == T ? 1 : 0;
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    gt += __shfl_xor(gt, off);
    eq += __shfl_xor(eq, off);
  }
  const int wave = threadIdx.x / kWave;
  if (lane_id() == 0) {
    red[0][wave] = gt;
    red[1][wave] = eq;
  }
  __syncthreads();
  if (threadIdx.x < kAdaCountChunks && cc * kAdaCountChunks + int(threadIdx.x) < nchunk) {
    constexpr int WPS = 256 / kWave;  // waves per sub-chunk
    int g = 0, e = 0;
    for (int w = 0; w < WPS; ++w) {
      g += red[0][threadIdx.x * WPS + w];
      e += red[1][threadIdx.x * WPS + w];
    }
    cnt[size_t(u) * nchunk + cc * kAdaCountChunks + threadIdx.x] = make_int2(g, e);
  }
}

// Each unit's kept positions (ascending) then the window's, and its count;
// workgroup c writes the positions chunk c selects.  mode 0: the cut;
// 1: every key (the budget covers them all); -1: none.
__global__ __launch_bounds__(256) void ada_emit_kernel(const float* __restrict__ pooled, int Hkv, int P, int W,
                                                      int nchunk, int mode, const AdaCut* __restrict__ cut,
                                                      const int2* __restrict__ cnt,
                                                      int32_t* __restrict__ kept, int kept_stride,
                                                      int32_t* __restrict__ counts) {
  constexpr int NWV = 256 / kWave;
  constexpr int RPW = kAdaEmitChunk / 256;  // rows of 64 positions per wave
  __shared__ int wsum[2][NWV];
  const int c = blockIdx.x, u = blockIdx.y;
  const int b = u / Hkv, h = u % Hkv;
  const int t = threadIdx.x, lane = lane_id(), wv = t / kWave;
  int32_t* ku = kept + size_t(u) * kept_stride;
  const int i0 = c * kAdaEmitChunk;
  const int i1 = min(i0 + kAdaEmitChunk, P);
  int n_sel;
  if (mode != 0) {
    if (mode == 1)
      for (int i = i0 + t; i < i1; i += 256) ku[i] = i;
    n_sel = mode == 1 ? P : 0;
  } else {
    const uint32_t T = cut[b].T;
    // sums over the sequence's chunk counts (every wave the same): keys
    // equal to T in lower heads, and this unit's counts before chunk c and
    // in total
    const int2* cb = cnt + size_t(b) * Hkv * nchunk;
    int eq_lower = 0, eq_u = 0, gt_u = 0, gt_pre = 0, eq_pre = 0, eq_c = 0;
    for (int j = lane; j < (h + 1) * nchunk; j += kWave) {
      const int2 v = cb[j];
      if (j < h * nchunk) {
        eq_lower += v.y;
      } else {
        const int cj = j - h * nchunk;
        eq_u += v.y;
        gt_u += v.x;
        gt_pre += cj < c ? v.x : 0;
        eq_pre += cj < c ? v.y : 0;
        eq_c += cj == c ? v.y : 0;
      }
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      eq_lower += __shfl_xor(eq_lower, off);
      eq_u += __shfl_xor(eq_u, off);
      gt_u += __shfl_xor(gt_u, off);
      gt_pre += __shfl_xor(gt_pre, off);
      eq_pre += __shfl_xor(eq_pre, off);
      eq_c += __shfl_xor(eq_c, off);
    }
    const int eq_take = max(0, min(cut[b].need - eq_lower, eq_u));  // this unit's keys equal to T
    const int eq_chunk = max(0, min(eq_take - eq_pre, eq_c));       // ... of them in chunk c
    // at most the room before the window (never exceeded by a consistent
    // cut; the bound keeps every store inside the unit's row regardless)
    const int room = kept_stride - W;
    n_sel = min(gt_u + eq_take, room);
    // wave wv holds positions [i0 + wv * 64 * RPW, +64 * RPW) of the chunk
    const unsigned long long below = (1ull << lane) - 1ull;
    const int r0 = i0 + wv * kWave * RPW;
    uint32_t kk[RPW];
    int g = 0, e = 0;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int i = r0 + r * kWave + lane;
      kk[r] = i < i1 ? order_key(pooled[size_t(u) * P + i]) : 0u;
      const bool in = i < i1;
      g += __popcll(ballot(in && kk[r] > T));
      e += __popcll(ballot(in && kk[r] == T));
    }
    if (lane == 0) {
      wsum[0][wv] = g;
      wsum[1][wv] = e;
    }
    __syncthreads();
    int g_w = 0, e_w = 0;
    for (int w = 0; w < wv; ++w) {
      g_w += wsum[0][w];
      e_w += wsum[1][w];
    }
    int base = gt_pre + min(eq_pre, eq_take) + g_w + min(e_w, eq_chunk);
    int eq_seen = e_w;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int i = r0 + r * kWave + lane;
      const bool in = i < i1;
      const bool eq = in && kk[r] == T;
      const unsigned long long em = ballot(eq);
      const bool sel = (in && kk[r] > T) || (eq && eq_seen + int(__popcll(em & below)) < eq_chunk);
      const unsigned long long sm = ballot(sel);
      const int pos = base + int(__popcll(sm & below));
      if (sel && pos < room) ku[pos] = i;
      base += __popcll(sm);
      eq_seen += __popcll(em);
    }
  }
  if (c == 0) {
    for (int w = t; w < W; w += 256) ku[n_sel + w] = P + w;
    if (t == 0) counts[u] = n_sel + W;
  }
}

// A sequence whose Hkv * P pooled keys (and a 4096-key candidate buffer) fit
// in LDS: one workgroup stages their order keys, takes the workgroup top-k of
// the flattened keys into tmp (ascending), then splits it by head.
__global__ __launch_bounds__(1024) void adakv_select_kernel(const float* __restrict__ pooled, int Hkv,
                                                            int P, int W, int kper, int cand_cap,
                                                            int32_t* __restrict__ tmp,
                                                            int32_t* __restrict__ kept, int kept_stride,
                                                            int32_t* __restrict__ counts) {
  extern __shared__ uint32_t skeys[];
  __shared__ TopkSmem<1024, 2048, 1> sm;
  __shared__ int start[kAdaMaxHeads + 1];
  const int b = blockIdx.x;
  const int n = Hkv * P;
  const int K = Hkv * kper;
  const float* pb = pooled + size_t(b) * n;
  int32_t* tb = tmp + size_t(b) * n;
  auto emit = [=](int r, int i) { tb[r] = i; };
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = threadIdx.x; i < n; i += 1024) {
    const uint32_t kk = order_key(pb[i]);
    skeys[i] = kk;
    lo = min(lo, kk);
    hi = max(hi, kk);
  }
  __syncthreads();
  wg_topk<1024, 2048>([&](int i) { return skeys[i]; }, n, K, emit, sm, true, lo, hi, skeys + n, cand_cap);
  __syncthreads();
  // start[h] = number of chosen indices below h * P (tb is ascending)
  if (int(threadIdx.x) <= Hkv) {
    const int target = int(threadIdx.x) * P;
    int lo = 0, hi = K;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (tb[mid] < target) lo = mid + 1; else hi = mid;
    }
    start[threadIdx.x] = lo;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < K; r += 1024) {
    const int i = tb[r];
    const int h = i / P;
    kept[(size_t(b) * Hkv + h) * kept_stride + (r - start[h])] = i - h * P;
  }
  for (int e = threadIdx.x; e < Hkv * W; e += 1024) {
    const int h = e / W, w = e % W;
    const int cnt = start[h + 1] - start[h];
    kept[(size_t(b) * Hkv + h) * kept_stride + cnt + w] = P + w;
    if (w == 0) counts[size_t(b) * Hkv + h] = cnt + W;
  }
}

// kept rows are kept_stride apart; with lens, unit u keeps lens[u] rows
// (Ada-KV budgets), else n_keep.
template <typename T, int D>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ k,
                                                     const T* __restrict__ v, int64_t kv_cap,
                                                     const int32_t* __restrict__ kept,
                                                     int n_keep_max, T* __restrict__ k_out,
                                                     T* __restrict__ v_out, int64_t out_cap,
                                                     int kept_stride,
                                                     const int32_t* __restrict__ lens) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int CPR = D / EPL;
  constexpr int RPP = 256 / CPR;  // rows per pass
  static_assert(64 % RPP == 0, "rows per workgroup");
  const int u = blockIdx.y;
  const int n0 = blockIdx.x * 64;
  const int ch = threadIdx.x % CPR;
  const int* ku = kept + size_t(u) * kept_stride;
  const int n_keep = lens ? min(lens[u], n_keep_max) : n_keep_max;
  // the workgroup's 64 rows: every index, then every K and V load, in flight
  // before any is used
  constexpr int NI = 64 / RPP;
  using R = decltype(Vec16<T>::raw);
  int src_row[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int n = n0 + threadIdx.x / CPR + i * RPP;
    src_row[i] = n < n_keep ? ku[n] : 0;
  }
  // rows past n_keep read the unit's row 0 (in bounds) and are dropped
  Vec16<T> kr[NI], vr[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const size_t src = (size_t(u) * size_t(kv_cap) + size_t(src_row[i])) * D + ch * EPL;
    kr[i] = load16(k + src);
    vr[i] = load16(v + src);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int n = n0 + threadIdx.x / CPR + i * RPP;
    if (n < n_keep) {
      const size_t dst = (size_t(u) * size_t(out_cap) + size_t(n)) * D + ch * EPL;
      *reinterpret_cast<R*>(k_out + dst) = kr[i].raw;
      *reinterpret_cast<R*>(v_out + dst) = vr[i].raw;
    }
  }
}

// The same compaction + aux for launches with many pages: one 512-thread
// workgroup per 32 pages (256-byte rows), each thread one 16-byte chunk of one
// page for all of the page's rows, read eight at a time (indices, then all
// K and V loads in flight; a short page repeats its last row for max/min and
// skips its store).  No row-group merge is needed, and each channel's aux run
// is a whole 64-byte line instead of 8 bytes (short runs are written back as
// partial lines, which the counters showed as ~20 % extra write traffic).
constexpr int kGatherWideThreads = 512;
template <typename T, int D>
__global__ __launch_bounds__(kGatherWideThreads, 4) void gather_aux_wide_kernel(
    const T* __restrict__ k, const T* __restrict__ v, int64_t kv_cap,
    const int32_t* __restrict__ kept, int n_keep_max, T* __restrict__ k_out, T* __restrict__ v_out,
    int64_t out_cap, int block, T* __restrict__ kmax, T* __restrict__ kmin, int64_t nblk_cap,
    int kept_stride, const int32_t* __restrict__ lens) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int CPR = D / EPL;
  constexpr int PPW = kGatherWideThreads / CPR;
  constexpr int RB = 8;
  static_assert(kGatherWideThreads % CPR == 0, "workgroup shape");
  __shared__ T smax[D][PPW + 1];
  __shared__ T smin[D][PPW + 1];
  const int t = threadIdx.x;
  const int c = t % CPR;
  const int j = t / CPR;
  const int u = blockIdx.y;
  const int n_keep = lens ? min(lens[u], n_keep_max) : n_keep_max;
  const int nblk = (n_keep + block - 1) / block;
  const int p0 = blockIdx.x * PPW;
  const int p = p0 + j;
  if (p < nblk) {
    const int n0 = p * block;
    const int n1 = min(n0 + block, n_keep);
    const int* ku = kept + size_t(u) * kept_stride;
    float mx[EPL], mn[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      mx[e] = -INFINITY;
      mn[e] = INFINITY;
    }
    for (int b0 = n0; b0 < n1; b0 += RB) {
      int src[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) src[i] = ku[min(b0 + i, n1 - 1)];
      Vec16<T> kr[RB], vr[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const size_t a = (size_t(u) * size_t(kv_cap) + size_t(src[i])) * D + c * EPL;
        // rows moved once: non-temporal loads and stores (at batch 32,
        // 201 -> 175 us for the copy with its aux; stores alone 184 us)
        kr[i] = load16_nt(k + a);
        vr[i] = load16_nt(v + a);
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (b0 + i < n1) {
          const size_t dst = (size_t(u) * size_t(out_cap) + size_t(b0 + i)) * D + c * EPL;
          store16_nt(k_out + dst, kr[i]);
          store16_nt(v_out + dst, vr[i]);
        }
        float x[EPL];
        unpack16(kr[i], x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          mx[e] = x[e] > mx[e] ? x[e] : mx[e];
          mn[e] = x[e] < mn[e] ? x[e] : mn[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      if constexpr (sizeof(T) == 2) {
        // the values came from bf16, so dropping the low half is exact
        smax[c * EPL + e][j].bits = uint16_t(__float_as_uint(mx[e]) >> 16);
        smin[c * EPL + e][j].bits = uint16_t(__float_as_uint(mn[e]) >> 16);
      } else {
        smax[c * EPL + e][j] = mx[e];
        smin[c * EPL + e][j] = mn[e];
      }
    }
  }
  __syncthreads();
  T* xu = kmax + size_t(u) * D * size_t(nblk_cap);
  T* nu = kmin + size_t(u) * D * size_t(nblk_cap);
  for (int e = t; e < D * PPW; e += kGatherWideThreads) {
    const int ch = e / PPW;
    const int jj = e % PPW;
    if (p0 + jj < nblk) {
      xu[size_t(ch) * nblk_cap + p0 + jj] = smax[ch][jj];
      nu[size_t(ch) * nblk_cap + p0 + jj] = smin[ch][jj];
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 window scoring on the matrix cores (v_mfma_f32_32x32x16_bf16).
//
// A workgroup (4 waves) walks a range of keys of one unit in 128-key tiles.
// Each tile is fetched with fully coalesced 16-byte loads (consecutive
// threads, consecutive bytes) into LDS with a padded row pitch, the next tile
// is prefetched into registers while the current one is multiplied, and the
// waves read their MFMA operand fragments from LDS.  The G*W window rows are
// cut into 32-row groups; a wave keeps its group's Q fragments (32 rows x d,
// bf16) in registers for the whole range.  With fewer than 4 row groups the
// waves split each tile's 32-key chunks instead.  Accumulator lane layout of
// v_mfma_f32_32x32x16_bf16 (verified on gfx950): lane l, element i holds row
// 8*(i/4) + 4*(l/32) + i%4 and column l%32 of the 32x32 product.
//   pass 1: product K_chunk * Q^T, so lane l owns window row l%32 of its group
//           and keeps that row's running (max, sum of exp2) in two registers
//   pass 2: product Q * K_chunk^T, so lane l owns key l%32 and sums
//           exp2(x - m_row - log2 Z_row) (= exp2(x - m_row) / Z_row, one
//           multiply and 16 registers fewer) over its 16 rows; row groups
//           are then added in order -> score
// Registers are held to 128 per lane so four workgroups share a CU (16
// waves): streaming K gains more from the extra resident waves than it
// loses to operand fragments being fetched closer to their use.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int TK = 128;              // keys per LDS tile

__device__ __forceinline__ bf16x8_t load_bf16x8(const bf16_t* p, bool ok) {
  uint4 r = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
  return __builtin_bit_cast(bf16x8_t, r);
}

template <int D, int PASS>
__global__ __launch_bounds__(256, 4) void ws_mfma_kernel(
    const bf16_t* __restrict__ q_win, const bf16_t* __restrict__ k, int64_t kv_cap, int S, int W,
    int G, int n_wg, int keys_per_wg, float scale_log2, float2* __restrict__ partials,
    const float2* __restrict__ stats, float* __restrict__ scores) {
  constexpr int KS = D / 16;
  constexpr int ROWB = D * 2 + 16;         // LDS row pitch in bytes (16 bytes of padding)
  constexpr int VPR = D * 2 / 16;          // 16-byte vectors per key row
  constexpr int LPT = TK * VPR / 256;      // vectors per thread per tile
  static_assert(TK * VPR % 256 == 0, "tile must split evenly over the workgroup");
  __shared__ __align__(16) unsigned char ktile[TK * ROWB];
  extern __shared__ float smem[];  // pass 1: items x 32 float2; pass 2: RG x TK floats
  const int M = G * W;
  const int RG = (M + 31) / 32;
  const int CS = RG >= 4 ? 1 : 4 / RG;  // waves sharing one row group
  const int items = RG * CS;
  // pass 2 walks the units in reverse: workgroups start in launch order, so
  // it begins with the K that pass 1 read last, still in the MALL
  const int u = PASS == 1 ? blockIdx.y : gridDim.y - 1 - blockIdx.y;
  const int wgi = blockIdx.x;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int half = lane >> 5;
  const int P = S - W;
  const int jlim = PASS == 1 ? S : P;
  const int kb = wgi * keys_per_wg;
  const int ke = min(kb + keys_per_wg, jlim);
  const bf16_t* qg = q_win + size_t(u) * M * D;
  const bf16_t* ku = k + size_t(u) * size_t(kv_cap) * D;
  // Wave w owns item w (row group it / CS, chunk class it % CS); the launcher
  // guarantees at most 4 items.  Its Q fragments stay in registers.
  const bool active = wave < items;
  const int rg = wave / CS, cs = wave % CS;
  bf16x8_t a[KS];
  {
    const int arow = rg * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      a[ks] = load_bf16x8(qg + size_t(arow) * D + ks * 16 + half * 8, active && arow < M);
  }
  // pass 1: (max, sum) of this lane's row; pass 2: m + log2 Z of its 16 rows
  // (rows past M get a huge offset, so they add zeros)
  float m1 = kNegBig, z1 = 0.f;
  float m2[16];
  if (PASS == 2 && active) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = rg * 32 + 8 * (i / 4) + 4 * half + (i & 3);
      const float2 st = row < M ? stats[size_t(u) * M + row] : make_float2(1.0e30f, 1.f);
      m2[i] = st.x - __builtin_amdgcn_logf(st.y);  // stats hold (m, 1/Z); logf is log2
    }
  }
  // the Q fragments and row statistics are ready before the tile loop, so its
  // first chunk need not wait for the next tile's loads
  wait_vector_loads();

  uint4 pre[LPT];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int x = 0; x < LPT; ++x) {
      const int vidx = threadIdx.x + 256 * x;
      const int key = t0 + vidx / VPR;
      // streamed once per pass: non-temporal (measured 8-15 % faster for pass 1)
      pre[x] = key < ke ? load_u4_nt(reinterpret_cast<const uint4*>(ku + size_t(key) * D) + vidx % VPR)
                        : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int x = 0; x < LPT; ++x) {
      const int vidx = threadIdx.x + 256 * x;
      *reinterpret_cast<uint4*>(ktile + (vidx / VPR) * ROWB + (vidx % VPR) * 16) = pre[x];
    }
  };
  if (kb < ke) {
    fetch(kb);
    stash();
  }
  __syncthreads();
  for (int t0 = kb; t0 < ke; t0 += TK) {
    const bool next = t0 + TK < ke;
    if (next) fetch(t0 + TK);             // in flight while this tile is multiplied
    const int nch = (min(t0 + TK, ke) - t0 + 31) / 32;
    if (active) {
      const int row1 = rg * 32 + (lane & 31);
      const int lim1 = S - W + (row1 % W);   // last key row1 may see
      for (int c = cs; c < nch; c += CS) {
        const unsigned char* fr = ktile + (c * 32 + (lane & 31)) * ROWB + half * 16;
        bf16x8_t b[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) b[ks] = *reinterpret_cast<const bf16x8_t*>(fr + ks * 32);
        f32x16_t acc = {};
        if (PASS == 1) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[ks], a[ks], acc, 0, 0, 0);
          if (t0 + c * 32 + 32 <= S - W) {
            // every key of the chunk is visible to every window row
            float cm = acc[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) cm = fmaxf(cm, acc[i]);
            const float mn = fmaxf(m1, cm * scale_log2);
            float zz = z1 * fast_exp2(m1 - mn);
#pragma unroll
            for (int i = 0; i < 16; ++i) zz += fast_exp2(fmaf(acc[i], scale_log2, -mn));
            z1 = zz;
            m1 = mn;
          } else {
            // causal window / past S: masked without branches
            const int kbase = t0 + c * 32 + 4 * half;  // key of element i: kbase + 8*(i/4) + i%4
            bool ok[16];
            float cm = kNegBig;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kbase + 8 * (i / 4) + (i & 3);
              ok[i] = key < S && key <= lim1;
              cm = fmaxf(cm, ok[i] ? acc[i] : kNegBig);
            }
            const float mn = fmaxf(m1, cm * scale_log2);
            float zz = z1 * fast_exp2(m1 - mn);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float e = fast_exp2(fmaf(acc[i], scale_log2, -mn));
              zz += ok[i] ? e : 0.f;
            }
            z1 = zz;
            m1 = mn;
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], b[ks], acc, 0, 0, 0);
          float cs_sum = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) cs_sum += fast_exp2(fmaf(acc[i], scale_log2, -m2[i]));
          cs_sum += __shfl_xor(cs_sum, 32);
          if (lane < 32) smem[rg * TK + c * 32 + lane] = cs_sum;
        }
      }
    }
    __syncthreads();
    // the next tile goes to LDS first: the score stores below must not sit
    // in front of the wait for its loads
    if (next) stash();
    if (PASS == 2) {
      for (int cidx = threadIdx.x; cidx < TK; cidx += 256) {
        const int j = t0 + cidx;
        if (j >= ke) continue;
        float sacc = 0.f;
        for (int rg = 0; rg < RG; ++rg) sacc += smem[rg * TK + cidx];
        scores[size_t(u) * P + j] = sacc;
      }
    }
    __syncthreads();
  }
  if (PASS == 1) {
    if (wave < items) {
      // the two half-waves hold disjoint keys of the same 32 rows
      const float mo = __shfl_xor(m1, 32);
      const float zo = __shfl_xor(z1, 32);
      const float mn = fmaxf(m1, mo);
      const float zz = (lane < 32) ? z1 * fast_exp2(m1 - mn) + zo * fast_exp2(mo - mn)
                                   : zo * fast_exp2(mo - mn) + z1 * fast_exp2(m1 - mn);
      if (lane < 32) reinterpret_cast<float2*>(smem)[wave * 32 + lane] = make_float2(mn, zz);
    }
    __syncthreads();
    const float2* mz = reinterpret_cast<const float2*>(smem);
    for (int r = threadIdx.x; r < RG * 32; r += 256) {
      if (r >= M) continue;
      const int rg = r / 32, rl = r % 32;
      float mm = kNegBig, zz = 0.f;
      for (int c = 0; c < CS; ++c) {  // column splits in order
        const float2 pz = mz[(rg * CS + c) * 32 + rl];
        const float mn = fmaxf(mm, pz.x);
        zz = zz * fast_exp2(mm - mn) + pz.y * fast_exp2(pz.x - mn);
        mm = mn;
      }
      partials[(size_t(u) * n_wg + wgi) * M + r] = make_float2(mm, zz);
    }
  }
}

// Compaction with the HSA step-1 aux built on the way (the compact K is not
// read again).  One workgroup per (PPW pages, unit): a page's rows are split
// over RG row groups of CPR threads (one 16-byte chunk of a row each), which
// copy their rows of K and V and keep running max/min; the groups merge
// through LDS and the workgroup writes its pages' Kmax/Kmin channel-major.
// Exact: max/min only.
template <typename T, int D>
__global__ __launch_bounds__(256) void gather_aux_kernel(
    const T* __restrict__ k, const T* __restrict__ v, int64_t kv_cap,
    const int32_t* __restrict__ kept, int n_keep_max, T* __restrict__ k_out, T* __restrict__ v_out,
    int64_t out_cap, int block, T* __restrict__ kmax, T* __restrict__ kmin, int64_t nblk_cap,
    int kept_stride, const int32_t* __restrict__ lens) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int CPR = D / EPL;
  constexpr int RG = 4;
  constexpr int PPW = 256 / (CPR * RG);
  static_assert(PPW >= 1 && 256 % (CPR * RG) == 0, "workgroup shape");
  __shared__ float smx[PPW][RG][D];
  __shared__ float smn[PPW][RG][D];
  const int t = threadIdx.x;
  const int c = t % CPR;
  const int g = (t / CPR) % RG;
  const int j = t / (CPR * RG);
  const int u = blockIdx.y;
  const int n_keep = lens ? min(lens[u], n_keep_max) : n_keep_max;
  const int nblk = (n_keep + block - 1) / block;
  const int p0 = blockIdx.x * PPW;
  const int p = p0 + j;
  float mx[EPL], mn[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    mx[e] = -INFINITY;
    mn[e] = INFINITY;
  }
  if (p < nblk) {
    const int n1 = min((p + 1) * block, n_keep);
    const int* ku = kept + size_t(u) * kept_stride;
    using Rw = decltype(Vec16<T>::raw);
    // NI rows per round: all their indices, then all their K and V loads,
    // are in flight before any is used (the index -> row chain is the latency)
    constexpr int NI = 4;
    for (int n0 = p * block + g; n0 < n1; n0 += NI * RG) {
      int src_row[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) src_row[i] = n0 + i * RG < n1 ? ku[n0 + i * RG] : 0;
      // rows past the page read the unit's row 0 (in bounds) and are dropped
      Vec16<T> kr[NI], vr[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const size_t src = (size_t(u) * size_t(kv_cap) + size_t(src_row[i])) * D + c * EPL;
        kr[i] = load16(k + src);
        vr[i] = load16(v + src);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int n = n0 + i * RG;
        if (n < n1) {
          const size_t dst = (size_t(u) * size_t(out_cap) + size_t(n)) * D + c * EPL;
          *reinterpret_cast<Rw*>(k_out + dst) = kr[i].raw;
          *reinterpret_cast<Rw*>(v_out + dst) = vr[i].raw;
          float x[EPL];
          unpack16(kr[i], x);
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            mx[e] = x[e] > mx[e] ? x[e] : mx[e];
            mn[e] = x[e] < mn[e] ? x[e] : mn[e];
          }
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    smx[j][g][c * EPL + e] = mx[e];
    smn[j][g][c * EPL + e] = mn[e];
  }
  __syncthreads();
  T* xu = kmax + size_t(u) * D * size_t(nblk_cap);
  T* nu = kmin + size_t(u) * D * size_t(nblk_cap);
  for (int e = t; e < D * PPW; e += 256) {
    const int ch = e / PPW;
    const int jj = e % PPW;
    if (p0 + jj < nblk) {
      float a = smx[jj][0][ch], b = smn[jj][0][ch];
#pragma unroll
      for (int gg = 1; gg < RG; ++gg) {
        const float x = smx[jj][gg][ch], y = smn[jj][gg][ch];
        a = x > a ? x : a;
        b = y < b ? y : b;
      }
      if constexpr (sizeof(T) == 2) {
        // the values came from bf16, so dropping the low half is exact
        xu[size_t(ch) * nblk_cap + p0 + jj].bits = uint16_t(__float_as_uint(a) >> 16);
        nu[size_t(ch) * nblk_cap + p0 + jj].bits = uint16_t(__float_as_uint(b) >> 16);
      } else {
        xu[size_t(ch) * nblk_cap + p0 + jj] = a;
        nu[size_t(ch) * nblk_cap + p0 + jj] = b;
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_evict_t(const Dims& d, const void* q_win, const void* k, const void* v,
                          int64_t kv_cap, int64_t S64, int W, int pool_kernel, int pool_op,
                          int64_t n_keep, int32_t* kept, void* k_out, void* v_out, int64_t out_cap,
                          float* pooled_opt, void* kmax, void* kmin, int64_t nblk_cap, int block,
                          void* ws, hipStream_t s, int32_t* ada_counts) {
  const int S = int(S64);
  const int P = S - W;
  // Ada-KV budgets: kept rows are out_cap apart and unit u keeps
  // ada_counts[u] of them (at most n_rows), else every unit keeps n_keep
  const bool ada = ada_counts != nullptr;
  const int kept_stride = ada ? int(out_cap) : int(n_keep);
  const int n_rows = ada ? int(std::min<int64_t>(S64, int64_t(d.Hkv) * (n_keep - W) + W)) : int(n_keep);
  const EvictWs lay = evict_ws_layout(d, S64, W);
  char* wsb = static_cast<char*>(ws);
  float2* partials = reinterpret_cast<float2*>(wsb + lay.partials);
  float2* stats = reinterpret_cast<float2*>(wsb + lay.stats);
  float* scores = reinterpret_cast<float*>(wsb + lay.scores);
  float* pooled = pooled_opt ? pooled_opt : reinterpret_cast<float*>(wsb + lay.pooled);
  const int units = d.units();
  const int M = d.G * W;
  const float scale_log2 = float(1.4426950408889634 / sqrt(double(D)));
  const T* qw = static_cast<const T*>(q_win);
  const T* kk = static_cast<const T*>(k);

  // bf16 on the matrix cores when G*W fits 4 waves of 32-row groups (one
  // group per wave), otherwise (and for float32) on the vector ALUs
  constexpr bool kBf16 = sizeof(T) == 2;
  const bool mfma = kBf16 && M <= 128;
  const int RG = (M + 31) / 32;
  const int CS = RG >= 4 ? 1 : 4 / RG;
  // keys per workgroup: about 8192 workgroups per pass (8 per CU slot; at
  // batch 32, 2048 measured 8 % slower and 16384 slower again), in whole
  // 128-key tiles, but at least 4 tiles, so each workgroup's window-row fetch
  // is spread over a streamed run of K (at batch 1, with non-temporal tile
  // loads, four-tile workgroups measured 1 % (32K prompt) and 3-5 % (109K
  // prompt) faster for the whole eviction than two-tile ones, eight-tile
  // ones 1-5 % slower).  Splitting the passes over unit chunks small enough
  // for the second pass to re-read K from the MALL measured slower: the
  // smaller launches lose more than the re-read gains.
  auto range = [&](int keys) {
    const int wpu = (8192 + units - 1) / units;
    int kpw = (keys + wpu - 1) / wpu;
    kpw = (kpw + TK - 1) / TK * TK;
    return kpw < 4 * TK ? 4 * TK : kpw;
  };
  const int kpw1 = range(S);
  const int n_wg1 = mfma ? (S + kpw1 - 1) / kpw1 : lay.n_tiles;
  const int n_tiles = n_wg1;
  const size_t lds1 = size_t(RG * CS) * 32 * sizeof(float2);
  const size_t lds2 = size_t(RG) * TK * sizeof(float);
  if (mfma) {
    RK_LAUNCH("ws_pass1", (ws_mfma_kernel<D, 1>), dim3(n_wg1, units), dim3(256), lds1, s,
              reinterpret_cast<const bf16_t*>(qw), reinterpret_cast<const bf16_t*>(kk), kv_cap, S,
              W, d.G, n_wg1, kpw1, scale_log2, partials, nullptr, nullptr);
  } else {
    RK_LAUNCH("ws_pass1", (ws_pass1_kernel<T, D>), dim3(n_tiles, units), dim3(256), 0, s, qw, kk,
              kv_cap, S, W, d.G, n_tiles, scale_log2, partials);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  RK_LAUNCH("ws_stats", ws_stats_kernel, dim3((units * M + 63) / 64), dim3(1024), 0, s, partials, M,
            n_tiles, units, stats);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (P > 0) {
    if (mfma) {
      const int kpw2 = range(P);
      RK_LAUNCH("ws_pass2", (ws_mfma_kernel<D, 2>), dim3((P + kpw2 - 1) / kpw2, units), dim3(256),
                lds2, s, reinterpret_cast<const bf16_t*>(qw), reinterpret_cast<const bf16_t*>(kk),
                kv_cap, S, W, d.G, 0, kpw2, scale_log2, nullptr, stats, scores);
    } else {
      RK_LAUNCH("ws_pass2", (ws_pass2_kernel<T, D>), dim3((P + TN - 1) / TN, units), dim3(256), 0,
                s, qw, kk, kv_cap, S, W, d.G, scale_log2, stats, scores);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  static bool attr_set = false;
  if (!attr_set) {
    for (const void* f : {reinterpret_cast<const void*>(&select_kernel),
                          reinterpret_cast<const void*>(&select_pool_kernel<31>),
                          reinterpret_cast<const void*>(&select_pool_kernel<31, true>),
                          reinterpret_cast<const void*>(&select_chunk_kernel),
                          reinterpret_cast<const void*>(&select_final_kernel),
                          reinterpret_cast<const void*>(&adakv_select_kernel)}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         int(kSelectKeysLds));
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  const int h = (pool_kernel - 1) / 2;
  const bool mx = pool_op == 1;  // max pooling (else sums)
  // the pooling launch of the paths that pool separately
  auto pool = [&]() {
    if (h == 31) {
      if (mx)
        RK_LAUNCH("pool_sum", (pool_sum_reg_kernel<31, true>), dim3((P + 2047) / 2048, units), dim3(256), 0,
                  s, scores, P, pooled);
      else
        RK_LAUNCH("pool_sum", pool_sum_reg_kernel<31>, dim3((P + 2047) / 2048, units), dim3(256), 0, s,
                  scores, P, pooled);
    } else {
      if (mx)
        RK_LAUNCH("pool_sum", pool_sum_kernel<true>, dim3((P + 255) / 256, units), dim3(256),
                  size_t(256 + 2 * h) * sizeof(float), s, scores, P, h, pooled);
      else
        RK_LAUNCH("pool_sum", pool_sum_kernel<false>, dim3((P + 255) / 256, units), dim3(256),
                  size_t(256 + 2 * h) * sizeof(float), s, scores, P, h, pooled);
    }
  };
  if (ada) {
    // pooling of every unit first (the shared choice reads all heads of a
    // sequence), then the shared choice: one workgroup per sequence when
    // its keys fit in LDS (the spent window scores hold its chosen flattened
    // indices), else the radix select over many workgroups
    if (P > 0) {
      pool();
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const size_t nkeys = size_t(d.Hkv) * P;
    if ((nkeys + 4096) * 4 <= kSelectKeysLds) {
      RK_LAUNCH("select_tokens", adakv_select_kernel, dim3(d.B), dim3(1024), (nkeys + 4096) * 4, s,
                pooled, d.Hkv, P, W, int(n_keep) - W, 4096, reinterpret_cast<int32_t*>(scores), kept,
                kept_stride, ada_counts);
    } else {
      // more keys than one workgroup's LDS: the radix select spread over
      // many workgroups (one workgroup per sequence took 645 us at batch 1 x
      // 8 heads x 32K keys).  Its histograms, cuts and chunk counts live in
      // the spent window-score region: B * 24 KB + units * P / 512 bytes,
      // well below its units * P * 4 bytes (over 137 KB per sequence here).
      const int n = int(nkeys);
      const int K = d.Hkv * (int(n_keep) - W);
      const int nchunk = (P + kAdaEmitChunk - 1) / kAdaEmitChunk;
      uint32_t* hist = reinterpret_cast<uint32_t*>(scores);  // [3][B][kAdaBins]
      AdaCut* cutp = reinterpret_cast<AdaCut*>(hist + size_t(3) * d.B * kAdaBins);
      int2* cntp = reinterpret_cast<int2*>(cutp + d.B);
      const size_t ws_need = size_t(3) * d.B * kAdaBins * 4 + size_t(d.B) * sizeof(AdaCut) +
                             size_t(units) * nchunk * sizeof(int2);
      if (ws_need > size_t(units) * P * sizeof(float)) return hipErrorInvalidValue;
      const int mode = K <= 0 ? -1 : K >= n ? 1 : 0;
      if (mode == 0) {
        const int words = 3 * d.B * kAdaBins;
        RK_LAUNCH("select_tokens", ada_clear_kernel, dim3((words + 255) / 256), dim3(256), 0, s, hist, words);
        for (int pass = 0; pass < 3; ++pass)
          RK_LAUNCH("select_tokens", ada_hist_kernel, dim3((n + kAdaChunk - 1) / kAdaChunk, d.B), dim3(1024),
                    0, s, pooled, d.B, n, pass, K, hist);
        RK_LAUNCH("select_tokens", ada_count_kernel,
                  dim3((nchunk + kAdaCountChunks - 1) / kAdaCountChunks, units), dim3(1024), 0, s, pooled,
                  d.B, d.Hkv, P, nchunk, K, hist, cutp, cntp);
      }
      RK_LAUNCH("select_tokens", ada_emit_kernel, dim3(nchunk, units), dim3(256), 0, s, pooled, d.Hkv, P, W,
                nchunk, mode, cutp, cntp, kept, kept_stride, ada_counts);
    }
  } else {
  // kernel 63 with the haloed scores in LDS and enough units to spread the
  // pooling over the CUs: pooling inside the select launch (at batch 32,
  // 49 -> 41 us for both; at batch 1 the 8 workgroups' LDS reads of the
  // pooling windows cost more than the separate launch, 30 -> 36 us)
  constexpr int kPoolH = 31;
  const size_t pool_words = size_t((P + 7) / 8 * 8 + 2 * kPoolH + 8);
  if (P > 0 && h == kPoolH && pool_words * 4 <= kSelectKeysLds && units >= kComputeUnits / 4) {
    const size_t words = std::max(pool_words, size_t(P) + 4096);
    const int cand_cap = int(std::min<size_t>(4096, kSelectKeysLds / 4 - size_t(P)));
    if (mx)
      RK_LAUNCH("select_tokens", (select_pool_kernel<kPoolH, true>), dim3(units), dim3(1024),
                std::min(words, kSelectKeysLds / 4) * 4, s, scores, S, W, int(n_keep), cand_cap,
                pooled_opt, kept);
    else
      RK_LAUNCH("select_tokens", select_pool_kernel<kPoolH>, dim3(units), dim3(1024),
                std::min(words, kSelectKeysLds / 4) * 4, s, scores, S, W, int(n_keep), cand_cap,
                pooled_opt, kept);
  } else {
    if (P > 0) {
      pool();
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const int staged = size_t(P) * 4 <= kSelectKeysLds ? 1 : 0;
    // more keys than LDS holds: chunked select when the candidates of all
    // chunks (positions and keys) fit in LDS, else the global-key path
    const int C = int(kSelectKeysLds / 4) / 64 * 64;
    const int k_sel = int(n_keep) - W;
    const int n_chunks = (P + C - 1) / C;
    int n_cand = 0;
    for (int c = 0; c < n_chunks; ++c) n_cand += std::min(std::min(k_sel, C), P - c * C);
    if (!staged && size_t(n_cand) * 8 <= kSelectKeysLds) {
      int32_t* cand = reinterpret_cast<int32_t*>(scores);  // the scores are spent once pooled
      RK_LAUNCH("select_chunk", select_chunk_kernel, dim3(n_chunks, units), dim3(1024),
                size_t(C) * 4, s, pooled, P, C, k_sel, cand);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      RK_LAUNCH("select_tokens", select_final_kernel, dim3(units), dim3(1024), size_t(n_cand) * 8,
                s, pooled, S, W, C, int(n_keep), cand, kept);
    } else {
      // staged keys, then up to 4096 words of radix candidates in what LDS is left
      const int cand_cap =
          staged ? int(std::min<size_t>(4096, (kSelectKeysLds - size_t(P) * 4) / 4)) : 0;
      RK_LAUNCH("select_tokens", select_kernel, dim3(units), dim3(1024),
                staged ? size_t(P + cand_cap) * 4 : size_t(0), s, pooled, S, W, int(n_keep), staged,
                cand_cap, kept);
    }
  }
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int32_t* lens = ada ? ada_counts : nullptr;
  if (k_out && kmax) {
    // wide workgroups (whole-line aux runs) unless they would leave most CUs
    // idle: at batch 1 with 32K keys (152 of them) they measured as fast as
    // the 4-page form, and twice as fast with 3-token pages; the 109K needle
    // (8 of them) keeps 4-page workgroups, which spread its copy over more CUs
    constexpr int PPW = 256 / ((D / Vec16<T>::N) * 4);
    constexpr int PPW_WIDE = kGatherWideThreads / (D / Vec16<T>::N);
    const int64_t nblk = (n_rows + block - 1) / block;
    const int64_t wide_wgs = (nblk + PPW_WIDE - 1) / PPW_WIDE * units;
    if (wide_wgs >= kComputeUnits / 4)
      RK_LAUNCH("gather_kv", (gather_aux_wide_kernel<T, D>),
                dim3(unsigned((nblk + PPW_WIDE - 1) / PPW_WIDE), units), dim3(kGatherWideThreads),
                0, s, kk, static_cast<const T*>(v), kv_cap, kept, n_rows,
                static_cast<T*>(k_out), static_cast<T*>(v_out), out_cap, block,
                static_cast<T*>(kmax), static_cast<T*>(kmin), nblk_cap, kept_stride, lens);
    else
      RK_LAUNCH("gather_kv", (gather_aux_kernel<T, D>), dim3(unsigned((nblk + PPW - 1) / PPW), units),
                dim3(256), 0, s, kk, static_cast<const T*>(v), kv_cap, kept, n_rows,
                static_cast<T*>(k_out), static_cast<T*>(v_out), out_cap, block,
                static_cast<T*>(kmax), static_cast<T*>(kmin), nblk_cap, kept_stride, lens);
    err = hipGetLastError();
  } else if (k_out) {
    RK_LAUNCH("gather_kv", (gather_kernel<T, D>), dim3(unsigned((n_rows + 63) / 64), units),
                       dim3(256), 0, s, kk, static_cast<const T*>(v), kv_cap, kept, n_rows,
                       static_cast<T*>(k_out), static_cast<T*>(v_out), out_cap, kept_stride, lens);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace

hipError_t launch_snapkv_evict(const Dims& d, const void* q_win, const void* k, const void* v,
                               int64_t kv_cap, int64_t S, int W, int pool_kernel, int pool_op,
                               int64_t n_keep, int32_t* kept, void* k_out, void* v_out,
                               int64_t out_cap, float* pooled_opt, void* kmax, void* kmin,
                               int64_t nblk_cap, int block, void* ws, hipStream_t s,
                               int32_t* ada_counts) {
#define RK_EVICT(TT, DD)                                                                  \
  return launch_evict_t<TT, DD>(d, q_win, k, v, kv_cap, S, W, pool_kernel, pool_op, n_keep, \
                                kept, k_out, v_out, out_cap, pooled_opt, kmax, kmin,        \
                                nblk_cap, block, ws, s, ada_counts)
  if (d.bf16) {
    if (d.D == 128) RK_EVICT(bf16_t, 128);
    RK_EVICT(bf16_t, 64);
  }
  if (d.D == 128) RK_EVICT(float, 128);
  RK_EVICT(float, 64);
#undef RK_EVICT
}

}  // namespace rk

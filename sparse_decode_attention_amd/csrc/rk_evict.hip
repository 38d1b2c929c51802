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
//   ws_pass1   logits of the group's G*W window rows against a 64-key tile,
//              causal on the window keys; per row, the tile's max and sum of
//              exp2 (log2 domain) -> partials
//   ws_stats   merge the tile partials of each row in tile order -> (m, 1/Z)
//   ws_pass2   recompute the prefix logits, p = exp2(x - m) / Z, sum over the
//              G*W rows in a fixed order -> score[j], j < S-W
//   pool       windowed sum of width pool_kernel, left to right -> pooled
//   select     workgroup radix top-k (ties to the lower position) + window
//   gather     compaction of K and V rows (skipped for the RocketKV-MT form)
#include <math.h>

#include "rk_device.hpp"
#include "rk_internal.hpp"

namespace rk {
namespace {

constexpr float kNegBig = -1.0e30f;
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
      if (j < S && j <= lim) z += exp2f(Ls[row][col] - mx);
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) z += __shfl_xor(z, off);
    if (part == 0 && r_all < M) partials[(size_t(u) * n_tiles + tile) * M + r_all] = make_float2(mx, z);
    __syncthreads();
  }
}

// Merge the tile partials of every row, in tile order: (m, 1/Z).
__global__ __launch_bounds__(256) void ws_stats_kernel(const float2* __restrict__ partials,
                                                       int M, int n_tiles,
                                                       float2* __restrict__ stats) {
  const int u = blockIdx.y;
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= M) return;
  const float2* pu = partials + size_t(u) * n_tiles * M + row;
  float mm = kNegBig;
  for (int t = 0; t < n_tiles; ++t) mm = fmaxf(mm, pu[size_t(t) * M].x);
  float z = 0.f;
  for (int t = 0; t < n_tiles; ++t) {
    const float2 p = pu[size_t(t) * M];
    z += p.y * exp2f(p.x - mm);
  }
  stats[size_t(u) * M + row] = make_float2(mm, 1.0f / z);
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
        s += exp2f(Ls[part * 8 + i][col] - mz.x) * mz.y;
      }
    }
    red[part][col] = s;
    __syncthreads();
    if (part == 0) total += ((red[0][col] + red[1][col]) + red[2][col]) + red[3][col];
    __syncthreads();
  }
  if (part == 0 && j0 + col < P) scores[size_t(u) * P + j0 + col] = total;
}

// pooled[j] = sum_{i=j-h}^{j+h} score[i] (zero outside [0, P)), left to right.
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
    if (src >= 0 && src < P) acc = __fadd_rn(acc, tile[threadIdx.x + i]);
  }
  pooled[size_t(u) * P + j] = acc;
}

// Top (n_keep - W) prefix positions by pooled score, ascending, then the window.
__global__ __launch_bounds__(1024) void select_kernel(const float* __restrict__ pooled, int S,
                                                      int W, int n_keep,
                                                      int32_t* __restrict__ kept) {
  __shared__ TopkSmem<1024> sm;
  const int u = blockIdx.x;
  const int P = S - W;
  const float* pu = pooled + size_t(u) * P;
  int32_t* ku = kept + size_t(u) * n_keep;
  wg_topk<1024>([&](int i) { return order_key(pu[i]); }, P, n_keep - W,
                [&](int r, int i) { ku[r] = i; }, sm);
  for (int r = threadIdx.x; r < W; r += 1024) ku[n_keep - W + r] = P + r;
}

// Compact cache rows: out[n] = in[kept[n]] for K and V.
template <typename T, int D>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ k,
                                                     const T* __restrict__ v, int64_t kv_cap,
                                                     const int32_t* __restrict__ kept,
                                                     int n_keep, T* __restrict__ k_out,
                                                     T* __restrict__ v_out, int64_t out_cap) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int CPR = D / EPL;
  constexpr int RPP = 256 / CPR;  // rows per pass
  const int u = blockIdx.y;
  const int n0 = blockIdx.x * 64;
  const int ch = threadIdx.x % CPR;
  const int* ku = kept + size_t(u) * n_keep;
  for (int rr = threadIdx.x / CPR; rr < 64; rr += RPP) {
    const int n = n0 + rr;
    if (n >= n_keep) break;
    const size_t src = (size_t(u) * size_t(kv_cap) + size_t(ku[n])) * D + ch * EPL;
    const size_t dst = (size_t(u) * size_t(out_cap) + size_t(n)) * D + ch * EPL;
    using R = decltype(Vec16<T>::raw);
    *reinterpret_cast<R*>(k_out + dst) = *reinterpret_cast<const R*>(k + src);
    *reinterpret_cast<R*>(v_out + dst) = *reinterpret_cast<const R*>(v + src);
  }
}

template <typename T, int D>
hipError_t launch_evict_t(const Dims& d, const void* q_win, const void* k, const void* v,
                          int64_t kv_cap, int64_t S64, int W, int pool_kernel, int64_t n_keep,
                          int32_t* kept, void* k_out, void* v_out, int64_t out_cap,
                          float* pooled_opt, void* ws, hipStream_t s) {
  const int S = int(S64);
  const int P = S - W;
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

  hipLaunchKernelGGL((ws_pass1_kernel<T, D>), dim3(lay.n_tiles, units), dim3(256), 0, s, qw, kk,
                     kv_cap, S, W, d.G, lay.n_tiles, scale_log2, partials);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(ws_stats_kernel, dim3((M + 255) / 256, units), dim3(256), 0, s, partials, M,
                     lay.n_tiles, stats);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (P > 0) {
    hipLaunchKernelGGL((ws_pass2_kernel<T, D>), dim3((P + TN - 1) / TN, units), dim3(256), 0, s,
                       qw, kk, kv_cap, S, W, d.G, scale_log2, stats, scores);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int h = (pool_kernel - 1) / 2;
    hipLaunchKernelGGL(pool_sum_kernel, dim3((P + 255) / 256, units), dim3(256),
                       size_t(256 + 2 * h) * sizeof(float), s, scores, P, h, pooled);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(select_kernel, dim3(units), dim3(1024), 0, s, pooled, S, W, int(n_keep),
                     kept);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (k_out) {
    hipLaunchKernelGGL((gather_kernel<T, D>), dim3(unsigned((n_keep + 63) / 64), units),
                       dim3(256), 0, s, kk, static_cast<const T*>(v), kv_cap, kept, int(n_keep),
                       static_cast<T*>(k_out), static_cast<T*>(v_out), out_cap);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace

hipError_t launch_snapkv_evict(const Dims& d, const void* q_win, const void* k, const void* v,
                               int64_t kv_cap, int64_t S, int W, int pool_kernel,
                               int64_t n_keep, int32_t* kept, void* k_out, void* v_out,
                               int64_t out_cap, float* pooled_opt, void* ws, hipStream_t s) {
  if (d.bf16) {
    if (d.D == 128)
      return launch_evict_t<bf16_t, 128>(d, q_win, k, v, kv_cap, S, W, pool_kernel, n_keep,
                                         kept, k_out, v_out, out_cap, pooled_opt, ws, s);
    return launch_evict_t<bf16_t, 64>(d, q_win, k, v, kv_cap, S, W, pool_kernel, n_keep, kept,
                                      k_out, v_out, out_cap, pooled_opt, ws, s);
  }
  if (d.D == 128)
    return launch_evict_t<float, 128>(d, q_win, k, v, kv_cap, S, W, pool_kernel, n_keep, kept,
                                      k_out, v_out, out_cap, pooled_opt, ws, s);
  return launch_evict_t<float, 64>(d, q_win, k, v, kv_cap, S, W, pool_kernel, n_keep, kept,
                                   k_out, v_out, out_cap, pooled_opt, ws, s);
}

}  // namespace rk

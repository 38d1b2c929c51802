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
    if (part == 0 && r_all < M) partials[(size_t(u) * M + r_all) * n_tiles + tile] = make_float2(mx, z);
    __syncthreads();
  }
}

// Merge the tile partials of every row: (m, 1/Z).  One wave per (unit, row);
// lane l takes tiles l, l+64, ... in order, then a fixed butterfly merges lanes.
__global__ __launch_bounds__(256) void ws_stats_kernel(const float2* __restrict__ partials,
                                                       int M, int n_tiles, int units,
                                                       float2* __restrict__ stats) {
  const int wi = blockIdx.x * 4 + threadIdx.x / kWave;
  if (wi >= units * M) return;
  const int lane = lane_id();
  const float2* pr = partials + size_t(wi) * n_tiles;
  float mm = kNegBig;
  for (int t = lane; t < n_tiles; t += kWave) mm = fmaxf(mm, pr[t].x);
  mm = wave_max(mm);
  float z = 0.f;
  for (int t = lane; t < n_tiles; t += kWave) {
    const float2 p = pr[t];
    z += p.y * exp2f(p.x - mm);
  }
  z = wave_sum(z);
  if (lane == 0) stats[wi] = make_float2(mm, 1.0f / z);
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
// When the P = S - W keys fit, they are converted to order keys once and held
// in LDS (dynamic, P words) for all radix passes and the compaction.
__global__ __launch_bounds__(1024) void select_kernel(const float* __restrict__ pooled, int S,
                                                      int W, int n_keep, int staged,
                                                      int32_t* __restrict__ kept) {
  extern __shared__ uint32_t skeys[];
  __shared__ TopkSmem<1024> sm;
  const int u = blockIdx.x;
  const int P = S - W;
  const float* pu = pooled + size_t(u) * P;
  int32_t* ku = kept + size_t(u) * n_keep;
  auto emit = [&](int r, int i) { ku[r] = i; };
  RK_PHASE(0);
  if (staged) {
    // 16-byte loads where the row allows it, all of a thread's loads in flight
    const bool vec = (reinterpret_cast<uintptr_t>(pu) & 15u) == 0;
    const int P4 = vec ? P / 4 : 0;
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
          skeys[4 * i] = order_key(buf[x].x);
          skeys[4 * i + 1] = order_key(buf[x].y);
          skeys[4 * i + 2] = order_key(buf[x].z);
          skeys[4 * i + 3] = order_key(buf[x].w);
        }
      }
    }
    for (int i = 4 * P4 + threadIdx.x; i < P; i += 1024) skeys[i] = order_key(pu[i]);
    __syncthreads();
    wg_topk<1024>([&](int i) { return skeys[i]; }, P, n_keep - W, emit, sm);
  } else {
    wg_topk<1024>([&](int i) { return order_key(pu[i]); }, P, n_keep - W, emit, sm);
  }
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

// ---------------------------------------------------------------------------
// bf16 window scoring on the matrix cores (v_mfma_f32_32x32x16_bf16).
//
// A workgroup (4 waves) owns 256 consecutive keys of one unit.  The G*W window
// rows are cut into 32-row groups; a wave keeps the A operand of its row group
// (32 rows x d, bf16) in registers for the whole tile and streams 32-key
// chunks of K straight from memory as the B operand (each lane fetches 16
// contiguous bytes of one key row), prefetching the next chunk while the
// current one is multiplied.  With fewer than 4 row groups the waves split
// the tile's chunks instead.  Accumulator lane layout (verified on gfx950):
// lane l, element i holds row 8*(i/4) + 4*(l/32) + i%4 of the group and key
// column l%32 of the chunk.
//   pass 1: per row, online max / sum of exp2 over the tile -> partials
//   pass 2: exp2(x - m_row) / Z_row summed over all rows of the group for each
//           key, then over the row groups in order -> score
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int TNM = 256;             // keys per workgroup
constexpr int NCH = TNM / 32;        // 32-key chunks per workgroup

__device__ __forceinline__ bf16x8_t load_bf16x8(const bf16_t* p, bool ok) {
  uint4 r = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
  return __builtin_bit_cast(bf16x8_t, r);
}

template <int D, int PASS>
__global__ __launch_bounds__(256) void ws_mfma_kernel(
    const bf16_t* __restrict__ q_win, const bf16_t* __restrict__ k, int64_t kv_cap, int S, int W,
    int G, int n_tiles, float scale_log2, float2* __restrict__ partials,
    const float2* __restrict__ stats, float* __restrict__ scores) {
  constexpr int KS = D / 16;
  extern __shared__ float smem[];  // pass 1: items x 32 float2; pass 2: RG x TNM floats
  const int M = G * W;
  const int RG = (M + 31) / 32;
  const int CS = RG >= 4 ? 1 : 4 / RG;  // waves sharing one row group
  const int items = RG * CS;
  const int u = blockIdx.y;
  const int tile = blockIdx.x;
  const int j0 = tile * TNM;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int half = lane >> 5;
  const int P = S - W;
  const int jlim = PASS == 1 ? S : P;
  const bf16_t* qg = q_win + size_t(u) * M * D;
  const bf16_t* ku = k + size_t(u) * size_t(kv_cap) * D + half * 8;

  for (int it = wave; it < items; it += 4) {
    const int rg = it / CS;
    const int cs = it % CS;
    bf16x8_t a[KS];
    {
      const int arow = rg * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        a[ks] = load_bf16x8(qg + size_t(arow) * D + ks * 16 + half * 8, arow < M);
    }
    float m[16], z[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = rg * 32 + 8 * (i / 4) + 4 * half + (i & 3);
      if (PASS == 1) {
        m[i] = kNegBig;
        z[i] = 0.f;
      } else {
        const float2 st = row < M ? stats[size_t(u) * M + row] : make_float2(1.0e30f, 0.f);
        m[i] = st.x;  // row max (log2 domain)
        z[i] = st.y;  // 1 / row sum
      }
    }
    int cc = cs;
    int col = j0 + cc * 32 + (lane & 31);
    bf16x8_t b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) b[ks] = load_bf16x8(ku + size_t(col) * D + ks * 16, col < jlim);
    for (; cc < NCH && j0 + cc * 32 < jlim; cc += CS) {
      const int ncol = col + 32 * CS;
      const bool more = cc + CS < NCH && j0 + (cc + CS) * 32 < jlim;
      bf16x8_t bn[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        bn[ks] = load_bf16x8(ku + size_t(ncol) * D + ks * 16, more && ncol < jlim);
      f32x16_t acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], b[ks], acc, 0, 0, 0);
      if (PASS == 1) {
        const bool edge = j0 + cc * 32 + 32 > S - W;  // chunk reaches the causal window or S
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = acc[i] * scale_log2;
          bool ok = true;
          if (edge) {
            const int row = rg * 32 + 8 * (i / 4) + 4 * half + (i & 3);
            ok = col < S && col <= S - W + (row % W);
          }
          if (ok) {
            const float mn = fmaxf(m[i], x);
            z[i] = z[i] * exp2f(m[i] - mn) + exp2f(x - mn);
            m[i] = mn;
          }
        }
      } else {
        float cs_sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) cs_sum += exp2f(acc[i] * scale_log2 - m[i]) * z[i];
        cs_sum += __shfl_xor(cs_sum, 32);
        if (lane < 32) smem[rg * TNM + cc * 32 + lane] = cs_sum;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) b[ks] = bn[ks];
      col = ncol;
    }
    if (PASS == 1) {
      // merge the 32 key columns held by the lanes of each half-wave
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float mo = __shfl_xor(m[i], off);
          const float zo = __shfl_xor(z[i], off);
          const float mn = fmaxf(m[i], mo);
          z[i] = z[i] * exp2f(m[i] - mn) + zo * exp2f(mo - mn);
          m[i] = mn;
        }
      }
      if ((lane & 31) == 0) {
        float2* mz = reinterpret_cast<float2*>(smem) + it * 32;
#pragma unroll
        for (int i = 0; i < 16; ++i) mz[8 * (i / 4) + 4 * half + (i & 3)] = make_float2(m[i], z[i]);
      }
    }
  }
  __syncthreads();
  if (PASS == 1) {
    const float2* mz = reinterpret_cast<const float2*>(smem);
    for (int r = threadIdx.x; r < RG * 32; r += 256) {
      if (r >= M) continue;
      const int rg = r / 32, rl = r % 32;
      float mm = kNegBig, zz = 0.f;
      for (int c = 0; c < CS; ++c) {  // column splits in order
        const float2 p = mz[(rg * CS + c) * 32 + rl];
        const float mn = fmaxf(mm, p.x);
        zz = zz * exp2f(mm - mn) + p.y * exp2f(p.x - mn);
        mm = mn;
      }
      partials[(size_t(u) * M + r) * n_tiles + tile] = make_float2(mm, zz);
    }
  } else {
    for (int c = threadIdx.x; c < TNM; c += 256) {
      const int j = j0 + c;
      if (j >= P) continue;
      float sacc = 0.f;
      for (int rg = 0; rg < RG; ++rg) sacc += smem[rg * TNM + c];
      scores[size_t(u) * P + j] = sacc;
    }
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

  constexpr bool kMfma = sizeof(T) == 2;  // bf16 on the matrix cores, float32 on the vector ALUs
  const int n_tiles = kMfma ? (S + TNM - 1) / TNM : lay.n_tiles;
  const int RG = (M + 31) / 32;
  const int CS = RG >= 4 ? 1 : 4 / RG;
  const size_t lds1 = size_t(RG * CS) * 32 * sizeof(float2);
  const size_t lds2 = size_t(RG) * TNM * sizeof(float);
  if constexpr (kMfma) {
    RK_LAUNCH("ws_pass1", (ws_mfma_kernel<D, 1>), dim3(n_tiles, units), dim3(256), lds1, s,
              reinterpret_cast<const bf16_t*>(qw), reinterpret_cast<const bf16_t*>(kk), kv_cap, S,
              W, d.G, n_tiles, scale_log2, partials, nullptr, nullptr);
  } else {
    RK_LAUNCH("ws_pass1", (ws_pass1_kernel<T, D>), dim3(n_tiles, units), dim3(256), 0, s, qw, kk,
              kv_cap, S, W, d.G, n_tiles, scale_log2, partials);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  RK_LAUNCH("ws_stats", ws_stats_kernel, dim3((units * M + 3) / 4), dim3(256), 0, s, partials, M,
            n_tiles, units, stats);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (P > 0) {
    if constexpr (kMfma) {
      RK_LAUNCH("ws_pass2", (ws_mfma_kernel<D, 2>), dim3((P + TNM - 1) / TNM, units), dim3(256),
                lds2, s, reinterpret_cast<const bf16_t*>(qw), reinterpret_cast<const bf16_t*>(kk),
                kv_cap, S, W, d.G, n_tiles, scale_log2, nullptr, stats, scores);
    } else {
      RK_LAUNCH("ws_pass2", (ws_pass2_kernel<T, D>), dim3((P + TN - 1) / TN, units), dim3(256), 0,
                s, qw, kk, kv_cap, S, W, d.G, scale_log2, stats, scores);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int h = (pool_kernel - 1) / 2;
    RK_LAUNCH("pool_sum", pool_sum_kernel, dim3((P + 255) / 256, units), dim3(256),
                       size_t(256 + 2 * h) * sizeof(float), s, scores, P, h, pooled);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int staged = size_t(P) * 4 <= kSelectKeysLds ? 1 : 0;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       int(kSelectKeysLds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  RK_LAUNCH("select_tokens", select_kernel, dim3(units), dim3(1024),
            staged ? size_t(P) * 4 : size_t(0), s, pooled, S, W, int(n_keep), staged, kept);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (k_out) {
    RK_LAUNCH("gather_kv", (gather_kernel<T, D>), dim3(unsigned((n_keep + 63) / 64), units),
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

// rk_aux.hip -- HSA step 1: per-page element-wise Kmax / Kmin.
//
// Source: papercache notes "RocketKV: Accelerating Long-Context LLM Inference
// via Two-Stage KV Cache Compression", method details, HSA step 1 (pages of
// consecutive keys, element-wise max/min kept as auxiliary data laid out
// along the head dimension, refreshed as new keys arrive) and RocketKV-MT
// (pages over the stage-1 candidate list of the full cache).  Also the
// decode-time append: one new row per unit folded into its page.
//
// One 512-thread workgroup covers PPW consecutive pages of one unit (32 for
// 256-byte rows, so each channel's output run is a whole 64-byte line).  Each
// thread owns one 16-byte channel chunk of one page: it reads the page's rows
// eight at a time (their indices, then all eight coalesced 16-byte loads in
// flight; a short page repeats its last row, which max/min ignore), keeps
// the running max/min in registers, then the tile is transposed through LDS
// so the channel-major output is written in contiguous page runs.
// Bandwidth bound: bytes = rows read + 2 * d * pages * sizeof(T) written.
#include <type_traits>

#include "rk_device.hpp"
#include "rk_internal.hpp"

namespace rk {
namespace {

constexpr int kAuxThreads = 512;

template <typename T, int D, bool PAGED = false>
__global__ __launch_bounds__(kAuxThreads) void aux_build_kernel(
    const T* __restrict__ k, int64_t k_cap, const int32_t* __restrict__ idx, int64_t idx_stride,
    int n_tokens, int first_block, int nblk, int block, T* __restrict__ kmax,
    T* __restrict__ kmin, int64_t nblk_cap, PagedArgs pga) {
  constexpr int EPL = Vec16<T>::N;   // elements per 16-byte chunk
  constexpr int CPR = D / EPL;       // chunks per row
  constexpr int PPW = kAuxThreads / CPR;  // pages per workgroup
  constexpr int RB = 8;              // rows in flight per thread
  static_assert(D % EPL == 0 && kAuxThreads % CPR == 0, "row must split into 16-byte chunks");
  __shared__ T smax[D][PPW + 1];
  __shared__ T smin[D][PPW + 1];

  const int u = blockIdx.y;
  const int t = threadIdx.x;
  const int c = t % CPR;
  const int j = t / CPR;
  const int p0 = first_block + blockIdx.x * PPW;
  const int p = p0 + j;
  // PAGED: rows are pool rows (the unit's sequence row of the block table)
  const T* ku = k + (PAGED ? size_t(0) : size_t(u) * size_t(k_cap) * D) + c * EPL;
  const int32_t* iu = idx ? idx + size_t(u) * size_t(idx_stride) : nullptr;
  const int32_t* tab = PAGED ? pga.table + size_t(u / pga.hkv) * pga.table_stride : nullptr;

  if (p < nblk) {
    const int n0 = p * block;
    const int n1 = min(n0 + block, n_tokens);
    float mx[EPL], mn[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      mx[e] = -INFINITY;
      mn[e] = INFINITY;
    }
    for (int b0 = n0; b0 < n1; b0 += RB) {
      int row[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int n = min(b0 + i, n1 - 1);
        if constexpr (PAGED)
          row[i] = paged_row(tab, n, pga.n_phys, pga.shift, pga.hkv, u % pga.hkv);
        else
          row[i] = iu ? clamp_row(iu[n], k_cap) : n;
      }
      Vec16<T> xr[RB];
#pragma unroll
      // each row is read once per build: non-temporal (RocketKV-MT's build over
      // 6517 scattered candidate rows per unit at batch 8 x 32 heads: 117 ->
      // 97 us; 16 rows in flight instead of 8 changed nothing)
      for (int i = 0; i < RB; ++i) xr[i] = load16_nt(ku + size_t(row[i]) * D);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        float x[EPL];
        unpack16(xr[i], x);
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
        // values came from bf16, so dropping the low half is exact
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
  T* nu = kmin ? kmin + size_t(u) * D * size_t(nblk_cap) : nullptr;  // NULL: only Kmax is wanted
  for (int e = t; e < D * PPW; e += kAuxThreads) {
    const int ch = e / PPW;
    const int jj = e % PPW;
    const int pp = p0 + jj;
    if (pp < nblk) {
      xu[size_t(ch) * nblk_cap + pp] = smax[ch][jj];
      if (kmin) nu[size_t(ch) * nblk_cap + pp] = smin[ch][jj];
    }
  }
}

template <typename T, int D>
hipError_t launch_aux_t(const Dims& d, const void* k, int64_t k_cap, const int32_t* idx,
                        int64_t idx_stride, int64_t n_tokens, int64_t first_block, int block,
                        void* kmax, void* kmin, int64_t nblk_cap, hipStream_t s,
                        const PagedArgs* paged) {
  constexpr int PPW = kAuxThreads / (D / Vec16<T>::N);
  const int64_t nblk = (n_tokens + block - 1) / block;
  const int64_t npages = nblk - first_block;
  dim3 grid(unsigned((npages + PPW - 1) / PPW), unsigned(d.units()));
  constexpr bool kPagedBuilt = std::is_same_v<T, bf16_t>;
  if (paged && !kPagedBuilt) return hipErrorInvalidValue;
  if (paged)
    RK_LAUNCH("aux_build", (aux_build_kernel<T, D, kPagedBuilt>), grid, dim3(kAuxThreads), 0, s,
              static_cast<const T*>(k), k_cap, idx, idx_stride, int(n_tokens), int(first_block),
              int(nblk), block, static_cast<T*>(kmax), static_cast<T*>(kmin), nblk_cap, *paged);
  else
    RK_LAUNCH("aux_build", (aux_build_kernel<T, D>), grid, dim3(kAuxThreads), 0, s,
              static_cast<const T*>(k), k_cap, idx, idx_stride, int(n_tokens), int(first_block),
              int(nblk), block, static_cast<T*>(kmax), static_cast<T*>(kmin), nblk_cap, PagedArgs{});
  return hipGetLastError();
}

// One thread per (unit, channel): write the new K/V element at row pos and
// fold it into the page's max/min (a fresh page takes the value itself).
template <typename T, int D, bool PAGED = false>
__global__ __launch_bounds__(256) void append_kv_kernel(const T* __restrict__ k_new,
                                                        const T* __restrict__ v_new,
                                                        T* __restrict__ k, T* __restrict__ v,
                                                        int64_t kv_cap, int64_t pos, int units,
                                                        T* __restrict__ kmax, T* __restrict__ kmin,
                                                        int64_t nblk_cap, int block, PagedArgs pga) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  if (gid >= units * D) return;
  const int u = gid / D, ch = gid % D;
  const T kn = k_new[size_t(u) * D + ch];
  const size_t row = PAGED ? size_t(paged_row(pga.table + size_t(u / pga.hkv) * pga.table_stride, int(pos),
                                              pga.n_phys, pga.shift, pga.hkv, u % pga.hkv))
                           : size_t(u) * kv_cap + pos;
  k[row * D + ch] = kn;
  v[row * D + ch] = v_new[size_t(u) * D + ch];
  const size_t a = (size_t(u) * D + ch) * nblk_cap + pos / block;
  if (pos % block == 0) {
    kmax[a] = kn;
    kmin[a] = kn;
  } else {
    const float x = to_f32(kn);
    if (x > to_f32(kmax[a])) kmax[a] = kn;
    if (x < to_f32(kmin[a])) kmin[a] = kn;
  }
}

template <typename T, int D>
hipError_t launch_append_t(const Dims& d, const void* k_new, const void* v_new, void* k, void* v,
                           int64_t kv_cap, int64_t pos, void* kmax, void* kmin, int64_t nblk_cap,
                           int block, hipStream_t s, const PagedArgs* paged) {
  const int units = d.units();
  constexpr bool kPagedBuilt = std::is_same_v<T, bf16_t>;
  if (paged && !kPagedBuilt) return hipErrorInvalidValue;
  if (paged)
    RK_LAUNCH("append_kv", (append_kv_kernel<T, D, kPagedBuilt>), dim3((units * D + 255) / 256), dim3(256),
              0, s, static_cast<const T*>(k_new), static_cast<const T*>(v_new), static_cast<T*>(k),
              static_cast<T*>(v), kv_cap, pos, units, static_cast<T*>(kmax), static_cast<T*>(kmin),
              nblk_cap, block, *paged);
  else
    RK_LAUNCH("append_kv", (append_kv_kernel<T, D>), dim3((units * D + 255) / 256), dim3(256), 0, s,
              static_cast<const T*>(k_new), static_cast<const T*>(v_new), static_cast<T*>(k),
              static_cast<T*>(v), kv_cap, pos, units, static_cast<T*>(kmax), static_cast<T*>(kmin),
              nblk_cap, block, PagedArgs{});
  return hipGetLastError();
}

// Dense rows [first, first + n) of every unit to the same token positions of
// a paged pool: one thread per 16-byte chunk, both tensors.
template <int D>
__global__ __launch_bounds__(256) void paged_write_kernel(const bf16_t* __restrict__ ks,
                                                          const bf16_t* __restrict__ vs, int64_t src_cap,
                                                          int first, int n, bf16_t* __restrict__ kp,
                                                          bf16_t* __restrict__ vp, PagedArgs pga) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const int u = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n * CPR) return;
  const int r = e / CPR, c = e % CPR;
  const int tok = first + r;
  const size_t src = (size_t(u) * size_t(src_cap) + size_t(tok)) * D + c * 8;
  const size_t dst = size_t(paged_row(pga.table + size_t(u / pga.hkv) * pga.table_stride, tok, pga.n_phys,
                                      pga.shift, pga.hkv, u % pga.hkv)) * D + c * 8;
  *reinterpret_cast<uint4*>(kp + dst) = *reinterpret_cast<const uint4*>(ks + src);
  *reinterpret_cast<uint4*>(vp + dst) = *reinterpret_cast<const uint4*>(vs + src);
}

}  // namespace

hipError_t launch_append_kv(const Dims& d, const void* k_new, const void* v_new, void* k, void* v,
                            int64_t kv_cap, int64_t pos, void* kmax, void* kmin,
                            int64_t nblk_cap, int block, hipStream_t s, const PagedArgs* paged) {
  if (d.bf16) {
    if (d.D == 128)
      return launch_append_t<bf16_t, 128>(d, k_new, v_new, k, v, kv_cap, pos, kmax, kmin, nblk_cap,
                                          block, s, paged);
    return launch_append_t<bf16_t, 64>(d, k_new, v_new, k, v, kv_cap, pos, kmax, kmin, nblk_cap,
                                       block, s, paged);
  }
  if (d.D == 128)
    return launch_append_t<float, 128>(d, k_new, v_new, k, v, kv_cap, pos, kmax, kmin, nblk_cap,
                                       block, s, paged);
  return launch_append_t<float, 64>(d, k_new, v_new, k, v, kv_cap, pos, kmax, kmin, nblk_cap, block,
                                    s, paged);
}

hipError_t launch_build_aux(const Dims& d, const void* k, int64_t k_cap, const int32_t* idx,
                            int64_t idx_stride, int64_t n_tokens, int64_t first_block,
                            int block, void* kmax, void* kmin, int64_t nblk_cap,
                            hipStream_t s, const PagedArgs* paged) {
  if (d.bf16) {
    if (d.D == 128)
      return launch_aux_t<bf16_t, 128>(d, k, k_cap, idx, idx_stride, n_tokens, first_block,
                                       block, kmax, kmin, nblk_cap, s, paged);
    return launch_aux_t<bf16_t, 64>(d, k, k_cap, idx, idx_stride, n_tokens, first_block, block,
                                    kmax, kmin, nblk_cap, s, paged);
  }
  if (d.D == 128)
    return launch_aux_t<float, 128>(d, k, k_cap, idx, idx_stride, n_tokens, first_block, block,
                                    kmax, kmin, nblk_cap, s, paged);
  return launch_aux_t<float, 64>(d, k, k_cap, idx, idx_stride, n_tokens, first_block, block,
                                 kmax, kmin, nblk_cap, s, paged);
}

hipError_t launch_paged_write(const Dims& d, const void* k_src, const void* v_src, int64_t src_cap,
                              int64_t first, int64_t n, void* k_pool, void* v_pool,
                              const PagedArgs& paged, hipStream_t s) {
  if (!d.bf16) return hipErrorInvalidValue;
  const int units = d.units();
  const int chunks = int(n) * (d.D / 8);
  const dim3 grid(unsigned((chunks + 255) / 256), unsigned(units));
  if (d.D == 128)
    RK_LAUNCH("paged_write", paged_write_kernel<128>, grid, dim3(256), 0, s,
              static_cast<const bf16_t*>(k_src), static_cast<const bf16_t*>(v_src), src_cap, int(first),
              int(n), static_cast<bf16_t*>(k_pool), static_cast<bf16_t*>(v_pool), paged);
  else
    RK_LAUNCH("paged_write", paged_write_kernel<64>, grid, dim3(256), 0, s,
              static_cast<const bf16_t*>(k_src), static_cast<const bf16_t*>(v_src), src_cap, int(first),
              int(n), static_cast<bf16_t*>(k_pool), static_cast<bf16_t*>(v_pool), paged);
  return hipGetLastError();
}

}  // namespace rk

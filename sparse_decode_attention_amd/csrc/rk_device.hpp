// rk_device.hpp -- device-side helpers shared by the RocketKV kernels (gfx950,
// wave64): element loads, order-preserving float keys, workgroup scans and the
// workgroup top-k selection used for tokens (stage 1), channels and pages
// (HSA step 2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Phase marker for external timing probes; compiles to nothing in the library.
#ifndef RK_PHASE
#define RK_PHASE(slot)
#endif

namespace rk {

constexpr int kWave = 64;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

// bf16 is carried as raw uint16 bits (the upper half of an IEEE float32).
struct bf16_t {
  uint16_t bits;
};

// 2^x with the hardware instruction alone.  Used where x <= 0 (arguments are
// differences from a running maximum): results below 2^-126, if flushed,
// are negligible next to the sums of >= 1 they are added to.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x.bits) << 16); }

// 16-byte vector of elements: 4 float or 8 bf16.
template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  float4 raw;
  __device__ __forceinline__ float get(int i) const {
    return i == 0 ? raw.x : i == 1 ? raw.y : i == 2 ? raw.z : raw.w;
  }
};
template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
  uint4 raw;
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = i < 2 ? raw.x : i < 4 ? raw.y : i < 6 ? raw.z : raw.w;
    return (i & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};

template <typename T>
__device__ __forceinline__ Vec16<T> load16(const T* p) {
  Vec16<T> v;
  v.raw = *reinterpret_cast<const decltype(v.raw)*>(p);
  return v;
}

template <typename T>
__device__ __forceinline__ void unpack16(const Vec16<T>& v, float* out) {
#pragma unroll
  for (int i = 0; i < Vec16<T>::N; ++i) out[i] = v.get(i);
}

// Order-preserving map float -> uint32: a > b  <=>  key(a) > key(b); -0 and +0
// share one key (they compare equal as floats).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// A caller-supplied row index forced into [0, cap): out-of-range indices give
// unspecified values, never out-of-bounds reads.
__device__ __forceinline__ int clamp_row(int32_t row, int64_t cap) {
  return uint64_t(uint32_t(row)) < uint64_t(cap) ? row : 0;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Exclusive prefix sum of v over the workgroup (NT threads, wave64).  `tmp`
// must hold NT/64 + 1 ints of LDS.  Returns the exclusive prefix; *total gets
// the workgroup sum.  Contains barriers: every thread must call it.
template <int NT>
__device__ __forceinline__ int wg_excl_scan(int v, int* tmp, int* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(x, off);
    if (lane >= off) x += t;
  }
  if (lane == kWave - 1) tmp[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NT / kWave; ++w) {
      const int t = tmp[w];
      tmp[w] = run;
      run += t;
    }
    tmp[NT / kWave] = run;
  }
  __syncthreads();
  const int res = tmp[wave] + x - v;
  *total = tmp[NT / kWave];
  __syncthreads();
  return res;
}

// Exclusive prefix sums of a pair (a, b) over the workgroup in one pass.
template <int NT>
__device__ __forceinline__ int2 wg_excl_scan2(int a, int b, int* tmp) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  int xa = a, xb = b;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int ta = __shfl_up(xa, off);
    const int tb = __shfl_up(xb, off);
    if (lane >= off) {
      xa += ta;
      xb += tb;
    }
  }
  if (lane == kWave - 1) {
    tmp[2 * wave] = xa;
    tmp[2 * wave + 1] = xb;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int ra = 0, rb = 0;
    for (int w = 0; w < NT / kWave; ++w) {
      const int ta = tmp[2 * w], tb = tmp[2 * w + 1];
      tmp[2 * w] = ra;
      tmp[2 * w + 1] = rb;
      ra += ta;
      rb += tb;
    }
  }
  __syncthreads();
  const int2 res = make_int2(tmp[2 * wave] + xa - a, tmp[2 * wave + 1] + xb - b);
  __syncthreads();
  return res;
}

// Exclusive prefix count of a predicate over the workgroup (ballot based).
template <int NT>
__device__ __forceinline__ int wg_excl_count(bool p, int* tmp, int* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const unsigned long long b = __ballot(p);
  const int below = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) tmp[wave] = __popcll(b);
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NT / kWave; ++w) {
      const int t = tmp[w];
      tmp[w] = run;
      run += t;
    }
    tmp[NT / kWave] = run;
  }
  __syncthreads();
  const int res = tmp[wave] + below;
  *total = tmp[NT / kWave];
  __syncthreads();
  return res;
}

template <int NT>
struct TopkSmem {
  static constexpr int kBins = 2048;
  uint32_t hist[kBins];
  int tmp[2 * (NT / kWave) + 2];
  int found[2];
};

// Workgroup top-k: calls emit(rank, position) for the k largest keys among
// key(0..n-1), ties broken toward the lower position; ranks 0..k-1 follow
// ascending position order.  Selected <=> #{i : key_i > key_j or (key_i == key_j and
// i < j)} < k.  Radix select over 11/11/10-bit digits finds the exact k-th
// key T and how many keys equal to T are taken; an ordered scan then writes
// the selection.  0 <= k <= n.  All threads of the workgroup must call it.
template <int NT, typename KeyFn, typename EmitFn>
__device__ void wg_topk(const KeyFn& key, int n, int k, const EmitFn& emit, TopkSmem<NT>& sm) {
  const int t = threadIdx.x;
  if (k <= 0) return;
  if (k >= n) {
    for (int i = t; i < n; i += NT) emit(i, i);
    return;
  }
  uint32_t prefix = 0, mask = 0;
  int need = k;  // keys still to take among those matching `prefix`
  constexpr int kShift[3] = {21, 10, 0};
  constexpr int kBits[3] = {11, 11, 10};
  constexpr int kPer = TopkSmem<NT>::kBins / NT;  // bins owned by one thread
  static_assert(kPer >= 1 && TopkSmem<NT>::kBins % NT == 0, "bins per thread");
  // Histogram order: lane l of every wave walks the run [l*rows, (l+1)*rows)
  // (rows odd), so the 64 lanes of one instruction touch keys far apart.
  // Neighbouring keys are often nearly equal (pooled scores), and a wave whose
  // lanes all hit one bin would serialise its LDS atomics.
  const int rows = ((n + kWave - 1) / kWave) | 1;
  const int lane = lane_id();
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = kShift[pass];
    const uint32_t dmask = (1u << kBits[pass]) - 1u;
    for (int b = t; b < TopkSmem<NT>::kBins; b += NT) sm.hist[b] = 0u;
    __syncthreads();
    for (int c = t / kWave; c < rows; c += NT / kWave) {
      const int i = lane * rows + c;
      if (i < n) {
        const uint32_t kk = key(i);
        if ((kk & mask) == prefix) atomicAdd(&sm.hist[(kk >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    RK_PHASE(1 + pass);
    // Thread t owns bins [top - (t+1)*kPer, top - t*kPer): thread 0 the highest.
    const int hi = TopkSmem<NT>::kBins - t * kPer;
    int own = 0;
#pragma unroll
    for (int j = 1; j <= kPer; ++j) own += int(sm.hist[hi - j]);
    int total;
    int above = wg_excl_scan<NT>(own, sm.tmp, &total);
#pragma unroll
    for (int j = 1; j <= kPer; ++j) {
      const int c = int(sm.hist[hi - j]);
      if (above < need && above + c >= need) {
        sm.found[0] = hi - j;
        sm.found[1] = need - above;
      }
      above += c;
    }
    __syncthreads();
    prefix |= uint32_t(sm.found[0]) << shift;
    mask |= dmask << shift;
    need = sm.found[1];
    __syncthreads();
  }
  // prefix == T (the k-th largest key); take `need` of the keys equal to T,
  // lowest positions first, and every key above T.  Thread t owns the
  // contiguous positions [t*seg, (t+1)*seg): it counts its keys above and
  // equal to T, one workgroup scan gives the counts before it, then it emits
  // its selected positions in order.
  const uint32_t T = prefix;
  const int need_eq = need;
  const int seg = ((n + NT - 1) / NT) | 1;  // odd: spreads LDS banks
  const int lo = min(t * seg, n);
  const int hi = min(lo + seg, n);
  int n_gt = 0, n_eq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t kk = key(i);
    n_gt += kk > T;
    n_eq += kk == T;
  }
  RK_PHASE(4);
  const int2 before = wg_excl_scan2<NT>(n_gt, n_eq, sm.tmp);
  int eq_seen = before.y;
  int pos = before.x + min(before.y, need_eq);
  for (int i = lo; i < hi; ++i) {
    const uint32_t kk = key(i);
    bool sel = kk > T;
    if (kk == T) {
      sel = eq_seen < need_eq;
      ++eq_seen;
    }
    if (sel) emit(pos++, i);
  }
  RK_PHASE(5);
}

// Workgroup top-k for a small key set held in LDS (n up to a few thousand):
// element j is selected iff #{i : key_i > key_j or (key_i == key_j and
// i < j)} < k, counted directly (4 keys per LDS read, broadcast to the wave);
// emit(rank, j) in ascending j order as wg_topk.  `keys` must be 16-byte
// aligned with room for n rounded up to 4 (the padding is never counted).
template <int NT, typename EmitFn>
__device__ void wg_topk_rank(const uint32_t* keys, int n, int k, const EmitFn& emit, int* tmp) {
  const int t = threadIdx.x;
  if (k <= 0) return;
  if (k >= n) {
    for (int i = t; i < n; i += NT) emit(i, i);
    return;
  }
  const int n4 = n & ~3;
  int base = 0;
  for (int c0 = 0; c0 < n; c0 += NT) {
    const int j = c0 + t;
    bool sel = false;
    if (j < n) {
      const uint32_t kj = keys[j];
      int rank = 0;
      const int n32 = n & ~31;
      int i = 0;
      for (; i < n32; i += 32) {  // eight 16-byte LDS reads in flight
        uint4 kk[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) kk[x] = *reinterpret_cast<const uint4*>(keys + i + 4 * x);
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int b = i + 4 * x;
          rank += int(kk[x].x > kj || (kk[x].x == kj && b < j));
          rank += int(kk[x].y > kj || (kk[x].y == kj && b + 1 < j));
          rank += int(kk[x].z > kj || (kk[x].z == kj && b + 2 < j));
          rank += int(kk[x].w > kj || (kk[x].w == kj && b + 3 < j));
        }
      }
      for (; i < n4; i += 4) {
        const uint4 kk = *reinterpret_cast<const uint4*>(keys + i);
        rank += int(kk.x > kj || (kk.x == kj && i < j));
        rank += int(kk.y > kj || (kk.y == kj && i + 1 < j));
        rank += int(kk.z > kj || (kk.z == kj && i + 2 < j));
        rank += int(kk.w > kj || (kk.w == kj && i + 3 < j));
      }
      for (; i < n; ++i) rank += int(keys[i] > kj || (keys[i] == kj && i < j));
      sel = rank < k;
    }
    int tot;
    const int pos = base + wg_excl_count<NT>(sel, tmp, &tot);
    if (sel) emit(pos, j);
    base += tot;
  }
}

// Sum over aligned groups of N lanes (N = 2, 4, 8, 16, 32), result in every
// lane of the group.  Up to 16 lanes it uses DPP row permutations (quad swaps,
// then the half-row and row mirrors), which stay in the ALU; the step across
// 16-lane rows uses a lane shuffle.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32, "group size");
  if (N >= 2) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));  // quad [1,0,3,2]
  if (N >= 4) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));  // quad [2,3,0,1]
  if (N >= 8) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false)); // row_half_mirror
  if (N >= 16) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false)); // row_mirror
  if (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

// Wave-wide reductions (all 64 lanes take part).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

}  // namespace rk

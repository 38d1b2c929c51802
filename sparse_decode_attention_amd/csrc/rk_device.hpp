// rk_device.hpp -- device-side helpers shared by the RocketKV kernels (gfx950,
// wave64): element loads, order-preserving float keys, workgroup scans and the
// workgroup top-k selection used for tokens (stage 1), channels and pages
// (HSA step 2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Wait until this wave's vector memory loads have all returned (s_waitcnt
// vmcnt(0); expcnt and lgkmcnt left at their maxima).  Placed after loads
// made once before a loop whose body also issues loads, it lets the
// compiler's wait counting see those registers as ready inside the loop;
// otherwise it may wait for every load in flight at the loop head.
__device__ __forceinline__ void wait_vector_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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

// Non-temporal forms, for data read once per launch (the chosen K/V rows of
// a decode step, streamed keys): the load is marked as streaming, so it does
// not displace data that is reused (page keys, aux rows of other units).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ Vec16<T> load16_nt(const T* p) {
  Vec16<T> v;
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  v.raw = __builtin_bit_cast(decltype(v.raw), x);
  return v;
}
__device__ __forceinline__ uint4 load_u4_nt(const uint4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

// 16-byte non-temporal store (a vector store with the streaming hint).
template <typename T>
__device__ __forceinline__ void store16_nt(T* p, const Vec16<T>& v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v.raw), reinterpret_cast<u32x4_t*>(p));
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

// Pool row of token `tok` of one unit in a paged K/V pool (see PagedArgs):
// `table` is the unit's sequence row of the block table, `h` its head.
__device__ __forceinline__ int paged_row(const int32_t* table, int tok, int64_t n_phys, int shift,
                                         int hkv, int h) {
  const int pg = clamp_row(table[tok >> shift], n_phys);
  return ((pg * hkv + h) << shift) + (tok & ((1 << shift) - 1));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Lanes of the wave where b holds, straight from the compare (no bool -> int
// round trip, which costs two extra instructions per call).
__device__ __forceinline__ unsigned long long ballot(bool b) { return __builtin_amdgcn_ballot_w64(b); }

// a.lo * b.lo + a.hi * b.hi + c over packed bf16 pairs (v_dot2c_f32_bf16)
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a), __builtin_bit_cast(bf16x2_v, b), c,
                                         false);
}

// XCD-aware work mapping.  MI355X deals the workgroups of a launch out to its
// 8 XCDs round robin (workgroup L to XCD L mod 8), and each XCD has its own
// L2.  With a 1-D grid of 8 * ceil(n/8) workgroups, XCD x here takes the
// contiguous work items [x * per, (x + 1) * per), so neighbouring items
// (pages of one unit, splits of one unit) share an L2.  Returns the item of
// this workgroup; items >= n are padding and do nothing.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_local_item(int n_items) {
  const int per = (n_items + kXcds - 1) / kXcds;
  const int L = blockIdx.x;
  return (L % kXcds) * per + L / kXcds;
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts build the
// sums inside each 16-lane row (zero fill at the row edge), then the totals of
// the earlier rows come in through lane reads.  No LDS traffic.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane_id() >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Minimum / maximum of uint32 over the wave (DPP inside rows, lane reads across).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), 0xB1, 0xf, 0xf, false)));
  x = min(x, uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), 0x4E, 0xf, 0xf, false)));
  x = min(x, uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), 0x141, 0xf, 0xf, false)));
  x = min(x, uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), 0x140, 0xf, 0xf, false)));
  const uint32_t a = uint32_t(__builtin_amdgcn_readlane(int(x), 0));
  const uint32_t b = uint32_t(__builtin_amdgcn_readlane(int(x), 16));
  const uint32_t c = uint32_t(__builtin_amdgcn_readlane(int(x), 32));
  const uint32_t d = uint32_t(__builtin_amdgcn_readlane(int(x), 48));
  return min(min(a, b), min(c, d));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), 0xB1, 0xf, 0xf, false)));
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), 0x4E, 0xf, 0xf, false)));
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), 0x141, 0xf, 0xf, false)));
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), 0x140, 0xf, 0xf, false)));
  const uint32_t a = uint32_t(__builtin_amdgcn_readlane(int(x), 0));
  const uint32_t b = uint32_t(__builtin_amdgcn_readlane(int(x), 16));
  const uint32_t c = uint32_t(__builtin_amdgcn_readlane(int(x), 32));
  const uint32_t d = uint32_t(__builtin_amdgcn_readlane(int(x), 48));
  return max(max(a, b), max(c, d));
}

// Exclusive prefix sum of v over the workgroup (NT threads, wave64).  `tmp`
// must hold 2*(NT/64) + 2 ints of LDS.  Returns the exclusive prefix; *total
// gets the workgroup sum.  Every thread reads the wave totals itself (no
// serial pass).  Contains barriers: every thread must call it.
template <int NT>
__device__ __forceinline__ int wg_excl_scan(int v, int* tmp, int* total) {
  constexpr int NW = NT / kWave;
  const int wave = threadIdx.x / kWave;
  const int x = wave_incl_scan(v);
  if (lane_id() == kWave - 1) tmp[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = tmp[w];
    before += w < wave ? c : 0;
    all += c;
  }
  *total = all;
  __syncthreads();
  return before + x - v;
}

// Exclusive prefix sums of a pair (a, b) over the workgroup in one pass.
template <int NT>
__device__ __forceinline__ int2 wg_excl_scan2(int a, int b, int* tmp) {
  constexpr int NW = NT / kWave;
  const int wave = threadIdx.x / kWave;
  const int xa = wave_incl_scan(a);
  const int xb = wave_incl_scan(b);
  if (lane_id() == kWave - 1) {
    tmp[2 * wave] = xa;
    tmp[2 * wave + 1] = xb;
  }
  __syncthreads();
  int ba = 0, bb = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) {
      ba += tmp[2 * w];
      bb += tmp[2 * w + 1];
    }
  }
  __syncthreads();
  return make_int2(ba + xa - a, bb + xb - b);
}

// Ordered emission of a top-k: with the threshold key T, every key above it
// is taken and `need_eq` of the keys equal to it, lowest positions first (or,
// when all_eq, every key >= T: one comparison per key).  Thread t owns the
// contiguous positions [t*seg, (t+1)*seg): it counts its selected keys, one
// workgroup scan gives the counts before it, then it emits its selected
// positions in order.  (Per-thread runs beat per-row ballots here: a row of
// 64 positions costs a dozen wave-wide instructions, a thread's key two.)
template <int NT, typename KeyFn, typename EmitFn>
__device__ __forceinline__ void wg_topk_emit(const KeyFn& key, int n, uint32_t T, int need_eq,
                                             bool all_eq, const EmitFn& emit, int* tmp) {
  const int t = threadIdx.x;
  const int seg = ((n + NT - 1) / NT) | 1;  // odd: spreads LDS banks
  const int lo = min(t * seg, n);
  const int hi = min(lo + seg, n);
  if (all_eq) {
    int n_ge = 0;
    for (int i = lo; i < hi; ++i) n_ge += key(i) >= T ? 1 : 0;
    int total;
    int pos = wg_excl_scan<NT>(n_ge, tmp, &total);
    for (int i = lo; i < hi; ++i)
      if (key(i) >= T) emit(pos++, i);
    return;
  }
  int n_gt = 0, n_eq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t kk = key(i);
    n_gt += kk > T;
    n_eq += kk == T;
  }
  const int2 before = wg_excl_scan2<NT>(n_gt, n_eq, tmp);
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
}

// Workgroup top-k: calls emit(rank, position) for the k largest keys among
// key(0..n-1), ties broken toward the lower position; ranks 0..k-1 follow
// ascending position order.  Selected <=> #{i : key_i > key_j or (key_i ==
// key_j and i < j)} < k.  0 <= k <= n; all threads of the workgroup call it,
// and emitted results are complete after the caller's next barrier.
//
// Range-adaptive radix select.  A pass buckets the candidate keys, those in
// [lo, hi], by (key - lo) >> shift, with shift chosen so the candidates' span
// fills the BINS bins (the first pass takes lo, hi = min, max of all keys):
// keys close in value still spread over many bins, so the LDS atomics rarely
// collide and the boundary bin usually holds one or two keys.  Every wave
// then finds the bin of the k-th largest key from the histogram by itself
// (no barrier): keys above it are taken, keys below dropped.  It ends when the
// boundary bin is one key value or is taken whole, after one pass in most
// cases; each pass narrows the span by a factor BINS, so at most
// ceil(32 / log2(BINS)) passes.  With NBUF = 2 histograms alternate between
// two buffers so a pass needs two barriers; NBUF = 1 saves the LDS for a
// third barrier per pass after the first.
template <int NT, int BINS, int NBUF = 2>
struct TopkSmem {
  alignas(16) uint32_t hist[NBUF][BINS];
  uint32_t red[2 * (NT / kWave)];
  int tmp[2 * (NT / kWave) + 2];
  int n_cand;  // keys gathered into the caller's candidate buffer
};

// The bin holding the need-th largest key, counting from the top bin, and
// how many keys it holds and are still needed from it.  Lane l reads bins
// [BINS - (l+1)*BPL, BINS - l*BPL); a wave scan gives the count above each
// lane, the lane that crosses `need` walks its bins.  Wave-uniform result.
template <int BINS>
__device__ __forceinline__ int3 wave_find_bin(const uint32_t* hist, int need) {
  constexpr int BPL = BINS / kWave;
  static_assert(BPL % 4 == 0, "bins per lane");
  const int lane = lane_id();
  const int base = BINS - (lane + 1) * BPL;
  uint32_t c[BPL];
#pragma unroll
  for (int j = 0; j < BPL; j += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(hist + base + j);
    c[j] = v.x;
    c[j + 1] = v.y;
    c[j + 2] = v.z;
    c[j + 3] = v.w;
  }
  int own = 0;
#pragma unroll
  for (int j = 0; j < BPL; ++j) own += int(c[j]);
  const int incl = wave_incl_scan(own);
  int above = incl - own;
  const unsigned long long hit = ballot(above < need && incl >= need);
  const int L = __ffsll(static_cast<long long>(hit)) - 1;
  int bin = 0, nin = 0, cnt = 0;
#pragma unroll
  for (int j = BPL - 1; j >= 0; --j) {
    const int cj = int(c[j]);
    if (above < need && above + cj >= need) {
      bin = base + j;
      nin = need - above;
      cnt = cj;
    }
    above += cj;
  }
  return make_int3(__builtin_amdgcn_readlane(bin, L), __builtin_amdgcn_readlane(nin, L),
                   __builtin_amdgcn_readlane(cnt, L));
}

// Ordered emission by one wave (n small): 64 positions per step, ballots give
// each selected position its rank and each equal key its order among equals.
template <typename KeyFn, typename EmitFn>
__device__ __forceinline__ void wave_topk_emit(const KeyFn& key, int n, uint32_t T, int need_eq,
                                               const EmitFn& emit) {
  const int lane = lane_id();
  const unsigned long long below = (1ull << lane) - 1ull;
  int base = 0, eq_seen = 0;
  // two rows of 64 per iteration, unrolled by hand (a row past n selects
  // nothing): the ballots are convergent, so the compiler cannot unroll a
  // loop of unknown trip count itself
  for (int c0 = 0; c0 < n; c0 += 2 * kWave) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = c0 + h * kWave + lane;
      const uint32_t kk = i < n ? key(i) : 0u;
      const bool eq = i < n && kk == T;
      const unsigned long long em = ballot(eq);
      const bool sel = (i < n && kk > T) || (eq && eq_seen + int(__popcll(em & below)) < need_eq);
      const unsigned long long sm = ballot(sel);
      if (sel) emit(base + __popcll(sm & below), i);
      base += __popcll(sm);
      eq_seen += __popcll(em);
    }
  }
}

// Keys ranked against each other once the radix bin holding the cut has at
// most this many keys (one wave's passes stop there).
constexpr int kWaveRankMax = 16;

// Exact cut among the c <= kWaveRankMax keys of [lo, hi] (lo >= 1): the keys are packed
// into LDS slots (position order), lane l takes slot l and counts the slots
// above it (gt) and at or above it (ge) with broadcast reads; the lane with
// gt < need <= ge holds T, the need-th largest of the range.  Returns T, the
// keys still needed at T (need - gt) and how many keys equal T (ge - gt).
template <int R>
__device__ __forceinline__ uint3 wave_rank_range(const uint32_t (&kz)[R], int /*n*/, uint32_t lo,
                                                 uint32_t hi, int need, uint32_t* slots) {
  const int lane = lane_id();
  const unsigned long long below = (1ull << lane) - 1ull;
  // every row's candidate mask first (independent compares), then the
  // packing of the rows that hold any
  const uint32_t span = hi - lo;
  // unused slots read as 0, below every candidate (lo >= 1 here)
  if (lane < kWaveRankMax / 4) reinterpret_cast<uint4*>(slots)[lane] = make_uint4(0u, 0u, 0u, 0u);
  unsigned long long m[R];
#pragma unroll
  for (int r = 0; r < R; ++r) m[r] = ballot(kz[r] - lo <= span);  // padding 0 < lo falls out
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (m[r]) {
      if ((m[r] >> lane) & 1ull) slots[cnt + __popcll(m[r] & below)] = kz[r];
      cnt += __popcll(m[r]);
    }
  }
  __builtin_amdgcn_wave_barrier();
  const uint32_t mine = lane < cnt ? slots[lane] : 0u;
  int gt = 0, ge = 0;
#pragma unroll
  for (int j = 0; j < kWaveRankMax; j += 4) {
    const uint4 s4 = *reinterpret_cast<const uint4*>(slots + j);
    const uint32_t sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gt += sv[e] > mine ? 1 : 0;
      ge += sv[e] >= mine ? 1 : 0;
    }
  }
  const unsigned long long hit = ballot(lane < cnt && gt < need && ge >= need);
  const int L = __ffsll(static_cast<long long>(hit)) - 1;
  const int gtL = __builtin_amdgcn_readlane(gt, L), geL = __builtin_amdgcn_readlane(ge, L);
  return make_uint3(uint32_t(__builtin_amdgcn_readlane(int(mine), L)), uint32_t(need - gtL),
                    uint32_t(geL - gtL));
}

// Where a top-k cuts: every key > T, then the first need_eq keys equal to T
// (position order); when `fast`, exactly the keys >= thr.
struct TopkCut {
  uint32_t T, thr;
  int need_eq;
  bool fast;
};

// Keys of one lane's rows with 0 at positions >= n and every real key >= 1
// (key 0 is a NaN pattern; merging it with key 1, another NaN, changes no
// order that matters), so padding never falls in a key range [lo, hi]; and
// the wave's key range.
template <int R>
__device__ __forceinline__ void topk_prepare(const uint32_t (&kr)[R], int n, uint32_t (&kz)[R],
                                             uint32_t& lo, uint32_t& hi) {
  const int lane = lane_id();
  lo = 0xffffffffu;
  hi = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool valid = r * kWave + lane < n;
    kz[r] = valid ? max(kr[r], 1u) : 0u;
    if (valid) {
      lo = min(lo, kz[r]);
      hi = max(hi, kz[r]);
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
}

// The cut of a top-k (0 < k < n) over keys held by one wave: range-adaptive
// radix passes, each a histogram of the live key range [lo, hi] over BINS
// bins of LDS (hist: BINS words, 16-byte aligned, the wave's own; LDS
// operations of one wave complete in order, so it is read right after its
// atomics with no barrier), narrowing to the bin that holds the cut; once
// that bin holds at most kWaveRankMax keys they are ranked against each
// other instead.  Padding keys (0) never fall in the range.
template <int R, int BINS>
__device__ __forceinline__ TopkCut wave_topk_cut(const uint32_t (&kz)[R], int n, int k,
                                                 uint32_t lo, uint32_t hi, uint32_t* hist) {
  constexpr int LOG_BINS = BINS == 256 ? 8 : BINS == 512 ? 9 : BINS == 1024 ? 10 : 11;
  static_assert((1 << LOG_BINS) == BINS && BINS <= 2048 && BINS >= 256, "bins");
  const int lane = lane_id();
  // state: [lo, hi] holds the cut, `need` more keys come from it, and it
  // holds in_range keys (need <= in_range)
  int need = k, in_range = n;
  TopkCut cut{0u, 0u, 0, false};
#pragma unroll 1
  while (true) {
    if (need == in_range) {  // the whole range is taken
      cut.thr = lo;
      cut.fast = true;
      return cut;
    }
    if (lo == hi) {
      cut.T = lo;
      cut.need_eq = need;
      return cut;
    }
    if (in_range <= kWaveRankMax) {
      const uint3 c = wave_rank_range(kz, n, lo, hi, need, hist);
      cut.T = cut.thr = c.x;
      cut.need_eq = int(c.y);
      cut.fast = c.y == c.z;
      return cut;
    }
    const int span_bits = 32 - __clz(int(hi - lo));
    const int shift = span_bits > LOG_BINS ? span_bits - LOG_BINS : 0;
#pragma unroll
    for (int j = 0; j < BINS / kWave; j += 4)
      *reinterpret_cast<uint4*>(hist + lane * (BINS / kWave) + j) = make_uint4(0u, 0u, 0u, 0u);
    const uint32_t span = hi - lo;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // one unsigned compare tests lo <= key <= hi; padding zeros fall out
      const uint32_t off = kz[r] - lo;
      if (off <= span) atomicAdd(&hist[off >> shift], 1u);
    }
    const int3 f = wave_find_bin<BINS>(hist, need);
    const uint32_t blo = lo + (uint32_t(f.x) << shift);
    const uint64_t bhi = uint64_t(blo) + ((uint64_t(1) << shift) - 1u);
    hi = bhi < uint64_t(hi) ? uint32_t(bhi) : hi;
    lo = blo;
    need = f.y;
    in_range = f.z;
  }
}

// Emission of a cut by one wave: calls emit(rank, position) for the selected
// keys whose rank lies in [rank_lo, rank_hi); the rows' selection masks come
// first, so rows outside that rank window are skipped whole.
template <int R, typename EmitFn>
__device__ __forceinline__ void wave_emit_cut(const uint32_t (&kz)[R], int n, const TopkCut& cut,
                                              const EmitFn& emit, int rank_lo, int rank_hi) {
  const int lane = lane_id();
  const unsigned long long below = (1ull << lane) - 1ull;
  if (cut.fast) {
    unsigned long long sm[R];  // padding zeros fall below the threshold (>= 1)
#pragma unroll
    for (int r = 0; r < R; ++r) sm[r] = ballot(kz[r] >= cut.thr);
    int base = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int cnt = __popcll(sm[r]);
      if (cnt > 0 && base < rank_hi && base + cnt > rank_lo) {
        const int rank = base + __popcll(sm[r] & below);
        if (((sm[r] >> lane) & 1ull) && rank >= rank_lo && rank < rank_hi)
          emit(rank, r * kWave + lane);
      }
      base += cnt;
    }
    return;
  }
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = r * kWave + lane;
    const bool eq = i < n && kz[r] == cut.T;
    const unsigned long long em = ballot(eq);
    const bool sel =
        (i < n && kz[r] > cut.T) || (eq && eq_seen + int(__popcll(em & below)) < cut.need_eq);
    const unsigned long long sm = ballot(sel);
    const int rank = base + __popcll(sm & below);
    if (sel && rank >= rank_lo && rank < rank_hi) emit(rank, i);
    base += __popcll(sm);
    eq_seen += __popcll(em);
  }
}

// Top-k by one wave over n <= 64*R keys held in registers: lane l holds the
// key of position l + 64 r in kr[r] (positions >= n are ignored).  Same
// selection and emission order as wg_topk (every key above the threshold,
// then the keys equal to it in position order); emit(rank, position) is
// called for ranks in [rank_lo, rank_hi) only.  hist: 256 words of LDS,
// 16-byte aligned, the wave's own.
template <int R, typename EmitFn>
__device__ __forceinline__ void wave_topk(const uint32_t (&kr)[R], int n, int k, const EmitFn& emit,
                                          uint32_t* hist, int rank_lo = 0, int rank_hi = 1 << 30) {
  if (k <= 0) return;
  if (k >= n) {
    const int lane = lane_id();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = r * kWave + lane;
      if (i < n && i >= rank_lo && i < rank_hi) emit(i, i);
    }
    return;
  }
  uint32_t kz[R], lo, hi;
  topk_prepare(kr, n, kz, lo, hi);
  const TopkCut cut = wave_topk_cut<R, 256>(kz, n, k, lo, hi, hist);
  wave_emit_cut(kz, n, cut, emit, rank_lo, rank_hi);
}

// One wave's top-k over n <= 16*64 keys read through key(i), with the
// register rows sized to n (4, 8, 12 or 16 rows of 64 keys), since the
// passes and the emission cost per row.
template <int R, typename KeyFn, typename EmitFn>
__device__ __forceinline__ void wave_topk_load(const KeyFn& key, int n, int k, const EmitFn& emit,
                                               uint32_t* hist, int rank_lo, int rank_hi) {
  const int lane = lane_id();
  // every read unconditional (positions past n re-read key n-1 and are masked
  // later), so all R are in flight together rather than each behind a branch
  uint32_t kr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) kr[r] = key(min(r * kWave + lane, n - 1));
  wave_topk<R>(kr, n, k, emit, hist, rank_lo, rank_hi);
}
template <typename KeyFn, typename EmitFn>
__device__ __forceinline__ void wave_topk_rows(const KeyFn& key, int n, int k, const EmitFn& emit,
                                               uint32_t* hist, int rank_lo, int rank_hi) {
  const int rows = (n + kWave - 1) / kWave;
  if (rows <= 4)
    wave_topk_load<4>(key, n, k, emit, hist, rank_lo, rank_hi);
  else if (rows <= 8)
    wave_topk_load<8>(key, n, k, emit, hist, rank_lo, rank_hi);
  else if (rows <= 12)
    wave_topk_load<12>(key, n, k, emit, hist, rank_lo, rank_hi);
  else
    wave_topk_load<16>(key, n, k, emit, hist, rank_lo, rank_hi);
}

// Most keys one wave emits; above it the workgroup emits (scan based).
constexpr int kWaveEmitMax = 1024;

template <int NT, int BINS, int NBUF, typename KeyFn, typename EmitFn>
__device__ __forceinline__ void wg_topk(const KeyFn& key, int n, int k, const EmitFn& emit,
                                        TopkSmem<NT, BINS, NBUF>& sm, bool have_range = false,
                                        uint32_t lo_in = 0xffffffffu, uint32_t hi_in = 0u,
                                        uint32_t* cand = nullptr, int cand_cap = 0) {
  constexpr int NW = NT / kWave;
  constexpr int LOG_BINS = BINS == 256 ? 8 : BINS == 512 ? 9 : BINS == 1024 ? 10 : 11;
  static_assert(BINS % NT == 0 || NT % BINS == 0, "bins");
  static_assert((1 << LOG_BINS) == BINS && BINS <= 2048 && BINS >= 256, "bins");
  const int t = threadIdx.x;
  const int wave = t / kWave;
  const int lane = lane_id();
  if (k <= 0) return;
  if (k >= n) {
    for (int i = t; i < n; i += NT) emit(i, i);
    return;
  }
  // key range: this thread's share of it from the caller (have_range) or
  // from a pass over the keys
  uint32_t lo = lo_in, hi = hi_in;
  if (!have_range) {
    for (int i = t; i < n; i += NT) {
      const uint32_t kk = key(i);
      lo = min(lo, kk);
      hi = max(hi, kk);
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    sm.red[wave] = lo;
    sm.red[NW + wave] = hi;
  }
  for (int b = t; b < BINS; b += NT) sm.hist[0][b] = 0u;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = min(lo, sm.red[w]);
    hi = max(hi, sm.red[NW + w]);
  }
  int need = k;      // keys still to take among the candidates [lo, hi]
  int in_range = n;  // candidates in [lo, hi]
  uint32_t T;        // threshold: keys above are taken, need_eq of the keys equal to it
  int need_eq;
  bool all_eq;       // every key equal to T is taken: the choice is key >= T
  // histogram order: lane l of a wave walks an odd-length run of positions,
  // so one instruction's lanes touch keys far apart
  const int rows = ((n + kWave - 1) / kWave) | 1;
  // with a candidate buffer (cand_cap words of LDS), the second pass also
  // gathers its candidates there when they fit, and later passes read only
  // them instead of all n keys
  bool from_cand = false;
  if (t == 0) sm.n_cand = 0;
#pragma unroll 1
  for (int pass = 0;; ++pass) {
    if (lo == hi) {  // every candidate has one value
      T = lo;
      need_eq = need;
      all_eq = need == in_range;
      break;
    }
    const int span_bits = 32 - __clz(int(hi - lo));
    const int shift = span_bits > LOG_BINS ? span_bits - LOG_BINS : 0;
    uint32_t* h = sm.hist[pass % NBUF];
    if (pass > 0) {
      if (NBUF == 1) __syncthreads();  // every wave has read the last histogram
      for (int b = t; b < BINS; b += NT) h[b] = 0u;
      __syncthreads();
    }
    const bool gather = cand && pass == 1 && in_range <= cand_cap;
    if (from_cand) {  // the gathered keys of the second pass's range hold this one's
      const int nc = sm.n_cand;
      for (int i = t; i < nc; i += NT) {
        const uint32_t kk = cand[i];
        if (kk >= lo && kk <= hi) atomicAdd(&h[(kk - lo) >> shift], 1u);
      }
    } else {
      // UR keys of a lane read before any is used (one LDS round trip per UR)
      constexpr int UR = 8;
      for (int c0 = wave; c0 < rows; c0 += NW * UR) {
        uint32_t kr[UR];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
          const int i = lane * rows + c0 + u * NW;
          kr[u] = c0 + u * NW < rows && i < n ? key(i) : 0u;
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) {
          const int i = lane * rows + c0 + u * NW;
          const uint32_t kk = kr[u];
          if (c0 + u * NW < rows && i < n && kk >= lo && kk <= hi) {
            atomicAdd(&h[(kk - lo) >> shift], 1u);
            if (gather) cand[atomicAdd(&sm.n_cand, 1)] = kk;  // order is irrelevant to counts
          }
        }
      }
    }
    from_cand = from_cand || gather;
    __syncthreads();
    int3 f;
    if constexpr (NW > 4) {
      // one wave walks the histogram and shares the result: with several
      // waves per SIMD, redundant walks would queue behind each other
      if (wave == 0) {
        f = wave_find_bin<BINS>(h, need);
        if (lane == 0) {
          sm.tmp[0] = f.x;
          sm.tmp[1] = f.y;
          sm.tmp[2] = f.z;
        }
      }
      __syncthreads();
      f = make_int3(sm.tmp[0], sm.tmp[1], sm.tmp[2]);
    } else {
      f = wave_find_bin<BINS>(h, need);
    }
    const uint32_t blo = lo + (uint32_t(f.x) << shift);
    if (shift == 0) {  // the boundary bin is one key value
      T = blo;
      need_eq = f.y;
      all_eq = f.y == f.z;
      break;
    }
    if (f.y == f.z) {
      // the whole bin is taken: the selection is every key >= blo (keys above
      // the candidate interval were taken by earlier passes)
      T = blo;
      need_eq = f.y;
      all_eq = true;
      break;
    }
    const uint64_t bhi = uint64_t(blo) + ((uint64_t(1) << shift) - 1u);
    hi = bhi < uint64_t(hi) ? uint32_t(bhi) : hi;
    lo = blo;
    need = f.y;
    in_range = f.z;
  }
  if (n <= kWaveEmitMax) {
    if (wave == 0) {
      if (all_eq)  // keys >= T: keys above T - 1 (T >= 1 here, else all n keys would be taken)
        wave_topk_emit(key, n, T - 1u, 0, emit);
      else
        wave_topk_emit(key, n, T, need_eq, emit);
    }
  } else {
    wg_topk_emit<NT>(key, n, T, need_eq, all_eq, emit, sm.tmp);
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

// Wave-wide reductions (all 64 lanes take part, every lane gets the result):
// within each 16-lane row by DPP (the ALU's own lane moves), then the four
// row results read as scalars, in row order; no LDS permutes in the chain.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false)));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (a + b) + (c + d);
}

}  // namespace rk

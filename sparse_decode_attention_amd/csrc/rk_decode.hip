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
// Three launches per call:
//   hsa_select  one workgroup per unit: channel sums, top-k1, page scores
//               over the k1 sign-selected aux rows (coalesced row reads), top-k2
//   hsa_attn    split-K over the selected pages: a wave streams whole pages,
//               16-byte K/V loads, online softmax in the exp2 domain, one
//               partial (m, l, o[d]) per head per workgroup
//   hsa_combine merges the partials of each head in split order.
// HBM-bound: bytes per unit = q + k1*nblk aux elements + 2*d*|T| K/V elements.
#include <math.h>

#include "rk_device.hpp"
#include "rk_internal.hpp"

namespace rk {
namespace {

constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void hsa_select_kernel(
    const T* __restrict__ q, const T* __restrict__ kmax, const T* __restrict__ kmin,
    int64_t nblk_cap, int nblk, int k1, int nsel, int32_t* __restrict__ sel_ws,
    int32_t* __restrict__ sel_opt, int32_t* __restrict__ chan_opt, float* __restrict__ s1_opt) {
  extern __shared__ uint32_t page_keys[];  // [nblk]
  __shared__ uint32_t chan_keys[D];
  __shared__ float qbar[D];
  __shared__ int i1[D];
  __shared__ TopkSmem<256> sm;

  const int u = blockIdx.x;
  const int t = threadIdx.x;
  if (t < D) {
    float a = 0.f, qb = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {  // g ascending, float32, as the group sums are defined
      const float x = to_f32(q[(size_t(u) * G + g) * D + t]);
      a = __fadd_rn(a, fabsf(x));
      qb = __fadd_rn(qb, x);
    }
    chan_keys[t] = order_key(a);
    qbar[t] = qb;
  }
  __syncthreads();
  wg_topk<256>([&](int i) { return chan_keys[i]; }, D, k1, [&](int r, int i) { i1[r] = i; }, sm);
  __syncthreads();
  if (chan_opt)
    for (int j = t; j < k1; j += 256) chan_opt[size_t(u) * k1 + j] = i1[j];

  const T* xu = kmax + size_t(u) * D * size_t(nblk_cap);
  const T* nu = kmin + size_t(u) * D * size_t(nblk_cap);
  for (int b = t; b < nblk; b += 256) {
    // one rounded multiply and one rounded add per term: no fused multiply-add
#pragma clang fp contract(off)
    float s = 0.f;
    for (int j = 0; j < k1; ++j) {
      const int ch = i1[j];
      const float qv = qbar[ch];
      const T* row = (qv >= 0.f ? xu : nu) + size_t(ch) * nblk_cap;
      const float prod = qv * to_f32(row[b]);
      s = s + prod;
    }
    page_keys[b] = order_key(s);
    if (s1_opt) s1_opt[size_t(u) * nblk + b] = s;
  }
  __syncthreads();
  int32_t* su = sel_ws + size_t(u) * nsel;
  int32_t* so = sel_opt ? sel_opt + size_t(u) * nsel : nullptr;
  wg_topk<256>(
      [&](int i) { return page_keys[i]; }, nblk, nsel,
      [&](int r, int i) {
        su[r] = i;
        if (so) so[r] = i;
      },
      sm);
}

// One workgroup = 4 waves; a wave streams whole pages.  Lanes split a row into
// LPR 16-byte chunks, so SLOTS tokens are in flight per wave and each slot
// takes TPS tokens per chunk before one softmax rescale.
template <typename T, int D, int G, bool MT>
__global__ __launch_bounds__(256) void hsa_attn_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t kv_cap,
    const int32_t* __restrict__ cand, int64_t cand_stride, const int32_t* __restrict__ sel,
    int nsel, int pages_per_split, int n_split, int n_tokens, int block, float scale_log2,
    float* __restrict__ partials) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPR = D / EPL;
  constexpr int SLOTS = kWave / LPR;
  constexpr int TPS = 4;
  constexpr int CHUNK = SLOTS * TPS;
  constexpr int NW = 4;
  static_assert(kWave % LPR == 0, "row chunks must tile a wave");
  __shared__ float wm[NW][G], wl[NW][G];
  __shared__ float wo[NW][G][D];

  const int u = blockIdx.y;
  const int split = blockIdx.x;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int slot = lane / LPR;
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

  const T* ku = k + size_t(u) * size_t(kv_cap) * D + c * EPL;
  const T* vu = v + size_t(u) * size_t(kv_cap) * D + c * EPL;
  const int32_t* cu = MT ? cand + size_t(u) * size_t(cand_stride) : nullptr;
  const int32_t* su = sel + size_t(u) * nsel;
  const int e0 = split * pages_per_split;
  const int e1 = min(e0 + pages_per_split, nsel);

  for (int e = e0 + wave; e < e1; e += NW) {
    const int t0 = su[e] * block;
    const int t1 = min(t0 + block, n_tokens);
    for (int tc = t0; tc < t1; tc += CHUNK) {
      Vec16<T> kr[TPS], vr[TPS];
      bool ok[TPS];
#pragma unroll
      for (int i = 0; i < TPS; ++i) {
        const int tok = tc + slot + SLOTS * i;
        ok[i] = tok < t1;
        const int row = ok[i] ? (MT ? clamp_row(cu[tok], kv_cap) : tok) : 0;
        if (ok[i]) {
          kr[i] = load16(ku + size_t(row) * D);
          vr[i] = load16(vu + size_t(row) * D);
        } else {
          kr[i].raw = {};
          vr[i].raw = {};
        }
      }
      float x[G][TPS];
#pragma unroll
      for (int i = 0; i < TPS; ++i) {
        float kf[EPL];
        unpack16(kr[i], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float s = 0.f;
#pragma unroll
          for (int ee = 0; ee < EPL; ++ee) s += qf[g][ee] * kf[ee];
#pragma unroll
          for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off);
          x[g][i] = s * scale_log2;
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float cm = kNegBig;
#pragma unroll
        for (int i = 0; i < TPS; ++i)
          if (ok[i]) cm = fmaxf(cm, x[g][i]);
        const float mn = fmaxf(m[g], cm);
        const float corr = exp2f(m[g] - mn);
        float p[TPS];
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < TPS; ++i) {
          p[i] = ok[i] ? exp2f(x[g][i] - mn) : 0.f;
          ps += p[i];
        }
        l[g] = l[g] * corr + ps;
        m[g] = mn;
#pragma unroll
        for (int ee = 0; ee < EPL; ++ee) {
          float acc = o[g][ee] * corr;
#pragma unroll
          for (int i = 0; i < TPS; ++i) acc += p[i] * vr[i].get(ee);
          o[g][ee] = acc;
        }
      }
    }
  }

  // merge the SLOTS token slots of the wave (lanes that share a channel chunk)
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float a = exp2f(m[g] - mn), b = exp2f(mo - mn);
      l[g] = l[g] * a + lo * b;
#pragma unroll
      for (int ee = 0; ee < EPL; ++ee) {
        const float oo = __shfl_xor(o[g][ee], off);
        o[g][ee] = o[g][ee] * a + oo * b;
      }
      m[g] = mn;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (c == 0) {
        wm[wave][g] = m[g];
        wl[wave][g] = l[g];
      }
#pragma unroll
      for (int ee = 0; ee < EPL; ++ee) wo[wave][g][c * EPL + ee] = o[g][ee];
    }
  }
  __syncthreads();
  // merge the 4 waves in order and write this split's partial per head
  float* pu = partials + (size_t(u) * n_split + split) * G * (D + 2);
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int g = idx / D;
    const int ch = idx % D;
    float mm = kNegBig;
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, wm[w][g]);
    float ll = 0.f, oo = 0.f;
    for (int w = 0; w < NW; ++w) {
      const float a = exp2f(wm[w][g] - mm);
      ll += wl[w][g] * a;
      oo += wo[w][g][ch] * a;
    }
    float* pg = pu + size_t(g) * (D + 2);
    pg[2 + ch] = oo;
    if (ch == 0) {
      pg[0] = mm;
      pg[1] = ll;
    }
  }
}

template <int D, int G>
__global__ __launch_bounds__(256) void hsa_combine_kernel(const float* __restrict__ partials,
                                                          int n_split, float* __restrict__ out) {
  const int u = blockIdx.x;
  const float* pu = partials + size_t(u) * n_split * G * (D + 2);
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int g = idx / D;
    const int ch = idx % D;
    float mm = kNegBig;
    for (int s = 0; s < n_split; ++s) mm = fmaxf(mm, pu[(size_t(s) * G + g) * (D + 2)]);
    float ll = 0.f, oo = 0.f;
    for (int s = 0; s < n_split; ++s) {
      const float* pg = pu + (size_t(s) * G + g) * (D + 2);
      const float a = exp2f(pg[0] - mm);
      ll += pg[1] * a;
      oo += pg[2 + ch] * a;
    }
    out[(size_t(u) * G + g) * D + ch] = oo / ll;
  }
}

template <typename T, int D, int G>
hipError_t launch_decode_t(const Dims& d, const void* q, const void* k, const void* v,
                           int64_t kv_cap, const int32_t* cand, int64_t cand_stride,
                           const void* kmax, const void* kmin, int64_t nblk_cap,
                           int64_t n_tokens, int block, int k1, int k2, float* out,
                           int32_t* sel_opt, int32_t* chan_opt, float* s1_opt, void* ws,
                           hipStream_t s) {
  const int nblk = int((n_tokens + block - 1) / block);
  const DecodeWs lay = decode_ws_layout(d, nblk, k2);
  char* wsb = static_cast<char*>(ws);
  int32_t* sel = reinterpret_cast<int32_t*>(wsb + lay.sel);
  float* part = reinterpret_cast<float*>(wsb + lay.partials);
  const int units = d.units();

  const size_t lds = size_t(nblk) * sizeof(uint32_t);
  hipLaunchKernelGGL((hsa_select_kernel<T, D, G>), dim3(units), dim3(256), lds, s,
                     static_cast<const T*>(q), static_cast<const T*>(kmax),
                     static_cast<const T*>(kmin), nblk_cap, nblk, k1, lay.nsel, sel, sel_opt,
                     chan_opt, s1_opt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // split-K sizing: aim for ~2048 workgroups over the whole launch, at least
  // kMinPagesPerSplit pages (one per wave) per workgroup
  const int64_t total_pages = int64_t(units) * lay.nsel;
  int pps = int((total_pages + 2047) / 2048);
  pps = pps < kMinPagesPerSplit ? kMinPagesPerSplit : pps;
  pps = (pps + 3) / 4 * 4;
  const int n_split = (lay.nsel + pps - 1) / pps;
  const float scale_log2 = float(1.4426950408889634 / sqrt(double(D)));
  if (cand)
    hipLaunchKernelGGL((hsa_attn_kernel<T, D, G, true>), dim3(n_split, units), dim3(256), 0, s,
                       static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), kv_cap, cand, cand_stride, sel, lay.nsel, pps,
                       n_split, int(n_tokens), block, scale_log2, part);
  else
    hipLaunchKernelGGL((hsa_attn_kernel<T, D, G, false>), dim3(n_split, units), dim3(256), 0, s,
                       static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), kv_cap, cand, cand_stride, sel, lay.nsel, pps,
                       n_split, int(n_tokens), block, scale_log2, part);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((hsa_combine_kernel<D, G>), dim3(units), dim3(256), 0, s, part, n_split,
                     out);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_d(const Dims& d, const void* q, const void* k, const void* v,
                           int64_t kv_cap, const int32_t* cand, int64_t cand_stride,
                           const void* kmax, const void* kmin, int64_t nblk_cap,
                           int64_t n_tokens, int block, int k1, int k2, float* out,
                           int32_t* sel_opt, int32_t* chan_opt, float* s1_opt, void* ws,
                           hipStream_t s) {
#define RK_DECODE_G(GG)                                                                        \
  case GG:                                                                                     \
    return launch_decode_t<T, D, GG>(d, q, k, v, kv_cap, cand, cand_stride, kmax, kmin,       \
                                     nblk_cap, n_tokens, block, k1, k2, out, sel_opt,         \
                                     chan_opt, s1_opt, ws, s);
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
                             hipStream_t s) {
  if (d.bf16) {
    if (d.D == 128)
      return launch_decode_d<bf16_t, 128>(d, q, k, v, kv_cap, cand, cand_stride, kmax, kmin,
                                          nblk_cap, n_tokens, block, k1, k2, out, sel_opt,
                                          chan_opt, s1_opt, ws, s);
    return launch_decode_d<bf16_t, 64>(d, q, k, v, kv_cap, cand, cand_stride, kmax, kmin,
                                       nblk_cap, n_tokens, block, k1, k2, out, sel_opt,
                                       chan_opt, s1_opt, ws, s);
  }
  if (d.D == 128)
    return launch_decode_d<float, 128>(d, q, k, v, kv_cap, cand, cand_stride, kmax, kmin,
                                       nblk_cap, n_tokens, block, k1, k2, out, sel_opt,
                                       chan_opt, s1_opt, ws, s);
  return launch_decode_d<float, 64>(d, q, k, v, kv_cap, cand, cand_stride, kmax, kmin,
                                    nblk_cap, n_tokens, block, k1, k2, out, sel_opt, chan_opt,
                                    s1_opt, ws, s);
}

}  // namespace rk

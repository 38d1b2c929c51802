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
//   hsa_select  one workgroup per unit: channel sums and top-k1; the k1
//               sign-selected aux rows are staged into LDS with 16-byte loads
//               (one memory round trip), pages are scored from LDS, top-k2 by
//               radix select
//   hsa_attn    split-K over the selected pages: a wave streams whole pages
//               with 16-byte K/V loads, online softmax in the exp2 domain, one
//               partial (m, l, o[d]) per head per workgroup
//   hsa_combine one wave per (unit, head) merges the partials
// HBM-bound: bytes per unit = q + k1*nblk aux elements + 2*d*|T| K/V elements.
#include <math.h>

#include "rk_device.hpp"
#include "rk_internal.hpp"

namespace rk {
namespace {

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void hsa_select_kernel(
    const T* __restrict__ q, const T* __restrict__ kmax, const T* __restrict__ kmin,
    int64_t nblk_cap, int nblk, int k1, int nsel, int npc, int32_t* __restrict__ sel_ws,
    int32_t* __restrict__ sel_opt, int32_t* __restrict__ chan_opt,
    float* __restrict__ s1_opt) {
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  extern __shared__ __align__(16) unsigned char dyn_lds[];
  uint32_t* page_keys = reinterpret_cast<uint32_t*>(dyn_lds);  // [nblk rounded up to 4]
  T* stage = reinterpret_cast<T*>(dyn_lds + (size_t((nblk + 3) & ~3) * 4 + 15) / 16 * 16);
  __shared__ __align__(16) uint32_t chan_keys[D];
  __shared__ float qbar[D];
  __shared__ int i1[D];
  __shared__ __align__(16) float i1_q[D + 16];
  __shared__ int i1_off[D];  // element offset of the sign-selected row; < 0: Kmin
  __shared__ TopkSmem<256> sm;

  const int u = blockIdx.x;
  const int t = threadIdx.x;
  RK_PHASE(0);
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
  wg_topk_rank<256>(chan_keys, D, k1, [&](int r, int i) { i1[r] = i; }, sm.tmp);
  __syncthreads();
  RK_PHASE(8);
  const T* xu = kmax + size_t(u) * D * size_t(nblk_cap);
  const T* nu = kmin + size_t(u) * D * size_t(nblk_cap);
  for (int j = t; j < k1; j += 256) {
    const int ch = i1[j];
    const float qv = qbar[ch];
    i1_q[j] = qv;
    i1_off[j] = qv >= 0.f ? ch : -1 - ch;  // sign selects the Kmax or the Kmin row
    if (chan_opt) chan_opt[size_t(u) * k1 + j] = ch;
  }
  __syncthreads();

  // Pages in chunks of npc (a multiple of 8).  Staging: thread (channel j,
  // vector slot) fetches 16-byte runs of row j (EPV consecutive pages) with
  // all of its loads in flight, and scatters them transposed into LDS as
  // stage[page][channel] (row pitch k1p, a multiple of EPV plus one vector of
  // padding).  Scoring: s1[b] = sum over i1 (ascending) of q_bar_i * P_i[b],
  // read back as 16-byte vectors of channels.
  const int k1p = (k1 + 15) / 16 * 16 + EPV;  // 16-channel blocks plus one vector of padding
  const int groups = 256 / k1;  // vector slots per channel (k1 <= 128)
  for (int p0 = 0; p0 < nblk; p0 += npc) {
    const int np = min(npc, nblk - p0);
    const int nv = (np + EPV - 1) / EPV;  // vectors per row slice (stays inside nblk_cap)
    if (t < groups * k1) {
      const int j = t % k1;
      const int off = i1_off[j];
      const T* row = (off >= 0 ? xu + size_t(off) * nblk_cap : nu + size_t(-1 - off) * nblk_cap) + p0;
      constexpr int NB = 20;
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
    __syncthreads();
    RK_PHASE(9);
    {
      // Each thread scores up to 4 pages (b = t + 256 p) together.  Channels go
      // in blocks of 16: the block's q_bar values come from LDS once (float4
      // broadcasts) and each page's 16 staged values as 16-byte reads, so all
      // reads of a block are in flight before the ordered multiply-adds.
      // One rounded multiply and one rounded add per term: no fused multiply-add.
#pragma clang fp contract(off)
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      const T* sp[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) sp[p] = stage + size_t(min(t + 256 * p, np - 1)) * k1p;
      const int npp = np > t ? (np - t + 255) / 256 : 0;  // pages of this thread (<= 4 when np <= npc)
      for (int j0 = 0; j0 < k1; j0 += 16) {
        float qv[16];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float4 q4 = *reinterpret_cast<const float4*>(i1_q + j0 + 4 * x);
          qv[4 * x] = q4.x;
          qv[4 * x + 1] = q4.y;
          qv[4 * x + 2] = q4.z;
          qv[4 * x + 3] = q4.w;
        }
        float sv[4][16];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
#pragma unroll
          for (int x = 0; x < 16 / EPV; ++x) {
            const Vec16<T> vv = load16(sp[p] + j0 + x * EPV);
#pragma unroll
            for (int e = 0; e < EPV; ++e) sv[p][x * EPV + e] = vv.get(e);
          }
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          if (p < npp) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (j0 + e < k1) acc[p] = acc[p] + qv[e] * sv[p][e];
          }
        }
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int b = t + 256 * p;
        if (p < npp) {
          page_keys[p0 + b] = order_key(acc[p]);
          if (s1_opt) s1_opt[size_t(u) * nblk + p0 + b] = acc[p];
        }
      }
    }
    __syncthreads();
    RK_PHASE(10);
  }
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
  constexpr int TPS = G >= 4 ? 2 : 4;  // fewer tokens per step for wide groups (registers)
  constexpr int CHUNK = SLOTS * TPS;
  constexpr int NW = 4;
  constexpr int PF = D + 4;  // floats per head partial: m, l, pad, pad, o[D]
  static_assert(kWave % LPR == 0, "row chunks must tile a wave");
  __shared__ float wm[NW][G], wl[NW][G];
  __shared__ __align__(16) float wo[NW][G][D];

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
          x[g][i] = group_sum<LPR>(s) * scale_log2;
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float cm = kNegBig;
#pragma unroll
        for (int i = 0; i < TPS; ++i)
          if (ok[i]) cm = fmaxf(cm, x[g][i]);
        const float mn = fmaxf(m[g], cm);
        const float corr = fast_exp2(m[g] - mn);
        float p[TPS];
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < TPS; ++i) {
          p[i] = ok[i] ? fast_exp2(x[g][i] - mn) : 0.f;
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
  float* pu = partials + size_t(u) * n_split * G * PF;
  float* pw = pu + size_t(split) * G * PF;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int g = idx / D;
    const int ch = idx % D;
    float mm = kNegBig;
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, wm[w][g]);
    float ll = 0.f, oo = 0.f;
    for (int w = 0; w < NW; ++w) {
      const float a = fast_exp2(wm[w][g] - mm);
      ll += wl[w][g] * a;
      oo += wo[w][g][ch] * a;
    }
    float* pg = pw + size_t(g) * PF;
    pg[4 + ch] = oo;
    if (ch == 0) {
      pg[0] = mm;
      pg[1] = ll;
    }
  }
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
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = cls + i * CLASSES;
    const float w = __shfl(a, s < kWave ? s : 0);
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
                           hipStream_t s) {
  const int nblk = int((n_tokens + block - 1) / block);
  const DecodeWs lay = decode_ws_layout(d, nblk, k2);
  char* wsb = static_cast<char*>(ws);
  int32_t* sel = reinterpret_cast<int32_t*>(wsb + lay.sel);
  float* part = reinterpret_cast<float*>(wsb + lay.partials);
  const int units = d.units();

  // LDS of the select workgroup: page keys, then the staged aux slices
  const size_t keys_bytes = (size_t((nblk + 3) & ~3) * 4 + 15) / 16 * 16;
  const size_t stage_budget = kSelectLdsBudget - keys_bytes;
  constexpr int EPV = 16 / sizeof(T);
  const int k1p = (k1 + 15) / 16 * 16 + EPV;
  int npc = int(stage_budget / (size_t(k1p) * sizeof(T))) / 8 * 8;
  npc = npc > 1024 ? 1024 : npc;  // at most 4 pages per scoring thread
  const int nblk8 = (nblk + 7) / 8 * 8;
  npc = npc > nblk8 ? nblk8 : npc;
  if (npc < 8) return hipErrorInvalidValue;
  const size_t lds = keys_bytes + size_t(k1p) * npc * sizeof(T);
  static bool attr_set = false;  // once per template instantiation
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&hsa_select_kernel<T, D, G>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       int(kSelectLdsBudget));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  RK_LAUNCH("hsa_select", (hsa_select_kernel<T, D, G>), dim3(units), dim3(256), lds, s,
            static_cast<const T*>(q), static_cast<const T*>(kmax), static_cast<const T*>(kmin),
            nblk_cap, nblk, k1, lay.nsel, npc, sel, sel_opt, chan_opt, s1_opt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // split-K sizing: aim for ~2048 workgroups over the whole launch, at least
  // kMinPagesPerSplit pages (one per wave) and at most kMaxSplits splits per unit
  const int64_t total_pages = int64_t(units) * lay.nsel;
  int pps = int((total_pages + 2047) / 2048);
  pps = pps < kMinPagesPerSplit ? kMinPagesPerSplit : pps;
  const int pps_cap = (lay.nsel + kMaxSplits - 1) / kMaxSplits;
  pps = pps < pps_cap ? pps_cap : pps;
  pps = (pps + 3) / 4 * 4;
  const int n_split = (lay.nsel + pps - 1) / pps;
  const float scale_log2 = float(1.4426950408889634 / sqrt(double(D)));
  if (cand)
    RK_LAUNCH("hsa_attn_mt", (hsa_attn_kernel<T, D, G, true>), dim3(n_split, units), dim3(256), 0,
              s, static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
              kv_cap, cand, cand_stride, sel, lay.nsel, pps, n_split, int(n_tokens), block,
              scale_log2, part);
  else
    RK_LAUNCH("hsa_attn", (hsa_attn_kernel<T, D, G, false>), dim3(n_split, units), dim3(256), 0,
              s, static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
              kv_cap, cand, cand_stride, sel, lay.nsel, pps, n_split, int(n_tokens), block,
              scale_log2, part);
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

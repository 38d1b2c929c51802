// rk_internal.hpp -- host-side interface between the C ABI (rk_api.hip) and the
// kernel launchers.  Arguments are validated by the caller; launchers only
// pick a kernel instance and a grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rk {

// Largest page count whose top-k runs inside the attention workgroups, from
// keys held in LDS (4 bytes each).  Beyond it (and for token-level scoring
// over key rows) a select launch of its own writes the chosen pages, which
// the attention workgroups then read; kMaxPagesGlobal bounds that path.
constexpr int64_t kMaxPages = 12288;
constexpr int64_t kMaxPagesGlobal = int64_t(1) << 22;
// Stage-1 column tile of the window-score passes (partials are sized by it).
constexpr int kWsTile = 64;
// Pages handled by one attention workgroup at least (split-K granularity),
// and the most workgroups one unit's attention is split over.
constexpr int kComputeUnits = 256;  // MI355X
constexpr int kMinPagesPerSplit = 4;
constexpr int kMaxSplits = 64;
// Stage-1 selection keeps the order keys of up to this many bytes in LDS
// (160 KB per workgroup on gfx950, minus the radix histogram and scan space).
constexpr size_t kSelectKeysLds = 160 * 1024 - 10 * 1024;
// LDS budget of the page-scoring workgroup (gfx950: 160 KB per workgroup).
constexpr size_t kSelectLdsBudget = 160 * 1024 - 16 * 1024;
// Page scoring fetches every channel's Kmax and Kmin rows (not only the k1
// chosen ones) when they total at most this many bytes over the launch.
constexpr size_t kScoreAllBytes = size_t(8) << 20;
// Up to this many pages the attention workgroup's page top-k runs in one
// wave from registers (a multiple of 64).
constexpr int kWaveTopkPages = 1024;
// Decode calls with at least this many units (the units alone fill the 256
// CUs), or with at most one chosen page per wave, run steps 2 and 3 in one
// workgroup per unit, with at most this much dynamic LDS per workgroup.
constexpr int kFusedMinUnits = 160;
constexpr int kFusedThreads = 1024;
// Workgroup size of the large-batch fused decode for groups of four heads.
constexpr int kFusedThreadsWide = 512;
constexpr size_t kFusedLdsBudget = 144 * 1024;
// Dynamic LDS of an attention workgroup at most: the unit's page keys and the
// pages of its split, kMaxPages 4-byte entries each.
constexpr size_t kAttnDynLds = size_t(2 * kMaxPages) * 4;

struct Dims {
  int B, Hq, Hkv, G, D;
  bool bf16;
  int units() const { return B * Hkv; }
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---- workspace layouts (shared by *_workspace_bytes and the calls) ----
struct EvictWs {
  size_t partials, stats, scores, pooled, total;
  int n_tiles, m_rows;
};
inline EvictWs evict_ws_layout(const Dims& d, int64_t S, int W) {
  EvictWs w{};
  w.m_rows = d.G * W;
  w.n_tiles = int((S + kWsTile - 1) / kWsTile);
  const size_t u = size_t(d.units());
  size_t off = 0;
  w.partials = off; off += align256(u * w.n_tiles * w.m_rows * 2 * sizeof(float));
  w.stats = off;    off += align256(u * w.m_rows * 2 * sizeof(float));
  w.scores = off;   off += align256(u * size_t(S - W) * sizeof(float));
  w.pooled = off;   off += align256(u * size_t(S - W) * sizeof(float));
  w.total = off;
  return w;
}

// Split-K partial of one head: m, l, two pad floats, then o[D] (16-byte aligned).
inline int partial_floats(int D) { return D + 4; }

struct DecodeWs {
  size_t keys, partials, sel, total;
  int n_split_max, nsel, keys_pitch;
};
inline DecodeWs decode_ws_layout(const Dims& d, int64_t nblk, int k2) {
  DecodeWs w{};
  w.nsel = int(nblk < k2 ? nblk : k2);
  w.keys_pitch = int((nblk + 3) & ~int64_t(3));
  const int by_pages = (w.nsel + kMinPagesPerSplit - 1) / kMinPagesPerSplit;
  w.n_split_max = by_pages < kMaxSplits ? by_pages : kMaxSplits;
  const size_t u = size_t(d.units());
  size_t off = 0;
  w.keys = off;     off += align256(u * size_t(w.keys_pitch) * sizeof(uint32_t));
  w.partials = off; off += align256(u * w.n_split_max * d.G * partial_floats(d.D) * sizeof(float));
  w.sel = off;      off += align256(u * size_t(w.nsel) * sizeof(int32_t));  // chosen pages (select launch)
  w.total = off;
  return w;
}

// ---- kernel timing (rk_profile_begin / rk_profile_end) ----
bool prof_enabled();
void prof_before(const char* name, hipStream_t s);
void prof_after(hipStream_t s);

// Launch a kernel; when kernel timing is on, bracket it with HIP events on
// its stream.  `kern` must be parenthesised if it contains commas.
#define RK_LAUNCH(name, kern, grid, block, lds, stream, ...)        \
  do {                                                              \
    const bool rk_prof_on_ = ::rk::prof_enabled();                  \
    if (rk_prof_on_) ::rk::prof_before(name, stream);               \
    hipLaunchKernelGGL(kern, grid, block, lds, stream, __VA_ARGS__); \
    if (rk_prof_on_) ::rk::prof_after(stream);                      \
  } while (0)

// Paged K/V: a pool of physical pages [n_phys, Hkv, P, D] (P = 1 << shift
// tokens) shared by the batch; token n of sequence b, head h lives at pool
// row (table[b * table_stride + n / P] * Hkv + h) * P + n % P.  Page numbers
// are clamped into [0, n_phys) in-kernel.
struct PagedArgs {
  const int32_t* table;
  int64_t table_stride;
  int64_t n_phys;
  int shift;
  int hkv;
};

// ---- launchers ----
hipError_t launch_build_aux(const Dims& d, const void* k, int64_t k_cap, const int32_t* idx,
                            int64_t idx_stride, int64_t n_tokens, int64_t first_block,
                            int block, void* kmax, void* kmin, int64_t nblk_cap,
                            hipStream_t s, const PagedArgs* paged = nullptr);

hipError_t launch_append_kv(const Dims& d, const void* k_new, const void* v_new, void* k, void* v,
                            int64_t kv_cap, int64_t pos, void* kmax, void* kmin,
                            int64_t nblk_cap, int block, hipStream_t s,
                            const PagedArgs* paged = nullptr);

// Rows [first, first + n) of a dense [B, Hkv, src_cap, D] cache written to
// the same token positions of a paged pool (bf16).
hipError_t launch_paged_write(const Dims& d, const void* k_src, const void* v_src, int64_t src_cap,
                              int64_t first, int64_t n, void* k_pool, void* v_pool,
                              const PagedArgs& paged, hipStream_t s);

// A decode step that first appends token n_tokens - 1 (rk_append_kv's
// effect): the new rows and the buffers it writes.
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k;
  void* v;
  void* kmax;
  void* kmin;
};

// exact_rows: page scores are the exact group logits q_bar . k_n over the
// key rows (pages of one token, every channel; kmax/kmin unused), the
// Exact-TopK selection; otherwise HSA step 2 over kmax/kmin.
hipError_t launch_hsa_decode(const Dims& d, const void* q, const void* k, const void* v,
                             int64_t kv_cap, const int32_t* cand, int64_t cand_stride,
                             const void* kmax, const void* kmin, int64_t nblk_cap,
                             int64_t n_tokens, int block, int k1, int k2, float* out,
                             int32_t* sel_opt, int32_t* chan_opt, float* s1_opt, void* ws,
                             hipStream_t s, const AppendArgs* app = nullptr,
                             bool exact_rows = false, const PagedArgs* paged = nullptr,
                             const int32_t* lens = nullptr);

hipError_t launch_snapkv_evict(const Dims& d, const void* q_win, const void* k, const void* v,
                               int64_t kv_cap, int64_t S, int W, int pool_kernel, int pool_op,
                               int64_t n_keep, int32_t* kept, void* k_out, void* v_out,
                               int64_t out_cap, float* pooled_opt, void* kmax, void* kmin,
                               int64_t nblk_cap, int block, void* ws, hipStream_t s,
                               int32_t* ada_counts = nullptr);

}  // namespace rk

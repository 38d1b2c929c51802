// rk_api.hip -- the C ABI of librocketkv.so: argument validation, workspace
// sizing, the host-side split arithmetic and dispatch to the HIP launchers.
// The contract of every entry point is documented in include/rocketkv.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/rocketkv.h"
#include "rk_internal.hpp"

namespace {

thread_local std::string g_last_error;

rk_status fail(rk_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
rk_status fail(rk_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

rk_status device_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return RK_OK;
  return fail(RK_EDEVICE, "%s: %s", what, hipGetErrorString(err));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every device entry point.
rk_status check_shape(const rk_shape* sh, rk::Dims* d) {
  if (!sh) return fail(RK_EINVAL, "shape is NULL");
  if (sh->batch < 1 || sh->n_q_heads < 1 || sh->n_kv_heads < 1 || sh->head_dim < 1)
    return fail(RK_EINVAL, "batch, heads and head_dim must be positive");
  if (sh->n_q_heads % sh->n_kv_heads)
    return fail(RK_EINVAL, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                sh->n_q_heads, sh->n_kv_heads);
  if (sh->dtype != RK_F32 && sh->dtype != RK_BF16) return fail(RK_EINVAL, "unknown dtype");
  if (sh->head_dim != 64 && sh->head_dim != 128)
    return fail(RK_EUNSUPPORTED, "head_dim %d not built (64, 128)", sh->head_dim);
  if (int64_t(sh->batch) * sh->n_kv_heads > 65535)
    return fail(RK_EUNSUPPORTED, "batch * n_kv_heads above 65535");
  d->B = sh->batch;
  d->Hq = sh->n_q_heads;
  d->Hkv = sh->n_kv_heads;
  d->G = sh->n_q_heads / sh->n_kv_heads;
  d->D = sh->head_dim;
  d->bf16 = sh->dtype == RK_BF16;
  return RK_OK;
}

rk_status check_ws(void* ws, size_t have, size_t need) {
  if (need && !ws) return fail(RK_EINVAL, "workspace is NULL");
  if (have < need) return fail(RK_EWORKSPACE, "workspace %zu bytes, need %zu", have, need);
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(RK_EINVAL, "workspace not 256-byte aligned");
  return RK_OK;
}

rk_status decode_common(const rk_shape* shape, const void* q, const void* k, const void* v,
                        int64_t kv_cap, const int32_t* cand, int64_t cand_stride,
                        const void* kmax, const void* kmin, int64_t nblk_cap, int64_t n_tokens,
                        int32_t block, int32_t k1, int32_t k2, float* out, int32_t* sel_opt,
                        int32_t* chan_opt, float* s1_opt, void* ws, size_t ws_bytes,
                        rk_stream stream, bool mt, const rk::AppendArgs* app = nullptr,
                        bool exact_rows = false, const rk::PagedArgs* paged = nullptr,
                        const int32_t* lens = nullptr) {
  rk::Dims d;
  rk_status st = check_shape(shape, &d);
  if (st != RK_OK) return st;
  if (!q || !k || !v || !out || (!exact_rows && (!kmax || !kmin)))
    return fail(RK_EINVAL, "null tensor argument");
  if (mt && !cand) return fail(RK_EINVAL, "cand_idx is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (!exact_rows && (!aligned16(kmax) || !aligned16(kmin))))
    return fail(RK_EINVAL, "q, k, v, kmax, kmin and out must be 16-byte aligned");
  if (d.G != 1 && d.G != 2 && d.G != 4 && d.G != 8)
    return fail(RK_EUNSUPPORTED, "group size %d not built (1, 2, 4, 8)", d.G);
  if (block < 1) return fail(RK_EINVAL, "block must be >= 1");
  if (n_tokens < 1) return fail(RK_EINVAL, "n_tokens must be >= 1");
  if (n_tokens > (int64_t(1) << 31) - 1) return fail(RK_EINVAL, "n_tokens too large");
  if (paged) {
    if (n_tokens > (paged->table_stride << paged->shift))
      return fail(RK_EINVAL, "n_tokens exceeds the pages of the block table row");
  } else if (mt) {
    if (n_tokens > cand_stride) return fail(RK_EINVAL, "n_cand exceeds cand_stride");
    if (kv_cap < 1) return fail(RK_EINVAL, "kv_cap must be >= 1");
  } else if (n_tokens > kv_cap) {
    return fail(RK_EINVAL, "n_tokens (%lld) exceeds kv_cap (%lld)", (long long)n_tokens,
                (long long)kv_cap);
  }
  const int64_t nblk = (n_tokens + block - 1) / block;
  if (!exact_rows) {
    if (nblk > nblk_cap) return fail(RK_EINVAL, "pages (%lld) exceed nblk_cap", (long long)nblk);
    if (nblk_cap % 8) return fail(RK_EINVAL, "nblk_cap must be a multiple of 8");
  }
  if (nblk > rk::kMaxPagesGlobal)
    return fail(RK_EUNSUPPORTED, "pages (%lld) above %lld", (long long)nblk,
                (long long)rk::kMaxPagesGlobal);
  if (k1 < 1 || k1 > d.D) return fail(RK_EINVAL, "k1 (%d) outside [1, head_dim]", k1);
  if (k2 < 1) return fail(RK_EINVAL, "k2 must be >= 1");
  if (lens) {
    if (reinterpret_cast<uintptr_t>(lens) & 3u) return fail(RK_EINVAL, "unit_tokens misaligned");
    if (nblk > rk::kMaxPages)
      return fail(RK_EUNSUPPORTED, "ragged units with more than %lld pages", (long long)rk::kMaxPages);
  }
  const rk::DecodeWs lay = rk::decode_ws_layout(d, nblk, k2);
  if ((st = check_ws(ws, ws_bytes, lay.total)) != RK_OK) return st;
  return device_status(
      rk::launch_hsa_decode(d, q, k, v, kv_cap, mt ? cand : nullptr, cand_stride, kmax, kmin,
                            nblk_cap, n_tokens, block, k1, k2, out, sel_opt, chan_opt, s1_opt,
                            ws, static_cast<hipStream_t>(stream), app, exact_rows, paged, lens),
      mt ? "rk_hsa_decode_mt launch" : app ? "rk_hsa_append_decode launch" : "rk_hsa_decode launch");
}

// Checks a paged-pool descriptor against the shape and converts it.
rk_status check_paged(const rk_paged_kv* pk, const rk::Dims& d, rk::PagedArgs* out) {
  if (!pk) return fail(RK_EINVAL, "paged descriptor is NULL");
  if (!d.bf16) return fail(RK_EUNSUPPORTED, "paged pools are built for bf16");
  if (!pk->block_table || (reinterpret_cast<uintptr_t>(pk->block_table) & 3u))
    return fail(RK_EINVAL, "block_table is NULL or misaligned");
  const int32_t P = pk->page_tokens;
  if (P < 1 || P > (1 << 15) || (P & (P - 1)))
    return fail(RK_EINVAL, "page_tokens must be a power of two in [1, 32768]");
  if (pk->n_pages < 1 || pk->table_stride < 1) return fail(RK_EINVAL, "n_pages and table_stride must be >= 1");
  if (pk->n_pages * int64_t(d.Hkv) * P > (int64_t(1) << 31) - 1)
    return fail(RK_EUNSUPPORTED, "the pool holds 2^31 or more rows");
  int shift = 0;
  while ((1 << shift) < P) ++shift;
  *out = rk::PagedArgs{pk->block_table, pk->table_stride, pk->n_pages, shift, d.Hkv};
  return RK_OK;
}

// ---- static scratch of rk_hsa_decode_noalloc -----------------------------
// Device memory that the library owns for callers that cannot allocate: the
// split-K decode's workspace (page keys and partials) lives here instead of a
// caller workspace.  Each GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is ever handed to kernels.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, per device

// The current device's address of `scratch` (looked up on the first call on
// that device, with it current).
rk_status scratch_address(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return device_status(err, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(RK_EUNSUPPORTED, "device %d beyond the %d the static scratch tracks", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return device_status(err, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(RK_EDEVICE, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RK_OK;
}

}  // namespace

extern "C" {

const char* rk_status_string(rk_status s) {
  switch (s) {
    case RK_OK: return "RK_OK";
    case RK_EINVAL: return "RK_EINVAL";
    case RK_EUNSUPPORTED: return "RK_EUNSUPPORTED";
    case RK_EWORKSPACE: return "RK_EWORKSPACE";
    case RK_EDEVICE: return "RK_EDEVICE";
  }
  return "RK_UNKNOWN";
}

const char* rk_last_error(void) { return g_last_error.c_str(); }

rk_status rk_split(double c, int64_t seq_len, int32_t window, int32_t block, int32_t head_dim,
                   rk_split_out* out) {
  if (!out) return fail(RK_EINVAL, "out is NULL");
  if (!(c >= 1.0) || !isfinite(c)) return fail(RK_EINVAL, "compression ratio must be >= 1");
  if (window < 1 || window > seq_len) return fail(RK_EINVAL, "window outside [1, seq_len]");
  if (block < 1 || head_dim < 1) return fail(RK_EINVAL, "block and head_dim must be >= 1");
  double r = 0.2 + 0.06 * log2(c);
  r = r < 0.2 ? 0.2 : (r > 0.8 ? 0.8 : r);
  const double c1 = pow(c, r);
  const double c2 = pow(c, 1.0 - r);
  const double t = double(seq_len) / c;
  int64_t keep = int64_t(ceil(double(seq_len) / c1));
  keep = keep < window ? window : keep;
  keep = keep > seq_len ? seq_len : keep;
  int64_t k2 = int64_t(ceil(t / double(block)));
  k2 = k2 < 1 ? 1 : k2;
  const int32_t page = int32_t(ceil(pow(c, (1.0 - r) / 2.0)));
  out->r = r;
  out->c1 = c1;
  out->c2 = c2;
  out->budget_t = t;
  out->n_keep = keep;
  out->k2_blocks = int32_t(k2 > INT32_MAX ? INT32_MAX : k2);
  out->paper_page = page;
  out->paper_k1 = double(head_dim) / (c2 / double(page));
  int64_t k1p = int64_t(floor(out->paper_k1 + 0.5));
  k1p = k1p < 1 ? 1 : (k1p > head_dim ? head_dim : k1p);
  out->paper_k1_channels = int32_t(k1p);
  int64_t k2p = int64_t(ceil(t / 2.0 / double(page)));
  k2p = k2p < 1 ? 1 : k2p;
  out->paper_k2_blocks = int32_t(k2p > INT32_MAX ? INT32_MAX : k2p);
  return RK_OK;
}

size_t rk_snapkv_workspace_bytes(const rk_shape* shape, int64_t seq_len, int32_t window) {
  rk::Dims d;
  if (check_shape(shape, &d) != RK_OK || window < 1 || window > seq_len) return 0;
  return rk::evict_ws_layout(d, seq_len, window).total;
}

rk_status rk_snapkv_evict(const rk_shape* shape, const void* q_win, const void* k,
                          const void* v, int64_t kv_cap, int64_t seq_len, int32_t window,
                          int32_t pool_kernel, int64_t n_keep, int32_t* kept_idx, void* k_out,
                          void* v_out, int64_t out_cap, float* pooled_opt, void* kmax_opt,
                          void* kmin_opt, int64_t nblk_cap, int32_t block, void* ws,
                          size_t ws_bytes, rk_stream stream) {
  return rk_snapkv_evict_pool(shape, q_win, k, v, kv_cap, seq_len, window, pool_kernel, RK_POOL_SUM,
                              n_keep, kept_idx, k_out, v_out, out_cap, pooled_opt, kmax_opt,
                              kmin_opt, nblk_cap, block, ws, ws_bytes, stream);
}

rk_status rk_snapkv_evict_pool(const rk_shape* shape, const void* q_win, const void* k,
                               const void* v, int64_t kv_cap, int64_t seq_len, int32_t window,
                               int32_t pool_kernel, int32_t pool_op, int64_t n_keep,
                               int32_t* kept_idx, void* k_out, void* v_out, int64_t out_cap,
                               float* pooled_opt, void* kmax_opt, void* kmin_opt, int64_t nblk_cap,
                               int32_t block, void* ws, size_t ws_bytes, rk_stream stream) {
  rk::Dims d;
  rk_status st = check_shape(shape, &d);
  if (st != RK_OK) return st;
  if (!q_win || !k || !kept_idx) return fail(RK_EINVAL, "null tensor argument");
  if ((k_out == nullptr) != (v_out == nullptr))
    return fail(RK_EINVAL, "k_out and v_out must both be given or both be NULL");
  if (k_out && !v) return fail(RK_EINVAL, "v is NULL but a compact cache is requested");
  if (!aligned16(q_win) || !aligned16(k) || (v && !aligned16(v)) ||
      (k_out && (!aligned16(k_out) || !aligned16(v_out))))
    return fail(RK_EINVAL, "tensors must be 16-byte aligned");
  if (window < 1 || window > seq_len) return fail(RK_EINVAL, "window outside [1, seq_len]");
  if (seq_len > kv_cap) return fail(RK_EINVAL, "seq_len exceeds kv_cap");
  if (seq_len > (int64_t(1) << 31) - 1) return fail(RK_EINVAL, "seq_len too large");
  if (n_keep < window || n_keep > seq_len) return fail(RK_EINVAL, "n_keep outside [W, S]");
  if (pool_kernel < 1 || (pool_kernel % 2) == 0 || pool_kernel > 4097)
    return fail(RK_EINVAL, "pool_kernel must be odd, in [1, 4097]");
  if (pool_op != RK_POOL_SUM && pool_op != RK_POOL_MAX)
    return fail(RK_EINVAL, "pool_op must be RK_POOL_SUM or RK_POOL_MAX");
  if (k_out && out_cap < n_keep) return fail(RK_EINVAL, "out_cap below n_keep");
  if ((kmax_opt == nullptr) != (kmin_opt == nullptr))
    return fail(RK_EINVAL, "kmax_opt and kmin_opt must both be given or both be NULL");
  if (kmax_opt) {
    if (!k_out) return fail(RK_EINVAL, "the aux outputs need the compact cache (k_out)");
    if (!aligned16(kmax_opt) || !aligned16(kmin_opt))
      return fail(RK_EINVAL, "kmax and kmin must be 16-byte aligned");
    if (block < 1) return fail(RK_EINVAL, "block must be >= 1");
    if ((n_keep + block - 1) / block > nblk_cap)
      return fail(RK_EINVAL, "nblk_cap below the page count of n_keep tokens");
    if (nblk_cap % 8 != 0) return fail(RK_EINVAL, "nblk_cap must be a multiple of 8");
  }
  if (int64_t(d.G) * window > 1024)
    return fail(RK_EUNSUPPORTED, "group * window above 1024 rows");
  const rk::EvictWs lay = rk::evict_ws_layout(d, seq_len, window);
  if ((st = check_ws(ws, ws_bytes, lay.total)) != RK_OK) return st;
  return device_status(
      rk::launch_snapkv_evict(d, q_win, k, v, kv_cap, seq_len, window, pool_kernel, pool_op,
                              n_keep, kept_idx, k_out, v_out, out_cap, pooled_opt, kmax_opt,
                              kmin_opt, nblk_cap, block, ws, static_cast<hipStream_t>(stream)),
      "rk_snapkv_evict launch");
}

rk_status rk_hsa_build_aux(const rk_shape* shape, const void* k, int64_t k_cap,
                           const int32_t* idx_opt, int64_t idx_stride, int64_t n_tokens,
                           int64_t first_token, int32_t block, void* kmax, void* kmin,
                           int64_t nblk_cap, rk_stream stream) {
  rk::Dims d;
  rk_status st = check_shape(shape, &d);
  if (st != RK_OK) return st;
  if (!k || !kmax) return fail(RK_EINVAL, "null tensor argument");
  if (!aligned16(k) || !aligned16(kmax) || (kmin && !aligned16(kmin)))
    return fail(RK_EINVAL, "k, kmax and kmin must be 16-byte aligned");
  if (block < 1) return fail(RK_EINVAL, "block must be >= 1");
  if (n_tokens < 1 || n_tokens > (int64_t(1) << 31) - 1)
    return fail(RK_EINVAL, "n_tokens outside [1, 2^31)");
  if (first_token < 0 || first_token >= n_tokens)
    return fail(RK_EINVAL, "first_token outside [0, n_tokens)");
  if (idx_opt ? n_tokens > idx_stride : n_tokens > k_cap)
    return fail(RK_EINVAL, "n_tokens exceeds %s", idx_opt ? "idx_stride" : "k_cap");
  const int64_t nblk = (n_tokens + block - 1) / block;
  if (nblk > nblk_cap) return fail(RK_EINVAL, "pages (%lld) exceed nblk_cap", (long long)nblk);
  if (nblk_cap % 8) return fail(RK_EINVAL, "nblk_cap must be a multiple of 8");
  return device_status(rk::launch_build_aux(d, k, k_cap, idx_opt, idx_stride, n_tokens,
                                            first_token / block, block, kmax, kmin, nblk_cap,
                                            static_cast<hipStream_t>(stream)),
                       "rk_hsa_build_aux launch");
}

rk_status rk_append_kv(const rk_shape* shape, const void* k_new, const void* v_new, void* k,
                       void* v, int64_t kv_cap, int64_t pos, void* kmax, void* kmin,
                       int64_t nblk_cap, int32_t block, rk_stream stream) {
  rk::Dims d;
  rk_status st = check_shape(shape, &d);
  if (st != RK_OK) return st;
  if (!k_new || !v_new || !k || !v || !kmax || !kmin) return fail(RK_EINVAL, "null tensor argument");
  if (block < 1) return fail(RK_EINVAL, "block must be >= 1");
  if (pos < 0 || pos >= kv_cap) return fail(RK_EINVAL, "pos outside [0, kv_cap)");
  if (pos / block >= nblk_cap) return fail(RK_EINVAL, "page of pos beyond nblk_cap");
  if (nblk_cap % 8) return fail(RK_EINVAL, "nblk_cap must be a multiple of 8");
  return device_status(rk::launch_append_kv(d, k_new, v_new, k, v, kv_cap, pos, kmax, kmin,
                                            nblk_cap, block, static_cast<hipStream_t>(stream)),
                       "rk_append_kv launch");
}

size_t rk_hsa_workspace_bytes(const rk_shape* shape, int64_t n_tokens, int32_t block, int32_t k1,
                              int32_t k2) {
  rk::Dims d;
  if (check_shape(shape, &d) != RK_OK || n_tokens < 1 || block < 1 || k1 < 1 || k2 < 1) return 0;
  return rk::decode_ws_layout(d, (n_tokens + block - 1) / block, k2).total;
}

rk_status rk_hsa_decode(const rk_shape* shape, const void* q, const void* k, const void* v,
                        int64_t kv_cap, const void* kmax, const void* kmin, int64_t nblk_cap,
                        int64_t n_tokens, int32_t block, int32_t k1, int32_t k2, float* out,
                        int32_t* sel_blocks_opt, int32_t* sel_channels_opt,
                        float* block_scores_opt, void* ws, size_t ws_bytes, rk_stream stream) {
  return decode_common(shape, q, k, v, kv_cap, nullptr, 0, kmax, kmin, nblk_cap, n_tokens, block,
                       k1, k2, out, sel_blocks_opt, sel_channels_opt, block_scores_opt, ws,
                       ws_bytes, stream, false);
}

rk_status rk_hsa_append_decode(const rk_shape* shape, const void* q, const void* k_new,
                               const void* v_new, void* k, void* v, int64_t kv_cap, int64_t pos,
                               void* kmax, void* kmin, int64_t nblk_cap, int32_t block, int32_t k1,
                               int32_t k2, float* out, int32_t* sel_blocks_opt,
                               int32_t* sel_channels_opt, float* block_scores_opt, void* ws,
                               size_t ws_bytes, rk_stream stream) {
  if (!k_new || !v_new) return fail(RK_EINVAL, "null tensor argument");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(RK_EINVAL, "k_new and v_new must be 16-byte aligned");
  if (pos < 0 || pos >= kv_cap) return fail(RK_EINVAL, "pos outside [0, kv_cap)");
  const rk::AppendArgs app{k_new, v_new, k, v, kmax, kmin};
  return decode_common(shape, q, k, v, kv_cap, nullptr, 0, kmax, kmin, nblk_cap, pos + 1, block,
                       k1, k2, out, sel_blocks_opt, sel_channels_opt, block_scores_opt, ws,
                       ws_bytes, stream, false, &app);
}

rk_status rk_hsa_decode_noalloc(const rk_shape* shape, const void* q, const void* k,
                                const void* v, int64_t kv_cap, const void* kmax, const void* kmin,
                                int64_t nblk_cap, int64_t n_tokens, int32_t block, int32_t k1,
                                int32_t k2, float* out, int32_t* sel_blocks_opt,
                                int32_t* sel_channels_opt, float* block_scores_opt,
                                rk_stream stream) {
  // the size check comes first: a call the scratch cannot hold touches no device
  rk::Dims d;
  rk_status st = check_shape(shape, &d);
  if (st != RK_OK) return st;
  if (block < 1 || k2 < 1 || n_tokens < 1) return fail(RK_EINVAL, "block, k2 and n_tokens must be >= 1");
  const size_t need = rk::decode_ws_layout(d, (n_tokens + block - 1) / block, k2).total;
  if (need > kScratchBytes)
    return fail(RK_EWORKSPACE,
                "rk_hsa_decode_noalloc: the call needs %zu bytes of scratch, the static scratch "
                "holds %zu; use rk_hsa_decode with a workspace",
                need, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != RK_OK) return st;
  return decode_common(shape, q, k, v, kv_cap, nullptr, 0, kmax, kmin, nblk_cap, n_tokens, block,
                       k1, k2, out, sel_blocks_opt, sel_channels_opt, block_scores_opt, ws,
                       kScratchBytes, stream, false);
}

size_t rk_hsa_decode_noalloc_max_bytes(void) { return kScratchBytes; }

rk_status rk_select_plan(rk_select_method method, double c, int64_t seq_len, int32_t head_dim,
                         rk_select_plan_out* out) {
  if (!out) return fail(RK_EINVAL, "out is NULL");
  if (!(c >= 1.0) || !isfinite(c)) return fail(RK_EINVAL, "compression ratio must be >= 1");
  if (seq_len < 1 || head_dim < 1) return fail(RK_EINVAL, "seq_len and head_dim must be >= 1");
  const double t = double(seq_len) / c;
  const int32_t d = head_dim;
  auto clamp_d = [d](double x) {
    int64_t v = int64_t(floor(x + 0.5));
    return int32_t(v < 1 ? 1 : (v > d ? d : v));
  };
  auto pages_for = [](double tokens, int64_t page) {
    const int64_t k = int64_t(ceil(tokens / double(page)));
    return int32_t(k < 1 ? 1 : (k > INT32_MAX ? INT32_MAX : k));
  };
  int64_t page = 1;
  int32_t channels = d, k2 = 1;
  switch (method) {
    case RK_SEL_HSA:
      page = int64_t(ceil(sqrt(c)));
      channels = clamp_d(double(d) * double(page) / c);
      k2 = pages_for(t / 2.0, page);
      break;
    case RK_SEL_QUEST:
      page = int64_t(ceil(c));
      channels = d;
      k2 = pages_for(t / 2.0, page);
      break;
    case RK_SEL_SPARQ:
      page = 1;
      channels = clamp_d(double(d) / c);
      k2 = pages_for(t / 2.0, 1);
      break;
    case RK_SEL_EXACT:
      page = 1;
      channels = d;
      k2 = pages_for(t, 1);
      break;
    default:
      return fail(RK_EINVAL, "unknown selection method %d", int(method));
  }
  if (page > INT32_MAX) return fail(RK_EINVAL, "page size too large");
  const int64_t n_pages = (seq_len + page - 1) / page;
  out->page = int32_t(page);
  out->channels = channels;
  out->k2 = k2;
  out->attn_tokens = int64_t(k2) * page < seq_len ? int64_t(k2) * page : seq_len;
  out->budget_t = t;
  out->est_pairs = double(channels) * double(n_pages) / (2.0 * double(d));
  return RK_OK;
}

rk_status rk_select_decode(const rk_shape* shape, rk_select_method method, const void* q,
                           const void* k, const void* v, int64_t kv_cap, const void* kmax,
                           const void* kmin, int64_t nblk_cap, int64_t n_tokens, int32_t page,
                           int32_t channels, int32_t k2, float* out, int32_t* sel_opt,
                           float* scores_opt, void* ws, size_t ws_bytes, rk_stream stream) {
  if (!shape) return fail(RK_EINVAL, "shape is NULL");
  switch (method) {
    case RK_SEL_HSA:
      break;
    case RK_SEL_QUEST:
      if (channels != shape->head_dim)
        return fail(RK_EINVAL, "Quest reads every channel: channels must equal head_dim");
      break;
    case RK_SEL_SPARQ:
      if (page != 1) return fail(RK_EINVAL, "SparQ selects tokens: page must be 1");
      kmin = kmax;  // pages of one token: Kmax = Kmin = the key row, channel-major
      break;
    case RK_SEL_EXACT:
      if (page != 1 || channels != shape->head_dim)
        return fail(RK_EINVAL, "Exact-TopK selects tokens over every channel: page 1, channels = head_dim");
      return decode_common(shape, q, k, v, kv_cap, nullptr, 0, nullptr, nullptr, 0, n_tokens, 1,
                           channels, k2, out, sel_opt, nullptr, scores_opt, ws, ws_bytes, stream,
                           false, nullptr, true);
    default:
      return fail(RK_EINVAL, "unknown selection method %d", int(method));
  }
  return decode_common(shape, q, k, v, kv_cap, nullptr, 0, kmax, kmin, nblk_cap, n_tokens, page,
                       channels, k2, out, sel_opt, nullptr, scores_opt, ws, ws_bytes, stream, false);
}

rk_status rk_paged_write_kv(const rk_shape* shape, const void* k_src, const void* v_src,
                           int64_t src_cap, int64_t first_token, int64_t n_tokens, void* k_pool,
                           void* v_pool, const rk_paged_kv* pages, rk_stream stream) {
  rk::Dims d;
  rk_status st = check_shape(shape, &d);
  if (st != RK_OK) return st;
  rk::PagedArgs pg;
  if ((st = check_paged(pages, d, &pg)) != RK_OK) return st;
  if (!k_src || !v_src || !k_pool || !v_pool) return fail(RK_EINVAL, "null tensor argument");
  if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(RK_EINVAL, "tensors must be 16-byte aligned");
  if (first_token < 0 || n_tokens < 1 || first_token + n_tokens > src_cap)
    return fail(RK_EINVAL, "rows [first_token, first_token + n_tokens) outside the source");
  if (first_token + n_tokens > (pg.table_stride << pg.shift) || first_token + n_tokens > (int64_t(1) << 31) - 1)
    return fail(RK_EINVAL, "rows beyond the pages of the block table row");
  return device_status(rk::launch_paged_write(d, k_src, v_src, src_cap, first_token, n_tokens, k_pool,
                                              v_pool, pg, static_cast<hipStream_t>(stream)),
                       "rk_paged_write_kv launch");
}

rk_status rk_paged_build_aux(const rk_shape* shape, const void* k_pool, const rk_paged_kv* pages,
                             int64_t n_tokens, int64_t first_token, int32_t block, void* kmax,
                             void* kmin, int64_t nblk_cap, rk_stream stream) {
  rk::Dims d;
  rk_status st = check_shape(shape, &d);
  if (st != RK_OK) return st;
  rk::PagedArgs pg;
  if ((st = check_paged(pages, d, &pg)) != RK_OK) return st;
  if (!k_pool || !kmax) return fail(RK_EINVAL, "null tensor argument");
  if (!aligned16(k_pool) || !aligned16(kmax) || (kmin && !aligned16(kmin)))
    return fail(RK_EINVAL, "k_pool, kmax and kmin must be 16-byte aligned");
  if (block < 1) return fail(RK_EINVAL, "block must be >= 1");
  if (n_tokens < 1 || n_tokens > (pg.table_stride << pg.shift) || n_tokens > (int64_t(1) << 31) - 1)
    return fail(RK_EINVAL, "n_tokens outside [1, pages of the block table row]");
  if (first_token < 0 || first_token >= n_tokens)
    return fail(RK_EINVAL, "first_token outside [0, n_tokens)");
  const int64_t nblk = (n_tokens + block - 1) / block;
  if (nblk > nblk_cap) return fail(RK_EINVAL, "pages (%lld) exceed nblk_cap", (long long)nblk);
  if (nblk_cap % 8) return fail(RK_EINVAL, "nblk_cap must be a multiple of 8");
  return device_status(rk::launch_build_aux(d, k_pool, 0, nullptr, 0, n_tokens, first_token / block, block,
                                            kmax, kmin, nblk_cap, static_cast<hipStream_t>(stream), &pg),
                       "rk_paged_build_aux launch");
}

rk_status rk_paged_append_kv(const rk_shape* shape, const void* k_new, const void* v_new,
                             void* k_pool, void* v_pool, const rk_paged_kv* pages, int64_t pos,
                             void* kmax, void* kmin, int64_t nblk_cap, int32_t block,
                             rk_stream stream) {
  rk::Dims d;
  rk_status st = check_shape(shape, &d);
  if (st != RK_OK) return st;
  rk::PagedArgs pg;
  if ((st = check_paged(pages, d, &pg)) != RK_OK) return st;
  if (!k_new || !v_new || !k_pool || !v_pool || !kmax || !kmin)
    return fail(RK_EINVAL, "null tensor argument");
  if (block < 1) return fail(RK_EINVAL, "block must be >= 1");
  if (pos < 0 || pos >= (pg.table_stride << pg.shift) || pos > (int64_t(1) << 31) - 2)
    return fail(RK_EINVAL, "pos outside the pages of the block table row");
  if (pos / block >= nblk_cap) return fail(RK_EINVAL, "page of pos beyond nblk_cap");
  if (nblk_cap % 8) return fail(RK_EINVAL, "nblk_cap must be a multiple of 8");
  return device_status(rk::launch_append_kv(d, k_new, v_new, k_pool, v_pool, 0, pos, kmax, kmin, nblk_cap,
                                            block, static_cast<hipStream_t>(stream), &pg),
                       "rk_paged_append_kv launch");
}

rk_status rk_paged_hsa_decode(const rk_shape* shape, const void* q, const void* k_pool,
                              const void* v_pool, const rk_paged_kv* pages, const void* kmax,
                              const void* kmin, int64_t nblk_cap, int64_t n_tokens, int32_t block,
                              int32_t k1, int32_t k2, float* out, int32_t* sel_blocks_opt,
                              int32_t* sel_channels_opt, float* block_scores_opt, void* ws,
                              size_t ws_bytes, rk_stream stream) {
  rk::Dims d;
  rk_status st = check_shape(shape, &d);
  if (st != RK_OK) return st;
  rk::PagedArgs pg;
  if ((st = check_paged(pages, d, &pg)) != RK_OK) return st;
  return decode_common(shape, q, k_pool, v_pool, 0, nullptr, 0, kmax, kmin, nblk_cap, n_tokens, block,
                       k1, k2, out, sel_blocks_opt, sel_channels_opt, block_scores_opt, ws, ws_bytes,
                       stream, false, nullptr, false, &pg);
}

rk_status rk_paged_hsa_append_decode(const rk_shape* shape, const void* q, const void* k_new,
                                     const void* v_new, void* k_pool, void* v_pool,
                                     const rk_paged_kv* pages, int64_t pos, void* kmax, void* kmin,
                                     int64_t nblk_cap, int32_t block, int32_t k1, int32_t k2,
                                     float* out, int32_t* sel_blocks_opt, int32_t* sel_channels_opt,
                                     float* block_scores_opt, void* ws, size_t ws_bytes,
                                     rk_stream stream) {
  rk::Dims d;
  rk_status st = check_shape(shape, &d);
  if (st != RK_OK) return st;
  rk::PagedArgs pg;
  if ((st = check_paged(pages, d, &pg)) != RK_OK) return st;
  if (!k_new || !v_new) return fail(RK_EINVAL, "null tensor argument");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(RK_EINVAL, "k_new and v_new must be 16-byte aligned");
  if (pos < 0 || pos >= (pg.table_stride << pg.shift))
    return fail(RK_EINVAL, "pos outside the pages of the block table row");
  const rk::AppendArgs app{k_new, v_new, k_pool, v_pool, kmax, kmin};
  return decode_common(shape, q, k_pool, v_pool, 0, nullptr, 0, kmax, kmin, nblk_cap, pos + 1, block,
                       k1, k2, out, sel_blocks_opt, sel_channels_opt, block_scores_opt, ws, ws_bytes,
                       stream, false, &app, false, &pg);
}

rk_status rk_adakv_evict(const rk_shape* shape, const void* q_win, const void* k, const void* v,
                         int64_t kv_cap, int64_t seq_len, int32_t window, int32_t pool_kernel,
                         int64_t n_keep, int32_t* kept_idx, int32_t* kept_count, void* k_out,
                         void* v_out, int64_t out_cap, float* pooled_opt, void* kmax_opt,
                         void* kmin_opt, int64_t nblk_cap, int32_t block, void* ws, size_t ws_bytes,
                         rk_stream stream) {
  return rk_adakv_evict_pool(shape, q_win, k, v, kv_cap, seq_len, window, pool_kernel, RK_POOL_SUM,
                             n_keep, kept_idx, kept_count, k_out, v_out, out_cap, pooled_opt,
                             kmax_opt, kmin_opt, nblk_cap, block, ws, ws_bytes, stream);
}

rk_status rk_adakv_evict_pool(const rk_shape* shape, const void* q_win, const void* k, const void* v,
                              int64_t kv_cap, int64_t seq_len, int32_t window, int32_t pool_kernel,
                              int32_t pool_op, int64_t n_keep, int32_t* kept_idx,
                              int32_t* kept_count, void* k_out, void* v_out, int64_t out_cap,
                              float* pooled_opt, void* kmax_opt, void* kmin_opt, int64_t nblk_cap,
                              int32_t block, void* ws, size_t ws_bytes, rk_stream stream) {
  rk::Dims d;
  rk_status st = check_shape(shape, &d);
  if (st != RK_OK) return st;
  if (!q_win || !k || !kept_idx || !kept_count) return fail(RK_EINVAL, "null tensor argument");
  if ((k_out == nullptr) != (v_out == nullptr))
    return fail(RK_EINVAL, "k_out and v_out must both be given or both be NULL");
  if (k_out && !v) return fail(RK_EINVAL, "v is NULL but a compact cache is requested");
  if (!aligned16(q_win) || !aligned16(k) || (v && !aligned16(v)) ||
      (k_out && (!aligned16(k_out) || !aligned16(v_out))) ||
      (reinterpret_cast<uintptr_t>(kept_idx) & 3u) || (reinterpret_cast<uintptr_t>(kept_count) & 3u))
    return fail(RK_EINVAL, "tensors misaligned");
  if (d.Hkv > 64) return fail(RK_EUNSUPPORTED, "shared budgets over more than 64 KV heads");
  if (window < 1 || window > seq_len) return fail(RK_EINVAL, "window outside [1, seq_len]");
  if (seq_len > kv_cap) return fail(RK_EINVAL, "seq_len exceeds kv_cap");
  if (seq_len > (int64_t(1) << 31) - 1) return fail(RK_EINVAL, "seq_len too large");
  if (n_keep < window || n_keep > seq_len) return fail(RK_EINVAL, "n_keep outside [W, S]");
  if (int64_t(d.Hkv) * (seq_len - window) > (int64_t(1) << 31) - 1)
    return fail(RK_EUNSUPPORTED, "Hkv * (seq_len - window) too large");
  if (pool_kernel < 1 || (pool_kernel % 2) == 0 || pool_kernel > 4097)
    return fail(RK_EINVAL, "pool_kernel must be odd, in [1, 4097]");
  if (pool_op != RK_POOL_SUM && pool_op != RK_POOL_MAX)
    return fail(RK_EINVAL, "pool_op must be RK_POOL_SUM or RK_POOL_MAX");
  const int64_t worst = std::min<int64_t>(seq_len, int64_t(d.Hkv) * (n_keep - window) + window);
  if (out_cap < worst)
    return fail(RK_EINVAL, "out_cap (%lld) below min(seq_len, Hkv * (n_keep - W) + W) = %lld",
                (long long)out_cap, (long long)worst);
  if ((kmax_opt == nullptr) != (kmin_opt == nullptr))
    return fail(RK_EINVAL, "kmax_opt and kmin_opt must both be given or both be NULL");
  if (kmax_opt) {
    if (!k_out) return fail(RK_EINVAL, "the aux outputs need the compact cache (k_out)");
    if (!aligned16(kmax_opt) || !aligned16(kmin_opt))
      return fail(RK_EINVAL, "kmax and kmin must be 16-byte aligned");
    if (block < 1) return fail(RK_EINVAL, "block must be >= 1");
    if ((worst + block - 1) / block > nblk_cap)
      return fail(RK_EINVAL, "nblk_cap below the page count of out_cap's worst case");
    if (nblk_cap % 8 != 0) return fail(RK_EINVAL, "nblk_cap must be a multiple of 8");
  }
  if (int64_t(d.G) * window > 1024) return fail(RK_EUNSUPPORTED, "group * window above 1024 rows");
  const rk::EvictWs lay = rk::evict_ws_layout(d, seq_len, window);
  if ((st = check_ws(ws, ws_bytes, lay.total)) != RK_OK) return st;
  return device_status(
      rk::launch_snapkv_evict(d, q_win, k, v, kv_cap, seq_len, window, pool_kernel, pool_op,
                              n_keep, kept_idx, k_out, v_out, out_cap, pooled_opt, kmax_opt,
                              kmin_opt, nblk_cap, block, ws, static_cast<hipStream_t>(stream),
                              kept_count),
      "rk_adakv_evict launch");
}

rk_status rk_hsa_decode_ragged(const rk_shape* shape, const void* q, const void* k, const void* v,
                               int64_t kv_cap, const void* kmax, const void* kmin, int64_t nblk_cap,
                               const int32_t* unit_tokens, int64_t max_tokens, int32_t block,
                               int32_t k1, int32_t k2, float* out, int32_t* sel_blocks_opt,
                               int32_t* sel_channels_opt, float* block_scores_opt, void* ws,
                               size_t ws_bytes, rk_stream stream) {
  if (!unit_tokens) return fail(RK_EINVAL, "unit_tokens is NULL");
  return decode_common(shape, q, k, v, kv_cap, nullptr, 0, kmax, kmin, nblk_cap, max_tokens, block, k1,
                       k2, out, sel_blocks_opt, sel_channels_opt, block_scores_opt, ws, ws_bytes, stream,
                       false, nullptr, false, nullptr, unit_tokens);
}

rk_status rk_hsa_decode_mt(const rk_shape* shape, const void* q, const void* k, const void* v,
                           int64_t kv_cap, const int32_t* cand_idx, int64_t cand_stride,
                           int64_t n_cand, const void* kmax, const void* kmin, int64_t nblk_cap,
                           int32_t block, int32_t k1, int32_t k2, float* out,
                           int32_t* sel_blocks_opt, int32_t* sel_channels_opt,
                           float* block_scores_opt, void* ws, size_t ws_bytes,
                           rk_stream stream) {
  return decode_common(shape, q, k, v, kv_cap, cand_idx, cand_stride, kmax, kmin, nblk_cap,
                       n_cand, block, k1, k2, out, sel_blocks_opt, sel_channels_opt,
                       block_scores_opt, ws, ws_bytes, stream, true);
}

}  // extern "C"

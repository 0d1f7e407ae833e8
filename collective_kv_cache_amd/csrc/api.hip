// C ABI entry points: argument checks, dispatch to the HIP launchers,
// error reporting.  No C++ exception crosses this boundary.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "common.h"

// Scratch of tdx_select_important_noalloc: one copy per GPU, resident until
// the process ends.  In host code this name is only a stand-in for the
// device symbol; its device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[TDX_SELECT_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return TDX_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TDX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

#define REQ(cond, code, ...)                 \
  do {                                       \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define REQ_PTR(p) REQ((p) != nullptr && aligned16(p), TDX_EINVAL, "%s is null or not 16-byte aligned", #p)
#define REQ_PTR4(p) \
  REQ((p) != nullptr && (reinterpret_cast<uintptr_t>(p) & 3u) == 0, TDX_EINVAL, "%s is null or not 4-byte aligned", #p)

// Shape checks common to all calls.
int check_shape(const tdx_shape* s, tdx::Dims* d) {
  REQ(s != nullptr, TDX_EINVAL, "shape is null");
  REQ(s->dtype == TDX_F32 || s->dtype == TDX_BF16, TDX_EINVAL, "dtype %d is not TDX_F32/TDX_BF16", s->dtype);
  REQ(s->n_layers >= 1, TDX_EINVAL, "n_layers %d < 1", s->n_layers);
  REQ(s->n_kv_heads >= 1 && s->n_q_heads >= 1, TDX_EINVAL, "head counts must be >= 1");
  REQ(s->n_q_heads % s->n_kv_heads == 0, TDX_EINVAL, "n_q_heads %d is not a multiple of n_kv_heads %d",
      s->n_q_heads, s->n_kv_heads);
  REQ(s->head_dim == 64 || s->head_dim == 128, TDX_EUNSUPPORTED, "head_dim %d not in {64, 128}", s->head_dim);
  REQ(s->rope_theta > 1.0, TDX_EINVAL, "rope_theta must be > 1");
  REQ(s->n_kv_heads <= 16, TDX_EUNSUPPORTED, "n_kv_heads %d > 16", s->n_kv_heads);
  d->L = s->n_layers;
  d->Hkv = s->n_kv_heads;
  d->Hq = s->n_q_heads;
  d->D = s->head_dim;
  d->dtype = s->dtype;
  d->theta = s->rope_theta;
  return TDX_OK;
}

// The restore calls count every (agent, layer) row's tiles (its history up
// to max_priv, then the shared tokens) in 32-bit integers.
bool restore_tiles_fit(const tdx::Dims& d, int32_t max_priv) {
  const long long per_row = ((long long)max_priv + TDX_DIFF_BLOCK - 1) / TDX_DIFF_BLOCK + d.T / TDX_DIFF_BLOCK;
  return max_priv >= 0 && (long long)d.N * d.L * per_row <= 0x7fffffffLL;
}
int check_restore_tiles(const tdx::Dims& d, int32_t max_priv) {
  REQ(restore_tiles_fit(d, max_priv), TDX_EUNSUPPORTED,
      "n_agents * n_layers * (max_priv + n_tokens) / 16 exceeds 2^31 - 1 tiles");
  return TDX_OK;
}

int check_layout(const tdx_layout* lay, tdx::Dims* d, bool need_pos) {
  REQ(lay != nullptr, TDX_EINVAL, "layout is null");
  REQ(lay->n_agents >= 1, TDX_EINVAL, "n_agents %d < 1", lay->n_agents);
  REQ(lay->n_blocks >= 1, TDX_EINVAL, "n_blocks %d < 1", lay->n_blocks);
  REQ(lay->n_tokens >= 1, TDX_EINVAL, "n_tokens %d < 1", lay->n_tokens);
  REQ(lay->n_agents <= 1024, TDX_EUNSUPPORTED, "n_agents %d > 1024", lay->n_agents);
  REQ(lay->n_blocks <= 4096, TDX_EUNSUPPORTED, "n_blocks %d > 4096", lay->n_blocks);
  if (need_pos) {
    REQ_PTR4(lay->blk_start);
    REQ_PTR4(lay->src_pos);
    REQ_PTR4(lay->dst_pos);
  }
  d->N = lay->n_agents;
  d->B = lay->n_blocks;
  d->T = lay->n_tokens;
  return TDX_OK;
}

// A paged view: pools 16-byte aligned (v_pool only where needed), page table
// 4-byte aligned, n_pages >= 1, row stride >= the pages a row needs when
// there is more than one row.
int check_paged(const tdx_paged_kv* p, const char* what, bool need_v, int64_t rows, int64_t per_row,
                tdx::PageMap* m) {
  REQ(p != nullptr, TDX_EINVAL, "%s is null", what);
  REQ(p->k_pool != nullptr && aligned16(p->k_pool), TDX_EINVAL, "%s.k_pool is null or not 16-byte aligned", what);
  if (need_v)
    REQ(p->v_pool != nullptr && aligned16(p->v_pool), TDX_EINVAL, "%s.v_pool is null or not 16-byte aligned",
        what);
  REQ(p->n_pages >= 1, TDX_EINVAL, "%s.n_pages < 1", what);
  REQ(p->pages != nullptr && aligned4(p->pages), TDX_EINVAL, "%s.pages is null or not 4-byte aligned", what);
  REQ(rows <= 1 || p->stride >= per_row, TDX_EINVAL, "%s.stride %lld < %lld pages per row", what,
      (long long)p->stride, (long long)per_row);
  *m = tdx::PageMap{p->pages, (long long)p->stride, (long long)p->n_pages};
  return TDX_OK;
}

#define GUARD_BEGIN try {
#define GUARD_END                                                   \
  }                                                                 \
  catch (...) {                                                     \
    return fail(TDX_EINTERNAL, "unexpected exception in %s", __func__); \
  }

}  // namespace

namespace tdx {
// error reporting for the host-only entry points compiled in other files
int report(int code, const char* msg) {
  if (code == TDX_OK) return ok();
  return fail(code, "%s", msg);
}
}  // namespace tdx

extern "C" {

int tdx_version(void) { return TDX_VERSION; }

const char* tdx_strerror(int code) {
  switch (code) {
    case TDX_OK: return "success";
    case TDX_EINVAL: return "invalid argument";
    case TDX_EUNSUPPORTED: return "unsupported shape";
    case TDX_EHIP: return "HIP runtime error";
    case TDX_EINTERNAL: return "internal error";
    case TDX_EWORKSPACE: return "workspace missing or too small";
    default: return "unknown error code";
  }
}

const char* tdx_last_error(void) { return g_last_error.c_str(); }

int32_t tdx_topk_count(int32_t pct, int32_t n_tokens) {
  if (n_tokens < 1 || pct < 0 || pct > 100) return 0;
  int64_t k = ((int64_t)pct * n_tokens + 99) / 100;
  if (k < 1) k = 1;
  if (k > n_tokens) k = n_tokens;
  return (int32_t)k;
}

int tdx_rerotate(const tdx_shape* shape, const tdx_layout* layout, const void* k_cached,
                 void* k_out, void* stream) {
  GUARD_BEGIN
  tdx::Dims d{};
  int rc;
  if ((rc = check_shape(shape, &d)) != TDX_OK) return rc;
  if ((rc = check_layout(layout, &d, true)) != TDX_OK) return rc;
  REQ_PTR(k_cached);
  REQ_PTR(k_out);
  hipError_t e = tdx::launch_rerotate(d, *layout, k_cached, k_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tdx_rerotate launch");
  return ok();
  GUARD_END
}

size_t tdx_select_workspace(const tdx_shape* shape, const tdx_layout* layout) {
  tdx::Dims d{};
  if (check_shape(shape, &d) != TDX_OK || check_layout(layout, &d, false) != TDX_OK) return 0;
  return tdx::select_ws_bytes(d);
}

}  // extern "C"

namespace {
// Argument checks shared by tdx_select_important and its no-allocation variant.
int check_select(const tdx_shape* shape, const tdx_layout* layout, int32_t check_layer, const void* k_reuse,
                 const void* k_recomp, int32_t k, const float* dev, const float* score, const float* agent_dev,
                 const int32_t* selected, const int32_t* master, tdx::Dims* dd) {
  tdx::Dims& d = *dd;
  int rc;
  if ((rc = check_shape(shape, &d)) != TDX_OK) return rc;
  if ((rc = check_layout(layout, &d, false)) != TDX_OK) return rc;
  REQ(check_layer >= 0 && check_layer < d.L, TDX_EINVAL, "check_layer %d outside [0, %d)", check_layer, d.L);
  REQ(k >= 1 && k <= d.T, TDX_EINVAL, "k %d outside [1, %d]", k, d.T);
  REQ_PTR(k_reuse);
  REQ_PTR(k_recomp);
  REQ_PTR4(dev);
  REQ_PTR4(score);
  REQ_PTR4(agent_dev);
  REQ_PTR4(selected);
  REQ_PTR4(master);
  return TDX_OK;
}

// Device address of `scratch` on the calling thread's current device, looked
// up once per device (the symbol's address differs from GPU to GPU).
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

int scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  REQ(dev >= 0 && dev < kMaxScratchDevices, TDX_EUNSUPPORTED, "device %d beyond the %d the scratch table serves", dev,
      kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    REQ(p != nullptr && aligned16(p), TDX_EINTERNAL, "scratch address %p is null or unaligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TDX_OK;
}
}  // namespace

extern "C" {

int tdx_select_important_noalloc(const tdx_shape* shape, const tdx_layout* layout, int32_t check_layer,
                                 const void* k_reuse, const void* k_recomp, int32_t k, float* dev, float* score,
                                 float* agent_dev, int32_t* selected, int32_t* master, void* stream) {
  GUARD_BEGIN
  tdx::Dims d{};
  int rc;
  if ((rc = check_select(shape, layout, check_layer, k_reuse, k_recomp, k, dev, score, agent_dev, selected, master,
                         &d)) != TDX_OK)
    return rc;
  const size_t need = tdx::select_ws_bytes(d);
  REQ(need <= (size_t)TDX_SELECT_SCRATCH_BYTES, TDX_EUNSUPPORTED,
      "the round needs %zu bytes of scratch, more than the static %zu (N * ceil(T/8) * 8 bytes)", need,
      (size_t)TDX_SELECT_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((rc = scratch_on_current_device(&ws)) != TDX_OK) return rc;
  hipError_t e = tdx::launch_select(d, *layout, check_layer, k_reuse, k_recomp, k, dev, score, agent_dev, selected,
                                    master, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tdx_select_important_noalloc launch");
  return ok();
  GUARD_END
}

int tdx_select_important(const tdx_shape* shape, const tdx_layout* layout, int32_t check_layer,
                         const void* k_reuse, const void* k_recomp, int32_t k, float* dev,
                         float* score, float* agent_dev, int32_t* selected, int32_t* master,
                         void* ws, size_t ws_bytes, void* stream) {
  GUARD_BEGIN
  tdx::Dims d{};
  int rc;
  if ((rc = check_select(shape, layout, check_layer, k_reuse, k_recomp, k, dev, score, agent_dev, selected, master,
                         &d)) != TDX_OK)
    return rc;
  const size_t need = tdx::select_ws_bytes(d);
  REQ(ws != nullptr && aligned16(ws) && ws_bytes >= need, TDX_EWORKSPACE,
      "workspace needs %zu bytes (16-byte aligned), got %zu", need, ws_bytes);
  hipError_t e = tdx::launch_select(d, *layout, check_layer, k_reuse, k_recomp, k, dev, score,
                                    agent_dev, selected, master, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tdx_select_important launch");
  return ok();
  GUARD_END
}

size_t tdx_diff_encode_workspace(const tdx_shape* shape, const tdx_layout* layout) {
  tdx::Dims d{};
  if (check_shape(shape, &d) != TDX_OK || check_layout(layout, &d, false) != TDX_OK) return 0;
  return tdx::encode_ws_bytes(d);
}

int tdx_diff_encode(const tdx_shape* shape, const tdx_layout* layout, const int32_t* master,
                    const void* agents_k, const void* agents_v, int64_t cap_blocks,
                    int32_t* diff_off, int32_t* diff_idx, void* diff_k, void* diff_v,
                    int64_t* nnz, void* master_k_out, void* master_v_out, void* ws,
                    size_t ws_bytes, void* stream) {
  GUARD_BEGIN
  tdx::Dims d{};
  int rc;
  if ((rc = check_shape(shape, &d)) != TDX_OK) return rc;
  if ((rc = check_layout(layout, &d, false)) != TDX_OK) return rc;
  REQ(d.T % TDX_DIFF_BLOCK == 0, TDX_EINVAL, "n_tokens %d is not a multiple of 16", d.T);
  REQ(cap_blocks >= 0, TDX_EINVAL, "cap_blocks < 0");
  REQ((int64_t)d.N * d.L <= INT32_MAX, TDX_EUNSUPPORTED, "too many CSR rows");
  REQ_PTR4(master);
  REQ_PTR(agents_k);
  REQ_PTR(agents_v);
  REQ_PTR4(diff_off);
  REQ((reinterpret_cast<uintptr_t>(nnz) & 7u) == 0 && nnz != nullptr, TDX_EINVAL, "nnz is null or not 8-byte aligned");
  if (cap_blocks > 0) {
    REQ_PTR4(diff_idx);
    REQ_PTR(diff_k);
    REQ_PTR(diff_v);
  }
  REQ((master_k_out == nullptr) == (master_v_out == nullptr), TDX_EINVAL,
      "master_k_out and master_v_out must both be set or both be NULL");
  if (master_k_out != nullptr) {
    REQ_PTR(master_k_out);
    REQ_PTR(master_v_out);
  }
  const size_t need = tdx::encode_ws_bytes(d);
  REQ(ws != nullptr && aligned16(ws) && ws_bytes >= need, TDX_EWORKSPACE,
      "workspace needs %zu bytes (16-byte aligned), got %zu", need, ws_bytes);
  hipError_t e = tdx::launch_encode(d, master, agents_k, agents_v, cap_blocks, diff_off, diff_idx,
                                    diff_k, diff_v, nnz, master_k_out, master_v_out, ws,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tdx_diff_encode launch");
  return ok();
  GUARD_END
}

size_t tdx_restore_attn_workspace(const tdx_shape* shape, const tdx_layout* layout, int32_t max_priv) {
  tdx::Dims d{};
  if (check_shape(shape, &d) != TDX_OK || check_layout(layout, &d, false) != TDX_OK || !restore_tiles_fit(d, max_priv))
    return 0;
  return tdx::restore_attn_ws_bytes(d, max_priv);
}

int tdx_restore_attn(const tdx_shape* shape, const tdx_layout* layout, const void* q,
                     const int32_t* priv_off, const void* priv_k, const void* priv_v,
                     int32_t max_priv, const void* master_k, const void* master_v,
                     const int32_t* master_sel, int64_t master_stride,
                     const int32_t* diff_off, const int32_t* diff_idx, const void* diff_k,
                     const void* diff_v, float scale, void* out, void* ws, size_t ws_bytes,
                     void* stream) {
  GUARD_BEGIN
  tdx::Dims d{};
  int rc;
  if ((rc = check_shape(shape, &d)) != TDX_OK) return rc;
  if ((rc = check_layout(layout, &d, true)) != TDX_OK) return rc;
  REQ(d.T % TDX_DIFF_BLOCK == 0, TDX_EINVAL, "n_tokens %d is not a multiple of 16", d.T);
  REQ(d.Hq / d.Hkv <= 16, TDX_EUNSUPPORTED, "more than 16 query heads per KV head");
  REQ(max_priv >= 0, TDX_EINVAL, "max_priv < 0");
  if ((rc = check_restore_tiles(d, max_priv)) != TDX_OK) return rc;
  REQ(scale > 0.0f, TDX_EINVAL, "scale must be > 0");
  REQ_PTR(q);
  REQ_PTR4(priv_off);
  if (max_priv > 0) {
    REQ_PTR(priv_k);
    REQ_PTR(priv_v);
  }
  REQ_PTR(master_k);
  REQ_PTR(master_v);
  REQ(master_sel == nullptr || aligned4(master_sel), TDX_EINVAL, "master_sel not 4-byte aligned");
  REQ(master_sel == nullptr || (master_stride >= 0 && master_stride % (d.dtype == TDX_BF16 ? 8 : 4) == 0),
      TDX_EINVAL, "master_stride %lld is negative or breaks 16-byte alignment", (long long)master_stride);
  REQ_PTR4(diff_off);
  // diff arrays may be empty (all rows empty) but must then still be valid
  // pointers to zero-length storage; they are only read through diff_off.
  REQ(diff_idx != nullptr && diff_k != nullptr && diff_v != nullptr, TDX_EINVAL, "diff arrays are null");
  REQ(aligned16(diff_k) && aligned16(diff_v), TDX_EINVAL, "diff_k/diff_v not 16-byte aligned");
  REQ_PTR(out);
  const size_t need = tdx::restore_attn_ws_bytes(d, max_priv);
  REQ(ws != nullptr && aligned16(ws) && ws_bytes >= need, TDX_EWORKSPACE,
      "workspace needs %zu bytes (16-byte aligned), got %zu", need, ws_bytes);
  const tdx::MasterRef mref{master_k, master_v, master_sel, master_sel ? master_stride : 0};
  hipError_t e = tdx::launch_restore_attn(d, *layout, q, priv_off, priv_k, priv_v, max_priv, mref,
                                          diff_off, diff_idx, diff_k, diff_v, scale, out, ws,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tdx_restore_attn launch");
  return ok();
  GUARD_END
}

// ---- paged KV layout ----------------------------------------------------------


int tdx_rerotate_paged(const tdx_shape* shape, const tdx_layout* layout, const tdx_paged_kv* cached,
                       const tdx_paged_kv* out, void* stream) {
  GUARD_BEGIN
  tdx::Dims d{};
  int rc;
  if ((rc = check_shape(shape, &d)) != TDX_OK) return rc;
  if ((rc = check_layout(layout, &d, true)) != TDX_OK) return rc;
  const int64_t np = (d.T + TDX_DIFF_BLOCK - 1) / TDX_DIFF_BLOCK;
  tdx::PageMap pin{}, pout{};
  if ((rc = check_paged(cached, "cached", false, 1, np, &pin)) != TDX_OK) return rc;
  if ((rc = check_paged(out, "out", false, d.N, np, &pout)) != TDX_OK) return rc;
  hipError_t e = tdx::launch_rerotate_paged(d, *layout, cached->k_pool, pin, out->k_pool, pout,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tdx_rerotate_paged launch");
  return ok();
  GUARD_END
}

int tdx_select_important_paged(const tdx_shape* shape, const tdx_layout* layout, int32_t check_layer,
                               const tdx_paged_kv* k_reuse, const void* k_recomp, int32_t k, float* dev,
                               float* score, float* agent_dev, int32_t* selected, int32_t* master, void* ws,
                               size_t ws_bytes, void* stream) {
  GUARD_BEGIN
  tdx::Dims d{};
  int rc;
  if ((rc = check_shape(shape, &d)) != TDX_OK) return rc;
  if ((rc = check_layout(layout, &d, false)) != TDX_OK) return rc;
  REQ(check_layer >= 0 && check_layer < d.L, TDX_EINVAL, "check_layer %d outside [0, %d)", check_layer, d.L);
  REQ(k >= 1 && k <= d.T, TDX_EINVAL, "k %d outside [1, %d]", k, d.T);
  tdx::PageMap pm{};
  if ((rc = check_paged(k_reuse, "k_reuse", false, d.N, (d.T + TDX_DIFF_BLOCK - 1) / TDX_DIFF_BLOCK, &pm)) !=
      TDX_OK)
    return rc;
  REQ_PTR(k_recomp);
  REQ_PTR4(dev);
  REQ_PTR4(score);
  REQ_PTR4(agent_dev);
  REQ_PTR4(selected);
  REQ_PTR4(master);
  const size_t need = tdx::select_ws_bytes(d);
  REQ(ws != nullptr && aligned16(ws) && ws_bytes >= need, TDX_EWORKSPACE,
      "workspace needs %zu bytes (16-byte aligned), got %zu", need, ws_bytes);
  hipError_t e = tdx::launch_select_paged(d, check_layer, k_reuse->k_pool, pm, k_recomp, k, dev, score, agent_dev,
                                          selected, master, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tdx_select_important_paged launch");
  return ok();
  GUARD_END
}

int tdx_diff_encode_paged(const tdx_shape* shape, const tdx_layout* layout, const int32_t* master,
                          const tdx_paged_kv* agents, int64_t cap_blocks, int32_t* diff_off, int32_t* diff_idx,
                          int32_t* diff_page, void* diff_k, void* diff_v, int64_t* nnz, void* ws, size_t ws_bytes,
                          void* stream) {
  GUARD_BEGIN
  tdx::Dims d{};
  int rc;
  if ((rc = check_shape(shape, &d)) != TDX_OK) return rc;
  if ((rc = check_layout(layout, &d, false)) != TDX_OK) return rc;
  REQ(d.T % TDX_DIFF_BLOCK == 0, TDX_EINVAL, "n_tokens %d is not a multiple of 16", d.T);
  REQ(cap_blocks >= 0, TDX_EINVAL, "cap_blocks < 0");
  REQ((int64_t)d.N * d.L <= INT32_MAX, TDX_EUNSUPPORTED, "too many CSR rows");
  REQ_PTR4(master);
  tdx::PageMap pm{};
  if ((rc = check_paged(agents, "agents", true, d.N, d.T / TDX_DIFF_BLOCK, &pm)) != TDX_OK) return rc;
  REQ_PTR4(diff_off);
  REQ((reinterpret_cast<uintptr_t>(nnz) & 7u) == 0 && nnz != nullptr, TDX_EINVAL, "nnz is null or not 8-byte aligned");
  REQ((diff_k == nullptr) == (diff_v == nullptr), TDX_EINVAL, "diff_k and diff_v must both be set or both be NULL");
  if (cap_blocks > 0) {
    REQ_PTR4(diff_idx);
    REQ_PTR4(diff_page);
    if (diff_k != nullptr) {
      REQ_PTR(diff_k);
      REQ_PTR(diff_v);
    }
  }
  const size_t need = tdx::encode_ws_bytes(d);
  REQ(ws != nullptr && aligned16(ws) && ws_bytes >= need, TDX_EWORKSPACE,
      "workspace needs %zu bytes (16-byte aligned), got %zu", need, ws_bytes);
  hipError_t e = tdx::launch_encode_paged(d, master, agents->k_pool, agents->v_pool, pm, cap_blocks, diff_off,
                                          diff_idx, diff_page, diff_k, diff_v, nnz, ws,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tdx_diff_encode_paged launch");
  return ok();
  GUARD_END
}

int tdx_restore_attn_paged(const tdx_shape* shape, const tdx_layout* layout, const void* q,
                           const int32_t* priv_off, const tdx_paged_kv* priv, int32_t max_priv,
                           const tdx_paged_kv* agents, const int32_t* master_sel, const int32_t* diff_off,
                           const int32_t* diff_idx, const int32_t* diff_page, float scale, void* out, void* ws,
                           size_t ws_bytes, void* stream) {
  GUARD_BEGIN
  tdx::Dims d{};
  int rc;
  if ((rc = check_shape(shape, &d)) != TDX_OK) return rc;
  if ((rc = check_layout(layout, &d, true)) != TDX_OK) return rc;
  REQ(d.T % TDX_DIFF_BLOCK == 0, TDX_EINVAL, "n_tokens %d is not a multiple of 16", d.T);
  REQ(d.Hq / d.Hkv <= 16, TDX_EUNSUPPORTED, "more than 16 query heads per KV head");
  REQ(max_priv >= 0, TDX_EINVAL, "max_priv < 0");
  if ((rc = check_restore_tiles(d, max_priv)) != TDX_OK) return rc;
  REQ(scale > 0.0f, TDX_EINVAL, "scale must be > 0");
  REQ_PTR(q);
  REQ_PTR4(priv_off);
  tdx::PageMap ppm{nullptr, 0, 1}, apm{};
  if (max_priv > 0 &&
      (rc = check_paged(priv, "priv", true, d.N, (max_priv + TDX_DIFF_BLOCK - 1) / TDX_DIFF_BLOCK, &ppm)) != TDX_OK)
    return rc;
  if ((rc = check_paged(agents, "agents", true, d.N, d.T / TDX_DIFF_BLOCK, &apm)) != TDX_OK) return rc;
  REQ(master_sel == nullptr || aligned4(master_sel), TDX_EINVAL, "master_sel not 4-byte aligned");
  REQ_PTR4(diff_off);
  // diff arrays may be empty (all rows empty) but must then still be valid
  // pointers to zero-length storage; they are only read through diff_off.
  REQ(diff_idx != nullptr && diff_page != nullptr, TDX_EINVAL, "diff arrays are null");
  REQ_PTR(out);
  const size_t need = tdx::restore_attn_ws_bytes(d, max_priv);
  REQ(ws != nullptr && aligned16(ws) && ws_bytes >= need, TDX_EWORKSPACE,
      "workspace needs %zu bytes (16-byte aligned), got %zu", need, ws_bytes);
  const void* pk = max_priv > 0 ? priv->k_pool : agents->k_pool;  // not read when max_priv = 0
  const void* pv = max_priv > 0 ? priv->v_pool : agents->v_pool;
  hipError_t e = tdx::launch_restore_attn_paged(d, *layout, q, priv_off, pk, pv, ppm, max_priv, agents->k_pool,
                                                agents->v_pool, apm, master_sel, diff_off, diff_idx, diff_page,
                                                scale, out, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tdx_restore_attn_paged launch");
  return ok();
  GUARD_END
}

// The GPU can read p: device memory or registered (pinned) host memory.
bool gpu_readable(const void* p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of an unregistered pointer
    return false;
  }
  return at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeHost || at.type == hipMemoryTypeManaged;
}

size_t tdx_restore_transfer_workspace(const tdx_shape* shape, const tdx_layout* layout, int32_t n_req,
                                      int32_t layer_begin, int32_t layer_end) {
  tdx::Dims d{};
  if (check_shape(shape, &d) != TDX_OK || check_layout(layout, &d, false) != TDX_OK) return 0;
  if (n_req < 1 || layer_begin < 0 || layer_end <= layer_begin || layer_end > d.L) return 0;
  return tdx::transfer_ws_bytes(d, n_req, layer_end - layer_begin);
}

}  // extern "C"

namespace {
// Shared by the dense-output and paged-output transfer restores: out_paged
// null = dense k_out/v_out [n_req][L][T][Hkv][D].
int restore_transfer_impl(const char* what, const tdx_shape* shape, const tdx_layout* layout, const void* master_k,
                          const void* master_v, const int32_t* diff_off, const int32_t* diff_idx,
                          const void* diff_k, const void* diff_v, const int32_t* agents, int32_t n_req,
                          int32_t layer_begin, int32_t layer_end, void* k_out, void* v_out,
                          const tdx_paged_kv* out_paged, void* ws, size_t ws_bytes, void* stream) {
  tdx::Dims d{};
  int rc;
  if ((rc = check_shape(shape, &d)) != TDX_OK) return rc;
  if ((rc = check_layout(layout, &d, true)) != TDX_OK) return rc;
  REQ(d.T % TDX_DIFF_BLOCK == 0, TDX_EINVAL, "n_tokens %d is not a multiple of 16", d.T);
  REQ(n_req >= 1, TDX_EINVAL, "n_req %d < 1", n_req);
  REQ(layer_begin >= 0 && layer_begin < layer_end && layer_end <= d.L, TDX_EINVAL,
      "layer range [%d, %d) is not inside [0, %d)", layer_begin, layer_end, d.L);
  REQ((long long)n_req * (layer_end - layer_begin) <= (1LL << 31) - 1, TDX_EUNSUPPORTED, "too many rows");
  REQ_PTR(master_k);
  REQ_PTR(master_v);
  REQ_PTR4(diff_off);
  REQ(diff_idx != nullptr && diff_k != nullptr && diff_v != nullptr, TDX_EINVAL, "diff arrays are null");
  REQ(aligned16(diff_k) && aligned16(diff_v), TDX_EINVAL, "diff_k/diff_v not 16-byte aligned");
  REQ_PTR4(agents);
  tdx::PageMap opm{nullptr, 0, 1};
  if (out_paged != nullptr) {
    if ((rc = check_paged(out_paged, "out", true, n_req, d.T / TDX_DIFF_BLOCK, &opm)) != TDX_OK) return rc;
    k_out = out_paged->k_pool;
    v_out = out_paged->v_pool;
  } else {
    REQ_PTR(k_out);
    REQ_PTR(v_out);
  }
  const size_t need = tdx::transfer_ws_bytes(d, n_req, layer_end - layer_begin);
  REQ(ws != nullptr && aligned16(ws) && ws_bytes >= need, TDX_EWORKSPACE, "workspace of %zu bytes < %zu", ws_bytes, need);
  REQ(gpu_readable(master_k) && gpu_readable(master_v) && gpu_readable(diff_off) && gpu_readable(diff_idx) &&
          gpu_readable(diff_k) && gpu_readable(diff_v),
      TDX_EINVAL, "Master and diff record must be device memory or pinned host memory");
  tdx::TransferArgs t{};
  t.mk = master_k;
  t.mv = master_v;
  t.diff_off = diff_off;
  t.diff_idx = diff_idx;
  t.dk = diff_k;
  t.dv = diff_v;
  t.agents = agents;
  t.n_req = n_req;
  t.l0 = layer_begin;
  t.l1 = layer_end;
  t.blk_start = layout->blk_start;
  t.src_pos = layout->src_pos;
  t.dst_pos = layout->dst_pos;
  t.k_out = k_out;
  t.v_out = v_out;
  t.ws = ws;
  t.out_pages = opm;
  hipError_t e = tdx::launch_transfer(d, t, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, what);
  return ok();
}
}  // namespace

extern "C" {

int tdx_restore_transfer(const tdx_shape* shape, const tdx_layout* layout, const void* master_k,
                         const void* master_v, const int32_t* diff_off, const int32_t* diff_idx,
                         const void* diff_k, const void* diff_v, const int32_t* agents, int32_t n_req,
                         int32_t layer_begin, int32_t layer_end, void* k_out, void* v_out, void* ws,
                         size_t ws_bytes, void* stream) {
  GUARD_BEGIN
  return restore_transfer_impl("tdx_restore_transfer launch", shape, layout, master_k, master_v, diff_off, diff_idx,
                               diff_k, diff_v, agents, n_req, layer_begin, layer_end, k_out, v_out, nullptr, ws,
                               ws_bytes, stream);
  GUARD_END
}

int tdx_restore_transfer_paged(const tdx_shape* shape, const tdx_layout* layout, const void* master_k,
                               const void* master_v, const int32_t* diff_off, const int32_t* diff_idx,
                               const void* diff_k, const void* diff_v, const int32_t* agents, int32_t n_req,
                               int32_t layer_begin, int32_t layer_end, const tdx_paged_kv* out, void* ws,
                               size_t ws_bytes, void* stream) {
  GUARD_BEGIN
  REQ(out != nullptr, TDX_EINVAL, "out is null");
  return restore_transfer_impl("tdx_restore_transfer_paged launch", shape, layout, master_k, master_v, diff_off,
                               diff_idx, diff_k, diff_v, agents, n_req, layer_begin, layer_end, nullptr, nullptr,
                               out, ws, ws_bytes, stream);
  GUARD_END
}

int tdx_restore_dense(const tdx_shape* shape, const tdx_layout* layout, const void* master_k,
                      const void* master_v, const int32_t* master_sel, int64_t master_stride,
                      const int32_t* diff_off, const int32_t* diff_idx,
                      const void* diff_k, const void* diff_v, void* k_dense, void* v_dense,
                      void* stream) {
  GUARD_BEGIN
  tdx::Dims d{};
  int rc;
  if ((rc = check_shape(shape, &d)) != TDX_OK) return rc;
  if ((rc = check_layout(layout, &d, true)) != TDX_OK) return rc;
  REQ(d.T % TDX_DIFF_BLOCK == 0, TDX_EINVAL, "n_tokens %d is not a multiple of 16", d.T);
  REQ_PTR(master_k);
  REQ_PTR(master_v);
  REQ(master_sel == nullptr || aligned4(master_sel), TDX_EINVAL, "master_sel not 4-byte aligned");
  REQ(master_sel == nullptr || (master_stride >= 0 && master_stride % (d.dtype == TDX_BF16 ? 8 : 4) == 0),
      TDX_EINVAL, "master_stride %lld is negative or breaks 16-byte alignment", (long long)master_stride);
  REQ_PTR4(diff_off);
  REQ(diff_idx != nullptr && diff_k != nullptr && diff_v != nullptr, TDX_EINVAL, "diff arrays are null");
  REQ(aligned16(diff_k) && aligned16(diff_v), TDX_EINVAL, "diff_k/diff_v not 16-byte aligned");
  REQ_PTR(k_dense);
  REQ_PTR(v_dense);
  const tdx::MasterRef mref{master_k, master_v, master_sel, master_sel ? master_stride : 0};
  hipError_t e = tdx::launch_restore_dense(d, *layout, mref, diff_off, diff_idx, diff_k, diff_v,
                                           k_dense, v_dense, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tdx_restore_dense launch");
  return ok();
  GUARD_END
}

size_t tdx_decode_attn_dense_workspace(const tdx_shape* shape, const tdx_layout* layout,
                                       int32_t max_priv) {
  tdx::Dims d{};
  if (check_shape(shape, &d) != TDX_OK || check_layout(layout, &d, false) != TDX_OK || !restore_tiles_fit(d, max_priv))
    return 0;
  return tdx::dense_attn_ws_bytes(d, max_priv);
}

int tdx_decode_attn_dense(const tdx_shape* shape, const tdx_layout* layout, const void* q,
                          const int32_t* priv_off, const void* priv_k, const void* priv_v,
                          int32_t max_priv, const void* k_dense, const void* v_dense, float scale,
                          void* out, void* ws, size_t ws_bytes, void* stream) {
  GUARD_BEGIN
  tdx::Dims d{};
  int rc;
  if ((rc = check_shape(shape, &d)) != TDX_OK) return rc;
  if ((rc = check_layout(layout, &d, false)) != TDX_OK) return rc;
  REQ(d.T % TDX_DIFF_BLOCK == 0, TDX_EINVAL, "n_tokens %d is not a multiple of 16", d.T);
  REQ(d.Hq / d.Hkv <= 16, TDX_EUNSUPPORTED, "more than 16 query heads per KV head");
  REQ(max_priv >= 0, TDX_EINVAL, "max_priv < 0");
  if ((rc = check_restore_tiles(d, max_priv)) != TDX_OK) return rc;
  REQ(scale > 0.0f, TDX_EINVAL, "scale must be > 0");
  REQ_PTR(q);
  REQ_PTR4(priv_off);
  if (max_priv > 0) {
    REQ_PTR(priv_k);
    REQ_PTR(priv_v);
  }
  REQ_PTR(k_dense);
  REQ_PTR(v_dense);
  REQ_PTR(out);
  const size_t need = tdx::dense_attn_ws_bytes(d, max_priv);
  REQ(ws != nullptr && aligned16(ws) && ws_bytes >= need, TDX_EWORKSPACE,
      "workspace needs %zu bytes (16-byte aligned), got %zu", need, ws_bytes);
  hipError_t e = tdx::launch_dense_attn(d, q, priv_off, priv_k, priv_v, max_priv, k_dense, v_dense,
                                        scale, out, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tdx_decode_attn_dense launch");
  return ok();
  GUARD_END
}

}  // extern "C"

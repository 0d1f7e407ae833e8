// Device helpers shared by the tdx HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tdx.h"

namespace tdx {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlock = TDX_DIFF_BLOCK;  // 16-token diff block

// ---- element formats -------------------------------------------------------
// A 16-byte vector holds 8 bf16 or 4 fp32 values.  bf16 is kept as raw bits.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// (lo, hi) fp32 -> packed bf16 bits with one v_cvt_pk_bf16_f32: round to
// nearest, ties to even, denormals kept, NaN -> quiet NaN with the upper
// payload bits (the same bits as ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) for
// non-NaN u and (u >> 16) | 0x40 for NaN; checked on gfx950 for all 2^32 inputs).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// fp32 -> bf16 bits (as pack_bf16)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16(f, 0.0f) & 0xFFFFu; }

template <typename E>
struct Fmt;

template <>
struct Fmt<uint16_t> {  // bf16 bits
  static constexpr int VEC = 8;
  __device__ static __forceinline__ void unpack(const u32x4& v, float* x) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_lo(v[k]);
      x[2 * k + 1] = bf16_hi(v[k]);
    }
  }
  __device__ static __forceinline__ u32x4 pack(const float* x) {
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = pack_bf16(x[2 * k], x[2 * k + 1]);
    return v;
  }
};

template <>
struct Fmt<float> {
  static constexpr int VEC = 4;
  __device__ static __forceinline__ void unpack(const u32x4& v, float* x) {
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(v[k]);
  }
  __device__ static __forceinline__ u32x4 pack(const float* x) {
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __float_as_uint(x[k]);
    return v;
  }
};

template <typename E>
__device__ __forceinline__ u32x4 ld16(const E* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
template <typename E>
__device__ __forceinline__ void st16(E* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
// Streaming load: data this kernel reads once (non-temporal hint, so the
// stream does not displace lines that are reused from the caches).
#ifndef TDX_NT_LOADS
#define TDX_NT_LOADS 1
#endif
template <typename E>
__device__ __forceinline__ u32x4 ld16_nt(const E* p) {
#if TDX_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}
// Streaming store: the written data is not re-read by this kernel.
template <typename E>
__device__ __forceinline__ void st16_nt(E* p, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// A paged KV pool: page p of layer l holds 16 token rows of Hkv*D elements
// at pool + (l * n_pages + p) * 16 * Hkv * D; row r of the page table starts
// at pages + r * stride.  Page IDs outside [0, n_pages) are clamped, so a bad
// table reads or writes a wrong page of the pool but never outside it.
struct PageMap {
  const int32_t* pages;
  long long stride;
  long long n_pages;
};
__device__ __forceinline__ long long page_at(const PageMap& m, long long row, long long j) {
  const long long p = m.pages[row * m.stride + j];
  return p < 0 ? 0 : (p >= m.n_pages ? m.n_pages - 1 : p);
}

// RoPE inverse frequency theta^(-2e/D) in double precision.
__device__ __forceinline__ double rope_inv_freq(double theta, int e, int D) {
  return pow(theta, -2.0 * (double)e / (double)D);
}

// Element offset of the Master's cache: (*sel clamped to [0, N)) * stride,
// 0 without a selector.
__device__ __forceinline__ size_t master_offset(const int32_t* sel, long long stride, int N) {
  if (sel == nullptr) return 0;
  const int m = min(max(sel[0], 0), N - 1);
  return (size_t)m * (size_t)stride;
}

// Restore-attention modes: FUSED = the Master patched with diff records
// tile by tile; DENSE = the comparator's attention over materialised caches.
enum AttnMode { FUSED = 0, DENSE = 1 };

}  // namespace tdx

// ---- internal launchers (implemented per kernel file, called by api.hip) ----
// Each returns hipSuccess or the launch error.  Arguments are already checked.
namespace tdx {

struct Dims {
  int N, B, T, L, Hkv, Hq, D;
  int dtype;
  double theta;
};

hipError_t launch_rerotate(const Dims& d, const tdx_layout& lay, const void* kc, void* out,
                           hipStream_t s);
// paged: cached K in pages cin (row 0), agent i's output in pages cout row i
hipError_t launch_rerotate_paged(const Dims& d, const tdx_layout& lay, const void* kc, const PageMap& cin,
                                 void* out, const PageMap& cout, hipStream_t s);

size_t select_ws_bytes(const Dims& d);
hipError_t launch_select(const Dims& d, const tdx_layout& lay, int check_layer,
                         const void* k_reuse, const void* k_recomp, int k, float* dev,
                         float* score, float* agent_dev, int32_t* selected, int32_t* master,
                         void* ws, hipStream_t s);

// paged: agent i's reused K at the check layer in pages pm row i of the pool
hipError_t launch_select_paged(const Dims& d, int check_layer, const void* kr_pool, const PageMap& pm,
                               const void* k_recomp, int k, float* dev, float* score, float* agent_dev,
                               int32_t* selected, int32_t* master, void* ws, hipStream_t s);

size_t encode_ws_bytes(const Dims& d);
hipError_t launch_encode(const Dims& d, const int32_t* master, const void* ak, const void* av,
                         int64_t cap, int32_t* diff_off, int32_t* diff_idx, void* diff_k,
                         void* diff_v, int64_t* nnz, void* mk_out, void* mv_out, void* ws,
                         hipStream_t s);

// paged: agent a's block beta is page pm[a][beta] of the K and V pools; the
// record holds each entry's page (diff_page) and, when diff_k is set, copies
hipError_t launch_encode_paged(const Dims& d, const int32_t* master, const void* k_pool, const void* v_pool,
                               const PageMap& pm, int64_t cap, int32_t* diff_off, int32_t* diff_idx,
                               int32_t* diff_page, void* diff_k, void* diff_v, int64_t* nnz, void* ws,
                               hipStream_t s);

size_t restore_attn_ws_bytes(const Dims& d, int max_priv);
// The Master's cache: k/v + m * stride elements, m = *sel clamped to [0, N)
// (m = 0 when sel is null).
struct MasterRef {
  const void* k;
  const void* v;
  const int32_t* sel;
  int64_t stride;
};

hipError_t launch_restore_attn(const Dims& d, const tdx_layout& lay, const void* q,
                               const int32_t* priv_off, const void* pk, const void* pv,
                               int max_priv, const MasterRef& master,
                               const int32_t* diff_off, const int32_t* diff_idx,
                               const void* dk, const void* dv, float scale, void* out, void* ws,
                               hipStream_t s);

// paged: agent i's private history in pages ppm row i of the private pools;
// the Master (agent *master_sel) and the diff blocks in pages of the agents'
// pools (the Master's row of apm; entry e's page diff_page[e])
hipError_t launch_restore_attn_paged(const Dims& d, const tdx_layout& lay, const void* q, const int32_t* priv_off,
                                     const void* pk_pool, const void* pv_pool, const PageMap& ppm, int max_priv,
                                     const void* ak_pool, const void* av_pool, const PageMap& apm,
                                     const int32_t* master_sel, const int32_t* diff_off, const int32_t* diff_idx,
                                     const int32_t* diff_page, float scale, void* out, void* ws, hipStream_t s);

hipError_t launch_restore_dense(const Dims& d, const tdx_layout& lay, const MasterRef& master,
                                const int32_t* diff_off,
                                const int32_t* diff_idx, const void* dk, const void* dv,
                                void* kd, void* vd, hipStream_t s);

size_t dense_attn_ws_bytes(const Dims& d, int max_priv);
hipError_t launch_dense_attn(const Dims& d, const void* q, const int32_t* priv_off,
                             const void* pk, const void* pv, int max_priv, const void* kd,
                             const void* vd, float scale, void* out, void* ws, hipStream_t s);

// fp32 caches: restore-attention on the fp32 vector units (attn_f32.hip).
// Pointers as in the bf16 path; sk/sv = the Master (or, with msel, every
// agent's cache at stride mstride) for FUSED, the dense caches
// [N][L][T][Hkv][D] for DENSE; paged (FUSED only): sk/sv/dk/dv are the
// agents' pools and pk/pv the private pools, mapped by mpm / dpm / ppm.
struct F32AttnArgs {
  const float* q;  // [N][L][Hq][D]
  const int32_t* priv_off;
  const float* pk;
  const float* pv;
  const float* sk;
  const float* sv;
  const int32_t* msel;
  long long mstride;
  const int32_t* diff_off;
  const int32_t* diff_idx;
  const float* dk;
  const float* dv;
  const int32_t* blk_start;
  const int32_t* src_pos;
  const int32_t* dst_pos;
  PageMap mpm, dpm, ppm;
  float scale_log2;  // softmax scale * log2(e)
  float* out;        // [N][L][Hq][D]
  // set by launch_attn_f32
  const float2* tab;
  float* part;
  int N, L, T, B, Hkv, Hq, pmax;
};
size_t f32_attn_ws_bytes(const Dims& d, int max_priv, bool fused);
hipError_t launch_attn_f32(const Dims& d, int mode, bool paged, F32AttnArgs a, int max_priv, void* ws,
                           hipStream_t s);

// Transfer-path restore: Master and diff records readable by the GPU
// (pinned host storage or device memory), requested agents, layer range.
struct TransferArgs {
  const void* mk;
  const void* mv;
  const int32_t* diff_off;
  const int32_t* diff_idx;
  const void* dk;
  const void* dv;
  const int32_t* agents;  // device [n_req]
  int n_req, l0, l1;
  const int32_t* blk_start;
  const int32_t* src_pos;
  const int32_t* dst_pos;
  void* k_out;  // [n_req][L][T][Hkv][D], or the output pools when out_pages is set
  void* v_out;
  void* ws;
  PageMap out_pages;  // pages: null for the dense output; row j = requested agent j's T/16 pages
};
size_t transfer_tab_off(const Dims& d, int n_req, int nl);
size_t transfer_ws_bytes(const Dims& d, int n_req, int nl);
hipError_t launch_transfer(const Dims& d, const TransferArgs& t, hipStream_t s);

}  // namespace tdx

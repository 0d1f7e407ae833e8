// a1: batched RoPE delta re-rotation of the cached shared K to all N agents.
//
// TokenDance notes, Summary "Method" and Figure 7 (path T3): the K of the
// shared blocks is corrected to every agent's absolute offsets by one
// group-wide RoPE pass instead of one pass per agent; Deep Analysis §0: the
// position difference of a block is fixed by one rotation R(Delta).
//
// Design (gfx950): the pass reads each cached K tile once and writes N
// rotated copies, so it is bound by HBM writes.  A workgroup owns a tile of
// up to 16 canonical tokens that lies inside one shared block, for a group of
// layers.  It evaluates cos/sin(Delta(i,b) * theta^(-2e/D)) for up to 32
// agents in double precision into LDS once, then streams: every lane holds the
// 16-byte chunk at dims [e0, e0+VEC) and its rotate-half partner at
// [e0+D/2, e0+D/2+VEC) in registers and emits both rotated chunks for every
// agent with 16-byte stores.  Loads and stores are plain: non-temporal stores
// were slower, and plain loads of the cached K slightly faster than
// non-temporal ones amid the write stream.
#include "common.h"

namespace tdx {
namespace {

constexpr int kThreads = 256;
#ifndef TDX_RR_TILE
#define TDX_RR_TILE 16
#endif
constexpr int kTileTok = TDX_RR_TILE;  // canonical tokens per workgroup
constexpr int kAgentChunk = 32;  // agents whose cos/sin sit in LDS at once
#ifndef TDX_RR_ITEMS
#define TDX_RR_ITEMS 2
#endif
constexpr int kItems = TDX_RR_ITEMS;  // (token, head) rows per lane per batch

#ifndef TDX_RR_TARGET_WG
#define TDX_RR_TARGET_WG 16384
#endif
#ifndef TDX_RR_NT_STORES
#define TDX_RR_NT_STORES 0
#endif

template <typename E>
__device__ __forceinline__ void st_out(E* p, const u32x4& v) {
#if TDX_RR_NT_STORES
  st16_nt(p, v);
#else
  st16(p, v);
#endif
}

// Column of element e in an agent's cos/sin row in LDS: each lane reads the
// VEC pairs of its chunk, and the groups of VEC pairs are padded by 2 pairs so
// that the lanes' 16-byte reads of neighbouring groups fall in different banks.
template <int VEC>
__device__ __forceinline__ int tab_col(int e) {
  return e + (e / VEC) * 2;
}

// One workgroup: canonical tokens [t0, t0+16) for layers [l0, l0+lpg).  The
// (layer, batch) steps run in sequence and the next step's input is loaded
// while the current one is written out for every agent.
//
// PAGED: the cached K and every agent's output live in 16-token pages of
// pools (a workgroup's tile is one page); pin row 0 lists the cached K's
// pages, pout row i agent i's pages, both in canonical token order.
template <typename E, int D, bool PAGED>
__global__ __launch_bounds__(kThreads) void rerotate_kernel(
    const E* __restrict__ kc, E* __restrict__ out, const int32_t* __restrict__ blk_start,
    const int32_t* __restrict__ src_pos, const int32_t* __restrict__ dst_pos, int N, int B,
    int T, int L, int Hkv, int lpg, int apg, double theta, PageMap pin, PageMap pout) {
  static_assert(!PAGED || kTileTok == kBlock, "a paged tile is one page");
  constexpr int VEC = Fmt<E>::VEC;
  constexpr int HALF = D / 2;
  constexpr int G = HALF / VEC;       // lanes per (token, head) row
  constexpr int RPP = kThreads / G;   // rows covered by the workgroup per item
  constexpr int TROW = HALF + 2 * G;  // padded cos/sin row of one agent (float2)
  extern __shared__ __align__(16) unsigned char smem[];
  float2* tab = reinterpret_cast<float2*>(smem);                      // [kAgentChunk][HALF]
  double* invf = reinterpret_cast<double*>(tab + kAgentChunk * TROW);  // [HALF]
  long long* opage = reinterpret_cast<long long*>(invf + HALF);        // [kAgentChunk] (paged)
  int32_t* szero = reinterpret_cast<int32_t*>(opage + kAgentChunk);    // [kAgentChunk] Delta == 0
  int32_t* sblk = szero + kAgentChunk;                                 // [B+1]

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTileTok;
  const int t1 = min(t0 + kTileTok, T);
  const int l0 = blockIdx.y * lpg;
  const int l1 = min(l0 + lpg, L);
  const int ab = blockIdx.z * apg;  // this workgroup's agents [ab, ae)
  const int ae = min(ab + apg, N);
  if (t0 >= T || l0 >= L || ab >= ae) return;  // uniform over the workgroup

  for (int b = tid; b <= B; b += kThreads) sblk[b] = blk_start[b];
  for (int e = tid; e < HALF; e += kThreads) invf[e] = rope_inv_freq(theta, e, D);
  __syncthreads();

  // first block containing t0: largest b with sblk[b] <= t0 (skips empty blocks)
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (sblk[mid] <= t0) lo = mid; else hi = mid - 1;
  }

  const int e0 = (tid % G) * VEC;
  const int row_base = tid / G;
  const size_t rowD = (size_t)Hkv * D;
  const int pj = t0 / kBlock;                         // paged: the tile's page column
  const long long ipage = PAGED ? page_at(pin, 0, pj) : 0;

  for (int b = lo; b < B && sblk[b] < t1; ++b) {
    const int ta = max(t0, sblk[b]);
    const int tb = min(t1, sblk[b + 1]);
    if (ta >= tb) continue;
    const int nrows = (tb - ta) * Hkv;
    const int nbatch = (nrows + RPP * kItems - 1) / (RPP * kItems);
    const int nsteps = (l1 - l0) * nbatch;
    const int sp = src_pos[b];
    for (int a0 = ab; a0 < ae; a0 += kAgentChunk) {
      const int na = min(kAgentChunk, ae - a0);
      __syncthreads();  // previous users of tab are done
      for (int x = tid; x < na * HALF; x += kThreads) {
        const int a = x / HALF, e = x % HALF;
        const double delta = (double)(dst_pos[(size_t)(a0 + a) * B + b] - sp);
        double sn, cs;
        sincos(delta * invf[e], &sn, &cs);
        tab[a * TROW + tab_col<VEC>(e)] = make_float2((float)cs, (float)sn);
      }
      for (int a = tid; a < na; a += kThreads) {
        if constexpr (PAGED) opage[a] = page_at(pout, a0 + a, pj);
        szero[a] = dst_pos[(size_t)(a0 + a) * B + b] == sp;
      }
      __syncthreads();
      // step = (layer, batch of rows)
      u32x4 xl[kItems], xh[kItems], nl[kItems], nh[kItems];
      auto load_step = [&](int step, u32x4* lo_, u32x4* hi_) {
        const int l = l0 + step / nbatch;
        const int rb = (step % nbatch) * RPP * kItems;
        const E* src = PAGED ? kc + (((size_t)l * pin.n_pages + ipage) * kBlock + (ta - t0)) * rowD
                             : kc + ((size_t)l * T + ta) * rowD;
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
          const int r = rb + row_base + k * RPP;
          if (r < nrows) {
            lo_[k] = ld16(src + (size_t)r * D + e0);
            hi_[k] = ld16(src + (size_t)r * D + HALF + e0);
          }
        }
      };
      load_step(0, xl, xh);
      for (int step = 0; step < nsteps; ++step) {
        if (step + 1 < nsteps) load_step(step + 1, nl, nh);  // in flight during the stores
        const int l = l0 + step / nbatch;
        const int rb = (step % nbatch) * RPP * kItems;
        for (int a = 0; a < na; ++a) {
          // R(0) is the identity: a zero shift stores the cached bits as
          // they are (signed zeros and non-finite values included), which
          // x*1 - y*0 would not (workgroup-uniform branch)
          if (szero[a]) {
            E* dst = PAGED ? out + (((size_t)l * pout.n_pages + opage[a]) * kBlock + (ta - t0)) * rowD
                           : out + ((size_t)(a0 + a) * L + l) * (size_t)T * rowD + (size_t)ta * rowD;
#pragma unroll
            for (int k = 0; k < kItems; ++k) {
              const int r = rb + row_base + k * RPP;
              if (r < nrows) {
                st_out(dst + (size_t)r * D + e0, xl[k]);
                st_out(dst + (size_t)r * D + HALF + e0, xh[k]);
              }
            }
            continue;
          }
          float cs[VEC], sn[VEC];
#pragma unroll
          for (int j = 0; j < VEC; ++j) {
            const float2 v = tab[a * TROW + tab_col<VEC>(e0 + j)];
            cs[j] = v.x;
            sn[j] = v.y;
          }
          E* dst = PAGED ? out + (((size_t)l * pout.n_pages + opage[a]) * kBlock + (ta - t0)) * rowD
                         : out + ((size_t)(a0 + a) * L + l) * (size_t)T * rowD + (size_t)ta * rowD;
#pragma unroll
          for (int k = 0; k < kItems; ++k) {
            const int r = rb + row_base + k * RPP;
            if (r < nrows) {
              float x[VEC], y[VEC], ox[VEC], oy[VEC];
              Fmt<E>::unpack(xl[k], x);
              Fmt<E>::unpack(xh[k], y);
#pragma unroll
              for (int j = 0; j < VEC; ++j) {
                ox[j] = x[j] * cs[j] - y[j] * sn[j];
                oy[j] = y[j] * cs[j] + x[j] * sn[j];
              }
              st_out(dst + (size_t)r * D + e0, Fmt<E>::pack(ox));
              st_out(dst + (size_t)r * D + HALF + e0, Fmt<E>::pack(oy));
            }
          }
        }
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
          xl[k] = nl[k];
          xh[k] = nh[k];
        }
      }
    }
  }
}

template <typename E, int D, bool PAGED>
hipError_t launch_t(const Dims& d, const tdx_layout& lay, const void* kc, void* out, const PageMap& pin,
                    const PageMap& pout, hipStream_t s) {
  const int tiles = (d.T + kTileTok - 1) / kTileTok;
  // enough workgroups to fill 256 CUs several times over: layers split
  // first (>= 1 layer each), then agents
  int groups = (TDX_RR_TARGET_WG + tiles - 1) / tiles;
  groups = groups < 1 ? 1 : (groups > d.L ? d.L : groups);
  const int lpg = (d.L + groups - 1) / groups;
  groups = (d.L + lpg - 1) / lpg;
  int asplit = (2048 + tiles * groups - 1) / (tiles * groups);  // only for small rounds
  asplit = asplit < 1 ? 1 : (asplit > d.N ? d.N : asplit);
  const int apg = (d.N + asplit - 1) / asplit;
  asplit = (d.N + apg - 1) / apg;
  dim3 grid(tiles, groups, asplit);
  const size_t lds = (size_t)kAgentChunk * (D / 2 + 2 * (D / 2 / Fmt<E>::VEC)) * 8 + (D / 2) * 8 +
                     (size_t)kAgentChunk * 8 + (size_t)kAgentChunk * 4 + (size_t)(d.B + 1) * 4;
  hipLaunchKernelGGL((rerotate_kernel<E, D, PAGED>), grid, dim3(kThreads), lds, s,
                     static_cast<const E*>(kc), static_cast<E*>(out), lay.blk_start,
                     lay.src_pos, lay.dst_pos, d.N, d.B, d.T, d.L, d.Hkv, lpg, apg, d.theta, pin, pout);
  return hipGetLastError();
}

template <bool PAGED>
hipError_t dispatch(const Dims& d, const tdx_layout& lay, const void* kc, void* out, const PageMap& pin,
                    const PageMap& pout, hipStream_t s) {
  if (d.dtype == TDX_BF16) {
    return d.D == 128 ? launch_t<uint16_t, 128, PAGED>(d, lay, kc, out, pin, pout, s)
                      : launch_t<uint16_t, 64, PAGED>(d, lay, kc, out, pin, pout, s);
  }
  return d.D == 128 ? launch_t<float, 128, PAGED>(d, lay, kc, out, pin, pout, s)
                    : launch_t<float, 64, PAGED>(d, lay, kc, out, pin, pout, s);
}

}  // namespace

hipError_t launch_rerotate(const Dims& d, const tdx_layout& lay, const void* kc, void* out,
                           hipStream_t s) {
  const PageMap none{nullptr, 0, 1};
  return dispatch<false>(d, lay, kc, out, none, none, s);
}

hipError_t launch_rerotate_paged(const Dims& d, const tdx_layout& lay, const void* kc, const PageMap& cin,
                                 void* out, const PageMap& cout, hipStream_t s) {
  return dispatch<true>(d, lay, kc, out, cin, cout, s);
}

}  // namespace tdx

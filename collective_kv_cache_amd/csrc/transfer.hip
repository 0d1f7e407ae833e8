// NEXT: transfer-path restore of Mirrors from host storage.
//
// TokenDance notes, Summary "Method" and §3d (Algorithm 1, "Fused Diff
// Restore"), blog §4.4: the Master and the Mirrors' block-sparse diffs live
// in storage outside the GPU (LMCache's CPU backend); a Mirror's KV is
// rebuilt layer by layer on the way in: the Master's layer chunk and the
// Mirror's diff blocks are transferred, merged block by block and
// RoPE-recovered into the agent's KV, with no dense Mirror built in between.
//
// Design (gfx950): the pages stage each layer through two GPU buffers filled
// by DMA on a copy stream (ping-pong) so that transfer and merge overlap.  On
// this GPU a kernel that reads pinned host memory directly reaches the same
// PCIe rate as a DMA copy, so the merge kernel reads the Master chunk and the
// diff blocks straight from host storage and writes the restored rows:
// one pass, no staging buffer, no second stream; the overlap of transfer and
// merge happens between the many workgroups in flight.  One launch covers a
// layer range, so a caller can restore layer l+1 while attention runs on
// layer l on another stream.
//
//  transfer_slot_kernel   one workgroup per (requested agent, layer): the
//                         diff entry of every 16-token block of the row, or -1
//  transfer_tab_kernel    cos/sin of Delta(agent, b) * theta^(-2e/D) in double,
//                         stored as fp32, per (requested agent, block, e)
//  transfer_kernel        one workgroup per (16-token block, layer): the
//                         Master's rows are read once and serve every
//                         requested agent; an agent whose diff holds the block
//                         takes its own rows instead; K rows are rotated by the
//                         shift of the shared block holding them and rounded,
//                         V rows are copied.
#include "common.h"

namespace tdx {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = kBlock;               // 16-token diff block
constexpr int kMaxTileBlocks = kTile;       // a 16-token tile touches at most 16 blocks

__global__ __launch_bounds__(kThreads) void transfer_slot_kernel(const int32_t* __restrict__ agents,
                                                                 const int32_t* __restrict__ diff_off,
                                                                 const int32_t* __restrict__ diff_idx,
                                                                 int N, int L, int l0, int nl, int nb,
                                                                 int32_t* __restrict__ slot) {
  const int j = blockIdx.x / nl, ll = blockIdx.x % nl;
  const int r = min(max(agents[j], 0), N - 1) * L + l0 + ll;
  int32_t* row = slot + (size_t)blockIdx.x * nb;
  for (int b = threadIdx.x; b < nb; b += kThreads) row[b] = -1;
  __syncthreads();
  const int e0 = diff_off[r];
  const int e1 = e0 + min(max(diff_off[r + 1] - e0, 0), nb);
  for (int e = e0 + threadIdx.x; e < e1; e += kThreads) {
    const int beta = diff_idx[e];
    if (beta >= 0 && beta < nb) row[beta] = e;
  }
}

__global__ __launch_bounds__(kThreads) void transfer_tab_kernel(const int32_t* __restrict__ agents,
                                                                const int32_t* __restrict__ src_pos,
                                                                const int32_t* __restrict__ dst_pos,
                                                                int N, int n_req, int B, int D, double theta,
                                                                float2* __restrict__ tab) {
  const int half = D / 2;
  const size_t n = (size_t)n_req * B * half;
  for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(x % half);
    const size_t jb = x / half;
    const int b = (int)(jb % B);
    const int j = (int)(jb / B);
    const double delta = (double)(dst_pos[(size_t)min(max(agents[j], 0), N - 1) * B + b] - src_pos[b]);
    double sn, cs;
    sincos(delta * rope_inv_freq(theta, e, D), &sn, &cs);
    tab[x] = make_float2((float)cs, (float)sn);
  }
}

// Rows of one (block, layer): (token, head) row = 16-byte chunks at dims
// [e0, e0 + VEC) and [e0 + D/2, e0 + D/2 + VEC), G lanes per row, RPP rows per
// pass, NP passes cover the tile's 16 * Hkv rows.  PAGED: requested agent
// j's tile is page opm[j][beta] of the output pools (16 rows of layer l).
template <typename E, int D, int NP, bool PAGED>
__global__ __launch_bounds__(kThreads) void transfer_kernel(
    const E* __restrict__ mk, const E* __restrict__ mv, const int32_t* __restrict__ slot,
    const E* __restrict__ dk, const E* __restrict__ dv, const float2* __restrict__ tab,
    const int32_t* __restrict__ blk_start, const int32_t* __restrict__ agents, const int32_t* __restrict__ src_pos,
    const int32_t* __restrict__ dst_pos, int N, int n_req, int B, int T, int L, int l0, int nl, int Hkv,
    E* __restrict__ k_out, E* __restrict__ v_out, PageMap opm) {
  constexpr int VEC = Fmt<E>::VEC;
  constexpr int HALF = D / 2;
  constexpr int G = HALF / VEC;
  constexpr int RPP = kThreads / G;
  __shared__ int32_t sst[kMaxTileBlocks], sid[kMaxTileBlocks];  // non-empty blocks of the tile
  __shared__ int s_nb;
  const int beta = blockIdx.x;
  const int ll = blockIdx.y;
  const int l = l0 + ll;
  const int tid = threadIdx.x;
  const int t0 = beta * kTile;
  const int nb = T / kTile;
  if (tid == 0) {
    // the non-empty shared blocks holding tokens of [t0, t0 + 16): the one
    // holding t0, then those starting inside the tile (at most 16 in all)
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (blk_start[mid] <= t0) lo = mid; else hi = mid - 1;
    }
    int n = 0;
    for (int b = lo; b < B && blk_start[b] < t0 + kTile && n < kMaxTileBlocks; ++b)
      if (blk_start[b + 1] > blk_start[b]) {
        sst[n] = blk_start[b];
        sid[n] = b;
        ++n;
      }
    s_nb = n;
  }
  __syncthreads();
  const int nbk = s_nb;

  const int e0 = (tid % G) * VEC;
  const int nrows = kTile * Hkv;
  const size_t rowHD = (size_t)Hkv * D;
  const size_t tile_off = ((size_t)l * T + t0) * rowHD;
  // this thread's rows of the Master tile: row0 + p * RPP, p < NP, from the
  // workgroup's first row NP * RPP * blockIdx.z (the workgroups along z
  // cover all 16 * Hkv rows of the tile)
  const int row0 = (int)blockIdx.z * NP * RPP + tid / G;
  u32x4 mkl[NP], mkh[NP], mvl[NP], mvh[NP];
  int bb[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = min(row0 + p * RPP, nrows - 1);
    const size_t off = tile_off + (size_t)row * D + e0;
    mkl[p] = ld16_nt(mk + off);
    mkh[p] = ld16_nt(mk + off + HALF);
    mvl[p] = ld16_nt(mv + off);
    mvh[p] = ld16_nt(mv + off + HALF);
    const int tok = t0 + row / Hkv;
    int x = 0;
    while (x + 1 < nbk && sst[x + 1] <= tok) ++x;
    bb[p] = sid[x];
  }
  for (int j = 0; j < n_req; ++j) {
    const int e = slot[((size_t)j * nl + ll) * nb + beta];  // uniform
    const float2* cs_j = tab + (size_t)j * B * HALF;
    const int32_t* dst_j = dst_pos + (size_t)min(max(agents[j], 0), N - 1) * B;
    const size_t orow = PAGED ? ((size_t)l * opm.n_pages + page_at(opm, j, beta)) * kTile
                              : ((size_t)j * L + l) * T + t0;
    E* ko = k_out + orow * rowHD;
    E* vo = v_out + orow * rowHD;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = row0 + p * RPP;
      if (row >= nrows) continue;
      u32x4 xl = mkl[p], xh = mkh[p], yl = mvl[p], yh = mvh[p];
      if (e >= 0) {  // the agent's own rows (the diff entry's block)
        const size_t off = ((size_t)e * kTile * rowHD) + (size_t)row * D + e0;
        xl = ld16_nt(dk + off);
        xh = ld16_nt(dk + off + HALF);
        yl = ld16_nt(dv + off);
        yh = ld16_nt(dv + off + HALF);
      }
      const size_t o = (size_t)row * D + e0;
      if (dst_j[bb[p]] == src_pos[bb[p]]) {  // R(0) is the identity: the stored bits as they are
        st16(ko + o, xl);
        st16(ko + o + HALF, xh);
      } else {
        float x[VEC], y[VEC], ox[VEC], oy[VEC];
        Fmt<E>::unpack(xl, x);
        Fmt<E>::unpack(xh, y);
        const float2* cs = cs_j + (size_t)bb[p] * HALF + e0;
#pragma unroll
        for (int q = 0; q < VEC; ++q) {
          const float2 c = cs[q];
          ox[q] = x[q] * c.x - y[q] * c.y;
          oy[q] = y[q] * c.x + x[q] * c.y;
        }
        st16(ko + o, Fmt<E>::pack(ox));
        st16(ko + o + HALF, Fmt<E>::pack(oy));
      }
      st16(vo + o, yl);
      st16(vo + o + HALF, yh);
    }
  }
}

template <typename E, int D, bool PAGED>
hipError_t launch_t(const Dims& d, const TransferArgs& t, hipStream_t s) {
  constexpr int G = D / 2 / Fmt<E>::VEC;
  constexpr int RPP = kThreads / G;
  const int nb = d.T / kTile;
  const int nl = t.l1 - t.l0;
  int32_t* slot = static_cast<int32_t*>(t.ws);
  float2* tab = reinterpret_cast<float2*>(static_cast<unsigned char*>(t.ws) + transfer_tab_off(d, t.n_req, nl));
  hipLaunchKernelGGL(transfer_slot_kernel, dim3(t.n_req * nl), dim3(kThreads), 0, s, t.agents, t.diff_off,
                     t.diff_idx, d.N, d.L, t.l0, nl, nb, slot);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n = (size_t)t.n_req * d.B * (D / 2);
  const int blocks = (int)((n + kThreads - 1) / kThreads < 2048 ? (n + kThreads - 1) / kThreads : 2048);
  hipLaunchKernelGGL(transfer_tab_kernel, dim3(blocks), dim3(kThreads), 0, s, t.agents, t.src_pos, t.dst_pos,
                     d.N, t.n_req, d.B, D, d.theta, tab);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int rows = kTile * d.Hkv;
  // rows per workgroup: up to 8 per thread; more rows (fp32, 16 heads x
  // 128) go to further workgroups along z
  const int nz = (rows + 8 * RPP - 1) / (8 * RPP);
  const dim3 grid(nb, nl, nz);
#define TDX_TR(NP)                                                                                         \
  hipLaunchKernelGGL((transfer_kernel<E, D, NP, PAGED>), grid, dim3(kThreads), 0, s,                       \
                     static_cast<const E*>(t.mk), static_cast<const E*>(t.mv), slot,                       \
                     static_cast<const E*>(t.dk), static_cast<const E*>(t.dv), tab, t.blk_start, t.agents, \
                     t.src_pos, t.dst_pos, d.N, t.n_req, d.B, d.T, d.L, t.l0, nl, d.Hkv,                   \
                     static_cast<E*>(t.k_out), static_cast<E*>(t.v_out), t.out_pages)
  if (rows <= RPP) TDX_TR(1);
  else if (rows <= 2 * RPP) TDX_TR(2);
  else if (rows <= 4 * RPP) TDX_TR(4);
  else TDX_TR(8);
#undef TDX_TR
  return hipGetLastError();
}

}  // namespace

size_t transfer_tab_off(const Dims& d, int n_req, int nl) {
  const size_t slot_bytes = (size_t)n_req * nl * (d.T / kTile) * 4;
  return (slot_bytes + 255) & ~(size_t)255;
}

size_t transfer_ws_bytes(const Dims& d, int n_req, int nl) {
  return transfer_tab_off(d, n_req, nl) + (size_t)n_req * d.B * (d.D / 2) * 8;
}

namespace {
template <bool PAGED>
hipError_t transfer_t(const Dims& d, const TransferArgs& t, hipStream_t s) {
  if (d.dtype == TDX_BF16)
    return d.D == 128 ? launch_t<uint16_t, 128, PAGED>(d, t, s) : launch_t<uint16_t, 64, PAGED>(d, t, s);
  return d.D == 128 ? launch_t<float, 128, PAGED>(d, t, s) : launch_t<float, 64, PAGED>(d, t, s);
}
}  // namespace

hipError_t launch_transfer(const Dims& d, const TransferArgs& t, hipStream_t s) {
  return t.out_pages.pages != nullptr ? transfer_t<true>(d, t, s) : transfer_t<false>(d, t, s);
}

}  // namespace tdx

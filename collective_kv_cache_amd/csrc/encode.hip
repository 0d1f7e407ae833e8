// a4: Master-Mirror block-sparse diff encode.
//
// TokenDance notes, Figure 8 and §2b (blog §4.3): the least-deviation agent
// (the Master) keeps its full cache; every other agent (a Mirror) stores only
// the 16-token blocks that differ from the Master, as block-sparse
// (indices, values), one record per Mirror per layer.
//
// Kernels (all deterministic, no atomics on the data path):
//  flag_kernel    resident workgroups over the (block beta, layer l, chunk
//                 slice) items: per item the Master block's K and V are held
//                 in registers (16-byte chunks per lane) and every Mirror
//                 block is streamed once through a register pipeline that
//                 runs on across items, and compared bit for bit.  Optionally
//                 writes the dense Master copy from the same registers.
//  index_rows_kernel  rounds with one chunk slice and at most 256K row-blocks:
//                 one workgroup per CSR row (agent, layer) counts the flagged
//                 blocks of the earlier rows itself (popcount of the flag
//                 bytes), writes its row offset (and, last row, the end offset
//                 and nnz) and ranks its own row while writing its indices;
//                 it replaces the three kernels below.
//  rows_kernel    one workgroup per CSR row (agent, layer): OR of the slices'
//                 flags, count of flagged blocks and each block's rank inside
//                 its row.
//  offsets_kernel one workgroup: exclusive scan of the row counts -> row
//                 offsets (clamped to the capacity, so a record whose blocks
//                 overflow it still names only written entries) and the true
//                 total nnz.  Launched only for rounds of more than 4096
//                 rows; smaller rounds have index_kernel do it per row.
//  index_kernel   one workgroup per CSR row: the row offset (the sum of the
//                 earlier rows' counts, on rounds of at most 4096 rows), then
//                 the ascending block indices (and, paged, the Mirror's page)
//                 into their slots; entries at or past the capacity are
//                 dropped.
//  copy_kernel    slot-major: each workgroup copies the Mirror's K/V blocks of
//                 a few consecutive CSR entries.
#include "common.h"

namespace tdx {
namespace {

constexpr int kThreads = 256;
constexpr int kFlagThreads = 1024;
constexpr int kCopySlots = 2;       // diff entries per copy workgroup step
constexpr int kCopyMaxWg = 65536;  // copy grid (grid-stride beyond)
constexpr int kCopyUnroll = 8;
constexpr int kScanThreads = 1024;
constexpr int kMaxAgents = 1024;

// Persistent: workgroup g takes the items w = g, g + G, ... of the (block beta,
// layer l, chunk slice cs) grid, beta fastest.  Per item it streams N blocks:
// the Master's block first, then every Mirror's, through one PD-stage
// register pipeline that runs on across items (each thread holds KC 16-byte
// chunks of K and of V per stage).  The Master's chunks are kept aside and
// every Mirror chunk is compared with them bit for bit; a wave that sees a
// difference marks the Mirror in LDS (two mark buffers, by item parity), and
// after the item's last block one barrier publishes the marks as the item's
// flags.  The unrolled body has no branch around a load, so the wait before
// a block is used leaves the younger blocks' loads outstanding.
//
// PAGED: agent a's block beta of layer l is page pm[a][beta] of the K and V
// pools (ak, av), whose pages hold `chunks` 16-byte chunks each.
template <int KC, int PD, bool PAGED>
__global__ __launch_bounds__(kFlagThreads) void flag_kernel(
    const u32x4* __restrict__ ak, const u32x4* __restrict__ av,
    const int32_t* __restrict__ master_p, int N, int L, int nb, int chunks, int nslices,
    uint8_t* __restrict__ flags, u32x4* __restrict__ mk_out, u32x4* __restrict__ mv_out, PageMap pm) {
  __shared__ uint8_t mark[2][kMaxAgents];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int G = gridDim.x;
  const int nitems = nb * L * nslices;
  const int m = master_p[0];
  const size_t slice_flags = (size_t)N * L * nb;
  if (m < 0 || m >= N) {  // invalid Master: no reads; nnz is reported as -1
    for (int w = blockIdx.x; w < nitems; w += G) {
      const int beta = w % nb, l = (w / nb) % L, cs = w / (nb * L);
      for (int i = tid; i < N; i += kFlagThreads) flags[cs * slice_flags + ((size_t)i * L + l) * nb + beta] = 0;
    }
    return;
  }
  const int nw = (nitems - (int)blockIdx.x + G - 1) / G;  // this workgroup's items
  if (nw <= 0) return;
  for (int i = tid; i < 2 * kMaxAgents; i += kFlagThreads) (&mark[0][0])[i] = 0;
  __syncthreads();
  const size_t layer_chunks = (size_t)nb * chunks;
  const size_t agent_chunks = (size_t)L * layer_chunks;
  struct Blk {
    u32x4 k[KC], v[KC];
  };
  // Position in the block stream: block p = item p / N (w = blockIdx.x + G *
  // (p / N), beta = w % nb, l = (w / nb) % L, slice cs = w / (nb * L)), agent
  // slot j = p % N (slot 0 = the Master, slot j > 0 = Mirror j - 1 = agent
  // j - 1 + (j - 1 >= m)).  Advanced one block at a time: the divisions run
  // once per item, not per block.
  struct Cursor {
    int j, wi, beta, l, cs;
    size_t item;  // chunk offset of the item's block in a cache (layer l, block beta)
    __device__ void set_item(int w, int nb_, int L_, size_t lchunks, int chunks_) {
      beta = w % nb_;
      l = (w / nb_) % L_;
      cs = w / (nb_ * L_);
      item = (size_t)l * lchunks + (size_t)beta * chunks_;
    }
  };
  const int b0w = (int)blockIdx.x;
  Cursor lc{0, 0, 0, 0, 0, 0}, uc{0, 0, 0, 0, 0, 0};
  lc.set_item(b0w, nb, L, layer_chunks, chunks);
  uc = lc;
  const long long nblk = (long long)nw * N;
  long long lp = 0;  // blocks loaded
  auto advance = [&](Cursor& c) {
    if (++c.j == N) {
      c.j = 0;
      ++c.wi;
      c.set_item(b0w + c.wi * G, nb, L, layer_chunks, chunks);
    }
  };
  // the next block of the stream; past the end the last block is re-read
  // (its compare is not used)
  auto load = [&](Blk& B) {
    const int a = lc.j == 0 ? m : (lc.j - 1) + (lc.j - 1 >= m);
    const size_t base = PAGED ? ((size_t)lc.l * pm.n_pages + page_at(pm, a, lc.beta)) * chunks
                              : (size_t)a * agent_chunks + lc.item;
    const int c0 = lc.cs * KC * kFlagThreads;
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      const int c = min(c0 + tid + q * kFlagThreads, chunks - 1);
      B.k[q] = ld16_nt(ak + base + c);
      B.v[q] = ld16_nt(av + base + c);
    }
    if (++lp < nblk) advance(lc);
  };
  u32x4 mkr[KC], mvr[KC];
#pragma unroll
  for (int q = 0; q < KC; ++q) mkr[q] = mvr[q] = u32x4{0, 0, 0, 0};
  auto use = [&](const Blk& B) {
    const int j = uc.j;
    if (j == 0) {  // the Master's block (uniform)
#pragma unroll
      for (int q = 0; q < KC; ++q) {
        mkr[q] = B.k[q];
        mvr[q] = B.v[q];
      }
      if (mk_out != nullptr) {
#pragma unroll
        for (int q = 0; q < KC; ++q) {
          const int c = uc.cs * KC * kFlagThreads + tid + q * kFlagThreads;
          if (c < chunks) {
            __builtin_nontemporal_store(B.k[q], mk_out + uc.item + c);
            __builtin_nontemporal_store(B.v[q], mv_out + uc.item + c);
          }
        }
      }
    } else {
      uint32_t acc = 0;
#pragma unroll
      for (int q = 0; q < KC; ++q) {
        const u32x4 xk = B.k[q] ^ mkr[q];
        const u32x4 xv = B.v[q] ^ mvr[q];
        acc |= xk[0] | xk[1] | xk[2] | xk[3] | xv[0] | xv[1] | xv[2] | xv[3];
      }
      const int a = (j - 1) + (j - 1 >= m);
      if (__builtin_amdgcn_ballot_w64(acc != 0) != 0 && lane == 0) mark[uc.wi & 1][a] = 1;
    }
    if (j == N - 1) {  // the item's last block (uniform): publish its flags
      __syncthreads();
      for (int i = tid; i < N; i += kFlagThreads) {
        flags[uc.cs * slice_flags + ((size_t)i * L + uc.l) * nb + uc.beta] = mark[uc.wi & 1][i];
        mark[uc.wi & 1][i] = 0;  // item wi + 2 reuses the buffer after item wi + 1's barrier
      }
    }
    advance(uc);
  };
  // PD-stage register pipeline: the first PD-1 blocks are loaded ahead, then
  // each step loads one block and uses the oldest.  The unrolled body has no
  // branch around a load, so the wait before a block is used leaves the
  // younger blocks' loads outstanding.
  Blk S[PD] = {};
#pragma unroll
  for (int k = 0; k < PD - 1; ++k) load(S[k]);
  for (long long p0 = 0; p0 < nblk; p0 += PD) {
#pragma unroll
    for (int k = 0; k < PD; ++k) {
      if (p0 + k >= nblk) break;  // uniform; the stream's last step
      load(S[(k + PD - 1) % PD]);
      use(S[k]);
    }
  }
}

__device__ __forceinline__ int lanemask_count(uint64_t m, int lane) {
  return __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
}

// In-row exclusive ranks of the flagged blocks and the row count.  With
// several chunk slices the block flag is the OR of the slices' flags; it is
// stored back into slice 0 for copy_kernel.
__global__ __launch_bounds__(kThreads) void rows_kernel(uint8_t* __restrict__ flags, int nb,
                                                        int nslices, size_t slice_stride,
                                                        int32_t* __restrict__ rank,
                                                        int32_t* __restrict__ count) {
  constexpr int W = kThreads / kWave;
  __shared__ int wcnt[W];
  const size_t r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int carry = 0;
  for (int base = 0; base < nb; base += kThreads) {
    const int beta = base + tid;
    bool f = false;
    if (beta < nb) {
      for (int c = 0; c < nslices; ++c) f |= flags[c * slice_stride + r * nb + beta] != 0;
      if (nslices > 1) flags[r * nb + beta] = f ? 1 : 0;
    }
    const uint64_t m = __ballot(f);
    if (lane == 0) wcnt[wave] = __popcll(m);
    __syncthreads();
    int pre = carry, all = carry;
    for (int w = 0; w < W; ++w) {
      if (w < wave) pre += wcnt[w];
      all += wcnt[w];
    }
    if (beta < nb) rank[r * nb + beta] = pre + lanemask_count(m, lane);
    carry = all;
    __syncthreads();
  }
  if (tid == 0) count[r] = carry;
}

// Row offsets are written as min(true offset, cap): entries past the
// capacity are never written (index_kernel, copy_kernel), and with clamped
// offsets no row of the record reaches one of them, so every consumer that
// reads entries [off[r], off[r+1]) stays inside the written entries.  nnz
// keeps the true total, which tells the caller that the record is truncated.
__global__ __launch_bounds__(kScanThreads) void offsets_kernel(const int32_t* __restrict__ count,
                                                               int rows, int64_t cap,
                                                               int32_t* __restrict__ off,
                                                               int64_t* __restrict__ nnz,
                                                               const int32_t* __restrict__ master_p,
                                                               int N) {
  constexpr int W = kScanThreads / kWave;
  __shared__ long long wsum[W];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  long long carry = 0;
  for (int base = 0; base < rows; base += kScanThreads) {
    const int r = base + tid;
    long long v = r < rows ? count[r] : 0;
    // inclusive wave scan
    long long x = v;
    for (int o = 1; o < kWave; o <<= 1) {
      const long long y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    if (lane == kWave - 1) wsum[wave] = x;
    __syncthreads();
    long long pre = carry, all = carry;
    for (int w = 0; w < W; ++w) {
      if (w < wave) pre += wsum[w];
      all += wsum[w];
    }
    if (r < rows) off[r] = (int32_t)min(pre + x - v, (long long)cap);
    carry = all;
    __syncthreads();
  }
  if (tid == 0) {
    off[rows] = (int32_t)min(carry, (long long)cap);
    const int m = master_p[0];
    nnz[0] = (m < 0 || m >= N) ? -1 : carry;
  }
}

// The diff values are written with non-temporal stores: the restore that
// reads them next then finds no dirty lines of them in the last-level cache
// to write back first (with plain stores a diff record that fits in the
// cache is left there dirty in full).
#ifndef TDX_CP_NT_STORES
#define TDX_CP_NT_STORES 1
#endif
__device__ __forceinline__ void cp_store(const u32x4& v, u32x4* p) {
#if TDX_CP_NT_STORES
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// One workgroup per CSR row (agent, layer): the ascending block indices of the
// row's flagged blocks into their slots (entries at or past the capacity are
// dropped).  PAGED: also each entry's page, the Mirror's page pm[a][beta].
// With OWN_OFF (rounds of at most kOwnOffRows rows) the workgroup first sums
// the earlier rows' counts itself and writes its row offset as
// offsets_kernel would (the last row also the end offset and nnz), so no
// separate scan launch is needed; larger rounds read the offsets that
// offsets_kernel wrote.
constexpr int kOwnOffRows = 4096;
template <bool PAGED, bool OWN_OFF>
__global__ __launch_bounds__(kThreads) void index_kernel(const uint8_t* __restrict__ flags,
                                                         const int32_t* __restrict__ rank,
                                                         const int32_t* __restrict__ count, int rows,
                                                         int32_t* __restrict__ off, int64_t* __restrict__ nnz,
                                                         const int32_t* __restrict__ master_p, int N, int nb,
                                                         int64_t cap, int32_t* __restrict__ diff_idx, PageMap pm,
                                                         int L, int32_t* __restrict__ diff_page) {
  const size_t r = blockIdx.x;
  int64_t row_off;
  if constexpr (OWN_OFF) {
    constexpr int W = kThreads / kWave;
    __shared__ long long wsum[W];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    long long x = 0;
    for (size_t j = tid; j < r; j += kThreads) x += count[j];
    for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
    if (lane == 0) wsum[wave] = x;
    __syncthreads();
    long long pre = 0;
    for (int w = 0; w < W; ++w) pre += wsum[w];
    row_off = min(pre, (long long)cap);
    if (tid == 0) {
      off[r] = (int32_t)row_off;
      if ((int)r == rows - 1) {
        const long long total = pre + count[r];
        off[rows] = (int32_t)min(total, (long long)cap);
        const int m = master_p[0];
        nnz[0] = (m < 0 || m >= N) ? -1 : total;
      }
    }
  } else {
    row_off = off[r];
  }
  for (int beta = threadIdx.x; beta < nb; beta += kThreads) {
    if (!flags[r * nb + beta]) continue;
    const int64_t slot = row_off + rank[r * nb + beta];
    if (slot >= cap) continue;
    diff_idx[slot] = beta;
    if constexpr (PAGED) diff_page[slot] = (int32_t)page_at(pm, (long long)(r / L), beta);
  }
}

// index_kernel without the rows_kernel launch in front of it, for rounds
// whose flags have one chunk slice and whose flag array is small
// (rows * nb <= kRowsInIndexFlags): workgroup r sums the flags of the rows
// before it itself (the flags are 0/1 bytes, so a popcount of each 16-byte
// chunk counts them), writes its row offset (the last row also the end
// offset and nnz) and then ranks its own row's flags in ascending block order
// while it writes their indices.  Same outputs as rows_kernel + index_kernel.
constexpr long long kRowsInIndexFlags = 256 * 1024;
template <bool PAGED>
__global__ __launch_bounds__(kThreads) void index_rows_kernel(const uint8_t* __restrict__ flags, int rows,
                                                              int32_t* __restrict__ off, int64_t* __restrict__ nnz,
                                                              const int32_t* __restrict__ master_p, int N, int nb,
                                                              int64_t cap, int32_t* __restrict__ diff_idx,
                                                              PageMap pm, int L, int32_t* __restrict__ diff_page) {
  constexpr int W = kThreads / kWave;
  __shared__ int wsum[W];
  __shared__ int wcnt[W];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  // flagged blocks of rows [0, r): bytes [0, r * nb) of the flag array
  const long long nbytes = (long long)r * nb;
  const long long n16 = nbytes / 16;
  const u32x4* f4 = reinterpret_cast<const u32x4*>(flags);
  int x = 0;
  for (long long j = tid; j < n16; j += kThreads) {
    const u32x4 v = f4[j];
    x += __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
  }
  if (n16 * 16 + tid < nbytes) x += flags[n16 * 16 + tid] != 0;  // < 16 tail bytes
  for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  if (lane == 0) wsum[wave] = x;
  __syncthreads();
  long long pre = 0;
  for (int w = 0; w < W; ++w) pre += wsum[w];
  const int64_t row_off = min(pre, (long long)cap);
  // own row: in-row exclusive ranks by ballots, indices into their slots
  const uint8_t* fr = flags + nbytes;
  int carry = 0;
  for (int base = 0; base < nb; base += kThreads) {
    const int beta = base + tid;
    const bool f = beta < nb && fr[beta] != 0;
    const uint64_t m = __ballot(f);
    if (lane == 0) wcnt[wave] = __popcll(m);
    __syncthreads();
    int rk = carry, all = carry;
    for (int w = 0; w < W; ++w) {
      if (w < wave) rk += wcnt[w];
      all += wcnt[w];
    }
    if (f) {
      const int64_t slot = row_off + rk + lanemask_count(m, lane);
      if (slot < cap) {
        diff_idx[slot] = beta;
        if constexpr (PAGED) diff_page[slot] = (int32_t)page_at(pm, (long long)(r / L), beta);
      }
    }
    carry = all;
    __syncthreads();
  }
  if (tid == 0) {
    off[r] = (int32_t)row_off;
    if (r == rows - 1) {
      const long long total = pre + carry;
      off[rows] = (int32_t)min(total, (long long)cap);
      const int m = master_p[0];
      nnz[0] = (m < 0 || m >= N) ? -1 : total;
    }
  }
}

// Slot-major value copy: workgroup w copies CSR entries [w*S, w*S + S), then
// the groups of S a grid further on (of the min(nnz, cap) written entries),
// from the Mirrors' caches, kCopyUnroll chunks of K and of V per thread in
// flight.  An entry's row is found by walking the
// row offsets from a binary search at the workgroup's first entry; its block
// index comes from diff_idx (index_kernel).  PAGED: the source is the entry's
// page of the pools.
template <bool PAGED>
__global__ __launch_bounds__(kThreads) void copy_kernel(
    const u32x4* __restrict__ ak, const u32x4* __restrict__ av, const int32_t* __restrict__ off, int rows, int nb,
    int chunks, int64_t cap, const int32_t* __restrict__ diff_idx, const int32_t* __restrict__ diff_page,
    u32x4* __restrict__ dk, u32x4* __restrict__ dv, long long n_pages, int L) {
  const int tid = threadIdx.x;
  const int64_t total = min((int64_t)off[rows], cap);
  for (int64_t e0 = (int64_t)blockIdx.x * kCopySlots; e0 < total; e0 += (int64_t)gridDim.x * kCopySlots) {
  const int64_t e1 = min(e0 + kCopySlots, total);
  int lo = 0, hi = rows - 1;  // the row of e0: largest r with off[r] <= e0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= e0) lo = mid; else hi = mid - 1;
  }
  int r = lo;
  for (int64_t e = e0; e < e1; ++e) {
    while (off[r + 1] <= e) ++r;  // uniform
    const size_t src = PAGED ? ((size_t)(r % L) * (size_t)n_pages + (size_t)diff_page[e]) * chunks
                             : ((size_t)r * nb + (size_t)diff_idx[e]) * chunks;
    const size_t dst = (size_t)e * chunks;
    for (int c0 = tid; c0 < chunks; c0 += kThreads * kCopyUnroll) {
      u32x4 xk[kCopyUnroll], xv[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int c = min(c0 + u * kThreads, chunks - 1);
        xk[u] = ld16_nt(ak + src + c);
        xv[u] = ld16_nt(av + src + c);
      }
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int c = c0 + u * kThreads;
        if (c < chunks) {
          cp_store(xk[u], dk + dst + c);
          cp_store(xv[u], dv + dst + c);
        }
      }
    }
  }
  }
}

struct WsLayout {
  size_t flags, rank, count, total;
};

int block_chunks(const Dims& d) {  // 16-byte chunks per block per tensor
  return kBlock * d.Hkv * d.D * (d.dtype == TDX_BF16 ? 2 : 4) / 16;
}
int flag_kc(const Dims& d) { return block_chunks(d) <= kFlagThreads ? 1 : 2; }
int flag_slices(const Dims& d) {
  const int per = flag_kc(d) * kFlagThreads;
  return (block_chunks(d) + per - 1) / per;
}

WsLayout ws_layout(const Dims& d) {
  const size_t rows = (size_t)d.N * d.L;
  const size_t nb = (size_t)(d.T / kBlock);
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WsLayout w;
  w.flags = 0;
  w.rank = up(rows * nb * flag_slices(d));
  w.count = w.rank + up(rows * nb * 4);
  w.total = w.count + up(rows * 4);
  return w;
}

}  // namespace

size_t encode_ws_bytes(const Dims& d) { return ws_layout(d).total; }

namespace {
template <bool PAGED>
hipError_t encode_t(const Dims& d, const int32_t* master, const void* ak, const void* av, const PageMap& pm,
                    int64_t cap, int32_t* diff_off, int32_t* diff_idx, int32_t* diff_page, void* diff_k,
                    void* diff_v, int64_t* nnz, void* mk_out, void* mv_out, void* ws, hipStream_t s) {
  const int nb = d.T / kBlock;
  const int chunks = block_chunks(d);
  const int rows = d.N * d.L;
  const WsLayout w = ws_layout(d);
  uint8_t* flags = static_cast<uint8_t*>(ws) + w.flags;
  int32_t* rank = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + w.rank);
  int32_t* count = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + w.count);
  const u32x4* k4 = static_cast<const u32x4*>(ak);
  const u32x4* v4 = static_cast<const u32x4*>(av);
  u32x4* mk4 = static_cast<u32x4*>(mk_out);
  u32x4* mv4 = static_cast<u32x4*>(mv_out);
  {
    const int ns = flag_slices(d);
    const int nitems = nb * d.L * ns;
    hipError_t e;
    int dev = 0, ncu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    auto launch_flag = [&](auto kern) -> hipError_t {
      int per_cu = 0;
      hipError_t e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                                    kFlagThreads, 0);
      if (e2 != hipSuccess) return e2;
      int grid = ncu * (per_cu < 1 ? 1 : per_cu);  // resident workgroups
      if (grid > nitems) grid = nitems;
      if (grid < 1) grid = 1;
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kFlagThreads), 0, s, k4, v4, master, d.N, d.L, nb, chunks, ns,
                         flags, mk4, mv4, pm);
      return hipGetLastError();
    };
    e = flag_kc(d) == 1 ? launch_flag(flag_kernel<1, 8, PAGED>) : launch_flag(flag_kernel<2, 4, PAGED>);
    if (e != hipSuccess) return e;
    if (ns == 1 && (long long)rows * nb <= kRowsInIndexFlags) {
      hipLaunchKernelGGL((index_rows_kernel<PAGED>), dim3(rows), dim3(kThreads), 0, s, flags, rows, diff_off, nnz,
                         master, d.N, nb, cap, diff_idx, pm, d.L, diff_page);
    } else {
      hipLaunchKernelGGL(rows_kernel, dim3(rows), dim3(kThreads), 0, s, flags, nb, ns, (size_t)rows * nb, rank,
                         count);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipError_t e;
  if (flag_slices(d) == 1 && (long long)rows * nb <= kRowsInIndexFlags) {
    // index_rows_kernel has written the offsets, nnz and indices
  } else if (rows <= kOwnOffRows) {
    hipLaunchKernelGGL((index_kernel<PAGED, true>), dim3(rows), dim3(kThreads), 0, s, flags, rank, count, rows,
                       diff_off, nnz, master, d.N, nb, cap, diff_idx, pm, d.L, diff_page);
  } else {
    hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(kScanThreads), 0, s, count, rows, cap, diff_off, nnz,
                       master, d.N);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((index_kernel<PAGED, false>), dim3(rows), dim3(kThreads), 0, s, flags, rank, count, rows,
                       diff_off, nnz, master, d.N, nb, cap, diff_idx, pm, d.L, diff_page);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (diff_k == nullptr || cap <= 0) return hipSuccess;  // a paged record without value copies
  // every written entry has a slot below cap; surplus workgroups exit at once
  const int64_t cwg = min((cap + kCopySlots - 1) / kCopySlots, (int64_t)kCopyMaxWg);
  hipLaunchKernelGGL((copy_kernel<PAGED>), dim3((unsigned)cwg), dim3(kThreads), 0, s, k4, v4, diff_off, rows, nb,
                     chunks, cap, diff_idx, diff_page, static_cast<u32x4*>(diff_k), static_cast<u32x4*>(diff_v),
                     (long long)pm.n_pages, d.L);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_encode(const Dims& d, const int32_t* master, const void* ak, const void* av,
                         int64_t cap, int32_t* diff_off, int32_t* diff_idx, void* diff_k,
                         void* diff_v, int64_t* nnz, void* mk_out, void* mv_out, void* ws,
                         hipStream_t s) {
  const PageMap none{nullptr, 0, 1};
  return encode_t<false>(d, master, ak, av, none, cap, diff_off, diff_idx, nullptr, diff_k, diff_v, nnz, mk_out,
                         mv_out, ws, s);
}

hipError_t launch_encode_paged(const Dims& d, const int32_t* master, const void* k_pool, const void* v_pool,
                               const PageMap& pm, int64_t cap, int32_t* diff_off, int32_t* diff_idx,
                               int32_t* diff_page, void* diff_k, void* diff_v, int64_t* nnz, void* ws,
                               hipStream_t s) {
  return encode_t<true>(d, master, k_pool, v_pool, pm, cap, diff_off, diff_idx, diff_page, diff_k, diff_v, nnz,
                        nullptr, nullptr, ws, s);
}

}  // namespace tdx

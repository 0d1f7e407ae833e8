// a5 / a6: fused restore + decode attention, and the dense comparator.
//
// TokenDance notes §3d and §4 ("Fused Diff Restore"), blog §4.4: a Mirror is
// never rebuilt densely; its diff blocks are merged into the Master's tiles
// on chip, RoPE is recovered, and attention runs on the tile right away.  The
// dense comparator (restore every agent's cache, then attend) is what the
// fused path is measured against (notes §3d, §7b).
//
// Fused path = set-up kernels, two kernels writing split-K partial records,
// then one merge:
//
//  stream_plan_kernel  one launch, two roles: workgroup 0 lays the (agent,
//                      layer) rows' tiles end to end and cuts them into one
//                      equal piece per stream-kernel slot (a wave per KV
//                      head), a piece being one task per row it touches; the
//                      other workgroups fill the table
//                      cos/sin(Delta(i,b) * theta^(-2e/D)), computed in
//                      double and stored as fp32 pairs [N][B][D/2].
//  shared_kernel       first, one wave per (agent, layer) row: per diff entry,
//                      its shared block and that block's cos/sin row (a
//                      block straddling two shared blocks is marked, and its
//                      rows take their own rows); then one workgroup per
//                      (agent group, Master split, layer, KV head).  Each 16-token Master tile (= one diff
//                      block) arrives ONCE in an LDS ring through direct
//                      global-to-LDS loads and serves the query rows of every
//                      agent of the group, the agents' GQA query groups
//                      stacked into one 16-row MFMA tile per wave.  RoPE is
//                      recovered on the query side, q . R(Delta) k =
//                      (R(-Delta) q) . k, so one canonical Master tile serves
//                      all agents.  Rows of an agent whose diff record holds
//                      the tile are masked here.
//  stream_kernel       persistent waves, each running its slot's tasks: the
//                      agent's private history followed by its own diff
//                      blocks (K/V straight from the diff record, the keys
//                      rotated by their block's Delta in registers), through
//                      one register pipeline that runs across tasks; K and V
//                      go through wave-private LDS into the MFMA operands.
//  merge_kernel        combines the records of every (agent, layer, query
//                      head).
//
// Per tile: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (K rows in the A
// operand, query rows in B, so each lane ends up holding 4 logits of ONE
// query row), online softmax with rows in lanes, O^T += V^T P^T with
// v_mfma_f32_16x16x16_bf16.  The dense comparator is restore_dense_kernel
// (every agent's cache materialised) followed by stream_kernel reading the
// materialised caches instead of diff records.
// These kernels serve bf16 caches: the operands are the stored bf16 values
// (and bf16 softmax weights), softmax, accumulation and the merge run in
// fp32.  fp32 caches take the fp32 vector-unit kernels of attn_f32.hip,
// which round nothing to bf16.
#include <algorithm>
#include <utility>

#include "common.h"

namespace tdx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTile = 16;
#ifndef TDX_ST_TW
#define TDX_ST_TW 48
#endif
#ifndef TDX_ST_PD
#define TDX_ST_PD 3
#endif
constexpr int kTilesPerSplit = TDX_ST_TW;  // stream kernel: tiles per task (one partial record)
constexpr int kShThreads = 256;     // shared_kernel: 4 waves, one 16-row tile each
constexpr int kShWaves = kShThreads / kWave;
constexpr int kRowsPerGroup = 16 * kShWaves;
constexpr int kMaxSharedTiles = 256;
constexpr float kLog2e = 1.4426950408889634f;


// ---- bf16 operand helpers ---------------------------------------------------

// 8 consecutive bf16 elements -> 8 floats
__device__ __forceinline__ void load8(const uint16_t* p, float* x) { Fmt<uint16_t>::unpack(ld16(p), x); }

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ __forceinline__ f32x4 mfma32(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const i16x4& a, const i16x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Order this wave's LDS writes before its later LDS reads of other lanes'
// data.  A wave's LDS operations execute in order, so only compiler ordering
// is needed; the fence is restricted to LDS so that outstanding global loads
// (the next tile's prefetch) are not waited for.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}


// Largest b in [0, B) with blk[b] <= t (the block holding token t; skips
// empty blocks).  blk is an LDS copy of blk_start.
__device__ __forceinline__ int block_of(const int32_t* blk, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (blk[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---- RoPE table: tab[(i*B + b)*HALF + e] = (cos, sin)(Delta(i,b) * theta^(-2e/D))

// entries x0, x0 + stride, ... of the table
__device__ void rope_table_fill(const int32_t* __restrict__ src_pos, const int32_t* __restrict__ dst_pos,
                                int N, int B, int D, double theta, float2* __restrict__ tab, size_t x0,
                                size_t stride) {
  const int half = D / 2;
  const size_t n = (size_t)N * B * half;
  for (size_t x = x0; x < n; x += stride) {
    const int e = (int)(x % half);
    const size_t ib = x / half;
    const int b = (int)(ib % B);
    const double delta = (double)(dst_pos[ib] - src_pos[b]);
    double sn, cs;
    sincos(delta * rope_inv_freq(theta, e, D), &sn, &cs);
    tab[x] = make_float2((float)cs, (float)sn);
  }
}

// ---- shared state ----------------------------------------------------------------

struct AttnArgs {
  const void* q;             // [N][L][Hq][D]
  const int32_t* priv_off;   // [N+1]
  const void* pk;            // [L][Ptot][Hkv][D]
  const void* pv;
  const void* sk;            // fused: Master [L][T][Hkv][D]; dense: [N][L][T][Hkv][D]
  const int32_t* msel;       // fused: Master at sk/sv + (*msel) * mstride (null: + 0)
  long long mstride;
  const void* sv;
  const int32_t* diff_off;   // fused: [N*L+1]
  const int32_t* diff_idx;
  const void* dk;            // [nnz][16][Hkv][D]
  const void* dv;
  const int32_t* blk_start;  // [B+1]
  const float2* tab;         // fused: [N][B][D/2] cos/sin of each shift
  const int32_t* src_pos;    // fused: [B] and [N][B], the shifts the table is filled from
  const int32_t* dst_pos;
  double theta;
  const uint16_t* qplain;    // [N][L][Hq][D] bf16 queries (the input q)
  float* part;               // [N][L][Hq][S][D+4]: m, l, -, -, O[D]
  unsigned char* ws_base;    // the workspace (task list, per-diff-entry cos/sin rows)
  int N, L, T, B, Hkv, Hq, D;
  long long dcap;            // fused: diff entries covered by the per-entry cos/sin rows
  int SP;                    // stream-kernel record slots
  int SG;                    // shared-kernel record slots (after SP)
  int S;                     // SP + SG
  int AGS, NAG, TPG;         // shared kernel: agents per group, groups, tiles per split
  int n_sh_wg;               // shared kernel: real workgroups (grid is padded to 8)
  int n_dt_wg;               // fused: workgroups in front of the shared kernel's that prepare the
                             // per-diff-entry rows (a multiple of 8)
  float2* dcs;               // fused: [dcap][D/2] per-diff-entry cos/sin rows (written by those)
  int2* dinfo;               // fused: [dcap] per-diff-entry (beta, shared block)
  float scale_log2;
  // paged (fused): sk/sv, dk/dv are the agents' K/V pools and pk/pv the
  // private pools; the Master's pages are row *msel of mpm, the diff entries'
  // pages dpm[0][e], agent i's private pages row i of ppm
  PageMap mpm, dpm, ppm;
  int pmax;  // an agent's private tokens are capped at pmax (= max_priv;
             // paged: a page-table row holds ceil(pmax/16) pages)
};

template <int D>
struct RowState {
  static constexpr int DT = D / 16;
  f32x4 o[DT];  // O^T tile dt: dims dt*16 + 4*q4 + j of row lane%16
  float m;      // running max (log2 domain), uniform over the row's 4 lanes
  float l;      // lane-partial running sum
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }
};

// LDS transpose read (ds_read_b64_tr_b16, gfx950).  Every lane supplies the
// address of 4 consecutive 16-bit elements; within each 16-lane group G, lane
// 16G + i receives element i%4 of the rows addressed by lanes 16G + 4j + i/4,
// j = 0..3.  If lane s addresses row 4*(s/16) + (s%16)/4 at column c0 + 4*(s%4),
// lane l gets [row 4*(l/16) + j][column c0 + l%16] for j = 0..3: the B
// operand layout of v_mfma_f32_16x16x16_bf16 with tokens as the reduction index.
__device__ __forceinline__ i16x4 ld_tr16(const void* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Maximum over the four lanes that hold one query row (lanes l, l ^ 16,
// l ^ 32, l ^ 48): two row swaps on the VALU (v_permlane16_swap,
// v_permlane32_swap), each followed by a max of the two halves.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Maxima of logits, which are finite or -inf and never NaN, as single
// v_max_f32 / v_max3_f32 instructions: fmaxf would first quiet possible
// signalling NaNs in each operand with an extra v_max of the value with
// itself.  The operands are VALU or permlane results, never MFMA results.
__device__ __forceinline__ float max_nn(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_nn(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float row_max4(float x) {
  u32x2 r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The running reference m of a row may lag its true maximum by up to
// kRescaleLag (log2 units): weights exp2(z - m) then stay below
// 2^kRescaleLag, and O and l are rescaled only when some row of the wave
// passes its reference by more than that.  O / l is the same quotient
// whichever reference is used, and the records carry their reference.
constexpr float kRescaleLag = 8.0f;

// Online softmax + PV for one tile.  z: the 4 logits (log2 domain) of the
// lane's row at tokens 4*q4 .. 4*q4+3 (-inf = masked).  While a row has no
// valid key its reference is -inf and 0 is used in its place, so every
// weight is exp2(-inf) = 0 and nothing turns into NaN; the path stays
// wave-uniform around the MFMAs.
template <int D>
__device__ __forceinline__ void softmax_pv(RowState<D>& st, const float z[4], const i16x4* va) {
  constexpr int DT = D / 16;
  const float tmax = row_max4(max_nn(max3_nn(z[0], z[1], z[2]), z[3]));
  if (__builtin_amdgcn_ballot_w64(tmax > st.m + kRescaleLag) != 0) {
    const float mnew = fmaxf(st.m, tmax);
    const float alpha = st.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st.m - mnew);
    st.m = mnew;
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.o[dt] *= alpha;
  }
  const float mref = st.m == -INFINITY ? 0.0f : st.m;
  // weights in (0, 2^kRescaleLag]: v_exp_f32, then one v_cvt_pk_bf16_f32
  // (round to nearest even) per pair; the sum uses the same rounded weights
  const uint32_t w01 = pack_bf16(__builtin_amdgcn_exp2f(z[0] - mref), __builtin_amdgcn_exp2f(z[1] - mref));
  const uint32_t w23 = pack_bf16(__builtin_amdgcn_exp2f(z[2] - mref), __builtin_amdgcn_exp2f(z[3] - mref));
  const float psum = (__uint_as_float(w01 << 16) + __uint_as_float(w01 & 0xffff0000u)) +
                     (__uint_as_float(w23 << 16) + __uint_as_float(w23 & 0xffff0000u));
  i16x4 pb;
  pb[0] = (short)(w01 & 0xffffu);
  pb[1] = (short)(w01 >> 16);
  pb[2] = (short)(w23 & 0xffffu);
  pb[3] = (short)(w23 >> 16);
  st.l += psum;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) st.o[dt] = mfma16(va[dt], pb, st.o[dt]);
}

// Write a row's partial record (m, l, O unnormalised).
template <int D>
__device__ __forceinline__ void write_record(float* rec, const RowState<D>& st, float lsum, int q4,
                                             int c16) {
  constexpr int DT = D / 16;
  if (q4 == 0) {
    rec[0] = st.m;
    rec[1] = lsum;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<f32x4*>(rec + 4 + dt * 16 + 4 * q4) = st.o[dt];
}

// ---- shared_kernel: Master tiles staged once, all agents' query rows ------------
//
// One workgroup per (agent group, Master split, layer, KV head).  The split's
// 16-token Master tiles arrive in a ring of NB LDS slots through direct
// global-to-LDS loads (global_load_lds_dwordx4): each wave's load instruction
// moves 1 KB of a tile, RPI whole rows (4 rows of 128 dims or 8 of 64),
// straight into the slot, so NB-2 tiles stay in flight per workgroup without
// holding any in registers.  Within its 1 KB, the 16-byte chunks of those
// rows are placed in the order the MFMA operands are read back (ShTile), so
// that a lane's K chunks of successive 32-dim steps, and its V elements of
// successive 16-dim slices, sit at fixed distances from its first one: the
// operand reads take one base address per tile and immediate offsets, and
// 16 consecutive lanes of a read touch 16 distinct 16-byte (K) or 8-byte (V)
// units of one 256-byte or 128-byte span.
//
// Step n (tile n of the split): wait until this wave has at most the loads
// of tiles n+1 .. n+NB-2 outstanding, barrier (tile n is in LDS and every
// wave is done with tile n-1), issue the loads of tile n+NB-1 into tile
// n-1's slot, then use tile n.  Loads past the split's last tile re-read it
// into the freed slot, so every step issues the same number of loads and
// one wait count serves all steps.
//
// The wave's 16 query rows (agents stacked into one MFMA tile) are rotated
// once per shared block, R(-Delta(i,b)) q, which is RoPE recovery moved to
// the query side (q . R(Delta) k = (R(-Delta) q) . k), so the Master's
// canonical key rows are used as stored.  A tile that straddles shared
// blocks is used once for each, with the other blocks' rows masked; rows of
// an agent whose diff record holds the tile are masked here (the stream
// kernel attends that agent's own rows).

#ifndef TDX_SH_NB
#define TDX_SH_NB 6
#endif
#ifndef TDX_SH_TARGET_WG
#define TDX_SH_TARGET_WG 1024
#endif

typedef __attribute__((address_space(3))) void lds_void_t;

// One Master tile slot: [K rows][V rows], 16 rows of RB bytes each.  Load
// instruction g of a tensor fills bytes [1024 g, 1024 g + 1024) of the
// tensor's half with rows RPI*g + i, i < RPI.  There, 16-byte chunk c of row
// RPI*g + i is at 16-byte unit
//   K: (c / 4) * 4*RPI + i + RPI * ((c % 4) ^ g)
//   V: ((c / 2) ^ VX(g)) * 2*RPI + 2*i + (c % 2),  VX(g) = g % 2 for 128 dims, else 0
// so the K chunk 4k + q of a row is k * KSTEP bytes past chunk q, and the V
// chunks of 16-dim slice dt are dt * VSTEP bytes past those of slice 0 for
// even dt, and past slice 1's minus VSTEP for odd dt.  VX staggers the
// 128-dim slices of consecutive row groups by 128 bytes: the lanes of one
// transposed read that address rows 4 apart then hit different banks
// (measured: half the LDS bank-conflict cycles of the unstaggered layout).
template <int D>
struct ShTile {
  static constexpr int RB = D * 2;                         // bytes of one bf16 row of a head
  static constexpr int CPR = RB / 16;                      // 16-byte chunks per row
  static constexpr int BYTES = 2 * kTile * RB;             // K and V
  static constexpr int RPI = 1024 / RB;                    // rows per wave load instruction
  static constexpr int IPT = kTile * RB / 1024;            // load instructions per tensor
  static constexpr int LPT = BYTES / (kShThreads * 16);    // loads per thread per tile
  static constexpr int KSTEP = 4 * RPI * 16;               // bytes between a lane's K chunks of consecutive 32-dim steps
  static constexpr int VSTEP = 2 * RPI * 16;               // bytes between a lane's V reads of consecutive 16-dim slices
  static_assert(LPT * kShWaves == 2 * IPT, "every wave issues the same loads");
  static_assert(CPR % 4 == 0 && IPT <= 4, "K chunk groups, XOR of the instruction index into 2 bits");
  // byte offset of K chunk c of tile row r / of V chunk c of tile row r within the tensor's half
  __device__ static constexpr int kbyte(int r, int c) {
    return ((r / RPI) * 64 + (c / 4) * 4 * RPI + r % RPI + RPI * ((c % 4) ^ (r / RPI))) * 16;
  }
  __device__ static constexpr int vx(int g) { return D == 128 ? g % 2 : 0; }
  __device__ static constexpr int vbyte(int r, int c) {
    return ((r / RPI) * 64 + ((c / 2) ^ vx(r / RPI)) * 2 * RPI + 2 * (r % RPI) + c % 2) * 16;
  }
};

// ds_read_b64_tr_b16 (as ld_tr16) and ds_read_b128 issued as inline asm, at
// address p + OFF (OFF in the instruction's offset field): the compiler
// cannot tell a ring slot being read from the slot the pending global-to-LDS
// loads write, and would otherwise wait for every one of them before each
// read.  The caller waits for the results with lds_wait / lds_wait_k.
template <int OFF>
__device__ __forceinline__ i16x4 ld_tr16_nowait(uint32_t p) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  i16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(p), "n"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x4 ld_b128_nowait(uint32_t p) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(p), "n"(OFF) : "memory");
  return r;
}
// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Wait until at most N of this wave's LDS reads are outstanding (LDS reads
// complete in order); the operands tie the K operand read before them.
template <int N, int KD>
__device__ __forceinline__ void lds_wait_k(u32x4 (&k)[KD]) {
  static_assert(KD == 2 || KD == 4, "K chunks");
  if constexpr (KD == 4)
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]) : "n"(N));
  else
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(k[0]), "+v"(k[1]) : "n"(N));
}
// Wait for this wave's LDS reads; the operands tie the values read by
// ld_tr16_nowait to this point, so no use of them is scheduled before it.
template <int N>
__device__ __forceinline__ void lds_wait(i16x4 (&v)[N]) {
  static_assert(N == 4 || N == 8, "dim tiles");
  if constexpr (N == 8)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}

// s_waitcnt immediate (gfx9 layout): vmcnt <= V, lgkmcnt 0, expcnt not waited
template <int V>
struct VmWait {
  static_assert(V >= 0 && V < 64, "vmcnt range");
  static constexpr int imm = (V & 15) | (7 << 4) | ((V >> 4) << 14);
};

#ifndef TDX_SH_WPE
#define TDX_SH_WPE 3
#endif

// Per diff entry e of row r = i * L + l: dinfo[e] = (beta, b) with b the
// shared block holding the entry's first token (~b when the 16 tokens span
// more than one block), and dcs[e][0 .. D/2) = the (cos, sin) row of
// Delta(i, b) from the round's table.  One wave per row: lane j searches the
// block starts for entries j, j + 64, ... of the row (all lanes at once),
// then the wave copies the entries' rows, eight independent reads in flight
// per lane.  Entries at or past dcap are left out.
__device__ void diff_tab_row(const AttnArgs& a, int r, int lane) {
  const int half = a.D / 2;
  const int nb = a.T / kTile;
  const int i = r / a.L;
  const int e0 = a.diff_off[r];
  if (e0 < 0) return;  // uniform
  const long long n = std::min<long long>(std::min(std::max(a.diff_off[r + 1] - e0, 0), nb), a.dcap - e0);
  for (int c = 0; c < n; c += kWave) {
    const int m = (int)std::min<long long>(kWave, n - c);  // entries of this chunk
    int b = 0;
    if (lane < m) {
      const int e = e0 + c + lane;
      const int t0 = a.diff_idx[e] * kTile;
      // b = the largest block with blk_start[b] <= t0 (empty blocks skipped)
      int lo = 0, hi = a.B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.blk_start[mid] <= t0) lo = mid; else hi = mid - 1;
      }
      b = lo;
      const bool straddle = a.blk_start[b + 1] < t0 + kTile;
      a.dinfo[e] = make_int2(t0 / kTile, straddle ? ~b : b);
    }
    // the m rows of half (cos, sin) pairs, element f = j * half + x
    const int tot = m * half;
    for (int f0 = 0; f0 < tot; f0 += 8 * kWave) {
      float2 v[8];
      int fj[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int f = std::min(f0 + u * kWave + lane, tot - 1);
        const int j = f / half;
        const int bj = __shfl(b, j, kWave);
        v[u] = a.tab[((size_t)i * a.B + bj) * half + f % half];
        fj[u] = f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (f0 + u * kWave + lane < tot) a.dcs[(size_t)(e0 + c) * half + fj[u]] = v[u];
    }
  }
}
template <typename E, int D, int NB, bool PAGED>
__global__ __launch_bounds__(kShThreads) __attribute__((amdgpu_waves_per_eu(TDX_SH_WPE))) void shared_kernel(AttnArgs a) {
  using Tl = ShTile<D>;
  constexpr int KD = D / 32;
  constexpr int DT = D / 16;
  constexpr int HALF = D / 2;
  constexpr int RB = Tl::RB;
  static_assert(sizeof(E) == 2, "bf16 caches (fp32 ones take the fp32 kernel)");
  static_assert(NB >= 3, "ring slots");
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* ring = smem;                                            // [NB][BYTES]
  int32_t* sblk = reinterpret_cast<int32_t*>(smem + NB * Tl::BYTES);     // [B+1]
  const int NW = (a.TPG + 31) / 32;                                      // flag words per agent
  uint32_t* dbits = reinterpret_cast<uint32_t*>(sblk + a.B + 1);         // [AGS][NW]

  // The first n_dt_wg workgroups (fused) prepare the per-diff-entry rows
  // that the stream kernel reads, one row per wave; they run before the
  // Master-tile workgroups and touch no LDS.
  if ((int)blockIdx.x < a.n_dt_wg) {
    const int r = (int)blockIdx.x * kShWaves + (int)threadIdx.x / kWave;
    if (r < a.N * a.L) diff_tab_row(a, r, (int)threadIdx.x % kWave);
    return;
  }
  // Hardware deals workgroups round-robin to the 8 XCDs; give each XCD a
  // contiguous run of logical ids so that the agent groups sharing a Master
  // tile run on the same XCD (one L2) at the same time.
  const int nwg = gridDim.x - a.n_dt_wg;  // a multiple of 8, as is n_dt_wg
  const int w = blockIdx.x - a.n_dt_wg;
  const int logical = (w % 8) * (nwg / 8) + w / 8;
  if (logical >= a.n_sh_wg) return;
  const int ag = logical % a.NAG;
  const int rest = logical / a.NAG;
  const int gs = rest % a.SG;
  const int lh = rest / a.SG;
  const int l = lh / a.Hkv, h = lh % a.Hkv;
  const int g = a.Hq / a.Hkv;
  const int a0 = ag * a.AGS;
  const int na = min(a.AGS, a.N - a0);
  const int nrows = na * g;
  const int nb = a.T / kTile;
  const int b0 = gs * a.TPG;
  const int b1 = min(b0 + a.TPG, nb);
  if (b0 >= b1) return;  // uniform
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform per wave
  const int q4 = lane / 16, c16 = lane % 16;

  for (int x = tid; x <= a.B; x += kShThreads) sblk[x] = a.blk_start[x];
  for (int x = tid; x < a.AGS * NW; x += kShThreads) dbits[x] = 0;
  __syncthreads();
  // flag (agent, tile) pairs whose block is in the agent's diff row, one bit
  // per tile: those rows take the tile from the agent's own record (stream
  // kernel)
  for (int al = wave; al < na; al += kShWaves) {
    const int r = (a0 + al) * a.L + l;
    const int e1 = a.diff_off[r + 1];
    for (int e = a.diff_off[r] + lane; e < e1; e += kWave) {
      const int beta = a.diff_idx[e];
      if (beta >= b0 && beta < b1) atomicOr(&dbits[al * NW + ((beta - b0) >> 5)], 1u << ((beta - b0) & 31));
    }
  }

  // this wave's 16 query rows (row = agent-major, then the GQA group); rows
  // past the group load row 0's data and are masked
  const bool has_rows = wave * 16 < nrows;  // wave-uniform
  const int row = wave * 16 + c16;
  const bool valid = row < nrows;
  const int agent = a0 + (valid ? row / g : 0);
  const int hq = h * g + (valid ? row % g : 0);
  RowState<D> st;
  st.init();

  const size_t rowHD = (size_t)a.Hkv * D;
  // contiguous: Master token t at mk + t * rowHD; paged: at page
  // mpm[mrow][t / 16], row t % 16 of layer l
  const size_t moff = PAGED ? 0 : master_offset(a.msel, a.mstride, a.N) + (size_t)l * a.T * rowHD;
  const E* mk = static_cast<const E*>(a.sk) + moff + (size_t)h * D;
  const E* mv = static_cast<const E*>(a.sv) + moff + (size_t)h * D;
  const int mrow = (PAGED && a.msel != nullptr) ? min(max(a.msel[0], 0), a.N - 1) : 0;
  const E* qrow = static_cast<const E*>(a.q) + (((size_t)agent * a.L + l) * a.Hq + hq) * D;
  const float2* tabrow = a.tab + (size_t)agent * a.B * HALF;

  // the lane's query elements 32k + 8*q4 .. +7 (element e < D/2 pairs with
  // e + D/2, which sits in chunk k + KD/2 of the same lane)
  u32x4 qraw[KD];
#pragma unroll
  for (int k = 0; k < KD; ++k) qraw[k] = ld16(qrow + 32 * k + 8 * q4);
  // rotated by -Delta(agent, b) in fp32 and rounded to bf16
  u32x4 qr[KD];
  auto rotate = [&](int b) {
    const float2* cs = tabrow + (size_t)b * HALF;
#pragma unroll
    for (int k = 0; k < KD / 2; ++k) {
      const int e0 = 32 * k + 8 * q4;
      float lo[8], hi[8], olo[8], ohi[8];
      Fmt<uint16_t>::unpack(qraw[k], lo);
      Fmt<uint16_t>::unpack(qraw[k + KD / 2], hi);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float2 c = cs[e0 + j];
        // R(-phi): (x, y) -> (x cos + y sin, y cos - x sin)
        olo[j] = lo[j] * c.x + hi[j] * c.y;
        ohi[j] = hi[j] * c.x - lo[j] * c.y;
      }
      qr[k] = Fmt<uint16_t>::pack(olo);
      qr[k + KD / 2] = Fmt<uint16_t>::pack(ohi);
    }
  };
  __syncthreads();
  int b = block_of(sblk, a.B, b0 * kTile);  // the block of the split's first token
  int bs = sblk[b], be = sblk[b + 1];       // its tokens [bs, be)
  if (has_rows) rotate(b);
  // everything above is complete before the ring's loads start, so that the
  // ring's wait counts see only its own loads
  __builtin_amdgcn_s_waitcnt(0);

  // This thread's share of a tile's loads: load p is instruction
  // wave * LPT + p (K instructions first, then V), and the lane's 16-byte
  // chunk is the one its position in the instruction's 1 KB holds (ShTile);
  // loff[p] is that chunk's byte offset from the tile's first row.
  uint32_t loff[Tl::LPT];
#pragma unroll
  for (int p = 0; p < Tl::LPT; ++p) {
    const int inst = wave * Tl::LPT + p;
    const int g = inst % Tl::IPT;
    int r, c;
    if (inst < Tl::IPT) {  // K: lane = (c / 4) * 4*RPI + i + RPI * ((c % 4) ^ g)
      r = g * Tl::RPI + lane % Tl::RPI;
      c = (lane / (4 * Tl::RPI)) * 4 + (((lane % (4 * Tl::RPI)) / Tl::RPI) ^ g);
    } else {  // V: lane = ((c / 2) ^ VX(g)) * 2*RPI + 2*i + c % 2
      r = g * Tl::RPI + (lane % (2 * Tl::RPI)) / 2;
      c = ((lane / (2 * Tl::RPI)) ^ Tl::vx(g)) * 2 + lane % 2;
    }
    loff[p] = (uint32_t)(((size_t)r * rowHD + (size_t)c * 8) * sizeof(E));
  }

  // this thread's loads of tile u into slot s (tiles past the split re-read its last)
  auto issue = [&](int u, int s) {
    const int tile = min(u, b1 - 1);
    const size_t trow = PAGED ? ((size_t)l * a.mpm.n_pages + page_at(a.mpm, mrow, tile)) * kTile
                              : (size_t)tile * kTile;
    const unsigned char* kb = reinterpret_cast<const unsigned char*>(mk + trow * rowHD);
    const unsigned char* vb = reinterpret_cast<const unsigned char*>(mv + trow * rowHD);
    unsigned char* slot = ring + s * Tl::BYTES;
#pragma unroll
    for (int p = 0; p < Tl::LPT; ++p) {
      const int inst = wave * Tl::LPT + p;
      const int tensor = inst / Tl::IPT, g = inst % Tl::IPT;
      __builtin_amdgcn_global_load_lds((void*)((tensor ? vb : kb) + loff[p]),
                                       (lds_void_t*)(slot + tensor * kTile * RB + g * 1024), 16, 0, 0);
    }
  };

  // use tokens [t_lo, t_hi) of tile u (in slot s) with the current rotation;
  // fw: the lane's agent's diff-flag word of the tile
  // The lane's operand addresses within a slot: K chunk q4 of row c16 (the
  // chunk of step k is k * KSTEP further); for the PV operand, va[dt][j] =
  // V[token 4*q4 + j][dim 16*dt + c16], the lane addresses row 4*q4 + c16/4
  // at dims 16*dt + 4*(c16%4): slice dt is dt * VSTEP past voff0 (even dt)
  // or voff1 (odd dt).
  const int vrow = 4 * q4 + (c16 >> 2), vc = (c16 & 3) >> 1;
  const uint32_t koff = Tl::kbyte(c16, q4);
  const uint32_t voff0 = kTile * RB + Tl::vbyte(vrow, vc) + (c16 & 1) * 8;
  const uint32_t voff1 = kTile * RB + Tl::vbyte(vrow, 2 + vc) - Tl::VSTEP + (c16 & 1) * 8;
  auto compute = [&](int u, int s, int t_lo, int t_hi, uint32_t fw) {
    const uint32_t slot = lds_addr(ring + s * Tl::BYTES);
    const uint32_t ka = slot + koff, va0 = slot + voff0, va1 = slot + voff1;
    // the K and V operands of the tile in one round trip: K first, then V,
    // whose latency the QK products cover
    u32x4 kop[KD];
    static_for<KD>([&](auto k) { kop[decltype(k)::value] = ld_b128_nowait<decltype(k)::value * Tl::KSTEP>(ka); });
    i16x4 va[DT];
    static_for<DT>([&](auto dt) {
      constexpr int j = decltype(dt)::value;
      va[j] = ld_tr16_nowait<j * Tl::VSTEP>(j % 2 ? va1 : va0);
    });
    lds_wait_k<DT>(kop);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KD; ++k) acc = mfma32(kop[k], qr[k], acc);
    const bool on = valid && !((fw >> ((u - b0) & 31)) & 1u);
    float z[4];
    if (t_lo == u * kTile && t_hi == u * kTile + kTile) {  // the whole tile (uniform)
      const float bias = on ? 0.0f : -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) z[j] = fmaf(acc[j], a.scale_log2, bias);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tt = u * kTile + 4 * q4 + j;
        z[j] = (on && tt >= t_lo && tt < t_hi) ? acc[j] * a.scale_log2 : -INFINITY;
      }
    }
    lds_wait(va);
    softmax_pv<D>(st, z, va);
  };

  const int nt = b1 - b0;
  uint32_t fw = 0;  // the lane's agent's diff flags of the current 32 tiles
#pragma unroll
  for (int s = 0; s < NB - 1; ++s) issue(b0 + s, s);
  for (int n = 0; n < nt; ++n) {
    // tile n is in LDS once this wave's loads of it are done (the NB-2
    // younger tiles may stay in flight) and every wave has passed the barrier
    __builtin_amdgcn_s_waitcnt(VmWait<Tl::LPT * (NB - 2)>::imm);
    asm volatile("s_barrier" ::: "memory");
    issue(b0 + n + NB - 1, (n + NB - 1) % NB);
    if (has_rows) {  // wave-uniform: no loads or barriers inside
      const int u = b0 + n, t0 = u * kTile, t1 = t0 + kTile;
      if (((u - b0) & 31) == 0) fw = dbits[(agent - a0) * NW + ((u - b0) >> 5)];
      if (be <= t0) {  // the block ended before this tile: the one holding t0
        do {
          ++b;
          be = sblk[b + 1];
        } while (be <= t0);
        bs = sblk[b];
        rotate(b);
      }
      for (;;) {
        compute(u, n % NB, max(bs, t0), min(be, t1), fw);
        if (be >= t1) break;
        bs = be;  // the tile goes on in the next non-empty block
        do {
          ++b;
          be = sblk[b + 1];
        } while (be <= bs);
        rotate(b);
      }
    }
  }
  // no load may still write this workgroup's LDS once it exits
  __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);

  if (has_rows) {
    float lsum = st.l;
    lsum += __shfl_xor(lsum, 16, kWave);
    lsum += __shfl_xor(lsum, 32, kWave);
    if (valid) {
      float* dst = a.part + ((((size_t)agent * a.L + l) * a.Hq + hq) * a.S + a.SP + gs) * (D + 4);
      write_record<D>(dst, st, lsum, q4, c16);
    }
  }
}

// ---- stream_kernel: every agent's own tiles, persistent waves -------------------
//
// The agent-private work is a stream of 16-token tiles per (agent, layer, KV
// head): the agent's private history, then its own diff blocks (fused) or its
// materialised shared cache (dense comparator).  stream_plan_kernel gives
// every slot of Hkv waves (one per KV head) an equal share of all rows' tiles
// as a run of tasks, each task one row's part of the share and one partial
// softmax record per query row.  The waves of stream_kernel stay resident and
// run their slot's tasks in turn;
// each wave runs ONE PD-stage register pipeline across task boundaries, so the
// first tiles and the query of the next task are in flight while the current
// task drains, and no workgroup start-up or combine step sits between tasks.
// A task runs for at least PD-1 steps (shorter ones are padded with masked
// steps), so the load side is never more than one task ahead.
//
// Per tile: K and V rows arrive in registers (16-byte non-temporal loads, a
// quarter-wave per 256-byte row), go to wave-private LDS tiles, and come back
// as MFMA operands: K as the A operand of S^T = K Q^T, V transposed
// (ds_read_b64_tr_b16).  The query operand is the agent's plain query.  A
// diff block holds canonical keys: its rows are rotated to the agent's
// offsets in registers by the shift of the shared block that holds them
// (K' = R(Delta(i,b)) K, rounded to bf16 like a materialised cache), with the
// block's cos/sin row prepared per diff entry (diff_tab_row) in the
// Master-tile launch.

template <typename E, int D, int MODE>
struct Stage {
  static constexpr int KD = D / 32;                                   // 16-byte bf16 chunks of K/Q per lane
  static constexpr int NV = kTile * D * (int)sizeof(E) / 16 / kWave;  // K or V loads per lane
  u32x4 k[NV];
  u32x4 v[NV];
  float2 cs;  // fused: this lane's (cos, sin) pair of the diff entry's cos/sin row
  int2 info;  // fused: (beta, shared block b) of the diff entry; ~b when the block straddles
};

// K tile of one wave in LDS, stored as loaded: [16 rows][CPR 16-byte chunks],
// chunk ch of row t at position ch ^ (t % CPR) (CPR a power of two, so the
// position stays inside the row), so that the row-wise writes and the column
// reads of the MFMA operand spread over the banks.
template <int CPR>
__device__ __forceinline__ int klds_off(int t, int ch) {
  static_assert((CPR & (CPR - 1)) == 0, "chunks per row: a power of two");
  return (t * CPR + (ch ^ (t % CPR))) * 16;
}

// V tile of one wave in LDS: [16 rows][D] bf16, 16-byte chunk ch of row t
// stored at chunk position ch ^ (t % (D/8)) so that row-wise writes and the
// transposed reads spread over the banks.
template <int D>
__device__ __forceinline__ int vlds_off(int t, int ch) {
  constexpr int C = D / 8;
  return (t * C + (ch ^ (t % C))) * 16;
}

// One task of the agent stream: tiles [t0, t0 + cnt) of row r = i * L + l,
// run once per KV head.
struct __attribute__((aligned(32))) StreamTask {
  int32_t r;     // (agent, layer) row
  int32_t s;     // split index: the partial-record slot
  int32_t t0;    // first tile (0 = the agent's first private tile)
  int32_t cnt;   // tiles, >= 1
  int32_t ntp;   // private tiles of the agent
  int32_t P;     // private tokens of the agent
  int32_t prow;  // first private row of the agent in layer l: l * Ptot + priv_off[i]
  int32_t e0;    // first diff entry of the row (fused)
};

constexpr int kPlanThreads = 1024;
#ifndef TDX_ST_NW
#define TDX_ST_NW 4
#endif
#ifndef TDX_ST_WPE
#define TDX_ST_WPE 2
#endif
constexpr int kStreamNW = TDX_ST_NW;  // waves per stream workgroup

// stream-kernel slots the plan can feed: a slot is one wave per KV head
// working on the same tasks
constexpr int kMaxSlots = 8192;

// Task plan (one workgroup).  The (agent, layer) rows' tiles are laid end to
// end in row order and cut into nslot equal pieces of
// P = max(kTilesPerSplit, ceil(total / nslot)) tiles, one per slot; where a
// piece crosses a row boundary it becomes one task per row.  Every wave then
// runs at most P tiles whatever the mix of row lengths, and a row has at most
// ceil(tiles / P) + 1 <= SP tasks (one partial record each).  Tasks are
// stored slot by slot in row order.  Writes ctl[0] = tasks, ctl[1] = nslot,
// ctl[2 + s] = first task of slot s (s <= nslot) and nrec[r] = tasks of row r.
// Workgroups 1 .. gridDim.x - 1 (fused path) fill the cos/sin table instead.
template <int MODE>
__global__ __launch_bounds__(kPlanThreads) void stream_plan_kernel(AttnArgs a, int nslot,
                                                                   StreamTask* __restrict__ tasks,
                                                                   int32_t* __restrict__ ctl,
                                                                   int32_t* __restrict__ nrec) {
  if (blockIdx.x > 0) {  // workgroup-uniform
    if (MODE == FUSED)
      rope_table_fill(a.src_pos, a.dst_pos, a.N, a.B, a.D, a.theta, const_cast<float2*>(a.tab),
                      (size_t)(blockIdx.x - 1) * kPlanThreads + threadIdx.x,
                      (size_t)(gridDim.x - 1) * kPlanThreads);
    return;
  }
  constexpr int W = kPlanThreads / kWave;
  __shared__ int wsum[2][W];
  __shared__ int red[W];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int rows = a.N * a.L;
  const int nb = a.T / kTile;
  const int ptot = a.priv_off[a.N];
  int32_t* slot_start = ctl + 2;
  // row r's task fields and its tile count
  auto row_task = [&](int r, StreamTask& t) {
    const int i = r / a.L, l = r % a.L;
    const int p0 = a.priv_off[i];
    t.P = a.priv_off[i + 1] - p0;
    t.P = min(t.P, a.pmax);
    t.ntp = (t.P + kTile - 1) / kTile;
    t.prow = l * ptot + p0;
    int nx = nb;
    if (MODE == FUSED) {
      t.e0 = a.diff_off[r];
      nx = min(max(a.diff_off[r + 1] - t.e0, 0), nb);
    }
    t.r = r;
    return t.ntp + nx;
  };
  // inclusive wave scan of x
  auto wave_scan = [&](int x) {
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    return x;
  };

  // pass 1: the total
  int part = 0;
  for (int r = tid; r < rows; r += kPlanThreads) {
    StreamTask t{};
    part += row_task(r, t);
  }
  part = wave_scan(part);
  if (lane == kWave - 1) red[wave] = part;
  __syncthreads();
  int total = 0;
  for (int w = 0; w < W; ++w) total += red[w];
  const int P = max(kTilesPerSplit, (total + nslot - 1) / nslot);

  // pass 2: each row's first tile position R0 and first task index, then its
  // tasks: piece j covers slot R0 / P + j
  int carry0 = 0, carry1 = 0;
  for (int base = 0; base < rows; base += kPlanThreads) {
    const int r = base + tid;
    StreamTask t{};
    const int nt = r < rows ? row_task(r, t) : 0;
    const int x0 = wave_scan(nt);
    if (lane == kWave - 1) wsum[0][wave] = x0;
    __syncthreads();
    int pre0 = carry0, all0 = carry0;
    for (int w = 0; w < W; ++w) {
      if (w < wave) pre0 += wsum[0][w];
      all0 += wsum[0][w];
    }
    const int R0 = pre0 + x0 - nt;
    const int first = R0 / P;
    const int np = nt > 0 ? (R0 + nt - 1) / P - first + 1 : 0;
    const int x1 = wave_scan(np);
    if (lane == kWave - 1) wsum[1][wave] = x1;
    __syncthreads();
    int pre1 = carry1, all1 = carry1;
    for (int w = 0; w < W; ++w) {
      if (w < wave) pre1 += wsum[1][w];
      all1 += wsum[1][w];
    }
    pre1 += x1 - np;
    if (r < rows) {
      nrec[r] = np;
      for (int j = 0; j < np; ++j) {
        const int sl = first + j;
        const int lo = max(R0, sl * P), hi = min(R0 + nt, (sl + 1) * P);
        t.s = j;
        t.t0 = lo - R0;
        t.cnt = hi - lo;
        tasks[pre1 + j] = t;
        if (lo == sl * P) slot_start[sl] = pre1 + j;  // the slot's first task
      }
    }
    carry0 = all0;
    carry1 = all1;
    __syncthreads();
  }
  // slots past the last piece have no tasks
  const int used = (total + P - 1) / P;
  for (int sl = used + tid; sl <= nslot; sl += kPlanThreads) slot_start[sl] = carry1;
  if (tid == 0) {
    ctl[0] = carry1;
    ctl[1] = nslot;
  }
}

template <typename E, int D, int MODE, int PD, bool PAGED>
__global__ __launch_bounds__(kStreamNW * kWave) __attribute__((amdgpu_waves_per_eu(TDX_ST_WPE))) void stream_kernel(
    AttnArgs a, const StreamTask* __restrict__ tasks, const int32_t* __restrict__ ctl, const float2* __restrict__ dcs,
    const int2* __restrict__ dinfo) {
  static_assert(sizeof(E) == 2, "bf16 caches (fp32 ones take the fp32 kernel)");
  using St = Stage<E, D, MODE>;
  constexpr int KD = St::KD;
  constexpr int DT = D / 16;
  constexpr int HALF = D / 2;
  constexpr int RB = D * (int)sizeof(E);  // K/V row bytes of one head
  constexpr int CPR = RB / 16;            // 16-byte chunks per K/V row
  constexpr int KB = kTile * RB;          // K tile bytes (as stored)
  constexpr int VB = kTile * D * 2;       // bf16 V tile bytes
  constexpr int CB = MODE == FUSED ? HALF * 8 : 0;  // cos/sin row of a diff entry
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform per wave
  const int q4 = lane / 16, c16 = lane % 16;
  const int g = a.Hq / a.Hkv;
  const int Hkv = a.Hkv;
  // Wave gw runs the tasks of slot gw / Hkv, [slot_start[s], slot_start[s + 1])
  // (stream_plan_kernel), for KV head gw % Hkv: the waves of a workgroup
  // work on neighbouring KV heads of the same rows.
  const int gw = blockIdx.x * kStreamNW + wave;
  const int slot = gw / Hkv;
  if (slot >= ctl[1]) return;  // wave-uniform; the kernel has no workgroup barrier
  const int ts = ctl[2 + slot], te = ctl[3 + slot];
  if (ts >= te) return;

  unsigned char* kl = smem + (size_t)wave * (KB + VB + CB);  // this wave's K tile
  unsigned char* vl = kl + KB;                               // V tile
  float2* csl = reinterpret_cast<float2*>(vl + VB);          // cos/sin row
  const size_t rowHD = (size_t)Hkv * D;
  const size_t rowbytes = rowHD * sizeof(E);
  const unsigned char* pkb = static_cast<const unsigned char*>(a.pk);
  const unsigned char* pvb = static_cast<const unsigned char*>(a.pv);

  // Per-lane byte offsets inside a tile: 16-byte chunk p = 64 v + lane is
  // row p / CPR, chunk p % CPR.  A tile's loads are a uniform base plus these.
  uint32_t loff[St::NV], lcol[St::NV];
#pragma unroll
  for (int v = 0; v < St::NV; ++v) {
    const int p = v * kWave + lane;
    lcol[v] = (uint32_t)(p % CPR) * 16u;
    loff[v] = (uint32_t)(p / CPR) * (uint32_t)rowbytes + lcol[v];
  }
  auto steps = [](const StreamTask& t) { return max(t.cnt, PD - 1); };
  // the query rows of (agent, layer, KV head) as the B operand: row min(c16, g-1),
  // elements 32k + 8*q4 .. +7 (rows >= g repeat row g-1; their logits are unused)
  auto load_q = [&](const StreamTask& t, int h, u32x4* qv) {
    const uint16_t* qp = a.qplain + ((size_t)t.r * a.Hq + (size_t)h * g + min(c16, g - 1)) * D;
#pragma unroll
    for (int k = 0; k < KD; ++k) qv[k] = ld16(qp + 32 * k + 8 * q4);
  };
  // ---- load side: task lk, its descriptor LT, step lu; the next task nk
  // and its descriptor ND
  const int lh = gw % Hkv;
  int lk = ts, lu = 0;
  StreamTask LT = tasks[lk];
  u32x4 qn[KD];
  load_q(LT, lh, qn);
  int nk = lk + 1;
  StreamTask ND = LT;
  if (nk < te) ND = tasks[nk];
  bool ldone = false;

  // ---- compute side: task pk of descriptor PT at step pu; the first PD-1
  // steps only fill the pipeline
  int pk = ts, pu = -(PD - 1);
  StreamTask PT = LT;
  u32x4 qop[KD];
#pragma unroll
  for (int k = 0; k < KD; ++k) qop[k] = u32x4{0, 0, 0, 0};
  RowState<D> st;
  st.init();

  auto load = [&](St& S) {
    if (lu == steps(LT) && !ldone) {  // next task (uniform)
      if (nk < te) {
        lk = nk;
        LT = ND;
        lu = 0;
        load_q(LT, lh, qn);
        nk = lk + 1;
        if (nk < te) ND = tasks[nk];
      } else {
        ldone = true;  // no more work: keep re-reading the last tile (masked)
        lk = te;
      }
    }
    const int su = min(lu, steps(LT) - 1);
    const int u = LT.t0 + min(su, LT.cnt - 1);  // tile of the row (uniform)
    const unsigned char* kb;
    const unsigned char* vb;
    int rmax = kTile - 1;  // rows past the end of a partial tile re-read its last row
    size_t e = 0;
    if (u < LT.ntp) {
      const size_t prow = PAGED ? ((size_t)(LT.r % a.L) * a.ppm.n_pages + page_at(a.ppm, LT.r / a.L, u)) * kTile
                                : (size_t)LT.prow + (size_t)u * kTile;
      const size_t o = (prow * rowHD + (size_t)lh * D) * sizeof(E);
      kb = pkb + o;
      vb = pvb + o;
      rmax = min(kTile - 1, LT.P - 1 - u * kTile);
    } else if (MODE == FUSED) {
      e = (size_t)(LT.e0 + u - LT.ntp);
      const size_t drow = PAGED ? ((size_t)(LT.r % a.L) * a.dpm.n_pages + page_at(a.dpm, 0, (long long)e)) * kTile
                                : e * kTile;
      const size_t o = (drow * rowHD + (size_t)lh * D) * sizeof(E);
      kb = static_cast<const unsigned char*>(a.dk) + o;
      vb = static_cast<const unsigned char*>(a.dv) + o;
    } else {
      const size_t o = (((size_t)LT.r * a.T + (size_t)(u - LT.ntp) * kTile) * rowHD + (size_t)lh * D) * sizeof(E);
      kb = static_cast<const unsigned char*>(a.sk) + o;
      vb = static_cast<const unsigned char*>(a.sv) + o;
    }
    // min(row, rmax) * rowbytes + column = min(loff, rmax * rowbytes + column)
    const uint32_t rlim = (uint32_t)rmax * (uint32_t)rowbytes;
#pragma unroll
    for (int v = 0; v < St::NV; ++v) {
      const uint32_t o = min(loff[v], rlim + lcol[v]);
      S.k[v] = ld16_nt(kb + o);
      S.v[v] = ld16_nt(vb + o);
    }
    if (MODE == FUSED) {  // a private tile reads entry 0 (unused)
      const size_t ec = e < (size_t)a.dcap ? e : 0;
      S.cs = dcs[ec * HALF + (lane % HALF)];
      S.info = dinfo[ec];  // uniform address: a scalar load
    }
    if (!ldone) ++lu;
  };

  // compute side, before the step's loads: a new task starts with the load
  // side's current one (the load side is at most PD-2 tiles ahead and a task
  // has at least PD-1 steps)
  auto begin = [&]() {
    if (pu == 0) {
      PT = LT;
      pk = lk;
#pragma unroll
      for (int k = 0; k < KD; ++k) qop[k] = qn[k];
    }
  };

  auto process = [&](St& S) {
    const bool live = pk < te && pu >= 0 && pu < PT.cnt;
    const int u = PT.t0 + min(max(pu, 0), PT.cnt - 1);
    // K rows -> LDS as loaded, V rows -> bf16 LDS tile (a wave's LDS
    // operations run in order, so the previous tile's reads are done)
#pragma unroll
    for (int v = 0; v < St::NV; ++v) {
      const int p = v * kWave + lane;
      *reinterpret_cast<u32x4*>(kl + klds_off<CPR>(p / CPR, p % CPR)) = S.k[v];
      *reinterpret_cast<u32x4*>(vl + vlds_off<D>(p / CPR, p % CPR)) = S.v[v];
    }
    const bool rot = MODE == FUSED && u >= PT.ntp;  // the agent's own block (wave-uniform)
    if (MODE == FUSED && lane < HALF) csl[lane] = S.cs;
    wave_sync();
    // K operand of the QK product: kop[k] = K[row c16][32k + 8*q4 .. +7] as bf16
    u32x4 kop[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) kop[k] = *reinterpret_cast<const u32x4*>(kl + klds_off<CPR>(c16, 4 * k + q4));
    if (rot) {
      float x[KD][8];
#pragma unroll
      for (int k = 0; k < KD; ++k) Fmt<uint16_t>::unpack(kop[k], x[k]);
      // rotate this lane's key row by the shift of the shared block holding
      // it; pairs (e, e + D/2) are chunks k and k + KD/2
      auto rotate = [&](auto row) {
#pragma unroll
        for (int k = 0; k < KD / 2; ++k) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int ce = 2 * (32 * k + 8 * q4 + j);  // (cos, sin) of element 32k + 8*q4 + j
            const float cc = row[ce], sn = row[ce + 1];
            const float lo = x[k][j], hi = x[k + KD / 2][j];
            x[k][j] = lo * cc - hi * sn;
            x[k + KD / 2][j] = hi * cc + lo * sn;
          }
          kop[k] = Fmt<uint16_t>::pack(x[k]);
          kop[k + KD / 2] = Fmt<uint16_t>::pack(x[k + KD / 2]);
        }
      };
      if (S.info.y >= 0) {
        // the whole tile lies in one shared block: its cos/sin row in LDS
        typedef __attribute__((address_space(3))) const float lds_float;
        rotate((lds_float*)csl);
      } else {
        // rows in several shared blocks: each row's own block, from the round's table
        const int t = S.info.x * kTile + c16;
        int lo = 0, hi = a.B - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (a.blk_start[mid] <= t) lo = mid; else hi = mid - 1;
        }
        typedef __attribute__((address_space(1))) const float global_float;
        rotate((global_float*)(a.tab + ((size_t)(PT.r / a.L) * a.B + lo) * HALF));
      }
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KD; ++k) acc = mfma32(kop[k], qop[k], acc);
    // rows >= lim of the tile are masked (lim = 16 for a full tile, less for
    // the last private tile, 0 for a fill, pad or drain step)
    const int lim = !live ? 0 : (u < PT.ntp ? min(kTile, PT.P - u * kTile) : kTile);
    float z[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = 4 * q4 + j < lim ? acc[j] * a.scale_log2 : -INFINITY;
    // PV operand: va[dt][j] = V[token 4*q4 + j][dim 16*dt + c16]; this lane
    // addresses row 4*q4 + c16/4, dims 16*dt + 4*(c16%4)
    i16x4 va[DT];
    const int vrow = 4 * q4 + (c16 >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      va[dt] = ld_tr16(vl + vlds_off<D>(vrow, 2 * dt + ((c16 & 3) >> 1)) + (c16 & 1) * 8);
    softmax_pv<D>(st, z, va);
    // advance; at the end of a task write its record and start afresh
    if (pu < 0) {
      ++pu;
    } else if (++pu == steps(PT)) {
      if (pk < te) {
        float lsum = st.l;
        lsum += __shfl_xor(lsum, 16, kWave);
        lsum += __shfl_xor(lsum, 32, kWave);
        if (c16 < g) {
          float* rec = a.part + (((size_t)PT.r * a.Hq + (size_t)lh * g + c16) * a.S + PT.s) * (D + 4);
          write_record<D>(rec, st, lsum, q4, c16);
        }
      }
      st.init();
      pu = 0;
    }
  };

  // PD-stage register pipeline: step k of the unrolled body loads into
  // S[(k+PD-1) % PD] and uses S[k], with no branch around either, so every
  // stage lives in the same registers on every pass and the wait before a
  // stage is used leaves the PD-1 younger tiles in flight.  The loop runs
  // until the compute side has passed its last task (masked steps after it).
  St S[PD] = {};
  // the first query loads complete here, once: otherwise the compiler's wait
  // counting sees them outstanding at the top of the loop
  __builtin_amdgcn_s_waitcnt(0);
  do {
#pragma unroll
    for (int k = 0; k < PD; ++k) {
      begin();
      load(S[(k + PD - 1) % PD]);
      process(S[k]);
    }
  } while (pk < te);
}

// One wave per output row (agent, layer, query head): combine the stream
// kernel's records [0, nsp) of the row (nsp = nrec[agent * L + layer]) and
// the shared kernel's splits [SP, SP + SG).
template <typename E, int D, int MODE>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, const int32_t* __restrict__ nrec,
                                                     E* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const size_t row = (size_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= (size_t)a.N * a.L * a.Hq) return;
  const int i = (int)(row / ((size_t)a.L * a.Hq));
  const int l = (int)((row / a.Hq) % a.L);
  const int nsp = min(nrec[i * a.L + l], a.SP);
  const size_t rec = D + 4;
  const float* pr = a.part + row * a.S * rec;
  // the row's records: its nsp agent splits, then the Master splits [SP, S)
  // (slots [nsp, SP) belong to no task of this row); record j of that list
  const int nu = nsp + (a.S - a.SP);
  auto rec_of = [&](int j) { return (size_t)(j < nsp ? j : a.SP + (j - nsp)) * rec; };
  // the row maximum: lane j reads record j's m (up to 64 records at once)
  float mm = -INFINITY;
  for (int j0 = 0; j0 < nu; j0 += kWave) {
    const int j = j0 + lane;
    const float ms = pr[rec_of(min(j, nu - 1))];
    mm = fmaxf(mm, j < nu ? ms : -INFINITY);
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o, kWave));
  // rescale and add the records in list order, MG records' loads in flight at
  // a time
  constexpr int PER = D / kWave;
  constexpr int MG = 8;
  float o[PER] = {};
  float ls = 0.f;
  for (int j0 = 0; j0 < nu; j0 += MG) {
    float mv[MG], lv[MG], ov[MG][PER];
#pragma unroll
    for (int j = 0; j < MG; ++j) {
      const float* r = pr + rec_of(min(j0 + j, nu - 1));
      mv[j] = r[0];
      lv[j] = r[1];
#pragma unroll
      for (int k = 0; k < PER; ++k) ov[j][k] = r[4 + lane + k * kWave];
    }
#pragma unroll
    for (int j = 0; j < MG; ++j) {
      if (j0 + j >= nu) break;
      const float f = (mv[j] == -INFINITY) ? 0.f : exp2f(mv[j] - mm);
      ls += f * lv[j];
#pragma unroll
      for (int k = 0; k < PER; ++k) o[k] += f * ov[j][k];
    }
  }
  const float inv = ls > 0.f ? 1.0f / ls : 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    out[row * D + lane + k * kWave] = (uint16_t)f32_to_bf16(o[k] * inv);
  }
}

// ---- dense restore ---------------------------------------------------------------
// One workgroup per (diff block beta, agent i), looping over layers: K rows are
// taken from the diff record or the Master, rotated by Delta(i, b(t)) and
// rounded; V rows are copied.

constexpr int kMaxTileBlocks = kTile;  // a 16-token tile touches at most 16 blocks

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void restore_dense_kernel(
    const E* __restrict__ mk, const E* __restrict__ mv, const int32_t* __restrict__ msel,
    long long mstride, const int32_t* __restrict__ diff_off,
    const int32_t* __restrict__ diff_idx, const E* __restrict__ dk, const E* __restrict__ dv,
    const int32_t* __restrict__ blk_start, const int32_t* __restrict__ src_pos,
    const int32_t* __restrict__ dst_pos, int N, int B, int T, int L, int Hkv, double theta,
    E* __restrict__ kd, E* __restrict__ vd) {
  constexpr int VEC = Fmt<E>::VEC;
  constexpr int HALF = D / 2;
  constexpr int G = HALF / VEC;
  constexpr int RPP = kThreads / G;
  __shared__ float2 tab[kMaxTileBlocks * HALF];
  __shared__ int s_nb;
  __shared__ int32_t sst[kMaxTileBlocks], sid[kMaxTileBlocks];  // non-empty blocks of the tile
  __shared__ int32_t szero[kMaxTileBlocks];                       // the block's shift is 0
  const int beta = blockIdx.x;
  const int i = blockIdx.y;
  const int tid = threadIdx.x;
  const int t0 = beta * kTile;
  const size_t moff = master_offset(msel, mstride, N);
  mk += moff;
  mv += moff;
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
        szero[n] = dst_pos[(size_t)i * B + b] == src_pos[b];
        ++n;
      }
    s_nb = n;
  }
  __syncthreads();
  const int nbk = s_nb;
  for (int x = tid; x < nbk * HALF; x += kThreads) {
    const int bb = x / HALF, e = x % HALF;
    const double delta = (double)(dst_pos[(size_t)i * B + sid[bb]] - src_pos[sid[bb]]);
    double sn, cs;
    sincos(delta * rope_inv_freq(theta, e, D), &sn, &cs);
    tab[x] = make_float2((float)cs, (float)sn);
  }
  __syncthreads();
  const int e0 = (tid % G) * VEC;
  const int row0 = tid / G;
  const int nrows = kTile * Hkv;
  const size_t rowHD = (size_t)Hkv * D;
  for (int l = 0; l < L; ++l) {
    const int r = i * L + l;
    int lo = diff_off[r], hi = diff_off[r + 1];
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (diff_idx[mid] < beta) lo = mid + 1; else hi = mid;
    }
    const bool hit = lo < diff_off[r + 1] && diff_idx[lo] == beta;
    const E* ks = hit ? dk + (size_t)lo * kTile * rowHD : mk + ((size_t)l * T + t0) * rowHD;
    const E* vs = hit ? dv + (size_t)lo * kTile * rowHD : mv + ((size_t)l * T + t0) * rowHD;
    E* ko = kd + (((size_t)i * L + l) * T + t0) * rowHD;
    E* vo = vd + (((size_t)i * L + l) * T + t0) * rowHD;
    for (int row = row0; row < nrows; row += RPP) {
      const int tok = t0 + row / Hkv;
      int bb = 0;
      while (bb + 1 < nbk && sst[bb + 1] <= tok) ++bb;
      const size_t off = (size_t)row * D + e0;
      const u32x4 rl = ld16(ks + off), rh = ld16(ks + off + HALF);
      if (szero[bb]) {  // R(0) is the identity: the stored bits as they are
        st16_nt(ko + off, rl);
        st16_nt(ko + off + HALF, rh);
      } else {
        float x[VEC], y[VEC], ox[VEC], oy[VEC];
        Fmt<E>::unpack(rl, x);
        Fmt<E>::unpack(rh, y);
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const float2 cs = tab[bb * HALF + e0 + j];
          ox[j] = x[j] * cs.x - y[j] * cs.y;
          oy[j] = y[j] * cs.x + x[j] * cs.y;
        }
        st16_nt(ko + off, Fmt<E>::pack(ox));
        st16_nt(ko + off + HALF, Fmt<E>::pack(oy));
      }
      st16_nt(vo + off, ld16(vs + off));
      st16_nt(vo + off + HALF, ld16(vs + off + HALF));
    }
  }
}

// ---- host-side planning ------------------------------------------------------------

struct Plan {
  int SP, SG, AGS, NAG, TPG, n_sh_wg;
  long long dcap;
  size_t part_bytes, tab_off, task_off, ctl_off, nrec_off, dcs_off, dinfo_off, total;
};

Plan make_plan(const Dims& d, int max_priv, bool fused) {
  Plan p{};
  const int nb = d.T / kTile;
  // stream-kernel records per row: a row of at most SP0 * kTilesPerSplit
  // tiles, cut into pieces of at least kTilesPerSplit tiles at arbitrary
  // offsets, has at most SP0 + 1 of them
  const int SP0 = ((max_priv + kTile - 1) / kTile + nb + kTilesPerSplit - 1) / kTilesPerSplit;
  p.SP = (SP0 < 1 ? 1 : SP0) + 1;
  if (fused) {
    const int g = d.Hq / d.Hkv;
    p.AGS = kRowsPerGroup / g;
    if (p.AGS > d.N) p.AGS = d.N;
    if (p.AGS < 1) p.AGS = 1;
    p.NAG = (d.N + p.AGS - 1) / p.AGS;
    const long base = (long)p.NAG * d.L * d.Hkv;
    long sg = (TDX_SH_TARGET_WG + base - 1) / base;  // aim at this many workgroups
    if (sg < 1) sg = 1;
    if (sg > nb) sg = nb;
    p.TPG = (int)((nb + sg - 1) / sg);
    if (p.TPG > kMaxSharedTiles) p.TPG = kMaxSharedTiles;
    p.SG = (nb + p.TPG - 1) / p.TPG;
    p.n_sh_wg = p.NAG * p.SG * d.L * d.Hkv;
  }
  // a valid diff record has at most T/16 entries per (agent, layer) row
  p.dcap = fused ? (long long)d.N * d.L * nb : 0;
  if (p.dcap < 1) p.dcap = 1;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.part_bytes = (size_t)d.N * d.L * d.Hq * (p.SP + p.SG) * (d.D + 4) * 4;
  p.tab_off = up(p.part_bytes);
  p.task_off = p.tab_off + (fused ? up((size_t)d.N * d.B * (d.D / 2) * 8) : 0);
  p.ctl_off = p.task_off + up((size_t)d.N * d.L * p.SP * sizeof(StreamTask));
  p.nrec_off = p.ctl_off + up((size_t)(kMaxSlots + 3) * 4);
  p.dcs_off = p.nrec_off + up((size_t)d.N * d.L * 4);
  p.dinfo_off = p.dcs_off + (fused ? up((size_t)p.dcap * (d.D / 2) * 8) : 0);
  p.total = p.dinfo_off + (fused ? up((size_t)p.dcap * 8) : 0);
  return p;
}

// register stages of stream_kernel: PD stages keep PD-1 tiles in flight per wave
template <typename E, int D>
struct StreamCfg {
  static constexpr int PD = TDX_ST_PD;
  static constexpr size_t lds(bool fused) {
    return (size_t)kStreamNW * (kTile * D * sizeof(E) + kTile * D * 2 + (fused ? D / 2 * 8 : 0));
  }
};

// the Master-tile kernel's LDS: its tile ring of nb slots, blk_start, the
// diff flags (one bit per agent and tile)
size_t shared_lds(int D, int B, const Plan& p, int nb) {
  return (size_t)nb * 2 * kTile * D * 2 + (size_t)(B + 1) * 4 + (size_t)p.AGS * ((p.TPG + 31) / 32) * 4;
}

template <typename E, int D, int MODE, bool PAGED>
hipError_t launch_attn_t(const Dims& d, AttnArgs a, const Plan& p, E* out, hipStream_t s) {
  static_assert(!PAGED || MODE == FUSED, "paged caches: fused path only");
  a.SP = p.SP;
  a.SG = p.SG;
  a.S = p.SP + p.SG;
  a.AGS = p.AGS;
  a.NAG = p.NAG;
  a.TPG = p.TPG;
  a.n_sh_wg = p.n_sh_wg;
  a.dcap = p.dcap;
  hipError_t e;
  a.qplain = static_cast<const uint16_t*>(a.q);  // bf16 queries are the MFMA operand as stored
  constexpr int PD = StreamCfg<E, D>::PD;
  const size_t lds = StreamCfg<E, D>::lds(MODE == FUSED);
  auto kern = stream_kernel<E, D, MODE, PD, PAGED>;
  int dev = 0, ncu = 0, per_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                         kStreamNW * kWave, lds)) != hipSuccess)
    return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  // resident workgroups (at least one slot: one wave per KV head); slot s
  // is waves s * Hkv .. s * Hkv + Hkv - 1
  const int grid = std::max(ncu * per_cu, (d.Hkv + kStreamNW - 1) / kStreamNW);
  const int nslot = std::min(grid * kStreamNW / d.Hkv, kMaxSlots);
  StreamTask* tasks = reinterpret_cast<StreamTask*>(a.ws_base + p.task_off);
  int32_t* ctl = reinterpret_cast<int32_t*>(a.ws_base + p.ctl_off);  // task count, slots, slot starts
  int32_t* nrec = reinterpret_cast<int32_t*>(a.ws_base + p.nrec_off);
  const float2* dcs = reinterpret_cast<const float2*>(a.ws_base + p.dcs_off);
  const int2* dinfo = reinterpret_cast<const int2*>(a.ws_base + p.dinfo_off);
  // set-up: the task plan (workgroup 0) and, fused, the cos/sin table (the
  // other workgroups) in one launch
  int pgrid = 1;
  if (MODE == FUSED) {
    const size_t n = (size_t)d.N * d.B * (d.D / 2);
    pgrid += (int)std::min<size_t>((n + kPlanThreads - 1) / kPlanThreads, 64);
  }
  hipLaunchKernelGGL((stream_plan_kernel<MODE>), dim3(pgrid), dim3(kPlanThreads), 0, s, a, nslot, tasks, ctl, nrec);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (MODE == FUSED) {
    // in front of the Master-tile workgroups: per diff entry, its shared
    // block and that block's cos/sin row (one (agent, layer) row per wave)
    a.dcs = reinterpret_cast<float2*>(a.ws_base + p.dcs_off);
    a.dinfo = reinterpret_cast<int2*>(a.ws_base + p.dinfo_off);
    a.n_dt_wg = (d.N * d.L + kShWaves - 1) / kShWaves;
    a.n_dt_wg = (a.n_dt_wg + 7) / 8 * 8;
    // a ring of TDX_SH_NB slots, or of 3 when blk_start and the diff flags
    // leave too little of the 64 KB
    const int sgrid = a.n_dt_wg + (p.n_sh_wg + 7) / 8 * 8;
    const size_t slds = shared_lds(D, d.B, p, TDX_SH_NB);
    if (slds <= 64 * 1024) {
      hipLaunchKernelGGL((shared_kernel<E, D, TDX_SH_NB, PAGED>), dim3(sgrid), dim3(kShThreads), slds, s, a);
    } else {
      const size_t lds3 = shared_lds(D, d.B, p, 3);
      if (lds3 > 64 * 1024) return hipErrorInvalidValue;
      hipLaunchKernelGGL((shared_kernel<E, D, 3, PAGED>), dim3(sgrid), dim3(kShThreads), lds3, s, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kStreamNW * kWave), lds, s, a, tasks, ctl, dcs, dinfo);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t rows = (size_t)d.N * d.L * d.Hq;
  const int rpb = 256 / kWave;
  hipLaunchKernelGGL((merge_kernel<E, D, MODE>), dim3((rows + rpb - 1) / rpb), dim3(256), 0, s, a,
                     static_cast<const int32_t*>(nrec), out);
  return hipGetLastError();
}

// bf16 caches (fp32 ones take launch_attn_f32 before reaching here)
template <int MODE, bool PAGED = false>
hipError_t dispatch_attn(const Dims& d, AttnArgs a, const Plan& p, void* out, hipStream_t s) {
  if (d.dtype != TDX_BF16) return hipErrorInvalidValue;
  return d.D == 128 ? launch_attn_t<uint16_t, 128, MODE, PAGED>(d, a, p, static_cast<uint16_t*>(out), s)
                    : launch_attn_t<uint16_t, 64, MODE, PAGED>(d, a, p, static_cast<uint16_t*>(out), s);
}

AttnArgs common_args(const Dims& d, const void* q, const int32_t* priv_off, const void* pk,
                     const void* pv, int max_priv, float scale, void* ws) {
  AttnArgs a{};
  a.q = q;
  a.priv_off = priv_off;
  a.pk = pk;
  a.pv = pv;
  a.part = static_cast<float*>(ws);
  a.ws_base = static_cast<unsigned char*>(ws);
  a.N = d.N;
  a.L = d.L;
  a.T = d.T;
  a.B = d.B;
  a.Hkv = d.Hkv;
  a.Hq = d.Hq;
  a.D = d.D;
  a.scale_log2 = scale * kLog2e;
  // private histories are capped at max_priv: the splits are sized for it,
  // so a history past it can only lose its own tail, never the diff tiles
  // that follow it (paged: a page-table row holds no private page past it)
  a.pmax = max_priv;
  return a;
}

}  // namespace

size_t restore_attn_ws_bytes(const Dims& d, int max_priv) {
  return d.dtype == TDX_F32 ? f32_attn_ws_bytes(d, max_priv, true) : make_plan(d, max_priv, true).total;
}
size_t dense_attn_ws_bytes(const Dims& d, int max_priv) {
  return d.dtype == TDX_F32 ? f32_attn_ws_bytes(d, max_priv, false) : make_plan(d, max_priv, false).total;
}

namespace {
// fp32 caches take the fp32 vector-unit path (attn_f32.hip)
F32AttnArgs f32_args(const Dims& d, const tdx_layout* lay, const void* q, const int32_t* priv_off, const void* pk,
                     const void* pv, float scale, void* out) {
  F32AttnArgs a{};
  a.q = static_cast<const float*>(q);
  a.priv_off = priv_off;
  a.pk = static_cast<const float*>(pk);
  a.pv = static_cast<const float*>(pv);
  if (lay != nullptr) {
    a.blk_start = lay->blk_start;
    a.src_pos = lay->src_pos;
    a.dst_pos = lay->dst_pos;
  }
  a.scale_log2 = scale * kLog2e;
  a.out = static_cast<float*>(out);
  return a;
}
}  // namespace

namespace {
// The fused restore: set-up (task plan and cos/sin table, per-diff-entry rows), then the attention kernels.
template <bool PAGED>
hipError_t restore_attn_t(const Dims& d, const tdx_layout& lay, AttnArgs a, const int32_t* diff_off,
                          const int32_t* diff_idx, int max_priv, void* out, void* ws, hipStream_t s) {
  const Plan p = make_plan(d, max_priv, true);
  a.diff_off = diff_off;
  a.diff_idx = diff_idx;
  a.blk_start = lay.blk_start;
  a.tab = reinterpret_cast<float2*>(static_cast<unsigned char*>(ws) + p.tab_off);
  a.src_pos = lay.src_pos;
  a.dst_pos = lay.dst_pos;
  a.theta = d.theta;
  return dispatch_attn<FUSED, PAGED>(d, a, p, out, s);
}
}  // namespace

hipError_t launch_restore_attn(const Dims& d, const tdx_layout& lay, const void* q,
                               const int32_t* priv_off, const void* pk, const void* pv,
                               int max_priv, const MasterRef& master,
                               const int32_t* diff_off, const int32_t* diff_idx, const void* dk,
                               const void* dv, float scale, void* out, void* ws, hipStream_t s) {
  if (d.dtype == TDX_F32) {
    F32AttnArgs f = f32_args(d, &lay, q, priv_off, pk, pv, scale, out);
    f.sk = static_cast<const float*>(master.k);
    f.sv = static_cast<const float*>(master.v);
    f.msel = master.sel;
    f.mstride = master.stride;
    f.diff_off = diff_off;
    f.diff_idx = diff_idx;
    f.dk = static_cast<const float*>(dk);
    f.dv = static_cast<const float*>(dv);
    return launch_attn_f32(d, FUSED, false, f, max_priv, ws, s);
  }
  AttnArgs a = common_args(d, q, priv_off, pk, pv, max_priv, scale, ws);
  a.sk = master.k;
  a.sv = master.v;
  a.msel = master.sel;
  a.mstride = master.stride;
  a.dk = dk;
  a.dv = dv;
  return restore_attn_t<false>(d, lay, a, diff_off, diff_idx, max_priv, out, ws, s);
}

hipError_t launch_restore_attn_paged(const Dims& d, const tdx_layout& lay, const void* q, const int32_t* priv_off,
                                     const void* pk_pool, const void* pv_pool, const PageMap& ppm, int max_priv,
                                     const void* ak_pool, const void* av_pool, const PageMap& apm,
                                     const int32_t* master_sel, const int32_t* diff_off, const int32_t* diff_idx,
                                     const int32_t* diff_page, float scale, void* out, void* ws, hipStream_t s) {
  if (d.dtype == TDX_F32) {
    F32AttnArgs f = f32_args(d, &lay, q, priv_off, pk_pool, pv_pool, scale, out);
    f.sk = f.dk = static_cast<const float*>(ak_pool);  // Master and diff pages are agents' pages
    f.sv = f.dv = static_cast<const float*>(av_pool);
    f.msel = master_sel;
    f.mpm = apm;
    f.dpm = PageMap{diff_page, 0, apm.n_pages};
    f.ppm = ppm;
    f.diff_off = diff_off;
    f.diff_idx = diff_idx;
    return launch_attn_f32(d, FUSED, true, f, max_priv, ws, s);
  }
  AttnArgs a = common_args(d, q, priv_off, pk_pool, pv_pool, max_priv, scale, ws);
  a.sk = ak_pool;  // the Master's pages and the diff entries' pages are agents' pages
  a.sv = av_pool;
  a.dk = ak_pool;
  a.dv = av_pool;
  a.msel = master_sel;
  a.mpm = apm;
  a.dpm = PageMap{diff_page, 0, apm.n_pages};
  a.ppm = ppm;
  return restore_attn_t<true>(d, lay, a, diff_off, diff_idx, max_priv, out, ws, s);
}

hipError_t launch_restore_dense(const Dims& d, const tdx_layout& lay, const MasterRef& master,
                                const int32_t* diff_off, const int32_t* diff_idx, const void* dk,
                                const void* dv, void* kd, void* vd, hipStream_t s) {
  dim3 grid(d.T / kTile, d.N);
#define TDX_RD(E, DD)                                                                          \
  hipLaunchKernelGGL((restore_dense_kernel<E, DD>), grid, dim3(kThreads), 0, s,               \
                     static_cast<const E*>(master.k), static_cast<const E*>(master.v),         \
                     master.sel, (long long)master.stride, diff_off, diff_idx,                 \
                     static_cast<const E*>(dk), static_cast<const E*>(dv), lay.blk_start,      \
                     lay.src_pos, lay.dst_pos, d.N, d.B, d.T, d.L, d.Hkv, d.theta,             \
                     static_cast<E*>(kd), static_cast<E*>(vd))
  if (d.dtype == TDX_BF16) {
    if (d.D == 128) TDX_RD(uint16_t, 128); else TDX_RD(uint16_t, 64);
  } else {
    if (d.D == 128) TDX_RD(float, 128); else TDX_RD(float, 64);
  }
#undef TDX_RD
  return hipGetLastError();
}

hipError_t launch_dense_attn(const Dims& d, const void* q, const int32_t* priv_off,
                             const void* pk, const void* pv, int max_priv, const void* kd,
                             const void* vd, float scale, void* out, void* ws, hipStream_t s) {
  if (d.dtype == TDX_F32) {
    F32AttnArgs f = f32_args(d, nullptr, q, priv_off, pk, pv, scale, out);
    f.sk = static_cast<const float*>(kd);
    f.sv = static_cast<const float*>(vd);
    return launch_attn_f32(d, DENSE, false, f, max_priv, ws, s);
  }
  const Plan p = make_plan(d, max_priv, false);
  AttnArgs a = common_args(d, q, priv_off, pk, pv, max_priv, scale, ws);
  a.sk = kd;
  a.sv = vd;
  return dispatch_attn<DENSE>(d, a, p, out, s);
}

}  // namespace tdx

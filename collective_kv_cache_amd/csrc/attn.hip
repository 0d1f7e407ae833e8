// a5 / a6: fused restore + decode attention, and the dense comparator.
//
// TokenDance notes §3d and §4 ("Fused Diff Restore"), blog §4.4: a Mirror is
// never rebuilt densely; its diff blocks are merged into the Master's tiles
// on chip, RoPE is recovered, and attention runs on the tile right away.  The
// dense comparator (restore every agent's cache, then attend) is what the
// fused path is measured against (notes §3d, §7b).
//
// Split-K decode attention, one workgroup per (agent i, key split, layer l,
// KV head h), 4 waves.  Agent i's keys are its private history followed by
// the shared tokens; they are walked in 16-token tiles (a shared tile is
// exactly one 16-token diff block).  Per tile a wave:
//   * loads the K rows straight into MFMA A-operand registers: for a shared
//     tile in the fused path each lane takes its token's row from the diff
//     record when the block is in agent i's diff row, else from the Master;
//   * stages V in wave-private LDS;
//   * computes S^T = K Q'^T with v_mfma_f32_16x16x32_bf16, where Q' is the
//     GQA query group of KV head h.  RoPE is recovered on the query side:
//     q . R(Delta) k = (R(-Delta) q) . k, so a shared tile of block b uses
//     Q' = R(-Delta(i,b)) q (cos/sin from a double-precision table), and one
//     Master tile layout serves every agent;
//   * runs an online softmax per query row (rows live in lanes) and
//     accumulates O^T += V^T P^T with v_mfma_f32_16x16x16_bf16.
// The four waves combine in LDS; a merge kernel combines the splits.
// Operands are bf16 (fp32 K/V/q are rounded to bf16 for the MFMA); softmax,
// accumulation and the merge run in fp32.
#include "common.h"

namespace tdx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = 16;
constexpr int kTilesPerSplit = 64;  // 16 per wave
constexpr float kLog2e = 1.4426950408889634f;

enum Mode { FUSED = 0, DENSE = 1 };

// ---- bf16 operand helpers ---------------------------------------------------

__device__ __forceinline__ uint32_t bf16_bits(float f) { return f32_to_bf16(f); }

// 8 consecutive elements -> 8 floats
template <typename E>
__device__ __forceinline__ void load8(const E* p, float* x);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* x) {
  Fmt<uint16_t>::unpack(ld16(p), x);
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* x) {
  Fmt<float>::unpack(ld16(p), x);
  Fmt<float>::unpack(ld16(p + 4), x + 4);
}

// 8 consecutive elements as packed bf16 (4 dwords), no float round trip for bf16
template <typename E>
__device__ __forceinline__ u32x4 load8_bf16(const E* p);
template <>
__device__ __forceinline__ u32x4 load8_bf16<uint16_t>(const uint16_t* p) {
  return ld16(p);
}
template <>
__device__ __forceinline__ u32x4 load8_bf16<float>(const float* p) {
  float x[8];
  load8<float>(p, x);
  u32x4 v;
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = pack_bf16(x[2 * k], x[2 * k + 1]);
  return v;
}

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

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ---- RoPE table: tab[(i*B + b)*HALF + e] = (cos, sin)(Delta(i,b) * theta^(-2e/D))

__global__ __launch_bounds__(256) void rope_table_kernel(const int32_t* __restrict__ src_pos,
                                                         const int32_t* __restrict__ dst_pos,
                                                         int N, int B, int D, double theta,
                                                         float2* __restrict__ tab) {
  const int half = D / 2;
  const size_t n = (size_t)N * B * half;
  for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < n;
       x += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(x % half);
    const size_t ib = x / half;
    const int b = (int)(ib % B);
    const double delta = (double)(dst_pos[ib] - src_pos[b]);
    double sn, cs;
    sincos(delta * rope_inv_freq(theta, e, D), &sn, &cs);
    tab[x] = make_float2((float)cs, (float)sn);
  }
}

// ---- split attention ----------------------------------------------------------

struct AttnArgs {
  const void* q;          // [N][L][Hq][D]
  const int32_t* priv_off;
  const void* pk;         // [L][Ptot][Hkv][D]
  const void* pv;
  const void* sk;         // fused: master [L][T][Hkv][D]; dense: k_dense [N][L][T][Hkv][D]
  const void* sv;
  const int32_t* diff_off;  // fused only
  const int32_t* diff_idx;
  const void* dk;         // [nnz][16][Hkv][D]
  const void* dv;
  const int32_t* blk_start;  // fused only
  const float2* tab;         // fused only [N][B][D/2]
  float* part;               // [N][L][Hq][S][D+4]
  int N, L, T, B, Hkv, Hq, S;
  float scale_log2;
};

template <int D>
struct WaveState {
  static constexpr int DT = D / 16;
  f32x4 o[DT];  // O^T tile dt: dims dt*16 + 4q + j, row = lane % 16
  float m;      // running max (log2 domain), row-uniform
  float l;      // lane-partial running sum
};

// Online-softmax update and PV for one tile.  z: 4 logits (log2 domain) of
// the lane's row at tokens 4q..4q+3 (-inf when masked).  vt: wave-private
// V tile in LDS, [16][D + 8] bf16.
template <int D>
__device__ __forceinline__ void softmax_pv(WaveState<D>& st, float z[4], const uint16_t* vt,
                                           int lane) {
  constexpr int DT = D / 16;
  constexpr int VS = D + 8;
  float tmax = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
  const float mnew = fmaxf(st.m, tmax);
  // while a row has seen no valid key, mnew = -inf: use 0 as the reference so
  // that every exp2 below is of -inf (-> 0) and nothing turns into NaN; the
  // path stays uniform across the wave around the MFMAs
  const float mref = (mnew == -INFINITY) ? 0.0f : mnew;
  const float alpha = exp2f(st.m - mref);  // st.m = -inf -> 0
  st.m = mnew;
  i16x4 pb;
  float psum = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float p = exp2f(z[j] - mref);  // masked -> 0
    const uint32_t b = bf16_bits(p);
    pb[j] = (short)b;
    psum += __uint_as_float(b << 16);
  }
  st.l = st.l * alpha + psum;
  const int q = lane / 16, c = lane % 16;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    st.o[dt] *= alpha;
    i16x4 va;
#pragma unroll
    for (int j = 0; j < 4; ++j) va[j] = (short)vt[(4 * q + j) * VS + dt * 16 + c];
    st.o[dt] = mfma16(va, pb, st.o[dt]);
  }
}

template <typename E, int D, int MODE>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(AttnArgs a) {
  constexpr int KD = D / 32;       // 32-dim k-steps of the QK MFMA
  constexpr int DT = D / 16;
  constexpr int HALF = D / 2;
  constexpr int VS = D + 8;        // padded LDS row stride (bf16)
  extern __shared__ __align__(16) unsigned char smem[];
  // layout: [kWaves][16][VS] bf16 V tiles | combine area aliases it afterwards | blk_start
  uint16_t* vtile_all = reinterpret_cast<uint16_t*>(smem);
  const size_t vbytes = (size_t)kWaves * kTile * VS * 2;
  const size_t cbytes = (size_t)kWaves * 16 * (D + 4) * 4;
  int32_t* sblk = reinterpret_cast<int32_t*>(smem + (vbytes > cbytes ? vbytes : cbytes));

  const int i = blockIdx.x;
  const int s = blockIdx.y;
  const int l = blockIdx.z / a.Hkv;
  const int h = blockIdx.z % a.Hkv;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int q4 = lane / 16, c16 = lane % 16;
  const int g = a.Hq / a.Hkv;

  const size_t ptot = (size_t)a.priv_off[a.N];  // private rows per layer
  const int p0 = a.priv_off[i];
  const int P = a.priv_off[i + 1] - p0;
  const int ntp = (P + kTile - 1) / kTile;
  const int nts = a.T / kTile;
  const int ntiles = ntp + nts;
  const int tbeg = s * kTilesPerSplit;
  if (tbeg >= ntiles) return;  // uniform: this agent has fewer splits
  const int tend = min(tbeg + kTilesPerSplit, ntiles);

  if (MODE == FUSED) {
    for (int b = tid; b <= a.B; b += kThreads) sblk[b] = a.blk_start[b];
  }

  const E* qrow = static_cast<const E*>(a.q) + (((size_t)i * a.L + l) * a.Hq + (size_t)h * g) * D;
  // query operand: row c16 (valid when < g), dims 8*q4 + 32k .. +7
  float qf[KD][8];
  u32x4 qb[KD], qr[KD];
#pragma unroll
  for (int k = 0; k < KD; ++k) {
    if (c16 < g) {
      load8<E>(qrow + (size_t)c16 * D + 32 * k + 8 * q4, qf[k]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[k][j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[k][j] = pack_bf16(qf[k][2 * j], qf[k][2 * j + 1]);
    qr[k] = qb[k];
  }
  __syncthreads();  // sblk ready

  WaveState<D> st;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.0f;

  uint16_t* vt = vtile_all + (size_t)wave * kTile * VS;
  const size_t rowHD = (size_t)a.Hkv * D;
  const E* pk = static_cast<const E*>(a.pk) + ((size_t)l * ptot + p0) * rowHD + (size_t)h * D;
  const E* pv = static_cast<const E*>(a.pv) + ((size_t)l * ptot + p0) * rowHD + (size_t)h * D;

  // fused: cursor into agent i's diff row at layer l
  int dcur = 0, dend = 0;
  int bcur = -1;  // block whose rotation qr holds
  if (MODE == FUSED) {
    const int r = i * a.L + l;
    dcur = a.diff_off[r];
    dend = a.diff_off[r + 1];
    // first entry >= the first shared diff block this wave can visit
    int first = tbeg + wave - ntp;
    if (first < 0) first = 0;
    int lo = dcur, hi = dend;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (a.diff_idx[mid] < first) lo = mid + 1; else hi = mid;
    }
    dcur = lo;
  }

  for (int tile = tbeg + wave; tile < tend; tile += kWaves) {
    u32x4 kop[KD];
    const E* vsrc;
    float z[4];
    if (tile < ntp) {
      // ---- private tile
      const int p = tile * kTile + c16;
      const bool ok = p < P;
      const E* krow = pk + (size_t)(ok ? p : 0) * rowHD;
      vsrc = pv + (size_t)(ok ? p : 0) * rowHD;
#pragma unroll
      for (int k = 0; k < KD; ++k) kop[k] = ok ? load8_bf16<E>(krow + 32 * k + 8 * q4) : u32x4{0, 0, 0, 0};
      // V -> LDS
#pragma unroll
      for (int k = 0; k < KD; ++k) {
        const u32x4 v = ok ? load8_bf16<E>(vsrc + 32 * k + 8 * q4) : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(vt + c16 * VS + 32 * k + 8 * q4) = v;
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KD; ++k) acc = mfma32(kop[k], qb[k], acc);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        z[j] = (tile * kTile + 4 * q4 + j < P) ? acc[j] * a.scale_log2 : -INFINITY;
    } else {
      // ---- shared tile = diff block beta
      const int beta = tile - ntp;
      const int t = beta * kTile + c16;
      const E* krow;
      const E* vrow;
      if (MODE == FUSED) {
        while (dcur < dend && a.diff_idx[dcur] < beta) ++dcur;
        const bool hit = dcur < dend && a.diff_idx[dcur] == beta;
        if (hit) {
          const size_t o = ((size_t)dcur * kTile + c16) * rowHD + (size_t)h * D;
          krow = static_cast<const E*>(a.dk) + o;
          vrow = static_cast<const E*>(a.dv) + o;
        } else {
          const size_t o = ((size_t)l * a.T + t) * rowHD + (size_t)h * D;
          krow = static_cast<const E*>(a.sk) + o;
          vrow = static_cast<const E*>(a.sv) + o;
        }
      } else {
        const size_t o = (((size_t)i * a.L + l) * a.T + t) * rowHD + (size_t)h * D;
        krow = static_cast<const E*>(a.sk) + o;
        vrow = static_cast<const E*>(a.sv) + o;
      }
#pragma unroll
      for (int k = 0; k < KD; ++k) kop[k] = load8_bf16<E>(krow + 32 * k + 8 * q4);
#pragma unroll
      for (int k = 0; k < KD; ++k)
        *reinterpret_cast<u32x4*>(vt + c16 * VS + 32 * k + 8 * q4) = load8_bf16<E>(vrow + 32 * k + 8 * q4);
      if (MODE == DENSE) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KD; ++k) acc = mfma32(kop[k], qb[k], acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) z[j] = acc[j] * a.scale_log2;
      } else {
        // blocks covering tokens [16 beta, 16 beta + 16): usually one
        const int t0 = beta * kTile;
        int lo = 0, hi = a.B - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (sblk[mid] <= t0) lo = mid; else hi = mid - 1;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) z[j] = -INFINITY;
        for (int b = lo; b < a.B && sblk[b] < t0 + kTile; ++b) {
          if (sblk[b + 1] <= t0) continue;  // empty block
          if (b != bcur) {
            // Q' = R(-Delta(i,b)) q on the lane's pairs (k, k + KD/2)
            const float2* tb = a.tab + ((size_t)i * a.B + b) * HALF;
#pragma unroll
            for (int k = 0; k < KD / 2; ++k) {
              float lo_o[8], hi_o[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const float2 cs = tb[32 * k + 8 * q4 + j];
                const float x = qf[k][j], y = qf[k + KD / 2][j];
                lo_o[j] = x * cs.x + y * cs.y;
                hi_o[j] = y * cs.x - x * cs.y;
              }
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                qr[k][j] = pack_bf16(lo_o[2 * j], lo_o[2 * j + 1]);
                qr[k + KD / 2][j] = pack_bf16(hi_o[2 * j], hi_o[2 * j + 1]);
              }
            }
            bcur = b;
          }
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < KD; ++k) acc = mfma32(kop[k], qr[k], acc);
          const int bs = sblk[b], be = sblk[b + 1];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int tt = t0 + 4 * q4 + j;
            if (tt >= bs && tt < be) z[j] = acc[j] * a.scale_log2;
          }
        }
      }
    }
    wave_sync();  // V tile visible to the whole wave
    softmax_pv<D>(st, z, vt, lane);
    wave_sync();  // done reading before the next tile overwrites it
  }

  // ---- combine the four waves (LDS aliases the V tiles)
  __syncthreads();
  float* cm = reinterpret_cast<float*>(smem);   // [kWaves][16] max
  float* cl = cm + kWaves * 16;                  // [kWaves][16] sum
  float* co = cl + kWaves * 16;                  // [kWaves][16][D]
  float lsum = st.l;
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  if (q4 == 0) {
    cm[wave * 16 + c16] = st.m;
    cl[wave * 16 + c16] = lsum;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) co[((size_t)wave * 16 + c16) * D + dt * 16 + 4 * q4 + j] = st.o[dt][j];
  __syncthreads();
  const size_t rec = D + 4;
  for (int x = tid; x < g * D; x += kThreads) {
    const int r = x / D, d = x % D;
    float mm = -INFINITY;
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, cm[w * 16 + r]);
    float o = 0.f, ls = 0.f;
    if (mm != -INFINITY) {
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(cm[w * 16 + r] - mm);
        o += f * co[((size_t)w * 16 + r) * D + d];
        ls += f * cl[w * 16 + r];
      }
    }
    float* dst = a.part + ((((size_t)i * a.L + l) * a.Hq + (size_t)h * g + r) * a.S + s) * rec;
    dst[4 + d] = o;
    if (d == 0) {
      dst[0] = mm;
      dst[1] = ls;
    }
  }
}

// One wave per output row (agent, layer, query head): combine the splits.
template <typename E, int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part,
                                                   const int32_t* __restrict__ priv_off, int N,
                                                   int L, int Hq, int T, int S, E* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const size_t row = (size_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= (size_t)N * L * Hq) return;
  const int i = (int)(row / ((size_t)L * Hq));
  const int P = priv_off[i + 1] - priv_off[i];
  const int ntiles = (P + kTile - 1) / kTile + T / kTile;
  const int ns = min((ntiles + kTilesPerSplit - 1) / kTilesPerSplit, S);  // S bounds the record
  const size_t rec = D + 4;
  const float* pr = part + row * S * rec;
  float mm = -INFINITY;
  for (int s = 0; s < ns; ++s) mm = fmaxf(mm, pr[s * rec]);
  constexpr int PER = D / kWave;
  float o[PER] = {};
  float ls = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ms = pr[s * rec];
    const float f = (ms == -INFINITY) ? 0.f : exp2f(ms - mm);
    ls += f * pr[s * rec + 1];
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] += f * pr[s * rec + 4 + lane + k * kWave];
  }
  const float inv = ls > 0.f ? 1.0f / ls : 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const float v = o[k] * inv;
    if constexpr (sizeof(E) == 2) {
      out[row * D + lane + k * kWave] = (uint16_t)f32_to_bf16(v);
    } else {
      out[row * D + lane + k * kWave] = v;
    }
  }
}

// ---- dense restore ---------------------------------------------------------------
// One workgroup per (diff block beta, agent i), looping over layers: K rows are
// taken from the diff record or the Master, rotated by Delta(i, b(t)) and
// rounded; V rows are copied.

constexpr int kMaxTileBlocks = kTile;  // a 16-token tile touches at most 16 blocks

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void restore_dense_kernel(
    const E* __restrict__ mk, const E* __restrict__ mv, const int32_t* __restrict__ diff_off,
    const int32_t* __restrict__ diff_idx, const E* __restrict__ dk, const E* __restrict__ dv,
    const int32_t* __restrict__ blk_start, const int32_t* __restrict__ src_pos,
    const int32_t* __restrict__ dst_pos, int N, int B, int T, int L, int Hkv, double theta,
    E* __restrict__ kd, E* __restrict__ vd) {
  constexpr int VEC = Fmt<E>::VEC;
  constexpr int HALF = D / 2;
  constexpr int G = HALF / VEC;
  constexpr int RPP = kThreads / G;
  __shared__ float2 tab[kMaxTileBlocks * HALF];
  __shared__ int s_b0, s_nb;
  __shared__ int32_t sb[kMaxTileBlocks + 1];
  const int beta = blockIdx.x;
  const int i = blockIdx.y;
  const int tid = threadIdx.x;
  const int t0 = beta * kTile;
  if (tid == 0) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (blk_start[mid] <= t0) lo = mid; else hi = mid - 1;
    }
    int nbk = 0;
    for (int b = lo; b < B && blk_start[b] < t0 + kTile; ++b) ++nbk;
    s_b0 = lo;
    s_nb = nbk;
  }
  __syncthreads();
  const int b0 = s_b0, nbk = s_nb;
  for (int x = tid; x <= nbk; x += kThreads) sb[x] = blk_start[b0 + x];
  for (int x = tid; x < nbk * HALF; x += kThreads) {
    const int bb = x / HALF, e = x % HALF;
    const double delta = (double)(dst_pos[(size_t)i * B + b0 + bb] - src_pos[b0 + bb]);
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
      while (bb + 1 < nbk && sb[bb + 1] <= tok) ++bb;
      const size_t off = (size_t)row * D + e0;
      float x[VEC], y[VEC], ox[VEC], oy[VEC];
      Fmt<E>::unpack(ld16(ks + off), x);
      Fmt<E>::unpack(ld16(ks + off + HALF), y);
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float2 cs = tab[bb * HALF + e0 + j];
        ox[j] = x[j] * cs.x - y[j] * cs.y;
        oy[j] = y[j] * cs.x + x[j] * cs.y;
      }
      st16_nt(ko + off, Fmt<E>::pack(ox));
      st16_nt(ko + off + HALF, Fmt<E>::pack(oy));
      st16_nt(vo + off, ld16(vs + off));
      st16_nt(vo + off + HALF, ld16(vs + off + HALF));
    }
  }
}

// ---- host-side planning ------------------------------------------------------------

int max_splits(const Dims& d, int max_priv) {
  const int nt = (max_priv + kTile - 1) / kTile + d.T / kTile;
  return (nt + kTilesPerSplit - 1) / kTilesPerSplit;
}

struct AttnWs {
  size_t part, tab, total;
};

AttnWs attn_ws(const Dims& d, int max_priv, bool fused) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  AttnWs w;
  w.part = 0;
  const size_t nrec = (size_t)d.N * d.L * d.Hq * max_splits(d, max_priv);
  w.tab = up(nrec * (d.D + 4) * 4);
  w.total = w.tab + (fused ? up((size_t)d.N * d.B * (d.D / 2) * 8) : 0);
  return w;
}

size_t attn_lds_bytes(int D, int B, bool fused) {
  const size_t vbytes = (size_t)kWaves * kTile * (D + 8) * 2;
  const size_t cbytes = (size_t)kWaves * 16 * (D + 4) * 4 + 2 * kWaves * 16 * 4;
  return (vbytes > cbytes ? vbytes : cbytes) + (fused ? (size_t)(B + 1) * 4 : 0);
}

template <typename E, int D, int MODE>
hipError_t launch_attn_t(const Dims& d, AttnArgs a, int max_priv, E* out, hipStream_t s) {
  a.S = max_splits(d, max_priv);
  const size_t lds = attn_lds_bytes(D, d.B, MODE == FUSED);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  dim3 grid(d.N, a.S, d.L * d.Hkv);
  hipLaunchKernelGGL((attn_split_kernel<E, D, MODE>), grid, dim3(kThreads), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t rows = (size_t)d.N * d.L * d.Hq;
  const int rpb = 256 / kWave;
  hipLaunchKernelGGL((merge_kernel<E, D>), dim3((rows + rpb - 1) / rpb), dim3(256), 0, s, a.part,
                     a.priv_off, d.N, d.L, d.Hq, d.T, a.S, out);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch_attn(const Dims& d, AttnArgs a, int max_priv, void* out, hipStream_t s) {
  if (d.dtype == TDX_BF16)
    return d.D == 128 ? launch_attn_t<uint16_t, 128, MODE>(d, a, max_priv, static_cast<uint16_t*>(out), s)
                      : launch_attn_t<uint16_t, 64, MODE>(d, a, max_priv, static_cast<uint16_t*>(out), s);
  return d.D == 128 ? launch_attn_t<float, 128, MODE>(d, a, max_priv, static_cast<float*>(out), s)
                    : launch_attn_t<float, 64, MODE>(d, a, max_priv, static_cast<float*>(out), s);
}

AttnArgs common_args(const Dims& d, const void* q, const int32_t* priv_off, const void* pk,
                     const void* pv, float scale, void* ws) {
  AttnArgs a{};
  a.q = q;
  a.priv_off = priv_off;
  a.pk = pk;
  a.pv = pv;
  a.part = static_cast<float*>(ws);
  a.N = d.N;
  a.L = d.L;
  a.T = d.T;
  a.B = d.B;
  a.Hkv = d.Hkv;
  a.Hq = d.Hq;
  a.scale_log2 = scale * kLog2e;
  return a;
}

}  // namespace

size_t restore_attn_ws_bytes(const Dims& d, int max_priv) { return attn_ws(d, max_priv, true).total; }
size_t dense_attn_ws_bytes(const Dims& d, int max_priv) { return attn_ws(d, max_priv, false).total; }

hipError_t launch_restore_attn(const Dims& d, const tdx_layout& lay, const void* q,
                               const int32_t* priv_off, const void* pk, const void* pv,
                               int max_priv, const void* mk, const void* mv,
                               const int32_t* diff_off, const int32_t* diff_idx, const void* dk,
                               const void* dv, float scale, void* out, void* ws, hipStream_t s) {
  const AttnWs w = attn_ws(d, max_priv, true);
  AttnArgs a = common_args(d, q, priv_off, pk, pv, scale, ws);
  a.sk = mk;
  a.sv = mv;
  a.diff_off = diff_off;
  a.diff_idx = diff_idx;
  a.dk = dk;
  a.dv = dv;
  a.blk_start = lay.blk_start;
  float2* tab = reinterpret_cast<float2*>(static_cast<unsigned char*>(ws) + w.tab);
  a.tab = tab;
  const size_t n = (size_t)d.N * d.B * (d.D / 2);
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, s, lay.src_pos, lay.dst_pos,
                     d.N, d.B, d.D, d.theta, tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return dispatch_attn<FUSED>(d, a, max_priv, out, s);
}

hipError_t launch_restore_dense(const Dims& d, const tdx_layout& lay, const void* mk,
                                const void* mv, const int32_t* diff_off,
                                const int32_t* diff_idx, const void* dk, const void* dv,
                                void* kd, void* vd, hipStream_t s) {
  dim3 grid(d.T / kTile, d.N);
#define TDX_RD(E, DD)                                                                          \
  hipLaunchKernelGGL((restore_dense_kernel<E, DD>), grid, dim3(kThreads), 0, s,               \
                     static_cast<const E*>(mk), static_cast<const E*>(mv), diff_off, diff_idx, \
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
  AttnArgs a = common_args(d, q, priv_off, pk, pv, scale, ws);
  a.sk = kd;
  a.sv = vd;
  return dispatch_attn<DENSE>(d, a, max_priv, out, s);
}

}  // namespace tdx

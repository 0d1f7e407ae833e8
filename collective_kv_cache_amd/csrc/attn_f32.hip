// a5 / a6 for fp32 caches: the fused restore + decode attention and the
// dense comparator's attention, computed on the fp32 vector units.
//
// TokenDance notes §3d and §4 ("Fused Diff Restore"), blog §4.4: a Mirror's
// diff blocks are merged into the Master's tiles on chip and RoPE is
// recovered right before attention, with no dense Mirror written; the restore
// gives back the Mirror exactly (notes Figure 8).  The bf16 matrix-core
// kernels take bf16 operands; for fp32 caches that would round K, V, q and
// the softmax weights to 8 significant bits, so fp32 rounds take this path,
// where every operand, product and sum is fp32.
//
// One workgroup per (agent i, layer l, KV head h, key split s).  Agent i's
// key sequence is its private history in tiles of 16 rows, then the T/16
// canonical shared tiles, each exactly one 16-token diff block.  Per tile:
//   - the 256 threads stage the tile's 16 K and V rows of head h in LDS:
//     fused, a shared tile comes from agent i's diff entry when its record
//     holds the block and from the Master otherwise, and its K rows are
//     rotated by R(Delta(i, b(t))) in fp32 with a cos/sin table built in
//     double precision; dense, the materialised rows are used as they are;
//   - thread (query head j = tid / 16, key = tid % 16) forms one logit;
//   - the 16 lanes of query head j update its running maximum and sum;
//   - thread (dim d = tid % D, query heads tid / D + k * 256 / D) adds P V.
// Each split writes (m, l, O) per query head; the merge kernel combines
// the splits of every (agent, layer, query head) and writes the output.
#include "common.h"

namespace tdx {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 16;
constexpr int kMaxG = 16;         // query heads per KV head (checked by the ABI)
constexpr int kTilesPerSplit = 32;

// cos/sin of Delta(i, b) * theta^(-2e/D), evaluated in double, stored as fp32
__global__ __launch_bounds__(256) void f32_rope_table_kernel(const int32_t* __restrict__ src_pos,
                                                             const int32_t* __restrict__ dst_pos, int N, int B,
                                                             int D, double theta, float2* __restrict__ tab) {
  const int half = D / 2;
  const size_t n = (size_t)N * B * half;
  for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(x % half);
    const size_t ib = x / half;
    const int b = (int)(ib % B);
    const double delta = (double)(dst_pos[ib] - src_pos[b]);
    double sn, cs;
    sincos(delta * rope_inv_freq(theta, e, D), &sn, &cs);
    tab[x] = make_float2((float)cs, (float)sn);
  }
}

// Largest b in [0, B) with blk[b] <= t (the block holding t; skips empty blocks)
__device__ __forceinline__ int block_holding(const int32_t* __restrict__ blk, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (blk[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int D, int MODE, bool PAGED>
__global__ __launch_bounds__(kThreads) void f32_attn_kernel(F32AttnArgs a) {
  constexpr int HALF = D / 2;
  constexpr int PPT = HALF / 16;        // rotate-half pairs per staging thread
  constexpr int KS = D + 1;             // padded rows: the logit reads walk one row per lane
  constexpr int HPP = kThreads / D;     // query heads per P V pass
  constexpr int NPV = kMaxG / HPP;      // passes
  __shared__ float qs[kMaxG][KS];
  __shared__ float ks[kTile][KS];
  __shared__ float vs[kTile][D];
  __shared__ float ps[kMaxG][kTile];
  __shared__ float salpha[kMaxG];
  __shared__ float sml[kMaxG][2];

  const int tid = threadIdx.x;
  const int g = a.Hq / a.Hkv;
  const int row = blockIdx.x;  // (i * L + l) * Hkv + h
  const int h = row % a.Hkv;
  const int r = row / a.Hkv;   // (agent, layer) row
  const int i = r / a.L, l = r % a.L;
  const int s = blockIdx.y;
  const int nb = a.T / kTile;
  const int P = min(a.priv_off[i + 1] - a.priv_off[i], a.pmax);
  const int ntp = (P + kTile - 1) / kTile;
  const int u0 = s * kTilesPerSplit, u1 = min(u0 + kTilesPerSplit, ntp + nb);
  const size_t rowHD = (size_t)a.Hkv * D;

  for (int x = tid; x < g * D; x += kThreads)
    qs[x / D][x % D] = a.q[(((size_t)i * a.L + l) * a.Hq + (size_t)h * g + x / D) * D + x % D];

  // logit lanes: query head j, key kk; running state kept by all 16 lanes of j
  const int j = tid / kTile, kk = tid % kTile;
  float m = -INFINITY, lsum = 0.f;
  // P V lanes: dim d, query heads tid / D + p * HPP
  const int d = tid % D, h0 = tid / D;
  float o[NPV];
#pragma unroll
  for (int p = 0; p < NPV; ++p) o[p] = 0.f;

  // staging lanes: key row sr, pairs [sc * PPT, sc * PPT + PPT) and their partners
  const int sr = tid / 16, sc = tid % 16;
  const int mrow = (PAGED && a.msel != nullptr) ? min(max(a.msel[0], 0), a.N - 1) : 0;
  const size_t moff = PAGED ? 0 : master_offset(a.msel, a.mstride, a.N) + (size_t)l * a.T * rowHD;
  const int e0 = MODE == FUSED ? a.diff_off[r] : 0;
  const int ne = MODE == FUSED ? min(max(a.diff_off[r + 1] - e0, 0), nb) : 0;
  const size_t ptot = (size_t)a.priv_off[a.N];

  for (int u = u0; u < u1; ++u) {
    // ---- stage tile u: rows of head h, K rotated where it is a shared key
    const float* ksrc = nullptr;
    const float* vsrc = nullptr;
    bool valid = true, rot = false;
    int t = 0;  // canonical token (shared tiles)
    if (u < ntp) {
      const int x = u * kTile + sr;
      valid = x < P;
      const size_t prow = PAGED ? ((size_t)l * a.ppm.n_pages + page_at(a.ppm, i, u)) * kTile + sr
                                : (size_t)l * ptot + a.priv_off[i] + x;
      ksrc = a.pk + prow * rowHD + (size_t)h * D;
      vsrc = a.pv + prow * rowHD + (size_t)h * D;
    } else {
      const int beta = u - ntp;
      t = beta * kTile + sr;
      if (MODE == DENSE) {
        const size_t o2 = (((size_t)i * a.L + l) * a.T + t) * rowHD + (size_t)h * D;
        ksrc = a.sk + o2;
        vsrc = a.sv + o2;
      } else {
        rot = true;
        // agent i's diff entry of block beta (ascending indices), or -1
        int lo = 0, hi = ne;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (a.diff_idx[e0 + mid] < beta) lo = mid + 1; else hi = mid;
        }
        const int e = (lo < ne && a.diff_idx[e0 + lo] == beta) ? e0 + lo : -1;
        size_t src;
        if (e >= 0) {
          src = PAGED ? ((size_t)l * a.dpm.n_pages + page_at(a.dpm, 0, e)) * kTile + sr
                      : (size_t)e * kTile + sr;
          ksrc = a.dk + src * rowHD + (size_t)h * D;
          vsrc = a.dv + src * rowHD + (size_t)h * D;
        } else {
          src = PAGED ? ((size_t)l * a.mpm.n_pages + page_at(a.mpm, mrow, beta)) * kTile + sr : (size_t)t;
          ksrc = a.sk + moff + src * rowHD + (size_t)h * D;
          vsrc = a.sv + moff + src * rowHD + (size_t)h * D;
        }
      }
    }
    const float2* cs = nullptr;
    if (rot) cs = a.tab + ((size_t)i * a.B + block_holding(a.blk_start, a.B, t)) * HALF;
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
      const int e = sc * PPT + q;
      float kx = 0.f, ky = 0.f, vx = 0.f, vy = 0.f;
      if (valid) {
        kx = ksrc[e];
        ky = ksrc[e + HALF];
        vx = vsrc[e];
        vy = vsrc[e + HALF];
        if (rot) {
          const float2 c = cs[e];
          const float x0 = kx, y0 = ky;
          kx = x0 * c.x - y0 * c.y;
          ky = y0 * c.x + x0 * c.y;
        }
      }
      ks[sr][e] = kx;
      ks[sr][e + HALF] = ky;
      vs[sr][e] = vx;
      vs[sr][e + HALF] = vy;
    }
    const int nvalid = u < ntp ? min(kTile, P - u * kTile) : kTile;
    __syncthreads();

    // ---- logits and the running softmax state of query head j
    if (j < g) {
      float z = 0.f;
#pragma unroll 8
      for (int e = 0; e < D; ++e) z = fmaf(qs[j][e], ks[kk][e], z);
      z = kk < nvalid ? z * a.scale_log2 : -INFINITY;
      float tmax = z;
#pragma unroll
      for (int o2 = 8; o2 > 0; o2 >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o2, 16));
      const float mnew = fmaxf(m, tmax);
      const float ref = mnew == -INFINITY ? 0.f : mnew;
      const float p = exp2f(z - ref);
      const float alpha = exp2f(m - ref);
      float psum = p;
#pragma unroll
      for (int o2 = 8; o2 > 0; o2 >>= 1) psum += __shfl_xor(psum, o2, 16);
      lsum = lsum * alpha + psum;
      m = mnew;
      ps[j][kk] = p;
      if (kk == 0) salpha[j] = alpha;
    }
    __syncthreads();

    // ---- O = O * alpha + P V
#pragma unroll
    for (int p = 0; p < NPV; ++p) {
      const int hq = h0 + p * HPP;
      if (hq < g) {
        float acc = o[p] * salpha[hq];
#pragma unroll
        for (int k2 = 0; k2 < kTile; ++k2) acc = fmaf(ps[hq][k2], vs[k2][d], acc);
        o[p] = acc;
      }
    }
    __syncthreads();
  }

  // ---- this split's record per query head: m, l, -, -, O[D]
  if (j < g && kk == 0) {
    sml[j][0] = m;
    sml[j][1] = lsum;
  }
  __syncthreads();
  const int S = gridDim.y;
#pragma unroll
  for (int p = 0; p < NPV; ++p) {
    const int hq = h0 + p * HPP;
    if (hq < g) {
      float* rec = a.part + (((size_t)r * a.Hq + (size_t)h * g + hq) * S + s) * (D + 4);
      rec[4 + d] = o[p];
      if (d == 0) {
        rec[0] = sml[hq][0];
        rec[1] = sml[hq][1];
      }
    }
  }
}

// One wave per output row (agent, layer, query head): combine its S records.
template <int D>
__global__ __launch_bounds__(256) void f32_merge_kernel(const float* __restrict__ part, int rows, int S,
                                                        float* __restrict__ out) {
  constexpr int PER = D / kWave;
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const float* pr = part + (size_t)row * S * (D + 4);
  float mm = -INFINITY;
  for (int x = lane; x < S; x += kWave) mm = fmaxf(mm, pr[(size_t)x * (D + 4)]);
#pragma unroll
  for (int o2 = kWave / 2; o2 > 0; o2 >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o2, kWave));
  float acc[PER] = {};
  float ls = 0.f;
  for (int x = 0; x < S; ++x) {
    const float* rec = pr + (size_t)x * (D + 4);
    const float f = rec[0] == -INFINITY ? 0.f : exp2f(rec[0] - mm);
    ls += f * rec[1];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] += f * rec[4 + lane + k * kWave];
  }
  const float inv = ls > 0.f ? 1.0f / ls : 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) out[(size_t)row * D + lane + k * kWave] = acc[k] * inv;
}

struct F32Plan {
  int S;
  size_t part_bytes, tab_off, total;
};

F32Plan f32_plan(const Dims& d, int max_priv, bool fused) {
  F32Plan p{};
  const int tiles = (max_priv + kTile - 1) / kTile + d.T / kTile;
  p.S = (tiles + kTilesPerSplit - 1) / kTilesPerSplit;
  if (p.S < 1) p.S = 1;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.part_bytes = (size_t)d.N * d.L * d.Hq * p.S * (d.D + 4) * 4;
  p.tab_off = up(p.part_bytes);
  p.total = p.tab_off + (fused ? up((size_t)d.N * d.B * (d.D / 2) * 8) : 0);
  return p;
}

template <int D, int MODE, bool PAGED>
hipError_t launch_d(const Dims& d, F32AttnArgs a, const F32Plan& p, hipStream_t s) {
  hipLaunchKernelGGL((f32_attn_kernel<D, MODE, PAGED>), dim3(d.N * d.L * d.Hkv, p.S), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = d.N * d.L * d.Hq;
  hipLaunchKernelGGL((f32_merge_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, s, a.part, rows, p.S, a.out);
  return hipGetLastError();
}

}  // namespace

size_t f32_attn_ws_bytes(const Dims& d, int max_priv, bool fused) { return f32_plan(d, max_priv, fused).total; }

hipError_t launch_attn_f32(const Dims& d, int mode, bool paged, F32AttnArgs a, int max_priv, void* ws,
                           hipStream_t s) {
  static_assert(FUSED == 0 && DENSE == 1, "modes");
  const F32Plan p = f32_plan(d, max_priv, mode == FUSED);
  a.part = static_cast<float*>(ws);
  a.N = d.N;
  a.L = d.L;
  a.T = d.T;
  a.B = d.B;
  a.Hkv = d.Hkv;
  a.Hq = d.Hq;
  a.pmax = max_priv;
  if (mode == FUSED) {
    float2* tab = reinterpret_cast<float2*>(static_cast<unsigned char*>(ws) + p.tab_off);
    const size_t n = (size_t)d.N * d.B * (d.D / 2);
    const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(f32_rope_table_kernel, dim3(blocks), dim3(256), 0, s, a.src_pos, a.dst_pos, d.N, d.B, d.D,
                       d.theta, tab);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.tab = tab;
  }
  if (mode == DENSE) return d.D == 128 ? launch_d<128, DENSE, false>(d, a, p, s) : launch_d<64, DENSE, false>(d, a, p, s);
  if (paged) return d.D == 128 ? launch_d<128, FUSED, true>(d, a, p, s) : launch_d<64, FUSED, true>(d, a, p, s);
  return d.D == 128 ? launch_d<128, FUSED, false>(d, a, p, s) : launch_d<64, FUSED, false>(d, a, p, s);
}

}  // namespace tdx

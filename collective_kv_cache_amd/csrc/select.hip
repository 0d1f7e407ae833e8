// a2 + a3: check-layer key difference, one important-position set, Master.
//
// TokenDance notes, Summary "Method": the N requests' K at the check layer
// are batched for ONE key-difference analysis; the important positions it
// selects are reused by all later layers (§3c A3); the agent with the least
// deviation becomes the Master (§3c A2).
//
// Kernels:
//  deviation_kernel  one wave per canonical token: for each agent the lanes
//                    stream the (reused, recomputed) K rows with 16-byte loads,
//                    square-sum in double, reduce each head with xor shuffles,
//                    take the per-head norm and add the heads.  The wave sums
//                    its token over agents in index order (score) and writes
//                    per-workgroup agent partials for the Master total.
//  select_kernel     one 1024-thread workgroup: fixed-order agent totals and
//                    argmin, 4-pass 8-bit radix select of the k-th largest
//                    fp32 score bit pattern, then an ordered ballot compaction
//                    that takes ties in ascending token order.
#include "common.h"

namespace tdx {
namespace {

constexpr int kDevThreads = 256;
constexpr int kDevWaves = kDevThreads / kWave;
constexpr int kTokPerWave = 2;
constexpr int kTokPerWg = kDevWaves * kTokPerWave;
constexpr int kAgentUnroll = 4;
constexpr int kSelThreads = 1024;
constexpr int kMaxAgents = 1024;

__device__ __forceinline__ double wave_sum_xor(double v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// KCH = 16-byte chunks per lane per row (row = Hkv * D elements).
template <typename E, int D, int KCH>
__global__ __launch_bounds__(kDevThreads) void deviation_kernel(
    const E* __restrict__ kr, const E* __restrict__ kx, int N, int T, int Hkv,
    size_t kr_agent_stride, float* __restrict__ dev, float* __restrict__ score,
    double* __restrict__ part) {
  constexpr int VEC = Fmt<E>::VEC;
  constexpr int G = D / VEC;  // lanes per head
  extern __shared__ double wsum_dyn[];  // [kDevWaves][N] per-wave agent sums
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int rowE = Hkv * D;
  const int cpr = rowE / VEC;  // chunks per row
  double* wsum = wsum_dyn + (size_t)wave * N;

  for (int i = lane; i < N; i += kWave) wsum[i] = 0.0;
  __syncthreads();

  for (int j = 0; j < kTokPerWave; ++j) {
    const int t = blockIdx.x * kTokPerWg + wave * kTokPerWave + j;
    if (t >= T) break;  // uniform within the wave
    double s_t = 0.0;
    for (int i0 = 0; i0 < N; i0 += kAgentUnroll) {
      u32x4 a[kAgentUnroll][KCH], b[kAgentUnroll][KCH];
#pragma unroll
      for (int u = 0; u < kAgentUnroll; ++u) {
        const int i = i0 + u;
#pragma unroll
        for (int k = 0; k < KCH; ++k) {
          const int c = lane + k * kWave;
          if (i < N && c < cpr) {
            a[u][k] = ld16(kr + (size_t)i * kr_agent_stride + (size_t)t * rowE + c * VEC);
            b[u][k] = ld16(kx + ((size_t)i * T + t) * rowE + c * VEC);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kAgentUnroll; ++u) {
        const int i = i0 + u;
        if (i >= N) break;
        double d_it = 0.0;
#pragma unroll
        for (int k = 0; k < KCH; ++k) {
          const int c = lane + k * kWave;
          double ss = 0.0;
          if (c < cpr) {
            float x[VEC], y[VEC];
            Fmt<E>::unpack(a[u][k], x);
            Fmt<E>::unpack(b[u][k], y);
#pragma unroll
            for (int q = 0; q < VEC; ++q) {
              const double df = (double)y[q] - (double)x[q];
              ss = fma(df, df, ss);
            }
          }
          ss = wave_sum_xor(ss, G);  // every lane of a head holds the head's sum
          const bool leader = (lane % G) == 0 && c < cpr;
          d_it += leader ? sqrt(ss) : 0.0;
        }
        d_it = wave_sum_xor(d_it, kWave);  // add the heads
        s_t += d_it;
        if (lane == 0) {
          dev[(size_t)i * T + t] = (float)d_it;
          wsum[i] += d_it;
        }
      }
    }
    if (lane == 0) score[t] = (float)s_t;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += kDevThreads) {
    double acc = 0.0;
    for (int w = 0; w < kDevWaves; ++w) acc += wsum_dyn[(size_t)w * N + i];
    part[(size_t)blockIdx.x * N + i] = acc;
  }
}

// Inclusive wave prefix of a predicate via ballot; returns count of set lanes
// strictly below this lane and writes the wave total.
__device__ __forceinline__ int wave_rank(bool p, int lane, int* total) {
  const uint64_t m = __ballot(p);
  *total = __popcll(m);
  return __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ score, const double* __restrict__ part, int nparts, int N, int T,
    int k, float* __restrict__ agent_dev, int32_t* __restrict__ selected,
    int32_t* __restrict__ master) {
  constexpr int W = kSelThreads / kWave;
  __shared__ float s_adev[kMaxAgents];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_need;
  __shared__ int s_wcnt[2][W];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;

  // ---- agent totals (fixed order: lane-strided partials, xor tree) and Master
  for (int i = wave; i < N; i += W) {
    double acc = 0.0;
    for (int p = lane; p < nparts; p += kWave) acc += part[(size_t)p * N + i];
    acc = wave_sum_xor(acc, kWave);
    if (lane == 0) {
      const float a = (float)acc;
      agent_dev[i] = a;
      s_adev[i] = a;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int best = 0;
    for (int i = 1; i < N; ++i)
      if (s_adev[i] < s_adev[best]) best = i;
    master[0] = best;
  }

  // ---- radix select of the k-th largest key (scores are >= 0, so the fp32
  // bit pattern orders like the value)
  uint32_t prefix = 0, mask = 0, need = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int x = tid; x < 256; x += kSelThreads) hist[x] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += kSelThreads) {
      const uint32_t u = __float_as_uint(score[t]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns digits 4*lane .. 4*lane+3; suffix sums from the top digit
      uint32_t h[4], own = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[q] = hist[4 * lane + q];
        own += h[q];
      }
      // keys whose digit belongs to a higher lane (exclusive suffix sum)
      uint32_t above = 0;
      for (int src = kWave - 1; src > 0; --src) {
        const uint32_t v = __shfl(own, src, kWave);
        if (src > lane) above += v;
      }
      // digit d crosses when above + sum_{q > d} h[q] < need <= ... + h[d]
      uint32_t run = above;
      int found = -1;
      uint32_t need_in = 0;
      for (int q = 3; q >= 0; --q) {
        if (found < 0 && run < need && need <= run + h[q]) {
          found = 4 * lane + q;
          need_in = need - run;
        }
        run += h[q];
      }
      const uint64_t m = __ballot(found >= 0);
      const int src = __ffsll((unsigned long long)m) - 1;
      const int digit = __shfl(found, src, kWave);
      const uint32_t nin = __shfl(need_in, src, kWave);
      if (lane == 0) {
        s_prefix = prefix | ((uint32_t)digit << shift);
        s_need = nin;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    mask |= 255u << shift;
    __syncthreads();
  }

  // ---- ordered compaction: every key > thr, and the first `need` keys == thr
  const uint32_t thr = prefix;
  int carry_eq = 0, carry_sel = 0;
  for (int base = 0; base < T; base += kSelThreads) {
    const int t = base + tid;
    const bool valid = t < T;
    const uint32_t u = valid ? __float_as_uint(score[t]) : 0u;
    const bool gt = valid && u > thr;
    const bool eq = valid && u == thr;
    int tot_eq, tot_sel;
    const int r_eq = wave_rank(eq, lane, &tot_eq);
    if (lane == 0) s_wcnt[0][wave] = tot_eq;
    __syncthreads();
    int pre_eq = carry_eq, all_eq = carry_eq;
    for (int w = 0; w < W; ++w) {
      if (w < wave) pre_eq += s_wcnt[0][w];
      all_eq += s_wcnt[0][w];
    }
    const bool sel = gt || (eq && (uint32_t)(pre_eq + r_eq) < need);
    const int r_sel = wave_rank(sel, lane, &tot_sel);
    if (lane == 0) s_wcnt[1][wave] = tot_sel;
    __syncthreads();
    int pre_sel = carry_sel, all_sel = carry_sel;
    for (int w = 0; w < W; ++w) {
      if (w < wave) pre_sel += s_wcnt[1][w];
      all_sel += s_wcnt[1][w];
    }
    if (sel && pre_sel + r_sel < k) selected[pre_sel + r_sel] = t;
    carry_eq = all_eq;
    carry_sel = all_sel;
    __syncthreads();
  }
}

template <typename E, int D, int KCH>
hipError_t launch_dev(const Dims& d, int check_layer, const void* kr, const void* kx,
                      float* dev, float* score, double* part, int nparts, hipStream_t s) {
  const size_t rowE = (size_t)d.Hkv * d.D;
  const size_t stride = (size_t)d.L * d.T * rowE;
  const E* krl = static_cast<const E*>(kr) + (size_t)check_layer * d.T * rowE;
  hipLaunchKernelGGL((deviation_kernel<E, D, KCH>), dim3(nparts), dim3(kDevThreads),
                     kDevWaves * d.N * sizeof(double), s, krl,
                     static_cast<const E*>(kx), d.N, d.T, d.Hkv, stride, dev, score, part);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_dev_d(const Dims& d, int check_layer, const void* kr, const void* kx,
                        float* dev, float* score, double* part, int nparts, hipStream_t s) {
  const int cpr = d.Hkv * D / Fmt<E>::VEC;
  const int kch = (cpr + kWave - 1) / kWave;
  switch (kch) {
    case 1: return launch_dev<E, D, 1>(d, check_layer, kr, kx, dev, score, part, nparts, s);
    case 2: return launch_dev<E, D, 2>(d, check_layer, kr, kx, dev, score, part, nparts, s);
    case 3:
    case 4: return launch_dev<E, D, 4>(d, check_layer, kr, kx, dev, score, part, nparts, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

static int dev_parts(const Dims& d) { return (d.T + kTokPerWg - 1) / kTokPerWg; }

size_t select_ws_bytes(const Dims& d) {
  return (size_t)dev_parts(d) * d.N * sizeof(double);
}

hipError_t launch_select(const Dims& d, const tdx_layout& lay, int check_layer,
                         const void* k_reuse, const void* k_recomp, int k, float* dev,
                         float* score, float* agent_dev, int32_t* selected, int32_t* master,
                         void* ws, hipStream_t s) {
  (void)lay;
  if (d.N > kMaxAgents) return hipErrorInvalidValue;
  const int nparts = dev_parts(d);
  double* part = static_cast<double*>(ws);
  hipError_t e;
  if (d.dtype == TDX_BF16)
    e = d.D == 128 ? launch_dev_d<uint16_t, 128>(d, check_layer, k_reuse, k_recomp, dev, score, part, nparts, s)
                   : launch_dev_d<uint16_t, 64>(d, check_layer, k_reuse, k_recomp, dev, score, part, nparts, s);
  else
    e = d.D == 128 ? launch_dev_d<float, 128>(d, check_layer, k_reuse, k_recomp, dev, score, part, nparts, s)
                   : launch_dev_d<float, 64>(d, check_layer, k_reuse, k_recomp, dev, score, part, nparts, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel, dim3(1), dim3(kSelThreads), 0, s, score, part, nparts, d.N,
                     d.T, k, agent_dev, selected, master);
  return hipGetLastError();
}

}  // namespace tdx

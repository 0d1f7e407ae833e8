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
//                    square-sum in fp32, sum each head's lanes with DPP, take
//                    the per-head norm and add the heads.  The wave sums its
//                    token over agents in index order (score) and writes
//                    per-workgroup agent partials for the Master total.
//  select_kernel     two 1024-thread workgroups side by side: one runs an 8-bit
//                    radix select of the k-th largest fp32 score bit pattern
//                    from the highest bit in which the non-zero scores differ
//                    (no pass when the set takes every non-zero score, fewer
//                    once the k-th key's bin is taken whole), then an ordered
//                    compaction by one scan that takes ties in ascending token
//                    order; the other sums the agent totals in a fixed order
//                    and takes their argmin.
#include "common.h"

namespace tdx {
namespace {

// deviation_kernel workgroups: 8 waves (one token each) when every token's
// wave can be resident at once, else 4.  With 8, a workgroup reads 8
// consecutive rows of every agent and the selection sums half as many
// per-workgroup partials (64 agents: 692 instead of 1384 rows of N doubles).
constexpr int kDevMaxThreads = 512;
constexpr int kDevMinWaves = 4;
constexpr int kSelThreads = 1024;
constexpr int kMaxAgents = 1024;
constexpr int kSelLdsKeys = 12288;  // scores kept in LDS up to this many tokens

__device__ __forceinline__ double wave_sum_xor(double v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// DPP lane moves within a 16-lane row (VALU, no LDS round trip)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of G lanes (G = 8, 16 or 32), result in every lane
// of the group; a fixed butterfly, so the order of the additions is fixed.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror: groups of 8
  if constexpr (G >= 16) v += dpp<0x140>(v);  // row_mirror: groups of 16
  if constexpr (G >= 32) v += __shfl_xor(v, 16, kWave);
  return v;
}

// One wave per canonical token t: for every agent, the lanes stream the
// (reused, recomputed) K rows with 16-byte loads (all agents of a group of
// AU in flight together), square-sum each lane's elements in fp32,
// sum each head's lanes with DPP, take the head norms and add the heads.
// KCH = 16-byte chunks per lane per row (row = Hkv * D elements).
//
// PAGED: the reused K lives in 16-token pages of a pool; agent i's token t is
// row t % 16 of page pm[i][t / 16] at layer pl (kr is the pool).
template <typename E, int D, int KCH, int AU, bool PAGED>
__global__ __launch_bounds__(kDevMaxThreads) void deviation_kernel(
    const E* __restrict__ kr, const E* __restrict__ kx, int N, int T, int Hkv,
    size_t kr_agent_stride, float* __restrict__ dev, float* __restrict__ score,
    double* __restrict__ part, PageMap pm, long long pl) {
  constexpr int VEC = Fmt<E>::VEC;
  constexpr int G = D / VEC;  // lanes per head
  static_assert(G == 8 || G == 16 || G == 32, "lanes per head");
  extern __shared__ float wsum_dyn[];  // [waves][N] the wave's token's deviation per agent
  const int nw = blockDim.x / kWave;   // waves = tokens per workgroup
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int rowE = Hkv * D;
  const int cpr = rowE / VEC;  // chunks per row
  float* wsum = wsum_dyn + (size_t)wave * N;
  for (int i = lane; i < N; i += kWave) wsum[i] = 0.0f;
  __syncthreads();

  const int t = blockIdx.x * nw + wave;
  const bool live = t < T;  // uniform within the wave
  const int tc = live ? t : T - 1;
  double s_t = 0.0;
  for (int i0 = 0; i0 < N; i0 += AU) {
    u32x4 a[AU][KCH], b[AU][KCH];
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int i = min(i0 + u, N - 1);  // past N: re-read the last agent (unused)
#pragma unroll
      for (int k = 0; k < KCH; ++k) {
        const int c = min(lane + k * kWave, cpr - 1);
        const size_t ra = PAGED ? ((size_t)(pl * pm.n_pages + page_at(pm, i, tc / kBlock)) * kBlock + tc % kBlock) * rowE
                                : (size_t)i * kr_agent_stride + (size_t)tc * rowE;
        a[u][k] = ld16_nt(kr + ra + c * VEC);
        b[u][k] = ld16_nt(kx + ((size_t)i * T + tc) * rowE + c * VEC);
      }
    }
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int i = i0 + u;
      float d_it = 0.0f;
#pragma unroll
      for (int k = 0; k < KCH; ++k) {
        float x[VEC], y[VEC];
        Fmt<E>::unpack(a[u][k], x);
        Fmt<E>::unpack(b[u][k], y);
        float ss = 0.0f;
#pragma unroll
        for (int q = 0; q < VEC; ++q) {
          const float df = y[q] - x[q];
          ss = fmaf(df, df, ss);
        }
        const float nh = sqrtf(group_sum<G>(ss));  // this lane's head norm
        // add the norms of the heads covered by chunk k (one lane per head)
#pragma unroll
        for (int hl = 0; hl < kWave; hl += G) {
          if (hl + k * kWave < cpr) d_it += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(nh), hl));
        }
      }
      if (i < N) {  // uniform
        s_t += (double)d_it;
        if (lane == 0 && live) {
          dev[(size_t)i * T + t] = d_it;
          wsum[i] = d_it;
        }
      }
    }
  }
  if (lane == 0 && live) score[t] = (float)s_t;
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    double acc = 0.0;
    for (int w = 0; w < nw; ++w) acc += (double)wsum_dyn[(size_t)w * N + i];
    part[(size_t)blockIdx.x * N + i] = acc;
  }
}

// DPP moves of a 32-bit value within rows of 16 lanes; lanes whose source
// lies outside the row, or outside row_mask's rows, read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the wave's 64 lanes: a Hillis-Steele scan inside
// each row of 16 (row_shr 1, 2, 4, 8), then row 1 and 3 add the last lane of
// the row before (row_bcast:15) and rows 2 and 3 add lane 31 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_u<0x111>(x);
  x += dpp_u<0x112>(x);
  x += dpp_u<0x114>(x);
  x += dpp_u<0x118>(x);
  x += dpp_u<0x142, 0xA>(x);
  x += dpp_u<0x143, 0xC>(x);
  return x;
}

// Wave-wide max, min or sum of a 32-bit value, the same in every lane: a DPP
// butterfly inside each row of 16 (quad_perm [1,0,3,2], [2,3,0,1],
// row_half_mirror, row_mirror), then the four rows' results by readlane.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
  v = op(v, dpp_u<0xB1>(v));
  v = op(v, dpp_u<0x4E>(v));
  v = op(v, dpp_u<0x141>(v));
  v = op(v, dpp_u<0x140>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(r0, r1), op(r2, r3));
}

// Exclusive prefix over the wave of two counters at once (the lanes below this
// one) and the two wave totals.
__device__ __forceinline__ void wave_excl2(uint32_t a, uint32_t b, uint32_t* ea, uint32_t* eb, uint32_t* ta,
                                           uint32_t* tb) {
  const uint32_t ia = wave_incl_scan(a);
  const uint32_t ib = wave_incl_scan(b);
  *ea = ia - a;
  *eb = ib - b;
  *ta = (uint32_t)__builtin_amdgcn_readlane((int)ia, kWave - 1);
  *tb = (uint32_t)__builtin_amdgcn_readlane((int)ib, kWave - 1);
}

// Workgroup 0 of select_kernel: the k largest scores (ties to the lower
// token), written in ascending token order.
//
// KEYS_IN_LDS = 1: the scores fit in LDS (T <= kSelLdsKeys) and are read from
// there; 0: from global memory.  A compile-time choice, so every key read has
// one address space (a pointer that may be either makes each read wait for all
// outstanding loads).
template <int KEYS_IN_LDS>
__device__ __forceinline__ void topk_role(const float* __restrict__ score, int T, int k,
                                          int32_t* __restrict__ selected, uint32_t* s_key) {
  constexpr int W = kSelThreads / kWave;
  constexpr int KPT = kSelLdsKeys / kSelThreads;  // keys per thread when the scores fit in LDS
  __shared__ uint32_t hist[2][256];  // radix histograms, alternating between passes
  __shared__ uint32_t s_prefix, s_need, s_done;
  __shared__ uint32_t s_wtot[2][W];
  __shared__ uint32_t s_wmax[W], s_wmin[W], s_wnz[W];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  // the scores (>= 0, so their fp32 bit patterns order like the values)
  constexpr bool in_lds = KEYS_IN_LDS != 0;
  const uint32_t* sbits = reinterpret_cast<const uint32_t*>(score);
  const uint32_t* key = in_lds ? s_key : sbits;
  // the largest key, the smallest non-zero key and the count of non-zero keys
  uint32_t kmax = 0, kmin = 0xffffffffu, nz = 0;
  auto take = [&](int t, uint32_t u) {
    if (t < T) {
      kmax = max(kmax, u);
      if (u != 0) {
        kmin = min(kmin, u);
        ++nz;
      }
    }
  };
  if constexpr (in_lds) {
    // the launch gives room for kSelLdsKeys keys: slots past T get copies of
    // the last score and are never read
    uint32_t kreg[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) kreg[u] = sbits[min(tid + u * kSelThreads, T - 1)];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      s_key[tid + u * kSelThreads] = kreg[u];
      take(tid + u * kSelThreads, kreg[u]);
    }
  } else {
    for (int t = tid; t < T; t += kSelThreads) take(t, sbits[t]);
  }
  kmax = wave_reduce(kmax, [](uint32_t x, uint32_t y) { return max(x, y); });
  kmin = wave_reduce(kmin, [](uint32_t x, uint32_t y) { return min(x, y); });
  nz = wave_reduce(nz, [](uint32_t x, uint32_t y) { return x + y; });
  if (lane == 0) {
    s_wmax[wave] = kmax;
    s_wmin[wave] = kmin;
    s_wnz[wave] = nz;
  }
  for (int x = tid; x < 2 * 256; x += kSelThreads) hist[x / 256][x % 256] = 0;
  __syncthreads();
  kmax = 0;
  kmin = 0xffffffffu;
  nz = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    kmax = max(kmax, s_wmax[w]);
    kmin = min(kmin, s_wmin[w]);
    nz += s_wnz[w];
  }

  // ---- the k-th largest key by radix select, 8 bits per pass from the
  // highest bit in which the non-zero keys differ (the bits above it are the
  // same in all of them, and the zero keys rank below them).  A pass narrows
  // the keys to those sharing the k-th largest key's leading bits (prefix
  // under mask); `need` of them still belong to the set.  Once the k-th
  // key's bin holds exactly `need` keys, every key of the bin belongs to the
  // set and the remaining passes are skipped.  With k above the count of
  // non-zero keys the threshold is 0: every non-zero key and the lowest
  // k - nz zero keys; with all non-zero keys equal it is their value.
  uint32_t prefix, mask = 0xffffffffu, need;
  int hb = -1;  // highest differing bit of the non-zero keys, -1: no passes
  if ((uint32_t)k > nz) {
    prefix = 0;
    need = (uint32_t)k - nz;
  } else if (kmin == kmax) {
    prefix = kmax;
    need = (uint32_t)k;
  } else {
    hb = 31 - __builtin_clz(kmin ^ kmax);  // <= 30: the keys' sign bits are 0
    mask = ~((2u << hb) - 1u);
    prefix = kmax & mask;
    need = (uint32_t)k;
  }
  // a pass's digit is bits [sh, sh + 8) with sh = max(hb - 7 - 8 pass, 0);
  // when sh is clamped to 0 the digit also holds bits already resolved,
  // which the keys still in play share, so it ranks them the same way
  for (int pass = 0, sh = hb - 7; hb >= 0; ++pass, sh -= 8) {
    const int s0 = max(sh, 0);
    uint32_t* h = hist[pass & 1];
    for (int base = 0; base < T; base += kSelThreads) {
      const int t = base + tid;
      const uint32_t u = key[min(t, T - 1)];
      bool pend = t < T && (u & mask) == prefix;
      const uint32_t dg = (u >> s0) & 255u;
      // the wave's first pending digit with one atomic for all its lanes
      // (the common case of many equal digits), the others one per lane
      const uint64_t act = __ballot(pend);
      if (act) {
        const int ld = __builtin_ctzll(act);
        const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)dg, ld);
        const uint64_t m = __ballot(pend && dg == d0);
        if (lane == ld) atomicAdd(&h[d0], (uint32_t)__popcll(m));
        if (pend && dg != d0) atomicAdd(&h[dg], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns digits 4*lane .. 4*lane+3 (read, then cleared for the pass
      // after next)
      uint32_t hv[4], own = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hv[q] = h[4 * lane + q];
        h[4 * lane + q] = 0;
        own += hv[q];
      }
      // keys in the digits of the lanes above this one: the wave total less
      // the inclusive prefix sum up to this lane
      const uint32_t pre = wave_incl_scan(own);
      uint32_t run = (uint32_t)__builtin_amdgcn_readlane((int)pre, kWave - 1) - pre;  // lanes > lane
      // digit d crosses when run + sum_{q > d} hv[q] < need <= ... + hv[d]
      int found = -1;
      uint32_t need_in = 0, cnt = 0;
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        if (found < 0 && run < need && need <= run + hv[q]) {
          found = 4 * lane + q;
          need_in = need - run;
          cnt = hv[q];
        }
        run += hv[q];
      }
      if (found >= 0) {  // exactly one lane
        s_prefix = prefix | ((uint32_t)found << s0);
        s_need = need_in;
        s_done = need_in == cnt;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    mask |= 255u << s0;
    if (s_done || s0 == 0) break;  // uniform: read after the barrier by every thread
  }

  // ---- ordered compaction in one scan.  Thread j owns the contiguous run of
  // tokens [j*C, j*C + C).  A key whose leading bits (under mask) exceed the
  // prefix is selected, and the first `need` keys whose leading bits equal it
  // in token order; so a selected token's slot is (keys above before it) +
  // min(keys equal before it, need), and one exclusive scan of the two
  // per-run counts places every token.  With all bits resolved these are the
  // keys above the k-th and the lowest tokens tied with it; after an early
  // stop every key of the k-th key's bin is selected.
  const uint32_t thr = prefix;
  const int C = (T + kSelThreads - 1) / kSelThreads;
  const int t0 = min(tid * C, T), t1 = min(t0 + C, T);
  uint32_t ngt = 0, neq = 0;
  for (int t = t0; t < t1; ++t) {
    const uint32_t u = key[t] & mask;
    ngt += u > thr;
    neq += u == thr;
  }
  uint32_t egt, eeq, wgt, weq;
  wave_excl2(ngt, neq, &egt, &eeq, &wgt, &weq);
  if (lane == 0) {
    s_wtot[0][wave] = wgt;
    s_wtot[1][wave] = weq;
  }
  __syncthreads();
  for (int w = 0; w < wave; ++w) {
    egt += s_wtot[0][w];
    eeq += s_wtot[1][w];
  }
  for (int t = t0; t < t1; ++t) {
    const uint32_t u = key[t] & mask;
    if (u > thr) {
      const uint32_t pos = egt + min(eeq, need);
      if (pos < (uint32_t)k) selected[pos] = t;
      ++egt;
    } else if (u == thr) {
      if (eeq < need && egt + eeq < (uint32_t)k) selected[egt + eeq] = t;
      ++eeq;
    }
  }
}

// Workgroup 1 of select_kernel: agent totals D_i = sum over the deviation
// pass's per-workgroup partials, then the Master (argmin, ties to the lower
// index).  Thread (slice j, agent i) sums the partials p = j, j + S, ... of
// agent i in that order (S = 1024 / N slices), PB loads in flight (PB at
// least the thread's count where that fits, so one round trip serves it);
// agent i's S slice sums are then added by one wave (lane l takes slices l,
// l + 64, ... in order, then a fixed butterfly) when there are 8 or more,
// else by one thread in slice order, so the order of every addition is fixed.
template <int PB>
__device__ __forceinline__ void totals_role(const double* __restrict__ part, int nparts, int N,
                                            float* __restrict__ agent_dev, int32_t* __restrict__ master) {
  constexpr int W = kSelThreads / kWave;
  __shared__ float s_adev[kMaxAgents];
  __shared__ double s_at[kSelThreads];  // [S][N] slice sums
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int S = kSelThreads / N;  // N <= 1024
  const int ai = tid % N, sj = tid / N;
  if (sj < S) {
    double acc = 0.0;
    for (int p0 = sj; p0 < nparts; p0 += PB * S) {
      double v[PB];
#pragma unroll
      for (int u = 0; u < PB; ++u) v[u] = part[(size_t)min(p0 + u * S, nparts - 1) * N + ai];
#pragma unroll
      for (int u = 0; u < PB; ++u)
        if (p0 + u * S < nparts) acc += v[u];
    }
    s_at[sj * N + ai] = acc;
  }
  __syncthreads();
  if (S >= 8) {
    for (int a = wave; a < N; a += W) {
      double v = 0.0;
      for (int q = lane; q < S; q += kWave) v += s_at[q * N + a];
      v = wave_sum_xor(v, kWave);
      if (lane == 0) {
        agent_dev[a] = (float)v;
        s_adev[a] = (float)v;
      }
    }
  } else {
    for (int a = tid; a < N; a += kSelThreads) {
      double tot = 0.0;
      for (int q = 0; q < S; ++q) tot += s_at[q * N + a];
      agent_dev[a] = (float)tot;
      s_adev[a] = (float)tot;
    }
  }
  __syncthreads();

  // ---- Master: argmin over the fp32 totals, ties to the lower index (each
  // lane scans its agents in ascending order, then a butterfly that prefers
  // the lower index on equal values)
  if (wave == 0) {
    float bv = lane < N ? s_adev[lane] : INFINITY;
    int bi = lane < N ? lane : 0x7fffffff;
    for (int a = lane + kWave; a < N; a += kWave) {
      const float v = s_adev[a];
      if (v < bv) {
        bv = v;
        bi = a;
      }
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov < bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) master[0] = bi;
  }
}

// Two workgroups of 1024 threads that run side by side: workgroup 0 selects
// the important set, workgroup 1 sums the agent totals and picks the Master.
template <int KEYS_IN_LDS, int PB>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ score, const double* __restrict__ part, int nparts, int N, int T,
    int k, float* __restrict__ agent_dev, int32_t* __restrict__ selected,
    int32_t* __restrict__ master) {
  extern __shared__ uint32_t s_key_dyn[];  // [kSelLdsKeys] score bits, when they fit
  if (blockIdx.x == 0)
    topk_role<KEYS_IN_LDS>(score, T, k, selected, s_key_dyn);
  else
    totals_role<PB>(part, nparts, N, agent_dev, master);
}

template <typename E, int D, int KCH, bool PAGED>
hipError_t launch_dev(const Dims& d, int check_layer, const void* kr, const PageMap& pm, const void* kx,
                      float* dev, float* score, double* part, int* nparts, hipStream_t s) {
  const size_t rowE = (size_t)d.Hkv * d.D;
  const size_t stride = (size_t)d.L * d.T * rowE;
  const E* krl = PAGED ? static_cast<const E*>(kr) : static_cast<const E*>(kr) + (size_t)check_layer * d.T * rowE;
  // agents in flight per wave: the group size that wastes the fewest re-reads
  // of the last agent (ties to the larger group), within the 256 registers a
  // wave of a 512-thread workgroup has: rows of 3-4 chunks per lane keep at
  // most 5 agents in flight, rows of 8 chunks (fp32, 16 heads x 128) 2
  int best = KCH >= 8 ? 2 : (KCH >= 4 ? 5 : 8);
  if (KCH < 8) {
    for (int au : {8, 5, 4}) {
      if (KCH >= 4 && au > 5) continue;
      const int waste = (d.N + au - 1) / au * au - d.N;
      const int bw = (d.N + best - 1) / best * best - d.N;
      if (waste < bw) best = au;
    }
  }
  // 8-wave workgroups when the GPU holds every token's wave at once, else 4
  auto launch = [&](auto kern) -> hipError_t {
    int dv = 0, ncu = 0, per_cu = 0, waves = kDevMinWaves;
    hipError_t e;
    if ((e = hipGetDevice(&dv)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dv)) != hipSuccess) return e;
    const int big = kDevMaxThreads / kWave;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                           kDevMaxThreads, big * d.N * sizeof(float))) != hipSuccess)
      return e;
    if ((long long)per_cu * ncu * big >= d.T) waves = big;
    *nparts = (d.T + waves - 1) / waves;
    hipLaunchKernelGGL(kern, dim3(*nparts), dim3(waves * kWave), waves * d.N * sizeof(float), s, krl,
                       static_cast<const E*>(kx), d.N, d.T, d.Hkv, stride, dev, score, part, pm, (long long)check_layer);
    return hipGetLastError();
  };
#define TDX_DEV(AU) return launch(deviation_kernel<E, D, KCH, AU, PAGED>)
  if constexpr (KCH >= 8) {
    TDX_DEV(2);
  } else if constexpr (KCH >= 4) {
    if (best == 5) TDX_DEV(5);
    else TDX_DEV(4);
  } else {
    if (best == 8) TDX_DEV(8);
    else if (best == 5) TDX_DEV(5);
    else TDX_DEV(4);
  }
#undef TDX_DEV
}

template <typename E, int D, bool PAGED>
hipError_t launch_dev_d(const Dims& d, int check_layer, const void* kr, const PageMap& pm, const void* kx,
                        float* dev, float* score, double* part, int* nparts, hipStream_t s) {
  const int cpr = d.Hkv * D / Fmt<E>::VEC;
  const int kch = (cpr + kWave - 1) / kWave;
  switch (kch) {
    case 1: return launch_dev<E, D, 1, PAGED>(d, check_layer, kr, pm, kx, dev, score, part, nparts, s);
    case 2: return launch_dev<E, D, 2, PAGED>(d, check_layer, kr, pm, kx, dev, score, part, nparts, s);
    case 3:
    case 4: return launch_dev<E, D, 4, PAGED>(d, check_layer, kr, pm, kx, dev, score, part, nparts, s);
    case 5:
    case 6:
    case 7:
    case 8: return launch_dev<E, D, 8, PAGED>(d, check_layer, kr, pm, kx, dev, score, part, nparts, s);
    default: return hipErrorInvalidValue;  // rows past 16 heads x 128 fp32 are rejected before
  }
}


}  // namespace

// partials of the deviation pass: one row per workgroup of at least 4 tokens
static int dev_parts(const Dims& d) { return (d.T + kDevMinWaves - 1) / kDevMinWaves; }

size_t select_ws_bytes(const Dims& d) {
  return (size_t)dev_parts(d) * d.N * sizeof(double);
}

namespace {
template <bool PAGED>
hipError_t select_t(const Dims& d, int check_layer, const void* k_reuse, const PageMap& pm, const void* k_recomp,
                    int k, float* dev, float* score, float* agent_dev, int32_t* selected, int32_t* master,
                    void* ws, hipStream_t s) {
  if (d.N > kMaxAgents) return hipErrorInvalidValue;
  int nparts = dev_parts(d);
  double* part = static_cast<double*>(ws);
  hipError_t e;
  if (d.dtype == TDX_BF16)
    e = d.D == 128
            ? launch_dev_d<uint16_t, 128, PAGED>(d, check_layer, k_reuse, pm, k_recomp, dev, score, part, &nparts, s)
            : launch_dev_d<uint16_t, 64, PAGED>(d, check_layer, k_reuse, pm, k_recomp, dev, score, part, &nparts, s);
  else
    e = d.D == 128
            ? launch_dev_d<float, 128, PAGED>(d, check_layer, k_reuse, pm, k_recomp, dev, score, part, &nparts, s)
            : launch_dev_d<float, 64, PAGED>(d, check_layer, k_reuse, pm, k_recomp, dev, score, part, &nparts, s);
  if (e != hipSuccess) return e;
  const size_t lds = d.T <= kSelLdsKeys ? (size_t)kSelLdsKeys * sizeof(uint32_t) : 0;
  // partials per thread of the totals workgroup: the smallest batch of 8, 16
  // or 32 loads that holds them, else batches of 32
  const int per = (nparts + kSelThreads / d.N - 1) / (kSelThreads / d.N);
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(2), dim3(kSelThreads), lds, s, score, part, nparts, d.N, d.T, k, agent_dev,
                       selected, master);
  };
  if (d.T <= kSelLdsKeys) {
    if (per <= 8) launch(select_kernel<1, 8>);
    else if (per <= 16) launch(select_kernel<1, 16>);
    else launch(select_kernel<1, 32>);
  } else {
    if (per <= 8) launch(select_kernel<0, 8>);
    else if (per <= 16) launch(select_kernel<0, 16>);
    else launch(select_kernel<0, 32>);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_select(const Dims& d, const tdx_layout& lay, int check_layer,
                         const void* k_reuse, const void* k_recomp, int k, float* dev,
                         float* score, float* agent_dev, int32_t* selected, int32_t* master,
                         void* ws, hipStream_t s) {
  (void)lay;
  const PageMap none{nullptr, 0, 1};
  return select_t<false>(d, check_layer, k_reuse, none, k_recomp, k, dev, score, agent_dev, selected, master, ws,
                         s);
}

hipError_t launch_select_paged(const Dims& d, int check_layer, const void* kr_pool, const PageMap& pm,
                               const void* k_recomp, int k, float* dev, float* score, float* agent_dev,
                               int32_t* selected, int32_t* master, void* ws, hipStream_t s) {
  return select_t<true>(d, check_layer, kr_pool, pm, k_recomp, k, dev, score, agent_dev, selected, master, ws, s);
}

}  // namespace tdx

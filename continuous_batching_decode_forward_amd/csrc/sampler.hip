// sampler.hip -- the batched sampler that closes the step.
//
// Per emitting row (RWKV-Runner Albatross article, "Worker main loop" and
// the adapter's defaults: frequency/presence penalty with decay, temperature,
// top-k, top-p, one batched sampling call over the decode segment):
//   S1 l' = l - f*c - q*[c > 0]            (c: the slot's decayed counts)
//   S2 T == 0: lowest-id argmax of l'; else z = l' / T
//   S3 e = exp(z - max z)
//   S4 top-k: keep the k largest by (e desc, id asc)          (0 < k < V)
//   S5 top-p: in (e desc, id asc) order keep the shortest prefix whose
//      mass reaches p * (mass after S4); the crossing id stays  (p < 1)
//   S6 u = Philox4x64-10(counter (request id, step id, 0, 0), key (seed, 0))
//      word 0, top 24 bits * 2^-24; r = u * kept mass; token = first kept id
//      in ascending id order whose running kept mass exceeds r
//   S7 c = c * decay for every id, then c[token] += 1
//
// One workgroup of 1024 threads (16 waves) per row. Wave w owns the
// contiguous ids [w*C, (w+1)*C), C = 64*K, and lane l of it takes ids
// w*C + 64k + l, k = 0..K-1: every global access is coalesced, and the
// ascending-id order is (wave, k, lane), so ascending-id questions (the CDF
// of S6, ties at a threshold) take a ballot or a wave prefix per k plus a
// prefix over the 16 waves. The row's e values (dropped ids hold -1) live
// on chip when V <= 65536: a thread's first 28 in registers, the other 36
// in LDS (144 KB per workgroup), so the passes below never leave the CU;
// larger vocabularies keep them in a workspace row indexed by id (coalesced,
// L2/MALL-resident between passes). Top-k and top-p thresholds come from a
// bisection over the bit patterns of e (non-negative floats order like
// their bits): each step one count or mass sum over the row, with no atomics
// and no sort; ties at the threshold are kept in ascending id order.
// Masses (S4-S6) accumulate in double, so the decisions are those of the
// exact sums up to rounding of order 1e-16; the fp32 products of S1 and S7
// are rounded before the following add (no fused multiply-add), as written.
#include "common.h"
#include "kernels.h"

namespace cbd {

#define SMP_THREADS 1024
#define SMP_WAVES (SMP_THREADS / 64)

// ---------------------------------------------------------------- Philox

__device__ __forceinline__ void philox4x64_10(uint64_t x[4], uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t m0 = 0xD2E7470EE14C6C93ull, m1 = 0xCA5A826395121157ull;
    uint64_t hi0 = __umul64hi(m0, x[0]), lo0 = m0 * x[0];
    uint64_t hi1 = __umul64hi(m1, x[2]), lo1 = m1 * x[2];
    uint64_t y0 = hi1 ^ x[1] ^ k0, y2 = hi0 ^ x[3] ^ k1;
    x[0] = y0;
    x[1] = lo1;
    x[2] = y2;
    x[3] = lo0;
    k0 += 0x9E3779B97F4A7C15ull;
    k1 += 0xBB67AE8584CAA73Bull;
  }
}

__device__ __forceinline__ float draw_uniform24(uint64_t seed, uint64_t request_id, uint32_t step) {
  uint64_t x[4] = {request_id, (uint64_t)step, 0, 0};
  philox4x64_10(x, seed, 0);
  return (float)(x[0] >> 40) * (1.0f / 16777216.0f);
}

// ------------------------------------------------------- block reductions

struct SmpShared {
  double red_d[SMP_WAVES];
  double wave_d[SMP_WAVES];
  float red_f[SMP_WAVES];
  int red_i[SMP_WAVES];
  int red_i2[SMP_WAVES];
  int wave_i[SMP_WAVES];
  int n_cand;
  float cand[SMP_THREADS];  // threshold candidates, one per thread
};

// An fp32 product rounded on its own: the empty asm hides it from
// contraction into a following add.
__device__ __forceinline__ float mul_rounded(float a, float b) {
  float t = a * b;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ double smp_block_sum_d(double v, SmpShared& sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) sh.red_d[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < SMP_WAVES; ++w) s += sh.red_d[w];
  __syncthreads();
  return s;
}

__device__ float smp_block_max(float v, SmpShared& sh) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) sh.red_f[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = -INFINITY;
#pragma unroll
  for (int w = 0; w < SMP_WAVES; ++w) s = fmaxf(s, sh.red_f[w]);
  __syncthreads();
  return s;
}

__device__ int smp_block_sum_i(int v, SmpShared& sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) sh.red_i[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < SMP_WAVES; ++w) s += sh.red_i[w];
  __syncthreads();
  return s;
}

__device__ int smp_block_min_i(int v, SmpShared& sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) sh.red_i[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = 0x7fffffff;
#pragma unroll
  for (int w = 0; w < SMP_WAVES; ++w) s = min(s, sh.red_i[w]);
  __syncthreads();
  return s;
}

__device__ int smp_block_max_i(int v, SmpShared& sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) sh.red_i[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = -1;
#pragma unroll
  for (int w = 0; w < SMP_WAVES; ++w) s = max(s, sh.red_i[w]);
  __syncthreads();
  return s;
}

// Inclusive prefix sum over the 64 lanes of a wave, in lane order.
__device__ __forceinline__ double wave_incl_scan(double v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// The per-thread row values (ids base + 64 k, k < K). REGS (K <= SMP_KREG):
// the first SMP_KR in registers, the rest in LDS ([k - SMP_KR][thread], the
// caller's slice); otherwise the workspace row, indexed by id.
#define SMP_KREG 64
#define SMP_KR 28

// Loops over a thread's K values. With REGS the bound is the constant
// SMP_KREG, fully unrolled so that the register array is indexed statically,
// the iterations past K are skipped, and each body starts with a scheduling
// barrier: without it the compiler hoists every iteration's compares and
// ballots at once, which does not fit the 128 registers a 1024-thread
// workgroup leaves each wave.
#define SMP_FOR_K(k)                                                   \
  _Pragma("unroll") for (int k = 0; k < (REGS ? SMP_KREG : K); ++k) \
    if (!REGS || k < K)

// The same over groups of SMP_LB values (k0 = 0, SMP_LB, ...): the body
// handles k0 .. k0 + SMP_LB - 1 and checks k < K itself.
#define SMP_LB 16
#define SMP_FOR_KB(k0)                                                              \
  _Pragma("unroll") for (int k0 = 0; k0 < (REGS ? SMP_KREG : K); k0 += SMP_LB) \
    if (!REGS || k0 < K)

template <bool REGS>
struct RowVals {
  float r[REGS ? SMP_KR : 1];
  float* g;  // REGS: this thread's LDS slice; otherwise the workspace row
  __device__ __forceinline__ float get(int k, int id) const {
    if constexpr (REGS)
      return k < SMP_KR ? r[k] : g[(k - SMP_KR) * SMP_THREADS];
    else
      return g[id];
  }
  __device__ __forceinline__ void set(int k, int id, float v) {
    if constexpr (REGS) {
      if (k < SMP_KR)
        r[k] = v;
      else
        g[(k - SMP_KR) * SMP_THREADS] = v;
    } else {
      g[id] = v;
    }
  }
};

// Block sums of one double and one int, sharing the barriers.
__device__ void smp_block_sum2(double& f, int& a, SmpShared& sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    f += __shfl_xor(f, o, 64);
    a += __shfl_xor(a, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    sh.red_d[threadIdx.x >> 6] = f;
    sh.red_i[threadIdx.x >> 6] = a;
  }
  __syncthreads();
  f = 0.0;
  a = 0;
#pragma unroll
  for (int w = 0; w < SMP_WAVES; ++w) {
    f += sh.red_d[w];
    a += sh.red_i[w];
  }
  __syncthreads();
}

// Kept values are non-negative floats, whose bit patterns read as signed
// ints are >= 0 and order like the values; dropped ids hold -1.0f, whose
// pattern is negative. So "kept and at least tau" is one signed compare, and
// every pass below is free of branches.
__device__ __forceinline__ int smp_bits(float v) { return __float_as_int(v); }

// Sum over the 64 lanes of a wave, the same in every lane (lane 0's).
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return __shfl(v, 0, 64);
}

// Largest bit pattern tau (non-negative floats) with F(tau) >= need, where
// F(tau) = count (BY_MASS false) or mass (true) of the kept values >= tau.
// Bisection between the smallest and largest kept pattern. Each step over
// the row is one pass and one reduction of F(mid) and C(mid), the number of
// kept values >= mid; C at both ends of the range gives the number of
// values left inside it. Once that is at most one per thread, those values
// are gathered into LDS and the search finishes on them alone: F(m) = F(hi)
// + the candidates in [m, hi) (those at or above a lowered hi are in F(hi)
// already), where F(hi) was computed when hi was last lowered (0 for the
// initial hi above every value). The result is the same whatever cut points
// the search takes, so the final phase takes three per step (a four-way
// split) to halve its steps.
template <bool BY_MASS, bool REGS>
__device__ __forceinline__ uint32_t smp_threshold(const RowVals<REGS>& e, int K, int base, double need,
                                  SmpShared& sh) {
  int lo = 0x7f800000, hi = 0;
  int kept = 0;
  SMP_FOR_K(k) { __builtin_amdgcn_sched_barrier(0);
    const int u = smp_bits(e.get(k, base + 64 * k));
    lo = min(lo, u >= 0 ? u : 0x7f800000);
    hi = max(hi, u);
    kept += u >= 0;
  }
  lo = -smp_block_max_i(-lo, sh);    // block min
  hi = smp_block_max_i(hi, sh) + 1;  // F(hi) = 0 < need
  int c_lo = smp_block_sum_i(kept, sh), c_hi = 0;
  double f_hi = 0.0;
  while (hi - lo > 1 && c_lo - c_hi > SMP_THREADS) {
    const int mid = lo + (hi - lo) / 2;
    double f = 0.0;
    int c = 0;
    SMP_FOR_K(k) { __builtin_amdgcn_sched_barrier(0);
      const float v = e.get(k, base + 64 * k);
      const bool in = smp_bits(v) >= mid;
      if (BY_MASS) f += in ? (double)v : 0.0;
      c += in;
    }
    smp_block_sum2(f, c, sh);
    if (!BY_MASS) f = (double)c;
    if (f >= need) {
      lo = mid;
      c_lo = c;
    } else {
      hi = mid;
      f_hi = f;
      c_hi = c;
    }
  }
  if (hi - lo <= 1) return (uint32_t)lo;
  // Gather the values in [lo, hi) (at most SMP_THREADS of them) in (thread,
  // k) order: each thread's first slot is the block prefix of the per-thread
  // counts, so the candidates, and every sum taken over them below, come out
  // in the same order on every run.
  {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int cnt = 0;
    SMP_FOR_K(k) { __builtin_amdgcn_sched_barrier(0);
      const int u = smp_bits(e.get(k, base + 64 * k));
      cnt += u >= lo && u < hi;
    }
    int inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(inc, o, 64);
      if (lane >= o) inc += t;
    }
    if (lane == 63) sh.wave_i[w] = inc;
    __syncthreads();
    int at = inc - cnt;
    for (int x = 0; x < w; ++x) at += sh.wave_i[x];
    SMP_FOR_K(k) { __builtin_amdgcn_sched_barrier(0);
      const float v = e.get(k, base + 64 * k);
      const int u = smp_bits(v);
      if (u >= lo && u < hi) sh.cand[at++] = v;
    }
    if (threadIdx.x == SMP_THREADS - 1) sh.n_cand = at;
    __syncthreads();
  }
  // Wave 0 alone finishes the search on the (at most SMP_THREADS)
  // candidates, 16 per lane, with wave reductions only; every lane decides
  // on lane 0's sums, and the result goes to the other waves through LDS.
  // (A block reduction per step -- about 20 steps at top-p 0.3 over 65536
  // ids -- cost two barriers each.) Each step sums the candidates in [m, hi)
  // for three cuts m1 <= m2 <= m3 in (lo, hi); these sums, and so F, do not
  // increase from m1 to m3 (the same terms in the same order, fewer of them),
  // so the largest cut with F >= need is well defined.
  if (threadIdx.x < 64) {
    constexpr int CPL = SMP_THREADS / 64;
    const int n = sh.n_cand;
    float cv[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int j = (int)threadIdx.x + 64 * i;
      cv[i] = j < n ? sh.cand[j] : -1.f;
    }
    while (hi - lo > 1) {
      const int d = hi - lo;
      const int m0 = lo + max(1, d / 4), m1 = lo + max(1, d / 2);
      const int m2 = lo + max(1, (int)((3LL * d) / 4));
      double c0 = 0.0, c1 = 0.0, c2 = 0.0;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int u = smp_bits(cv[i]);
        const double x = BY_MASS ? (double)cv[i] : 1.0;
        const bool below_hi = u < hi;
        c0 += below_hi && u >= m0 ? x : 0.0;
        c1 += below_hi && u >= m1 ? x : 0.0;
        c2 += below_hi && u >= m2 ? x : 0.0;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        c0 += __shfl_xor(c0, o, 64);
        c1 += __shfl_xor(c1, o, 64);
        c2 += __shfl_xor(c2, o, 64);
      }
      const double f0 = f_hi + __shfl(c0, 0, 64), f1 = f_hi + __shfl(c1, 0, 64);
      const double f2 = f_hi + __shfl(c2, 0, 64);
      if (f2 >= need) {
        lo = m2;
      } else if (f1 >= need) {
        lo = m1;
        hi = m2;
        f_hi = f2;
      } else if (f0 >= need) {
        lo = m0;
        hi = m1;
        f_hi = f1;
      } else {
        hi = m0;
        f_hi = f0;
      }
    }
    if (threadIdx.x == 0) sh.red_i[0] = lo;
  }
  __syncthreads();
  lo = sh.red_i[0];
  __syncthreads();  // red_i is reused by the next reduction
  return (uint32_t)lo;
}

// Keep the values above tau and the first eq_keep values equal to tau in
// ascending id order; drop the rest (-1). Returns this thread's kept mass.
template <bool REGS>
__device__ __forceinline__ double smp_keep(RowVals<REGS>& e, int K, int base, uint32_t tau, int eq_keep,
                          SmpShared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = (int)tau;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int eq_wave = 0;  // equals in this wave's range (same in every lane)
  SMP_FOR_K(k) { __builtin_amdgcn_sched_barrier(0);
    eq_wave += __popcll(__ballot(smp_bits(e.get(k, base + 64 * k)) == t));
  }
  if (lane == 0) sh.wave_i[w] = eq_wave;
  __syncthreads();
  int eq_before = 0;
  for (int x = 0; x < w; ++x) eq_before += sh.wave_i[x];
  __syncthreads();
  double own = 0.0;
  SMP_FOR_K(k) { __builtin_amdgcn_sched_barrier(0);
    const int id = base + 64 * k;
    const float v = e.get(k, id);
    const int u = smp_bits(v);
    const uint64_t m = __ballot(u == t);
    const bool keep = u > t || (u == t && eq_before + __popcll(m & below) < eq_keep);
    eq_before += __popcll(m);
    own += keep ? (double)v : 0.0;
    e.set(k, id, keep ? v : -1.f);
  }
  return own;
}

template <bool REGS>
__device__ __forceinline__ void sampler_row(const float* __restrict__ lrow, float* __restrict__ crow,
                            float* __restrict__ scratch_row, int V, int K, const SlotParams& P,
                            uint32_t step, int32_t* __restrict__ token_out, SmpShared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int base = w * 64 * K + lane;  // this thread's id at k = 0; ids step by 64
  RowVals<REGS> e;
  e.g = scratch_row;  // REGS: the caller passes its LDS slice base + threadIdx.x

  // S1 penalties (+ S2 division), and the decay of S7 in the same pass:
  // penalties read the counts before the step, and nothing below reads them
  // again, so each id's decayed count is written as soon as it is read (the
  // token's +1 follows once it is drawn). The two row reads go out SMP_LB
  // ids at a time: with the scheduling barrier of every id they waited one
  // memory round trip per id.
  float zmax = -INFINITY;
  SMP_FOR_KB(k0) { __builtin_amdgcn_sched_barrier(0);
    float cv[SMP_LB], lv[SMP_LB];
#pragma unroll
    for (int u = 0; u < SMP_LB; ++u) {
      const int id = base + 64 * (k0 + u);
      const bool ok = k0 + u < K && id < V;
      cv[u] = ok ? crow[id] : 0.f;
      lv[u] = ok ? lrow[id] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < SMP_LB; ++u) {
      const int k = k0 + u;
      if (k < K) {
        const int id = base + 64 * k;
        float z = -INFINITY;
        if (id < V) {
          const float c = cv[u];
          crow[id] = mul_rounded(c, P.penalty_decay);
          float l = lv[u] - mul_rounded(P.freq_penalty, c);
          if (c > 0.f) l = l - P.presence_penalty;
          for (int f = 0; f < P.n_forbidden; ++f)  // forbidden ids: never drawn
            if (id == P.forbidden[f]) l = -INFINITY;
          z = P.temperature == 0.f ? l : l / P.temperature;
        }
        e.set(k, id, z);
        zmax = fmaxf(zmax, z);
      }
    }
  }
  zmax = smp_block_max(zmax, sh);
  int token;
  if (P.temperature == 0.f) {  // greedy on the penalised logits, lowest id
    int cand = 0x7fffffff;
    SMP_FOR_K(k) { __builtin_amdgcn_sched_barrier(0);
      const int id = base + 64 * k;
      if (id < V && e.get(k, id) == zmax) cand = min(cand, id);
    }
    token = smp_block_min_i(cand, sh);
    if (token == 0x7fffffff) token = 0;
  } else {
    // S3
    double own = 0.0;
    SMP_FOR_K(k) { __builtin_amdgcn_sched_barrier(0);
      const int id = base + 64 * k;
      float v = -1.f;
      if (id < V) {
        v = expf(e.get(k, id) - zmax);
        own += v;
      }
      e.set(k, id, v);
    }
    double sum_k = smp_block_sum_d(own, sh);
    // S4 top-k
    if (P.top_k > 0 && P.top_k < V) {
      const uint32_t tau = smp_threshold<false>(e, K, base, (float)P.top_k, sh);
      int above = 0;
      SMP_FOR_K(k) { __builtin_amdgcn_sched_barrier(0);
        above += smp_bits(e.get(k, base + 64 * k)) > (int)tau;
      }
      above = smp_block_sum_i(above, sh);
      own = smp_keep(e, K, base, tau, P.top_k - above, sh);
      sum_k = smp_block_sum_d(own, sh);
    }
    // S5 top-p
    if (P.top_p < 1.f) {
      const double target = (double)P.top_p * sum_k;
      const uint32_t tau = smp_threshold<true>(e, K, base, target, sh);
      const double tauf = (double)__uint_as_float(tau);
      double above = 0.0;
      SMP_FOR_K(k) { __builtin_amdgcn_sched_barrier(0);
        const float v = e.get(k, base + 64 * k);
        above += smp_bits(v) > (int)tau ? (double)v : 0.0;
      }
      above = smp_block_sum_d(above, sh);
      // ids equal to tau needed to reach the target, in ascending id order
      const double need = target - above;
      int eq_keep = 1;
      if (tauf > 0.0 && need > tauf) eq_keep = (int)ceil(need / tauf);
      own = smp_keep(e, K, base, tau, eq_keep, sh);
    }
    // S6 draw over the ascending-id CDF of the kept mass
    double wsum = own;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wsum += __shfl_xor(wsum, o, 64);
    if (lane == 0) sh.wave_d[w] = wsum;
    __syncthreads();
    double total = 0.0, prefix = 0.0;
#pragma unroll
    for (int x = 0; x < SMP_WAVES; ++x) {
      if (x < w) prefix += sh.wave_d[x];
      total += sh.wave_d[x];
    }
    __syncthreads();
    const float u = draw_uniform24(P.seed, P.request_id, step);
    const double r = (double)u * total;
    int cand = 0x7fffffff, last = -1;
    if (prefix + wsum > r) {  // this wave's range reaches past r
      // The wave's totals over groups of SMP_LB consecutive k (64 SMP_LB
      // consecutive ids each), in ascending order, find the group where the
      // running mass passes r; one wave prefix per k then runs from there
      // (from k = 0 with the wave's prefix if no group total passes r, as
      // rounding may have it).
      double carry = prefix;
      int k_from = -1;
      SMP_FOR_KB(k0) { __builtin_amdgcn_sched_barrier(0);
        if (k_from < 0) {
          double gs = 0.0;
#pragma unroll
          for (int uu = 0; uu < SMP_LB; ++uu) {
            const int k = k0 + uu;
            if (k < K) {
              const float v = e.get(k, base + 64 * k);
              gs += v >= 0.f ? (double)v : 0.0;
            }
          }
          gs = wave_sum_d(gs);
          if (carry + gs > r)
            k_from = k0;
          else
            carry += gs;
        }
      }
      if (k_from < 0) {
        k_from = 0;
        carry = prefix;
      }
      SMP_FOR_K(k) { __builtin_amdgcn_sched_barrier(0);
        if (k < k_from) continue;
        const int id = base + 64 * k;
        const float v = e.get(k, id);
        const double kv = v >= 0.f ? (double)v : 0.0;
        const double run = carry + wave_incl_scan(kv);
        const uint64_t hit = __ballot(v >= 0.f && run > r);
        if (hit) {
          const int first = __ffsll((long long)hit) - 1;
          cand = base - lane + 64 * k + first;
          break;
        }
        carry = __shfl(run, 63, 64);  // run already holds carry
      }
    }
    SMP_FOR_K(k) { __builtin_amdgcn_sched_barrier(0);
      const int id = base + 64 * k;
      if (e.get(k, id) >= 0.f) last = id;
    }
    token = smp_block_min_i(cand, sh);
    if (token == 0x7fffffff) token = smp_block_max_i(last, sh);
    if (token < 0) token = 0;
  }
  // S7: every id's count was decayed in the S1 pass; the token's owner
  // thread (the one that wrote it) adds the token's count.
  {
    const int rem = token % (64 * K);
    if (w == token / (64 * K) && lane == rem % 64) crow[token] = crow[token] + 1.0f;
  }
  if (threadIdx.x == 0) *token_out = token;
}

// REGS: the row values in registers and dynamic LDS (V <= SMP_KREG *
// SMP_THREADS); otherwise in the workspace row of this output.
template <bool REGS>
__global__ __launch_bounds__(SMP_THREADS) void sampler_kernel(
    const float* __restrict__ logits, int V, int K, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ step_ids, const int32_t* __restrict__ out_seq,
    const SlotParams* __restrict__ params, float* __restrict__ counts, int max_slots,
    float* __restrict__ scratch, int32_t* __restrict__ tokens, uint32_t* status) {
  __shared__ SmpShared sh;
  extern __shared__ float smp_lds[];  // REGS: [SMP_KREG - SMP_KR][SMP_THREADS]
  const int j = blockIdx.x;
  const int sidx = out_seq ? out_seq[j] : j;
  const int slot = slots[sidx];
  if (slot < 0 || slot >= max_slots) {
    if (threadIdx.x == 0) {
      raise_status(status, ST_BAD_SLOT);
      tokens[j] = 0;
    }
    return;
  }
  const SlotParams P = params[slot];
  const uint32_t step = (uint32_t)step_ids[sidx];
  const float* lrow = logits + (size_t)j * V;
  float* crow = counts + (size_t)slot * V;
  float* vals = REGS ? smp_lds + threadIdx.x : scratch + (size_t)j * K * SMP_THREADS;
  sampler_row<REGS>(lrow, crow, vals, V, K, P, step, tokens + j, sh);
}

int32_t sampler_row_floats(int32_t V) {
  const int K = (V + SMP_THREADS - 1) / SMP_THREADS;
  return K * SMP_THREADS;
}

hipError_t launch_sampler(const float* logits, int32_t n, int32_t V, const int32_t* slots,
                          const int32_t* step_ids, const int32_t* out_seq, const SlotParams* params,
                          float* counts, int32_t max_slots, float* scratch, int32_t* tokens,
                          uint32_t* status, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int K = sampler_row_floats(V) / SMP_THREADS;
  if (K <= SMP_KREG) {
    const size_t lds = (size_t)(SMP_KREG - SMP_KR) * SMP_THREADS * sizeof(float);
    static bool lds_set = false;  // above 64 KB the launch must be allowed first
    if (!lds_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&sampler_kernel<true>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      lds_set = true;
    }
    sampler_kernel<true><<<n, SMP_THREADS, lds, st>>>(logits, V, K, slots, step_ids, out_seq,
                                                       params, counts, max_slots, scratch, tokens,
                                                       status);
  } else {
    sampler_kernel<false><<<n, SMP_THREADS, 0, st>>>(logits, V, K, slots, step_ids, out_seq,
                                                      params, counts, max_slots, scratch, tokens,
                                                      status);
  }
  return hipGetLastError();
}

}  // namespace cbd

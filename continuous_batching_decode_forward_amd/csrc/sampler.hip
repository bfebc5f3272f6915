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
// One workgroup of 1024 threads per row. Thread t owns the contiguous ids
// [t*PER, (t+1)*PER), so every ascending-id question (the CDF of S6, ties at
// a threshold) is one block scan of per-thread totals. The row's e values
// live in a workspace scratch row (L2-resident) between passes; dropped ids
// hold -1. Top-k and top-p thresholds come from a radix select on the bit
// patterns of e (non-negative floats order like their bits): four 8-bit
// passes over LDS histograms, counting ids for top-k and summing mass for
// top-p; ties at the threshold are kept in ascending id order. No sort of
// the vocabulary.
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
  float red_f[SMP_WAVES];
  int red_i[SMP_WAVES];
  float scan_f[SMP_THREADS];
  int scan_i[SMP_THREADS];
  unsigned hist_cnt[256];
  float hist_mass[256];
  unsigned sel_digit;
  unsigned sel_above_cnt;
  float sel_above_mass;
};

__device__ float smp_block_sum(float v, SmpShared& sh) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sh.red_f[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < SMP_WAVES; ++w) s += sh.red_f[w];
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

// Exclusive prefix over threads, in thread order (Hillis-Steele).
__device__ float smp_excl_scan_f(float v, SmpShared& sh) {
  const int t = threadIdx.x;
  sh.scan_f[t] = v;
  __syncthreads();
  for (int o = 1; o < SMP_THREADS; o <<= 1) {
    float add = t >= o ? sh.scan_f[t - o] : 0.f;
    __syncthreads();
    sh.scan_f[t] += add;
    __syncthreads();
  }
  float r = sh.scan_f[t] - v;
  __syncthreads();
  return r;
}

__device__ int smp_excl_scan_i(int v, SmpShared& sh) {
  const int t = threadIdx.x;
  sh.scan_i[t] = v;
  __syncthreads();
  for (int o = 1; o < SMP_THREADS; o <<= 1) {
    int add = t >= o ? sh.scan_i[t - o] : 0;
    __syncthreads();
    sh.scan_i[t] += add;
    __syncthreads();
  }
  int r = sh.scan_i[t] - v;
  __syncthreads();
  return r;
}

// Radix select over the bit patterns of the kept e values (e >= 0) of the
// row; each thread reads its own ids [id0, id0 + per) from the scratch row.
// BY_MASS = false: the largest pattern tau with count(e >= tau) >= need.
// BY_MASS = true:  the largest pattern tau with mass(e >= tau) >= need.
// Also returns what lies strictly above tau (count and mass).
template <bool BY_MASS>
__device__ uint32_t radix_select(const float* __restrict__ e, int id0, int per, float need,
                                 SmpShared& sh, unsigned* above_cnt, float* above_mass) {
  uint32_t prefix = 0;
  unsigned acnt = 0;
  float amass = 0.f;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += SMP_THREADS) {
      sh.hist_cnt[b] = 0;
      sh.hist_mass[b] = 0.f;
    }
    __syncthreads();
    const uint32_t hmask = shift == 24 ? 0u : (0xffffffffu << (shift + 8));
    for (int i = 0; i < per; i += 4) {
      const float4 v4 = *reinterpret_cast<const float4*>(e + id0 + i);
      const float vs[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float v = vs[k];
        const uint32_t bits = __float_as_uint(v);
        if (v >= 0.f && (bits & hmask) == prefix) {
          const uint32_t dgt = (bits >> shift) & 255u;
          if (BY_MASS)
            atomicAdd(&sh.hist_mass[dgt], v);
          else
            atomicAdd(&sh.hist_cnt[dgt], 1u);
        }
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned c = acnt;
      float ms = amass;
      int d = 255;
      for (; d > 0; --d) {
        bool reach = BY_MASS ? (ms + sh.hist_mass[d] >= need)
                             : (c + sh.hist_cnt[d] >= (unsigned)need);
        if (reach) break;
        c += sh.hist_cnt[d];
        ms += sh.hist_mass[d];
      }
      sh.sel_digit = (unsigned)d;
      sh.sel_above_cnt = c;
      sh.sel_above_mass = ms;
    }
    __syncthreads();
    prefix |= sh.sel_digit << shift;
    acnt = sh.sel_above_cnt;
    amass = sh.sel_above_mass;
    __syncthreads();
  }
  *above_cnt = acnt;
  *above_mass = amass;
  return prefix;
}

// Keep ids with e above tau and the first eq_keep ids (ascending id order)
// whose e equals tau; drop the rest (e = -1). Returns the kept mass of this
// thread's ids.
__device__ float keep_threshold(float* __restrict__ e, int id0, int per, uint32_t tau,
                                int eq_keep, SmpShared& sh) {
  int eq_own = 0;
  for (int i = 0; i < per; ++i) {
    const float v = e[id0 + i];
    if (v >= 0.f && __float_as_uint(v) == tau) ++eq_own;
  }
  int eq_before = smp_excl_scan_i(eq_own, sh);
  float own = 0.f;
  for (int i = 0; i < per; ++i) {
    const float v = e[id0 + i];
    if (!(v >= 0.f)) continue;
    const uint32_t b = __float_as_uint(v);
    bool keep = b > tau;
    if (b == tau) {
      keep = eq_before < eq_keep;
      ++eq_before;
    }
    if (keep)
      own += v;
    else
      e[id0 + i] = -1.f;
  }
  return own;
}

__global__ __launch_bounds__(SMP_THREADS) void sampler_kernel(
    const float* __restrict__ logits, int V, int per, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ step_ids, const int32_t* __restrict__ out_seq,
    const SlotParams* __restrict__ params, float* __restrict__ counts, int max_slots,
    float* __restrict__ scratch, int32_t* __restrict__ tokens, uint32_t* status) {
  __shared__ SmpShared sh;
  const int j = blockIdx.x;
  const int t = threadIdx.x;
  const int sidx = out_seq ? out_seq[j] : j;
  const int slot = slots[sidx];
  if (slot < 0 || slot >= max_slots) {
    if (t == 0) {
      raise_status(status, ST_BAD_SLOT);
      tokens[j] = 0;
    }
    return;
  }
  const SlotParams P = params[slot];
  const uint32_t step = (uint32_t)step_ids[sidx];
  const float* lrow = logits + (size_t)j * V;
  float* crow = counts + (size_t)slot * V;
  float* e = scratch + (size_t)j * per * SMP_THREADS;
  const int id0 = t * per;

  // S1 penalties (+ S2 division), into the scratch row
  float zmax = -INFINITY;
  for (int i = 0; i < per; ++i) {
    const int id = id0 + i;
    float z = -INFINITY;
    if (id < V) {
      const float c = crow[id];
      float l = lrow[id] - P.freq_penalty * c;
      if (c > 0.f) l = l - P.presence_penalty;
      z = P.temperature == 0.f ? l : l / P.temperature;
    }
    e[id] = z;
    zmax = fmaxf(zmax, z);
  }
  zmax = smp_block_max(zmax, sh);
  int token;
  if (P.temperature == 0.f) {  // greedy on the penalised logits, lowest id
    int cand = 0x7fffffff;
    for (int i = per - 1; i >= 0; --i)
      if (id0 + i < V && e[id0 + i] == zmax) cand = id0 + i;
    token = smp_block_min_i(cand, sh);
    if (token == 0x7fffffff) token = 0;
  } else {
    // S3
    float own = 0.f;
    for (int i = 0; i < per; ++i) {
      const int id = id0 + i;
      float v = -1.f;
      if (id < V) {
        v = expf(e[id] - zmax);
        own += v;
      }
      e[id] = v;
    }
    float sum_k = smp_block_sum(own, sh);
    // S4 top-k
    if (P.top_k > 0 && P.top_k < V) {
      unsigned above;
      float unused;
      const uint32_t tau = radix_select<false>(e, id0, per, (float)P.top_k, sh, &above, &unused);
      own = keep_threshold(e, id0, per, tau, P.top_k - (int)above, sh);
      sum_k = smp_block_sum(own, sh);
    }
    // S5 top-p
    if (P.top_p < 1.f) {
      const float target = P.top_p * sum_k;
      unsigned unused_c;
      float above_mass;
      const uint32_t tau = radix_select<true>(e, id0, per, target, sh, &unused_c, &above_mass);
      const float tauf = __uint_as_float(tau);
      // ids equal to tau needed to reach the target, in ascending id order
      const float need = target - above_mass;
      int eq_keep = 1;
      if (tauf > 0.f && need > tauf) eq_keep = (int)ceilf(need / tauf);
      own = keep_threshold(e, id0, per, tau, eq_keep, sh);
    }
    // S6 draw over the ascending-id CDF of the kept mass
    const float total = smp_block_sum(own, sh);
    const float excl = smp_excl_scan_f(own, sh);
    const float u = draw_uniform24(P.seed, P.request_id, step);
    const float r = u * total;
    int cand = 0x7fffffff, last = -1;
    float run = excl;
    for (int i = 0; i < per; ++i) {
      const float v = e[id0 + i];
      if (!(v >= 0.f)) continue;
      run += v;
      last = id0 + i;
      if (run > r) {
        cand = id0 + i;
        break;
      }
    }
    token = smp_block_min_i(cand, sh);
    if (token == 0x7fffffff) token = smp_block_max_i(last, sh);
    if (token < 0) token = 0;
  }
  // S7 counts: decay every id, then count the token
  for (int id = t; id < V; id += SMP_THREADS) {
    float c = crow[id] * P.penalty_decay;
    if (id == token) c = c + 1.0f;
    crow[id] = c;
  }
  if (t == 0) tokens[j] = token;
}

int32_t sampler_row_floats(int32_t V) {
  int per = (V + SMP_THREADS - 1) / SMP_THREADS;
  per = (per + 3) / 4 * 4;
  return per * SMP_THREADS;
}

hipError_t launch_sampler(const float* logits, int32_t n, int32_t V, const int32_t* slots,
                          const int32_t* step_ids, const int32_t* out_seq, const SlotParams* params,
                          float* counts, int32_t max_slots, float* scratch, int32_t* tokens,
                          uint32_t* status, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int per = sampler_row_floats(V) / SMP_THREADS;
  sampler_kernel<<<n, SMP_THREADS, 0, st>>>(logits, V, per, slots, step_ids, out_seq, params,
                                             counts, max_slots, scratch, tokens, status);
  return hipGetLastError();
}

}  // namespace cbd

// attention.hip -- paged GQA attention for decode rows and prefill chunks.
//
// Selective batching (Go under the hood 20.3.2, after Orca): the projections
// run over all rows of the step together, attention runs per sequence at that
// sequence's own length, reading its K/V block by block through its block
// table (PagedAttention's fixed-size blocks, same section).
//
// Work item = (sequence, KV head g, query tile, key split). A query tile is
// 16 "query columns": up to 16/G consecutive rows of the sequence times the G
// query heads that share KV head g, so every K/V element fetched serves G
// heads (decode: 1 row x G heads, the other columns idle; a prefill chunk:
// 16/G rows x G heads, a dense contraction). Keys are split into chunks of
// split_len positions so that long contexts spread over many waves; a second
// kernel combines the splits' (max, sum, output) in split order.
//
// One wave per work item, 32 keys per iteration, two MFMAs shapes:
//   S[32 keys][16 cols] = K . Q^T       v_mfma_f32_16x16x32_bf16, A = K rows,
//                                       B = Q (its hi and lo bf16 terms, two
//                                       MFMAs), K-dim = head_dim
//   O^T[hd][16 cols]   += V^T . P^T     A = V^T rows, B = P, K-dim = 32 keys
// The key order inside the S tiles is chosen so that the four lane groups
// end up holding 8 consecutive keys each, which is exactly the B operand the
// PV MFMA needs (no shuffles), and the V tile is stored dimension-major in
// the pool so that its A operand is one 16-byte load per lane. Softmax is
// online in base 2 (scores pre-scaled by log2(e)/sqrt(hd)); P enters the PV
// MFMA as three bf16 terms that sum to its fp32 value, and the running sums
// use fp32 P.
#include "common.h"
#include "kernels.h"

namespace cbd {

#define ATT_WAVES 4

__device__ __forceinline__ int find_seq(const int32_t* __restrict__ item0, int n, int item) {
  int lo = 0, hi = n - 1;  // largest s with item0[s] <= item
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (item0[mid] <= item)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

template <int HD, bool WIDE_BLOCKS>
__global__ __launch_bounds__(64 * ATT_WAVES) void attention_kernel(
    const uint16_t* __restrict__ q_hi, const uint16_t* __restrict__ q_lo, StepMeta m,
    RowMaps maps, ModelDims md, AttnPlan ap,
    const uint16_t* __restrict__ pool_k, const uint16_t* __restrict__ pool_v,
    float* __restrict__ part_ml, float* __restrict__ part_o, uint32_t* status) {
  constexpr int QK_STEPS = HD / 32;  // MFMAs over head_dim
  constexpr int DT = HD / 16;        // output d tiles
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int item = blockIdx.x * ATT_WAVES + wave;
  const int n_seqs = m.n_seqs;
  if (item >= maps.item0[n_seqs]) return;
  const int s = find_seq(maps.item0, n_seqs, item);
  const int G = md.n_heads / md.n_kv_heads;
  const int rpt = 16 / G;  // rows per query tile
  const int nn = m.n_new[s], ctx = m.ctx_lens[s];
  const int qtiles = (nn * G + 15) / 16;
  const int splits = (ctx + nn + ap.split_len - 1) / ap.split_len;
  int local = item - maps.item0[s];
  const int qt = local % qtiles;
  local /= qtiles;
  const int sp = local % splits;
  const int g = local / splits;

  // This lane's query column.
  const int c_row = qt * rpt + lr / G;  // row within the sequence
  const int c_head = g * G + lr % G;
  const bool c_ok = lr < rpt * G && c_row < nn;
  const int row0 = maps.seq_row0[s];
  const int last_row = min(nn, (qt + 1) * rpt) - 1;
  const int k_lo = sp * ap.split_len;
  const int k_hi = min(k_lo + ap.split_len, ctx + last_row + 1);
  const int c_end = c_ok ? min(k_hi, ctx + c_row + 1) : k_lo;  // keys [k_lo, c_end)

  // Q as the B operand: lane (lr, lg) holds d = lg*HD/4 + 8j .. +8 of its
  // column, as the hi and the lo bf16 terms of the fp32 query.
  bf16x8_t qf[2][QK_STEPS];
  {
    const size_t at = ((size_t)(row0 + (c_ok ? c_row : 0)) * md.n_heads + c_head) * HD +
                      lg * (HD / 4);
#pragma unroll
    for (int j = 0; j < QK_STEPS; ++j) {
      qf[0][j] = as_bf16x8(c_ok ? reinterpret_cast<const uint4*>(q_hi + at)[j]
                                : make_uint4(0, 0, 0, 0));
      qf[1][j] = as_bf16x8(c_ok ? reinterpret_cast<const uint4*>(q_lo + at)[j]
                                : make_uint4(0, 0, 0, 0));
    }
  }

  const int32_t* table = m.block_tables + (size_t)s * m.max_blocks_per_seq;
  const int bs = md.block_size;
  const size_t kv_head_stride = (size_t)bs * HD;  // one (block, kv head) tile
  const float scale = 1.4426950408889634f / sqrtf((float)HD);

  floatx4_t o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  bool bad_block = false;

  for (int p0 = k_lo; p0 < k_hi; p0 += 32) {
    // ---- K rows for the two S tiles: row m -> key p0 + 8(m/4) + m%4 + 4t
    uint4 kf[2][QK_STEPS];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int p = p0 + 8 * (lr >> 2) + (lr & 3) + 4 * t;
      bool ok = p < k_hi;
      int blk = ok ? table[p / bs] : 0;
      if (ok && (blk < 0 || blk >= md.num_blocks)) {
        bad_block = true;
        ok = false;
      }
      const uint16_t* kp = pool_k + ((size_t)blk * md.n_kv_heads + g) * kv_head_stride +
                           (size_t)(p % bs) * HD + lg * (HD / 4);
#pragma unroll
      for (int j = 0; j < QK_STEPS; ++j)
        kf[t][j] = ok ? reinterpret_cast<const uint4*>(kp)[j] : make_uint4(0, 0, 0, 0);
    }
    // ---- V^T rows for the PV MFMA: d = 16 dt + lr, keys p0 + 8 lg .. +8
    uint4 vf[DT];
    {
      const int pv = p0 + 8 * lg;
      if (WIDE_BLOCKS) {  // 8 | block_size: the 8 keys share one block
        bool ok = pv < k_hi;
        int blk = ok ? table[pv / bs] : 0;
        if (ok && (blk < 0 || blk >= md.num_blocks)) {
          bad_block = true;
          ok = false;
        }
        const uint16_t* vp = pool_v + ((size_t)blk * md.n_kv_heads + g) * kv_head_stride +
                             (size_t)lr * bs + (pv % bs);
#pragma unroll
        for (int t = 0; t < DT; ++t)
          vf[t] = ok ? *reinterpret_cast<const uint4*>(vp + (size_t)16 * t * bs)
                     : make_uint4(0, 0, 0, 0);
        // keys at or beyond k_hi inside the 8: zero them (they may hold stale data)
        if (ok && pv + 8 > k_hi) {
          int valid = k_hi - pv;  // 1..7
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            uint32_t w[4] = {vf[t].x, vf[t].y, vf[t].z, vf[t].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (2 * e >= valid) w[e] = 0;
              else if (2 * e + 1 >= valid) w[e] &= 0xffffu;
            }
            vf[t] = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
      } else {  // 4-position blocks: two half loads
#pragma unroll
        for (int t = 0; t < DT; ++t) vf[t] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int ph = pv + 4 * half;
          bool ok = ph < k_hi;
          int blk = ok ? table[ph / bs] : 0;
          if (ok && (blk < 0 || blk >= md.num_blocks)) {
            bad_block = true;
            ok = false;
          }
          const uint16_t* vp = pool_v + ((size_t)blk * md.n_kv_heads + g) * kv_head_stride +
                               (size_t)lr * bs + (ph % bs);
          int valid = min(4, k_hi - ph);
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            uint2 v = ok ? *reinterpret_cast<const uint2*>(vp + (size_t)16 * t * bs)
                         : make_uint2(0, 0);
            if (ok && valid < 4) {
              if (valid <= 0) v = make_uint2(0, 0);
              else if (valid == 1) v = make_uint2(v.x & 0xffffu, 0);
              else if (valid == 2) v = make_uint2(v.x, 0);
              else v = make_uint2(v.x, v.y & 0xffffu);
            }
            if (half == 0) {
              vf[t].x = v.x;
              vf[t].y = v.y;
            } else {
              vf[t].z = v.x;
              vf[t].w = v.y;
            }
          }
        }
      }
    }
    // ---- S = K . Q^T for the two tiles
    floatx4_t sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < QK_STEPS; ++j) {
        sacc[t] = mfma16x16x32(as_bf16x8(kf[t][j]), qf[0][j], sacc[t]);
        sacc[t] = mfma16x16x32(as_bf16x8(kf[t][j]), qf[1][j], sacc[t]);
      }
    }
    // lane (lr, lg) now holds column lr for keys p0 + 8 lg + jj, jj = i + 4 t
    float sv[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = p0 + 8 * lg + i + 4 * t;
        float v = (p < c_end) ? sacc[t][i] * scale : -INFINITY;
        sv[i + 4 * t] = v;
        cmax = fmaxf(cmax, v);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_new = fmaxf(m_run, cmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    // P = P1 + P2 + P3, three bf16 terms: together they carry P's full fp32
    // significand, so the PV product rounds like an fp32 weighted sum.
    uint32_t p1[4], p2[4], p3[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = exp2f(sv[2 * e] - m_use);
      const float b = exp2f(sv[2 * e + 1] - m_use);
      psum += a + b;
      const float a1 = round_bf(a), b1 = round_bf(b);
      const float a2 = round_bf(a - a1), b2 = round_bf(b - b1);
      p1[e] = pack_bf2(a1, b1);
      p2[e] = pack_bf2(a2, b2);
      p3[e] = pack_bf2(a - a1 - a2, b - b1 - b2);
    }
    l_run = l_run * alpha + psum;
    const bf16x8_t pf1 = as_bf16x8(make_uint4(p1[0], p1[1], p1[2], p1[3]));
    const bf16x8_t pf2 = as_bf16x8(make_uint4(p2[0], p2[1], p2[2], p2[3]));
    const bf16x8_t pf3 = as_bf16x8(make_uint4(p3[0], p3[1], p3[2], p3[3]));
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      o[t] = o[t] * alpha;
      o[t] = mfma16x16x32(as_bf16x8(vf[t]), pf1, o[t]);
      o[t] = mfma16x16x32(as_bf16x8(vf[t]), pf2, o[t]);
      o[t] = mfma16x16x32(as_bf16x8(vf[t]), pf3, o[t]);
    }
  }
  if (bad_block) raise_status(status, ST_BAD_BLOCK);

  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!c_ok || k_lo >= c_end) return;  // this column has no keys in this split
  const size_t idx = ((size_t)(row0 + c_row) * md.n_heads + c_head) * ap.max_splits + sp;
  if (lg == 0) {
    part_ml[2 * idx] = m_run;
    part_ml[2 * idx + 1] = l_run;
  }
  // lane holds O^T[d = 16 t + 4 lg + i][col lr]
  float* op = part_o + idx * HD + 4 * lg;
#pragma unroll
  for (int t = 0; t < DT; ++t)
    *reinterpret_cast<float4*>(op + 16 * t) = make_float4(o[t][0], o[t][1], o[t][2], o[t][3]);
}

// Combine the splits of one (row, head): out = sum_j 2^(m_j - M) o_j /
// sum_j 2^(m_j - M) l_j over the splits that hold keys of this row, in split
// order. One wave per (row, head), 4 per workgroup.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(StepMeta m, RowMaps maps, ModelDims md,
                                                           AttnPlan ap, int R,
                                                           const float* __restrict__ part_ml,
                                                           const float* __restrict__ part_o,
                                                           uint16_t* __restrict__ out_hi,
                                                           uint16_t* __restrict__ out_lo) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= R * md.n_heads) return;
  const int r = w / md.n_heads, h = w % md.n_heads;
  constexpr int PER = HD / 64;  // dims per lane
  const size_t at = ((size_t)r * md.n_heads + h) * HD + lane * PER;
  const int s = maps.row_seq[r];
  if (s < 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) out_hi[at + e] = out_lo[at + e] = 0;
    return;
  }
  const int pos = maps.row_pos[r];
  const int n_sp = pos / ap.split_len + 1;  // splits holding keys 0..pos
  const size_t base = ((size_t)r * md.n_heads + h) * ap.max_splits;
  float M = -INFINITY;
  for (int j = 0; j < n_sp; ++j) M = fmaxf(M, part_ml[2 * (base + j)]);
  float acc[PER], den = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int j = 0; j < n_sp; ++j) {
    const float wj = exp2f(part_ml[2 * (base + j)] - M);
    den += wj * part_ml[2 * (base + j) + 1];
    const float* op = part_o + (base + j) * HD + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += wj * op[e];
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    bf16_t hi, lo;
    split_bf(acc[e] * inv, hi, lo);
    out_hi[at + e] = hi;
    out_lo[at + e] = lo;
  }
}

template <int HD>
static hipError_t launch_hd(const uint16_t* q_hi, const uint16_t* q_lo, int32_t R,
                            const StepMeta& m, const RowMaps& maps, const ModelDims& md,
                            const AttnPlan& ap, const uint16_t* pool_k, const uint16_t* pool_v,
                            float* part_ml, float* part_o, uint16_t* out_hi, uint16_t* out_lo,
                            uint32_t* status, hipStream_t st) {
  const int blocks = (ap.grid_items + ATT_WAVES - 1) / ATT_WAVES;
  if (blocks > 0) {
    if (md.block_size % 8 == 0)
      attention_kernel<HD, true><<<blocks, 64 * ATT_WAVES, 0, st>>>(
          q_hi, q_lo, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, status);
    else
      attention_kernel<HD, false><<<blocks, 64 * ATT_WAVES, 0, st>>>(
          q_hi, q_lo, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int waves = R * md.n_heads;
  attn_combine_kernel<HD><<<(waves + 3) / 4, 256, 0, st>>>(m, maps, md, ap, R, part_ml, part_o,
                                                            out_hi, out_lo);
  return hipGetLastError();
}

hipError_t launch_attention(const uint16_t* q_hi, const uint16_t* q_lo, int32_t R,
                            const StepMeta& m, const RowMaps& maps, const ModelDims& md,
                            const AttnPlan& ap, const uint16_t* pool_k, const uint16_t* pool_v,
                            float* part_ml, float* part_o, uint16_t* out_hi, uint16_t* out_lo,
                            uint32_t* status, hipStream_t st) {
  if (R <= 0) return hipSuccess;
  if (md.head_dim == 128)
    return launch_hd<128>(q_hi, q_lo, R, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, out_hi,
                          out_lo, status, st);
  return launch_hd<64>(q_hi, q_lo, R, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, out_hi,
                       out_lo, status, st);
}

}  // namespace cbd

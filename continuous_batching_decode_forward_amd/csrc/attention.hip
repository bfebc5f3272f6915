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
#include <type_traits>

#include "attn_sched.h"
#include "common.h"
#include "kernels.h"
#include "rope_append.h"

namespace cbd {

#define ATT_LDS_SEQS 1024  // item0 staged in LDS for up to this many sequences

// A value the whole wave shares, moved to a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// One 32-key step's operands in registers, as loaded: K rows of the two S
// tiles and the V^T pieces -- bf16, 8 values (16 bytes) per MFMA operand,
// or E4M3 codes, widened to bf16 when the step is computed: V^T 8 codes (8
// bytes) per operand, K 16 codes (16 bytes) per load, the operands of two
// MFMAs (see kdim below).
template <int HD, bool F8>
struct KVTile {
  using Frag = typename std::conditional<F8, uint2, uint4>::type;
  uint4 k[2][F8 ? HD / 64 : HD / 32];
  Frag v[HD / 16];
};

// The head dimensions that lane group lg holds (8 consecutive ones) for the
// j-th 32-wide slice of the S = K.Q^T contraction. Any assignment works as
// long as K and Q use the same one and it covers each dimension once: bf16
// takes dims 32 j + 8 lg; an 8-bit cache takes 64 (j / 2) + 16 lg + 8 (j % 2),
// so that one 16-byte load per lane holds the codes of slices j and j + 1
// and the four lane groups together read 64 consecutive bytes of a key row
// (8-byte loads at dims 32 j + 8 lg read 32 bytes of every 128-byte row per
// instruction).
template <bool F8>
__device__ __forceinline__ int kdim(int j, int lg) {
  return F8 ? 64 * (j >> 1) + 16 * lg + 8 * (j & 1) : 32 * j + 8 * lg;
}

__device__ __forceinline__ uint4 widen(uint4 v) { return v; }
__device__ __forceinline__ uint4 widen(uint2 v) { return e4m3x8_to_bf16x8(v); }
// 16 bytes at element `elem` of the pool (bf16 values or E4M3 codes).
template <bool F8>
__device__ __forceinline__ uint4 load16(const void* base, size_t elem) {
  return load_stream16(reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(base) +
                                                         elem * (F8 ? 1 : 2)));
}
template <bool F8>
__device__ __forceinline__ auto load_frag(const void* base, size_t elem) {
  if constexpr (F8)
    return load_stream8(static_cast<const uint8_t*>(base) + elem);
  else
    return load_stream16(static_cast<const uint16_t*>(base) + elem);
}

// Issue priority from a wave's progress: 3 in the first quarter of its key
// steps, down to 0 in the last. Two waves share each SIMD, and at equal
// priority the older one wins every arbitration once the memory pipeline is
// full, so with a fixed schedule the younger workgroup on a CU finished about
// 1.5x later than the older one and ran its tail at half occupancy. Ranking by
// progress lets the wave that is behind catch up (the schedule, and so the
// result, does not change).
__device__ __forceinline__ void progress_prio(int done, int total) {
  const int lvl = min(3, (4 * done) / max(total, 1));
  if (lvl == 0)
    __builtin_amdgcn_s_setprio(3);
  else if (lvl == 1)
    __builtin_amdgcn_s_setprio(2);
  else if (lvl == 2)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Where a segment's result goes. Each lane holds its query column's running
// maximum m and sum l (base 2) and O^T[d = 16 t + 4 lg + i][col] for t <
// HD / 16; `has_keys` is false for an idle column or one with no key in the
// segment. SegPartials: the partial slot (row, head, split) in global
// memory, merged later by the combine kernel.
struct SegPartials {
  float* part_ml;
  float* part_o;
  int max_splits, sp, n_heads;
  template <int DT>
  __device__ __forceinline__ void operator()(int row, int head, int lr, int lg, bool has_keys,
                                             float m_run, float l_run, const floatx4_t (&o)[DT],
                                             float vs) const {
    if (!has_keys) return;
    const size_t idx = ((size_t)row * n_heads + head) * max_splits + sp;
    if (lg == 0) {
      part_ml[2 * idx] = m_run;
      part_ml[2 * idx + 1] = l_run;
    }
    float* op = part_o + idx * (16 * DT) + 4 * lg;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      *reinterpret_cast<float4*>(op + 16 * t) =
          make_float4(o[t][0] * vs, o[t][1] * vs, o[t][2] * vs, o[t][3] * vs);
  }
};

// The row kernel's: the wave's slot in LDS, columns 0 .. ATT_ROW_G - 1 (one
// decode row, its G heads), merged by the workgroup afterwards.
struct SegLds {
  float* ml;  // [ATT_ROW_G][2]
  float* o;   // [ATT_ROW_G][HD]
  template <int DT>
  __device__ __forceinline__ void operator()(int row, int head, int lr, int lg, bool has_keys,
                                             float m_run, float l_run, const floatx4_t (&o_)[DT],
                                             float vs) const {
    if (!has_keys || lr >= ATT_ROW_G) return;
    if (lg == 0) {
      ml[2 * lr] = m_run;
      ml[2 * lr + 1] = l_run;
    }
    float* op = o + lr * (16 * DT) + 4 * lg;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      *reinterpret_cast<float4*>(op + 16 * t) =
          make_float4(o_[t][0] * vs, o_[t][1] * vs, o_[t][2] * vs, o_[t][3] * vs);
  }
};

// The loads are unconditional and branch-free: a key past the item's range
// reads a valid pool location (its score is masked to -inf, and its V
// element is zeroed on the last step), and a block id outside the pool is
// replaced by block 0 and reported. Block ids come from the wave's slice of
// the block table staged in LDS, so no K/V address waits on a global load.
// The kernel is held to 256 registers (accumulators included) so that two
// waves share each SIMD: one wave's loads stay in flight while the other
// computes (at one wave per SIMD the key stream stalls on every step).
template <int HD, int BS, bool F8, class Out>
__device__ __forceinline__ void attend_segment(
    const uint16_t* __restrict__ q_hi, const uint16_t* __restrict__ q_lo, const StepMeta& m,
    const RowMaps& maps, const ModelDims& md, const void* __restrict__ pool_k,
    const void* __restrict__ pool_v, const Out& out, uint32_t* status, int* tbl, int s, int g,
    int qt, int nn, int ctx, int k_lo, int k_hi, int done, int total) {
  constexpr int QK_STEPS = HD / 32;  // MFMAs over head_dim
  constexpr int DT = HD / 16;        // output d tiles
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int G = md.n_heads / md.n_kv_heads;
  const int rpt = 16 / G;  // rows per query tile
  // This lane's query column: row c_row of the sequence, query head c_head.
  const int c_row = qt * rpt + lr / G;
  const int c_head = g * G + lr % G;
  const bool c_ok = lr < rpt * G && c_row < nn;
  const int row0 = uniform(maps.seq_row0[s]);
  const int c_end = c_ok ? min(k_hi, ctx + c_row + 1) : k_lo;  // keys [k_lo, c_end)

  // Q as the B operand of S = K.Q^T: lane (lr, lg) holds d = 32 j + 8 lg .. +8
  // of its column for step j, as the hi and lo bf16 terms.
  bf16x8_t qf[2][QK_STEPS];
  {
    const size_t at = ((size_t)(row0 + min(c_row, nn - 1)) * md.n_heads + c_head) * HD +
                      (F8 ? 16 : 8) * lg;
#pragma unroll
    for (int j = 0; j < QK_STEPS; ++j) {
      const int d = kdim<F8>(j, 0);
      qf[0][j] = as_bf16x8(*reinterpret_cast<const uint4*>(q_hi + at + d));
      qf[1][j] = as_bf16x8(*reinterpret_cast<const uint4*>(q_lo + at + d));
    }
  }

  // The wave's block-table slice: entries for blocks b0 .. b0 + nb - 1.
  const int32_t* table = m.block_tables + (size_t)s * m.max_blocks_per_seq;
  const int b0 = k_lo / BS;
  const int nb = (k_hi - 1) / BS - b0 + 1;  // <= ATT_TBL (host-side piece cap)
  if (nb > ATT_TBL) {  // the host caps piece_hi; refuse rather than overrun LDS
    if (lane == 0) raise_status(status, ST_BAD_SHAPE);
    return;
  }
  // The previous segment's reads of the slice are done before it is
  // overwritten (LDS operations of one wave complete in order).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  bool bad_block = false;
  for (int i = lane; i < nb; i += 64) {
    int blk = table[b0 + i];
    if (blk < 0 || blk >= md.num_blocks) {
      bad_block = true;
      blk = 0;
    }
    tbl[i] = blk;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // Offsets below count stored values (bf16 or E4M3 codes).
  const size_t head_stride = (size_t)BS * HD;  // one (block, kv head) tile
  const size_t kv_off = (size_t)g * head_stride;
  const size_t blk_stride = (size_t)md.n_kv_heads * head_stride;
  // An 8-bit cache holds K / k_scale: the scale joins the softmax scale.
  const float scale = 1.4426950408889634f / sqrtf((float)HD) * (F8 ? md.k_scale : 1.0f);
  const int last = k_hi - 1;

  // Per-lane constant parts of the K and V^T addresses inside a block.
  // K row of tile t for this lane: key 8 (lr / 4) + lr % 4 + 4 t of the step.
  const int krow0 = 8 * (lr >> 2) + (lr & 3);
  auto load = [&](KVTile<HD, F8>& T, int p0) {
    if constexpr (BS >= 32) {
      // A 32-key step lies in one block (steps start on multiples of 32):
      // one block id for the wave, keys past the range read stale but valid
      // slots of the same block.
      const int blk = uniform(tbl[p0 / BS - b0]);
      const size_t kb = (size_t)blk * blk_stride + kv_off + (size_t)(p0 % BS) * HD;
      const size_t vb = (size_t)blk * blk_stride + kv_off + (p0 % BS);
      if constexpr (F8) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < QK_STEPS; j += 2)
            T.k[t][j / 2] = load16<F8>(pool_k, kb + (size_t)(krow0 + 4 * t) * HD + kdim<F8>(j, lg));
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < QK_STEPS; ++j)
            T.k[t][j] = load_frag<F8>(pool_k, kb + (size_t)(krow0 + 4 * t) * HD + 8 * lg + 32 * j);
      }
#pragma unroll
      for (int t = 0; t < DT; ++t)
        T.v[t] = load_frag<F8>(pool_v, vb + (size_t)(16 * t + lr) * BS + 8 * lg);
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int p = min(p0 + krow0 + 4 * t, last);
        const int blk = tbl[p / BS - b0];
        const size_t kp = (size_t)blk * blk_stride + kv_off + (size_t)(p % BS) * HD;
        if constexpr (F8) {
#pragma unroll
          for (int j = 0; j < QK_STEPS; j += 2) T.k[t][j / 2] = load16<F8>(pool_k, kp + kdim<F8>(j, lg));
        } else {
#pragma unroll
          for (int j = 0; j < QK_STEPS; ++j) T.k[t][j] = load_frag<F8>(pool_k, kp + 8 * lg + 32 * j);
        }
      }
      // V^T pieces: row d = 16 t + lr, keys pv .. pv + 7 (pv = p0 + 8 lg)
      const int pv = min(p0 + 8 * lg, last & ~7);
      if constexpr (BS >= 8) {
        const int blk = tbl[pv / BS - b0];
        const size_t vp = (size_t)blk * blk_stride + kv_off + (size_t)lr * BS + (pv % BS);
#pragma unroll
        for (int t = 0; t < DT; ++t) T.v[t] = load_frag<F8>(pool_v, vp + (size_t)16 * t * BS);
      } else {  // 4-position blocks (bf16 only): two 8-byte halves
        static_assert(!F8, "an 8-bit cache needs blocks of 8 positions or more");
        const int blk0 = tbl[pv / BS - b0];
        const int blk1 = tbl[min(pv + 4, last) / BS - b0];
        const uint16_t* v0 = static_cast<const uint16_t*>(pool_v) + (size_t)blk0 * blk_stride + kv_off + (size_t)lr * BS;
        const uint16_t* v1 = static_cast<const uint16_t*>(pool_v) + (size_t)blk1 * blk_stride + kv_off + (size_t)lr * BS;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const uint2 a = *reinterpret_cast<const uint2*>(v0 + (size_t)16 * t * BS);
          const uint2 b = *reinterpret_cast<const uint2*>(v1 + (size_t)16 * t * BS);
          T.v[t] = make_uint4(a.x, a.y, b.x, b.y);
        }
      }
    }
  };

  floatx4_t o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // Steps that end at or before every column's limit need no score mask.
  // Idle columns (c_ok false) take k_hi: their values are never written.
  const int col_end = c_ok ? c_end : k_hi;
  int mask_from = col_end;
#pragma unroll
  for (int o_ = 1; o_ < 16; o_ <<= 1) mask_from = min(mask_from, __shfl_xor(mask_from, o_, 64));
  mask_from = uniform(mask_from);

  auto compute = [&](KVTile<HD, F8>& T, int p0) {
    floatx4_t sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < QK_STEPS; ++j) {
        bf16x8_t kf;
        if constexpr (F8) {
          const uint4 c = T.k[t][j / 2];
          kf = as_bf16x8(e4m3x8_to_bf16x8((j & 1) ? make_uint2(c.z, c.w) : make_uint2(c.x, c.y)));
        } else {
          kf = as_bf16x8(T.k[t][j]);
        }
        sacc[t] = mfma16x16x32(kf, qf[0][j], sacc[t]);
        sacc[t] = mfma16x16x32(kf, qf[1][j], sacc[t]);
      }
    }
    uint4 vw[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) vw[t] = widen(T.v[t]);
    // lane (lr, lg) holds column lr for keys p0 + 8 lg + i + 4 t
    float sv[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i + 4 * t] = sacc[t][i] * scale;
    if (p0 + 32 > mask_from) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int p = p0 + 8 * lg + (e & 3) + 4 * (e >> 2);
        if (p >= col_end) sv[e] = -INFINITY;
      }
    }
    float cmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                       fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_new = fmaxf(m_run, cmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    // Stale V elements of keys past the range (last step only) are zeroed:
    // their P is 0, but 0 * NaN would not be.
    if (p0 + 32 > k_hi) {
      const int valid = k_hi - (p0 + 8 * lg);  // keys of this lane's piece in range
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        uint32_t w[4] = {vw[t].x, vw[t].y, vw[t].z, vw[t].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t keep = 2 * e + 1 < valid ? 0xffffffffu : (2 * e < valid ? 0xffffu : 0u);
          w[e] &= keep;
        }
        vw[t] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    // P = P1 + P2 + P3 exactly: each term keeps the top 8 significant bits
    // of what the previous ones left (truncation; the last remainder has at
    // most 8 bits and is itself a bf16), so the PV product accumulates like
    // an fp32 weighted sum. The terms of two keys pack into one register.
    uint32_t p1[4], p2[4], p3[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = __builtin_amdgcn_exp2f(sv[2 * e] - m_use);
      const float b = __builtin_amdgcn_exp2f(sv[2 * e + 1] - m_use);
      psum += a + b;
      const float a1 = __uint_as_float(__float_as_uint(a) & 0xffff0000u);
      const float b1 = __uint_as_float(__float_as_uint(b) & 0xffff0000u);
      const float ra = a - a1, rb = b - b1;
      const float a2 = __uint_as_float(__float_as_uint(ra) & 0xffff0000u);
      const float b2 = __uint_as_float(__float_as_uint(rb) & 0xffff0000u);
      const float a3 = ra - a2, b3 = rb - b2;
      // the high halves of a (low 16 bits of the result) and b (high 16)
      p1[e] = __builtin_amdgcn_perm(__float_as_uint(b1), __float_as_uint(a1), 0x07060302u);
      p2[e] = __builtin_amdgcn_perm(__float_as_uint(b2), __float_as_uint(a2), 0x07060302u);
      p3[e] = __builtin_amdgcn_perm(__float_as_uint(b3), __float_as_uint(a3), 0x07060302u);
    }
    l_run = l_run * alpha + psum;
    // Rescale the running output only when some column's maximum moved.
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] = o[t] * alpha;
    }
    const bf16x8_t pf1 = as_bf16x8(make_uint4(p1[0], p1[1], p1[2], p1[3]));
    const bf16x8_t pf2 = as_bf16x8(make_uint4(p2[0], p2[1], p2[2], p2[3]));
    const bf16x8_t pf3 = as_bf16x8(make_uint4(p3[0], p3[1], p3[2], p3[3]));
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = mfma16x16x32(as_bf16x8(vw[t]), pf1, o[t]);
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = mfma16x16x32(as_bf16x8(vw[t]), pf2, o[t]);
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = mfma16x16x32(as_bf16x8(vw[t]), pf3, o[t]);
  };

  // Two tiles in flight: the loads of step i + 1 are issued before step i is
  // computed (near the end they repeat the last step's addresses, which
  // the cache serves; those repeats are never computed). Every load starts
  // on a step boundary: the block-size >= 32 path's per-lane offsets assume
  // it (a start past the boundary would read beyond the block's tile).
  {
    const int n_it = (k_hi - k_lo + 31) / 32;
    const int last_step = k_lo + 32 * (n_it - 1);
    KVTile<HD, F8> A, B;
    load(A, k_lo);
    int i = 0;
    for (; i + 2 <= n_it; i += 2) {
      progress_prio(done + i, total);
      load(B, k_lo + 32 * (i + 1));
      compute(A, k_lo + 32 * i);
      load(A, min(k_lo + 32 * (i + 2), last_step));
      compute(B, k_lo + 32 * (i + 1));
    }
    if (i < n_it) compute(A, k_lo + 32 * i);
  }
  if (bad_block) raise_status(status, ST_BAD_BLOCK);

  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  // lane holds O^T[d = 16 t + 4 lg + i][col lr]; an 8-bit cache holds
  // V / v_scale
  out(row0 + c_row, c_head, lr, lg, c_ok && k_lo < c_end, m_run, l_run, o,
      F8 ? md.v_scale : 1.0f);
}

// The kernel is held to 256 registers (accumulators included) so that two
// waves share each SIMD: one wave's loads stay in flight while the other
// computes (at one wave per SIMD the key stream stalls on every step).
template <int HD, int BS, bool F8>
__global__ __launch_bounds__(64 * ATT_WAVES) __attribute__((amdgpu_waves_per_eu(2))) void attention_kernel(
    const uint16_t* __restrict__ q_hi, const uint16_t* __restrict__ q_lo, StepMeta m,
    RowMaps maps, ModelDims md, AttnPlan ap, const void* __restrict__ pool_k,
    const void* __restrict__ pool_v, float* __restrict__ part_ml,
    float* __restrict__ part_o, uint32_t* status) {
  __shared__ int s_item0[ATT_LDS_SEQS + 1];
  __shared__ int s_tbl[ATT_WAVES][ATT_TBL];
  const int wave = uniform(threadIdx.x >> 6);
  const int n_seqs = m.n_seqs;
  const bool lds_seqs = n_seqs <= ATT_LDS_SEQS;
  if (lds_seqs)
    for (int i = threadIdx.x; i <= n_seqs; i += 64 * ATT_WAVES) s_item0[i] = maps.item0[i];
  __syncthreads();  // no barrier below this point
  const int32_t* step0 = lds_seqs ? s_item0 : maps.item0;
  // Everything that selects a segment is the same for the whole wave;
  // readfirstlane makes that explicit so that the key loop is a scalar loop.
  const int T = uniform(step0[n_seqs]);
  const PieceSched ps = piece_sched(T, ap, md.n_kv_heads);
  const int n_pieces = ps.per_head * md.n_kv_heads;
  const int rpt = 16 / (md.n_heads / md.n_kv_heads);
  const int first = blockIdx.x * ATT_WAVES + wave;
  const int total = first < n_pieces ? ceil_div(n_pieces - first, ap.grid_items) * ps.len : 0;
  int done = 0;  // key steps of this wave so far
  for (int p = first; p < n_pieces; p += ap.grid_items) {
    const int g = p / ps.per_head, q = p % ps.per_head;
    int b = q * ps.len;
    const int b_end = min(T, b + ps.len);
    while (b < b_end) {
      const int s = uniform(find_seq(step0, n_seqs, b));
      const int nn = uniform(m.n_new[s]), ctx = uniform(m.ctx_lens[s]);
      const int s0 = uniform(step0[s]);
      const Segment sg = piece_segment(b, b_end, s0, nn, ctx, q, ps.len, rpt);
      if (sg.sp >= ap.max_splits) {  // the host's piece_lo rules this out
        if ((threadIdx.x & 63) == 0) raise_status(status, ST_BAD_SHAPE);
      } else {
        const SegPartials out{part_ml, part_o, ap.max_splits, sg.sp, md.n_heads};
        attend_segment<HD, BS, F8>(q_hi, q_lo, m, maps, md, pool_k, pool_v, out, status,
                                   s_tbl[wave], s, g, sg.qt, nn, ctx, sg.k_lo, sg.k_hi, done,
                                   total);
      }
      b += sg.steps;
      done += sg.steps;
    }
  }
}

// -------------------------------------------------------------- row kernel
//
// Decode-only steps over short contexts (every sequence one row, at most
// ATT_ROW_KEYS keys): workgroup (sequence s, KV head g) of ATT_ROW_WAVES
// waves. First the workgroup does the RoPE + KV append of its row for the
// slots only it reads -- K and V of head g and the G query heads of g --
// and a workgroup barrier orders those stores before its own loads (no
// other workgroup reads them, so no wider fence is needed). Then wave w
// takes the w-th equal run of the row's 32-key steps through the same
// segment code, leaves its (m, l, O) in LDS, and the workgroup merges the
// runs in key order with the combine kernel's arithmetic: no partial
// results in global memory, no RoPE/append launch before and no combine
// launch after. At these sizes a step is a chain of short launches, so the
// launches it saves are most of its gain. A sequence that does not have
// exactly one row is refused (status BAD_SHAPE, zero outputs; its rows are
// still appended, as the standalone RoPE/append kernel would); a row no
// valid sequence owns gets zero outputs from the workgroups whose sequence
// index equals it (rows number the sequences here).
template <int HD, int BS, bool F8>
__global__ __launch_bounds__(64 * ATT_ROW_WAVES) __attribute__((amdgpu_waves_per_eu(2))) void attention_row_kernel(
    RopeAppendArgs ra, StepMeta m, RowMaps maps, ModelDims md, int R,
    uint16_t* __restrict__ out_hi, uint16_t* __restrict__ out_lo, uint32_t* status) {
  __shared__ int s_tbl[ATT_ROW_WAVES][ATT_TBL];
  __shared__ float s_ml[ATT_ROW_WAVES][ATT_ROW_G][2];
  __shared__ float s_o[ATT_ROW_WAVES][ATT_ROW_G][HD];
  constexpr int LPP = HD / 8;  // merge threads per head, 8 dimensions each
  constexpr int T = 64 * ATT_ROW_WAVES;
  const int wave = uniform(threadIdx.x >> 6);
  const int s = blockIdx.x / md.n_kv_heads, g = blockIdx.x % md.n_kv_heads;
  const int G = md.n_heads / md.n_kv_heads;
  const int KB = (md.n_heads * HD + 31) / 32;
  auto zero_row = [&](int row) {  // this KV head's G outputs of one row
    for (int t = threadIdx.x; t < G * LPP; t += T) {
      const size_t at = tile_at(row, (g * G + t / LPP) * HD + 8 * (t % LPP), KB);
      *reinterpret_cast<uint4*>(out_hi + at) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(out_lo + at) = make_uint4(0, 0, 0, 0);
    }
  };
  // RoPE + append of row `row` for this KV head's slots: its G query heads,
  // its K head and its V head.
  auto rope_row = [&](int row) {
    constexpr int half = HD / 2;
    const int pos = maps.row_pos[row];
    for (int t = threadIdx.x; t < (G + 2) * half; t += T) {
      const int js = t / half;
      const int j = js < G ? g * G + js : md.n_heads + (js - G) * md.n_kv_heads + g;
      rope_append_one(ra, row, s, pos, j, t % half, status);
    }
  };
  if (s < R && maps.row_seq[s] < 0) zero_row(s);
  const int r = maps.seq_row0[s];
  const int nn = m.n_new[s];
  if (r < 0 || r >= R || maps.row_seq[r] != s) return;  // refused by prep (no rows to serve)
  if (nn != 1) {  // served rows, but more than one: not a decode row
    if (threadIdx.x == 0 && g == 0) raise_status(status, ST_BAD_SHAPE);
    for (int i = 0; i < nn && r + i < R; ++i) {
      rope_row(r + i);
      zero_row(r + i);
    }
    return;
  }
  rope_row(r);
  __syncthreads();  // the row's q, K and V stores before this workgroup reads them
  const int ctx = m.ctx_lens[s];
  const int n_steps = ceil_div(ctx + 1, 32);  // keys 0 .. ctx, the row's own included
  const int per = ceil_div(n_steps, ATT_ROW_WAVES);
  const int st0 = wave * per, st1 = min(n_steps, st0 + per);
  if (st0 < st1) {
    const SegLds out{&s_ml[wave][0][0], &s_o[wave][0][0]};
    attend_segment<HD, BS, F8>(ra.q_hi, ra.q_lo, m, maps, md, ra.pool_k, ra.pool_v, out, status,
                               s_tbl[wave], s, g, 0, 1, ctx, 32 * st0, min(ctx + 1, 32 * st1), 0,
                               st1 - st0);
  }
  __syncthreads();
  const int n_used = ceil_div(n_steps, per);
  for (int t = threadIdx.x; t < G * LPP; t += T) {
    const int j = t / LPP, sl = t % LPP;
    float M = -INFINITY;
    for (int w = 0; w < n_used; ++w) M = fmaxf(M, s_ml[w][j][0]);
    float acc[8], den = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int w = 0; w < n_used; ++w) {
      const float wj = exp2f(s_ml[w][j][0] - M);
      den += wj * s_ml[w][j][1];
      const float4 a = *reinterpret_cast<const float4*>(&s_o[w][j][8 * sl]);
      const float4 b = *reinterpret_cast<const float4*>(&s_o[w][j][8 * sl + 4]);
      acc[0] += wj * a.x; acc[1] += wj * a.y; acc[2] += wj * a.z; acc[3] += wj * a.w;
      acc[4] += wj * b.x; acc[5] += wj * b.y; acc[6] += wj * b.z; acc[7] += wj * b.w;
    }
    const float inv = 1.0f / den;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = acc[e] * inv;
    store_split8(out_hi, out_lo, tile_at(r, (g * G + j) * HD + 8 * sl, KB), y);
  }
}

// ------------------------------------------------------------ block kernel
//
// Prefill chunks: a work item is (sequence, KV head g, block of 256 query
// columns = 256/G consecutive rows x the G heads of g, key split), run by a
// workgroup of 8 waves, each owning two 16-column tiles (the per-tile
// kernel's tiles, so the MFMA algebra, the online softmax and the partial
// layout are the same and the same combine follows). The workgroup stages
// each 32-key step of K and V^T once in LDS for all 16 tiles, by direct
// global->LDS copies (16 KB per step at head_dim 128: 2 per wave) into a
// 6-step ring (4 steps in flight while one is computed), instead of every
// tile reading its own copy of the prefix.
// Per-lane copy sources lay the stage out conflict-free for the MFMA
// operand reads: K as [8-dim chunk][key] and V^T as [8-key chunk][dim], so
// the 16 lanes that read different keys (or dims) hit consecutive 16-byte
// slots. Block sizes of 32 and up only (a 32-key step lies in one block).
#define ATB_WAVES 8
#define ATB_CT 2                              // 16-column tiles per wave
#define ATB_COLS (ATB_WAVES * ATB_CT * 16)    // query columns per item
static_assert(ATB_COLS == ATT_BLOCK_COLS, "the host plans items of ATT_BLOCK_COLS columns");
#define ATB_STAGES 6

template <int HD, int BS>
__global__ __launch_bounds__(64 * ATB_WAVES) void attention_block_kernel(
    const uint16_t* __restrict__ q_hi, const uint16_t* __restrict__ q_lo, StepMeta m,
    RowMaps maps, ModelDims md, AttnPlan ap, const uint16_t* __restrict__ pool_k,
    const uint16_t* __restrict__ pool_v, float* __restrict__ part_ml,
    float* __restrict__ part_o, uint32_t* status) {
  static_assert(BS >= 32 && BS % 32 == 0, "a 32-key step must lie in one block");
  constexpr int QK_STEPS = HD / 32;   // MFMAs over head_dim
  constexpr int DT = HD / 16;         // output d tiles
  constexpr int NK = HD / 8 * 32;     // 16-byte K slots per step ([chunk][key])
  constexpr int NSLOT = 8 * HD;       // K + V^T slots per step
  constexpr int CPW = NSLOT / 64 / ATB_WAVES;  // copies per wave per step
  static_assert(NSLOT % (64 * ATB_WAVES) == 0, "copies per wave");
  extern __shared__ uint4 ring_lds[];  // [ATB_STAGES][NSLOT]
  __shared__ int s_tbl[ATT_TBL];
  auto ring = [&](int j) { return ring_lds + (size_t)j * NSLOT; };
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int n_seqs = m.n_seqs;
  const int item = blockIdx.x;
  const int total = uniform(maps.item0b[n_seqs]);
  if (item >= total) return;  // the whole workgroup
  const int s = uniform(find_seq(maps.item0b, n_seqs, item));
  const int G = md.n_heads / md.n_kv_heads;
  const int rpt = 16 / G;               // rows per 16-column tile
  const int nn = uniform(m.n_new[s]), ctx = uniform(m.ctx_lens[s]);
  const BlockItem bi = block_item(item - uniform(maps.item0b[s]), nn, ctx, ap);
  const int g = bi.g, sp = bi.sp, row_lo = bi.row_lo, last_row = bi.last_row;
  const int k_lo = bi.k_lo, k_hi = bi.k_hi;
  if (k_lo >= k_hi) return;  // no keys of this split for these rows: the whole workgroup

  // The item's block-table slice.
  const int32_t* table = m.block_tables + (size_t)s * m.max_blocks_per_seq;
  const int b0 = k_lo / BS;
  const int nb = (k_hi - 1) / BS - b0 + 1;  // <= ATT_TBL (host-side split cap)
  if (nb > ATT_TBL) {
    if (threadIdx.x == 0) raise_status(status, ST_BAD_SHAPE);
    return;  // the whole workgroup
  }
  bool bad_block = false;
  for (int i = threadIdx.x; i < nb; i += 64 * ATB_WAVES) {
    int blk = table[b0 + i];
    if (blk < 0 || blk >= md.num_blocks) {
      bad_block = true;
      blk = 0;
    }
    s_tbl[i] = blk;
  }

  // This wave's two tiles: column lr of tile ct is row c_row, head c_head.
  const int row0 = uniform(maps.seq_row0[s]);
  int c_row[ATB_CT], c_head[ATB_CT], col_end[ATB_CT], mask_from[ATB_CT], tile_hi[ATB_CT];
  bool c_ok[ATB_CT];
  bf16x8_t qf[ATB_CT][2][QK_STEPS];
  int wave_hi = k_lo;
#pragma unroll
  for (int ct = 0; ct < ATB_CT; ++ct) {
    const int t = wave * ATB_CT + ct;
    const int tr0 = row_lo + t * rpt;  // the tile's first row
    c_row[ct] = tr0 + lr / G;
    c_head[ct] = g * G + lr % G;
    c_ok[ct] = c_row[ct] <= last_row;
    const int c_end = c_ok[ct] ? min(k_hi, ctx + c_row[ct] + 1) : k_lo;
    // idle columns take k_hi: their values are never written
    col_end[ct] = c_ok[ct] ? c_end : k_hi;
    int mf = col_end[ct];
#pragma unroll
    for (int o_ = 1; o_ < 16; o_ <<= 1) mf = min(mf, __shfl_xor(mf, o_, 64));
    mask_from[ct] = uniform(mf);
    tile_hi[ct] = tr0 <= last_row ? min(k_hi, ctx + min(last_row, tr0 + rpt - 1) + 1) : k_lo;
    wave_hi = max(wave_hi, tile_hi[ct]);
    const size_t at =
        ((size_t)(row0 + min(c_row[ct], nn - 1)) * md.n_heads + c_head[ct]) * HD + 8 * lg;
#pragma unroll
    for (int j = 0; j < QK_STEPS; ++j) {
      qf[ct][0][j] = as_bf16x8(*reinterpret_cast<const uint4*>(q_hi + at + 32 * j));
      qf[ct][1][j] = as_bf16x8(*reinterpret_cast<const uint4*>(q_lo + at + 32 * j));
    }
  }
  __syncthreads();  // the table slice is staged

  const size_t head_stride = (size_t)BS * HD;  // one (block, kv head) tile
  const size_t blk_stride = (size_t)md.n_kv_heads * head_stride;
  const uint16_t* kbase = pool_k + (size_t)g * head_stride;
  const uint16_t* vbase = pool_v + (size_t)g * head_stride;
  const float scale = 1.4426950408889634f / sqrtf((float)HD);
  const int n_it = (k_hi - k_lo + 31) / 32;

  // Step c's copies into ring slot j: this wave's copies x = wave * CPW + i
  // cover slots x * 64 + lane; K slots [chunk][key], then V^T [key chunk][dim].
  auto issue = [&](int j, int c) {
    const int p0 = k_lo + 32 * c;
    const int blk = s_tbl[p0 / BS - b0];
    const int off0 = p0 % BS;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int slot = (wave * CPW + i) * 64 + lane;
      const uint16_t* src;
      if (slot < NK) {
        const int ch = slot / 32, key = slot % 32;
        src = kbase + (size_t)blk * blk_stride + (size_t)(off0 + key) * HD + 8 * ch;
      } else {
        const int v = slot - NK, q = v / HD, d = v % HD;
        src = vbase + (size_t)blk * blk_stride + (size_t)d * BS + off0 + 8 * q;
      }
      copy16_to_lds(src, ring(j) + (wave * CPW + i) * 64);
    }
  };

  floatx4_t o[ATB_CT][DT];
  float m_run[ATB_CT], l_run[ATB_CT];
#pragma unroll
  for (int ct = 0; ct < ATB_CT; ++ct) {
#pragma unroll
    for (int t = 0; t < DT; ++t) o[ct][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m_run[ct] = -INFINITY;
    l_run[ct] = 0.f;
  }
  const int krow0 = 8 * (lr >> 2) + (lr & 3);

  // One 32-key step of one tile: scores, online softmax, PV (the per-tile
  // kernel's arithmetic, with K and V^T fragments read from the stage).
  auto tile_step = [&](int ct, const uint4 (&kf)[2][QK_STEPS], uint4 (&vf)[DT], int p0) {
    floatx4_t sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < QK_STEPS; ++j) {
        sacc[t] = mfma16x16x32(as_bf16x8(kf[t][j]), qf[ct][0][j], sacc[t]);
        sacc[t] = mfma16x16x32(as_bf16x8(kf[t][j]), qf[ct][1][j], sacc[t]);
      }
    }
    float sv[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i + 4 * t] = sacc[t][i] * scale;
    if (p0 + 32 > mask_from[ct]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int p = p0 + 8 * lg + (e & 3) + 4 * (e >> 2);
        if (p >= col_end[ct]) sv[e] = -INFINITY;
      }
    }
    float cmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                       fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_new = fmaxf(m_run[ct], cmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run[ct] - m_use);
    m_run[ct] = m_new;
    uint32_t p1[4], p2[4], p3[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = __builtin_amdgcn_exp2f(sv[2 * e] - m_use);
      const float b = __builtin_amdgcn_exp2f(sv[2 * e + 1] - m_use);
      psum += a + b;
      const float a1 = __uint_as_float(__float_as_uint(a) & 0xffff0000u);
      const float b1 = __uint_as_float(__float_as_uint(b) & 0xffff0000u);
      const float ra = a - a1, rb = b - b1;
      const float a2 = __uint_as_float(__float_as_uint(ra) & 0xffff0000u);
      const float b2 = __uint_as_float(__float_as_uint(rb) & 0xffff0000u);
      const float a3 = ra - a2, b3 = rb - b2;
      p1[e] = __builtin_amdgcn_perm(__float_as_uint(b1), __float_as_uint(a1), 0x07060302u);
      p2[e] = __builtin_amdgcn_perm(__float_as_uint(b2), __float_as_uint(a2), 0x07060302u);
      p3[e] = __builtin_amdgcn_perm(__float_as_uint(b3), __float_as_uint(a3), 0x07060302u);
    }
    l_run[ct] = l_run[ct] * alpha + psum;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int t = 0; t < DT; ++t) o[ct][t] = o[ct][t] * alpha;
    }
    const bf16x8_t pf1 = as_bf16x8(make_uint4(p1[0], p1[1], p1[2], p1[3]));
    const bf16x8_t pf2 = as_bf16x8(make_uint4(p2[0], p2[1], p2[2], p2[3]));
    const bf16x8_t pf3 = as_bf16x8(make_uint4(p3[0], p3[1], p3[2], p3[3]));
#pragma unroll
    for (int t = 0; t < DT; ++t) o[ct][t] = mfma16x16x32(as_bf16x8(vf[t]), pf1, o[ct][t]);
#pragma unroll
    for (int t = 0; t < DT; ++t) o[ct][t] = mfma16x16x32(as_bf16x8(vf[t]), pf2, o[ct][t]);
#pragma unroll
    for (int t = 0; t < DT; ++t) o[ct][t] = mfma16x16x32(as_bf16x8(vf[t]), pf3, o[ct][t]);
  };

  // The ring: step c + ATB_STAGES - 1 is issued right after the barrier of
  // step c, and the wait for step c is an exact vector-memory count (every
  // issue is CPW copies per wave; past the last step the last step is
  // re-issued, never computed).
#pragma unroll
  for (int j = 0; j < ATB_STAGES - 1; ++j) issue(j, min(j, n_it - 1));
  for (int c = 0; c < n_it; ++c) {
    // step c's copies landed; those of the next ATB_STAGES - 2 steps may not have
    wait_vmem<(ATB_STAGES - 2) * CPW>();
    __syncthreads();
    issue((c + ATB_STAGES - 1) % ATB_STAGES, min(c + ATB_STAGES - 1, n_it - 1));
    const int p0 = k_lo + 32 * c;
    if (p0 < wave_hi) {
      const uint4* st = ring(c % ATB_STAGES);
      uint4 kf[2][QK_STEPS], vf[DT];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < QK_STEPS; ++j) kf[t][j] = st[(4 * j + lg) * 32 + krow0 + 4 * t];
#pragma unroll
      for (int t = 0; t < DT; ++t) vf[t] = st[NK + lg * HD + 16 * t + lr];
      // Stale V elements of keys past the range (last step only) are zeroed:
      // their P is 0, but 0 * NaN would not be.
      if (p0 + 32 > k_hi) {
        const int valid = k_hi - (p0 + 8 * lg);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          uint32_t w[4] = {vf[t].x, vf[t].y, vf[t].z, vf[t].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t keep = 2 * e + 1 < valid ? 0xffffffffu : (2 * e < valid ? 0xffffu : 0u);
            w[e] &= keep;
          }
          vf[t] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < ATB_CT; ++ct)
        if (p0 < tile_hi[ct]) tile_step(ct, kf, vf, p0);
    }
  }
  wait_vmem<0>();  // no LDS copy may land after the workgroup exits
  if (bad_block) raise_status(status, ST_BAD_BLOCK);

#pragma unroll
  for (int ct = 0; ct < ATB_CT; ++ct) {
    float l = l_run[ct];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int c_end = c_ok[ct] ? min(k_hi, ctx + c_row[ct] + 1) : k_lo;
    if (!c_ok[ct] || k_lo >= c_end) continue;  // this column has no keys in this split
    const size_t idx =
        ((size_t)(row0 + c_row[ct]) * md.n_heads + c_head[ct]) * ap.max_splits + sp;
    if (lg == 0) {
      part_ml[2 * idx] = m_run[ct];
      part_ml[2 * idx + 1] = l;
    }
    float* op = part_o + idx * HD + 4 * lg;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      *reinterpret_cast<float4*>(op + 16 * t) =
          make_float4(o[ct][t][0], o[ct][t][1], o[ct][t][2], o[ct][t][3]);
  }
}

// Combine the splits of one (row, head): out = sum_j 2^(m_j - M) o_j /
// sum_j 2^(m_j - M) l_j over the partial results that hold keys of this row,
// in key order. HD / 8 lanes per (row, head), 8 consecutive dims each, so
// that every lane writes one whole 16-byte run of an operand tile per plane.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(StepMeta m, RowMaps maps, ModelDims md,
                                                           AttnPlan ap, int R,
                                                           const float* __restrict__ part_ml,
                                                           const float* __restrict__ part_o,
                                                           uint16_t* __restrict__ out_hi,
                                                           uint16_t* __restrict__ out_lo) {
  constexpr int LPP = HD / 8;     // lanes per (row, head)
  constexpr int PPB = 256 / LPP;  // (row, head) pairs per workgroup
  const int sl = threadIdx.x % LPP;
  const int w = blockIdx.x * PPB + threadIdx.x / LPP;
  if (w >= R * md.n_heads) return;
  const int r = w / md.n_heads, h = w % md.n_heads;
  const size_t at = tile_at(r, h * HD + 8 * sl, (md.n_heads * HD + 31) / 32);
  const int s = maps.row_seq[r];
  if (s < 0) {
    *reinterpret_cast<uint4*>(out_hi + at) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(out_lo + at) = make_uint4(0, 0, 0, 0);
    return;
  }
  const int pos = maps.row_pos[r];
  const int nn = m.n_new[s];
  int n_sp;  // partial results holding keys 0..pos
  if (attn_on_block_kernel(nn, ap)) {  // block kernel: splits of split_len keys
    n_sp = block_partials(pos, ap);
  } else {  // per-tile kernel: the pieces over this row's (sequence, tile) steps
    const PieceSched ps = piece_sched(maps.item0[m.n_seqs], ap, md.n_kv_heads);
    const int rpt = 16 / (md.n_heads / md.n_kv_heads);
    const int qt = (r - maps.seq_row0[s]) / rpt;
    n_sp = piece_partials(tile_start(maps.item0[s], qt, nn, m.ctx_lens[s], rpt), pos, ps.len);
  }
  // Up to CB_ONE partial results are loaded at once, all in flight
  // together, then used in key order: one round trip. More take two passes
  // (the maximum, then the sums) that load four at a time. Both ways add
  // the same terms in the same order with the same maximum.
  const size_t base = ((size_t)r * md.n_heads + h) * ap.max_splits;
  float acc[8], den = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  auto add = [&](float2 ml, float4 a, float4 b, float M) {
    const float wj = exp2f(ml.x - M);
    den += wj * ml.y;
    acc[0] += wj * a.x; acc[1] += wj * a.y; acc[2] += wj * a.z; acc[3] += wj * a.w;
    acc[4] += wj * b.x; acc[5] += wj * b.y; acc[6] += wj * b.z; acc[7] += wj * b.w;
  };
  constexpr int CB_ONE = 16;
  if (n_sp <= CB_ONE) {
    float2 ml[CB_ONE];
    float4 oa[CB_ONE], ob[CB_ONE];
#pragma unroll
    for (int u = 0; u < CB_ONE; ++u)
      if (u < n_sp) {
        ml[u] = reinterpret_cast<const float2*>(part_ml)[base + u];
        const float4* op = reinterpret_cast<const float4*>(part_o + (base + u) * HD + 8 * sl);
        oa[u] = op[0];
        ob[u] = op[1];
      }
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < CB_ONE; ++u)
      if (u < n_sp) M = fmaxf(M, ml[u].x);
#pragma unroll
    for (int u = 0; u < CB_ONE; ++u)
      if (u < n_sp) add(ml[u], oa[u], ob[u], M);
  } else {
    float M = -INFINITY;
    for (int j0 = 0; j0 < n_sp; j0 += 4) {
      float mv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) mv[u] = j0 + u < n_sp ? part_ml[2 * (base + j0 + u)] : -INFINITY;
#pragma unroll
      for (int u = 0; u < 4; ++u) M = fmaxf(M, mv[u]);
    }
    for (int j0 = 0; j0 < n_sp; j0 += 4) {
      float2 ml[4];
      float4 oa[4], ob[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j0 + u < n_sp) {
          ml[u] = reinterpret_cast<const float2*>(part_ml)[base + j0 + u];
          const float4* op = reinterpret_cast<const float4*>(part_o + (base + j0 + u) * HD + 8 * sl);
          oa[u] = op[0];
          ob[u] = op[1];
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j0 + u < n_sp) add(ml[u], oa[u], ob[u], M);
    }
  }
  const float inv = 1.0f / den;
  bf16_t hi[8], lo[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) split_bf(acc[e] * inv, hi[e], lo[e]);
  *reinterpret_cast<uint4*>(out_hi + at) =
      make_uint4((uint32_t)hi[0] | ((uint32_t)hi[1] << 16), (uint32_t)hi[2] | ((uint32_t)hi[3] << 16),
                 (uint32_t)hi[4] | ((uint32_t)hi[5] << 16), (uint32_t)hi[6] | ((uint32_t)hi[7] << 16));
  *reinterpret_cast<uint4*>(out_lo + at) =
      make_uint4((uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16),
                 (uint32_t)lo[4] | ((uint32_t)lo[5] << 16), (uint32_t)lo[6] | ((uint32_t)lo[7] << 16));
}

template <int HD, int BS>
static void launch_items(int blocks, const uint16_t* q_hi, const uint16_t* q_lo, const StepMeta& m,
                         const RowMaps& maps, const ModelDims& md, const AttnPlan& ap,
                         const void* pool_k, const void* pool_v, float* part_ml,
                         float* part_o, uint32_t* status, hipStream_t st) {
  if constexpr (BS >= 8) {
    if (md.kv_fp8) {
      attention_kernel<HD, BS, true><<<blocks, 64 * ATT_WAVES, 0, st>>>(
          q_hi, q_lo, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, status);
      return;
    }
  }
  attention_kernel<HD, BS, false><<<blocks, 64 * ATT_WAVES, 0, st>>>(
      q_hi, q_lo, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, status);
}

template <int HD, int BS>
static void launch_rows(const RopeAppendArgs& ra, int32_t R, const StepMeta& m,
                        const RowMaps& maps, const ModelDims& md, uint16_t* out_hi,
                        uint16_t* out_lo, uint32_t* status, hipStream_t st) {
  const unsigned grid = (unsigned)(m.n_seqs * md.n_kv_heads);
  if constexpr (BS >= 8) {
    if (md.kv_fp8) {
      attention_row_kernel<HD, BS, true><<<grid, 64 * ATT_ROW_WAVES, 0, st>>>(
          ra, m, maps, md, R, out_hi, out_lo, status);
      return;
    }
  }
  attention_row_kernel<HD, BS, false><<<grid, 64 * ATT_ROW_WAVES, 0, st>>>(
      ra, m, maps, md, R, out_hi, out_lo, status);
}

// Dynamic LDS above 64 KB must be allowed per kernel before its first launch.
static hipError_t allow_lds(const void* kernel, size_t bytes) {
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int HD>
static hipError_t launch_hd(const uint16_t* q_hi, const uint16_t* q_lo, int32_t R,
                            const StepMeta& m, const RowMaps& maps, const ModelDims& md,
                            const AttnPlan& ap, const void* pool_k_, const void* pool_v_,
                            float* part_ml, float* part_o, uint16_t* out_hi, uint16_t* out_lo,
                            uint32_t* status, hipStream_t st) {
  if (ap.row_kernel) return hipErrorInvalidValue;  // launch_rope_attention_rows runs that plan
  // the block kernel reads a bf16 cache (an 8-bit cache plans no block items)
  const uint16_t* pool_k = static_cast<const uint16_t*>(pool_k_);
  const uint16_t* pool_v = static_cast<const uint16_t*>(pool_v_);
  if (ap.block_rows > 0 && ap.grid_items_b > 0) {
    if (md.kv_fp8) return hipErrorInvalidValue;
    const size_t lds = (size_t)ATB_STAGES * 8 * HD * 16;  // the K/V ring
    if (md.block_size == 32) {
      hipError_t e = allow_lds(reinterpret_cast<const void*>(&attention_block_kernel<HD, 32>), lds);
      if (e != hipSuccess) return e;
      attention_block_kernel<HD, 32><<<ap.grid_items_b, 64 * ATB_WAVES, lds, st>>>(
          q_hi, q_lo, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, status);
    } else if (md.block_size == 64) {
      hipError_t e = allow_lds(reinterpret_cast<const void*>(&attention_block_kernel<HD, 64>), lds);
      if (e != hipSuccess) return e;
      attention_block_kernel<HD, 64><<<ap.grid_items_b, 64 * ATB_WAVES, lds, st>>>(
          q_hi, q_lo, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, status);
    } else {
      return hipErrorInvalidValue;  // the host enables the block kernel for 32 and 64 only
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int blocks = (ap.grid_items + ATT_WAVES - 1) / ATT_WAVES;
  if (blocks > 0) {
    switch (md.block_size) {
      case 4: launch_items<HD, 4>(blocks, q_hi, q_lo, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, status, st); break;
      case 8: launch_items<HD, 8>(blocks, q_hi, q_lo, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, status, st); break;
      case 16: launch_items<HD, 16>(blocks, q_hi, q_lo, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, status, st); break;
      case 32: launch_items<HD, 32>(blocks, q_hi, q_lo, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, status, st); break;
      case 64: launch_items<HD, 64>(blocks, q_hi, q_lo, m, maps, md, ap, pool_k, pool_v, part_ml, part_o, status, st); break;
      default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int pairs = R * md.n_heads, per_block = 256 / (HD / 8);
  attn_combine_kernel<HD><<<(pairs + per_block - 1) / per_block, 256, 0, st>>>(
      m, maps, md, ap, R, part_ml, part_o, out_hi, out_lo);
  return hipGetLastError();
}

template <int HD>
static hipError_t launch_rows_hd(const RopeAppendArgs& ra, int32_t R, const StepMeta& m,
                                 const RowMaps& maps, const ModelDims& md, uint16_t* out_hi,
                                 uint16_t* out_lo, uint32_t* status, hipStream_t st) {
  switch (md.block_size) {
    case 4: launch_rows<HD, 4>(ra, R, m, maps, md, out_hi, out_lo, status, st); break;
    case 8: launch_rows<HD, 8>(ra, R, m, maps, md, out_hi, out_lo, status, st); break;
    case 16: launch_rows<HD, 16>(ra, R, m, maps, md, out_hi, out_lo, status, st); break;
    case 32: launch_rows<HD, 32>(ra, R, m, maps, md, out_hi, out_lo, status, st); break;
    case 64: launch_rows<HD, 64>(ra, R, m, maps, md, out_hi, out_lo, status, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rope_attention_rows(float* qkv, const float* part, int32_t S, int32_t R,
                                      const StepMeta& m, const RowMaps& maps,
                                      const double* rope_cs, const ModelDims& md,
                                      const AttnPlan& ap, uint16_t* q_hi, uint16_t* q_lo,
                                      void* pool_k, void* pool_v, uint16_t* out_hi,
                                      uint16_t* out_lo, uint32_t* status, hipStream_t st) {
  if (R <= 0) return hipSuccess;
  if (!ap.row_kernel || R != m.n_seqs) return hipErrorInvalidValue;
  const RopeAppendArgs ra =
      rope_append_args(qkv, part, S, R, m, rope_cs, md, q_hi, q_lo, pool_k, pool_v);
  if (md.head_dim == 128) return launch_rows_hd<128>(ra, R, m, maps, md, out_hi, out_lo, status, st);
  return launch_rows_hd<64>(ra, R, m, maps, md, out_hi, out_lo, status, st);
}

hipError_t launch_attention(const uint16_t* q_hi, const uint16_t* q_lo, int32_t R,
                            const StepMeta& m, const RowMaps& maps, const ModelDims& md,
                            const AttnPlan& ap, const void* pool_k, const void* pool_v,
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

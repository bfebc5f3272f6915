// kernels_misc.hip -- step metadata preparation, embedding + RMSNorm,
// RMSNorm, RoPE + KV append, argmax combine, fills.
#include <algorithm>

#include "attn_sched.h"
#include "common.h"
#include "kernels.h"
#include "rope_append.h"

namespace cbd {

// ------------------------------------------------------------------- prep
//
// One workgroup turns the per-sequence metadata into per-row maps: the
// sequence and position of every row (rows are the sequences' n_new entries
// laid end to end, in order), the row each emitting sequence takes its token
// from (its last row), and where each sequence's attention work starts (its
// first key step in the per-tile schedule, or its first block-kernel item).
// Sequences whose metadata is out of range keep their place in the row
// layout but are refused: their rows get row_seq = -1 and no attention work.

#define PREP_THREADS 1024
#define PREP_WAVES (PREP_THREADS / 64)
// Sequences with more rows than PREP_SHORT (prefill chunks) have their rows
// written by a whole wave after the scan instead of by their own thread;
// up to PREP_QUEUE of them per step (any further ones: their own thread).
#define PREP_SHORT 4
#define PREP_QUEUE 256

struct PrepQueued {
  int s, r, n, ctx, seq, orow;
};

// Exclusive prefix sums over the workgroup of four per-thread counts, and
// their totals: a shuffle scan inside each wave, then the 16 wave totals.
__device__ int4 block_scan4(int4 v, int4* wave_tot, int4* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int4 inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(inc.x, o, 64), b = __shfl_up(inc.y, o, 64);
    const int c = __shfl_up(inc.z, o, 64), d = __shfl_up(inc.w, o, 64);
    if (lane >= o) {
      inc.x += a;
      inc.y += b;
      inc.z += c;
      inc.w += d;
    }
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  int4 base = make_int4(0, 0, 0, 0), tot = make_int4(0, 0, 0, 0);
#pragma unroll
  for (int w = 0; w < PREP_WAVES; ++w) {
    const int4 t = wave_tot[w];
    if (w < wave) {
      base.x += t.x;
      base.y += t.y;
      base.z += t.z;
      base.w += t.w;
    }
    tot.x += t.x;
    tot.y += t.y;
    tot.z += t.z;
    tot.w += t.w;
  }
  *total = tot;
  return make_int4(base.x + inc.x - v.x, base.y + inc.y - v.y, base.z + inc.z - v.z,
                   base.w + inc.w - v.w);
}

__device__ __forceinline__ void prep_write_row(const RowMaps& maps, int row, int seq, int pos,
                                               int out) {
  maps.row_seq[row] = seq;
  maps.row_pos[row] = pos;
  maps.row_out[row] = out;
}

__device__ void prep_body(const StepMeta& m, const RowMaps& maps, const ModelDims& md,
                          const AttnPlan& ap, uint32_t* status) {
  __shared__ int4 wave_tot[PREP_WAVES];
  __shared__ PrepQueued queue[PREP_QUEUE];
  __shared__ int q_cnt;
  const int t = threadIdx.x;
  const int n = m.n_seqs;
  const int per = (n + PREP_THREADS - 1) / PREP_THREADS;
  const int s0 = min(n, t * per), s1 = min(n, s0 + per);
  const int G = md.n_heads / md.n_kv_heads;  // query heads per KV head
  const int cap = m.max_blocks_per_seq * md.block_size;
  if (t == 0) q_cnt = 0;  // ordered before any use by the scan's barrier

  // A sequence is served when its counts fit the cache, the key splits, the
  // positions and its slot; its attention goes to the block kernel (block
  // items) or the per-tile kernel (key steps of its query tiles).
  auto valid = [&](int s, int nn, int ctx) {
    return attn_seq_valid(nn, ctx, m.slots[s], cap, ap, md.max_position, md.max_slots);
  };
  auto add_items = [&](int nn, int ctx, int& steps, int& items_b) {
    attn_seq_work(nn, ctx, G, md.n_kv_heads, ap, &steps, &items_b);
  };

  int4 cnt = make_int4(0, 0, 0, 0);  // rows, key steps, block items, outputs
  for (int s = s0; s < s1; ++s) {
    const int nn = m.n_new[s], ctx = m.ctx_lens[s];
    const int slot = m.slots[s];
    const bool ok = valid(s, nn, ctx);
    if (slot < 0 || slot >= md.max_slots)
      raise_status(status, ST_BAD_SLOT);
    else if (!ok)
      raise_status(status, ST_BAD_SHAPE);
    cnt.x += max(0, min(nn, m.n_rows));
    if (ok) add_items(nn, ctx, cnt.y, cnt.z);
    cnt.w += m.want_token[s] ? 1 : 0;
  }
  int4 tot;
  const int4 base = block_scan4(cnt, wave_tot, &tot);
  const bool counts_ok = tot.x == m.n_rows && tot.w == m.n_out;
  if (t == 0 && !counts_ok) raise_status(status, ST_BAD_SHAPE);

  int r = base.x, it = base.y, itb = base.z, o = base.w;
  for (int s = s0; s < s1; ++s) {
    const int nn = m.n_new[s], ctx = m.ctx_lens[s];
    const int nn_layout = max(0, min(nn, m.n_rows));
    const bool ok = counts_ok && valid(s, nn, ctx);
    maps.item0[s] = it;
    maps.item0b[s] = itb;
    maps.seq_row0[s] = r;
    int orow = -1;  // output index of the last row
    if (m.want_token[s]) {
      if (o < m.n_out) {
        maps.out_row[o] = ok ? r + nn_layout - 1 : -1;
        maps.out_seq[o] = s;
        if (ok) orow = o;
      }
      ++o;
    }
    if (counts_ok && nn_layout > 0) {  // with counts_ok every row lies below n_rows
      int q = PREP_QUEUE;
      if (nn_layout > PREP_SHORT) q = atomicAdd(&q_cnt, 1);
      if (q < PREP_QUEUE) {
        queue[q] = PrepQueued{s, r, nn_layout, ctx, ok ? s : -1, orow};
      } else {
        for (int i = 0; i < nn_layout; ++i)
          prep_write_row(maps, r + i, ok ? s : -1, ctx + i, i == nn_layout - 1 ? orow : -1);
      }
    }
    if (ok) add_items(nn, ctx, it, itb);
    r += nn_layout;
  }
  __syncthreads();
  if (t == 0) {
    maps.item0[n] = counts_ok ? tot.y : 0;
    maps.item0b[n] = counts_ok ? tot.z : 0;
  }
  // The queued sequences' rows, one wave per sequence.
  const int lane = t & 63, wave = t >> 6;
  const int nq = min(q_cnt, PREP_QUEUE);
  for (int e = wave; e < nq; e += PREP_WAVES) {
    const PrepQueued qe = queue[e];
    for (int i = lane; i < qe.n; i += 64)
      prep_write_row(maps, qe.r + i, qe.seq, qe.ctx + i, i == qe.n - 1 ? qe.orow : -1);
  }
  if (!counts_ok) {  // the layout cannot be trusted: refuse every row
    for (int i = t; i < m.n_rows; i += PREP_THREADS) {
      maps.row_seq[i] = -1;
      maps.row_out[i] = -1;
    }
    for (int i = t; i < m.n_out; i += PREP_THREADS) maps.out_row[i] = -1;
    for (int i = t; i < n; i += PREP_THREADS) maps.item0[i] = maps.item0b[i] = 0;
  } else {
    for (int i = tot.x + t; i < m.n_rows; i += PREP_THREADS) {
      maps.row_seq[i] = -1;
      maps.row_out[i] = -1;
    }
  }
}

// The embedding rows of the step, gathered by the other workgroups of the
// prep launch: row r = blockIdx.x - 1 becomes x[r] = E[tokens[r]] (fp32) and
// its RMSNorm, split into hi and lo planes (a token outside the vocabulary
// gives a zero row and ST_BAD_TOKEN). Rows of refused sequences are gathered
// too: prep runs beside this, and nothing downstream reads them.
#define EN_MAX_CHUNKS 2  // 8-column chunks per thread: d_model <= 8 * 2 * PREP_THREADS

__device__ void embed_row(int r, const int32_t* __restrict__ tokens,
                          const uint16_t* __restrict__ embed, const uint16_t* __restrict__ gain,
                          int d, int vocab, float eps, float* __restrict__ x,
                          uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo,
                          uint32_t* status) {
  __shared__ float red[PREP_WAVES];
  const int t = threadIdx.x;
  const int nch = d >> 3;
  const int tok = tokens[r];
  const bool ok = tok >= 0 && tok < vocab;
  if (!ok && t == 0) raise_status(status, ST_BAD_TOKEN);
  float* xr = x + (size_t)r * d;
  float xv[EN_MAX_CHUNKS][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < EN_MAX_CHUNKS; ++c) {
    const int ch = t + c * PREP_THREADS;
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[c][e] = 0.f;
    if (ch < nch) {
      if (ok) {
        const uint4 q = reinterpret_cast<const uint4*>(embed + (size_t)tok * d)[ch];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[c][2 * e] = lo_bf(w[e]);
          xv[c][2 * e + 1] = hi_bf(w[e]);
        }
      }
      reinterpret_cast<float4*>(xr)[2 * ch] = make_float4(xv[c][0], xv[c][1], xv[c][2], xv[c][3]);
      reinterpret_cast<float4*>(xr)[2 * ch + 1] = make_float4(xv[c][4], xv[c][5], xv[c][6], xv[c][7]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += xv[c][e] * xv[c][e];
    }
  }
  ss = wave_sum(ss);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < PREP_WAVES; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  const int KB = (d + 31) / 32;
#pragma unroll
  for (int c = 0; c < EN_MAX_CHUNKS; ++c) {
    const int ch = t + c * PREP_THREADS;
    if (ch < nch) {
      const uint4 q = reinterpret_cast<const uint4*>(gain)[ch];
      const uint32_t g[4] = {q.x, q.y, q.z, q.w};
      float y[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[2 * e] = xv[c][2 * e] * inv * lo_bf(g[e]);
        y[2 * e + 1] = xv[c][2 * e + 1] * inv * hi_bf(g[e]);
      }
      store_split8(h_hi, h_lo, tile_at(r, 8 * ch, KB), y);
    }
  }
}

// One launch for the step's start: workgroup 0 builds the row maps and the
// attention schedule, workgroups 1 .. n_rows gather and normalise the
// embedding rows (the two depend on nothing of each other).
__global__ __launch_bounds__(PREP_THREADS) void prep_embed_kernel(
    StepMeta m, RowMaps maps, ModelDims md, AttnPlan ap, const uint16_t* __restrict__ embed,
    const uint16_t* __restrict__ gain, float* __restrict__ x, uint16_t* __restrict__ h_hi,
    uint16_t* __restrict__ h_lo, uint32_t* status) {
  if (blockIdx.x == 0)
    prep_body(m, maps, md, ap, status);
  else
    embed_row(blockIdx.x - 1, m.tokens, embed, gain, md.d_model, md.vocab, md.rms_eps, x, h_hi,
              h_lo, status);
}

hipError_t launch_prep_embed(const StepMeta& m, const RowMaps& maps, const ModelDims& md,
                             const AttnPlan& ap, const uint16_t* embed, const uint16_t* gain,
                             float* x, uint16_t* h_hi, uint16_t* h_lo, uint32_t* status,
                             hipStream_t st) {
  if ((md.d_model >> 3) > EN_MAX_CHUNKS * PREP_THREADS) return hipErrorInvalidValue;
  prep_embed_kernel<<<1 + m.n_rows, PREP_THREADS, 0, st>>>(m, maps, md, ap, embed, gain, x, h_hi,
                                                            h_lo, status);
  return hipGetLastError();
}

// ---------------------------------------------------------------- RMSNorm
//
// One workgroup per row, one 8-column chunk of the row per thread (up to
// RN_MAX_CHUNKS when the row is wider than the workgroup): the residual sum
// (the split partials of a chunk are loaded four splits at a time and added
// in split order), then the norm of the new x, stored as one 16-byte run of
// an operand tile per plane. Wide workgroups keep many loads in flight,
// since only one workgroup per row works here.
#define RN_MAX_CHUNKS 2

__global__ __launch_bounds__(1024) void resid_norm_kernel(
    float* __restrict__ x, const float* __restrict__ part, int S, int R,
    const int32_t* __restrict__ row_out, const int32_t* __restrict__ out_row,
    const uint16_t* __restrict__ gain, int d, float eps, uint16_t* __restrict__ h_hi,
    uint16_t* __restrict__ h_lo) {
  __shared__ float red[16];
  const int T = blockDim.x, t = threadIdx.x;
  const int nch = d >> 3;
  const int KB = (d + 31) / 32;
  const int r = blockIdx.x;
  if (r >= R) {  // output o = r - R with no row (refused): zeros, finite downstream
    const int o = r - R;
    if (out_row[o] >= 0) return;
    for (int ch = t; ch < nch; ch += T) {
      *reinterpret_cast<uint4*>(h_hi + tile_at(o, 8 * ch, KB)) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(h_lo + tile_at(o, 8 * ch, KB)) = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  float* xr = x + (size_t)r * d;
  const size_t pstride = (size_t)R * d / 4;  // one split's partials, in float4
  float4 xa[RN_MAX_CHUNKS], xb[RN_MAX_CHUNKS];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < RN_MAX_CHUNKS; ++c) {
    const int ch = t + c * T;
    xa[c] = xb[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ch < nch) {
      float4 a = reinterpret_cast<const float4*>(xr)[2 * ch];
      float4 b = reinterpret_cast<const float4*>(xr)[2 * ch + 1];
      if (S > 1) {
        const float4* p = reinterpret_cast<const float4*>(part + (size_t)r * d) + 2 * ch;
        for (int k0 = 0; k0 < S; k0 += 4) {
          float4 qa[4], qb[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (k0 + u < S) {
              qa[u] = p[(k0 + u) * pstride];
              qb[u] = p[(k0 + u) * pstride + 1];
            }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (k0 + u < S) {
              a.x += qa[u].x; a.y += qa[u].y; a.z += qa[u].z; a.w += qa[u].w;
              b.x += qb[u].x; b.y += qb[u].y; b.z += qb[u].z; b.w += qb[u].w;
            }
        }
        reinterpret_cast<float4*>(xr)[2 * ch] = a;
        reinterpret_cast<float4*>(xr)[2 * ch + 1] = b;
      }
      xa[c] = a;
      xb[c] = b;
      ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z +
            b.w * b.w;
    }
  }
  const int dst = row_out ? row_out[r] : r;
  if (dst < 0) return;  // the whole workgroup: no barrier below is skipped by part of it
  ss = wave_sum(ss);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < (T >> 6); ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int c = 0; c < RN_MAX_CHUNKS; ++c) {
    const int ch = t + c * T;
    if (ch < nch) {
      const uint4 g = reinterpret_cast<const uint4*>(gain)[ch];
      const float y[8] = {xa[c].x * inv * lo_bf(g.x), xa[c].y * inv * hi_bf(g.x),
                          xa[c].z * inv * lo_bf(g.y), xa[c].w * inv * hi_bf(g.y),
                          xb[c].x * inv * lo_bf(g.z), xb[c].y * inv * hi_bf(g.z),
                          xb[c].z * inv * lo_bf(g.w), xb[c].w * inv * hi_bf(g.w)};
      store_split8(h_hi, h_lo, tile_at(dst, 8 * ch, KB), y);
    }
  }
}

hipError_t launch_resid_norm(float* x, const float* part, int32_t S, int32_t R,
                             const int32_t* row_out, const int32_t* out_row, int32_t n_out,
                             const uint16_t* gain, int32_t d, float eps, uint16_t* h_hi,
                             uint16_t* h_lo, hipStream_t st) {
  if (R <= 0) return hipSuccess;
  const int nch = d / 8;
  int T = (nch + RN_MAX_CHUNKS - 1) / RN_MAX_CHUNKS;  // threads for at most RN_MAX_CHUNKS each
  T = std::max(T, std::min(nch, 1024));               // and up to one chunk per thread
  T = std::min(1024, (T + 63) / 64 * 64);
  if ((size_t)T * RN_MAX_CHUNKS < (size_t)nch) return hipErrorInvalidValue;
  const int extra = row_out ? n_out : 0;
  resid_norm_kernel<<<R + extra, T, 0, st>>>(x, part, S, R, row_out, out_row, gain, d, eps, h_hi,
                                             h_lo);
  return hipGetLastError();
}

// ------------------------------------------------------- RoPE + KV append
//
// Block (hd/2, 4): x = pair index i, y = one of four head slots of row r;
// each thread does one element pair (rope_append.h: the QKV split-K sum, the
// rotation in fp64, the query split into hi and lo planes, the K/V rounded
// once into the sequence's block).

__global__ void rope_append_kernel(RopeAppendArgs a, const int32_t* __restrict__ row_seq,
                                   const int32_t* __restrict__ row_pos, uint32_t* status) {
  const int slots = a.hq + 2 * a.hkv;
  const int groups = (slots + 3) / 4;
  const int r = blockIdx.x / groups;
  const int j = (blockIdx.x % groups) * 4 + threadIdx.y;
  if (r >= a.R || j >= slots) return;
  const int s = row_seq[r];
  if (s < 0) return;
  rope_append_one(a, r, s, row_pos[r], j, threadIdx.x, status);
}

RopeAppendArgs rope_append_args(float* qkv, const float* part, int32_t S, int32_t R,
                                const StepMeta& m, const double* rope_cs, const ModelDims& md,
                                uint16_t* q_hi, uint16_t* q_lo, void* pool_k, void* pool_v) {
  return RopeAppendArgs{qkv, part, S, R, reinterpret_cast<const double2*>(rope_cs),
                        m.block_tables, m.max_blocks_per_seq, md.n_heads, md.n_kv_heads,
                        md.head_dim, md.block_size, md.num_blocks, q_hi, q_lo, pool_k, pool_v,
                        md.kv_fp8, md.k_scale, md.v_scale};
}

hipError_t launch_rope_append(float* qkv, const float* part, int32_t S, int32_t R,
                              const StepMeta& m, const RowMaps& maps, const double* rope_cs,
                              const ModelDims& md, uint16_t* q_hi, uint16_t* q_lo,
                              void* pool_k, void* pool_v, uint32_t* status, hipStream_t st) {
  if (R <= 0) return hipSuccess;
  const int slots = md.n_heads + 2 * md.n_kv_heads;
  const int groups = (slots + 3) / 4;
  dim3 block(md.head_dim / 2, 4);
  rope_append_kernel<<<R * groups, block, 0, st>>>(
      rope_append_args(qkv, part, S, R, m, rope_cs, md, q_hi, q_lo, pool_k, pool_v), maps.row_seq,
      maps.row_pos, status);
  return hipGetLastError();
}

// ---------------------------------------------------------- argmax combine
//
// One workgroup of 256 threads per row: the maximum over the per-tile
// partials, lowest id on equal values (ids are unique per partial, so the
// order is total). Each thread scans a strided share, the four waves reduce
// by shuffles and then through LDS.

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void argmax_reduce_kernel(const float* __restrict__ val,
                                                            const int32_t* __restrict__ idx,
                                                            int n_tiles, int stride,
                                                            int32_t* __restrict__ tokens) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int j = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int t = threadIdx.x; t < n_tiles; t += 256) {
    const float v = val[(size_t)j * stride + t];
    const int i = idx[(size_t)j * stride + t];
    if (better(v, i, bv, bi)) {
      bv = v;
      bi = i;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v = __shfl_xor(bv, o, 64);
    const int i = __shfl_xor(bi, o, 64);
    if (better(v, i, bv, bi)) {
      bv = v;
      bi = i;
    }
  }
  if ((threadIdx.x & 63) == 0) {
    sv[threadIdx.x >> 6] = bv;
    si[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], bv, bi)) {
        bv = sv[w];
        bi = si[w];
      }
    tokens[j] = bi == 0x7fffffff ? 0 : bi;
  }
}

hipError_t launch_argmax_reduce(const float* amax_val, const int32_t* amax_idx, int32_t n_tiles,
                                int32_t stride, int32_t n, int32_t* tokens, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  argmax_reduce_kernel<<<n, 256, 0, st>>>(amax_val, amax_idx, n_tiles, stride, tokens);
  return hipGetLastError();
}

// ------------------------------------------------------------------- fill

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t step = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += step) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_u32_kernel<<<(unsigned)blocks, 256, 0, st>>>(p, value, n);
  return hipGetLastError();
}

}  // namespace cbd

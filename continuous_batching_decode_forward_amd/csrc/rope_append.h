// rope_append.h -- one element pair of the QKV split-K sum + RoPE + paged KV
// append, shared by the standalone RoPE/append kernel and the attention row
// kernel (which does this work for its own sequence and KV head before
// attending).
//
// Row r, head slot j, pair index i (element i pairs with i + hd/2). Head
// slots 0..Hq-1 are query heads (rotated into q, split into hi and lo
// planes), then Hkv key heads (rotated, rounded to bf16 -- or E4M3 codes of
// value / k_scale -- into the K tile [block][kvh][pos % bs][hd]) and Hkv
// value heads (rounded the same way, dimension-major, into the V tile
// [block][kvh][hd][pos % bs]). The rotation reads a host-built fp64 table
// of (cos, sin) per (position, i) and is evaluated in fp64, so a cached key
// is its exact rotation rounded once. The summed projection is written back
// to qkv (for inspection). The caller has checked that row r belongs to a
// served sequence s at position pos.
#pragma once

#include "common.h"
#include "kernels.h"

namespace cbd {

struct RopeAppendArgs {
  float* qkv;          // [R][slots * hd] fp32 projection (the sum when split)
  const float* part;   // S split partials of it, [S][R][slots * hd]
  int S, R;
  const double2* rope_cs;  // [max_position][hd / 2] (cos, sin)
  const int32_t* tables;   // block tables [n_seqs][max_blocks_per_seq]
  int max_blocks_per_seq;
  int hq, hkv, hd, bs, num_blocks;
  uint16_t* q_hi;
  uint16_t* q_lo;
  void* pool_k;
  void* pool_v;
  int kv_fp8;
  float k_scale, v_scale;
};

// The arguments of one step's RoPE + append (host).
RopeAppendArgs rope_append_args(float* qkv, const float* part, int32_t S, int32_t R,
                                const StepMeta& m, const double* rope_cs, const ModelDims& md,
                                uint16_t* q_hi, uint16_t* q_lo, void* pool_k, void* pool_v);

__device__ __forceinline__ void rope_append_one(const RopeAppendArgs& a, int r, int s, int pos,
                                                int j, int i, uint32_t* status) {
  const int slots = a.hq + 2 * a.hkv;
  const int hd = a.hd, half = hd >> 1, hq = a.hq, hkv = a.hkv, bs = a.bs;
  float* src = a.qkv + (size_t)r * slots * hd + (size_t)j * hd;
  float x, y;
  if (a.S > 1) {  // the projection's split partials, summed in split order
    const size_t stride = (size_t)a.R * slots * hd;
    const float* p = a.part + (size_t)r * slots * hd + (size_t)j * hd;
    x = p[i];
    y = p[i + half];
    for (int k = 1; k < a.S; ++k) {
      x += p[k * stride + i];
      y += p[k * stride + i + half];
    }
    src[i] = x;  // the projection itself, for inspection
    src[i + half] = y;
  } else {
    x = src[i];
    y = src[i + half];
  }
  if (j < hq + hkv) {
    const double2 cs = a.rope_cs[(size_t)pos * half + i];
    const double dx = x, dy = y;
    // fp64 -> fp32 -> bf16 for keys: the double rounding can only matter
    // within 2^-29 of a bf16 halfway point.
    x = (float)(dx * cs.x - dy * cs.y);
    y = (float)(dy * cs.x + dx * cs.y);
  }
  if (j < hq) {
    const size_t at = (size_t)r * hq * hd + (size_t)j * hd;
    bf16_t h, l;
    split_bf(x, h, l);
    a.q_hi[at + i] = h;
    a.q_lo[at + i] = l;
    split_bf(y, h, l);
    a.q_hi[at + i + half] = h;
    a.q_lo[at + i + half] = l;
    return;
  }
  const int blk = a.tables[(size_t)s * a.max_blocks_per_seq + pos / bs];
  if (blk < 0 || blk >= a.num_blocks) {
    if (i == 0) raise_status(status, ST_BAD_BLOCK);
    return;
  }
  const int off = pos % bs;
  if (a.kv_fp8) {  // E4M3 codes of value / scale
    if (j < hq + hkv) {
      const int g = j - hq;
      uint8_t* dst = static_cast<uint8_t*>(a.pool_k) + (((size_t)blk * hkv + g) * bs + off) * hd;
      dst[i] = f2e4m3(x / a.k_scale);
      dst[i + half] = f2e4m3(y / a.k_scale);
    } else {
      const int g = j - hq - hkv;
      uint8_t* dst = static_cast<uint8_t*>(a.pool_v) + ((size_t)blk * hkv + g) * hd * bs + off;
      dst[(size_t)i * bs] = f2e4m3(x / a.v_scale);
      dst[(size_t)(i + half) * bs] = f2e4m3(y / a.v_scale);
    }
    return;
  }
  if (j < hq + hkv) {
    const int g = j - hq;
    uint16_t* dst = static_cast<uint16_t*>(a.pool_k) + (((size_t)blk * hkv + g) * bs + off) * hd;
    dst[i] = f2bf(x);
    dst[i + half] = f2bf(y);
  } else {
    const int g = j - hq - hkv;
    uint16_t* dst = static_cast<uint16_t*>(a.pool_v) + ((size_t)blk * hkv + g) * hd * bs + off;
    dst[(size_t)i * bs] = f2bf(x);
    dst[(size_t)(i + half) * bs] = f2bf(y);
  }
}

}  // namespace cbd

// attn_sched.h -- the attention work schedule of one step, as plain integer
// arithmetic shared by the host (the launch plan, and a host replay of the
// schedule) and the device (the prep kernel's per-sequence counts, the two
// attention kernels' segment and item decoding, the combine's partial
// count). Selective batching (Go under the hood 20.3.2, after Orca):
// attention runs per sequence at its own length, reading its K/V through its
// block table (PagedAttention's fixed-size blocks, same section).
//
// Per-tile schedule. The key steps (32 keys) of every (sequence, query tile)
// on the per-tile kernel are laid end to end in sequence order, the same for
// each KV head: T steps per head, sequence s starting at step item0[s]. A
// query tile is 16 query columns: 16/G consecutive rows of the sequence
// times the G query heads of one KV head; tile qt holds keys 0 .. ctx + its
// last row. Each head's T steps are cut into pieces of `len` steps; piece q
// of head g is run by wave g * per_head + q (mod the launched waves). A piece
// may cross (sequence, tile) boundaries; each run of it inside one (sequence,
// tile) is a segment with its own partial result, stored at split index
// "piece - first piece of that (sequence, tile)".
//
// Block schedule (prefill chunks of block_min rows or more): work items are
// (row block of block_rows rows, key split of split_len keys, KV head), item
// numbering sequence by sequence from item0b[s].
#pragma once

#include <stdint.h>

#include "kernels.h"

#if defined(__HIP__)
#define CBD_HD __host__ __device__ __forceinline__
#else
#define CBD_HD inline
#endif

namespace cbd {

CBD_HD int imin(int a, int b) { return a < b ? a : b; }
CBD_HD int imax(int a, int b) { return a > b ? a : b; }
CBD_HD int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Partial-result slots per (row, head): one per 128 positions (at most 64),
// plus one for a piece of the per-tile schedule that starts inside the range.
CBD_HD int attn_cap_splits(int max_position) {
  return imax(1, imin(64, ceil_div(max_position, 128))) + 1;
}

// Longest key split (and piece): its block-table slice fits ATT_TBL entries.
CBD_HD int attn_split_cap(int block_size) { return (ATT_TBL - 1) * block_size / 32 * 32; }

// The launch plan of one step (host). cus_waves: resident waves of the
// per-tile kernel on the device (two per SIMD). n_rows, n_seqs, max_ctx: the
// step's host scalars. kv_fp8: an 8-bit cache, whose chunks stay on the
// per-tile kernel.
inline AttnPlan plan_attention(int n_heads, int n_kv_heads, int block_size, int max_position,
                               int cus_waves, int n_seqs, int n_rows, int max_ctx,
                               int kv_fp8 = 0) {
  AttnPlan ap;
  ap.max_splits = attn_cap_splits(max_position);
  ap.max_ctx = max_ctx;
  // Block kernel (prefill chunks): keys split into split_len pieces, enough
  // items to fill the chip (about 4096) without slivers shorter than 64
  // keys; never more splits than the partial buffers hold.
  long long want = (long long)max_ctx * n_seqs * n_kv_heads / 4096;
  if (want < 64) want = 64;
  if (want > 4096) want = 4096;
  int len = ((int)want + 31) / 32 * 32;
  int floor_len = ceil_div(max_ctx, ap.max_splits);
  floor_len = (floor_len + 31) / 32 * 32;
  ap.split_len = imax(imin(len, attn_split_cap(block_size)), floor_len);
  const int G = n_heads / n_kv_heads;
  const long long qt = ((long long)n_rows * G + 15) / 16 + n_seqs;
  const long long sp = ceil_div(max_ctx, ap.split_len);
  // Per-tile kernel: equal pieces of each KV head's key steps (a piece at
  // least 2 steps, and long enough that the pieces over one (sequence, tile)
  // fit the partial slots; at most what a block-table slice in LDS covers),
  // run by the chip's resident waves, or fewer when the step has few keys.
  // (A floor of 2 rather than 4 took the 2B 28-layer decode step at B = 8
  // from 2.04 to 1.98 ms; 1 was no better.)
  const int steps_max = ceil_div(max_ctx, 32);
  ap.piece_hi = attn_split_cap(block_size) / 32;
  ap.piece_lo = imax(2, ceil_div(steps_max, ap.max_splits - 1));
  const long long unit = (long long)n_kv_heads * ATT_WAVES;
  long long p_max = cus_waves / unit;
  if (p_max < 1) p_max = 1;
  p_max *= unit;
  const long long p_want = n_kv_heads * ((qt * steps_max + ap.piece_lo - 1) / ap.piece_lo);
  const long long p_fit = (p_want + unit - 1) / unit * unit;
  ap.grid_items = (int32_t)(p_max < p_fit ? p_max : p_fit);
  // Prefill chunks of 32+ rows run on the block kernel (block sizes that
  // are multiples of 32). Every sequence has at least one row, so a step
  // with fewer than block_min + n_seqs - 1 rows has no such chunk: it
  // launches no block kernel and every sequence runs on the per-tile kernel.
  ap.block_min = 32;
  ap.block_rows = block_size % 32 == 0 && !kv_fp8 ? ATT_BLOCK_COLS / G : 0;
  if ((long long)n_rows - n_seqs + 1 < ap.block_min) ap.block_rows = 0;
  ap.grid_items_b = 0;
  if (ap.block_rows > 0) {
    const long long qb = n_rows / ap.block_rows + n_seqs;
    long long items = qb * sp * n_kv_heads;
    if (items > (1LL << 30)) items = 1LL << 30;
    ap.grid_items_b = (int32_t)items;
  }
  // One row per sequence (every n_new is 1 when the rows number the
  // sequences) over at most ATT_ROW_KEYS keys, one (sequence, KV head)
  // workgroup per CU at most: the row kernel, whose workgroup merges its own
  // waves' results, so no combine launch follows. Measured against the
  // per-tile kernel + combine on the 8B layer over contexts U[16, 1023]:
  // 256 workgroups 37 -> 28 us; 512 and 2048 (more than one per CU, rows of
  // unequal length) 4 and 24 us slower; 8 (one row) 3 us slower. The 2B
  // 28-layer decode step at 64 and 256 workgroups: 2.0-2.1 -> 1.91 ms and
  // 2.41-2.43 -> 2.30 ms.
  const int row_wgs = n_seqs * n_kv_heads;
  ap.row_kernel = n_rows == n_seqs && max_ctx <= ATT_ROW_KEYS && G <= ATT_ROW_G &&
                  row_wgs >= ATT_ROW_MIN_WG && row_wgs <= cus_waves / ATT_ROW_WAVES;
  return ap;
}

// A sequence is served when its counts fit its block table (cap = max
// blocks per sequence x block size), the key splits, the positions, the
// launch bound and its slot; otherwise its rows are refused.
CBD_HD bool attn_seq_valid(int nn, int ctx, int slot, int cap, const AttnPlan& ap,
                           int max_position, int max_slots) {
  return nn >= 1 && ctx >= 0 && ctx + nn <= cap && ctx + nn <= ap.max_splits * ap.split_len &&
         ctx + nn <= max_position && ctx + nn <= ap.max_ctx && slot >= 0 && slot < max_slots;
}

// Whether a (served) sequence's attention runs on the block kernel.
CBD_HD bool attn_on_block_kernel(int nn, const AttnPlan& ap) {
  return ap.block_rows > 0 && nn >= ap.block_min;
}

// Key steps of query tile qt of a sequence (its keys are positions
// 0 .. ctx + its last row). rpt: rows per tile = 16 / G.
CBD_HD int tile_steps(int qt, int nn, int ctx, int rpt) {
  return ceil_div(ctx + imin(nn, (qt + 1) * rpt), 32);
}

// A served sequence's share of the schedule: per-tile key steps (per KV
// head) added to *steps, or block-kernel items added to *items_b.
CBD_HD void attn_seq_work(int nn, int ctx, int G, int n_kv_heads, const AttnPlan& ap, int* steps,
                          int* items_b) {
  if (attn_on_block_kernel(nn, ap)) {
    const int splits = ceil_div(ctx + nn, ap.split_len);
    *items_b += n_kv_heads * ceil_div(nn, ap.block_rows) * splits;
  } else {
    const int rpt = 16 / G, qtiles = ceil_div(nn * G, 16);
    for (int qt = 0; qt < qtiles; ++qt) *steps += tile_steps(qt, nn, ctx, rpt);
  }
}

// Largest s with item0[s] <= item (item0 ascending, item0[0] = 0).
CBD_HD int find_seq(const int32_t* item0, int n, int item) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (item0[mid] <= item)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

struct PieceSched {
  int len, per_head;
};

// The fewest rounds of the launched waves whose pieces fit in piece_hi
// steps, then the shortest pieces (not below piece_lo) that cover T steps in
// that many rounds.
CBD_HD PieceSched piece_sched(int T, const AttnPlan& ap, int n_kv_heads) {
  const int wh = imax(1, ap.grid_items / n_kv_heads);  // waves per KV head
  int rounds = imax(1, ceil_div(ceil_div(imax(T, 1), wh), ap.piece_hi));
  while (ceil_div(T, rounds * wh) > ap.piece_hi) ++rounds;
  const int len = imin(ap.piece_hi, imax(ap.piece_lo, ceil_div(T, rounds * wh)));
  PieceSched ps;
  ps.len = len;
  ps.per_head = ceil_div(T, len);
  return ps;
}

// The segment of piece q (steps [b, b_end) of one head) that starts at step
// b inside sequence s, whose schedule starts at step s0: its query tile, its
// keys [k_lo, k_hi), the partial slot sp it writes, and its length in steps.
struct Segment {
  int qt, k_lo, k_hi, sp, steps;
};

CBD_HD Segment piece_segment(int b, int b_end, int s0, int nn, int ctx, int q, int len,
                             int rpt) {
  const int off = b - s0;
  int qt = 0, qstart = 0, st = tile_steps(0, nn, ctx, rpt);
  while (off >= qstart + st) {
    qstart += st;
    st = tile_steps(++qt, nn, ctx, rpt);
  }
  const int rel = off - qstart;
  Segment sg;
  sg.qt = qt;
  sg.steps = imin(st - rel, b_end - b);
  sg.k_lo = 32 * rel;
  sg.k_hi = imin(ctx + imin(nn, (qt + 1) * rpt), 32 * (rel + sg.steps));
  sg.sp = q - (s0 + qstart) / len;
  return sg;
}

// Partial results the combine reads for the row at position pos of a
// per-tile sequence whose query tile qt starts at schedule step `start`:
// the pieces that hold steps start .. start + pos / 32.
CBD_HD int piece_partials(int start, int pos, int len) {
  return (start + pos / 32) / len - start / len + 1;
}

// First schedule step of query tile qt of a sequence starting at step s0.
CBD_HD int tile_start(int s0, int qt, int nn, int ctx, int rpt) {
  int start = s0;
  for (int t = 0; t < qt; ++t) start += tile_steps(t, nn, ctx, rpt);
  return start;
}

// Block-kernel item `local` (counted from the sequence's first item): its
// KV head g, split sp, rows [row_lo, last_row] of the chunk, keys
// [k_lo, k_hi) (empty when k_lo >= k_hi: the split lies past these rows).
struct BlockItem {
  int g, sp, row_lo, last_row, k_lo, k_hi;
};

CBD_HD BlockItem block_item(int local, int nn, int ctx, const AttnPlan& ap) {
  const int qblocks = ceil_div(nn, ap.block_rows);
  const int splits = ceil_div(ctx + nn, ap.split_len);
  BlockItem it;
  const int qb = local % qblocks;
  local /= qblocks;
  it.sp = local % splits;
  it.g = local / splits;
  it.row_lo = qb * ap.block_rows;
  it.last_row = imin(nn, it.row_lo + ap.block_rows) - 1;
  it.k_lo = it.sp * ap.split_len;
  it.k_hi = imin(it.k_lo + ap.split_len, ctx + it.last_row + 1);
  return it;
}

// Partial results the combine reads for a block-kernel row at position pos.
CBD_HD int block_partials(int pos, const AttnPlan& ap) { return pos / ap.split_len + 1; }

}  // namespace cbd

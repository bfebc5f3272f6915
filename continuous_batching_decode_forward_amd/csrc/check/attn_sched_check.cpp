// attn_sched_check.cpp -- a host replay of one step's attention schedule,
// built from the same schedule arithmetic the kernels run (attn_sched.h):
// the launch plan, the prep kernel's per-sequence counts, the per-tile
// kernel's piece and segment walk for every launched wave, the block
// kernel's item decoding for every launched workgroup, and the combine's
// partial counts. It checks, for a given step's metadata, every bound the
// kernels rely on without a device-side check:
//   - every segment and block item that loads K/V has keys (k_lo < k_hi);
//   - its block-table slice fits the LDS table (nb <= ATT_TBL) and lies
//     inside the sequence's table row, and the ids it stages are pool blocks;
//   - every partial slot written is below max_splits and belongs to a row
//     of the step, and no (row, head, slot) is written twice;
//   - every key step of every (sequence, KV head, query tile) is covered
//     exactly once, and the block kernel's grid holds every item;
//   - the combine reads exactly the partial slots that were written.
// Host-only; loaded by the tests, never by the library.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "../attn_sched.h"

using namespace cbd;

namespace {

struct Checker {
  int violations = 0;
  std::string first;
  void fail(const std::string& m) {
    if (violations++ == 0) first = m;
  }
};

}  // namespace

extern "C" {

// cfg: n_heads, n_kv_heads, head_dim, block_size, num_blocks, max_position,
// max_rows, max_slots, cus_waves, kv_fp8. Step arrays are host int32:
// slots[n_seqs], block_tables[n_seqs][mbps], ctx_lens[n_seqs],
// n_new[n_seqs]. stats (int64[8], nullable): per-tile segments, per-tile
// pieces, block items with keys, launched per-tile waves, block workgroups,
// the largest table slice, the largest partial slot, served sequences.
// Returns the number of violations; msg gets the first one.
int cbd_check_attention_schedule(const int32_t* cfg, int32_t n_seqs, int32_t n_rows,
                                 int32_t max_ctx, int32_t mbps, const int32_t* slots,
                                 const int32_t* block_tables, const int32_t* ctx_lens,
                                 const int32_t* n_new, int64_t* stats, char* msg,
                                 int32_t msg_len) {
  const int n_heads = cfg[0], kvh = cfg[1], bs = cfg[3], num_blocks = cfg[4];
  const int max_position = cfg[5], max_rows = cfg[6], max_slots = cfg[7], cus_waves = cfg[8];
  const int G = n_heads / kvh, rpt = 16 / G;
  Checker ck;
  char buf[256];
  const AttnPlan ap =
      plan_attention(n_heads, kvh, bs, max_position, cus_waves, n_seqs, n_rows, max_ctx, cfg[9]);
  int64_t st[8] = {0, 0, 0, 0, 0, 0, 0, 0};

  // The prep kernel: row layout, served sequences, schedule starts.
  const int cap = mbps * bs;
  std::vector<int32_t> item0(n_seqs + 1), item0b(n_seqs + 1), row0(n_seqs);
  std::vector<char> ok(n_seqs);
  long long rows = 0;
  for (int s = 0; s < n_seqs; ++s) rows += n_new[s] > 0 ? (n_new[s] < n_rows ? n_new[s] : n_rows) : 0;
  const bool counts_ok = rows == n_rows;
  int it = 0, itb = 0, r = 0;
  for (int s = 0; s < n_seqs; ++s) {
    ok[s] = counts_ok &&
            attn_seq_valid(n_new[s], ctx_lens[s], slots[s], cap, ap, max_position, max_slots);
    item0[s] = counts_ok ? it : 0;
    item0b[s] = counts_ok ? itb : 0;
    row0[s] = r;
    if (ok[s]) {
      attn_seq_work(n_new[s], ctx_lens[s], G, kvh, ap, &it, &itb);
      ++st[7];
    }
    r += n_new[s] > 0 ? n_new[s] : 0;
  }
  item0[n_seqs] = counts_ok ? it : 0;
  item0b[n_seqs] = counts_ok ? itb : 0;
  if (n_rows > max_rows) ck.fail("n_rows above max_rows");

  // (row, head, slot) written, and (sequence, head, tile, step) covered.
  std::set<std::tuple<int, int, int>> written;
  std::set<std::tuple<int, int, int, int>> covered;
  auto stage_table = [&](int s, int k_lo, int k_hi, const char* who) {
    const int b0 = k_lo / bs, nb = (k_hi - 1) / bs - b0 + 1;
    if (nb > ATT_TBL) {
      snprintf(buf, sizeof buf, "%s: seq %d keys [%d,%d) need %d table entries", who, s, k_lo, k_hi, nb);
      ck.fail(buf);
    }
    if (b0 + nb > mbps) {
      snprintf(buf, sizeof buf, "%s: seq %d table index %d past max_blocks_per_seq %d", who, s,
               b0 + nb - 1, mbps);
      ck.fail(buf);
      return;
    }
    for (int i = 0; i < nb; ++i) {
      const int blk = block_tables[(size_t)s * mbps + b0 + i];
      if (blk < 0 || blk >= num_blocks) {
        snprintf(buf, sizeof buf, "%s: seq %d block id %d at table index %d", who, s, blk, b0 + i);
        ck.fail(buf);
      }
    }
    if (nb > st[5]) st[5] = nb;
  };
  auto write_partial = [&](int row, int head, int sp, const char* who) {
    if (sp < 0 || sp >= ap.max_splits) {
      snprintf(buf, sizeof buf, "%s: partial slot %d outside [0, %d)", who, sp, ap.max_splits);
      ck.fail(buf);
    }
    if (row < 0 || row >= n_rows) {
      snprintf(buf, sizeof buf, "%s: partial of row %d outside the step", who, row);
      ck.fail(buf);
    }
    if (!written.insert(std::make_tuple(row, head, sp)).second) {
      snprintf(buf, sizeof buf, "%s: row %d head %d slot %d written twice", who, row, head, sp);
      ck.fail(buf);
    }
    if (sp > st[6]) st[6] = sp;
  };

  // The per-tile kernel: every launched wave walks its pieces.
  const int T = item0[n_seqs];
  const PieceSched ps = piece_sched(T, ap, kvh);
  const int n_pieces = ps.per_head * kvh;
  const int waves = ceil_div(ap.grid_items, ATT_WAVES) * ATT_WAVES;
  st[3] = waves;
  for (int first = 0; first < waves; ++first) {
    for (int p = first; p < n_pieces; p += ap.grid_items) {
      ++st[1];
      const int g = p / ps.per_head, q = p % ps.per_head;
      int b = q * ps.len;
      const int b_end = imin(T, b + ps.len);
      while (b < b_end) {
        const int s = find_seq(item0.data(), n_seqs, b);
        const int nn = n_new[s], ctx = ctx_lens[s];
        if (!ok[s] || attn_on_block_kernel(nn, ap)) {
          snprintf(buf, sizeof buf, "per-tile: step %d maps to seq %d, which has no per-tile work", b, s);
          ck.fail(buf);
          break;
        }
        const Segment sg = piece_segment(b, b_end, item0[s], nn, ctx, q, ps.len, rpt);
        ++st[0];
        if (sg.steps < 1) {
          ck.fail("per-tile: a segment of no steps");
          break;
        }
        if (sg.k_lo >= sg.k_hi) {
          snprintf(buf, sizeof buf, "per-tile: seq %d tile %d segment has no keys [%d,%d)", s, sg.qt,
                   sg.k_lo, sg.k_hi);
          ck.fail(buf);
        } else if (sg.sp < ap.max_splits) {  // the kernel refuses sp >= max_splits
          stage_table(s, sg.k_lo, sg.k_hi, "per-tile");
          for (int k = sg.k_lo / 32; k < ceil_div(sg.k_hi, 32); ++k)
            if (!covered.insert(std::make_tuple(s, g, sg.qt, k)).second) {
              snprintf(buf, sizeof buf, "per-tile: seq %d head %d tile %d step %d covered twice", s, g, sg.qt, k);
              ck.fail(buf);
            }
          for (int lr = 0; lr < 16; ++lr) {
            const int c_row = sg.qt * rpt + lr / G;
            if (lr >= rpt * G || c_row >= nn) continue;
            const int c_end = imin(sg.k_hi, ctx + c_row + 1);
            if (sg.k_lo < c_end) write_partial(row0[s] + c_row, g * G + lr % G, sg.sp, "per-tile");
          }
        } else {
          snprintf(buf, sizeof buf, "per-tile: seq %d partial slot %d >= max_splits %d", s, sg.sp,
                   ap.max_splits);
          ck.fail(buf);
        }
        b += sg.steps;
      }
    }
  }
  // Every key step of every per-tile (sequence, head, tile) was covered.
  for (int s = 0; s < n_seqs; ++s) {
    if (!ok[s] || attn_on_block_kernel(n_new[s], ap)) continue;
    for (int g = 0; g < kvh; ++g)
      for (int qt = 0; qt < ceil_div(n_new[s] * G, 16); ++qt)
        for (int k = 0; k < tile_steps(qt, n_new[s], ctx_lens[s], rpt); ++k)
          if (!covered.count(std::make_tuple(s, g, qt, k))) {
            snprintf(buf, sizeof buf, "per-tile: seq %d head %d tile %d step %d not covered", s, g, qt, k);
            ck.fail(buf);
          }
  }

  // The block kernel: every launched workgroup decodes its item.
  const int total_b = item0b[n_seqs];
  st[4] = ap.grid_items_b;
  if (total_b > 0 && ap.grid_items_b < total_b) {
    snprintf(buf, sizeof buf, "block: %d items but a grid of %d", total_b, ap.grid_items_b);
    ck.fail(buf);
  }
  for (int item = 0; item < ap.grid_items_b && item < total_b; ++item) {
    const int s = find_seq(item0b.data(), n_seqs, item);
    const int nn = n_new[s], ctx = ctx_lens[s];
    if (!ok[s] || !attn_on_block_kernel(nn, ap)) {
      snprintf(buf, sizeof buf, "block: item %d maps to seq %d, which has no block work", item, s);
      ck.fail(buf);
      continue;
    }
    const BlockItem bi = block_item(item - item0b[s], nn, ctx, ap);
    if (bi.g < 0 || bi.g >= kvh) {
      ck.fail("block: KV head out of range");
      continue;
    }
    if (bi.k_lo >= bi.k_hi) continue;  // the whole workgroup returns before any load
    ++st[2];
    stage_table(s, bi.k_lo, bi.k_hi, "block");
    for (int t = 0; t < ATT_BLOCK_COLS / 16; ++t)
      for (int lr = 0; lr < 16; ++lr) {
        const int c_row = bi.row_lo + t * rpt + lr / G;
        if (c_row > bi.last_row) continue;
        const int c_end = imin(bi.k_hi, ctx + c_row + 1);
        if (bi.k_lo < c_end) write_partial(row0[s] + c_row, bi.g * G + lr % G, bi.sp, "block");
      }
  }

  // The combine: each row reads exactly the partial slots that were written.
  for (int s = 0; s < n_seqs; ++s) {
    if (!ok[s]) continue;
    const int nn = n_new[s], ctx = ctx_lens[s];
    for (int i = 0; i < nn; ++i) {
      const int pos = ctx + i;
      int n_sp;
      if (attn_on_block_kernel(nn, ap))
        n_sp = block_partials(pos, ap);
      else
        n_sp = piece_partials(tile_start(item0[s], i / rpt, nn, ctx, rpt), pos, ps.len);
      if (n_sp < 1 || n_sp > ap.max_splits) {
        snprintf(buf, sizeof buf, "combine: row %d reads %d partials (max %d)", row0[s] + i, n_sp,
                 ap.max_splits);
        ck.fail(buf);
        continue;
      }
      for (int h = 0; h < n_heads; ++h) {
        for (int j = 0; j < n_sp; ++j)
          if (!written.count(std::make_tuple(row0[s] + i, h, j))) {
            snprintf(buf, sizeof buf, "combine: row %d head %d reads unwritten slot %d of %d",
                     row0[s] + i, h, j, n_sp);
            ck.fail(buf);
          }
        auto nxt = written.lower_bound(std::make_tuple(row0[s] + i, h, n_sp));
        if (nxt != written.end() && std::get<0>(*nxt) == row0[s] + i && std::get<1>(*nxt) == h) {
          snprintf(buf, sizeof buf, "combine: row %d head %d leaves slot %d unread", row0[s] + i,
                   h, std::get<2>(*nxt));
          ck.fail(buf);
        }
      }
    }
  }
  if (stats) memcpy(stats, st, sizeof st);
  if (msg && msg_len > 0) {
    strncpy(msg, ck.first.c_str(), (size_t)msg_len - 1);
    msg[msg_len - 1] = 0;
  }
  return ck.violations;
}

}  // extern "C"

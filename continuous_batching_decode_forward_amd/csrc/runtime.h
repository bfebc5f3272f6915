// runtime.h -- host runtime of the step: engine state, allocators, errors.
#pragma once

#include <stdint.h>

#include <deque>
#include <string>
#include <vector>

#include "../../include/cbd.h"
#include "kernels.h"

namespace cbd {

// Thread-local message of the last failure (cbd_last_error).
void set_error(const std::string& msg);
int fail(int code, const std::string& msg);

// Slot ids, lowest free first.
class SlotAllocator {
 public:
  void reset(int32_t n) {
    used_.assign((size_t)n, 0);
    n_free_ = n;
  }
  int32_t alloc() {
    for (size_t i = 0; i < used_.size(); ++i)
      if (!used_[i]) {
        used_[i] = 1;
        --n_free_;
        return (int32_t)i;
      }
    return -1;
  }
  bool release(int32_t s) {
    if (s < 0 || (size_t)s >= used_.size() || !used_[(size_t)s]) return false;
    used_[(size_t)s] = 0;
    ++n_free_;
    return true;
  }
  bool in_use(int32_t s) const { return s >= 0 && (size_t)s < used_.size() && used_[(size_t)s]; }
  int32_t n_free() const { return n_free_; }

 private:
  std::vector<uint8_t> used_;
  int32_t n_free_ = 0;
};

// Block ids: a FIFO free list seeded with a given order; allocation is
// all-or-nothing from the front, freed ids go to the back in the given order.
class BlockAllocator {
 public:
  bool reset(int32_t n, const int32_t* order) {
    free_.clear();
    used_.assign((size_t)n, 1);
    for (int32_t i = 0; i < n; ++i) {
      int32_t b = order ? order[i] : i;
      if (b < 0 || b >= n || !used_[(size_t)b]) return false;  // not a permutation
      used_[(size_t)b] = 0;
      free_.push_back(b);
    }
    return true;
  }
  bool alloc(int32_t n, int32_t* out) {
    if (n < 0 || (size_t)n > free_.size()) return false;
    for (int32_t i = 0; i < n; ++i) {
      out[i] = free_.front();
      free_.pop_front();
      used_[(size_t)out[i]] = 1;
    }
    return true;
  }
  bool release(int32_t n, const int32_t* ids) {
    for (int32_t i = 0; i < n; ++i)  // validate first: all or nothing
      if (ids[i] < 0 || (size_t)ids[i] >= used_.size() || !used_[(size_t)ids[i]]) return false;
    for (int32_t i = 0; i < n; ++i) {
      used_[(size_t)ids[i]] = 0;
      free_.push_back(ids[i]);
    }
    return true;
  }
  int32_t available() const { return (int32_t)free_.size(); }

 private:
  std::deque<int32_t> free_;
  std::vector<uint8_t> used_;
};

// Offsets (bytes) of everything the engine keeps in the caller's workspace.
struct WorkspaceLayout {
  size_t status, row_seq, row_pos, seq_row0, out_row, out_seq, item0, row_out, item0b;
  size_t x, h, qkv, q, attn, ffn, lm_in, logits, amax_val, amax_idx;
  size_t gemm_part, attn_ml, attn_o, rope, smp;
  size_t total;
  size_t gemm_part_floats;
  int32_t attn_max_splits;
  int32_t amax_stride;
};

struct SlotLayout {
  size_t params, counts, total;
};

// Element offsets of every projection matrix in the packed-weights buffer.
struct PackedLayout {
  std::vector<size_t> qkv, o, gate, up, down;  // per layer
  size_t lm_head;
  size_t total_elems;
};
PackedLayout packed_layout(const cbd_config& c);

int validate_config(const cbd_config* c);
WorkspaceLayout workspace_layout(const cbd_config& c);
SlotLayout slot_layout(const cbd_config& c);
size_t kv_pool_bytes(const cbd_config& c);

}  // namespace cbd

struct cbd_engine {
  cbd_config cfg;
  cbd::ModelDims md;
  cbd::WorkspaceLayout ws;
  cbd::SlotLayout sl;
  // weights (device pointers)
  const uint16_t* embed;
  const uint16_t* final_norm;
  const uint16_t* lm_head;
  std::vector<const uint16_t*> attn_norm, w_qkv, w_o, ffn_norm, w_gate, w_up, w_down;
  uint16_t* packed;
  cbd::PackedLayout pl;
  uint8_t* kv_pool;
  uint8_t* slot_state;
  uint8_t* workspace;
  hipStream_t stream;
  int32_t attn_waves;  // resident waves of the per-tile attention kernel (2 per SIMD)
  int32_t device;      // the device the engine was created on
  cbd::SlotAllocator slots;
  cbd::BlockAllocator blocks;
  std::vector<cbd::SlotParams> host_params;
  // recorded step graphs (cbd_step_forward_graph), least recently used first out
  struct GraphKey {
    cbd_step step;
    float* logits;
    int32_t* tokens;
  };
  struct GraphEntry {
    GraphKey key;
    hipGraphExec_t exec;
    uint64_t used;
  };
  std::vector<GraphEntry> graphs;
  uint64_t graph_clock = 0;
  int64_t graph_captures = 0, graph_replays = 0;
  // profiling: event pairs around launches of one kernel class
  int32_t prof_class = 0;
  std::vector<hipEvent_t> prof_events;  // created lazily, reused
  size_t prof_used = 0;
  ~cbd_engine();
  hipError_t prof_mark(int32_t cls, hipStream_t st);

  template <typename T>
  T* wsp(size_t off) const {
    return reinterpret_cast<T*>(workspace + off);
  }
  void* pool_k(int layer) const;  // bf16 values or E4M3 codes (cfg.kv_dtype)
  void* pool_v(int layer) const;
};

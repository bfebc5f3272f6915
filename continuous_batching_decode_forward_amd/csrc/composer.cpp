// composer.cpp -- the host step composer (Forma's "Scheduler", Go under the
// hood section 20.3.2), plus the library's error reporting.
//
// Each plan: admit what the policy allows, then compose the step:
//  1. prefill chunks of sequences that have no first token yet, in arrival
//     order, each min(chunk_size, remaining prompt, remaining row budget);
//  2. one row per decoding sequence while rows remain; sequences that have
//     waited longest for a row go first (ties by ascending slot), so a row
//     that does not fit waits one step and is then served -- nothing is ever
//     evicted.
// Other pacings (cbd_sched_config.pacing) compose the step differently:
// CBD_PACE_ALBATROSS puts decode rows first, feeds short prompts one token
// per step beside them, advances long prompts by a chunk only on every
// (ratio + 1)-th step while decode rows exist, and admits no more than
// max_prefill sequences into prefill at once; CBD_PACE_SEPARATE runs prefill
// chunks in steps of their own, without decode rows.
// Admission under CBD_ADMIT_RESERVE takes ceil((prompt + max_new) / block)
// blocks up front, which guarantees that every admitted request can finish
// (the deadlock the section describes -- all slots busy, pool empty, nobody
// can grow -- cannot arise). CBD_ADMIT_FREE_SLOT admits on a free slot and
// takes blocks as rows first write into them, and can stall.
// CBD_ADMIT_REQUEST_LEVEL admits a new group only once the batch is empty.
#include <string.h>

#include <algorithm>
#include <deque>
#include <list>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "runtime.h"

namespace cbd {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

}  // namespace cbd

using namespace cbd;

namespace {

struct Request {
  uint64_t id = 0;
  std::vector<int32_t> prompt;
  int32_t max_new = 0;
  cbd_sampling sp{};
  bool has_sp = false;
  int32_t slot = -1;
  std::vector<int32_t> blocks;
  int32_t ctx = 0;        // positions cached
  int32_t prefilled = 0;  // prompt tokens cached
  std::vector<int32_t> generated;
  int64_t last_row_step = -1;
};

struct Finished {
  uint64_t id;
  int32_t reason;
  int32_t n_generated;
};

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

}  // namespace

struct cbd_sched {
  cbd_sched_config cfg{};
  cbd_engine* engine = nullptr;
  SlotAllocator own_slots;
  BlockAllocator own_blocks;
  std::deque<std::unique_ptr<Request>> queue;
  std::map<int32_t, std::unique_ptr<Request>> active;  // by slot
  std::vector<Request*> order;                         // admitted, arrival order
  std::deque<Finished> finished;
  int64_t steps = 0, n_finished = 0;
  bool planned = false;
  // CBD_PACE_ALBATROSS: decode-carrying steps left before the next step
  // that may advance a long prompt
  int32_t seq_countdown = 0;
  int32_t max_prefill() const {
    return cfg.max_prefill > 0 ? cfg.max_prefill : std::max(cfg.max_slots / 8, 1);
  }
  int32_t ratio() const { return cfg.decode_prefill_ratio > 0 ? cfg.decode_prefill_ratio : 5; }
  int32_t min_fwd() const { return cfg.min_forward_seq_len > 0 ? cfg.min_forward_seq_len : 10; }
  int32_t n_prefilling() const {
    int32_t n = 0;
    for (const Request* r : order) n += r->prefilled < (int32_t)r->prompt.size();
    return n;
  }
  // the last plan
  std::vector<int32_t> p_slots, p_tables, p_ctx, p_new, p_tokens, p_want, p_step;
  std::vector<uint64_t> p_ids;
  std::vector<Request*> p_reqs;

  int32_t blocks_available() const {
    return engine ? cbd_blocks_available(engine) : own_blocks.available();
  }
  int32_t slots_free() const {
    if (!engine) return own_slots.n_free();
    return engine->slots.n_free();
  }
  bool take_blocks(int32_t n, std::vector<int32_t>& into) {
    if (n <= 0) return true;
    size_t at = into.size();
    into.resize(at + (size_t)n);
    bool ok = engine ? cbd_block_alloc(engine, n, into.data() + at) == CBD_OK
                     : own_blocks.alloc(n, into.data() + at);
    if (!ok) into.resize(at);
    return ok;
  }
  void give_blocks(std::vector<int32_t>& b) {
    if (b.empty()) return;
    if (engine)
      cbd_block_free(engine, (int32_t)b.size(), b.data());
    else
      own_blocks.release((int32_t)b.size(), b.data());
    b.clear();
  }
  int32_t take_slot(const Request& r) {
    if (!engine) return own_slots.alloc();
    int32_t s = -1;
    const cbd_sampling* p = r.has_sp ? &r.sp : nullptr;
    return cbd_slot_alloc(engine, p, r.id, &s) == CBD_OK ? s : -1;
  }
  void give_slot(int32_t s) {
    if (engine)
      cbd_slot_free(engine, s);
    else
      own_slots.release(s);
  }

  void retire(Request* r, int32_t reason) {
    give_blocks(r->blocks);
    give_slot(r->slot);
    finished.push_back({r->id, reason, (int32_t)r->generated.size()});
    ++n_finished;
    order.erase(std::find(order.begin(), order.end(), r));
    active.erase(r->slot);  // destroys r
  }

  void admit() {
    if (cfg.policy == CBD_ADMIT_REQUEST_LEVEL && !active.empty()) return;
    int32_t prefilling = n_prefilling();
    while (!queue.empty() && slots_free() > 0) {
      if (cfg.pacing == CBD_PACE_ALBATROSS && prefilling >= max_prefill()) break;
      Request& r = *queue.front();
      std::vector<int32_t> blocks;
      if (cfg.policy != CBD_ADMIT_FREE_SLOT) {
        int32_t need = ceil_div((int64_t)r.prompt.size() + r.max_new, cfg.block_size);
        if (blocks_available() < need || !take_blocks(need, blocks)) break;
      }
      int32_t slot = take_slot(r);
      if (slot < 0) {
        give_blocks(blocks);
        break;
      }
      std::unique_ptr<Request> up = std::move(queue.front());
      queue.pop_front();
      up->slot = slot;
      up->blocks = std::move(blocks);
      order.push_back(up.get());
      ++prefilling;
      active[slot] = std::move(up);
    }
  }

  // Free-slot-only policy: make r hold blocks for n_pos positions.
  bool grow(Request& r, int64_t n_pos) {
    int32_t need = ceil_div(n_pos, cfg.block_size) - (int32_t)r.blocks.size();
    if (need <= 0) return true;
    if (blocks_available() < need) return false;
    return take_blocks(need, r.blocks);
  }

  void emit(Request& r, const int32_t* toks, int32_t n, bool want) {
    r.last_row_step = steps;
    p_slots.push_back(r.slot);
    size_t at = p_tables.size();
    p_tables.resize(at + (size_t)cfg.max_blocks_per_seq, -1);
    std::copy(r.blocks.begin(), r.blocks.end(), p_tables.begin() + (ptrdiff_t)at);
    p_ctx.push_back(r.ctx);
    p_new.push_back(n);
    p_tokens.insert(p_tokens.end(), toks, toks + n);
    p_want.push_back(want ? 1 : 0);
    p_step.push_back((int32_t)r.generated.size());
    p_ids.push_back(r.id);
    p_reqs.push_back(&r);
  }
};

extern "C" {

int cbd_sched_create(const cbd_sched_config* cfg, cbd_engine* engine, const int32_t* block_order,
                     cbd_sched** out) {
  if (!cfg || !out) return fail(CBD_E_INVAL, "NULL config or output");
  if (cfg->max_slots < 1 || cfg->block_size < 1 || cfg->num_blocks < 1 ||
      cfg->max_blocks_per_seq < 1 || cfg->max_rows < 1 || cfg->chunk_size < 1 ||
      cfg->policy < CBD_ADMIT_RESERVE || cfg->policy > CBD_ADMIT_REQUEST_LEVEL ||
      cfg->pacing < CBD_PACE_PREFILL_FIRST || cfg->pacing > CBD_PACE_SEPARATE ||
      cfg->max_prefill < 0 || cfg->decode_prefill_ratio < 0 || cfg->min_forward_seq_len < 0 ||
      cfg->ctx_round < 0 || cfg->graph_decode < 0 || cfg->graph_decode > 1)
    return fail(CBD_E_INVAL, "composer config out of range");
  // With an engine, every plan the composer can make must be a step the
  // engine accepts: its sequences (at most max_slots) fit max_seqs, and a
  // sequence's positions (at most max_blocks_per_seq blocks) fit the RoPE
  // table, so the loop cannot fail in the middle of a run.
  if (engine && (engine->cfg.block_size != cfg->block_size ||
                 engine->cfg.num_blocks != cfg->num_blocks ||
                 engine->cfg.max_slots < cfg->max_slots ||
                 engine->cfg.max_seqs < cfg->max_slots ||
                 engine->cfg.max_blocks_per_seq < cfg->max_blocks_per_seq ||
                 (int64_t)engine->cfg.max_position <
                     (int64_t)cfg->max_blocks_per_seq * cfg->block_size ||
                 engine->cfg.max_rows < cfg->max_rows))
    return fail(CBD_E_INVAL, "composer config does not match the engine");
  std::unique_ptr<cbd_sched> s(new cbd_sched());
  s->cfg = *cfg;
  s->engine = engine;
  if (!engine) {
    s->own_slots.reset(cfg->max_slots);
    if (!s->own_blocks.reset(cfg->num_blocks, block_order))
      return fail(CBD_E_INVAL, "block_order is not a permutation of 0..num_blocks-1");
  }
  *out = s.release();
  return CBD_OK;
}

int cbd_sched_destroy(cbd_sched* s) {
  if (!s) return fail(CBD_E_INVAL, "composer is NULL");
  while (!s->order.empty()) s->retire(s->order.front(), CBD_FINISH_ABORT);
  delete s;
  return CBD_OK;
}

int cbd_sched_submit(cbd_sched* s, const int32_t* prompt, int32_t prompt_len, int32_t max_new,
                     const cbd_sampling* params, uint64_t request_id) {
  if (!s || !prompt || prompt_len < 1 || max_new < 1)
    return fail(CBD_E_INVAL, "empty prompt or max_new < 1");
  int32_t need = ceil_div((int64_t)prompt_len + max_new, s->cfg.block_size);
  if (need > s->cfg.max_blocks_per_seq || need > s->cfg.num_blocks)
    return fail(CBD_E_INVAL, "prompt + answer can never fit a sequence's block table or the pool");
  std::unique_ptr<Request> r(new Request());
  r->id = request_id;
  r->prompt.assign(prompt, prompt + prompt_len);
  r->max_new = max_new;
  if (params) {
    r->sp = *params;
    r->has_sp = true;
  }
  s->queue.push_back(std::move(r));
  return CBD_OK;
}

int cbd_sched_plan(cbd_sched* s, cbd_plan* out) {
  if (!s || !out) return fail(CBD_E_INVAL, "NULL composer or output");
  s->admit();
  s->p_slots.clear(); s->p_tables.clear(); s->p_ctx.clear(); s->p_new.clear();
  s->p_tokens.clear(); s->p_want.clear(); s->p_step.clear(); s->p_ids.clear();
  s->p_reqs.clear();
  int32_t budget = s->cfg.max_rows, n_prefill = 0, n_decode = 0;
  const int32_t pacing = s->cfg.pacing;
  // A prefill chunk of r: up to chunk_size rows (cut to the row budget);
  // under CBD_ADMIT_FREE_SLOT only when its blocks can be had.
  auto chunk = [&](Request* r, int32_t limit) {
    const int32_t left = (int32_t)r->prompt.size() - r->prefilled;
    const int32_t n = std::min({limit, left, budget});
    if (n <= 0) return false;
    if (s->cfg.policy == CBD_ADMIT_FREE_SLOT && !s->grow(*r, (int64_t)r->ctx + n)) return false;
    s->emit(*r, r->prompt.data() + r->prefilled, n, n == left);
    budget -= n;
    n_prefill += n;
    return true;
  };
  auto prefilling = [](const Request* r) { return r->prefilled < (int32_t)r->prompt.size(); };
  // One row per decoding sequence while rows remain, longest-waiting first.
  auto decode_rows = [&]() {
    std::vector<Request*> dec;
    for (auto& kv : s->active)
      if (!prefilling(kv.second.get())) dec.push_back(kv.second.get());
    std::stable_sort(dec.begin(), dec.end(), [](const Request* a, const Request* b) {
      if (a->last_row_step != b->last_row_step) return a->last_row_step < b->last_row_step;
      return a->slot < b->slot;
    });
    for (Request* r : dec) {
      if (budget <= 0) break;
      if (s->cfg.policy == CBD_ADMIT_FREE_SLOT && !s->grow(*r, (int64_t)r->ctx + 1)) continue;
      s->emit(*r, &r->generated.back(), 1, true);
      budget -= 1;
      ++n_decode;
    }
  };
  if (pacing == CBD_PACE_ALBATROSS) {
    decode_rows();
    for (Request* r : s->order)  // short prompts: one token per step
      if (budget > 0 && prefilling(r) && (int32_t)r->prompt.size() < s->min_fwd()) chunk(r, 1);
    if (s->seq_countdown == 0 || n_decode == 0) {
      bool ran = false;
      for (Request* r : s->order)  // long prompts: a chunk on this step
        if (budget > 0 && prefilling(r) && (int32_t)r->prompt.size() >= s->min_fwd())
          ran |= chunk(r, s->cfg.chunk_size);
      if (ran && n_decode > 0) s->seq_countdown = s->ratio();
    } else {
      --s->seq_countdown;
    }
  } else if (pacing == CBD_PACE_SEPARATE) {
    for (Request* r : s->order)
      if (budget > 0 && prefilling(r)) chunk(r, s->cfg.chunk_size);
    if (n_prefill == 0) decode_rows();
  } else {  // prefill first, arrival order; then the decode rows
    for (Request* r : s->order)
      if (budget > 0 && prefilling(r)) chunk(r, s->cfg.chunk_size);
    decode_rows();
  }
  out->n_seqs = (int32_t)s->p_slots.size();
  out->n_rows = (int32_t)s->p_tokens.size();
  out->n_out = 0;
  out->max_ctx = 0;
  for (size_t i = 0; i < s->p_slots.size(); ++i) {
    out->n_out += s->p_want[i];
    out->max_ctx = std::max(out->max_ctx, s->p_ctx[i] + s->p_new[i]);
  }
  out->max_blocks_per_seq = s->cfg.max_blocks_per_seq;
  out->n_prefill_rows = n_prefill;
  out->n_decode_rows = n_decode;
  out->stalled = (out->n_rows == 0 && !s->active.empty()) ? 1 : 0;
  out->slots = s->p_slots.data();
  out->block_tables = s->p_tables.data();
  out->ctx_lens = s->p_ctx.data();
  out->n_new = s->p_new.data();
  out->tokens = s->p_tokens.data();
  out->want_token = s->p_want.data();
  out->step_ids = s->p_step.data();
  out->request_ids = s->p_ids.data();
  s->planned = true;
  return CBD_OK;
}

int cbd_sched_commit(cbd_sched* s, const int32_t* tokens, int32_t n) {
  if (!s) return fail(CBD_E_INVAL, "composer is NULL");
  if (!s->planned) return fail(CBD_E_INVAL, "commit without a plan");
  int32_t want = 0;
  for (int32_t w : s->p_want) want += w;
  if (n != want || (n > 0 && !tokens)) return fail(CBD_E_INVAL, "token count does not match the plan");
  std::vector<std::pair<Request*, int32_t>> retire;
  int32_t o = 0;
  for (size_t i = 0; i < s->p_reqs.size(); ++i) {
    Request* r = s->p_reqs[i];
    r->ctx += s->p_new[i];
    if (r->prefilled < (int32_t)r->prompt.size()) r->prefilled += s->p_new[i];
    if (s->p_want[i]) {
      int32_t t = tokens[o++];
      r->generated.push_back(t);
      if (t == s->cfg.eos_id)
        retire.push_back({r, CBD_FINISH_EOS});
      else if ((int32_t)r->generated.size() >= r->max_new)
        retire.push_back({r, CBD_FINISH_LENGTH});
    }
  }
  for (auto& pr : retire) s->retire(pr.first, pr.second);
  s->p_reqs.clear();
  s->planned = false;
  ++s->steps;
  return CBD_OK;
}

int cbd_sched_abort(cbd_sched* s, uint64_t request_id) {
  if (!s) return fail(CBD_E_INVAL, "composer is NULL");
  if (s->planned) return fail(CBD_E_INVAL, "abort between plan and commit");
  for (Request* r : s->order)
    if (r->id == request_id) {
      s->retire(r, CBD_FINISH_ABORT);
      return CBD_OK;
    }
  for (auto it = s->queue.begin(); it != s->queue.end(); ++it)
    if ((*it)->id == request_id) {
      s->finished.push_back({request_id, CBD_FINISH_ABORT, 0});
      ++s->n_finished;
      s->queue.erase(it);
      return CBD_OK;
    }
  return fail(CBD_E_INVAL, "unknown request id");
}

int cbd_sched_pop_finished(cbd_sched* s, uint64_t* request_id, int32_t* reason,
                           int32_t* n_generated) {
  if (!s || !request_id || !reason || !n_generated) return fail(CBD_E_INVAL, "NULL argument");
  if (s->finished.empty()) return 0;
  Finished f = s->finished.front();
  s->finished.pop_front();
  *request_id = f.id;
  *reason = f.reason;
  *n_generated = f.n_generated;
  return 1;
}

int cbd_sched_stats_get(const cbd_sched* s, cbd_sched_stats* out) {
  if (!s || !out) return fail(CBD_E_INVAL, "NULL argument");
  out->queued = (int32_t)s->queue.size();
  out->active = (int32_t)s->active.size();
  out->free_slots = s->slots_free();
  out->free_blocks = s->blocks_available();
  out->steps = s->steps;
  out->finished = s->n_finished;
  return CBD_OK;
}

int cbd_sched_meta_ints(const cbd_sched_config* cfg, size_t* ints_out) {
  if (!cfg || !ints_out || cfg->max_slots < 1 || cfg->max_blocks_per_seq < 1 || cfg->max_rows < 1)
    return fail(CBD_E_INVAL, "NULL or out-of-range composer config");
  *ints_out = (size_t)cfg->max_slots * (5 + (size_t)cfg->max_blocks_per_seq) + cfg->max_rows;
  return CBD_OK;
}

int cbd_sched_step(cbd_sched* s, int32_t mode, int32_t* meta_dev, int32_t* host_stage,
                   int32_t* tokens_dev, float* logits_out, void* stream, cbd_plan* plan_out) {
  if (!s || !meta_dev || !host_stage || !tokens_dev)
    return fail(CBD_E_INVAL, "NULL composer or staging buffer");
  if (!s->engine) return fail(CBD_E_INVAL, "cbd_sched_step needs a composer created with an engine");
  if (mode != CBD_MODE_GREEDY && mode != CBD_MODE_SAMPLE) return fail(CBD_E_INVAL, "bad mode");
  cbd_plan p;
  int rc = cbd_sched_plan(s, &p);
  if (rc != CBD_OK) return rc;
  if (plan_out) *plan_out = p;
  if (p.n_rows == 0) return cbd_sched_commit(s, nullptr, 0);
  const size_t n = (size_t)p.n_seqs, mb = (size_t)p.max_blocks_per_seq;
  size_t o = 0;
  auto put = [&](const int32_t* src, size_t cnt) {
    memcpy(host_stage + o, src, cnt * sizeof(int32_t));
    const size_t at = o;
    o += cnt;
    return meta_dev + at;
  };
  cbd_step st;
  st.n_seqs = p.n_seqs;
  st.n_rows = p.n_rows;
  st.n_out = p.n_out;
  st.max_ctx = p.max_ctx;
  st.max_blocks_per_seq = p.max_blocks_per_seq;
  st.mode = mode;
  st.slots = put(p.slots, n);
  st.block_tables = put(p.block_tables, n * mb);
  st.ctx_lens = put(p.ctx_lens, n);
  st.n_new = put(p.n_new, n);
  st.tokens = put(p.tokens, (size_t)p.n_rows);
  st.want_token = put(p.want_token, n);
  st.step_ids = put(p.step_ids, n);
  // A decode-only step may take a rounded-up max_ctx (any upper bound is
  // valid) so that consecutive steps share one launch plan, and replay a
  // recorded graph of it.
  const bool decode_only = p.n_prefill_rows == 0;
  if (decode_only && s->cfg.ctx_round > 0) {
    const int64_t q = s->cfg.ctx_round;
    const int64_t r = ((int64_t)st.max_ctx + q - 1) / q * q;
    st.max_ctx = (int32_t)std::min<int64_t>(r, s->engine->cfg.max_position);
  }
  hipStream_t hs = (hipStream_t)stream;
  hipError_t he = hipMemcpyAsync(meta_dev, host_stage, o * sizeof(int32_t), hipMemcpyHostToDevice, hs);
  if (he != hipSuccess) return fail(CBD_E_DEVICE, std::string("step metadata upload: ") + hipGetErrorString(he));
  rc = decode_only && s->cfg.graph_decode
           ? cbd_step_forward_graph(s->engine, &st, logits_out, tokens_dev, stream)
           : cbd_step_forward(s->engine, &st, logits_out, tokens_dev, stream);
  if (rc != CBD_OK) {
    // The upload may still be reading host_stage: drain the stream before
    // handing the buffer back (the error message of the step is kept).
    const std::string msg = cbd_last_error();
    (void)hipStreamSynchronize(hs);
    return fail(rc, msg);
  }
  if (p.n_out > 0) {
    he = hipMemcpyAsync(host_stage, tokens_dev, (size_t)p.n_out * sizeof(int32_t),
                        hipMemcpyDeviceToHost, hs);
    if (he != hipSuccess) {
      (void)hipStreamSynchronize(hs);  // the upload may still read host_stage
      return fail(CBD_E_DEVICE, std::string("token download: ") + hipGetErrorString(he));
    }
  }
  he = hipStreamSynchronize(hs);
  if (he != hipSuccess) return fail(CBD_E_DEVICE, std::string("step: ") + hipGetErrorString(he));
  return cbd_sched_commit(s, host_stage, p.n_out);
}

const char* cbd_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

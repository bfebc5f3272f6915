// engine.cpp -- configuration checks, buffer layouts, engine lifecycle, slot
// and block allocation, and the per-step launch sequence.
#include <hip/hip_runtime.h>
#include <math.h>

#include <cmath>
#include <string.h>

#include <algorithm>
#include <string>
#include <utility>
#include <vector>

#include "attn_sched.h"
#include "runtime.h"

namespace cbd {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Per-row argmax partials of the LM head: one per 64-column wave tile of
// the stream path (in 8-wave groups, ceil(vocab / 512) * 8 <= vocab / 64 +
// 8) or per 128-column half tile of the dense path (ceil(vocab / 256) * 2).
static int32_t amax_stride(int32_t vocab) { return (vocab + 63) / 64 + 8; }

int validate_config(const cbd_config* c) {
  if (!c) return fail(CBD_E_INVAL, "config is NULL");
  if (c->n_layers < 1 || c->d_model < 1 || c->n_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 1 || c->ffn_dim < 1 || c->vocab < 2 || c->block_size < 1 ||
      c->num_blocks < 1 || c->max_blocks_per_seq < 1 || c->max_slots < 1 || c->max_rows < 1 ||
      c->max_seqs < 1 || c->max_position < 1 || !(c->rms_eps > 0.f) || !(c->rope_base > 1.0))
    return fail(CBD_E_INVAL, "config has a non-positive size or parameter");
  if (c->n_heads % c->n_kv_heads)
    return fail(CBD_E_INVAL, "n_heads must be a multiple of n_kv_heads");
  const int G = c->n_heads / c->n_kv_heads;
  if (16 % G)
    return fail(CBD_E_UNSUPPORTED, "query heads per KV head must divide 16 (1, 2, 4, 8, 16)");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(CBD_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->block_size != 4 && c->block_size != 8 && c->block_size != 16 && c->block_size != 32 &&
      c->block_size != 64)
    return fail(CBD_E_UNSUPPORTED, "block_size must be 4, 8, 16, 32 or 64");
  if (c->d_model % 16 || c->ffn_dim % 16 || c->vocab % 16)
    return fail(CBD_E_UNSUPPORTED, "d_model, ffn_dim and vocab must be multiples of 16");
  if (c->d_model > 8192) return fail(CBD_E_UNSUPPORTED, "d_model above 8192");
  if (c->kv_dtype != CBD_KV_BF16 && c->kv_dtype != CBD_KV_FP8_E4M3)
    return fail(CBD_E_INVAL, "unknown kv_dtype");
  if (!(c->k_scale >= 0.f) || !(c->v_scale >= 0.f) || !std::isfinite(c->k_scale) ||
      !std::isfinite(c->v_scale))
    return fail(CBD_E_INVAL, "k_scale and v_scale must be finite and non-negative");
  if (c->weight_dtype != CBD_W_BF16 && c->weight_dtype != CBD_W_INT8)
    return fail(CBD_E_INVAL, "unknown weight_dtype");
  if (c->kv_dtype == CBD_KV_FP8_E4M3 && c->block_size < 8)
    return fail(CBD_E_UNSUPPORTED, "an FP8 KV cache needs block_size 8, 16, 32 or 64");
  if (c->max_seqs > c->max_rows) return fail(CBD_E_INVAL, "max_seqs exceeds max_rows");
  if ((long long)(attn_cap_splits(c->max_position) - 1) * attn_split_cap(c->block_size) <
      c->max_position)
    return fail(CBD_E_UNSUPPORTED, "max_position too long for this block size");
  for (int32_t r = 1; r <= c->max_seqs; ++r)  // the LM head's plans at every output count
    if (gemm_amax_tiles(r, c->vocab, c->d_model, c->weight_dtype == CBD_W_INT8) >
        amax_stride(c->vocab))
      return fail(CBD_E_UNSUPPORTED, "LM-head argmax partials exceed their workspace stride");
  return CBD_OK;
}

WorkspaceLayout workspace_layout(const cbd_config& c) {
  WorkspaceLayout L;
  const size_t R = (size_t)c.max_rows, S = (size_t)c.max_seqs;
  const size_t d = (size_t)c.d_model, hd = (size_t)c.head_dim;
  const size_t qkv_n = (size_t)(c.n_heads + 2 * c.n_kv_heads) * hd;
  const size_t qd = (size_t)c.n_heads * hd;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.status = take(sizeof(uint32_t));
  L.row_seq = take(R * 4);
  L.row_pos = take(R * 4);
  L.seq_row0 = take(S * 4);
  L.out_row = take(R * 4);
  L.out_seq = take(R * 4);
  L.item0 = take((S + 1) * 4);
  L.row_out = take(R * 4);
  L.item0b = take((S + 1) * 4);
  // fp32 buffers [rows][w] and split buffers (hi plane bf16, then the lo
  // plane) both take 4 bytes per element; the split inputs of the
  // projections are in operand tiles, rows and columns padded to 16 and 32.
  L.x = take(R * d * 4);
  L.h = take(tile_plane_elems(R, d) * 4);
  L.qkv = take(R * qkv_n * 4);
  L.q = take(R * qd * 4);
  L.attn = take(tile_plane_elems(R, qd) * 4);
  L.ffn = take(tile_plane_elems(R, c.ffn_dim) * 4);
  L.lm_in = take(tile_plane_elems(S, d) * 4);
  L.logits = take(S * (size_t)c.vocab * 4);
  L.amax_stride = amax_stride(c.vocab);
  L.amax_val = take(S * (size_t)L.amax_stride * 4);
  L.amax_idx = take(S * (size_t)L.amax_stride * 4);
  size_t maxn = std::max({(size_t)2 * c.ffn_dim, qkv_n, d});
  L.gemm_part_floats = std::max<size_t>((size_t)16 << 20, 4 * R * maxn);
  L.gemm_part = take(L.gemm_part_floats * 4);
  L.attn_max_splits = attn_cap_splits(c.max_position);
  const size_t cols = R * (size_t)c.n_heads * (size_t)L.attn_max_splits;
  L.attn_ml = take(cols * 2 * 4);
  L.attn_o = take(cols * hd * 4);
  L.rope = take((size_t)c.max_position * (hd / 2) * 16);
  L.smp = take(S * (size_t)sampler_row_floats(c.vocab) * 4);
  L.total = o;
  return L;
}

SlotLayout slot_layout(const cbd_config& c) {
  SlotLayout L;
  L.params = 0;
  L.counts = align256((size_t)c.max_slots * sizeof(SlotParams));
  L.total = L.counts + align256((size_t)c.max_slots * (size_t)c.vocab * 4);
  return L;
}

PackedLayout packed_layout(const cbd_config& c) {
  PackedLayout L;
  const int qkv_n = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  const int qd = c.n_heads * c.head_dim;
  size_t o = 0;
  const bool w8 = c.weight_dtype == CBD_W_INT8;
  auto take = [&](int N, int K) {  // offsets in 16-bit units
    size_t at = o;
    o += w8 ? (packed8_bytes(N, K) + 1) / 2 : packed_elems(N, K);
    o = (o + 127) & ~(size_t)127;  // 256-byte aligned
    return at;
  };
  for (int l = 0; l < c.n_layers; ++l) {
    L.qkv.push_back(take(qkv_n, c.d_model));
    L.o.push_back(take(c.d_model, qd));
    L.gate.push_back(take(c.ffn_dim, c.d_model));
    L.up.push_back(take(c.ffn_dim, c.d_model));
    L.down.push_back(take(c.d_model, c.ffn_dim));
  }
  L.lm_head = take(c.vocab, c.d_model);
  L.total_elems = o;
  return L;
}

size_t kv_pool_bytes(const cbd_config& c) {
  const size_t esz = c.kv_dtype == CBD_KV_FP8_E4M3 ? 1 : 2;
  return (size_t)c.n_layers * 2 * (size_t)c.num_blocks * (size_t)c.n_kv_heads *
         (size_t)c.block_size * (size_t)c.head_dim * esz;
}

}  // namespace cbd

using namespace cbd;

// One layer's K or V region of the pool (bytes: values x element size).
static size_t kv_region_bytes(const cbd_config& c) {
  return (size_t)c.num_blocks * c.n_kv_heads * c.block_size * c.head_dim *
         (c.kv_dtype == CBD_KV_FP8_E4M3 ? 1 : 2);
}

void* cbd_engine::pool_k(int layer) const {
  return kv_pool + (size_t)layer * 2 * kv_region_bytes(cfg);
}

void* cbd_engine::pool_v(int layer) const {
  return kv_pool + ((size_t)layer * 2 + 1) * kv_region_bytes(cfg);
}

cbd_engine::~cbd_engine() {
  for (hipEvent_t ev : prof_events) (void)hipEventDestroy(ev);
  for (GraphEntry& g : graphs) (void)hipGraphExecDestroy(g.exec);
}

// Record one event of a start/stop pair when `cls` is being profiled.
hipError_t cbd_engine::prof_mark(int32_t cls, hipStream_t st) {
  if (cls != prof_class || prof_class == 0) return hipSuccess;
  if (prof_used >= 2 * 65536) return hipSuccess;
  if (prof_used == prof_events.size()) {
    // Timing events only, read after hipEventSynchronize: no system-scope
    // fence at each record (with it, a marked B = 64 step of the 8B layer
    // took about 4 us more, and the LM head between the marks 2 us more).
    hipEvent_t ev;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableSystemFence);
    if (e != hipSuccess) return e;
    prof_events.push_back(ev);
  }
  return hipEventRecord(prof_events[prof_used++], st);
}

#define HIP_TRY(expr)                                                        \
  do {                                                                       \
    hipError_t e_ = (expr);                                                  \
    if (e_ != hipSuccess)                                                    \
      return fail(CBD_E_DEVICE, std::string(#expr ": ") + hipGetErrorString(e_)); \
  } while (0)

extern "C" {

int cbd_kv_pool_bytes(const cbd_config* cfg, size_t* bytes) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!bytes) return fail(CBD_E_INVAL, "bytes is NULL");
  *bytes = kv_pool_bytes(*cfg);
  return CBD_OK;
}

int cbd_slot_state_bytes(const cbd_config* cfg, size_t* bytes) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!bytes) return fail(CBD_E_INVAL, "bytes is NULL");
  *bytes = slot_layout(*cfg).total;
  return CBD_OK;
}

int cbd_workspace_bytes(const cbd_config* cfg, size_t* bytes) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!bytes) return fail(CBD_E_INVAL, "bytes is NULL");
  *bytes = workspace_layout(*cfg).total;
  return CBD_OK;
}

int cbd_packed_weights_bytes(const cbd_config* cfg, size_t* bytes) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!bytes) return fail(CBD_E_INVAL, "bytes is NULL");
  *bytes = packed_layout(*cfg).total_elems * 2;
  return CBD_OK;
}

int cbd_engine_create(const cbd_config* cfg, const cbd_weights* w, void* packed_weights,
                      void* kv_pool, void* slot_state, void* workspace,
                      const int32_t* block_order, void* stream, cbd_engine** out) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!w || !packed_weights || !kv_pool || !slot_state || !workspace || !out)
    return fail(CBD_E_INVAL, "NULL weights, buffer or output handle");
  if (!w->embed || !w->final_norm || !w->lm_head || !w->attn_norm || !w->w_qkv || !w->w_o ||
      !w->ffn_norm || !w->w_gate || !w->w_up || !w->w_down)
    return fail(CBD_E_INVAL, "a weight pointer is NULL");
  for (int l = 0; l < cfg->n_layers; ++l)
    if (!w->attn_norm[l] || !w->w_qkv[l] || !w->w_o[l] || !w->ffn_norm[l] || !w->w_gate[l] ||
        !w->w_up[l] || !w->w_down[l])
      return fail(CBD_E_INVAL, "a per-layer weight pointer is NULL");
  const bool w8 = cfg->weight_dtype == CBD_W_INT8;
  if (w8) {
    if (!w->lm_head_scale || !w->s_qkv || !w->s_o || !w->s_gate || !w->s_up || !w->s_down)
      return fail(CBD_E_INVAL, "int8 weights need their scale pointers");
    for (int l = 0; l < cfg->n_layers; ++l)
      if (!w->s_qkv[l] || !w->s_o[l] || !w->s_gate[l] || !w->s_up[l] || !w->s_down[l])
        return fail(CBD_E_INVAL, "a per-layer scale pointer is NULL");
  }
  for (const void* p : {(const void*)packed_weights, (const void*)kv_pool,
                        (const void*)slot_state, (const void*)workspace})
    if ((uintptr_t)p % 256) return fail(CBD_E_INVAL, "device buffers must be 256-byte aligned");

  cbd_engine* e = new cbd_engine();
  e->cfg = *cfg;
  e->md = ModelDims{cfg->d_model, cfg->n_heads, cfg->n_kv_heads, cfg->head_dim, cfg->ffn_dim,
                    cfg->vocab, cfg->block_size, cfg->num_blocks, cfg->max_slots,
                    cfg->max_position, cfg->rms_eps, cfg->kv_dtype == CBD_KV_FP8_E4M3,
                    cfg->kv_dtype == CBD_KV_FP8_E4M3 && cfg->k_scale > 0.f ? cfg->k_scale : 1.f,
                    cfg->kv_dtype == CBD_KV_FP8_E4M3 && cfg->v_scale > 0.f ? cfg->v_scale : 1.f};
  e->ws = workspace_layout(*cfg);
  e->sl = slot_layout(*cfg);
  e->embed = (const uint16_t*)w->embed;
  e->final_norm = (const uint16_t*)w->final_norm;
  e->lm_head = (const uint16_t*)w->lm_head;
  for (int l = 0; l < cfg->n_layers; ++l) {
    e->attn_norm.push_back((const uint16_t*)w->attn_norm[l]);
    e->w_qkv.push_back((const uint16_t*)w->w_qkv[l]);
    e->w_o.push_back((const uint16_t*)w->w_o[l]);
    e->ffn_norm.push_back((const uint16_t*)w->ffn_norm[l]);
    e->w_gate.push_back((const uint16_t*)w->w_gate[l]);
    e->w_up.push_back((const uint16_t*)w->w_up[l]);
    e->w_down.push_back((const uint16_t*)w->w_down[l]);
  }
  e->packed = (uint16_t*)packed_weights;
  e->pl = packed_layout(*cfg);
  e->kv_pool = (uint8_t*)kv_pool;
  e->slot_state = (uint8_t*)slot_state;
  e->workspace = (uint8_t*)workspace;
  e->stream = (hipStream_t)stream;
  {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    e->attn_waves = cus * 4 * 2;
    e->device = dev;
  }
  {  // the fixed sampler scratch of this device, looked up at set-up
    float* p = nullptr;
    size_t n = 0;
    if (noalloc_scratch(&p, &n) != hipSuccess) {
      delete e;
      return fail(CBD_E_DEVICE, "sampler scratch symbol lookup failed");
    }
  }
  e->slots.reset(cfg->max_slots);
  if (!e->blocks.reset(cfg->num_blocks, block_order)) {
    delete e;
    return fail(CBD_E_INVAL, "block_order is not a permutation of 0..num_blocks-1");
  }
  e->host_params.assign((size_t)cfg->max_slots, SlotParams{});

  // RoPE table: angle pos * base^(-2i/hd), (cos, sin) in double.
  const int half = cfg->head_dim / 2;
  std::vector<double> cs((size_t)cfg->max_position * half * 2);
  for (int i = 0; i < half; ++i) {
    const double inv_freq = pow(cfg->rope_base, -2.0 * i / (double)cfg->head_dim);
    for (int p = 0; p < cfg->max_position; ++p) {
      const double th = (double)p * inv_freq;
      cs[((size_t)p * half + i) * 2] = cos(th);
      cs[((size_t)p * half + i) * 2 + 1] = sin(th);
    }
  }
  hipError_t he = hipMemcpyAsync(e->workspace + e->ws.rope, cs.data(), cs.size() * sizeof(double),
                                 hipMemcpyHostToDevice, e->stream);
  // Pack every projection matrix into the GEMM's tile order.
  const int qkv_n = (cfg->n_heads + 2 * cfg->n_kv_heads) * cfg->head_dim;
  const int qd = cfg->n_heads * cfg->head_dim;
  if (w8) {  // int8 codes in k-pairs, each matrix followed by its row scales
    auto pack8 = [&](const void* q, const void* sc, int N, int K, size_t off) {
      return launch_pack8((const int8_t*)q, (const float*)sc, N, K, (uint8_t*)(e->packed + off),
                          e->stream);
    };
    for (int l = 0; l < cfg->n_layers && he == hipSuccess; ++l) {
      he = pack8(w->w_qkv[l], w->s_qkv[l], qkv_n, cfg->d_model, e->pl.qkv[l]);
      if (he == hipSuccess) he = pack8(w->w_o[l], w->s_o[l], cfg->d_model, qd, e->pl.o[l]);
      if (he == hipSuccess)
        he = pack8(w->w_gate[l], w->s_gate[l], cfg->ffn_dim, cfg->d_model, e->pl.gate[l]);
      if (he == hipSuccess)
        he = pack8(w->w_up[l], w->s_up[l], cfg->ffn_dim, cfg->d_model, e->pl.up[l]);
      if (he == hipSuccess)
        he = pack8(w->w_down[l], w->s_down[l], cfg->d_model, cfg->ffn_dim, e->pl.down[l]);
    }
    if (he == hipSuccess)
      he = pack8(w->lm_head, w->lm_head_scale, cfg->vocab, cfg->d_model, e->pl.lm_head);
  }
  for (int l = 0; l < cfg->n_layers && he == hipSuccess && !w8; ++l) {
    he = launch_pack(e->w_qkv[l], qkv_n, cfg->d_model, e->packed + e->pl.qkv[l], e->stream);
    if (he == hipSuccess)
      he = launch_pack(e->w_o[l], cfg->d_model, qd, e->packed + e->pl.o[l], e->stream);
    if (he == hipSuccess)
      he = launch_pack(e->w_gate[l], cfg->ffn_dim, cfg->d_model, e->packed + e->pl.gate[l],
                       e->stream);
    if (he == hipSuccess)
      he = launch_pack(e->w_up[l], cfg->ffn_dim, cfg->d_model, e->packed + e->pl.up[l], e->stream);
    if (he == hipSuccess)
      he = launch_pack(e->w_down[l], cfg->d_model, cfg->ffn_dim, e->packed + e->pl.down[l],
                       e->stream);
  }
  if (he == hipSuccess && !w8)
    he = launch_pack(e->lm_head, cfg->vocab, cfg->d_model, e->packed + e->pl.lm_head, e->stream);
  if (he == hipSuccess)
    he = launch_fill_u32(e->wsp<uint32_t>(e->ws.status), 0u, 1, e->stream);
  // The operand-tile buffers start as zeros: their padding columns are read
  // by the contractions (against zero weights) and never written.
  {
    const size_t R = (size_t)cfg->max_rows, S = (size_t)cfg->max_seqs;
    const size_t qd = (size_t)cfg->n_heads * cfg->head_dim;
    const std::pair<size_t, size_t> tiled[] = {
        {e->ws.h, tile_plane_elems(R, cfg->d_model)}, {e->ws.attn, tile_plane_elems(R, qd)},
        {e->ws.ffn, tile_plane_elems(R, cfg->ffn_dim)}, {e->ws.lm_in, tile_plane_elems(S, cfg->d_model)}};
    for (const auto& t : tiled)  // two bf16 planes: one u32 per element
      if (he == hipSuccess) he = launch_fill_u32(e->wsp<uint32_t>(t.first), 0u, t.second, e->stream);
  }
  if (he == hipSuccess)
    he = launch_fill_u32((uint32_t*)e->slot_state, 0u, e->sl.total / 4, e->stream);
  if (he == hipSuccess) he = hipStreamSynchronize(e->stream);
  if (he != hipSuccess) {
    delete e;
    return fail(CBD_E_DEVICE, std::string("engine set-up: ") + hipGetErrorString(he));
  }
  *out = e;
  return CBD_OK;
}

int cbd_engine_destroy(cbd_engine* e) {
  if (!e) return fail(CBD_E_INVAL, "engine is NULL");
  delete e;
  return CBD_OK;
}

int cbd_slot_alloc(cbd_engine* e, const cbd_sampling* p, uint64_t request_id, int32_t* slot_out) {
  if (!e || !slot_out) return fail(CBD_E_INVAL, "NULL engine or output");
  cbd_sampling sp{};
  if (p) {
    sp = *p;
  } else {
    sp.temperature = 0.f;
    sp.top_p = 1.f;
    sp.penalty_decay = 1.f;
  }
  if (!(sp.temperature >= 0.f) || sp.top_k < 0 || !(sp.penalty_decay >= 0.f))
    return fail(CBD_E_INVAL, "sampling parameters out of range");
  static_assert(CBD_MAX_FORBIDDEN == SLOT_MAX_FORBIDDEN, "forbidden-id capacity");
  if (sp.n_forbidden < 0 || sp.n_forbidden > CBD_MAX_FORBIDDEN)
    return fail(CBD_E_INVAL, "n_forbidden out of range");
  for (int i = 0; i < sp.n_forbidden; ++i)
    if (sp.forbidden[i] < 0 || sp.forbidden[i] >= e->cfg.vocab)
      return fail(CBD_E_INVAL, "a forbidden id is outside the vocabulary");
  int32_t s = e->slots.alloc();
  if (s < 0) return fail(CBD_E_NOSLOT, "every slot is taken");
  SlotParams& hp = e->host_params[(size_t)s];
  hp = SlotParams{};
  hp.temperature = sp.temperature;
  hp.top_p = sp.top_p;
  hp.top_k = sp.top_k;
  hp.freq_penalty = sp.freq_penalty;
  hp.presence_penalty = sp.presence_penalty;
  hp.penalty_decay = sp.penalty_decay;
  hp.seed = sp.seed;
  hp.request_id = request_id;
  hp.n_forbidden = sp.n_forbidden;
  for (int i = 0; i < sp.n_forbidden; ++i) hp.forbidden[i] = sp.forbidden[i];
  hipError_t he = hipMemcpyAsync(e->slot_state + e->sl.params + (size_t)s * sizeof(SlotParams),
                                 &hp, sizeof(SlotParams), hipMemcpyHostToDevice, e->stream);
  if (he == hipSuccess)
    he = launch_fill_u32((uint32_t*)(e->slot_state + e->sl.counts) + (size_t)s * e->cfg.vocab, 0u,
                         (size_t)e->cfg.vocab, e->stream);
  if (he != hipSuccess) {
    e->slots.release(s);
    return fail(CBD_E_DEVICE, std::string("slot reset: ") + hipGetErrorString(he));
  }
  *slot_out = s;
  return CBD_OK;
}

int cbd_slot_free(cbd_engine* e, int32_t slot) {
  if (!e) return fail(CBD_E_INVAL, "engine is NULL");
  if (!e->slots.release(slot)) return fail(CBD_E_INVAL, "slot is not allocated");
  return CBD_OK;
}

int cbd_block_alloc(cbd_engine* e, int32_t n, int32_t* ids_out) {
  if (!e || (n > 0 && !ids_out) || n < 0) return fail(CBD_E_INVAL, "bad block_alloc arguments");
  if (!e->blocks.alloc(n, ids_out)) return fail(CBD_E_NOBLOCKS, "not enough free blocks");
  return CBD_OK;
}

int cbd_block_free(cbd_engine* e, int32_t n, const int32_t* ids) {
  if (!e || (n > 0 && !ids) || n < 0) return fail(CBD_E_INVAL, "bad block_free arguments");
  if (!e->blocks.release(n, ids)) return fail(CBD_E_INVAL, "freeing a block that is not allocated");
  return CBD_OK;
}

int cbd_blocks_available(const cbd_engine* e) {
  if (!e) return fail(CBD_E_INVAL, "engine is NULL");
  return e->blocks.available();
}

int cbd_engine_status(cbd_engine* e, void* stream, uint32_t* flags) {
  if (!e || !flags) return fail(CBD_E_INVAL, "NULL engine or output");
  hipStream_t st = (hipStream_t)stream;
  uint32_t v = 0;
  HIP_TRY(hipMemcpyAsync(&v, e->wsp<uint32_t>(e->ws.status), 4, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
  HIP_TRY(launch_fill_u32(e->wsp<uint32_t>(e->ws.status), 0u, 1, st));
  *flags = v;
  return CBD_OK;
}

// ---------------------------------------------------------------- the step

// Host-side checks of a step (before anything is enqueued).
static int check_step(cbd_engine* e, const cbd_step* s, const int32_t* tokens_out) {
  if (!e || !s) return fail(CBD_E_INVAL, "NULL engine or step");
  const cbd_config& c = e->cfg;
  if (s->n_seqs < 1 || s->n_seqs > c.max_seqs) return fail(CBD_E_INVAL, "n_seqs out of range");
  if (s->n_rows < s->n_seqs || s->n_rows > c.max_rows) return fail(CBD_E_INVAL, "n_rows out of range");
  if (s->n_out < 0 || s->n_out > s->n_seqs) return fail(CBD_E_INVAL, "n_out out of range");
  if (s->max_ctx < 1 || s->max_ctx > c.max_position)
    return fail(CBD_E_INVAL, "max_ctx must be in 1..max_position");
  if (s->max_blocks_per_seq < 1 || s->max_blocks_per_seq > c.max_blocks_per_seq)
    return fail(CBD_E_INVAL, "max_blocks_per_seq out of range");
  if (s->mode != CBD_MODE_GREEDY && s->mode != CBD_MODE_SAMPLE)
    return fail(CBD_E_INVAL, "unknown mode");
  if (!s->slots || !s->block_tables || !s->ctx_lens || !s->n_new || !s->tokens ||
      !s->want_token || (s->mode == CBD_MODE_SAMPLE && !s->step_ids))
    return fail(CBD_E_INVAL, "a step array is NULL");
  if (s->n_out > 0 && !tokens_out) return fail(CBD_E_INVAL, "tokens_out is NULL");
  return CBD_OK;
}

// The step's launches on `st` (a checked step).
static int enqueue_step(cbd_engine* e, const cbd_step* s, float* logits_out, int32_t* tokens_out,
                        hipStream_t st) {
  const cbd_config& c = e->cfg;
  // int8 weights: each packed matrix's row scales follow its codes
  const bool w8 = c.weight_dtype == CBD_W_INT8;
  auto scales8 = [&](size_t off, int N, int K) -> const float* {
    if (!w8) return nullptr;
    return reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(e->packed + off) +
                                          packed8_codes_bytes(N, K));
  };
  const int R = s->n_rows;
  uint32_t* status = e->wsp<uint32_t>(e->ws.status);
  StepMeta m{s->n_seqs, s->n_rows, s->n_out, s->max_blocks_per_seq, s->slots, s->block_tables,
             s->ctx_lens, s->n_new, s->tokens, s->want_token, s->step_ids};
  RowMaps maps{e->wsp<int32_t>(e->ws.row_seq), e->wsp<int32_t>(e->ws.row_pos),
               e->wsp<int32_t>(e->ws.seq_row0), e->wsp<int32_t>(e->ws.out_row),
               e->wsp<int32_t>(e->ws.out_seq), e->wsp<int32_t>(e->ws.item0),
               e->wsp<int32_t>(e->ws.row_out), e->wsp<int32_t>(e->ws.item0b)};
  const AttnPlan ap = plan_attention(c.n_heads, c.n_kv_heads, c.block_size, c.max_position,
                                     e->attn_waves, s->n_seqs, s->n_rows, s->max_ctx,
                                     c.kv_dtype == CBD_KV_FP8_E4M3);
  const int qkv_n = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  const int qd = c.n_heads * c.head_dim;
  const size_t MR = (size_t)c.max_rows;
  float* x = e->wsp<float>(e->ws.x);
  float* qkv = e->wsp<float>(e->ws.qkv);
  // split buffers: the lo plane follows the hi plane
  uint16_t* h = e->wsp<uint16_t>(e->ws.h);
  uint16_t* h_lo = h + tile_plane_elems(MR, c.d_model);
  uint16_t* q = e->wsp<uint16_t>(e->ws.q);
  uint16_t* q_lo = q + MR * qd;
  uint16_t* attn = e->wsp<uint16_t>(e->ws.attn);
  uint16_t* attn_lo = attn + tile_plane_elems(MR, qd);
  uint16_t* ffn = e->wsp<uint16_t>(e->ws.ffn);
  uint16_t* ffn_lo = ffn + tile_plane_elems(MR, c.ffn_dim);
  float* gpart = e->wsp<float>(e->ws.gemm_part);

  HIP_TRY(e->prof_mark(CBD_KERNEL_NORM, st));
  HIP_TRY(launch_prep_embed(m, maps, e->md, ap, e->embed, e->attn_norm[0], x, h, h_lo, status, st));
  HIP_TRY(e->prof_mark(CBD_KERNEL_NORM, st));
  // The norm in front of each projection is fused into the kernel that
  // finishes the previous residual projection (or the embedding gather):
  // per layer QKV -> RoPE/append (+ the QKV split sum) -> attention -> O ->
  // residual + pre-FFN norm -> gate/up -> down -> residual + the next norm.
  uint16_t* lm_in = e->wsp<uint16_t>(e->ws.lm_in);
  uint16_t* lm_in_lo = lm_in + tile_plane_elems(c.max_seqs, c.d_model);
  int32_t splits = 1;
  for (int l = 0; l < c.n_layers; ++l) {
    GemmArgs g{};
    g.partials = gpart;
    g.partials_cap = e->ws.gemm_part_floats;
    g.splits_out = &splits;
    g.X = h; g.Xlo = h_lo; g.R = R; g.K = c.d_model; g.W = e->packed + e->pl.qkv[l]; g.N = qkv_n;
    g.epi = EPI_F32; g.Y = qkv;
    g.w8 = w8;
    g.Ws = scales8(e->pl.qkv[l], qkv_n, c.d_model);
    HIP_TRY(e->prof_mark(CBD_KERNEL_QKV, st));
    HIP_TRY(launch_gemm(g, st));
    HIP_TRY(e->prof_mark(CBD_KERNEL_QKV, st));
    if (ap.row_kernel) {  // RoPE/append fused into the attention row kernel (timed as attention)
      HIP_TRY(e->prof_mark(CBD_KERNEL_ATTN, st));
      HIP_TRY(launch_rope_attention_rows(qkv, gpart, splits, R, m, maps, e->wsp<double>(e->ws.rope),
                                         e->md, ap, q, q_lo, e->pool_k(l), e->pool_v(l), attn,
                                         attn_lo, status, st));
      HIP_TRY(e->prof_mark(CBD_KERNEL_ATTN, st));
    } else {
      HIP_TRY(e->prof_mark(CBD_KERNEL_ROPE, st));
      HIP_TRY(launch_rope_append(qkv, gpart, splits, R, m, maps, e->wsp<double>(e->ws.rope),
                                 e->md, q, q_lo, e->pool_k(l), e->pool_v(l), status, st));
      HIP_TRY(e->prof_mark(CBD_KERNEL_ROPE, st));
      HIP_TRY(e->prof_mark(CBD_KERNEL_ATTN, st));
      HIP_TRY(launch_attention(q, q_lo, R, m, maps, e->md, ap, e->pool_k(l), e->pool_v(l),
                               e->wsp<float>(e->ws.attn_ml), e->wsp<float>(e->ws.attn_o), attn,
                               attn_lo, status, st));
      HIP_TRY(e->prof_mark(CBD_KERNEL_ATTN, st));
    }
    g.X = attn; g.Xlo = attn_lo; g.K = qd; g.W = e->packed + e->pl.o[l]; g.N = c.d_model;
    g.epi = EPI_RESID; g.Y = x;
    g.Ws = scales8(e->pl.o[l], c.d_model, qd);
    HIP_TRY(e->prof_mark(CBD_KERNEL_O, st));
    HIP_TRY(launch_gemm(g, st));
    HIP_TRY(e->prof_mark(CBD_KERNEL_O, st));
    HIP_TRY(e->prof_mark(CBD_KERNEL_NORM, st));
    HIP_TRY(launch_resid_norm(x, gpart, splits, R, nullptr, nullptr, 0, e->ffn_norm[l], c.d_model,
                              c.rms_eps, h, h_lo, st));
    HIP_TRY(e->prof_mark(CBD_KERNEL_NORM, st));
    g.X = h; g.Xlo = h_lo; g.K = c.d_model; g.W = e->packed + e->pl.gate[l];
    g.W2 = e->packed + e->pl.up[l]; g.N = c.ffn_dim;
    g.Ws = scales8(e->pl.gate[l], c.ffn_dim, c.d_model);
    g.Ws2 = scales8(e->pl.up[l], c.ffn_dim, c.d_model);
    g.epi = EPI_SWIGLU; g.Y = nullptr; g.Yh = ffn; g.Yl = ffn_lo; g.splits_out = nullptr;
    HIP_TRY(e->prof_mark(CBD_KERNEL_GATEUP, st));
    HIP_TRY(launch_gemm(g, st));
    HIP_TRY(e->prof_mark(CBD_KERNEL_GATEUP, st));
    g.X = ffn; g.Xlo = ffn_lo; g.K = c.ffn_dim; g.W = e->packed + e->pl.down[l]; g.W2 = nullptr;
    g.Ws = scales8(e->pl.down[l], c.d_model, c.ffn_dim);
    g.Ws2 = nullptr;
    g.N = c.d_model; g.epi = EPI_RESID; g.Y = x; g.Yh = g.Yl = nullptr; g.splits_out = &splits;
    HIP_TRY(e->prof_mark(CBD_KERNEL_DOWN, st));
    HIP_TRY(launch_gemm(g, st));
    HIP_TRY(e->prof_mark(CBD_KERNEL_DOWN, st));
    HIP_TRY(e->prof_mark(CBD_KERNEL_NORM, st));
    if (l + 1 < c.n_layers)
      HIP_TRY(launch_resid_norm(x, gpart, splits, R, nullptr, nullptr, 0, e->attn_norm[l + 1],
                                c.d_model, c.rms_eps, h, h_lo, st));
    else  // the final norm, only for the emitting rows, into the LM head's rows
      HIP_TRY(launch_resid_norm(x, gpart, splits, R, maps.row_out, maps.out_row, s->n_out,
                                e->final_norm, c.d_model, c.rms_eps, lm_in, lm_in_lo, st));
    HIP_TRY(e->prof_mark(CBD_KERNEL_NORM, st));
  }
  if (s->n_out == 0) return CBD_OK;
  float* logits = logits_out;
  if (!logits && s->mode == CBD_MODE_SAMPLE) logits = e->wsp<float>(e->ws.logits);
  GemmArgs g{};
  // The LM head is a bf16 contraction: it reads the hi plane of its input
  // alone (the final norm's output rounded to nearest bf16).
  g.X = lm_in; g.Xlo = nullptr; g.R = s->n_out; g.K = c.d_model; g.W = e->packed + e->pl.lm_head; g.N = c.vocab;
  g.w8 = w8;
  g.Ws = scales8(e->pl.lm_head, c.vocab, c.d_model);
  g.epi = EPI_LOGITS; g.logits = logits;
  g.amax_val = e->wsp<float>(e->ws.amax_val);
  g.amax_idx = e->wsp<int32_t>(e->ws.amax_idx);
  g.amax_stride = e->ws.amax_stride;
  g.partials = gpart;
  g.partials_cap = e->ws.gemm_part_floats;
  HIP_TRY(e->prof_mark(CBD_KERNEL_LM_HEAD, st));
  HIP_TRY(launch_gemm(g, st));
  HIP_TRY(e->prof_mark(CBD_KERNEL_LM_HEAD, st));
  HIP_TRY(e->prof_mark(CBD_KERNEL_SAMPLE, st));
  if (s->mode == CBD_MODE_GREEDY) {
    HIP_TRY(launch_argmax_reduce(g.amax_val, g.amax_idx, gemm_amax_tiles(s->n_out, c.vocab, c.d_model, w8),
                                 e->ws.amax_stride, s->n_out, tokens_out, st));
  } else {
    HIP_TRY(launch_sampler(logits, s->n_out, c.vocab, s->slots, s->step_ids, maps.out_seq,
                           reinterpret_cast<const SlotParams*>(e->slot_state + e->sl.params),
                           reinterpret_cast<float*>(e->slot_state + e->sl.counts), c.max_slots,
                           e->wsp<float>(e->ws.smp), tokens_out, status, st));
  }
  HIP_TRY(e->prof_mark(CBD_KERNEL_SAMPLE, st));
  return CBD_OK;
}

int cbd_step_forward(cbd_engine* e, const cbd_step* s, float* logits_out, int32_t* tokens_out,
                     void* stream) {
  const int rc = check_step(e, s, tokens_out);
  if (rc != CBD_OK) return rc;
  return enqueue_step(e, s, logits_out, tokens_out, (hipStream_t)stream);
}

// Graph replay: a step shape is every field of the step (host scalars and
// the device pointers the kernels are given) and the two output pointers;
// the launch plan and every kernel argument follow from it, so one recorded
// graph serves every step of that shape.
int cbd_step_forward_graph(cbd_engine* e, const cbd_step* s, float* logits_out,
                           int32_t* tokens_out, void* stream) {
  int rc = check_step(e, s, tokens_out);
  if (rc != CBD_OK) return rc;
  if (!stream) return fail(CBD_E_INVAL, "graph replay needs a stream other than the null stream");
  if (e->prof_class != 0) return fail(CBD_E_INVAL, "graph replay while a kernel class is profiled");
  hipStream_t st = (hipStream_t)stream;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  HIP_TRY(hipStreamIsCapturing(st, &cs));
  if (cs != hipStreamCaptureStatusNone) return enqueue_step(e, s, logits_out, tokens_out, st);
  cbd_engine::GraphKey key;
  memset(&key, 0, sizeof key);
  key.step = *s;
  key.logits = logits_out;
  key.tokens = tokens_out;
  ++e->graph_clock;
  for (cbd_engine::GraphEntry& g : e->graphs) {
    if (memcmp(&g.key, &key, sizeof key) == 0) {
      g.used = e->graph_clock;
      HIP_TRY(hipGraphLaunch(g.exec, st));
      ++e->graph_replays;
      return CBD_OK;
    }
  }
  // Record the step's launches (relaxed mode: the first launch of a kernel
  // with more than 64 KB of LDS sets its attribute during the capture).
  HIP_TRY(hipStreamBeginCapture(st, hipStreamCaptureModeRelaxed));
  rc = enqueue_step(e, s, logits_out, tokens_out, st);
  const std::string msg = rc != CBD_OK ? std::string(cbd_last_error()) : std::string();
  hipGraph_t graph = nullptr;
  const hipError_t ee = hipStreamEndCapture(st, &graph);
  if (rc != CBD_OK || ee != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    if (rc != CBD_OK) return fail(rc, msg);
    return fail(CBD_E_DEVICE, std::string("graph capture: ") + hipGetErrorString(ee));
  }
  hipGraphExec_t exec = nullptr;
  const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (ei != hipSuccess) return fail(CBD_E_DEVICE, std::string("graph instantiate: ") + hipGetErrorString(ei));
  if (e->graphs.size() >= CBD_GRAPH_CACHE) {  // drop the least recently used
    size_t old = 0;
    for (size_t i = 1; i < e->graphs.size(); ++i)
      if (e->graphs[i].used < e->graphs[old].used) old = i;
    // It may still be running, on this stream or on another one the caller
    // launched it on: wait for the device before destroying it.
    HIP_TRY(hipDeviceSynchronize());
    (void)hipGraphExecDestroy(e->graphs[old].exec);
    e->graphs.erase(e->graphs.begin() + old);
  }
  e->graphs.push_back(cbd_engine::GraphEntry{key, exec, e->graph_clock});
  ++e->graph_captures;
  HIP_TRY(hipGraphLaunch(exec, st));
  return CBD_OK;
}

int cbd_graph_stats(const cbd_engine* e, int64_t out[3]) {
  if (!e || !out) return fail(CBD_E_INVAL, "NULL engine or output");
  out[0] = e->graph_captures;
  out[1] = e->graph_replays;
  out[2] = (int64_t)e->graphs.size();
  return CBD_OK;
}

int cbd_read_probe(const void* buf, size_t bytes, uint32_t* out, int32_t blocks, void* stream) {
  if (!buf || !out || blocks < 1 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(CBD_E_INVAL, "bad read_probe arguments");
  HIP_TRY(launch_read_probe(buf, bytes, out, blocks, (hipStream_t)stream));
  return CBD_OK;
}

int cbd_sample_logits(cbd_engine* e, const float* logits, int32_t n, const int32_t* slots,
                      const int32_t* step_ids, int32_t* tokens_out, void* stream) {
  if (!e || !logits || !slots || !step_ids || !tokens_out || n < 1 || n > e->cfg.max_seqs)
    return fail(CBD_E_INVAL, "bad sample_logits arguments");
  HIP_TRY(launch_sampler(logits, n, e->cfg.vocab, slots, step_ids, nullptr,
                         reinterpret_cast<const SlotParams*>(e->slot_state + e->sl.params),
                         reinterpret_cast<float*>(e->slot_state + e->sl.counts), e->cfg.max_slots,
                         e->wsp<float>(e->ws.smp), tokens_out, e->wsp<uint32_t>(e->ws.status),
                         (hipStream_t)stream));
  return CBD_OK;
}

int cbd_sample_logits_noalloc(cbd_engine* e, const float* logits, int32_t n,
                              const int32_t* slots, const int32_t* step_ids, int32_t* tokens_out,
                              void* stream) {
  if (!e || !logits || !slots || !step_ids || !tokens_out || n < 1 || n > e->cfg.max_seqs)
    return fail(CBD_E_INVAL, "bad sample_logits_noalloc arguments");
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev != e->device)
    return fail(CBD_E_INVAL, "the engine's device is not the current device");
  float* scratch = nullptr;
  size_t cap = 0;
  HIP_TRY(noalloc_scratch(&scratch, &cap));
  // rows of vocabularies above 65536 are staged in the scratch, one
  // sampler_row_floats(vocab) run per row; smaller rows stay on chip
  const size_t need = e->cfg.vocab > 65536 ? (size_t)n * sampler_row_floats(e->cfg.vocab) : 0;
  if (need > cap)
    return fail(CBD_E_INVAL, "sample_logits_noalloc: " + std::to_string(n) + " rows of vocab " +
                                 std::to_string(e->cfg.vocab) + " need " + std::to_string(need) +
                                 " scratch floats, above the fixed " + std::to_string(cap));
  HIP_TRY(launch_sampler(logits, n, e->cfg.vocab, slots, step_ids, nullptr,
                         reinterpret_cast<const SlotParams*>(e->slot_state + e->sl.params),
                         reinterpret_cast<float*>(e->slot_state + e->sl.counts), e->cfg.max_slots,
                         scratch, tokens_out, e->wsp<uint32_t>(e->ws.status),
                         (hipStream_t)stream));
  return CBD_OK;
}

int cbd_debug_buffer(cbd_engine* e, int32_t which, void** ptr, size_t* bytes) {
  if (!e || !ptr || !bytes) return fail(CBD_E_INVAL, "NULL argument");
  const cbd_config& c = e->cfg;
  const size_t R = (size_t)c.max_rows;
  const size_t qkv_n = (size_t)(c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  const size_t qd = (size_t)c.n_heads * c.head_dim;
  size_t off, n;
  switch (which) {
    case CBD_BUF_X: off = e->ws.x; n = R * c.d_model; break;
    case CBD_BUF_H: off = e->ws.h; n = tile_plane_elems(R, c.d_model); break;
    case CBD_BUF_QKV: off = e->ws.qkv; n = R * qkv_n; break;
    case CBD_BUF_Q: off = e->ws.q; n = R * qd; break;
    case CBD_BUF_ATTN: off = e->ws.attn; n = tile_plane_elems(R, qd); break;
    case CBD_BUF_FFN: off = e->ws.ffn; n = tile_plane_elems(R, c.ffn_dim); break;
    case CBD_BUF_LM_IN: off = e->ws.lm_in; n = tile_plane_elems(c.max_seqs, c.d_model); break;
    default: return fail(CBD_E_INVAL, "unknown buffer");
  }
  *ptr = e->workspace + off;
  *bytes = n * 4;
  return CBD_OK;
}

int cbd_profile_begin(cbd_engine* e, int32_t kernel_class) {
  if (!e || kernel_class < CBD_KERNEL_QKV || kernel_class > CBD_KERNEL_NORM)
    return fail(CBD_E_INVAL, "unknown kernel class");
  e->prof_class = kernel_class;
  e->prof_used = 0;
  return CBD_OK;
}

int cbd_profile_end(cbd_engine* e, double* total_ms, int32_t* launches) {
  if (!e || !total_ms || !launches) return fail(CBD_E_INVAL, "NULL argument");
  double sum = 0.0;
  const size_t pairs = e->prof_used / 2;
  for (size_t i = 0; i < pairs; ++i) {
    HIP_TRY(hipEventSynchronize(e->prof_events[2 * i + 1]));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, e->prof_events[2 * i], e->prof_events[2 * i + 1]));
    sum += ms;
  }
  e->prof_class = 0;
  e->prof_used = 0;
  *total_ms = sum;
  *launches = (int32_t)pairs;
  return CBD_OK;
}

}  // extern "C"

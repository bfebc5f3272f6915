/*
 * cbd.h -- C ABI of the continuous-batching decode forward step for AMD
 * MI355X (gfx950).
 *
 * One call of cbd_step_forward is one iteration of iteration-level
 * scheduling: it reads the decoder weights once and produces one next token
 * for each in-flight sequence that asks for one (Go under the hood,
 * section 20.3.2: a step costs about (W + B*A)/beta -- W weight bytes, A
 * per-sequence bytes, beta bandwidth -- so B sequences share one weight
 * read). Per-sequence KV state lives in a paged pool of fixed-size blocks
 * reached through per-sequence block tables (same section: PagedAttention's
 * fixed-size blocks allocated on demand). A prefill chunk may share the step
 * with decode rows, and a batched sampler closes it (RWKV-Runner Albatross
 * article, "Worker main loop": penalties, temperature, top-p/top-k sampling
 * over the decode segment).
 *
 * Conventions for every function below:
 *  - Return value: CBD_OK (0) or a negative CBD_E_* code; the message of
 *    the last failure on the calling thread is cbd_last_error().
 *    No C++ exception crosses this boundary.
 *  - "device" pointers are HIP device memory; "host" pointers are ordinary
 *    host memory. The caller allocates and owns every device buffer
 *    (weights, KV pool, slot state, workspace, step metadata, outputs) and
 *    keeps it alive until the work that uses it has completed. The library
 *    allocates no device memory; it owns only host-side state (allocator
 *    free lists, the composer, the handle).
 *  - Streams are hipStream_t passed as void*; NULL is the default stream.
 *    Device work is enqueued asynchronously on the given stream.
 *  - One engine is driven by one host thread at a time (the Kestrel page,
 *    "0.8MB 跑通 Qwen" 14-1 section 2: a single engine thread is the only
 *    caller of the batched forward). Calls on one engine from several
 *    threads at once are not supported.
 *  - bf16 is the 16-bit brain float, stored as uint16_t bit patterns.
 *  - Precision: the bytes the step streams -- weights and the KV cache --
 *    are bf16 (a cached K or V value is rounded to bf16 once, when it is
 *    appended). Activations between the step's kernels are fp32; the
 *    matrix-core contractions of the layers take them as two bf16 terms
 *    (hi + lo) and accumulate in fp32. The LM head is a bf16 contraction:
 *    its input, the final norm's output, is rounded to nearest bf16, and it
 *    accumulates in fp32. Logits are fp32; the greedy id is the lowest id
 *    of their maximum.
 */
#ifndef CBD_H
#define CBD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CBD_OK 0
#define CBD_E_INVAL (-1)       /* bad argument, shape or metadata */
#define CBD_E_NOSLOT (-2)      /* every slot is taken */
#define CBD_E_NOBLOCKS (-3)    /* the block pool cannot satisfy the request;
                                  the caller waits, nothing is evicted */
#define CBD_E_UNSUPPORTED (-4) /* a shape outside what the kernels support;
                                  never silently replaced by another path */
#define CBD_E_DEVICE (-5)      /* a HIP runtime error */

/* Device-side status bits reported by cbd_engine_status (set by kernels
 * that met metadata they refused to act on; the offending rows are skipped
 * and their outputs are left unspecified). */
#define CBD_STATUS_BAD_BLOCK 0x1u   /* block id outside [0, num_blocks) */
#define CBD_STATUS_BAD_TOKEN 0x2u   /* token id outside [0, vocab) */
#define CBD_STATUS_BAD_SLOT 0x4u    /* slot outside [0, max_slots) */
#define CBD_STATUS_BAD_SHAPE 0x8u   /* n_new < 1, ctx < 0, ctx + n_new beyond
                                       the table, or the row/output counts
                                       disagree with the host scalars */

/* ------------------------------------------------------------------ config */

typedef struct cbd_config {
  /* decoder shape: pre-norm blocks (RMSNorm -> attention -> residual,
   * RMSNorm -> SwiGLU FFN -> residual), final RMSNorm, untied LM head */
  int32_t n_layers;
  int32_t d_model;
  int32_t n_heads;    /* query heads */
  int32_t n_kv_heads; /* KV heads; query head h reads KV head h*n_kv/n_heads */
  int32_t head_dim;   /* 64 or 128 */
  int32_t ffn_dim;
  int32_t vocab;      /* embedding rows = LM-head rows */
  /* paged KV pool */
  int32_t block_size; /* positions per block: 4, 8, 16, 32 or 64 */
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  /* per-step limits */
  int32_t max_slots;  /* sequences that may hold sampler state */
  int32_t max_rows;   /* rows per step (decode rows + prefill tokens) */
  int32_t max_seqs;   /* sequences per step */
  int32_t max_position; /* positions covered by the RoPE table */
  float rms_eps;
  float pad0_;
  double rope_base;
  /* KV cache storage: CBD_KV_BF16, or CBD_KV_FP8_E4M3 (an 8-bit float per
   * value, halving the per-sequence bytes the step streams; the "Continuous
   * Batching" practice article, section 6, recommends FP8 KV quantisation).
   * FP8 stores the OCP E4M3 code of value / scale (round to nearest even,
   * magnitudes past 448 saturated), read back as code value * scale; the
   * scales (0 means 1.0; powers of two keep the division exact) are per
   * engine, k_scale for keys (after RoPE) and v_scale for values. FP8 needs
   * block_size 8, 16, 32 or 64, and prefill chunks attend on the per-tile
   * kernel. */
  int32_t kv_dtype;
  float k_scale;
  float v_scale;
  /* Projection weights (QKV, O, gate, up, down, LM head): CBD_W_BF16, or
   * CBD_W_INT8 -- int8 codes q with one float32 scale per matrix row, read
   * as q * scale (weight-only quantisation, the follow-up "int8 weights" the
   * RWKV-Runner Albatross article lists; it halves W, the bytes every
   * decode step streams). The embedding and the norm gains stay bf16. The
   * int8 projections run on the streaming GEMM at every row count. */
  int32_t weight_dtype;
} cbd_config;

#define CBD_KV_BF16 0
#define CBD_KV_FP8_E4M3 1
#define CBD_W_BF16 0
#define CBD_W_INT8 1

/* Weights: every pointer is device memory holding bf16, row-major (the
 * projections int8 under CBD_W_INT8). Per-layer fields are HOST arrays of
 * n_layers device pointers; the engine copies the pointer values at create
 * time. */
typedef struct cbd_weights {
  const void* embed;        /* [vocab][d_model] */
  const void* final_norm;   /* [d_model] */
  const void* lm_head;      /* [vocab][d_model] */
  const void* const* attn_norm; /* [d_model] */
  const void* const* w_qkv;     /* [(n_heads + 2*n_kv_heads)*head_dim][d_model]:
                                   q rows, then k rows, then v rows */
  const void* const* w_o;       /* [d_model][n_heads*head_dim] */
  const void* const* ffn_norm;  /* [d_model] */
  const void* const* w_gate;    /* [ffn_dim][d_model] */
  const void* const* w_up;      /* [ffn_dim][d_model] */
  const void* const* w_down;    /* [d_model][ffn_dim] */
  /* CBD_W_INT8 only (NULL otherwise): float32 scales, one per row of the
   * matching matrix above; copied into the packed buffer at creation. */
  const void* lm_head_scale;    /* [vocab] */
  const void* const* s_qkv;     /* [(n_heads + 2*n_kv_heads)*head_dim] */
  const void* const* s_o;       /* [d_model] */
  const void* const* s_gate;    /* [ffn_dim] */
  const void* const* s_up;      /* [ffn_dim] */
  const void* const* s_down;    /* [d_model] */
} cbd_weights;

/* Per-slot sampling parameters (Albatross adapter defaults: temperature
 * 1.0, top_p 0.3, top_k 0, frequency penalty 1, penalty decay 0.996).
 * Forbidden ids (the Albatross worker masks forbidden tokens on the decode
 * segment before the penalties and the draw, worker main loop step 6): the
 * sampler sets their penalised logits to -infinity, so they are never drawn
 * (and never the greedy pick of temperature 0). Up to CBD_MAX_FORBIDDEN ids
 * in [0, vocab); the greedy step mode (CBD_MODE_GREEDY) does not read them. */
#define CBD_MAX_FORBIDDEN 8
typedef struct cbd_sampling {
  float temperature;      /* 0 = greedy on the penalised logits */
  float top_p;            /* >= 1 disables top-p */
  int32_t top_k;          /* 0 disables top-k */
  float freq_penalty;
  float presence_penalty;
  float penalty_decay;
  uint64_t seed;          /* key of the counter-based draw */
  int32_t n_forbidden;    /* 0 .. CBD_MAX_FORBIDDEN */
  int32_t forbidden[CBD_MAX_FORBIDDEN];
} cbd_sampling;

/* Buffer sizes for a configuration (bytes). The KV pool layout is
 * [n_layers][2][num_blocks][n_kv_heads][tile], one tile per (block, KV
 * head): K tiles are [block_size][head_dim] (position-major), V tiles are
 * [head_dim][block_size] (dimension-major), bf16 or E4M3 bytes (kv_dtype).
 * The block-id space is shared by all layers. */
int cbd_kv_pool_bytes(const cbd_config* cfg, size_t* bytes);
/* The packed-weights buffer: every projection matrix (QKV, O, gate, up,
 * down per layer, and the LM head) rearranged once, at engine creation, into
 * the GEMM's tile order (16 rows x 32 k tiles in MFMA operand order; int8
 * codes as 16 rows x 64 k pairs of such tiles, followed by the matrix's row
 * scales; see the engine source). After cbd_engine_create returns, the
 * engine reads only the embedding, the norm gains and this buffer, so the
 * caller may release the row-major projection matrices (and their scales). */
int cbd_packed_weights_bytes(const cbd_config* cfg, size_t* bytes);
int cbd_slot_state_bytes(const cbd_config* cfg, size_t* bytes);
int cbd_workspace_bytes(const cbd_config* cfg, size_t* bytes);

/* ------------------------------------------------------------------ engine */

typedef struct cbd_engine cbd_engine;

/* Create an engine over caller-owned device buffers of at least the sizes
 * above (all 256-byte aligned); fills packed_weights from the weights and
 * waits for that on `stream` before returning. block_order (host, nullable) seeds the FIFO block free list with a
 * permutation of 0..num_blocks-1 (NULL: ascending). stream: where the
 * engine's own set-up work and slot resets are enqueued. Returns
 * CBD_E_UNSUPPORTED for shapes the kernels do not handle (head_dim not in
 * {64, 128}, n_heads/n_kv_heads not dividing 16, block_size not in {4, 8,
 * 16, 32, 64}, d_model, ffn_dim or vocab not a multiple of 16, d_model above
 * 8192, max_position beyond the key splits of that block size). */
int cbd_engine_create(const cbd_config* cfg, const cbd_weights* weights, void* packed_weights,
                      void* kv_pool, void* slot_state, void* workspace,
                      const int32_t* block_order, void* stream, cbd_engine** out);
int cbd_engine_destroy(cbd_engine* e);

/* Slots (per-sequence sampler state: penalty counts over the vocabulary
 * and the sampling parameters; the Albatross worker keeps them as
 * preallocated per-slot tensors). cbd_slot_alloc returns the lowest free
 * slot id, stores params and request_id (the draw's counter) and enqueues a
 * reset of the slot's counts to zero on the engine stream. CBD_E_INVAL for
 * a negative temperature, top_k or decay, or forbidden ids out of range.
 * cbd_slot_free may be called at any step boundary (a request aborted by
 * its client stops alone). */
int cbd_slot_alloc(cbd_engine* e, const cbd_sampling* params, uint64_t request_id,
                   int32_t* slot_out);
int cbd_slot_free(cbd_engine* e, int32_t slot);

/* Blocks: the paged KV pool's fixed-size blocks, handed out by id (Go under
 * the hood section 20.3.2: PagedAttention stores the KV cache in fixed-size
 * blocks allocated as sequences grow, and Forma's scheduler takes a
 * request's blocks from one shared pool at admission, waiting -- never
 * evicting -- when the pool is short).
 * cbd_block_alloc (n >= 0, ids_out: host int32[n]) is all-or-nothing: it
 * pops n ids from the front of the FIFO free list into ids_out, or returns
 * CBD_E_NOBLOCKS and takes none (the caller waits for blocks to be freed).
 * cbd_block_free (ids: host int32[n]) appends the ids to the back of the
 * list, in the given order; if any id is out of range or not allocated
 * (a double free) it returns CBD_E_INVAL and frees none.
 * cbd_blocks_available returns the number of free blocks (or CBD_E_INVAL
 * for a NULL engine). The free list starts as the engine's block_order.
 * The ids index the pool for every layer. Host-only; nothing is enqueued. */
int cbd_block_alloc(cbd_engine* e, int32_t n, int32_t* ids_out);
int cbd_block_free(cbd_engine* e, int32_t n, const int32_t* ids);
int cbd_blocks_available(const cbd_engine* e);

/* ------------------------------------------------------------------- step */

#define CBD_MODE_GREEDY 0 /* argmax of the raw logits, lowest id on ties */
#define CBD_MODE_SAMPLE 1 /* the per-slot batched sampler */

/* One step. Host scalars size the launch; the arrays are DEVICE memory.
 * Sequences are taken in the given order; sequence s contributes n_new[s]
 * consecutive entries of `tokens` (decode rows: 1; a prefill chunk: up to
 * 512), at positions ctx_lens[s] .. ctx_lens[s] + n_new[s] - 1, where
 * ctx_lens[s] counts the positions already in the pool. Row i of a chunk
 * attends to positions 0 .. ctx_lens[s] + i. Every row's K and V are
 * appended through the sequence's block table before attention. */
typedef struct cbd_step {
  int32_t n_seqs;             /* 1 .. max_seqs */
  int32_t n_rows;             /* sum of n_new, 1 .. max_rows */
  int32_t n_out;              /* number of sequences with want_token != 0 */
  int32_t max_ctx;            /* host upper bound of ctx_lens[s] + n_new[s] */
  int32_t max_blocks_per_seq; /* row stride of block_tables */
  int32_t mode;               /* CBD_MODE_GREEDY or CBD_MODE_SAMPLE */
  const int32_t* slots;        /* [n_seqs] sampler slot of each sequence
                                  (distinct within a sampled step) */
  const int32_t* block_tables; /* [n_seqs][max_blocks_per_seq] block ids */
  const int32_t* ctx_lens;     /* [n_seqs] */
  const int32_t* n_new;        /* [n_seqs] */
  const int32_t* tokens;       /* [n_rows] */
  const int32_t* want_token;   /* [n_seqs] 0/1: emit a token from the last row */
  const int32_t* step_ids;     /* [n_seqs] index of the token being generated
                                  (the draw's counter); unused when greedy */
} cbd_step;

/* Run one step on `stream`. Outputs (device) have one entry per sequence
 * with want_token, in sequence order: logits_out [n_out][vocab] fp32
 * (nullable when not wanted) and tokens_out [n_out] int32. Asynchronous.
 * Host-checkable errors return CBD_E_INVAL before anything is enqueued;
 * bad device metadata is refused row by row on the device and reported
 * through cbd_engine_status. */
int cbd_step_forward(cbd_engine* e, const cbd_step* step, float* logits_out,
                     int32_t* tokens_out, void* stream);

/* The same step replayed from a HIP graph (the RWKV-Runner Albatross
 * article's follow-up route, "边界与后续路线": graph-captured decode).
 * Contract, checks and results are those of cbd_step_forward. The first
 * call for a step shape -- every field of `step` (the host scalars and the
 * device array pointers) together with logits_out and tokens_out -- records
 * the step's launches into a graph on `stream` and instantiates it; every
 * later call with the same shape launches that graph, which reads the
 * step's current metadata through the same device pointers. A caller that
 * wants replays keeps its metadata buffer in place and passes a max_ctx
 * that stays fixed across steps (any upper bound of ctx_lens + n_new is
 * valid, e.g. rounded up to a multiple of 256). The engine keeps the
 * CBD_GRAPH_CACHE most recently used graphs, destroying the oldest (after
 * waiting for the device, since it may still run on some stream).
 * `stream` must not be the null stream (CBD_E_INVAL; a graph is recorded
 * by stream capture). On a stream that is already being captured the
 * launches are recorded into the caller's capture, as cbd_step_forward's
 * would be. Not while a kernel class is being profiled (CBD_E_INVAL). */
#define CBD_GRAPH_CACHE 16
int cbd_step_forward_graph(cbd_engine* e, const cbd_step* step, float* logits_out,
                           int32_t* tokens_out, void* stream);
/* Graphs recorded (out[0]) and replayed (out[1]) by cbd_step_forward_graph
 * since the engine was created, and graphs cached now (out[2]). */
int cbd_graph_stats(const cbd_engine* e, int64_t out[3]);

/* Streaming-read probe of the device's HBM, for reading the step's rooflines
 * (not part of the step). The cost model of the step is bytes over the
 * memory bandwidth beta (Go under the hood 20.3.2, one weight read shared by
 * the batch); this measures the beta a plain stream reaches on the device,
 * beside the published peak. Reads the `bytes` bytes at `buf` (device,
 * 16-byte aligned, `bytes` a multiple of 16) once, front to back, with
 * `blocks` workgroups of 1024 threads and non-temporal 16-byte loads, on
 * `stream`, and writes each thread's XOR fold of the words it read to `out`
 * (device, blocks * 1024 uint32; the caller's). Asynchronous: time it with
 * events on `stream`. Errors: CBD_E_INVAL (NULL pointer, blocks < 1, a
 * misaligned `buf` or `bytes`), CBD_E_DEVICE (launch). */
int cbd_read_probe(const void* buf, size_t bytes, uint32_t* out, int32_t blocks, void* stream);

/* The batched sampler alone, over caller-given fp32 logits [n][vocab]
 * (device): row j uses slot slots[j] and draw counter step_ids[j] (device
 * arrays). Updates the slots' penalty counts like a sampled step. The slots
 * of one call must be distinct (each row rewrites its slot's counts; rows
 * sharing a slot race). */
int cbd_sample_logits(cbd_engine* e, const float* logits, int32_t n, const int32_t* slots,
                      const int32_t* step_ids, int32_t* tokens_out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * cbd_sample_logits with the same arguments, results and errors, except that
 * the per-row scratch of vocabularies above 65536 comes from a fixed static
 * device array of 4 Mi floats (16 MiB) per GPU instead of the engine's
 * workspace, so n * 1024 * ceil(vocab / 1024) must stay within 4 Mi
 * (vocab 151936: at most 27 rows), else CBD_E_INVAL before anything is
 * enqueued; vocabularies up to 65536 use no scratch (n up to max_seqs).
 * Allocates nothing. The engine's device must be the current device. All
 * calls on one GPU share its array and leave its contents behind (nothing
 * needs clearing: each row's scratch is written before it is read); calls
 * that overlap on one GPU race. */
int cbd_sample_logits_noalloc(cbd_engine* e, const float* logits, int32_t n,
                              const int32_t* slots, const int32_t* step_ids, int32_t* tokens_out,
                              void* stream);

/* Wait for the engine's device status word on `stream`, return it in
 * *flags and clear it (CBD_STATUS_* bits). */
int cbd_engine_status(cbd_engine* e, void* stream, uint32_t* flags);

const char* cbd_last_error(void);

/* ----------------------------------------------------------- inspection */

/* Activation buffers inside the workspace, as the last step left them (for
 * multi-layer models: the last layer's). Row i is the i-th row of the step
 * (for CBD_BUF_LM_IN: the i-th emitting sequence). Activations are fp32
 * values. "fp32" buffers hold float [rows][w]. "split" buffers hold the
 * value as two bf16 terms, a hi plane followed by a lo plane, value = hi +
 * lo (hi = bf16(v), lo = bf16(v - hi)); the contractions consume them that
 * way. A "row-major" split plane is [rows][w]. A "tiled" split plane (the
 * inputs of the projections) is in operand tiles: rows padded to a multiple
 * of 16 (R16) and columns to a multiple of 32 (KB = w32 / 32 blocks), element
 * (r, k) at ((r / 16 * KB + k / 32) * 64 + (k / 8 % 4) * 16 + r % 16) * 8 +
 * k % 8, i.e. 1 KB tiles of 16 rows x 32 columns; each plane holds
 * R16 * w32 elements. rows = max_rows (max_seqs for CBD_BUF_LM_IN). */
#define CBD_BUF_X 1      /* fp32: residual stream after the step [rows][d_model] */
#define CBD_BUF_H 2      /* split, tiled: last RMSNorm output, the FFN input [rows][d_model] */
#define CBD_BUF_QKV 3    /* fp32: QKV projection [rows][(n_heads+2*n_kv_heads)*head_dim] */
#define CBD_BUF_Q 4      /* split, row-major: rotated queries [rows][n_heads*head_dim] */
#define CBD_BUF_ATTN 5   /* split, tiled: attention output [rows][n_heads*head_dim] */
#define CBD_BUF_FFN 6    /* split, tiled: SwiGLU output [rows][ffn_dim] */
#define CBD_BUF_LM_IN 7  /* split, tiled: final-norm rows [rows][d_model]; the LM head
                            reads their hi plane (the rows rounded to bf16) */
/* Device address and size in bytes of one of them (no copy, no sync). */
int cbd_debug_buffer(cbd_engine* e, int32_t which, void** ptr, size_t* bytes);

/* ------------------------------------------------------------- profiling */

/* Kernel classes that can be timed inside cbd_step_forward. */
#define CBD_KERNEL_QKV 1       /* QKV projection */
#define CBD_KERNEL_ROPE 2      /* RoPE + KV append */
#define CBD_KERNEL_ATTN 3      /* paged attention + split combine */
#define CBD_KERNEL_O 4         /* O projection + residual */
#define CBD_KERNEL_GATEUP 5    /* gate/up projection + SwiGLU */
#define CBD_KERNEL_DOWN 6      /* down projection + residual */
#define CBD_KERNEL_LM_HEAD 7   /* final norm's consumer: LM head + argmax partials */
#define CBD_KERNEL_SAMPLE 8    /* argmax combine or the sampler */
#define CBD_KERNEL_NORM 9      /* embedding + RMSNorms */

/* From now on, every launch of that class inside cbd_step_forward is
 * bracketed by a pair of HIP events recorded on the step's stream (a marker
 * each, nothing else changes). At most 65536 launches are kept. */
int cbd_profile_begin(cbd_engine* e, int32_t kernel_class);
/* Stop recording, wait for the recorded events, and return the summed
 * duration (milliseconds) and the number of launches timed. */
int cbd_profile_end(cbd_engine* e, double* total_ms, int32_t* launches);

/* --------------------------------------------------------------- composer */

/* The host step composer: Forma's "Scheduler" (Go under the hood section
 * 20.3.2), kept apart from the step so that an admission bug and a batching
 * bug can be told apart. */

#define CBD_ADMIT_RESERVE 0       /* reserve prompt + answer blocks at
                                     admission (every admitted request can
                                     finish) */
#define CBD_ADMIT_FREE_SLOT 1     /* admit on any free slot, take blocks on
                                     demand (can exhaust the pool) */
#define CBD_ADMIT_REQUEST_LEVEL 2 /* static batching: admit a new group only
                                     when the batch is empty */

#define CBD_FINISH_EOS 1
#define CBD_FINISH_LENGTH 2
#define CBD_FINISH_ABORT 3

/* How prefill work is paced against decode rows (step composition). */
#define CBD_PACE_PREFILL_FIRST 0 /* Forma (Go under the hood 20.3.2): every step
                                    takes prefill chunks first (arrival order),
                                    then one row per decoding sequence */
#define CBD_PACE_ALBATROSS 1     /* the Albatross worker loop (RWKV-Runner
                                    Albatross article, worker main loop steps 4
                                    and 5 and the pacing parameters after it):
                                    at most max_prefill sequences in prefill at
                                    once (admission waits otherwise); decode rows
                                    first; prompts shorter than
                                    min_forward_seq_len are fed one token per
                                    step beside the decode rows; longer prompts
                                    advance by a chunk only on every
                                    (decode_prefill_ratio + 1)-th step while
                                    decode rows exist (every step otherwise) */
#define CBD_PACE_SEPARATE 2      /* prefill apart from decode (the Kestrel
                                    engine prefills under the engine mutex,
                                    outside the batched forward: "0.8MB 跑通
                                    Qwen" 14-1 section 2): a step that carries
                                    prefill chunks carries no decode rows */

typedef struct cbd_sched_config {
  int32_t max_slots;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_rows;   /* row budget of one step */
  int32_t chunk_size; /* prefill chunk length (Forma: 512) */
  int32_t eos_id;
  int32_t policy;     /* CBD_ADMIT_* */
  int32_t pacing;     /* CBD_PACE_* (0: prefill first) */
  /* CBD_PACE_ALBATROSS parameters; 0 takes the article's value:
   * max_prefill = max(floor(0.125 * max_slots), 1), decode_prefill_ratio = 5,
   * min_forward_seq_len = 10 */
  int32_t max_prefill;
  int32_t decode_prefill_ratio;
  int32_t min_forward_seq_len;
  /* Decode-only steps (no prefill rows) in cbd_sched_step: ctx_round > 0
   * rounds the step's max_ctx up to a multiple of ctx_round (at most the
   * engine's max_position), so that it stays fixed over many steps;
   * graph_decode = 1 runs them through cbd_step_forward_graph. */
  int32_t ctx_round;
  int32_t graph_decode;
} cbd_sched_config;

/* One planned step, in host memory owned by the composer and valid until
 * the next cbd_sched_plan. Copy the arrays to the device and fill a
 * cbd_step from them. block_tables is [n_seqs][max_blocks_per_seq], unused
 * entries -1. */
typedef struct cbd_plan {
  int32_t n_seqs, n_rows, n_out, max_ctx, max_blocks_per_seq;
  int32_t n_prefill_rows, n_decode_rows;
  int32_t stalled; /* no row can run although sequences are active */
  const int32_t* slots;
  const int32_t* block_tables;
  const int32_t* ctx_lens;
  const int32_t* n_new;
  const int32_t* tokens;
  const int32_t* want_token;
  const int32_t* step_ids;
  const uint64_t* request_ids;
} cbd_plan;

typedef struct cbd_sched_stats {
  int32_t queued, active, free_slots, free_blocks;
  int64_t steps, finished;
} cbd_sched_stats;

typedef struct cbd_sched cbd_sched;

/* engine (nullable): when given, slots and blocks come from the engine's
 * allocators (slot allocation resets the slot's sampler state on the
 * device), and block_order is ignored; when NULL the composer keeps its own
 * host-only allocators seeded by block_order (nullable, ascending).
 * With an engine the configs must agree: the same block_size and
 * num_blocks, and max_slots, max_rows and max_blocks_per_seq no larger than
 * the engine's (max_slots also within its max_seqs, and
 * max_blocks_per_seq * block_size within its max_position); otherwise
 * CBD_E_INVAL. */
int cbd_sched_create(const cbd_sched_config* cfg, cbd_engine* engine,
                     const int32_t* block_order, cbd_sched** out);
int cbd_sched_destroy(cbd_sched* s);
/* Queue a request (host prompt). CBD_E_INVAL if the prompt is empty,
 * max_new < 1 or prompt + answer can never fit a sequence's table or the
 * pool. params may be NULL (greedy defaults). */
int cbd_sched_submit(cbd_sched* s, const int32_t* prompt, int32_t prompt_len,
                     int32_t max_new, const cbd_sampling* params, uint64_t request_id);
/* Retire nothing, admit what the policy allows, compose the next step. */
int cbd_sched_plan(cbd_sched* s, cbd_plan* out);
/* Hand back the step's tokens (host, n = plan.n_out, sequence order):
 * append, advance positions, retire on EOS or length (freeing slot and
 * blocks). */
int cbd_sched_commit(cbd_sched* s, const int32_t* tokens, int32_t n);
/* Abort a queued or active request at a step boundary. CBD_E_INVAL if
 * unknown. */
int cbd_sched_abort(cbd_sched* s, uint64_t request_id);
/* Pop the oldest finished request: returns 1 and fills the outputs, or 0
 * when none is left. */
int cbd_sched_pop_finished(cbd_sched* s, uint64_t* request_id, int32_t* reason,
                           int32_t* n_generated);
int cbd_sched_stats_get(const cbd_sched* s, cbd_sched_stats* out);

/* The loop of Go under the hood section 20.3.2 (plan a step, run it on the
 * batch, hand its tokens back) as one host call, for a composer created
 * with an engine.
 *
 * cbd_sched_meta_ints: the int32 count of the staging buffers below,
 * max_slots * (5 + max_blocks_per_seq) + max_rows.
 *
 * cbd_sched_step: plan (admit, compose); pack the plan's arrays (slots,
 * block tables, ctx_lens, n_new, tokens, want_token, step_ids, in that
 * order) into host_stage (host, cbd_sched_meta_ints int32; page-locked
 * memory makes the upload asynchronous) and copy them to meta_dev (device,
 * same size); run cbd_step_forward with `mode` on `stream` (a decode-only
 * step with graph_decode set: cbd_step_forward_graph, which needs a stream
 * other than the null stream, with max_ctx rounded up by ctx_round; the
 * staging buffers' fixed addresses let one recorded graph serve every such
 * step of a batch size); copy the step's
 * tokens (tokens_dev: device int32 [max_slots]) back into host_stage; wait
 * for the stream; commit them. logits_out (device [max_slots][vocab] fp32)
 * is nullable. plan_out (nullable) receives the plan that ran; its arrays
 * stay valid until the next plan. A step with no rows (nothing admitted, or
 * stalled under CBD_ADMIT_FREE_SLOT: see plan_out->stalled) runs nothing and
 * commits an empty step. All buffers are the caller's. Blocks until the
 * step's tokens are on the host. Errors: CBD_E_INVAL (NULL argument, no
 * engine, bad mode), CBD_E_DEVICE; after an error inside the step the
 * stream has been drained (host_stage is free again), the plan stays
 * uncommitted and the composer should be destroyed. */
int cbd_sched_meta_ints(const cbd_sched_config* cfg, size_t* ints_out);
int cbd_sched_step(cbd_sched* s, int32_t mode, int32_t* meta_dev, int32_t* host_stage,
                   int32_t* tokens_dev, float* logits_out, void* stream, cbd_plan* plan_out);

#ifdef __cplusplus
}
#endif

#endif /* CBD_H */

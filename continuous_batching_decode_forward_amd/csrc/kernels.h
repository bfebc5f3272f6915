// kernels.h -- host-side launch interface of the step's gfx950 kernels.
// Every launcher enqueues on the given stream and returns the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cbd {

// ------------------------------------------------------------------ metadata

struct StepMeta {
  int32_t n_seqs, n_rows, n_out, max_blocks_per_seq;
  const int32_t* slots;
  const int32_t* block_tables;
  const int32_t* ctx_lens;
  const int32_t* n_new;
  const int32_t* tokens;
  const int32_t* want_token;
  const int32_t* step_ids;
};

// Row maps built on the device from the step metadata (workspace).
struct RowMaps {
  int32_t* row_seq;    // [max_rows] sequence of each row, -1 = refused
  int32_t* row_pos;    // [max_rows] position of each row
  int32_t* seq_row0;   // [max_seqs] first row of each sequence
  int32_t* out_row;    // [max_rows] row of the j-th emitting sequence, -1 = none
  int32_t* out_seq;    // [max_rows] that sequence
  int32_t* item0;      // [max_seqs + 1] first key step per sequence of the per-tile schedule
  int32_t* row_out;    // [max_rows] output index of each row, -1 = emits nothing
  int32_t* item0b;     // [max_seqs + 1] first block work item per sequence (chunks)
};

struct ModelDims {
  int32_t d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  int32_t block_size, num_blocks, max_slots, max_position;
  float rms_eps;
  int32_t kv_fp8;          // the KV pool holds E4M3 codes of value / scale (else bf16)
  float k_scale, v_scale;  // fp8 scales (1 for bf16)
};

// Waves per workgroup of the per-tile attention kernel.
#define ATT_WAVES 4

// Block-table entries one attention work item stages in LDS (a wave's
// slice); split_len is capped so that a split spans at most this many
// blocks.
#define ATT_TBL 512

// Query columns (rows x heads of one KV head) per block-kernel work item.
#define ATT_BLOCK_COLS 256

// Row kernel: waves per workgroup, the longest context (keys) it takes, the
// most query heads per KV head it merges, and the fewest workgroups
// (sequences x KV heads) it runs with.
#define ATT_ROW_WAVES 8
#define ATT_ROW_KEYS 1024
#define ATT_ROW_G 8
#define ATT_ROW_MIN_WG 64

// Attention work decomposition chosen by the host for one step.
struct AttnPlan {
  int32_t split_len;   // keys per block-kernel work item (multiple of 32)
  int32_t max_splits;  // stride of the partial buffers
  int32_t grid_items;  // waves of the per-tile kernel (a multiple of its workgroup)
  int32_t max_ctx;     // host bound on ctx + n_new that sized the launch
  // Piece lengths of the per-tile schedule, in 32-key steps: at least
  // piece_lo (so that no (sequence, tile) spans more than max_splits
  // pieces), at most piece_hi (a piece's block-table slice fits in LDS).
  int32_t piece_lo, piece_hi;
  // Sequences with at least block_min new rows (prefill chunks) run on the
  // block kernel, block_rows rows per work item (0: every sequence runs on
  // the per-tile kernel); grid_items_b bounds its work items.
  int32_t block_min, block_rows, grid_items_b;
  // Decode-only steps over short contexts: one workgroup per (sequence, KV
  // head), its waves splitting the keys and merging in LDS (no combine).
  int32_t row_kernel;
};

// Row maps and attention schedule (one workgroup) together with the
// embedding gather + first RMSNorm of every row (x, and h as hi/lo planes).
hipError_t launch_prep_embed(const StepMeta& m, const RowMaps& maps, const ModelDims& md,
                             const AttnPlan& ap, const uint16_t* embed, const uint16_t* gain,
                             float* x, uint16_t* h_hi, uint16_t* h_lo, uint32_t* status,
                             hipStream_t st);

// Activation storage. The residual stream x and the QKV projection are fp32
// [rows][width]. Activations that feed an MFMA contraction (norm outputs,
// rotated queries, attention output, SwiGLU product) are "split": two bf16
// planes hi and lo with hi + lo = the fp32 value (split_bf in common.h). The
// rotated queries are row-major planes [rows][width]; the inputs of the
// projections are in operand tiles (tile_at in common.h).

// x[r] = embed[tokens[r]] (fp32), h[r] = rmsnorm(x[r]) * gain (split).

// The end of a residual projection and the norm that follows it, per row r:
// x[r] += sum over s < S of part[s][r] (S > 1: the projection's split-K
// partials, summed in split order; S <= 1: the projection already added
// itself to x), then h[dst] = rmsnorm(x[r]) * gain (split), with dst =
// row_out ? row_out[r] : r and no norm where dst < 0. With row_out, the
// n_out output rows whose out_row is -1 (refused) are zeroed.
hipError_t launch_resid_norm(float* x, const float* part, int32_t S, int32_t R,
                             const int32_t* row_out, const int32_t* out_row, int32_t n_out,
                             const uint16_t* gain, int32_t d, float eps, uint16_t* h_hi,
                             uint16_t* h_lo, hipStream_t st);

// RoPE on q and k of every row at its position; q to q_out (split), k and v
// rounded to bf16 and appended into the layer's K and V regions of the pool
// through the block tables. S > 1: the projection is the sum of the S split
// partials part[s][r][.] (in split order), also stored into qkv; otherwise
// it is read from qkv.
hipError_t launch_rope_append(float* qkv, const float* part, int32_t S, int32_t R,
                              const StepMeta& m, const RowMaps& maps, const double* rope_cs,
                              const ModelDims& md, uint16_t* q_hi, uint16_t* q_lo,
                              void* pool_k, void* pool_v, uint32_t* status, hipStream_t st);

// Paged GQA attention for every row (decode rows and prefill chunks), split
// over keys, then the split combine into out [R][n_heads*head_dim] (split).
// Not for a plan that takes the row kernel (ap.row_kernel): see below.
hipError_t launch_attention(const uint16_t* q_hi, const uint16_t* q_lo, int32_t R,
                            const StepMeta& m, const RowMaps& maps, const ModelDims& md,
                            const AttnPlan& ap, const void* pool_k, const void* pool_v,
                            float* part_ml, float* part_o, uint16_t* out_hi, uint16_t* out_lo,
                            uint32_t* status, hipStream_t st);

// Decode-only steps whose plan takes the row kernel (ap.row_kernel): the
// step's RoPE + KV append and attention in one launch. Workgroup (sequence,
// KV head g) rotates and appends its row's K and V of head g and its G
// query heads (what launch_rope_append does for them), then attends over
// the sequence's keys, merging its waves' results in LDS.
hipError_t launch_rope_attention_rows(float* qkv, const float* part, int32_t S, int32_t R,
                                      const StepMeta& m, const RowMaps& maps,
                                      const double* rope_cs, const ModelDims& md,
                                      const AttnPlan& ap, uint16_t* q_hi, uint16_t* q_lo,
                                      void* pool_k, void* pool_v, uint16_t* out_hi,
                                      uint16_t* out_lo, uint32_t* status, hipStream_t st);

// --------------------------------------------------------------------- GEMM

enum GemmEpilogue { EPI_F32 = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

// Weights reach the GEMM in a packed layout: tiles of 16 rows x 32 k, tile
// (nb, kb) at element offset (nb * ceil(K/32) + kb) * 512, and inside a tile
// lane l's 8 values (row nb*16 + l%16, k kb*32 + 8*(l/16) .. +8) at l * 8.
// Rows past N and k past K are zero.
size_t packed_elems(int32_t N, int32_t K);
// int8 weights: the padded codes (k-pair order), then the float32 row scales.
size_t packed8_codes_bytes(int32_t N, int32_t K);
size_t packed8_bytes(int32_t N, int32_t K);
hipError_t launch_pack8(const int8_t* W, const float* scale, int32_t N, int32_t K, uint8_t* out,
                        hipStream_t st);
hipError_t launch_pack(const uint16_t* W, int32_t N, int32_t K, uint16_t* out, hipStream_t st);

// Elements of one plane of a split activation buffer in operand tiles
// (rows and columns rounded up to 16 and 32; the padding columns must hold
// zeros -- the engine clears these buffers once -- because the contractions
// read whole tiles).
inline size_t tile_plane_elems(size_t rows, size_t w) {
  return (rows + 15) / 16 * 16 * ((w + 31) / 32 * 32);
}

struct GemmArgs {
  const uint16_t* X;    // [R][K] split activation in operand tiles: hi plane
  const uint16_t* Xlo;  //                                             lo plane
                        // (not read by EPI_LOGITS: the LM head takes hi alone)
  int32_t R, K;
  const uint16_t* W;    // [N][K] bf16, packed (int8 k-pairs when w8)
  const uint16_t* W2;   // second packed matrix for EPI_SWIGLU (up), [N][K]
  const float* Ws;      // w8: float32 row scales of W (padded to 256 rows)
  const float* Ws2;     //     and of W2
  int32_t w8;           // the weights are int8 codes
  int32_t N;
  int32_t epi;
  float* Y;             // EPI_F32 out [R][N]; EPI_RESID in/out [R][N] (fp32)
  uint16_t* Yh;         // EPI_SWIGLU out [R][N] split, operand tiles: hi plane
  uint16_t* Yl;         //                                         lo plane
  float* logits;        // EPI_LOGITS out [R][N] (nullable: argmax only)
  float* amax_val;      // EPI_LOGITS per-(row, column tile) maxima [R][amax_stride]
  int32_t* amax_idx;
  int32_t amax_stride;
  float* partials;      // split-K partial sums
  size_t partials_cap;  // floats available there
  int32_t* splits_out;  // nullable: the launch leaves S > 1 partials unsummed
                        // for the caller (EPI_F32, EPI_RESID) and stores S here
};

// Number of argmax partials per row the logits GEMM writes (column tiles).
int32_t gemm_amax_tiles(int32_t R, int32_t N, int32_t K, int32_t w8);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);

// tokens[j] = lowest id of the row maximum over the argmax partials.
hipError_t launch_argmax_reduce(const float* amax_val, const int32_t* amax_idx, int32_t n_tiles,
                                int32_t stride, int32_t n, int32_t* tokens, hipStream_t st);

// ------------------------------------------------------------------ sampler

// Per-slot sampler state in the caller's slot buffer.
#define SLOT_MAX_FORBIDDEN 8
struct SlotParams {
  float temperature, top_p;
  int32_t top_k;
  float freq_penalty, presence_penalty, penalty_decay;
  uint64_t seed;
  uint64_t request_id;
  int32_t n_forbidden;
  int32_t forbidden[SLOT_MAX_FORBIDDEN];  // ids whose penalised logit is -inf
  int32_t pad_;
};
static_assert(sizeof(SlotParams) == 80, "slot parameter layout");

// Floats of sampler scratch per row for a vocabulary of V.
int32_t sampler_row_floats(int32_t V);
hipError_t launch_sampler(const float* logits, int32_t n, int32_t V, const int32_t* slots,
                          const int32_t* step_ids, const int32_t* out_seq, const SlotParams* params,
                          float* counts, int32_t max_slots, float* scratch, int32_t* tokens,
                          uint32_t* status, hipStream_t st);

// Streaming-read probe (probe.hip): `blocks` x 1024 threads read `bytes`
// (a multiple of 16) at `buf` once; one XOR fold per thread to `out`.
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, int32_t blocks,
                             hipStream_t st);

// The current device's fixed sampler scratch (a static device array of
// *floats floats), for the allocation-free sampler entry point; looked up once
// per device.
hipError_t noalloc_scratch(float** ptr, size_t* floats);

// -------------------------------------------------------------------- misc

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, size_t n, hipStream_t st);

}  // namespace cbd

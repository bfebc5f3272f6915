// gemm.hip -- the weight-streaming skinny GEMM of the step, on MFMA.
//
//   Y[r][n] = sum_k X[r][k] * W[n][k]      X: [R][K] fp32 as bf16 hi + lo
//                                          W: [N][K] bf16 (read once)
//
// Decode is weight-bandwidth bound: every weight byte is used by the R rows of
// the step (Go under the hood 20.3.2: one weight read serves the whole batch),
// so the kernel streams W from HBM exactly once per column tile and keeps X
// close (it is small and shared by every workgroup through L2 and L1).
//
// Mapping onto v_mfma_f32_16x16x32_bf16: the A operand is a 16-row fragment
// of W (16 output columns), the B operand a 16-row fragment of X, so one
// instruction yields a 16 (columns) x 16 (rows) tile. Lane l holds 8
// consecutive k of row (l % 16) of each operand; the four lane groups
// (l / 16) hold consecutive 8-k pieces. The weights are stored pre-packed in
// exactly that operand order (16 x 32 tiles, lane-major), so every
// wave-wide weight load is one contiguous 1 KB tile. Tiles are grouped by
// 16 column blocks (256 columns): a group stores the 16 blocks' tiles of
// k-tile 0, then of k-tile 1, and so on, so that a workgroup that covers
// 256 columns reads one contiguous 16 KB run per 32 k (the DRAM sees a few
// long runs instead of 16 scattered ones; measured about 5-10% faster on the
// LM head than blocks stored one after another).
//
// The layer projections' activations are fp32 values carried as two bf16
// planes (hi, lo), so each weight fragment meets two B operands: acc +=
// W.X_hi, acc += W.X_lo. Both products are exact in the fp32 accumulator,
// and the result is the fp32 dot product of W with X to within 2^-17
// relative per term. The second MFMA costs nothing while the weights stream
// from HBM (a 16 x 32 weight tile per 2 x 16 rows of MFMA work leaves the
// matrix cores idle most of the time at these row counts). The LM head is a
// bf16 contraction: its input is the hi plane alone (the final norm's
// output rounded to nearest bf16), one MFMA per weight fragment and row
// fragment, which halves its matrix work where that is what bounds it (at
// 128-256 rows on the dense path).
//
// Up to 64 rows run on the stream path below, more rows on the dense path.
// S workgroups along K leave fp32 partials that a second kernel (or the
// consumer of the result) sums in fixed split order and passes through the
// epilogue. Epilogues: fp32 store,
// fp32 residual add (x += acc), SwiGLU over a gate/up pair
// (a = silu(g) * u, stored split), and fp32 logits with per-tile argmax
// partials (lowest id on ties).
#include "common.h"
#include "kernels.h"

namespace cbd {

// Element offset of k-tile kt of 16-column block nb in a packed matrix with
// KT k-tiles, and the distance between consecutive k-tiles of one block.
__device__ __forceinline__ size_t wtile(int nb, int kt, int KT) {
  return (((size_t)(nb >> 4) * KT + kt) * 16 + (nb & 15)) * 512;
}
#define WT_NEXT (16 * 512)

// int8 codes are packed in k-pairs: two consecutive 32-k tiles of one
// 16-column block, lane l's 16 bytes holding its 8 codes of the first tile
// and then its 8 codes of the second, so one 16-byte load per lane feeds a
// whole 64-k stage. Byte offset of pair kp of block nb (KP pairs per
// block), grouped by 16 blocks like the bf16 tiles, and the distance
// between consecutive pairs of one block. The matrix's float32 row scales
// follow its codes.
__device__ __forceinline__ size_t wpair8(int nb, int kp, int KP) {
  return (((size_t)(nb >> 4) * KP + kp) * 16 + (nb & 15)) * 1024;
}
#define WP8_NEXT (16 * 1024)

// Eight int8 codes (a uint2, code i in byte i) -> eight bf16 values in MFMA
// operand order (a uint4, value i in half-word i). |q| <= 127 has at most 8
// significant bits, so the float of q truncated to bf16 is exact.
__device__ __forceinline__ uint4 i8x8_to_bf16x8(uint2 c) {
  auto two = [](uint32_t w, int b) {  // bytes b and b + 1 of w
    const float x = (float)((int32_t)(w << (24 - 8 * b)) >> 24);
    const float y = (float)((int32_t)(w << (16 - 8 * b)) >> 24);
    return __builtin_amdgcn_perm(__float_as_uint(y), __float_as_uint(x), 0x07060302u);
  };
  return make_uint4(two(c.x, 0), two(c.x, 2), two(c.y, 0), two(c.y, 2));
}

template <int EPI>
struct EpiTraits {
  static constexpr int NM = EPI == EPI_SWIGLU ? 2 : 1;  // weight matrices
  static constexpr int PL = EPI == EPI_LOGITS ? 1 : 2;  // activation planes (hi, lo)
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// Apply the epilogue to 4 consecutive columns n..n+3 of row r.
template <int EPI>
__device__ __forceinline__ void epilogue4(const GemmArgs& a, int r, int n, const float* v0,
                                          const float* v1) {
  const size_t at = (size_t)r * a.N + n;
  if (EPI == EPI_F32) {
    *reinterpret_cast<float4*>(a.Y + at) = make_float4(v0[0], v0[1], v0[2], v0[3]);
  } else if (EPI == EPI_RESID) {
    float4* p = reinterpret_cast<float4*>(a.Y + at);
    float4 x = *p;
    x.x += v0[0];
    x.y += v0[1];
    x.z += v0[2];
    x.w += v0[3];
    *p = x;
  } else if (EPI == EPI_SWIGLU) {
    store_split4(a.Yh, a.Yl, tile_at(r, n, (a.N + 31) / 32), silu_f(v0[0]) * v1[0], silu_f(v0[1]) * v1[1],
                 silu_f(v0[2]) * v1[2], silu_f(v0[3]) * v1[3]);
  } else {  // EPI_LOGITS
    if (a.logits)
      *reinterpret_cast<float4*>(a.logits + at) = make_float4(v0[0], v0[1], v0[2], v0[3]);
  }
}

// Write a wave's accumulators: lane l holds columns n0 + 16 nt + 4 lg + (0..3)
// of row r0 + 16 rt + lr. With a K split (S > 1) they go to the partials of
// split ks; otherwise through the epilogue, and the logits epilogue also
// leaves this wave's per-row maximum (lowest column on ties) in argmax
// partial `tile`.
template <int RT, int NT, int EPI>
__device__ __forceinline__ void store_tile(const GemmArgs& a,
                                           const floatx4_t (&acc)[EpiTraits<EPI>::NM][NT][RT],
                                           int r0, int n0, int ks, int S, int tile) {
  constexpr int NM = EpiTraits<EPI>::NM;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int R = a.R, N = a.N;
  if (S > 1) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          int r = r0 + 16 * rt + lr, n = n0 + 16 * nt + 4 * lg;
          if (r < R && n < N)
            *reinterpret_cast<float4*>(a.partials + (((size_t)ks * NM + m) * R + r) * N + n) =
                make_float4(acc[m][nt][rt][0], acc[m][nt][rt][1], acc[m][nt][rt][2],
                            acc[m][nt][rt][3]);
        }
    return;
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = r0 + 16 * rt + lr;
    float best = -INFINITY;
    int bidx = 0x7fffffff;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + 16 * nt + 4 * lg;
      float v0[4], v1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v0[i] = acc[0][nt][rt][i];
        v1[i] = acc[NM - 1][nt][rt][i];
      }
      if (r < R && n < N) {
        epilogue4<EPI>(a, r, n, v0, v1);
        if (EPI == EPI_LOGITS) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v0[i] > best) {  // ascending columns: first maximum wins
              best = v0[i];
              bidx = n + i;
            }
        }
      }
    }
    if (EPI == EPI_LOGITS) {
#pragma unroll
      for (int o = 16; o < 64; o <<= 1) {
        float v = __shfl_xor(best, o, 64);
        int i = __shfl_xor(bidx, o, 64);
        if (v > best || (v == best && i < bidx)) {
          best = v;
          bidx = i;
        }
      }
      if (lg == 0 && r < R) {
        a.amax_val[(size_t)r * a.amax_stride + tile] = best;
        a.amax_idx[(size_t)r * a.amax_stride + tile] = bidx;
      }
    }
  }
}

// ------------------------------------------------------- the stream path
//
// One kernel for any row count. A workgroup is NW waves side by side along N
// (each NT column fragments, RT row fragments) over one K range. Per 64-k
// stage the workgroup's activation tile (RT x 16 rows x 64 k per plane:
// RT x 4 KB with hi and lo, RT x 2 KB for the LM head's one plane, kept in
// MFMA operand order -- block (rt, plane, 32-k half) is 64 lanes x 16
// bytes) is copied by direct global->LDS loads into a ring of
// D LDS stages, with no registers involved; each wave's weights stream
// through a ring of D register stages. The loads of stage c + D - 1 are
// issued right after the barrier of stage c, so D - 2 later stages stay in
// flight while stage c waits: the wait is an explicit vector-memory count
// (the LDS copies carry no register the compiler could wait on), exact
// because every stage issues the same number of loads per wave and the
// barrier orders the stages. Stages are padded to a multiple of D; the
// activation pieces at or beyond kend (padding, a K tail) are zeroed in LDS
// after their copy lands, so the weights read there meet zeros.
// Two waves per SIMD (256 registers, accumulators included). A workgroup
// has NW = 4 or 8 waves: 8 halve the activation copies per weight byte, which
// pays on the LM head (64 rows: 173 -> 163 us) but not on the narrower layer
// matrices, whose grids then leave CUs idle. The LM head's 8-wave
// workgroups cover 512 columns, 251 of them for a 128256-column vocabulary,
// one per CU at every row count: at 17-32 rows, 501 workgroups of 4 waves
// finished unevenly (per-workgroup timestamps: half by about 105 us, the
// rest at up to 168) and the launch took 172 us against 161 with 8 waves.
// A vocabulary past 256 such workgroups takes 4-wave ones (see the plan).
// The grid is one-dimensional with the K split varying fastest: workgroup i
// runs on XCD i mod 8, so at 8 splits each XCD holds one split (and reads
// one eighth of the activation into its L2), at 4 splits each split sits on
// two XCDs. Numbered column-group first, every XCD would fetch the whole
// activation: at 64 rows that was 8 of the 46 MB the O projection moved.
// W8: int8 weights (k-pair packing above; one 16-byte load per column
// fragment per stage, widened to bf16 in registers), the row scales applied
// to the accumulators before the epilogue.
template <int RT, int NT, int D, int NW, int EPI, bool W8>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void gemm_stream_kernel(GemmArgs a, int kc, int S, int n_groups) {
  constexpr int NM = EpiTraits<EPI>::NM;
  constexpr int PL = EpiTraits<EPI>::PL;
  constexpr int BLK = RT * 2 * PL;            // 1 KB activation blocks per stage
  constexpr int CPW = (BLK + NW - 1) / NW;    // activation copies per wave per stage
  constexpr int BLKP = CPW * NW;              // LDS blocks per stage (see below)
  constexpr int WL = W8 ? 1 : 2;              // weight loads per column fragment per stage
  constexpr int LPS = NM * NT * WL + CPW;     // loads per stage per wave
  static_assert(D >= 3, "ring depth");
  extern __shared__ uint4 xs[];               // [D][BLKP][64]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int ks = blockIdx.x % S;
  const int grp = blockIdx.x / S;
  const int tile = (grp % n_groups) * NW + wave;
  const int n0 = tile * (16 * NT);
  const int r0 = (grp / n_groups) * (16 * RT);
  const int K = a.K, N = a.N, R = a.R;
  const int kbeg = ks * kc;                   // a multiple of 64
  const int kend = min(K, kbeg + kc);
  const int nst0 = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;
  const int nst = (nst0 + D - 1) / D * D;     // padded to whole ring turns

  const int KT = (K + 31) / 32;
  const int KP = (K + 63) / 64;  // int8 k-pairs per block
  const uint16_t* wp[NM][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int nb = (n0 >> 4) + nt;
    if (nb * 16 >= N) nb = 0;  // past N: read block 0, never stored
    if constexpr (W8) {  // byte offsets into the int8 codes
      const size_t off = wpair8(nb, kbeg / 64, KP) + lane * 16;
      wp[0][nt] = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.W) + off);
      if (NM == 2)
        wp[NM - 1][nt] = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.W2) + off);
    } else {
      const size_t off = wtile(nb, kbeg / 32, KT) + lane * 8;
      wp[0][nt] = a.W + off;
      if (NM == 2) wp[NM - 1][nt] = a.W2 + off;
    }
  }
  // This wave copies blocks b = wave + NW i of every stage; block (rt, pl, h)
  // of stage c is the operand tile (row fragment r0 / 16 + rt, k-block
  // kbeg / 32 + 2 c + h) of plane pl: lane `lane` holds row r0 + 16 rt + lr,
  // k + 32 h + 8 lg. Fragments past R read the last one (their outputs are
  // never stored). With more waves than blocks (one row fragment, 8 waves)
  // the waves past BLK copy such a clamped tile into a spare LDS block that
  // is never read, so that every wave issues the same loads per stage and
  // the vector-memory wait counts stay exact.
  const uint16_t* xsrc[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int b = wave + NW * i;
    const int rt = b / (2 * PL), pl = (b >> 1) % PL;
    const int f = min(r0 / 16 + rt, (R - 1) >> 4);
    xsrc[i] = (pl ? a.Xlo : a.X) + (size_t)f * KT * 512 + lane * 8;
  }

  floatx4_t acc[NM][NT][RT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[m][nt][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  uint4 w[D][NM][NT][WL];
  // Issue every load of stage c (clamped into range; see above) into slot j.
  auto issue = [&](int j, int c) {
    if constexpr (W8) {
      const int t = min(kbeg / 64 + c, KP - 1) - kbeg / 64;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          w[j][m][nt][0] = load_stream16(reinterpret_cast<const uint16_t*>(
              reinterpret_cast<const uint8_t*>(wp[m][nt]) + (size_t)t * WP8_NEXT));
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = min(kbeg / 32 + 2 * c + h, KT - 1) - kbeg / 32;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            w[j][m][nt][h] = load_stream16(wp[m][nt] + (size_t)t * WT_NEXT);
      }
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int b = wave + NW * i;
      const int kb = min(kbeg / 32 + 2 * c + (b & 1), KT - 1);
      copy16_to_lds(xsrc[i] + (size_t)kb * 512, xs + ((size_t)j * BLKP + b) * 64);
    }
  };
  auto compute = [&](int j, int c) {
    const uint4* buf = xs + (size_t)j * BLKP * 64;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 xf[RT][PL];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int pl = 0; pl < PL; ++pl) xf[rt][pl] = buf[((rt * PL + pl) * 2 + h) * 64 + lane];
      bf16x8_t wf[NM][NT];
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if constexpr (W8) {
            const uint4 q = w[j][m][nt][0];
            wf[m][nt] = as_bf16x8(i8x8_to_bf16x8(h ? make_uint2(q.z, q.w) : make_uint2(q.x, q.y)));
          } else {
            wf[m][nt] = as_bf16x8(w[j][m][nt][h]);
          }
        }
#pragma unroll
      for (int pl = 0; pl < PL; ++pl)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              acc[m][nt][rt] = mfma16x16x32(wf[m][nt], as_bf16x8(xf[rt][pl]), acc[m][nt][rt]);
    }
  };

  if (nst > 0) {
#pragma unroll
    for (int j = 0; j < D - 1; ++j) issue(j, j);
    for (int c0 = 0; c0 < nst; c0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int c = c0 + j;
        // Stage c's loads were followed by those of stages c + 1 .. c + D - 2.
        wait_vmem<(D - 2) * LPS>();
        if (kbeg + 64 * c + 64 > kend) {  // K tail or padding: zero what lies past kend
#pragma unroll
          for (int i = 0; i < CPW; ++i) {
            const int b = wave + NW * i;
            if (kbeg + 64 * c + 32 * (b & 1) + 8 * lg >= kend)
              xs[((size_t)j * BLKP + b) * 64 + lane] = make_uint4(0, 0, 0, 0);
          }
        }
        __syncthreads();
        issue((j + D - 1) % D, min(c + D - 1, nst - 1));
        compute(j, c);
      }
    }
  }
  wait_vmem<0>();  // no LDS copy may land after the workgroup exits
  if constexpr (W8) {  // the row scales of the weights (this lane's 4 output columns)
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = n0 + 16 * nt + 4 * lg;
        float4 sc = make_float4(0.f, 0.f, 0.f, 0.f);  // past N (never stored)
        if (n < N) sc = *reinterpret_cast<const float4*>((m ? a.Ws2 : a.Ws) + n);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          acc[m][nt][rt][0] *= sc.x;
          acc[m][nt][rt][1] *= sc.y;
          acc[m][nt][rt][2] *= sc.z;
          acc[m][nt][rt][3] *= sc.w;
        }
      }
  }
  store_tile<RT, NT, EPI>(a, acc, r0, n0, ks, S, tile);
}

// ------------------------------------------------------- the dense path
//
// For many rows (a prefill chunk, a large batch) the projection is a dense
// contraction and the aim is MFMA time. A workgroup of 8 waves (2 along N
// x 4 along R) owns a 256-column x 16 RF-row tile; each wave a 128-column x
// 4 RF-row block: per 32-k stage it reads 8 weight fragments and RF/4
// activation fragments per plane (hi and lo; the LM head's hi alone) from
// LDS and issues 2 RF MFMAs per plane, and the activation tile is fetched
// once per 256 columns. Both operands reach
// LDS by direct global->LDS copies into a D-stage ring: 16 weight tiles
// (1 KB each, straight from the packed layout) and RF fragments per plane.
// The ring discipline is the stream path's: stage c + D - 1 is issued right
// after the barrier of stage c, and the wait for stage c is an exact
// vector-memory count (every issue is the same LPS copies per wave; past
// the last stage the last stage is re-issued, never computed).
// The workgroups that share a weight tile (its row groups and K splits) are
// numbered so that they land on one XCD (workgroup i runs on XCD i mod 8):
// their repeated weight reads meet in that XCD's L2. Past K the packed
// weights and the operand tiles' padding columns are zero, so a K tail
// needs no masking (every split but the last ends on a 32-k boundary).
#define DENSE_TN 256

#define DENSE_WAVES 8

template <int RF, int D, int EPI>
__global__ __launch_bounds__(64 * DENSE_WAVES) void gemm_dense_kernel(GemmArgs a, int kc, int S,
                                                                      int n_tiles, int r_groups) {
  constexpr int NM = EpiTraits<EPI>::NM;
  constexpr int PL = EpiTraits<EPI>::PL;
  constexpr int NT = 8 / NM;       // column fragments per matrix per wave
  constexpr int WR = DENSE_WAVES / 2;  // waves along R
  constexpr int RH = RF / WR;      // row fragments per wave
  constexpr int TW = 16;           // weight tiles per stage
  constexpr int TS = TW + PL * RF; // 1 KB tiles per stage
  constexpr int LPS = TS / DENSE_WAVES;  // copies per stage per wave
  static_assert(TS % DENSE_WAVES == 0 && RF % WR == 0, "tile counts");
  static_assert(D >= 3 && (D - 2) * LPS < 64, "ring depth");
  extern __shared__ uint4 ring[];  // [D][TS][64]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wr = wave >> 1;
  const int lr = lane & 15, lg = lane >> 4;
  const int id = blockIdx.x;
  const int per = r_groups * S;
  const int q = id >> 3;
  const int n_tile = (q / per) * 8 + (id & 7);
  if (n_tile >= n_tiles) return;  // padding of the XCD numbering; no barrier yet
  const int rg = (q % per) / S, ks = (q % per) % S;
  const int K = a.K, R = a.R, N = a.N;
  const int r_base = rg * 16 * RF;
  const int kbeg = ks * kc;  // a multiple of 32
  const int kend = min(K, kbeg + kc);
  const int nst = kend > kbeg ? (kend - kbeg + 31) / 32 : 0;
  const int KT = (K + 31) / 32;
  constexpr int CB = 2 * NT;  // 16-column blocks per matrix per workgroup

  // Copy sources: this wave issues tiles t = wave + 8 i; t < 16 are weight
  // tiles (matrix t / CB, column block t % CB), the rest activation operand
  // tiles (u = t - 16: row fragment u / PL, plane u % PL; fragments past R
  // read the last one, whose outputs are never stored).
  const uint16_t* src[LPS];
#pragma unroll
  for (int i = 0; i < LPS; ++i) {
    const int t = wave + DENSE_WAVES * i;
    if (i < TW / DENSE_WAVES) {
      const int m = t / CB;
      int nb = n_tile * CB + t % CB;
      if (nb * 16 >= N) nb = 0;  // past N: read block 0, never stored
      src[i] = (m ? a.W2 : a.W) + wtile(nb, kbeg / 32, KT) + lane * 8;
    } else {
      const int u = t - TW;
      const int f = min(r_base / 16 + u / PL, (R - 1) >> 4);
      src[i] = (u % PL ? a.Xlo : a.X) + (size_t)f * KT * 512 + lane * 8;
    }
  }
  auto issue = [&](int slot, int c) {
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const int t = wave + DENSE_WAVES * i;
      if (i < TW / DENSE_WAVES)  // weights: streamed once, kept out of L2's way
        copy16_to_lds_nt(src[i] + (size_t)c * WT_NEXT, ring + ((size_t)slot * TS + t) * 64);
      else  // activations: re-read by every column tile, kept in L2
        copy16_to_lds(src[i] + (size_t)min(kbeg / 32 + c, KT - 1) * 512,
                      ring + ((size_t)slot * TS + t) * 64);
    }
  };

  floatx4_t acc[NM][NT][RH];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int rh = 0; rh < RH; ++rh) acc[m][nt][rh] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // The hi products of every accumulator, then the lo products: two MFMAs
  // on one accumulator are 8 RH apart, never back to back (one plane: 8 RH
  // independent accumulators in a row). A wave raises its
  // issue priority for its run of MFMAs, so that the matrix pipe stays fed
  // while the other wave of the SIMD issues its LDS reads and copies (2-5%
  // on the dense launches at 256-560 rows).
  auto compute = [&](int slot) {
    const uint4* buf = ring + (size_t)slot * TS * 64;
    uint4 wf[NM][NT], xf[PL][RH];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) wf[m][nt] = buf[(m * CB + wn * NT + nt) * 64 + lane];
#pragma unroll
    for (int rh = 0; rh < RH; ++rh)
#pragma unroll
      for (int pl = 0; pl < PL; ++pl) xf[pl][rh] = buf[(TW + PL * (wr * RH + rh) + pl) * 64 + lane];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int pl = 0; pl < PL; ++pl)
#pragma unroll
      for (int rh = 0; rh < RH; ++rh)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[m][nt][rh] = mfma16x16x32(as_bf16x8(wf[m][nt]), as_bf16x8(xf[pl][rh]), acc[m][nt][rh]);
    __builtin_amdgcn_s_setprio(0);
  };

  if (nst > 0) {
#pragma unroll
    for (int j = 0; j < D - 1; ++j) issue(j, min(j, nst - 1));
    for (int c = 0; c < nst; ++c) {
      // Stage c's copies were followed by those of stages c + 1 .. c + D - 2.
      wait_vmem<(D - 2) * LPS>();
      __syncthreads();
      issue((c + D - 1) % D, min(c + D - 1, nst - 1));
      compute(c % D);
    }
  }
  wait_vmem<0>();  // no LDS copy may land after the workgroup exits
  store_tile<RH, NT, EPI>(a, acc, r_base + 16 * RH * wr, n_tile * (DENSE_TN / NM) + 16 * NT * wn,
                          ks, S, n_tile * 2 + wn);
}

// Sum the S split partials in split order, then the epilogue (no argmax:
// the logits GEMM never splits K).
template <int EPI>
__global__ void gemm_reduce_kernel(GemmArgs a, int S) {
  constexpr int NM = EpiTraits<EPI>::NM;
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // group of 4 columns
  const int groups = a.N / 4;
  if (q >= (size_t)a.R * groups) return;
  const int r = (int)(q / groups), n = (int)(q % groups) * 4;
  float v[NM][4];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) v[m][i] = 0.f;
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      float4 p = *reinterpret_cast<const float4*>(a.partials + (((size_t)s * NM + m) * a.R + r) * a.N + n);
      v[m][0] += p.x;
      v[m][1] += p.y;
      v[m][2] += p.z;
      v[m][3] += p.w;
    }
  epilogue4<EPI>(a, r, n, v[0], v[NM - 1]);
}

// ------------------------------------------------------------- host side

size_t packed_elems(int32_t N, int32_t K) {
  return (size_t)((N + 255) / 256) * 16 * (size_t)((K + 31) / 32) * 512;
}

__global__ void pack_kernel(const uint16_t* __restrict__ W, int N, int K,
                            uint16_t* __restrict__ out, size_t n16) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // one 16-byte piece
  if (i >= n16) return;
  const int KT = (K + 31) / 32;
  const int lane = (int)(i & 63);
  const size_t tile = i >> 6;
  const int kb = (int)(tile % KT);
  const int nb = (int)(tile / KT);
  const int n = nb * 16 + (lane & 15);
  const int k = kb * 32 + 8 * (lane >> 4);
  uint4 v = make_uint4(0, 0, 0, 0);
  if (n < N && k < K) v = *reinterpret_cast<const uint4*>(W + (size_t)n * K + k);
  reinterpret_cast<uint4*>(out)[(wtile(nb, kb, KT) >> 3) + lane] = v;
}

hipError_t launch_pack(const uint16_t* W, int32_t N, int32_t K, uint16_t* out, hipStream_t st) {
  const size_t n16 = packed_elems(N, K) / 8;
  pack_kernel<<<(unsigned)((n16 + 255) / 256), 256, 0, st>>>(W, N, K, out, n16);
  return hipGetLastError();
}

// int8: codes of the padded matrix (N up to a multiple of 256, K up to 64),
// then its float32 row scales (zero past N).
size_t packed8_codes_bytes(int32_t N, int32_t K) {
  return (size_t)((N + 255) / 256) * 256 * (size_t)((K + 63) / 64) * 64;
}
size_t packed8_bytes(int32_t N, int32_t K) {
  return packed8_codes_bytes(N, K) + (size_t)((N + 255) / 256) * 256 * 4;
}

// One 16-byte piece per thread: lane `lane` of k-pair (nb, kp) holds codes
// k0 .. k0 + 7 and k0 + 32 .. k0 + 39 of row 16 nb + lane % 16, k0 = 64 kp +
// 8 (lane / 16); K is a multiple of 16, so an 8-code run is all in or all
// out of the matrix.
__global__ void pack8_kernel(const int8_t* __restrict__ W, int N, int K, uint8_t* __restrict__ out,
                             size_t n16) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n16) return;
  const int KP = (K + 63) / 64;
  const int lane = (int)(i & 63);
  const size_t pair = i >> 6;
  const int kp = (int)(pair % KP);
  const int nb = (int)(pair / KP);
  const int n = nb * 16 + (lane & 15);
  const int k0 = kp * 64 + 8 * (lane >> 4);
  uint2 a = make_uint2(0, 0), b = make_uint2(0, 0);
  if (n < N && k0 < K) a = *reinterpret_cast<const uint2*>(W + (size_t)n * K + k0);
  if (n < N && k0 + 32 < K) b = *reinterpret_cast<const uint2*>(W + (size_t)n * K + k0 + 32);
  *reinterpret_cast<uint4*>(out + wpair8(nb, kp, KP) + (size_t)lane * 16) = make_uint4(a.x, a.y, b.x, b.y);
}

__global__ void pack_scales_kernel(const float* __restrict__ scale, int N, float* __restrict__ out,
                                   int n_pad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_pad) out[i] = i < N ? scale[i] : 0.f;
}

hipError_t launch_pack8(const int8_t* W, const float* scale, int32_t N, int32_t K, uint8_t* out,
                        hipStream_t st) {
  const size_t codes = packed8_codes_bytes(N, K);
  const size_t n16 = codes / 16;
  pack8_kernel<<<(unsigned)((n16 + 255) / 256), 256, 0, st>>>(W, N, K, out, n16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_pad = (N + 255) / 256 * 256;
  pack_scales_kernel<<<(n_pad + 255) / 256, 256, 0, st>>>(scale, N,
                                                          reinterpret_cast<float*>(out + codes), n_pad);
  return hipGetLastError();
}

// How one projection runs. Up to 64 rows: the stream kernel with RT row
// fragments (16, 32 or 64 rows), NW waves of NT column fragments sharing
// the activation tile, S workgroups splitting K. Measured on the 8B shapes
// at 1-64 rows on MI355X: the LM head wants 64-column waves, 8 to a
// workgroup (each 256-column half of it reads one contiguous run per
// stage); the gate/up pair 16-column waves, 4 to a workgroup, over the
// whole K (no partials, no separate SwiGLU pass); the single matrices
// 32-column waves, 4 to a workgroup, with K split until the grid would
// pass one workgroup per CU. More rows: the dense kernel (see above).
struct GemmPlan {
  bool dense;
  int RT, NT, D, NW, S;
};

// Rows at or above which the dense path runs: past one stream row group
// (64 rows) the stream path would fetch every weight once per group.
#define DENSE_MIN_ROWS 65

// Estimated time (us) of a dense launch: rounds of one workgroup per CU
// (a projection's dense ring needs 96-144 KB of LDS; the LM head's 72 KB
// ring at 8 fragments fits two per CU, which the estimate leaves out: for
// the LM head it only picks the tile height, and measured at 96-256 rows
// it picks the faster one) times the 32-k stages of a
// workgroup times the stage time, which grows with the tile height (fitted
// on the 8B matrices at 128-560 rows: 0.87, 1.19 and 1.5 us at RF = 8, 12,
// 16), plus the split partials written and read back at about 6 TB/s, plus
// the reduce launch a split SwiGLU needs.
static double dense_cost(int R, int N, int K, int NM, int rf, int S) {
  const long long tiles = (long long)((N + DENSE_TN / NM - 1) / (DENSE_TN / NM)) *
                          ((R + 16 * rf - 1) / (16 * rf));
  const long long rounds = (tiles * S + 255) / 256;
  const int stages = ((K + S - 1) / S + 31) / 32;
  double t = (double)rounds * stages * (0.25 + 0.078 * rf);
  if (S > 1) t += (double)S * R * N * NM * 8.0 / 6e6 + (NM == 2 ? 5.0 : 0.0);
  return t;
}

static GemmPlan plan_gemm(int R, int N, int K, int NM, bool logits, size_t partials_cap,
                          bool w8) {
  GemmPlan p{};
  // Row fragments per dense workgroup: the fewest padded rows, then the
  // larger tile (fewer weight re-reads).
  int best = 0, waste = 1 << 30;
  for (int rf : {16, 12, 8}) {
    const int w = (R + 16 * rf - 1) / (16 * rf) * 16 * rf - R;
    if (w < waste) {
      waste = w;
      best = rf;
    }
  }
  const int dense_tiles =
      (N + DENSE_TN / NM - 1) / (DENSE_TN / NM) * ((R + 16 * best - 1) / (16 * best));
  // The dense path wants enough tiles to spread without deep K splits (or a
  // long K, where splitting is cheap); narrow matrices at moderate row
  // counts stay on the stream path.
  // int8 weights always stream (row groups of 64 rows past 64 rows).
  if (!w8 && R >= DENSE_MIN_ROWS && (dense_tiles >= 32 || K >= 8192)) {
    // The tile height and K split with the lowest estimate (the logits
    // epilogue never splits; splits must fit the partial buffer and keep at
    // least 256 k each).
    double t_best = 1e30;
    for (int rf : {16, 12, 8}) {
      if (logits && rf == 12) continue;  // the one-plane tile wants 8 or 16 fragments
      for (int S = 1; S <= (logits ? 1 : 16); ++S) {
        if (S > 1 && (K / S < 256 || (size_t)S * NM * R * N > partials_cap)) break;
        const double t = dense_cost(R, N, K, NM, rf, S);
        if (t < t_best) {
          t_best = t;
          p.RT = rf;
          p.S = S;
        }
      }
    }
    p.dense = true;
    p.NT = 4 / NM;
    p.D = p.RT == 8 && !logits ? 4 : 3;
    return p;
  }
  p.RT = R <= 16 ? 1 : (R <= 32 ? 2 : 4);
  p.NT = logits ? 4 : (NM == 2 ? 1 : 2);
  p.D = 4;
  // The LM head's 512-column workgroups while they fit one per CU (a
  // 128256-column vocabulary: 251); past that, 256-column ones (a 151936-
  // column vocabulary: 297 would leave 41 CUs running two, 126 us per launch
  // at 2048 k against 104 with 594 of 4 waves).
  p.NW = logits && (N + 511) / 512 <= 256 ? 8 : 4;
  p.S = 1;
  if (!logits) {
    const int cols = 16 * p.NW * p.NT;
    const int groups = (N + cols - 1) / cols * ((R + 16 * p.RT - 1) / (16 * p.RT));
    while (groups * p.S * 2 <= 256 && K / (p.S * 2) >= 512) p.S *= 2;
  }
  return p;
}

int32_t gemm_amax_tiles(int32_t R, int32_t N, int32_t K, int32_t w8) {
  const GemmPlan p = plan_gemm(R, N, K, 1, true, 0, w8 != 0);
  if (p.dense) return (N + DENSE_TN - 1) / DENSE_TN * 2;
  const int cols = 16 * p.NT;
  return (N + cols * p.NW - 1) / (cols * p.NW) * p.NW;
}

// The split-K sum for the SwiGLU product, whose output is in operand tiles:
// one wave per output tile, lane 16 j + i summing columns 8 j .. 8 j + 7 of
// tile row i (32-byte runs of the partials, four lanes per 128 bytes of a
// row) in split order, so that the wave writes the tile as one contiguous
// kilobyte per plane. (Four columns per thread in row order scattered 8-byte
// pieces over the tiles and took 54 us at 560 rows against 33 us.)
__global__ __launch_bounds__(256) void gemm_reduce_swiglu_kernel(GemmArgs a, int S) {
  const int lane = threadIdx.x & 63;
  const int KB = (a.N + 31) / 32;
  const size_t t = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // output tile
  if (t >= (size_t)((a.R + 15) / 16) * KB) return;
  const int r = (int)(t / KB) * 16 + (lane & 15);
  const int n = (int)(t % KB) * 32 + 8 * (lane >> 4);
  if (r >= a.R || n >= a.N) return;  // N % 16 == 0: an 8-column run is all in or all out
  float g[8], u[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) g[e] = u[e] = 0.f;
  for (int s = 0; s < S; ++s) {
    const float4* pg = reinterpret_cast<const float4*>(a.partials + (((size_t)s * 2) * a.R + r) * a.N + n);
    const float4* pu = reinterpret_cast<const float4*>(a.partials + (((size_t)s * 2 + 1) * a.R + r) * a.N + n);
    const float4 g0 = pg[0], g1 = pg[1], u0 = pu[0], u1 = pu[1];
    g[0] += g0.x; g[1] += g0.y; g[2] += g0.z; g[3] += g0.w;
    g[4] += g1.x; g[5] += g1.y; g[6] += g1.z; g[7] += g1.w;
    u[0] += u0.x; u[1] += u0.y; u[2] += u0.z; u[3] += u0.w;
    u[4] += u1.x; u[5] += u1.y; u[6] += u1.z; u[7] += u1.w;
  }
  bf16_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) split_bf(silu_f(g[e]) * u[e], h[e], l[e]);
  const size_t at = t * 512 + (size_t)lane * 8;  // = tile_at(r, n, KB)
  *reinterpret_cast<uint4*>(a.Yh + at) =
      make_uint4((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16),
                 (uint32_t)h[4] | ((uint32_t)h[5] << 16), (uint32_t)h[6] | ((uint32_t)h[7] << 16));
  *reinterpret_cast<uint4*>(a.Yl + at) =
      make_uint4((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16),
                 (uint32_t)l[4] | ((uint32_t)l[5] << 16), (uint32_t)l[6] | ((uint32_t)l[7] << 16));
}

template <int EPI>
static hipError_t launch_reduce(const GemmArgs& a, int S, hipStream_t st) {
  if constexpr (EPI == EPI_SWIGLU) {
    const size_t tiles = (size_t)((a.R + 15) / 16) * ((a.N + 31) / 32);
    gemm_reduce_swiglu_kernel<<<(unsigned)((tiles + 3) / 4), 256, 0, st>>>(a, S);
  } else {
    const size_t threads = (size_t)a.R * (a.N / 4);
    gemm_reduce_kernel<EPI><<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(a, S);
  }
  return hipGetLastError();
}

// After the GEMM launch: the split-K sum, unless the caller takes the
// partials (splits_out, fp32 and residual epilogues only).
template <int EPI>
static hipError_t finish_splits(const GemmArgs& a, int S, hipStream_t st) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool defer = a.splits_out && (EPI == EPI_F32 || EPI == EPI_RESID);
  if (defer) *a.splits_out = S;
  if (S == 1 || defer) return hipSuccess;
  return launch_reduce<EPI>(a, S, st);
}

// K range per split: a multiple of `align`; returns the split count that
// covers K (the requested one, possibly fewer).
static int split_k(int K, int S, int align, int* kc) {
  int c = (K + S - 1) / S;
  c = (c + align - 1) / align * align;
  *kc = c;
  return (K + c - 1) / c;
}

template <int RT, int NT, int D, int NW, int EPI, bool W8>
static hipError_t launch_stream(const GemmArgs& a, int S, hipStream_t st) {
  constexpr int NM = EpiTraits<EPI>::NM;
  const int cols = 16 * NT * NW;
  const int n_groups = (a.N + cols - 1) / cols;
  const int r_groups = (a.R + 16 * RT - 1) / (16 * RT);
  int kc;
  S = split_k(a.K, S, 64, &kc);
  if (S > 1 && (size_t)S * NM * a.R * a.N > a.partials_cap) S = split_k(a.K, 1, 64, &kc);
  constexpr int PL = EpiTraits<EPI>::PL;
  const size_t lds = (size_t)D * ((RT * 2 * PL + NW - 1) / NW * NW) * 1024;  // <= 64 KB as instantiated
  gemm_stream_kernel<RT, NT, D, NW, EPI, W8><<<(unsigned)(n_groups * S * r_groups), 64 * NW, lds, st>>>(
      a, kc, S, n_groups);
  return finish_splits<EPI>(a, S, st);
}

template <int RF, int D, int EPI>
static hipError_t launch_dense(const GemmArgs& a, int S, hipStream_t st) {
  constexpr int NM = EpiTraits<EPI>::NM;
  const int n_tiles = (a.N + DENSE_TN / NM - 1) / (DENSE_TN / NM);
  const int r_groups = (a.R + 16 * RF - 1) / (16 * RF);
  int kc;
  S = split_k(a.K, S, 32, &kc);
  if (S > 1 && (size_t)S * NM * a.R * a.N > a.partials_cap) S = split_k(a.K, 1, 32, &kc);
  const size_t lds = (size_t)D * (16 + EpiTraits<EPI>::PL * RF) * 1024;
  static bool lds_set = false;  // above 64 KB the launch must be allowed first
  if (!lds_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_dense_kernel<RF, D, EPI>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_set = true;
  }
  const unsigned grid = (unsigned)((n_tiles + 7) / 8 * 8 * r_groups * S);
  gemm_dense_kernel<RF, D, EPI><<<grid, 64 * DENSE_WAVES, lds, st>>>(a, kc, S, n_tiles, r_groups);
  return finish_splits<EPI>(a, S, st);
}

template <int EPI, bool W8>
static hipError_t launch_stream_plan(const GemmArgs& a, const GemmPlan& p, hipStream_t st) {
  constexpr int NM = EpiTraits<EPI>::NM;
#define ST(RT_, NT_, NW_)                                \
  if (p.RT == RT_ && p.NT == NT_ && p.NW == NW_) \
    return launch_stream<RT_, NT_, 4, NW_, EPI, W8>(a, p.S, st);
  if constexpr (NM == 2) {
    ST(1, 1, 4) ST(2, 1, 4)
    return launch_stream<4, 1, 4, 4, EPI, W8>(a, p.S, st);
  } else if constexpr (EPI == EPI_LOGITS) {
    ST(1, 4, 8) ST(2, 4, 8) ST(1, 4, 4) ST(2, 4, 4) ST(4, 4, 4)
    return launch_stream<4, 4, 4, 8, EPI, W8>(a, p.S, st);
  } else {
    ST(1, 2, 4) ST(2, 2, 4)
    return launch_stream<4, 2, 4, 4, EPI, W8>(a, p.S, st);
  }
#undef ST
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& a, hipStream_t st) {
  constexpr int NM = EpiTraits<EPI>::NM;
  const GemmPlan p = plan_gemm(a.R, a.N, a.K, NM, EPI == EPI_LOGITS, a.partials_cap, a.w8 != 0);
  if (a.w8) return launch_stream_plan<EPI, true>(a, p, st);
  if (p.dense) {
    if (p.RT == 16) return launch_dense<16, 3, EPI>(a, p.S, st);
    if constexpr (EPI == EPI_LOGITS) {
      // One plane at 8 fragments: a 3-stage ring is 72 KB, two workgroups
      // per CU, so the 501 column tiles of a 128k vocabulary run in one round
      // (LM head at 96-128 rows 187-196 -> 178-187 us against 4 stages).
      // 12 fragments do not split over 8 waves.
      return launch_dense<8, 3, EPI>(a, p.S, st);
    } else {
      if (p.RT == 12) return launch_dense<12, 3, EPI>(a, p.S, st);
      return launch_dense<8, 4, EPI>(a, p.S, st);
    }
  }
  return launch_stream_plan<EPI, false>(a, p, st);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.R <= 0) return hipSuccess;
  switch (a.epi) {
    case EPI_F32: return launch_epi<EPI_F32>(a, st);
    case EPI_RESID: return launch_epi<EPI_RESID>(a, st);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(a, st);
    default: return launch_epi<EPI_LOGITS>(a, st);
  }
}

}  // namespace cbd

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
// wave-wide weight load is one contiguous 1 KB tile and a wave streams each
// 16-row block front to back -- the DRAM sees long sequential runs instead
// of 16 scattered 64-byte pieces per instruction. Two register stages of
// loads are kept in flight while the previous stage feeds the MFMAs.
//
// The activations are fp32 values carried as two bf16 planes (hi, lo), so
// each weight fragment meets two B operands: acc += W.X_hi, acc += W.X_lo.
// Both products are exact in the fp32 accumulator, and the result is the
// fp32 dot product of W with X to within 2^-17 relative per term. The
// second MFMA costs nothing while the weights stream from HBM (a 16 x 32
// weight tile per 2 x 16 rows of MFMA work leaves the matrix cores idle
// most of the time at these row counts).
//
// A wave owns NT column fragments x RT row fragments. KW waves of a workgroup
// split K and reduce through LDS in fixed wave order; S workgroups along
// grid.y split K further and leave fp32 partials that a second kernel sums in
// fixed split order and passes through the epilogue. Epilogues: fp32 store,
// fp32 residual add (x += acc), SwiGLU over a gate/up pair
// (a = silu(g) * u, stored split), and fp32 logits with per-tile argmax
// partials (lowest id on ties).
#include "common.h"
#include "kernels.h"

namespace cbd {

template <int EPI>
struct EpiTraits {
  static constexpr int NM = EPI == EPI_SWIGLU ? 2 : 1;  // weight matrices
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
    store_split4(a.Yh, a.Yl, at, silu_f(v0[0]) * v1[0], silu_f(v0[1]) * v1[1],
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

template <int RT, int NT, int KW, int EPI>
__global__ __launch_bounds__(64 * KW) void gemm_kernel(GemmArgs a, int kc, int S) {
  constexpr int NM = EpiTraits<EPI>::NM;
  extern __shared__ float lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * (16 * NT);
  const int ks = blockIdx.y;
  const int r0 = blockIdx.z * (16 * RT);
  const int K = a.K, N = a.N, R = a.R;

  const int kw_len = kc / KW;  // a multiple of 64: waves start on tile boundaries
  const int kbeg = ks * kc + wave * kw_len;
  const int kend = min(K, kbeg + kw_len);

  // Weight pointers into the packed layout, at this wave's first tile and
  // this lane's 16 bytes: a wave-wide load reads one whole 1 KB tile. Row
  // blocks past N read block 0 (valid memory; those outputs are never
  // stored). Activation rows past R likewise read row 0.
  const int KT = (K + 31) / 32;
  const uint16_t* wp[NM][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int nb = (n0 >> 4) + nt;
    if (nb * 16 >= N) nb = 0;
    const size_t off = ((size_t)nb * KT + kbeg / 32) * 512 + lane * 8;
    wp[0][nt] = a.W + off;
    if (NM == 2) wp[NM - 1][nt] = a.W2 + off;
  }
  const uint16_t* xp[RT][2];  // hi and lo planes
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = r0 + 16 * rt + lr;
    const size_t off = (size_t)(r < R ? r : 0) * K + kbeg + 8 * lg;
    xp[rt][0] = a.X + off;
    xp[rt][1] = a.Xlo + off;
  }

  floatx4_t acc[NM][NT][RT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[m][nt][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // One stage = ST super-steps of 64 k; two stages in registers, so the
  // loads of stage i+1 are in flight while stage i feeds the MFMAs.
  constexpr int ST = RT * NM <= 1 ? 2 : 1;
  struct Stage {
    uint4 w[ST][NM][NT][2];
    uint4 x[ST][RT][2][2];  // [u][rt][32-k half][hi, lo]
  };
  auto load = [&](Stage& sg, int k) {
#pragma unroll
    for (int u = 0; u < ST; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int off = k + 64 * u + 32 * h;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            sg.w[u][m][nt][h] = load_stream16(wp[m][nt] + (size_t)(off / 32) * 512);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int pl = 0; pl < 2; ++pl)
            sg.x[u][rt][h][pl] = *reinterpret_cast<const uint4*>(xp[rt][pl] + off);
      }
  };
  auto compute = [&](const Stage& sg) {
#pragma unroll
    for (int u = 0; u < ST; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int rt = 0; rt < RT; ++rt)
                acc[m][nt][rt] = mfma16x16x32(as_bf16x8(sg.w[u][m][nt][h]),
                                              as_bf16x8(sg.x[u][rt][h][pl]), acc[m][nt][rt]);
  };

  const int span = kend - kbeg;  // this wave's k count (a multiple of 8, or <= 0)
  const int stride = 64 * ST;
  const int nfull = span > 0 ? span / stride : 0;
  {
    Stage A, B;
    int it = 0;
    if (nfull > 0) load(A, 0);
    for (; it + 2 <= nfull; it += 2) {
      load(B, (it + 1) * stride);
      compute(A);
      if (it + 2 < nfull) load(A, (it + 2) * stride);
      compute(B);
    }
    if (it < nfull) compute(A);
  }
  // Tail: the last < 64*ST k, in 32-k halves predicated per lane group.
  for (int k = nfull * stride; k < span; k += 32) {
    const bool kin = k + 8 * lg < span;
    uint4 w[NM][NT], x[RT][2];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        w[m][nt] = kin ? load_stream16(wp[m][nt] + (size_t)(k / 32) * 512) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int pl = 0; pl < 2; ++pl)
        x[rt][pl] = kin ? *reinterpret_cast<const uint4*>(xp[rt][pl] + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int pl = 0; pl < 2; ++pl)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            acc[m][nt][rt] = mfma16x16x32(as_bf16x8(w[m][nt]), as_bf16x8(x[rt][pl]), acc[m][nt][rt]);
  }

  // Reduce the KW waves' partial sums through LDS, in wave order.
  if (KW > 1) {
    constexpr int TILE = NM * NT * RT * 4;  // floats per lane
    if (wave > 0) {
      float* dst = lds + ((size_t)(wave - 1) * 64 + lane) * TILE;
      int q = 0;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[q++] = acc[m][nt][rt][i];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < KW; ++w) {
      const float* src = lds + ((size_t)(w - 1) * 64 + lane) * TILE;
      int q = 0;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][nt][rt][i] += src[q++];
    }
  }

  store_tile<RT, NT, EPI>(a, acc, r0, n0, ks, S, blockIdx.x);
}

// ------------------------------------------------------- the wide-row path
//
// For 17..64 rows per weight read. A workgroup is NW = 4 waves side by side
// along N (each NT column fragments) over the same K range and all RT row
// fragments, so the activation tile of a 64-k stage (RT x 16 rows x 64 k, hi
// and lo: RT x 4 KB) is fetched once per workgroup into LDS instead of once
// per wave. The LDS tile is kept in MFMA operand order -- block
// (rt, plane, 32-k half) is 64 lanes x 16 bytes -- so each wave reads its B
// operands with one conflict-free 16-byte LDS read per lane.
//
// Each wave streams its weights through a ring of D register stages (64 k
// each), issuing stage c + D - 1 before it computes stage c, so D - 1 stages
// of weight reads are in flight per wave. The activation copy for a stage is
// issued with that stage's weights (the vector-memory counter retires loads
// in order, so a later-issued activation load would hold back the wait for
// the weights behind it). Per stage: copy the arrived activation rows into
// LDS buffer c % 2, barrier, then the MFMAs of stage c.
#define WIDE_NW 4

template <int RT, int NT, int D, int EPI>
__global__ __launch_bounds__(64 * WIDE_NW) void gemm_wide_kernel(GemmArgs a, int kc, int S) {
  constexpr int NM = EpiTraits<EPI>::NM;
  constexpr int BLK = RT * 4;  // LDS blocks per stage: (rt, plane, half)
  __shared__ uint4 xs[2][BLK * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int tile = blockIdx.x * WIDE_NW + wave;  // this wave's column tile
  const int n0 = tile * (16 * NT);
  const int ks = blockIdx.y;
  const int r0 = blockIdx.z * (16 * RT);
  const int K = a.K, N = a.N, R = a.R;
  const int kbeg = ks * kc;                 // a multiple of 64
  const int kend = min(K, kbeg + kc);
  const int nst = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;

  const int KT = (K + 31) / 32;
  const uint16_t* wp[NM][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int nb = (n0 >> 4) + nt;
    if (nb * 16 >= N) nb = 0;  // past N: read block 0, never stored
    const size_t off = ((size_t)nb * KT + kbeg / 32) * 512 + lane * 8;
    wp[0][nt] = a.W + off;
    if (NM == 2) wp[NM - 1][nt] = a.W2 + off;
  }
  // This thread's share of the activation copy: block b = wave + 4 i of
  // every stage, lane `lane` of it. Rows past R read row 0 and are zeroed
  // when written to LDS.
  const uint16_t* xsrc[RT];
  bool xrow[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int b = wave + WIDE_NW * i;
    const int rt = b >> 2, pl = (b >> 1) & 1;
    const int r = r0 + 16 * rt + lr;
    xrow[i] = r < R;
    xsrc[i] = (pl ? a.Xlo : a.X) + (size_t)(xrow[i] ? r : 0) * K;
  }

  floatx4_t acc[NM][NT][RT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[m][nt][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // The loads carry no conditions (a condition would become a branch, and
  // the counter waits at its join drain every outstanding load): weight
  // tiles are clamped into the matrix and activation pieces into the row,
  // and pieces at or beyond kend are zeroed when the activations are
  // written to LDS -- weights there then meet zeros.
  uint4 w[D][NM][NT][2];
  uint4 xc[D][RT];
  auto load = [&](int j, int c) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = min(kbeg / 32 + 2 * c + h, KT - 1) - kbeg / 32;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          w[j][m][nt][h] = load_stream16(wp[m][nt] + (size_t)t * 512);
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int b = wave + WIDE_NW * i;
      const int k = min(kbeg + 64 * c + 32 * (b & 1) + 8 * lg, K - 8);
      xc[j][i] = *reinterpret_cast<const uint4*>(xsrc[i] + k);
    }
  };
  auto stage = [&](int j, int c) {
    uint4* buf = xs[c & 1];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int b = wave + WIDE_NW * i;
      const bool ok = xrow[i] && kbeg + 64 * c + 32 * (b & 1) + 8 * lg < kend;
      buf[b * 64 + lane] = ok ? xc[j][i] : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 xf[RT][2];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) xf[rt][pl] = buf[((rt * 2 + pl) * 2 + h) * 64 + lane];
#pragma unroll
      for (int pl = 0; pl < 2; ++pl)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              acc[m][nt][rt] = mfma16x16x32(as_bf16x8(w[j][m][nt][h]), as_bf16x8(xf[rt][pl]),
                                            acc[m][nt][rt]);
    }
  };

  if (nst > 0) {
    // Stage s lives in ring slot s % D; the loads of stage c + D - 1 are
    // issued before stage c is computed (clamped to the last stage near the
    // end: those repeats are cache hits and never computed).
#pragma unroll
    for (int j = 0; j < D - 1; ++j) load(j, min(j, nst - 1));
    const int groups = nst / D;
    for (int g = 0; g < groups; ++g) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int c = g * D + j;
        load((j + D - 1) % D, min(c + D - 1, nst - 1));
        stage(j, c);
      }
    }
    const int rest = nst - groups * D;  // < D, already loaded in slots 0..rest-1
#pragma unroll
    for (int j = 0; j < D - 1; ++j)
      if (j < rest) stage(j, groups * D + j);
  }
  store_tile<RT, NT, EPI>(a, acc, r0, n0, ks, S, tile);
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
  return (size_t)((N + 15) / 16) * (size_t)((K + 31) / 32) * 512;
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
  reinterpret_cast<uint4*>(out)[i] = v;
}

hipError_t launch_pack(const uint16_t* W, int32_t N, int32_t K, uint16_t* out, hipStream_t st) {
  const size_t n16 = packed_elems(N, K) / 8;
  pack_kernel<<<(unsigned)((n16 + 255) / 256), 256, 0, st>>>(W, N, K, out, n16);
  return hipGetLastError();
}

struct Shape {
  int RT, NT;
};

// Up to 16 rows: the per-wave kernel with one row fragment and four column
// fragments (the waves of a workgroup split K). Beyond 16 rows: the wide-row
// kernel, 64 rows (four row fragments; two up to 32 rows) per weight read,
// and row groups past 64 re-read the weights -- the repeats are served by
// the Infinity Cache for matrices up to its size.
static bool use_wide(int R) { return R > 16; }

static Shape wide_shape(int R, int NM) {
  return {R <= 32 ? 2 : 4, NM == 2 ? 2 : 4};
}

int32_t gemm_amax_tiles(int32_t R, int32_t N, int32_t K) {
  (void)K;
  if (use_wide(R)) {
    const int cols = 16 * wide_shape(R, 1).NT;
    return (N + cols * WIDE_NW - 1) / (cols * WIDE_NW) * WIDE_NW;
  }
  return (N + 63) / 64;
}

template <int EPI>
static hipError_t launch_reduce(const GemmArgs& a, int S, hipStream_t st) {
  const size_t threads = (size_t)a.R * (a.N / 4);
  gemm_reduce_kernel<EPI><<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(a, S);
  return hipGetLastError();
}

template <int RT, int NT, int EPI>
static hipError_t launch_shape(const GemmArgs& a, hipStream_t st) {
  constexpr int NM = EpiTraits<EPI>::NM;
  const int n_tiles = (a.N + 16 * NT - 1) / (16 * NT);
  const int r_groups = (a.R + 16 * RT - 1) / (16 * RT);
  const int base = n_tiles * r_groups;
  // Enough waves to cover the chip: when the column tiles alone give fewer
  // than ~1024 waves, split K inside the workgroup (up to 4 waves, >= 256 k
  // each) and then across workgroups (>= 512 k each) when the partials fit.
  // LDS for the in-workgroup reduction stays within 64 KB.
  const size_t lds_per_wave = (size_t)64 * NM * NT * RT * 4 * sizeof(float);
  int KW = 1;
  while (base * KW < 1024 && KW < 4 && a.K / (KW * 2) >= 256 &&
         (size_t)(KW * 2 - 1) * lds_per_wave <= 65536)
    KW *= 2;
  int S = 1;
  if (EPI != EPI_LOGITS) {
    while (base * KW * S < 2048 && a.K / (S * 2) >= 512 &&
           (size_t)(S * 2) * NM * a.R * a.N <= a.partials_cap)
      S *= 2;
  }
  // Waves start on 64-k (two-tile) boundaries.
  int kc = (a.K + S - 1) / S;
  kc = (kc + 64 * KW - 1) / (64 * KW) * (64 * KW);
  S = (a.K + kc - 1) / kc;
  dim3 grid(n_tiles, S, r_groups);
  size_t lds = KW > 1 ? (size_t)(KW - 1) * 64 * NM * NT * RT * 4 * sizeof(float) : 0;
  switch (KW) {
    case 1: gemm_kernel<RT, NT, 1, EPI><<<grid, 64, lds, st>>>(a, kc, S); break;
    case 2: gemm_kernel<RT, NT, 2, EPI><<<grid, 128, lds, st>>>(a, kc, S); break;
    default: gemm_kernel<RT, NT, 4, EPI><<<grid, 256, lds, st>>>(a, kc, S); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  return launch_reduce<EPI>(a, S, st);
}

// The wide-row kernel over (column groups of 4 waves) x (K splits) x (row
// groups). A K split is used only while the column groups alone leave the
// chip short of workgroups and each split keeps >= 1024 k; the logits never
// split (their argmax is fused).
template <int RT, int NT, int D, int EPI>
static hipError_t launch_wide(const GemmArgs& a, int S_force, hipStream_t st) {
  constexpr int NM = EpiTraits<EPI>::NM;
  const int cols = 16 * NT * WIDE_NW;
  const int n_groups = (a.N + cols - 1) / cols;
  const int r_groups = (a.R + 16 * RT - 1) / (16 * RT);
  int S = 1;
  if (S_force > 0) {
    S = S_force;
  } else if (EPI != EPI_LOGITS) {
    while (n_groups * r_groups * S < 512 && a.K / (S * 2) >= 1024 &&
           (size_t)(S * 2) * NM * a.R * a.N <= a.partials_cap)
      S *= 2;
  }
  if (EPI == EPI_LOGITS) S = 1;
  int kc = (a.K + S - 1) / S;
  kc = (kc + 63) / 64 * 64;
  S = (a.K + kc - 1) / kc;
  if (S > 1 && (size_t)S * NM * a.R * a.N > a.partials_cap) return hipErrorInvalidValue;
  dim3 grid(n_groups, S, r_groups);
  gemm_wide_kernel<RT, NT, D, EPI><<<grid, 64 * WIDE_NW, 0, st>>>(a, kc, S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  return launch_reduce<EPI>(a, S, st);
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& a, hipStream_t st) {
  if (!use_wide(a.R)) return launch_shape<1, 4, EPI>(a, st);
  constexpr int NT = EpiTraits<EPI>::NM == 2 ? 2 : 4;
  if (a.R <= 32) return launch_wide<2, NT, 4, EPI>(a, 0, st);
  return launch_wide<4, NT, 4, EPI>(a, 0, st);
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

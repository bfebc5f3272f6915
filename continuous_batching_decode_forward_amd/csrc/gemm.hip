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

  // Lane l holds columns n0 + 16 nt + 4 lg + (0..3) of row r0 + 16 rt + lr.
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
        a.amax_val[(size_t)r * a.amax_stride + blockIdx.x] = best;
        a.amax_idx[(size_t)r * a.amax_stride + blockIdx.x] = bidx;
      }
    }
  }
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

// Tile shape by rows. Up to 16 rows: one row fragment, four column
// fragments. Beyond that up to 64 rows share one weight read per wave (four
// row fragments; two for the dual-matrix SwiGLU, whose accumulators double),
// and row groups past 64 re-read the weights -- the repeats are served by
// the Infinity Cache for matrices up to its size.
static Shape pick_shape(int R, int NM) {
  if (R <= 16) return {1, 4};
  if (NM == 2) return {2, 4};
  return {4, 4};
}

int32_t gemm_amax_tiles(int32_t R, int32_t N, int32_t K) {
  (void)K;
  Shape s = pick_shape(R, 1);
  return (N + 16 * s.NT - 1) / (16 * s.NT);
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
  const size_t threads = (size_t)a.R * (a.N / 4);
  gemm_reduce_kernel<EPI><<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(a, S);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& a, hipStream_t st) {
  const Shape s = pick_shape(a.R, EpiTraits<EPI>::NM);
  if (s.RT == 1) return launch_shape<1, 4, EPI>(a, st);
  if constexpr (EpiTraits<EPI>::NM == 2) return launch_shape<2, 4, EPI>(a, st);
  else return launch_shape<4, 4, EPI>(a, st);
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

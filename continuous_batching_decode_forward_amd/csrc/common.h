// common.h -- device helpers shared by the gfx950 kernels of the step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define CBD_WAVE 64

// bf16 <-> fp32. bf16 is the top half of a binary32; the narrowing rounds to
// nearest even (NaN kept quiet).
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ float round_bf(float f) { return bf2f(f2bf(f)); }

// fp32 -> OCP E4M3 code (the 8-bit cache format): round to nearest even,
// magnitudes beyond 448 saturated to 448, NaN to 0x7f (the conversion
// instruction alone turns out-of-range values into NaN, hence the clamp).
__device__ __forceinline__ uint8_t f2e4m3(float f) {
  if (f != f) return 0x7f;
  f = fminf(fmaxf(f, -448.0f), 448.0f);
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(f, 0.0f, 0, false) & 0xff);
}

// Eight E4M3 codes (a uint2, code i in byte i) -> eight bf16 values in MFMA
// operand order (a uint4, value i in half-word i). Every E4M3 value is
// exactly a bf16 value.
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, 1.0f, true);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, 1.0f, false);
  const bf16x2_t e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, 1.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, d), __builtin_bit_cast(uint32_t, e));
}

// Two bf16 packed in a uint32 (low half first).
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// An fp32 activation travels to the MFMAs as two bf16 terms: hi = bf16(v)
// and lo = bf16(v - hi). v - hi is exact in fp32, so hi + lo equals v to
// within 2^-17 |v|, and a product with a bf16 weight is the sum of two bf16
// products, each exact in the fp32 accumulator.
__device__ __forceinline__ void split_bf(float v, bf16_t& hi, bf16_t& lo) {
  hi = f2bf(v);
  lo = f2bf(v - bf2f(hi));
}

// Split activations that feed a contraction are kept in operand tiles: each
// plane [rows][w] is cut into 1 KB tiles of 16 rows x 32 columns, tile
// (f, kb) at element (f * KB + kb) * 512 with KB = ceil(w / 32), and inside
// a tile columns 32 kb + 8 j .. + 7 of row 16 f + i sit at (16 j + i) * 8.
// A 64-lane copy of 16 bytes per lane then moves one whole tile, contiguous,
// into exactly the order the MFMA B operand is read in (lane 16 j + i: row
// i, columns 8 j ..). Row-major rows instead make every copy touch 16 rows
// of 64 bytes, which the vector memory path serves at about a third of the
// rate of a contiguous kilobyte.
__host__ __device__ __forceinline__ size_t tile_at(int r, int k, int KB) {
  return (((size_t)(r >> 4) * KB + (k >> 5)) * 64 + ((k >> 3) & 3) * 16 + (r & 15)) * 8 + (k & 7);
}

// Split four consecutive values and store them to the hi and lo planes
// (8-byte stores; `at` must be a multiple of 4: in operand tiles the four
// columns 4 m .. 4 m + 3 of a row are contiguous).
__device__ __forceinline__ void store_split4(uint16_t* hi, uint16_t* lo, size_t at, float a,
                                             float b, float c, float d) {
  bf16_t h[4], l[4];
  split_bf(a, h[0], l[0]);
  split_bf(b, h[1], l[1]);
  split_bf(c, h[2], l[2]);
  split_bf(d, h[3], l[3]);
  *reinterpret_cast<uint2*>(hi + at) =
      make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
  *reinterpret_cast<uint2*>(lo + at) =
      make_uint2((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16));
}

// Split eight consecutive values and store them to the hi and lo planes
// (16-byte stores: one whole 8-column run of an operand tile per plane).
__device__ __forceinline__ void store_split8(uint16_t* hi, uint16_t* lo, size_t at, const float* v) {
  bf16_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) split_bf(v[e], h[e], l[e]);
  *reinterpret_cast<uint4*>(hi + at) =
      make_uint4((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16),
                 (uint32_t)h[4] | ((uint32_t)h[5] << 16), (uint32_t)h[6] | ((uint32_t)h[7] << 16));
  *reinterpret_cast<uint4*>(lo + at) =
      make_uint4((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16),
                 (uint32_t)l[4] | ((uint32_t)l[5] << 16), (uint32_t)l[6] | ((uint32_t)l[7] << 16));
}

// 16-byte load that asks the memory system not to keep the line (weights
// are streamed once per step).
__device__ __forceinline__ uint4 load_stream16(const uint16_t* p) {
  u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The same for 8 bytes.
__device__ __forceinline__ uint2 load_stream8(const uint8_t* p) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// 16 bytes per lane from global memory straight into LDS: lane i of the
// wave writes lds_base + 16 i (lds_base must be the same for the whole
// wave). Counts as a vector-memory load for s_waitcnt vmcnt. Issued as
// inline assembly on purpose: the compiler would otherwise make every later
// LDS access wait for all outstanding loads (it cannot tell which LDS
// bytes the copy writes), so the caller orders the copy itself with
// wait_vmem and a barrier.
__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(size_t)(__attribute__((address_space(3))) void*)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
#endif
}

// The same copy with the non-temporal cache policy: for data read once
// (a weight stream), so that it does not push reused data out of L2.
__device__ __forceinline__ void copy16_to_lds_nt(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(size_t)(__attribute__((address_space(3))) void*)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
#endif
}

// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
#if defined(__HIP_DEVICE_COMPILE__)
  // s_waitcnt simm16: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
#endif
}

__device__ __forceinline__ floatx4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Wave-wide reductions over 64 lanes (xor butterfly, fixed order).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, CBD_WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, CBD_WAVE));
  return v;
}

// Device status bits (same values as CBD_STATUS_* in cbd.h).
#define ST_BAD_BLOCK 0x1u
#define ST_BAD_TOKEN 0x2u
#define ST_BAD_SLOT 0x4u
#define ST_BAD_SHAPE 0x8u

__device__ __forceinline__ void raise_status(uint32_t* status, uint32_t bit) {
  atomicOr(status, bit);
}

// common.h -- device types and the exact dequantization routines shared by
// every kernel of the library (gfx950 / CDNA4, wave64).
//
// Dequantization, INT4 ([P3] "LLM 量化技术详解" §2.1 asymmetric with zero point,
// §2.2 group-wise): w = round16(fp32(q - z) * fp32(s)).  (q - z) is a 5-bit
// integer and s has an 11-bit significand, so the product is exact in fp32 and
// the only rounding is the final one to fp16/bf16 (nearest-even).
//
//  * fp16: the code is turned into the fp16 value 1024 + q by OR-ing it into
//    the significand of 1024.0 (bits 0x6400 | q); subtracting 1024 + z is then
//    exact, and one packed fp16 multiply by s rounds the exact product once.
//  * bf16: there is no packed bf16 add on gfx950, so each code goes to fp32
//    (v_cvt_f32_ubyte*), (q - z) * s is formed exactly in fp32 and
//    v_cvt_pk_bf16_f32 rounds two results at a time.
//
// Repacked word format: a 32-bit word holds the 8 codes of one column for 8
// consecutive (permuted) input columns e = 0..7 at nibble slot
// (e >> 1) + 4 * (e & 1).  Extracting nibble pairs (r, r + 4) therefore yields
// the element pairs (2r, 2r + 1), i.e. the natural order of the 8-element MFMA
// operand of v_mfma_f32_16x16x32_{f16,bf16}.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

enum { DT_F16 = 0, DT_BF16 = 1 };

// 8-element MFMA operand type for a dtype.
template <int DT> struct Op;
template <> struct Op<DT_F16> { typedef half8_t vec; };
template <> struct Op<DT_BF16> { typedef bf16x8_t vec; };

template <int DT>
__device__ __forceinline__ float4_t mfma16x16x32(const typename Op<DT>::vec& a,
                                                 const typename Op<DT>::vec& b, float4_t c);
template <>
__device__ __forceinline__ float4_t mfma16x16x32<DT_F16>(const half8_t& a, const half8_t& b,
                                                         float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ float4_t mfma16x16x32<DT_BF16>(const bf16x8_t& a, const bf16x8_t& b,
                                                          float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Per-(column, group) quantization parameters in the form each dtype's
// dequant routine consumes.
template <int DT> struct QParam;
template <> struct QParam<DT_F16> {
  half2_t hz;  // (1024 + z) in both halves
  half2_t s2;  // s in both halves
  __device__ __forceinline__ void set(uint32_t scale_bits, uint32_t z) {
    uint32_t hzb = 0x6400u | z;
    hz = __builtin_bit_cast(half2_t, hzb | (hzb << 16));
    s2 = __builtin_bit_cast(half2_t, scale_bits | (scale_bits << 16));
  }
};
template <> struct QParam<DT_BF16> {
  float zf, sf;
  __device__ __forceinline__ void set(uint32_t scale_bits, uint32_t z) {
    zf = (float)z;
    sf = (float)__builtin_bit_cast(_Float16, (uint16_t)scale_bits);
  }
};

// Exact dequantization of one repacked word into an 8-element MFMA operand.
__device__ __forceinline__ half8_t dequant_word(uint32_t w, const QParam<DT_F16>& p) {
  half2_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t t = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;  // (1024+q_2i, 1024+q_2i+1)
    r[i] = (__builtin_bit_cast(half2_t, t) - p.hz) * p.s2;       // exact sub, one rounding
  }
  return half8_t{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
}

__device__ __forceinline__ bf16x8_t dequant_word(uint32_t w, const QParam<DT_BF16>& p) {
  // nibble slot s holds element e with s = (e >> 1) + 4 (e & 1):
  //   lo = w & 0x0F0F0F0F  bytes = slots 0, 2, 4, 6 = elements 0, 4, 1, 5
  //   hi = (w >> 4) & ...  bytes = slots 1, 3, 5, 7 = elements 2, 6, 3, 7
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  float f[8];
  f[0] = (float)(lo & 0xFFu);
  f[1] = (float)((lo >> 16) & 0xFFu);
  f[2] = (float)(hi & 0xFFu);
  f[3] = (float)((hi >> 16) & 0xFFu);
  f[4] = (float)((lo >> 8) & 0xFFu);
  f[5] = (float)((lo >> 24) & 0xFFu);
  f[6] = (float)((hi >> 8) & 0xFFu);
  f[7] = (float)((hi >> 24) & 0xFFu);
  bf16x8_t out;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (__bf16)((f[e] - p.zf) * p.sf);
  return out;
}

// Round an fp32 value to the 16-bit output type and return its bits.
template <int DT> __device__ __forceinline__ uint16_t round16(float v);
template <> __device__ __forceinline__ uint16_t round16<DT_F16>(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}
template <> __device__ __forceinline__ uint16_t round16<DT_BF16>(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Exact widening of 16-bit input bits to fp32.
template <int DT> __device__ __forceinline__ float widen16(uint16_t b);
template <> __device__ __forceinline__ float widen16<DT_F16>(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
template <> __device__ __forceinline__ float widen16<DT_BF16>(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace w4a16

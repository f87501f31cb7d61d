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
//  * bf16: there is no packed bf16 add on gfx950; (q - z) is formed exactly in
//    fp16 as above, widened, multiplied by s in fp32 (exact) and
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
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

enum { DT_F16 = 0, DT_BF16 = 1 };

// 0x64006400 (two fp16 1024.0) held in a VGPR: a literal cannot be an operand
// of the 3-operand v_and_or_b32 on gfx9, so without this the compiler splits
// the nibble insert into v_and_b32 + v_or_b32.
__device__ __forceinline__ uint32_t opaque_magic() {
  uint32_t m;
  asm("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

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
  uint32_t magic;  // 0x64006400 in a register, so the nibble insert is one v_and_or_b32
  // 4-bit words (HI4): the codes of the odd element pairs are inserted at
  // bits 4-7 of 0x5400, which is 64 + q exactly (see dequant_word4_f16)
  half2_t hz_hi;      // (64 + z) in both halves
  uint32_t magic_hi;  // 0x54005400 in a register
  template <bool HI4 = false>
  __device__ __forceinline__ void set(uint32_t scale_bits, uint32_t z) {
    magic = opaque_magic();
    uint32_t hzb = 0x6400u | z;
    hz = __builtin_bit_cast(half2_t, hzb | (hzb << 16));
    s2 = __builtin_bit_cast(half2_t, scale_bits | (scale_bits << 16));
    if constexpr (HI4) {
      asm("v_mov_b32 %0, 0x54005400" : "=v"(magic_hi));
      const uint32_t h = 0x5400u | (z << 4);
      hz_hi = __builtin_bit_cast(half2_t, h | (h << 16));
    }
  }
};
template <> struct QParam<DT_BF16> {
  half2_t hz;  // (1024 + z) in both halves
  float sf;    // s
  float nz;    // -0.0, opaque to the compiler so that the fma below stays an fma
  float nc;    // -(1024 + z) s, exact in fp32 (an 11-bit integer times an 11-bit significand)
  uint32_t magic;  // 0x64006400 in a register, so the nibble insert is one v_and_or_b32
  template <bool HI4 = false>
  __device__ __forceinline__ void set(uint32_t scale_bits, uint32_t z) {
    magic = opaque_magic();
    uint32_t hzb = 0x6400u | z;
    hz = __builtin_bit_cast(half2_t, hzb | (hzb << 16));
    sf = (float)__builtin_bit_cast(_Float16, (uint16_t)scale_bits);
    nc = -(float)(1024u + z) * sf;
    uint32_t m;
    asm("v_mov_b32 %0, 0x80000000" : "=v"(m));
    nz = __builtin_bit_cast(float, m);
  }
};

// Exact dequantization of a pair of codes held in the low bits of the two
// 16-bit halves of f (codes < 1024): 0x6400 | q is the fp16 value 1024 + q,
// so (1024 + q) - (1024 + z) = q - z exactly, then one rounding of (q - z) s.
// Returned as two packed 16-bit values.
//
// ZS (zero sign): the bf16 form below keeps the IEEE sign of an exactly-zero
// product ((q - z) s = -0 when q == z and s is negative or -0).  The GEMM
// kernels use ZS = false, a cheaper form whose only difference is +0 there:
// their fp32 accumulators start at +0, and a sum of signed zeros with a +0
// term is +0, so no output can tell the two apart.  The dequant export, which
// is compared bit for bit, uses ZS = true.
template <bool ZS = true>
__device__ __forceinline__ uint32_t dequant_fields(uint32_t f, const QParam<DT_F16>& p) {
  const uint32_t t = f | p.magic;                                     // (1024+q_lo, 1024+q_hi)
  const half2_t r = (__builtin_bit_cast(half2_t, t) - p.hz) * p.s2;  // exact sub, one rounding
  return __builtin_bit_cast(uint32_t, r);
}

template <bool ZS = true>
__device__ __forceinline__ uint32_t dequant_fields(uint32_t f, const QParam<DT_BF16>& p) {
  const uint32_t t = f | p.magic;
  if constexpr (ZS) {
    // (q - z) exactly in fp16 as on the fp16 path, then the exact fp32
    // product with s as fma(q - z, s, -0) (v_fma_mix widens the fp16 half in
    // place; adding -0 keeps every signed zero of the plain product) and the
    // one rounding to bf16.
    const half2_t d = __builtin_bit_cast(half2_t, t) - p.hz;
    const bf16x2_t r = {(__bf16)__builtin_fmaf((float)d[0], p.sf, p.nz),
                        (__bf16)__builtin_fmaf((float)d[1], p.sf, p.nz)};
    return __builtin_bit_cast(uint32_t, r);
  } else {
    // (1024 + q) s - (1024 + z) s in one fma: both products are exact in fp32
    // and so is their difference (q - z) s, which is then rounded once to bf16
    const half2_t th = __builtin_bit_cast(half2_t, t);
    const bf16x2_t r = {(__bf16)__builtin_fmaf((float)th[0], p.sf, p.nc),
                        (__bf16)__builtin_fmaf((float)th[1], p.sf, p.nc)};
    return __builtin_bit_cast(uint32_t, r);
  }
}

// Element pair i (elements 2i, 2i + 1, nibble slots i and i + 4) of one
// repacked 4-bit word.
template <bool ZS = true, class QP>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t w, int i, const QP& p) {
  return dequant_fields<ZS>((w >> (4 * i)) & 0x000F000Fu, p);
}

// The codes alone as MFMA operand values, for kernels that apply the scale and
// zero after summing over a group: 0x6400 | q is the fp16 value 1024 + q and
// 0x4300 | q the bf16 value 128 + q (q < 128), both exact: o + q with o = 1024
// or 128.
//
// Such a kernel forms, per group and output, s * (T - Z) with
// T = sum_k x_k (o + q_k) and Z = sum_k x_k (o + z), both from MFMAs over the
// same activation operand in the same accumulation order: Z uses the zero
// operand below (o + z in all 8 elements) in place of the codes.  Where every
// code of the group equals its zero the two MFMAs see identical inputs, so
// T - Z is exactly 0 and the output is exactly 0, as with the per-weight
// dequant (q - z) s = 0.
template <int DT> struct RawQ {
  uint32_t magic;     // in a register, so the insert is one v_and_or_b32
  uint32_t magic_hi;  // fp16 4-bit words: 0x54005400 (odd element pairs, 64 + q)
  __device__ __forceinline__ RawQ() {
    magic = DT == DT_F16 ? 0x64006400u : 0x43004300u;
    magic_hi = 0x54005400u;
    asm("" : "+v"(magic));
    if constexpr (DT == DT_F16) asm("" : "+v"(magic_hi));
  }
  // The zero operand: o + z in every element of an MFMA operand, with o the
  // offset of each element's code form (z < 1024 in fp16, < 128 in bf16; for
  // 4-bit codes in fp16 the odd element pairs carry 64 + z, as their codes
  // carry 64 + q).
  // (The fields of z land on zero bits of the offsets, so the sums below are
  // the bitwise ors, and each is one multiply-add.)
  template <int BITS>
  __device__ __forceinline__ typename Op<DT>::vec zero_operand(uint32_t z) const {
    const uint32_t v = magic + z * 0x00010001u;
    if constexpr (DT == DT_F16 && BITS == 4) {
      const uint32_t h = magic_hi + z * 0x00100010u;
      return __builtin_bit_cast(typename Op<DT>::vec, u32x4_t{v, h, v, h});
    } else {
      return __builtin_bit_cast(typename Op<DT>::vec, u32x4_t{v, v, v, v});
    }
  }
};
template <bool ZS = true, int DT>
__device__ __forceinline__ uint32_t dequant_fields(uint32_t f, const RawQ<DT>& p) {
  return f | p.magic;
}

// One repacked 4-bit word into an fp16 MFMA operand with a single shift.  The
// pairs (0, 1) and (4, 5) have their codes at bits 0-3 / 16-19 of w and of
// w >> 8, the pairs (2, 3) and (6, 7) at bits 4-7 / 20-23: 0x6400 | q is the
// fp16 value 1024 + q, and 0x5400 | (q << 4) is 64 + q exactly (the fp16 ulp
// at 64 is 1/16), so every code is inserted where it lies.  With a QParam the
// dequant then subtracts 1024 + z or 64 + z (exact) and multiplies by s (one
// rounding): the same value as the routine above.  With a RawQ the operand
// holds the codes alone, o + q with o = 1024 or 64 by element, and the zero
// operand carries the same offsets.
__device__ __forceinline__ uint32_t f16_hi_fields(uint32_t f, const QParam<DT_F16>& p) {
  const half2_t r = (__builtin_bit_cast(half2_t, f | p.magic_hi) - p.hz_hi) * p.s2;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t f16_hi_fields(uint32_t f, const RawQ<DT_F16>& p) {
  return f | p.magic_hi;
}
template <bool ZS, class QP>
__device__ __forceinline__ half8_t dequant_word4_f16(uint32_t w, const QP& p) {
  const uint32_t t = w >> 8;
  const u32x4_t r = {dequant_fields<ZS>(w & 0x000F000Fu, p), f16_hi_fields(w & 0x00F000F0u, p),
                     dequant_fields<ZS>(t & 0x000F000Fu, p), f16_hi_fields(t & 0x00F000F0u, p)};
  return __builtin_bit_cast(half8_t, r);
}

// Exact dequantization of one repacked 4-bit word into an 8-element MFMA operand
// (with a RawQ: the codes alone).
template <int DT, bool ZS = true, class QP>
__device__ __forceinline__ typename Op<DT>::vec dequant_word(uint32_t w, const QP& p) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = dequant_pair<ZS>(w, i, p);
  return __builtin_bit_cast(typename Op<DT>::vec, r);
}

// NF4 operand of one 32-bit code word (element e in nibble e): w = round16(L[c]
// a') with the fp32 product.  The levels come from a 256-entry table of pairs
// in LDS: entry b (8 bytes) holds {L[b & 15], L[b >> 4]}, the levels of the two
// codes one byte of w carries (low nibble: element 2 j, high nibble: element
// 2 j + 1), so one 8-byte lookup serves two codes and its address is the byte
// shifted by 3 (one shift with a byte-select operand).
template <int DT>
__device__ __forceinline__ typename Op<DT>::vec nf4_pair_operand(uint32_t w, const float2* lut2,
                                                                float a) {
  typename Op<DT>::vec v;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float2 l = lut2[(w >> (8 * j)) & 0xFFu];
    const float f0 = l.x * a, f1 = l.y * a;
    if constexpr (DT == DT_F16) {
      v[2 * j] = (_Float16)f0;
      v[2 * j + 1] = (_Float16)f1;
    } else {
      v[2 * j] = (__bf16)f0;
      v[2 * j + 1] = (__bf16)f1;
    }
  }
  return v;
}

// ---- b-bit integer codes.  One lane's codes of one K tile (32 codes: the 8
// inputs of each of the 4 MFMA steps j) in the repacked form of each width:
//  * 4 bits: 4 dwords, dword j = step j, nibble slot (e >> 1) + 4 (e & 1).
//  * 8 bits: 8 dwords (two 16-byte halves, half j >> 1); step j is dwords
//    2 (j & 1) and 2 (j & 1) + 1 of its half, each holding elements
//    [e0, e2, e1, e3] of its 4 so that (d >> 8 r) & 0x00FF00FF is a pair.
//  * 3 bits: 3 dwords; the low 2 bits of code (j, e) at bit 16 (e & 1) +
//    2 (4 (j & 1) + (e >> 1)) of dword j >> 1, its high bit at bit
//    16 (e & 1) + 4 j + (e >> 1) of dword 2.
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
template <int BITS> struct Codes;
template <> struct Codes<4> { u32x4_t w; };
template <> struct Codes<3> { u32x3_t w; };
template <> struct Codes<8> { u32x4_t lo, hi; };

// Width of a repacked zero field, and the XOR that turns the zero fields a
// symmetric weight reads as 0 into its implicit zero 2^(b-1).
__host__ __device__ constexpr int zero_field_bits(int bits) { return bits == 8 ? 8 : 4; }
__host__ __device__ constexpr uint32_t sym_zero_xor(int bits) {
  return bits == 8 ? 0x80808080u : bits == 4 ? 0x88888888u : 0x44444444u;
}

// The 8-element B operand of MFMA step j (0..3) from a lane's codes (p a
// QParam, or a RawQ for the codes alone).
template <int DT, bool ZS = true, class QP>
__device__ __forceinline__ typename Op<DT>::vec dequant_step(const Codes<4>& c, int j,
                                                             const QP& p) {
  if constexpr (DT == DT_F16) return dequant_word4_f16<ZS>(c.w[j], p);
  else return dequant_word<DT, ZS>(c.w[j], p);
}
template <int DT, bool ZS = true, class QP>
__device__ __forceinline__ typename Op<DT>::vec dequant_step(const Codes<8>& c, int j,
                                                             const QP& p) {
  const u32x4_t h = (j >> 1) ? c.hi : c.lo;
  const uint32_t a = h[2 * (j & 1)], b = h[2 * (j & 1) + 1];
  u32x4_t r;
  r[0] = dequant_fields<ZS>(a & 0x00FF00FFu, p);
  r[1] = dequant_fields<ZS>((a >> 8) & 0x00FF00FFu, p);
  r[2] = dequant_fields<ZS>(b & 0x00FF00FFu, p);
  r[3] = dequant_fields<ZS>((b >> 8) & 0x00FF00FFu, p);
  return __builtin_bit_cast(typename Op<DT>::vec, r);
}
template <int DT, bool ZS = true, class QP>
__device__ __forceinline__ typename Op<DT>::vec dequant_step(const Codes<3>& c, int j,
                                                             const QP& p) {
  const uint32_t lo = c.w[j >> 1], hi = c.w[2];
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t f = ((lo >> (8 * (j & 1) + 2 * i)) & 0x00030003u) |
                       (((hi >> (4 * j + i)) & 0x00010001u) << 2);
    r[i] = dequant_fields<ZS>(f, p);
  }
  return __builtin_bit_cast(typename Op<DT>::vec, r);
}

// AWQ input scaling of 16-bit activations: x / s as the fp32 product of x
// with the fp32 reciprocal of s (v_rcp_f32, within 1 ulp), rounded once to
// the activation type.  Shared by the decode kernel's staged rows and the
// activation preparation pass, so both produce the same operand bits.
template <int DT>
__device__ __forceinline__ float f16bits_to_f32(uint16_t v) {
  if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, v);
  else return __builtin_bit_cast(float, (uint32_t)v << 16);
}
template <int DT>
__device__ __forceinline__ float recip_scale(uint16_t s) {
  return __builtin_amdgcn_rcpf(f16bits_to_f32<DT>(s));
}
template <int DT>
__device__ __forceinline__ uint16_t mul_round16(uint16_t x, float r) {
  const float f = f16bits_to_f32<DT>(x) * r;
  if constexpr (DT == DT_F16) return __builtin_bit_cast(uint16_t, (_Float16)f);
  else return __builtin_bit_cast(uint16_t, (__bf16)f);
}
template <int DT>
__device__ __forceinline__ uint16_t div_scale1(uint16_t x, uint16_t s) {
  return mul_round16<DT>(x, recip_scale<DT>(s));
}

// ---- raw buffer loads (gfx9-family descriptors).  A load whose per-lane
// offset is at or past the descriptor's byte range returns 0, which is how
// kernels read rows past M, codes past a tail and padding without branches;
// every kernel keeps the in-range part of an address in the per-lane offset
// and only a wave-uniform, in-range tile step in the scalar offset.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;
// A per-lane offset past every descriptor's range.
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
__device__ __forceinline__ u32x4_t bld128(rsrc_t r, uint32_t voff, int soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x3_t bld96(rsrc_t r, uint32_t voff, int soff) {
  return __builtin_bit_cast(u32x3_t, __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2_t bld64(rsrc_t r, uint32_t voff, int soff) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t bld32(rsrc_t r, uint32_t voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bld16(rsrc_t r, uint32_t voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
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

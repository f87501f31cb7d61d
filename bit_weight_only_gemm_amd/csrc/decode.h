// decode.h -- the skinny-M (decode) fused dequantize-and-multiply kernel
// templates, shared by the translation units that instantiate them (one per
// weight code width, compiled in parallel).  See gemm.hip for the design.
#pragma once
#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"
#include "launch.h"

namespace w4a16 {

constexpr int DW = 4;                   // waves per decode workgroup
constexpr int RUN = 8;                  // K tiles per meta run and ring pass
constexpr int64_t kWideMinN = 16384;    // narrowest layer of the wide packed decode

// Activation modes.  PACKED: M <= 4, one 16-byte load per lane and K tile
// carries the 4 MFMA steps (rows 4 j + m).  FULL: 16 MT rows, 4 MT loads per
// tile.  FULLT: FULL with the loads taking whole lines and an LDS transpose
// to the MFMA layout.  XGATHER: PACKED for an act-order weight, with the M
// rows of x (in their original column order) and the permutation staged in
// LDS once per workgroup; the loop gathers each operand from LDS,
// x[m][perm[k]], two tiles ahead of its use (one row: the 4 lanes of a quad,
// which carry the same inputs, gather 2 of the 8 each and share them by DPP),
// so neither a permutation pass nor a permute phase before the loop runs.
// Measured on MI355X against permuting the staged rows in place before the
// loop, whole calls in a graph, fp16: 11008 x 4096 at M = 4 11.57 -> 10.19
// us, M = 3 10.57 -> 9.86; 4096 x 11008 at M = 4 10.87 -> 9.98, M = 1 8.49 ->
// 7.77; 4096 x 4096 at M = 4 6.56 -> 5.56; 11008 x 4096 at M = 1 level (8.07
// -> 8.14).  XSTAGED:
// PACKED with the M rows of x staged in LDS and read from there (used with
// AWQ input scales, below).  With input scales (XS) the staged rows are
// divided by s in place, once per workgroup, before the loop: each x element
// is scaled once per workgroup instead of once per use.  GGATHER: FULL with
// one row tile, each operand element gathered from global memory,
// x[m][perm[k]] (and divided by s[perm[k]] with input scales): the form of
// every call that has a permutation or input scales, no workspace for a
// preparation pass and no room to stage its rows on chip; correct at any M,
// not fast.  TILED: FULL with the activations prepared by the preparation
// pass in the operand layout itself (tile t, row tile R, step j, lane l: the
// 16 bytes lane l feeds to MFMA step j of row tile R), so that each operand
// is one 1 KB coalesced load per wave and no transpose runs.
enum { AM_PACKED = 0, AM_FULL = 1, AM_XGATHER = 2, AM_XSTAGED = 3, AM_FULLT = 4, AM_GGATHER = 5,
       AM_TILED = 6 };
constexpr bool is_full(int am) {
  return am == AM_FULL || am == AM_FULLT || am == AM_GGATHER || am == AM_TILED;
}
constexpr bool is_packed(int am) { return !is_full(am); }
constexpr bool is_staged(int am) { return am == AM_XGATHER || am == AM_XSTAGED; }

// Largest LDS footprint of the staged activations (+ permutation, + input
// scales) per workgroup: past it the staging costs more than the separate
// preparation pass it saves (measured on MI355X; 72 rather than 56 KB takes
// the 11008 x 4096 layer at M = 1, 66 KB with its permutation, from 11.7 to
// 10.8 us per call), and with the reduction buffer it leaves room for two
// workgroups in a CU's 160 KB.
constexpr int64_t kMaxXlds = 72 * 1024;
// On a grid of at most 256 workgroups (one per CU anyway) a workgroup may take
// up to this much LDS for its staged rows, permutation and input scales (with
// the 4 KB reduction buffer, within a CU's 160 KB).
constexpr int64_t kMaxXldsOne = 152 * 1024;

// Multiply-accumulate the 4 MFMA steps of one K tile given its 4 B operands.
template <int DT, int AM, int MT, int NA, int NACC>
__device__ __forceinline__ void mma_tile(const typename Op<DT>::vec b[4],
                                         const typename Op<DT>::vec (&a)[NA],
                                         float4_t (&acc)[NACC]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (is_packed(AM)) {
      acc[j] = mfma16x16x32<DT>(a[0], b[j], acc[j]);
    } else {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        // NACC / MT accumulators per row tile take the steps in turn, so that
        // consecutive MFMAs do not wait on each other's results
        constexpr int PER = NACC / MT;
        acc[m * PER + j % PER] = mfma16x16x32<DT>(a[m * 4 + j], b[j], acc[m * PER + j % PER]);
      }
    }
  }
}

// Value of the meta unit that MFMA step g = lane >> 4 of a K tile uses, out
// of the tile's U candidates (unit g U / 4: g >> 1 for U = 2, g for U = 4),
// blended bitwise on the bits of the lane group: a chain of equality tests
// would become divergent branches, and a select between two elements of one
// local array can be turned into a load at a per-lane index, which puts the
// array in scratch memory.
template <int U, class T>
__device__ __forceinline__ T sel_unit(const T (&v)[U], int lane) {
  static_assert(sizeof(T) == 4, "32-bit values");
  if constexpr (U == 1) {
    return v[0];
  } else {
    uint32_t b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) b[u] = __builtin_bit_cast(uint32_t, v[u]);
    const uint32_t m5 = 0u - (uint32_t)((lane >> 5) & 1);
    if constexpr (U == 2) {
      return __builtin_bit_cast(T, b[0] ^ ((b[0] ^ b[1]) & m5));
    } else {
      const uint32_t m4 = 0u - (uint32_t)((lane >> 4) & 1);
      const uint32_t lo = b[0] ^ ((b[0] ^ b[1]) & m4), hi = b[2] ^ ((b[2] ^ b[3]) & m4);
      return __builtin_bit_cast(T, lo ^ ((lo ^ hi) & m5));
    }
  }
}

// ------------------------------------------------------ b-bit integer policy --
// Column tile ct = 4p + c of panel p.  Word j of lane l covers K = 128t + 32j +
// 8(l >> 4) + e, so lane-group b feeds x[row][128t + 32j + 8b ...] in step j.
// BITS-bit codes (3, 4 or 8; the Codes<BITS> forms of common.h): a column
// tile's K tile is 256 BITS bytes, lane l's codes at 12 l (3 bits), 16 l
// (4 bits) or 16 l and 1024 + 16 l (8 bits).  U meta units per K tile (group
// size 128 / U, or >= 128 for U = 1); word j of tile slot s uses unit
// r = sU + jU/4 of the run.  Zero fields are 4 bits wide (8 for 8-bit codes).
// A symmetric weight has no zeros (empty descriptor range, loads read 0) and
// zx turns each field into the implicit zero 2^(BITS-1).
template <int DT, int U, int BITS>
struct IntW {
  static constexpr bool kRaggedK = false;  // K % 128 == 0 for this format
  static constexpr int kTile = 256 * BITS;                 // bytes per column tile, K tile
  static constexpr int kZW = zero_field_bits(BITS);        // zero field width
  static constexpr int kZWords = U * kZW / 4;              // zero dwords per column and run
  typedef Codes<BITS> CodeT;
  // the codes exact as o + q in the operand type: the packed modes may apply
  // the scale and zero after each step's MFMA (a step never spans two meta
  // units)
  static constexpr bool kFold = !(BITS == 8 && DT == DT_BF16);
  static constexpr int kU = U;
  const uint8_t* codes;
  const uint8_t* scales;
  const uint8_t* zeros;
  int KT;
  uint32_t zx;  // sym_zero_xor(BITS) for a symmetric weight, else 0
  rsrc_t rc, rs, rz;
  uint32_t voc, vos, voz;
  int c;
  struct Meta {
    u32x4_t s[U];          // 8U fp16 scales of this lane's column, unit r at half r
    uint32_t z[kZWords];   // 8U zero fields, unit r at field r of the array
  };
  __device__ __forceinline__ void init(int ct, int lane, int /*N*/, int /*K*/) {
    const int p = ct >> 2;
    c = ct & 3;
    const int i = lane & 15;
    const int KT8 = (KT + RUN - 1) / RUN;
    // one descriptor per array, based at this panel: offsets stay 32-bit
    rc = make_rsrc(codes + (size_t)p * KT * 4 * kTile, (uint32_t)KT * 4u * kTile);
    rs = make_rsrc(scales + (size_t)p * KT8 * 1024 * U, (uint32_t)KT8 * 1024u * U);
    rz = make_rsrc(zeros + (size_t)p * KT8 * 256 * kZWords,
                   zx ? 0u : (uint32_t)KT8 * 256u * kZWords);
    voc = (uint32_t)(c * kTile + lane * (BITS == 3 ? 12 : 16));
    vos = (uint32_t)((c * 16 + i) * 16 * U);
    voz = (uint32_t)((c * 16 + i) * 4 * kZWords);
  }
  __device__ static __forceinline__ Meta zero_meta() {
    Meta m;
#pragma unroll
    for (int k = 0; k < U; ++k) m.s[k] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < kZWords; ++k) m.z[k] = 0u;
    return m;
  }
  __device__ __forceinline__ Meta load_meta(int run) const {
    Meta m;
#pragma unroll
    for (int k = 0; k < U; ++k) m.s[k] = bld128(rs, vos + 16u * k, run * 1024 * U);
    const int zs = run * 256 * kZWords;
    if constexpr (kZWords == 1) {
      m.z[0] = bld32(rz, voz, zs);
    } else if constexpr (kZWords == 2) {
      const u32x2_t z = bld64(rz, voz, zs);
      m.z[0] = z[0];
      m.z[1] = z[1];
    } else {
#pragma unroll
      for (int h = 0; h < kZWords / 4; ++h) {
        const u32x4_t z = bld128(rz, voz + 16u * h, zs);
#pragma unroll
        for (int k = 0; k < 4; ++k) m.z[4 * h + k] = z[k];
      }
    }
#pragma unroll
    for (int k = 0; k < kZWords; ++k) m.z[k] ^= zx;
    return m;
  }
  __device__ __forceinline__ CodeT load_codes(int t, int /*lane*/) const {
    CodeT w;
    if constexpr (BITS == 4) {
      w.w = bld128(rc, voc, t * 4 * kTile);
    } else if constexpr (BITS == 3) {
      w.w = bld96(rc, voc, t * 4 * kTile);
    } else {
      w.lo = bld128(rc, voc, t * 4 * kTile);
      w.hi = bld128(rc, voc + 1024u, t * 4 * kTile);
    }
    return w;
  }
  __device__ static __forceinline__ void unit_param(const Meta& m, int r, QParam<DT>& qp) {
    constexpr int per = 32 / kZW;  // fields per dword
    qp.template set<BITS == 4>((m.s[r >> 3][(r & 7) >> 1] >> (16 * (r & 1))) & 0xFFFFu,
                               (m.z[r / per] >> (kZW * (r % per))) & ((1u << kZW) - 1u));
  }
  // B operands of tile slot s (0..7 within the run) from the exact dequant.
  __device__ __forceinline__ void operands(const CodeT& w, int s, const Meta& m,
                                           typename Op<DT>::vec b[4]) const {
    QParam<DT> qp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j * U % 4 == 0) unit_param(m, s * U + j * U / 4, qp);  // a new unit
      b[j] = dequant_step<DT, false>(w, j, qp);
    }
  }
  // The codes alone (o + q, RawQ) as the B operands of tile slot s, and, for
  // the fold, the scale of step g of slot s (unit sU + gU/4; g is the lane
  // group, so the U candidates are formed and selected on its bits rather
  // than indexed) and the zero operands (o + z) of the slot's U units.
  __device__ __forceinline__ void raw_operands(const CodeT& w, const RawQ<DT>& rq,
                                               typename Op<DT>::vec b[4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = dequant_step<DT, false>(w, j, rq);
  }
  __device__ static __forceinline__ float unit_scale(const Meta& m, int r) {
    return (float)__builtin_bit_cast(
        _Float16, (uint16_t)((m.s[r >> 3][(r & 7) >> 1] >> (16 * (r & 1))) & 0xFFFFu));
  }
  __device__ static __forceinline__ uint32_t unit_zero(const Meta& m, int r) {
    constexpr int per = 32 / kZW;
    return (m.z[r / per] >> (kZW * (r % per))) & ((1u << kZW) - 1u);
  }
  __device__ static __forceinline__ float fold_scale(const Meta& m, int s, int lane) {
    if constexpr (U == 1) {
      return unit_scale(m, s);
    } else {
      float a[U];
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = unit_scale(m, s * U + u);
      return sel_unit<U>(a, lane);
    }
  }
  __device__ static __forceinline__ void zero_operands(const Meta& m, int s, const RawQ<DT>& rq,
                                                       typename Op<DT>::vec (&bz)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) bz[u] = rq.template zero_operand<BITS>(unit_zero(m, s * U + u));
  }
  __device__ static __forceinline__ int xk(int j, int b) { return 32 * j + 8 * b; }
};

// ---------------------------------------------------------------- NF4 policy --
// Raw layout: row n of qweight holds K/2 bytes, element 2j in the low nibble of
// byte j.  Lane (column n = 16 ct + (l & 15), group b = l >> 4) loads 16 bytes =
// elements 128t + 32b .. +31 of its row, all in one 64-element absmax block;
// word j feeds MFMA step j.  Dequant is the definition: a' = fp32(absmax_q) *
// absmax_scale, w = round16(fp32(L[c] * a')), L from a 16-entry LDS table.
// BATCH (K % 1024 == 0): the 16 absmax bytes of a run of 8 tiles of a row are
// one aligned 16-byte load and share one double-quant scale (a run of 16
// blocks never straddles a group of 256); otherwise they are loaded per tile.
// RP: the codes repacked into 1 KB tiles (nf4_repack): lane l's 16 bytes of
// K tile t are at byte 1024 t + 16 l of its column tile's run of tiles, so a
// wave's load of a tile is one contiguous 1 KB block (the canonical rows put
// its 16 rows of 64 bytes a row pitch apart).
template <int DT, bool BATCH, bool RP = false>
struct Nf4W {
  static constexpr bool kRaggedK = true;  // K % 64 == 0 only: a last tile may be half
  static constexpr bool kFold = false;
  static constexpr int kU = 1;
  typedef u32x4_t CodeT;
  const uint8_t* q;
  const uint8_t* aq;
  const float* asc;
  const float2* lut2;
  int N, K;
  rsrc_t rq, raq, ras;
  int kb;
  uint32_t voq, vob, blk0;
  struct Meta {
    // BATCH: a16 = 16 absmax codes of the run, sc = its double-quant scale.
    // otherwise: a[s] = dequantized absmax of tile slot s for this lane.
    u32x4_t a16;
    float sc;
    float a[BATCH ? 1 : RUN];
  };
  __device__ __forceinline__ void init(int ct, int lane, int N_, int K_) {
    N = N_;
    K = K_;
    const size_t n0 = (size_t)ct * 16;
    const int nloc = lane & 15;
    kb = lane >> 4;
    if constexpr (RP) {
      const uint32_t KTc = (uint32_t)(K + 127) / 128u;
      rq = make_rsrc(q + (size_t)ct * KTc * 1024, KTc * 1024u);
    } else {
      rq = make_rsrc(q + n0 * (K >> 1), 16u * (uint32_t)(K >> 1));
    }
    raq = make_rsrc(aq + n0 * (K >> 6), 16u * (uint32_t)(K >> 6));
    const size_t nblocks = (size_t)N * (K >> 6);
    ras = make_rsrc(asc, (uint32_t)(((nblocks + 255) >> 8) * 4));
    blk0 = (uint32_t)(n0 * (K >> 6));
    voq = RP ? (uint32_t)lane * 16u : (uint32_t)(nloc * (K >> 1) + 16 * kb);
    vob = (uint32_t)(nloc * (K >> 6));
  }
  __device__ static __forceinline__ Meta zero_meta() {
    Meta m;
    m.a16 = u32x4_t{0u, 0u, 0u, 0u};
    m.sc = 0.0f;
#pragma unroll
    for (int s = 0; s < (BATCH ? 1 : RUN); ++s) m.a[s] = 0.0f;
    return m;
  }
  __device__ __forceinline__ Meta load_meta(int run) const {
    Meta m = zero_meta();
    if constexpr (BATCH) {
      m.a16 = bld128(raq, vob + (uint32_t)(16 * run), 0);
      m.sc = __builtin_bit_cast(float, bld32(ras, ((blk0 + vob + 16u * run) >> 8) * 4u, 0));
    } else {
#pragma unroll
      for (int s = 0; s < RUN; ++s) {
        // block of (row, tile 8 run + s, lane group); reads past the row meet
        // zero activations
        const uint32_t bl = vob + (uint32_t)(2 * (RUN * run + s) + (kb >> 1));
        const uint32_t qa = __builtin_amdgcn_raw_buffer_load_b8(raq, bl, 0, 0);
        const float sa = __builtin_bit_cast(float, bld32(ras, ((blk0 + bl) >> 8) * 4u, 0));
        m.a[s] = (float)qa * sa;
      }
    }
    return m;
  }
  // t is a valid K tile.  In a half-filled last tile the lanes past K use an
  // out-of-range per-lane offset and read zeros.
  __device__ __forceinline__ u32x4_t load_codes(int t, int /*lane*/) const {
    const uint32_t vq = (t * 128 + 32 * kb < K) ? voq : kOutOfRange;
    return bld128(rq, vq, t * (RP ? 1024 : 64));
  }
  __device__ __forceinline__ void operands(const u32x4_t& w4, int s, const Meta& m,
                                           typename Op<DT>::vec b[4]) const {
    float a;
    if constexpr (BATCH) {
      // absmax code of block 2 s + (b >> 1) of the run: byte 2 (s & 1) + (b >> 1)
      // of word s >> 1
      const uint32_t qa = (m.a16[s >> 1] >> (16 * (s & 1) + 8 * (kb >> 1))) & 0xFFu;
      a = (float)qa * m.sc;
    } else {
      a = m.a[s];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = nf4_pair_operand<DT>(w4[j], lut2, a);
  }
  __device__ static __forceinline__ int xk(int j, int b) { return 32 * b + 8 * j; }
};

// Activations of one K tile.  PACKED: one vector, lane row r = 4 j + m holds
// step j of batch row m.  FULL: MT x 4 vectors, vector 4m + j the A operand
// of row tile m, step j (lane row r = batch row: 16 rows x 64 bytes per
// load).  FULLT: vector 4m + i of lane l is 16-byte chunk l & 15 of row
// 4i + (l >> 4) of row tile m (whole 128-byte lines per load), which xpose_a
// puts into the MFMA layout through LDS.  Rows >= M read 0 through the
// descriptor range; k >= K (only in a half NF4 tile) uses an out-of-range
// offset.
// Staged activations in LDS: x rows [M][K] at xl, row m at m * pitch
// (XGATHER: the rows in their original column order and the permutation at
// pl, gathered per operand in the loop).
// GGATHER: the permutation (when perm) and the input scales in global memory,
// behind the descriptors rp and rs.  TILED: rt row tiles in the prepared
// buffer, rt0 the workgroup's first.
struct XLds {
  const uint8_t* xl;
  const uint8_t* pl;
  uint32_t pitch;
  int M;
  rsrc_t rp, rs;
  bool perm;
  int rt, rt0;
};

template <int DT, int AM, int MT, int NA, class WP, bool XS = false>
__device__ __forceinline__ void load_a(rsrc_t rx, int K, int t, int lane,
                                       typename Op<DT>::vec (&a)[NA], const XLds& xs) {
  typedef typename Op<DT>::vec vec;
  const int r = lane & 15, b = lane >> 4;
  static_assert(AM != AM_XGATHER, "XGATHER operands are gathered by xg_perm / xg_gather");
  if constexpr (AM == AM_GGATHER) {
    // one row tile: lane row r, 8 inputs of step j per operand; rows past M
    // read 0 through the descriptor range of rx, as does any input of a
    // permutation entry outside the row
    const uint32_t rowoff = (uint32_t)r * (uint32_t)K * 2u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kg = t * 128 + WP::xk(j, b);
      uint32_t src[8];
      if (xs.perm) {
        const u32x4_t p0 = bld128(xs.rp, (uint32_t)kg * 4u, 0);
        const u32x4_t p1 = bld128(xs.rp, (uint32_t)kg * 4u + 16u, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          src[e] = min(p0[e], (uint32_t)K);
          src[4 + e] = min(p1[e], (uint32_t)K);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) src[e] = (uint32_t)(kg + e);
      }
      uint32_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = bld16(rx, rowoff + src[e] * 2u, 0);
        if constexpr (XS) v[e] = div_scale1<DT>((uint16_t)v[e], (uint16_t)bld16(xs.rs, src[e] * 2u, 0));
      }
      const u32x4_t w = {v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16),
                         v[6] | (v[7] << 16)};
      a[j] = __builtin_bit_cast(vec, w);
    }
  } else if constexpr (AM == AM_XSTAGED) {
    const int j = r >> 2, m = min(r & 3, xs.M - 1);
    const uint32_t kg = (uint32_t)(t * 128 + WP::xk(j, b));
    a[0] = *(const vec*)(xs.xl + ((uint32_t)m * (uint32_t)K + kg) * 2u);
  } else if constexpr (AM == AM_PACKED) {
    const int j = r >> 2, m = r & 3;
    const int kin = WP::xk(j, b);
    uint32_t off = (uint32_t)m * (uint32_t)K * 2u + (uint32_t)kin * 2u;
    if constexpr (WP::kRaggedK) off = (t * 128 + kin < K) ? off : kOutOfRange;
    a[0] = __builtin_bit_cast(typename Op<DT>::vec, bld128(rx, off, t * 256));
  } else if constexpr (AM == AM_TILED) {
    // rx covers the whole prepared buffer (row tiles past it read 0)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a[m * 4 + j] = __builtin_bit_cast(
            typename Op<DT>::vec,
            bld128(rx, (uint32_t)(j * 1024 + lane * 16), (t * xs.rt + xs.rt0 + m) * 4096));
    }
  } else if constexpr (AM == AM_FULLT) {
    const int c = lane & 15;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t row = (uint32_t)(m * 16 + 4 * i + b);
        uint32_t off = row * (uint32_t)K * 2u + (uint32_t)c * 16u;
        if constexpr (WP::kRaggedK) off = (t * 128 + c * 8 < K) ? off : kOutOfRange;
        a[m * 4 + i] = __builtin_bit_cast(typename Op<DT>::vec, bld128(rx, off, t * 256));
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint32_t rowoff = (uint32_t)(m * 16 + r) * (uint32_t)K * 2u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kin = WP::xk(j, b);
        uint32_t off = rowoff + (uint32_t)kin * 2u;
        if constexpr (WP::kRaggedK) off = (t * 128 + kin < K) ? off : kOutOfRange;
        a[m * 4 + j] = __builtin_bit_cast(typename Op<DT>::vec, bld128(rx, off, t * 256));
      }
    }
  }
}

// FULLT mode: the contiguous chunks of load_a to the A operands of the 4 MFMA
// steps, through this wave's 4 KB per row tile of LDS at xw.  Chunk c of row R
// sits in 16-byte slot 16 R + (c ^ R): the stores (a row per 16 lanes) and the
// loads (16 rows of one chunk per 16 lanes) each cover all 64 banks.
template <int DT, int MT, class WP>
__device__ __forceinline__ void xpose_a(const typename Op<DT>::vec (&a)[MT * 4],
                                        typename Op<DT>::vec (&o)[MT * 4], uint8_t* xw,
                                        int lane) {
  typedef typename Op<DT>::vec vec;
  const int c = lane & 15, b = lane >> 4, r = lane & 15;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int R = 4 * i + b;
      *(vec*)(xw + (m * 256 + R * 16 + (c ^ R)) * 16) = a[m * 4 + i];
    }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ch = WP::xk(j, b) >> 3;
      o[m * 4 + j] = *(const vec*)(xw + (m * 256 + r * 16 + (ch ^ r)) * 16);
    }
}

// Whether the FULLT mode applies the scale and zero after each K tile's sum:
// integer codes with the fold's exact o + q operands and one meta unit per K
// tile (G >= 128).
template <class WP>
constexpr bool full_fold() {
  if constexpr (WP::kFold) return WP::kU == 1;
  else return false;
}

// LDS bytes of the FULLT mode's transpose: 4 KB per row tile and wave.
__host__ __device__ constexpr uint32_t xpose_bytes(int MT) { return (uint32_t)(DW * MT * 4096); }

// Staged LDS layout, each region rounded up to whole 1 KB blocks: x rows
// [M][K] at a pitch of 2 K bytes (XSTAGED) or 2 K + 32 (XGATHER: the 4 rows
// that one gather reads for an input sit 8 banks apart), then (input
// scales) s [K], then (XGATHER) the permutation [K] as int32.  XGATHER keeps
// the rows in their original column order: the loop gathers each operand
// from them through the staged permutation (xg_perm, xg_gather).
__host__ __device__ constexpr uint32_t xlds_pitch(int K, bool perm) {
  return (uint32_t)(2 * K + (perm ? 32 : 0));
}
__host__ __device__ constexpr uint32_t xlds_x_bytes(int M, int K, bool perm) {
  return (uint32_t)(((int64_t)M * xlds_pitch(K, perm) + 1023) / 1024 * 1024);
}
__host__ __device__ constexpr uint32_t xlds_s_bytes(int K, bool xs) {
  return xs ? (uint32_t)((K * 2 + 1023) / 1024 * 1024) : 0u;
}
__host__ __device__ constexpr uint32_t xlds_p_bytes(int K, bool perm) {
  return perm ? (uint32_t)((K * 4 + 1023) / 1024 * 1024) : 0u;
}
// what each workgroup reads from memory besides the weights: the rows, the
// permutation and the input scales
__host__ __device__ constexpr uint32_t xlds_staged_bytes(int M, int K, bool perm, bool xs) {
  return (uint32_t)(M * K * 2) + (perm ? (uint32_t)(K * 4) : 0u) + (xs ? (uint32_t)(K * 2) : 0u);
}
// the LDS footprint
__host__ __device__ constexpr uint32_t xlds_bytes(int M, int K, bool perm, bool xs) {
  return xlds_x_bytes(M, K, perm) + xlds_s_bytes(K, xs) + xlds_p_bytes(K, perm);
}

// 16 bytes per lane from a buffer straight into LDS: lane l's data lands at
// lds + 16 l (the LDS base is wave-uniform).
__device__ __forceinline__ void lds_dma16(rsrc_t r, uint8_t* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// Copy `bytes` (rounded up to 1 KB; the tail reads 0 through the descriptor
// range) from `src` to LDS, 1 KB per wave instruction.
__device__ __forceinline__ void stage_lds(const void* src, uint32_t bytes, uint8_t* lds,
                                          int wave, int lane) {
  const rsrc_t r = make_rsrc(src, bytes);
  const int nblk = (int)((bytes + 1023) / 1024);
  for (int blk = wave; blk < nblk; blk += DW)
    lds_dma16(r, lds + blk * 1024, (uint32_t)(blk * 1024 + lane * 16), 0);
}

// Copy exactly `bytes` (a multiple of 256) from offset `off` of r to LDS: whole
// 1 KB blocks by 16-byte lanes, the rest by 4-byte lanes (256 bytes per wave
// instruction), so nothing past the span is written.
__device__ __forceinline__ void stage_exact(rsrc_t r, uint32_t off, uint32_t bytes, uint8_t* lds,
                                            int wave, int lane) {
  const int nk = (int)(bytes >> 10);
  for (int blk = wave; blk < nk; blk += DW)
    lds_dma16(r, lds + blk * 1024, off + (uint32_t)(blk * 1024 + lane * 16), 0);
  const int nq = (int)((bytes & 1023u) >> 8);
  if (wave < nq)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(lds + nk * 1024 + wave * 256), 4,
        off + (uint32_t)(nk * 1024 + wave * 256 + lane * 4), 0, 0, 0);
}

// A workgroup barrier for LDS data: this wave's LDS writes (and LDS DMA) are
// complete before it, other waves' are visible after it; loads from global
// memory in flight are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// XGATHER: the 8 permutation entries of this lane's operand of tile t (inputs
// 128 t + 32 j + 8 b .. + 7 of A row 4 j + m, lane group b), from the staged
// permutation.
template <class WP>
__device__ __forceinline__ void xg_perm(const XLds& xs, int t, int lane, u32x4_t (&pq)[2]) {
  const int j = (lane & 15) >> 2, b = lane >> 4;
  const uint8_t* pp = xs.pl + (uint32_t)(t * 128 + WP::xk(j, b)) * 4u;
  pq[0] = *(const u32x4_t*)pp;
  pq[1] = *(const u32x4_t*)(pp + 16);
}
// ... and the operand itself, x[m][perm[k]] for those 8 inputs, gathered from
// the staged row (rows m >= M only feed output rows that are never stored,
// so they read row M - 1).
template <int DT>
__device__ __forceinline__ typename Op<DT>::vec xg_gather(const XLds& xs, int lane,
                                                          const u32x4_t (&pq)[2]) {
  const uint8_t* rb = xs.xl + (uint32_t)min(lane & 3, xs.M - 1) * xs.pitch;
  // (16-bit values as pairs built from two loads: the odd one loads into the
  // high half in place)
  u32x4_t w;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    half2_t h;
    h[0] = *(const _Float16*)(rb + pq[q >> 1][2 * (q & 1)] * 2u);
    h[1] = *(const _Float16*)(rb + pq[q >> 1][2 * (q & 1) + 1] * 2u);
    w[q] = __builtin_bit_cast(uint32_t, h);
  }
  return __builtin_bit_cast(typename Op<DT>::vec, w);
}

// The same for one batch row (M == 1), shared by the 4 lanes of a quad (lane
// bits 0-1, which hold the 4 rows of A that only that row feeds): lane q of
// the quad gathers inputs 2q and 2q + 1 of the 8 (xg_perm1, xg_gather1) and
// the operand is assembled at its use from the quad's 4 pairs by DPP
// broadcasts (xg_assemble1).
template <class WP>
__device__ __forceinline__ u32x2_t xg_perm1(const XLds& xs, int t, int lane) {
  const int j = (lane & 15) >> 2, b = lane >> 4;
  return *(const u32x2_t*)(xs.pl + (uint32_t)(t * 128 + WP::xk(j, b) + 2 * (lane & 3)) * 4u);
}
__device__ __forceinline__ uint32_t xg_gather1(const XLds& xs, u32x2_t p) {
  half2_t h;
  h[0] = *(const _Float16*)(xs.xl + p[0] * 2u);
  h[1] = *(const _Float16*)(xs.xl + p[1] * 2u);
  return __builtin_bit_cast(uint32_t, h);
}
template <int DT>
__device__ __forceinline__ typename Op<DT>::vec xg_assemble1(uint32_t d) {
  // quad_perm [q, q, q, q]: every lane of the quad takes lane q's pair
  const u32x4_t w = {(uint32_t)__builtin_amdgcn_mov_dpp((int)d, 0x00, 0xF, 0xF, false),
                     (uint32_t)__builtin_amdgcn_mov_dpp((int)d, 0x55, 0xF, 0xF, false),
                     (uint32_t)__builtin_amdgcn_mov_dpp((int)d, 0xAA, 0xF, 0xF, false),
                     (uint32_t)__builtin_amdgcn_mov_dpp((int)d, 0xFF, 0xF, 0xF, false)};
  return __builtin_bit_cast(typename Op<DT>::vec, w);
}

// XS: divide the staged activations by the AWQ input scales xsc [K] (staged
// modes only).  ONE: a single batch row (M == 1) in a packed mode with the
// fold, which then keeps only element 0 of each lane's step tiles (row 4g of
// the A operand; the others are rows past M): a quarter of the fold's selects
// and multiply-adds.
template <int DT, int MT, int AM, bool XS, bool ONE = false, class WP>
__device__ __forceinline__ void decode_body(const uint16_t* __restrict__ x,
                                            const uint16_t* __restrict__ xsc, WP& wp,
                                            uint16_t* __restrict__ out, int M, int N, int K,
                                            int KT, float* red, const int32_t* perm,
                                            uint8_t* xlds) {
  static_assert(!XS || is_staged(AM) || AM == AM_GGATHER,
                "input scales are applied to staged or gathered rows");
  static_assert(AM != AM_GGATHER || MT == 1, "the global gather takes one row tile");
  static_assert(AM != AM_XSTAGED || XS, "rows are staged for input scales");
  constexpr int NA = is_packed(AM) ? 1 : MT * 4;                   // A vectors per tile
  constexpr int NACC = is_packed(AM) ? 4 : MT * (MT == 1 ? 4 : (MT == 2 ? 2 : 1));  // acc tiles
  // A ring depth (XGATHER: operands gathered two tiles ahead, their
  // permutation entries read one tile before that)
  constexpr int PA = AM == AM_XGATHER ? 2 : (is_packed(AM) ? RUN : (MT == 1 ? 2 : 1));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ct = blockIdx.x;
  const int row0 = blockIdx.y * 16 * MT;
  wp.init(ct, lane, N, K);
  const int nrun = (KT + RUN - 1) / RUN;
  const int r0 = (nrun * wave) / DW, r1 = (nrun * (wave + 1)) / DW;
  const int t0 = r0 * RUN;
  const int n = min(KT, r1 * RUN) - t0;  // tiles of this wave (wave-uniform)
  const int vrows = min(16 * MT, M - row0);
  const int rtiles = (M + 15) >> 4;
  const rsrc_t rx = AM == AM_TILED
                        ? make_rsrc(x, (uint32_t)rtiles * 32u * (uint32_t)K)
                        : make_rsrc(x + (size_t)row0 * K, (uint32_t)vrows * (uint32_t)K * 2u);

  float4_t acc[NACC];
#pragma unroll
  for (int q = 0; q < NACC; ++q) acc[q] = float4_t{0.f, 0.f, 0.f, 0.f};
  // FOLD (packed modes, integer codes): the B operands are the codes alone
  // (o + q, exact), each K tile's 4 steps go to fresh step tiles at[j], and
  // MFMAs of the same A against the zero operands (o + z, one per meta unit
  // of the tile) give az[u].  Lane group g's rows are step g's, so the lane
  // keeps
  //   yf += s (at[g] - az[unit of step g]),
  // s of its own column and step g's meta unit: the scale and zero cost a
  // subtract and a multiply-add per accumulator and tile instead of VALU work
  // in every operand.  The weights are never rounded to 16 bits in this form
  // (a one-hot row still gives round16((q - z) s) exactly), and a group whose
  // codes all equal its zero gives at[g] == az bit for bit, so exactly 0.
  constexpr bool FOLD = is_packed(AM) && WP::kFold;
  static_assert(!ONE || FOLD, "the one-row form is a form of the fold");
  // FFOLD (FULLT with one row tile, integer codes, G >= 128): per K tile, the
  // 4 steps' o + q products and the products with the zero operand (o + z)
  // each go to a fresh tile; yfm += s (accT - accZ) with the lane's column's
  // s.  Measured on MI355X, act-order whole calls at M = 16 (with the row sums
  // then taken against ones): fp16 2-5 % faster than the exact dequant
  // (4096 x 11008 15.6 -> 15.0 us), bf16 6-8 % (11008 x 4096 17.8 -> 16.6);
  // with two row tiles (M = 24) the doubled MFMAs cost more than the dequant
  // they save (5120 x 5120 14.2 -> 15.2).
  constexpr bool FFOLD = (AM == AM_FULLT || AM == AM_TILED) && MT == 1 && full_fold<WP>();
  float4_t yfm[FFOLD ? MT : 1];
#pragma unroll
  for (int m = 0; m < (FFOLD ? MT : 1); ++m) yfm[m] = float4_t{0.f, 0.f, 0.f, 0.f};
  constexpr int FE = ONE ? 1 : 4;  // fold elements per lane
  float4_t yf = float4_t{0.f, 0.f, 0.f, 0.f};
  // Deferred fold (FOLD, FFOLD): a tile's MFMA results are folded into the
  // accumulators in the next tile's slot, after that tile's MFMAs have been
  // issued, so each tile's MFMA latency is covered by the other tile's work
  // instead of stalling the wave (one wave per SIMD on most decode grids).
  // The tiles are still folded one after another in K order, so the sums are
  // the same bit for bit; the pending results start at zero (a fold of zeros
  // leaves the accumulators unchanged) and the last tile is folded after the
  // loop.
  constexpr int PDA = FOLD ? 4 : (FFOLD ? MT : 1), PDZ = FOLD ? WP::kU : (FFOLD ? MT : 1);
  // NB = 2: two sets of pending results, by the parity of the tile (a run of
  // RUN tiles is even and the slots are unrolled, so each slot's set is
  // fixed): a tile's results go to its own set while the other set, the
  // previous tile's, is folded, so they need not be copied between registers
  // (4-13 fewer VALU instructions per K tile).  The packed modes over several
  // rows without the on-chip gather keep one set (a copy per tile): with two
  // they pass 128 VGPRs, which would cut the waves a CU holds from 4 to 3.
  static_assert(RUN % 2 == 0, "the pending sets alternate by slot parity");
  constexpr int NB = (is_packed(AM) && AM != AM_XGATHER && !ONE) ? 1 : 2;
  float4_t pat[NB][PDA], paz[NB][PDZ];
  float psf[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    psf[b] = 0.f;
#pragma unroll
    for (int q = 0; q < PDA; ++q) pat[b][q] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < PDZ; ++q) paz[b][q] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  // FOLD, FFOLD: the offsets of the raw code and zero operands, set once and
  // held in registers for the whole loop (made per tile, each tile's branch
  // would set them again)
  const RawQ<DT> rq;
  // FOLD: yf += s (at[lane group] - az[unit of the lane group's step]), the
  // step tile taken as two levels of selects on the bits of the lane group
  // (a chain of equality tests becomes branches)
  auto fold_packed = [&](const float4_t (&a)[PDA], const float4_t (&z)[PDZ], float sf) {
    if constexpr (FOLD) {
      const bool h0 = lane & 16, h1 = lane & 32;
#pragma unroll
      for (int e = 0; e < FE; ++e) {
        const float v01 = h0 ? a[1][e] : a[0][e], v23 = h0 ? a[3][e] : a[2][e];
        float zu[WP::kU];
#pragma unroll
        for (int u = 0; u < WP::kU; ++u) zu[u] = z[u][e];
        yf[e] = __builtin_fmaf(sf, (h1 ? v23 : v01) - sel_unit<WP::kU>(zu, lane), yf[e]);
      }
    }
  };
  // FFOLD: yfm += s (accT - accZ) per row tile
  auto fold_full = [&](const float4_t (&a)[PDA], const float4_t (&z)[PDZ], float sf) {
    if constexpr (FFOLD) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) yfm[m][e] = __builtin_fmaf(sf, a[m][e] - z[m][e], yfm[m][e]);
    }
  };

  // Ring of RUN tiles: slot s holds tile i + s of the current pass.  The
  // fill (tiles 0 .. RUN - 1 and the first run's meta) is issued first; each
  // pass then computes slot s and refills it with tile i + s + RUN (clamped
  // into range: the tail re-reads the last tile from cache, and slots past
  // the wave's range are not computed).  The meta of a run is double-buffered.
  // Scheduling barriers keep slot order in the instruction stream so each
  // slot's wait covers only its own loads.
  typename WP::CodeT ring[RUN];
  typename Op<DT>::vec ra[PA][NA];
  typename WP::Meta mc, mn = WP::zero_meta();
  constexpr bool XG = AM == AM_XGATHER;
  XLds xs{xlds, xlds + xlds_x_bytes(M, K, XG) + xlds_s_bytes(K, XS), xlds_pitch(K, XG), M,
          make_rsrc(perm, 0u), make_rsrc(xsc, 0u), perm != nullptr, rtiles,
          (int)blockIdx.y * MT};
  if constexpr (AM == AM_GGATHER) {
    xs.rp = make_rsrc(perm, perm ? (uint32_t)K * 4u : 0u);
    xs.rs = make_rsrc(xsc, XS ? (uint32_t)K * 2u : 0u);
  }
  // Staged modes: the LDS DMA of the rows (and input scales, and the
  // permutation) goes out before the first code tiles, so the staging
  // barrier waits only for it while the tiles stay in flight.
  if constexpr (XG) {
    const rsrc_t rxa = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    for (int m = 0; m < M; ++m)
      stage_exact(rxa, (uint32_t)m * (uint32_t)K * 2u, (uint32_t)K * 2u, xlds + m * xs.pitch, wave,
                  lane);
    if constexpr (XS)
      stage_exact(make_rsrc(xsc, (uint32_t)K * 2u), 0u, (uint32_t)K * 2u,
                  xlds + xlds_x_bytes(M, K, true), wave, lane);
    stage_exact(make_rsrc(perm, (uint32_t)K * 4u), 0u, (uint32_t)K * 4u, const_cast<uint8_t*>(xs.pl),
                wave, lane);
  } else if constexpr (is_staged(AM)) {
    stage_lds(x, (uint32_t)(M * K * 2), xlds, wave, lane);
    if constexpr (XS) stage_lds(xsc, (uint32_t)(K * 2), xlds + xlds_x_bytes(M, K, false), wave, lane);
  }
  // (staged: unconditional, a wave without tiles reading its first tile, so
  // that the staging barrier's wait counts the same loads on every path)
  if constexpr (is_staged(AM)) __builtin_amdgcn_sched_barrier(0);
  if (is_staged(AM) || n > 0) {
    mn = wp.load_meta(r0);
#pragma unroll
    for (int s = 0; s < RUN; ++s) ring[s] = wp.load_codes(t0 + max(min(s, n - 1), 0), lane);
  }
  if constexpr (is_staged(AM)) __builtin_amdgcn_sched_barrier(0);
  if constexpr (is_staged(AM)) {
    lds_barrier();
    if constexpr (XS) {
      // x[m][k] / s[k] in place (original column order): a pair of columns per
      // step, their reciprocals shared by the M rows
      const uint32_t* sw = (const uint32_t*)(xlds + xlds_x_bytes(M, K, XG));
      const int half = K >> 1;
      for (int kp = threadIdx.x; kp < half; kp += 64 * DW) {
        const uint32_t sv = sw[kp];
        const float r0 = recip_scale<DT>((uint16_t)(sv & 0xFFFFu));
        const float r1 = recip_scale<DT>((uint16_t)(sv >> 16));
        for (int m = 0; m < M; ++m) {
          uint32_t* xw = (uint32_t*)(xlds + m * xs.pitch) + kp;
          const uint32_t v = *xw;
          *xw = (uint32_t)mul_round16<DT>((uint16_t)(v & 0xFFFFu), r0) |
                ((uint32_t)mul_round16<DT>((uint16_t)(v >> 16), r1) << 16);
        }
      }
      lds_barrier();
    }
  }
  u32x4_t pq[2];   // XGATHER: permutation entries of the next operand to gather
  u32x2_t pq1;     // (one row: this lane's 2 of them)
  uint32_t g1[PA];  // (one row: this lane's gathered pair per ring slot)
  if (n > 0) {
    if constexpr (XG && ONE) {
      pq1 = xg_perm1<WP>(xs, t0, lane);
#pragma unroll
      for (int s = 0; s < PA; ++s) {
        g1[s] = xg_gather1(xs, pq1);
        pq1 = xg_perm1<WP>(xs, t0 + min(s + 1, n - 1), lane);
      }
    } else if constexpr (XG) {
      xg_perm<WP>(xs, t0, lane, pq);
#pragma unroll
      for (int s = 0; s < PA; ++s) {
        ra[s][0] = xg_gather<DT>(xs, lane, pq);
        xg_perm<WP>(xs, t0 + min(s + 1, n - 1), lane, pq);
      }
    } else {
#pragma unroll
      for (int s = 0; s < PA; ++s) load_a<DT, AM, MT, NA, WP, XS>(rx, K, t0 + min(s, n - 1), lane, ra[s], xs);
    }
    for (int i = 0; i < n; i += RUN) {
      mc = mn;
      mn = wp.load_meta(r0 + min(i / RUN + 1, (n - 1) / RUN));
#pragma unroll
      for (int s = 0; s < RUN; ++s) {
        const int sa = s % PA;
        if (i + s < n) {  // wave-uniform
          typename Op<DT>::vec b[4];
          if constexpr (FOLD) {
            const float4_t z4 = float4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (XG && ONE) ra[sa][0] = xg_assemble1<DT>(g1[sa]);
            wp.raw_operands(ring[s], rq, b);
            // this tile's set and the previous tile's (unrolled: fixed)
            const int cb = NB == 2 ? (s & 1) : 0, pb = NB == 2 ? (cb ^ 1) : 0;
            float4_t at[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) at[j] = mfma16x16x32<DT>(ra[sa][0], b[j], z4);
            typename Op<DT>::vec bz[WP::kU];
            WP::zero_operands(mc, s, rq, bz);
            float4_t az[WP::kU];
#pragma unroll
            for (int u = 0; u < WP::kU; ++u) az[u] = mfma16x16x32<DT>(ra[sa][0], bz[u], z4);
            const float sf = WP::fold_scale(mc, s, lane);
            // the previous tile's results, while this tile's MFMAs run
            fold_packed(pat[pb], paz[pb], psf[pb]);
#pragma unroll
            for (int j = 0; j < 4; ++j) pat[cb][j] = at[j];
#pragma unroll
            for (int u = 0; u < WP::kU; ++u) paz[cb][u] = az[u];
            psf[cb] = sf;
          } else {
            if constexpr (FFOLD) wp.raw_operands(ring[s], rq, b);
            else wp.operands(ring[s], s, mc, b);
            if constexpr (AM == AM_FULLT || AM == AM_TILED) {
              typename Op<DT>::vec at[NA];
              if constexpr (AM == AM_FULLT) {
                xpose_a<DT, MT, WP>(ra[sa], at, xlds + wave * MT * 4096, lane);
              } else {
#pragma unroll
                for (int q = 0; q < NA; ++q) at[q] = ra[sa][q];
              }
              if constexpr (FFOLD) {
                typename Op<DT>::vec bz[1];
                WP::zero_operands(mc, s, rq, bz);
                // this tile's set and the previous tile's (unrolled: fixed)
                const int cb = s & 1, pb = cb ^ 1;
                psf[cb] = WP::fold_scale(mc, s, lane);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                  pat[cb][m] = float4_t{0.f, 0.f, 0.f, 0.f};
                  paz[cb][m] = pat[cb][m];
#pragma unroll
                  for (int j = 0; j < 4; ++j) {
                    pat[cb][m] = mfma16x16x32<DT>(at[m * 4 + j], b[j], pat[cb][m]);
                    paz[cb][m] = mfma16x16x32<DT>(at[m * 4 + j], bz[0], paz[cb][m]);
                  }
                }
                // the previous tile's sums, while this tile's MFMAs run
                fold_full(pat[pb], paz[pb], psf[pb]);
              } else {
                mma_tile<DT, AM, MT, NA, NACC>(b, at, acc);
              }
            } else {
              mma_tile<DT, AM, MT, NA, NACC>(b, ra[sa], acc);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        ring[s] = wp.load_codes(t0 + min(i + s + RUN, n - 1), lane);
        if constexpr (XG && ONE) {
          g1[sa] = xg_gather1(xs, pq1);
          pq1 = xg_perm1<WP>(xs, t0 + min(i + s + PA + 1, n - 1), lane);
        } else if constexpr (XG) {
          // pq holds the entries of tile i + s + PA (clamped)
          ra[sa][0] = xg_gather<DT>(xs, lane, pq);
          xg_perm<WP>(xs, t0 + min(i + s + PA + 1, n - 1), lane, pq);
        } else {
          load_a<DT, AM, MT, NA, WP, XS>(rx, K, t0 + min(i + s + PA, n - 1), lane, ra[sa], xs);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the last tile's results: its set is that of its slot, (n - 1) % RUN,
    // whose parity is that of n - 1
    if (NB == 2 && ((n - 1) & 1)) {
      fold_packed(pat[NB - 1], paz[NB - 1], psf[NB - 1]);
      fold_full(pat[NB - 1], paz[NB - 1], psf[NB - 1]);
    } else {
      fold_packed(pat[0], paz[0], psf[0]);
      fold_full(pat[0], paz[0], psf[0]);
    }
  }

  // ---- v_mfma_f32_16x16x32 result layout: element e of lane l is row
  // 4 (l >> 4) + e, column l & 15 of the 16x16 tile.
  float4_t res[MT];
  if constexpr (is_packed(AM)) {
    // rows 4g .. 4g+3 of step tile acc[g] (g = lane group) are batch rows
    // 0..3 of step g: take them and add the 4 lane groups (a shuffle
    // reduction across the wave); lane group 0 then holds rows 0..3.
    const int g = lane >> 4;
    float4_t v = FOLD ? yf : (g == 0 ? acc[0] : (g == 1 ? acc[1] : (g == 2 ? acc[2] : acc[3])));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] += __shfl_xor(v[e], 16, 64);
      v[e] += __shfl_xor(v[e], 32, 64);
    }
    res[0] = g == 0 ? v : float4_t{0.f, 0.f, 0.f, 0.f};
  } else {
    constexpr int PER = NACC / MT;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if constexpr (FFOLD) {
        res[m] = yfm[m];
        continue;
      }
      res[m] = acc[m * PER];
#pragma unroll
      for (int q = 1; q < PER; ++q) {
        res[m][0] += acc[m * PER + q][0];
        res[m][1] += acc[m * PER + q][1];
        res[m][2] += acc[m * PER + q][2];
        res[m][3] += acc[m * PER + q][3];
      }
    }
  }

  // ---- wave partials -> LDS, summed in wave order
#pragma unroll
  for (int m = 0; m < MT; ++m)
    *(float4_t*)(red + ((wave * MT + m) * 64 + lane) * 4) = res[m];
  __syncthreads();
  if (wave < MT) {
    const int m = wave;
    float4_t s = *(const float4_t*)(red + ((0 * MT + m) * 64 + lane) * 4);
#pragma unroll
    for (int w = 1; w < DW; ++w) {
      const float4_t v = *(const float4_t*)(red + ((w * MT + m) * 64 + lane) * 4);
      s[0] += v[0];
      s[1] += v[1];
      s[2] += v[2];
      s[3] += v[3];
    }
    const int col = ct * 16 + (lane & 15);
    if (col < N) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = row0 + m * 16 + 4 * (lane >> 4) + e;
        if (row < M) out[(size_t)row * N + col] = round16<DT>(s[e]);
      }
    }
  }
}

// Wide packed decode (M <= 4, integer codes, plain activations): each wave
// owns NC column tiles and feeds every activation load to all of them, so
// the rows of x are read from L2 once per NC column tiles instead of once per
// tile (at M = 4 on a 5120 x 55296 layer those re-reads are as many bytes as
// the weights).  Otherwise as the packed mode of decode_body with the scale
// and zero applied after each step's MFMA: DW waves split the K tiles of the
// workgroup's NC column tiles in runs of WRUN tiles, ring of WRUN tiles per
// column tile, wave partials added in wave order through LDS.
template <int DT, int U, int BITS, int NC, int WRUN>
__global__ void __launch_bounds__(64 * DW)
intb_decode_wide_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
                        const uint8_t* __restrict__ scales, const uint8_t* __restrict__ zeros,
                        uint32_t zx, uint16_t* __restrict__ out, int M, int N, int K, int KT) {
  typedef IntW<DT, U, BITS> WP;
  typedef typename Op<DT>::vec vec;
  static_assert(WP::kFold, "the wide mode applies the scale and zero after the sum");
  static_assert(RUN % WRUN == 0, "a ring pass stays inside one meta run");
  __shared__ float red[DW * NC * 64 * 4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  WP wp[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    wp[c].codes = codes;
    wp[c].scales = scales;
    wp[c].zeros = zeros;
    wp[c].zx = zx;
    wp[c].KT = KT;
    // (column tiles past N lie in the last panel's padding: read, never stored)
    wp[c].init(blockIdx.x * NC + c, lane, N, K);
  }
  const int nrun = (KT + RUN - 1) / RUN;
  const int r0 = (nrun * wave) / DW, r1 = (nrun * (wave + 1)) / DW;
  const int t0 = r0 * RUN;
  const int n = min(KT, r1 * RUN) - t0;  // tiles of this wave (wave-uniform)
  const rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const float4_t z4 = float4_t{0.f, 0.f, 0.f, 0.f};
  const XLds none{nullptr, nullptr, 0u, M, make_rsrc(nullptr, 0u), make_rsrc(nullptr, 0u), false, 0, 0};
  const bool g0 = lane & 16, g1 = lane & 32;
  // the operand offsets, held in registers for the whole loop
  const RawQ<DT> rq;

  float4_t yf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) yf[c] = z4;
  typename WP::CodeT ring[WRUN][NC];
  vec ra[WRUN][1];
  typename WP::Meta mc[NC], mn[NC];  // the meta of a run, double-buffered
  if (n > 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c) mn[c] = wp[c].load_meta(r0);
#pragma unroll
    for (int s = 0; s < WRUN; ++s) {
#pragma unroll
      for (int c = 0; c < NC; ++c) ring[s][c] = wp[c].load_codes(t0 + min(s, n - 1), lane);
      load_a<DT, AM_PACKED, 1, 1, WP>(rx, K, t0 + min(s, n - 1), lane, ra[s], none);
    }
    for (int i = 0; i < n; i += WRUN) {
      if (i % RUN == 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          mc[c] = mn[c];
          mn[c] = wp[c].load_meta(r0 + min(i / RUN + 1, (n - 1) / RUN));
        }
      }
#pragma unroll
      for (int s = 0; s < WRUN; ++s) {
        if (i + s < n) {  // wave-uniform
          const int slot = (i % RUN) + s;  // tile slot within the meta run
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            vec b[4];
            wp[c].raw_operands(ring[s][c], rq, b);
            float4_t at[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) at[j] = mfma16x16x32<DT>(ra[s][0], b[j], z4);
            vec bz[U];
            WP::zero_operands(mc[c], slot, rq, bz);
            float4_t az[U];
#pragma unroll
            for (int u = 0; u < U; ++u) az[u] = mfma16x16x32<DT>(ra[s][0], bz[u], z4);
            const float sf = WP::fold_scale(mc[c], slot, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float v01 = g0 ? at[1][e] : at[0][e], v23 = g0 ? at[3][e] : at[2][e];
              float zu[U];
#pragma unroll
              for (int u = 0; u < U; ++u) zu[u] = az[u][e];
              yf[c][e] = __builtin_fmaf(sf, (g1 ? v23 : v01) - sel_unit<U>(zu, lane), yf[c][e]);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < NC; ++c)
          ring[s][c] = wp[c].load_codes(t0 + min(i + s + WRUN, n - 1), lane);
        load_a<DT, AM_PACKED, 1, 1, WP>(rx, K, t0 + min(i + s + WRUN, n - 1), lane, ra[s], none);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // lane group g holds batch rows 0..3 of step g: add the 4 lane groups, then
  // the DW waves' partials through LDS in wave order
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      yf[c][e] += __shfl_xor(yf[c][e], 16, 64);
      yf[c][e] += __shfl_xor(yf[c][e], 32, 64);
    }
    *(float4_t*)(red + ((wave * NC + c) * 64 + lane) * 4) = yf[c];
  }
  __syncthreads();
  if (wave < NC && lane < 16) {
    const int c = wave;
    float4_t s4 = *(const float4_t*)(red + ((0 * NC + c) * 64 + lane) * 4);
#pragma unroll
    for (int w = 1; w < DW; ++w) {
      const float4_t v = *(const float4_t*)(red + ((w * NC + c) * 64 + lane) * 4);
      s4[0] += v[0];
      s4[1] += v[1];
      s4[2] += v[2];
      s4[3] += v[3];
    }
    const int col = (blockIdx.x * NC + c) * 16 + lane;
    if (col < N) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < M) out[(size_t)e * N + col] = round16<DT>(s4[e]);
    }
  }
}

template <int DT, int MT, int AM, int U, bool XS, int BITS, bool ONE>
__global__ void __launch_bounds__(64 * DW)
intb_decode_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ xsc,
                   const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                   const uint8_t* __restrict__ zeros, uint32_t zx,
                   const int32_t* __restrict__ perm, uint16_t* __restrict__ out, int M, int N,
                   int K, int KT) {
  __shared__ float red[DW * MT * 64 * 4];
  extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
  IntW<DT, U, BITS> wp;
  wp.codes = codes;
  wp.scales = scales;
  wp.zeros = zeros;
  wp.zx = zx;
  wp.KT = KT;
  decode_body<DT, MT, AM, XS, ONE>(x, xsc, wp, out, M, N, K, KT, red, perm, xlds);
}

template <int DT, int MT, int AM, bool BATCH, bool RP>
__device__ __forceinline__ void nf4_decode(const uint16_t* __restrict__ x,
                                           const uint8_t* __restrict__ q,
                                           const uint8_t* __restrict__ aq,
                                           const float* __restrict__ asc, const Nf4Table& L,
                                           uint16_t* __restrict__ out, int M, int N, int K,
                                           int KT) {
  __shared__ float red[DW * MT * 64 * 4];
  // the levels of every code byte (64 * DW == 256 threads, one entry each)
  __shared__ float2 lut2[256];
  static_assert(64 * DW == 256, "one thread per code byte");
  lut2[threadIdx.x] = make_float2(L.v[threadIdx.x & 15u], L.v[threadIdx.x >> 4]);
  __syncthreads();
  extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
  Nf4W<DT, BATCH, RP> wp;
  wp.q = q;
  wp.aq = aq;
  wp.asc = asc;
  wp.lut2 = lut2;
  decode_body<DT, MT, AM, false>(x, nullptr, wp, out, M, N, K, KT, red, nullptr, xlds);
}

template <int DT, int MT, int AM, bool BATCH>
__global__ void __launch_bounds__(64 * DW)
nf4_decode_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q,
                  const uint8_t* __restrict__ aq, const float* __restrict__ asc, Nf4Table L,
                  uint16_t* __restrict__ out, int M, int N, int K, int KT) {
  nf4_decode<DT, MT, AM, BATCH, false>(x, q, aq, asc, L, out, M, N, K, KT);
}

// The same on the repacked codes (nf4_repack).
template <int DT, int MT, int AM, bool BATCH>
__global__ void __launch_bounds__(64 * DW)
nf4r_decode_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q,
                   const uint8_t* __restrict__ aq, const float* __restrict__ asc, Nf4Table L,
                   uint16_t* __restrict__ out, int M, int N, int K, int KT) {
  nf4_decode<DT, MT, AM, BATCH, true>(x, q, aq, asc, L, out, M, N, K, KT);
}

// ---------------------------------------------------------------- planning --

// Raise a kernel's dynamic LDS limit to what a CU holds beside the kernel's
// static LDS, at most kMaxXldsOne (once per kernel; the call is idempotent,
// so a race between host threads is harmless).  A refusal is consumed here
// so it cannot be reported by a later launch: a launch that then asks for
// more than the old limit fails on its own.
static void allow_dynamic_lds(const void* kernel) {
  constexpr int kLdsPerCu = 160 * 1024;
  static thread_local const void* done[32];
  static thread_local int ndone = 0;
  for (int i = 0; i < ndone; ++i)
    if (done[i] == kernel) return;
  hipFuncAttributes fa{};
  int limit = (int)kMaxXlds;
  if (hipFuncGetAttributes(&fa, kernel) == hipSuccess)
    limit = (int)std::min<int64_t>(kMaxXldsOne, kLdsPerCu - (int64_t)fa.sharedSizeBytes);
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, limit) !=
      hipSuccess)
    (void)hipGetLastError();
  if (ndone < 32) done[ndone++] = kernel;
}

// Largest total of staged bytes (workgroups x bytes each) for which staging
// beats a separate preparation pass: every workgroup copies the rows (and the
// permutation and scales) from L2, so the cost grows with the grid, while the
// pass costs about one launch.  Measured on MI355X, whole calls in a graph,
// with the rows' DMA ahead of the code tiles and the rows permuted in place
// before the loop: staging saved 0.9 - 1.8 us on 4096 x 11008 at 2 - 4 rows
// (688 workgroups x up to 48 KB, 33 MB) and 1.7 us on 11008 x 4096 at 2 rows;
// it cost ~10 us on 5120 x 55296 layers (3456 workgroups).
constexpr int64_t kMaxStagedTotal = (int64_t)40 << 20;

// Activation mode and row tiles per workgroup row block for M rows of a
// [N, K] layer; gather: an act-order permutation is to be applied, xs: AWQ
// input scales.  For M <= 4 both are done on the rows staged in LDS when they
// fit and the grid is small enough (staging x alone does not beat per-tile
// loads).  Otherwise the caller prepares x first.  More rows: FULLT, except
// for at most 8 rows on layers of at most 4096 columns (at most one
// workgroup per CU, one wave per SIMD), where the transpose's LDS round trip
// is not hidden and the direct loads (fewer rows, fewer lines) are faster.
// Measured on MI355X, act-order whole calls, FULL -> FULLT: 11008 x 4096 at
// M = 5 14.8 -> 16.3 us, M = 8 15.9 -> 16.5, M = 12 17.8 -> 16.8, M = 16
// 19.3 -> 17.0; 4096 x 11008 at M = 8 16.6 -> 14.1; 5120 x 5120 at M = 12
// 13.6 -> 11.1; NF4 28672 x 8192 at M = 8 65.5 -> 54.1.
static int pick_mode(int64_t M, int64_t N, int64_t K, bool gather, bool xs, int* mt) {
  if (M <= 4) {
    *mt = 1;
    const int64_t wgs = ceil_div(N, 16);
    const int64_t lds = xlds_bytes((int)M, (int)K, gather, xs);
    const int64_t staged = xlds_staged_bytes((int)M, (int)K, gather, xs);
    if ((gather || xs) && lds <= (wgs <= 256 ? kMaxXldsOne : kMaxXlds) &&
        wgs * staged <= kMaxStagedTotal)
      return gather ? AM_XGATHER : AM_XSTAGED;
    return AM_PACKED;
  }
  *mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  return (M <= 8 && N <= 4096) ? AM_FULL : AM_FULLT;
}

// One decode launch.  a: the call's arguments (xsc non-null only when the
// kernel scales the activations itself).
struct DecodeArgs {
  const void *x, *xsc, *codes, *scales, *zeros;
  const int32_t* perm;
  void* out;
  int64_t M, N, K;
  hipStream_t stream;
  bool one, wide;  // the plan's one-row form and wide kernel
};

template <int DT, int MT, int AM, int U, bool XS, int BITS, bool ONE = false>
static void launch_intb_v(const DecodeArgs& a) {
  const dim3 grid((unsigned)ceil_div(a.N, 16), (unsigned)ceil_div(a.M, 16 * MT));
  const size_t lds = is_staged(AM) ? xlds_bytes((int)a.M, (int)a.K, AM == AM_XGATHER, XS)
                                   : (AM == AM_FULLT ? xpose_bytes(MT) : 0);
  if (lds) allow_dynamic_lds((const void*)intb_decode_kernel<DT, MT, AM, U, XS, BITS, ONE>);
  // a symmetric weight: the zeros descriptor gets an empty range over a valid
  // base and every zero field reads 0 ^ 2^(BITS-1)
  const uint32_t zx = a.zeros ? 0u : sym_zero_xor(BITS);
  launch_timed(intb_decode_kernel<DT, MT, AM, U, XS, BITS, ONE>, grid, dim3(64 * DW), lds, a.stream,
               (const uint16_t*)a.x, (const uint16_t*)a.xsc, (const uint8_t*)a.codes,
               (const uint8_t*)a.scales, (const uint8_t*)(a.zeros ? a.zeros : a.scales), zx,
               AM == AM_XGATHER || AM == AM_GGATHER ? a.perm : nullptr, (uint16_t*)a.out,
               (int)a.M, (int)a.N,
               (int)a.K, (int)(a.K / 128));
}

// Wide packed decode: 2 column tiles per wave, for 3 or 4 rows on layers of at
// least kWideMinN
// columns (measured on MI355X, 5120 x 55296: 50.4 -> 43.3 us per call at M = 4;
// within run-to-run noise at M = 2 and no gain at M = 1, where most of each
// activation load is rows past M; slower on 11008 columns, where half as many
// waves fill the GPU; 3 or 4 column tiles per wave were slower than 2).
template <int DT, int U, int BITS>
static void launch_intb_wide(const DecodeArgs& a) {
  constexpr int NC = 2, WR = RUN;
  const dim3 grid((unsigned)ceil_div(a.N, (int64_t)16 * NC));
  const uint32_t zx = a.zeros ? 0u : sym_zero_xor(BITS);
  launch_timed(intb_decode_wide_kernel<DT, U, BITS, NC, WR>, grid, dim3(64 * DW), 0, a.stream,
               (const uint16_t*)a.x, (const uint8_t*)a.codes, (const uint8_t*)a.scales,
               (const uint8_t*)(a.zeros ? a.zeros : a.scales), zx, (uint16_t*)a.out, (int)a.M,
               (int)a.N, (int)a.K, (int)(a.K / 128));
}

// A packed mode; one batch row takes the one-row form of the fold (measured on
// MI355X at M = 1, fp16, whole calls: 4096 x 11008 8.9 -> 8.5 us, 11008 x 4096
// 9.5 -> 8.9, 5120 x 55296 34.6 -> 33.3; a wave-uniform branch on M inside
// the loop instead gained nothing).
template <int DT, int AM, int U, bool XS, int BITS>
static void launch_intb_packed(const DecodeArgs& a) {
  if constexpr (IntW<DT, U, BITS>::kFold) {
    if (a.one) return launch_intb_v<DT, 1, AM, U, XS, BITS, true>(a);
  }
  launch_intb_v<DT, 1, AM, U, XS, BITS, false>(a);
}

template <int DT, int U, bool XS, int BITS>
static void launch_intb_mode(int am, int mt, const DecodeArgs& a) {
  if (am == AM_GGATHER) return launch_intb_v<DT, 1, AM_GGATHER, U, XS, BITS>(a);
  if (am == AM_XGATHER) return launch_intb_packed<DT, AM_XGATHER, U, XS, BITS>(a);
  if constexpr (XS) {
    launch_intb_packed<DT, AM_XSTAGED, U, true, BITS>(a);  // the only other mode that scales
  } else {
    if constexpr (IntW<DT, U, BITS>::kFold) {
      if (a.wide) return launch_intb_wide<DT, U, BITS>(a);
    }
    if (am == AM_PACKED) launch_intb_packed<DT, AM_PACKED, U, false, BITS>(a);
    else if (am == AM_TILED) {
      if (mt == 1) launch_intb_v<DT, 1, AM_TILED, U, false, BITS>(a);
      else if (mt == 2) launch_intb_v<DT, 2, AM_TILED, U, false, BITS>(a);
      else launch_intb_v<DT, 4, AM_TILED, U, false, BITS>(a);
    } else if (am == AM_FULL) launch_intb_v<DT, 1, AM_FULL, U, false, BITS>(a);
    else if (mt == 1) launch_intb_v<DT, 1, AM_FULLT, U, false, BITS>(a);
    else if (mt == 2) launch_intb_v<DT, 2, AM_FULLT, U, false, BITS>(a);
    else launch_intb_v<DT, 4, AM_FULLT, U, false, BITS>(a);
  }
}

template <int DT, bool XS, int BITS>
static void launch_intb_dt(int am, int mt, int G, const DecodeArgs& a) {
  const int U = units_per_tile(G);
  if (U == 1) launch_intb_mode<DT, 1, XS, BITS>(am, mt, a);
  else if (U == 2) launch_intb_mode<DT, 2, XS, BITS>(am, mt, a);
  else launch_intb_mode<DT, 4, XS, BITS>(am, mt, a);
}

// One decode launch of BITS-bit codes (instantiated once per width, each in
// its own translation unit).
template <int BITS>
void launch_intb_decode(int dtype, bool xs, int am, int mt, int G, const DecodeArgs& a) {
  if (dtype == DT_F16) {
    if (xs) launch_intb_dt<DT_F16, true, BITS>(am, mt, G, a);
    else launch_intb_dt<DT_F16, false, BITS>(am, mt, G, a);
  } else {
    if (xs) launch_intb_dt<DT_BF16, true, BITS>(am, mt, G, a);
    else launch_intb_dt<DT_BF16, false, BITS>(am, mt, G, a);
  }
}
extern template void launch_intb_decode<3>(int, bool, int, int, int, const DecodeArgs&);
extern template void launch_intb_decode<4>(int, bool, int, int, int, const DecodeArgs&);
extern template void launch_intb_decode<8>(int, bool, int, int, int, const DecodeArgs&);

}  // namespace w4a16

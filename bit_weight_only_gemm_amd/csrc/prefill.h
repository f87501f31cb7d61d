// prefill.h -- the large-M fused dequantize-and-multiply kernel template and
// its launchers, shared by the translation units that instantiate them (one
// per weight code width, compiled in parallel).  See prefill.hip for the
// design.
#pragma once
#include "common.h"
#include "kernels.h"
#include "launch.h"

namespace w4a16 {


constexpr int PF_WAVES = 4;                  // waves per workgroup
constexpr int PF_ROWB = 256;                 // LDS bytes of one row of a K tile
// Rows per workgroup BM in {32, 64, 128, 192, 256}: BM / 32 MFMA row tiles per wave,
// an LDS stage of BM x 256 bytes, BM / 16 16-byte activation loads per lane.

constexpr int PF_DMA_STEPS = 8;             // steps the activation loads spread over

typedef float float16_t __attribute__((ext_vector_type(16)));

template <int DT>
__device__ __forceinline__ float16_t mfma32x32x16(const typename Op<DT>::vec& a,
                                                  const typename Op<DT>::vec& b,
                                                  const float16_t& c);
template <>
__device__ __forceinline__ float16_t mfma32x32x16<DT_F16>(const half8_t& a, const half8_t& b,
                                                          const float16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ float16_t mfma32x32x16<DT_BF16>(const bf16x8_t& a, const bf16x8_t& b,
                                                           const float16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16 bytes per lane from a buffer straight into LDS: lane l's data lands at
// lds + 16 l (the LDS base is wave-uniform).
__device__ __forceinline__ void lds_dma16(rsrc_t r, uint8_t* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// TAIL: the row block may hold fewer than BM rows; the row of each load is
// then part of the per-lane offset so that rows past M read 0 (a launch of
// this form may also cover whole row blocks).  Full blocks put it in the
// scalar offset (fewer registers).  Row block of a workgroup: rb0 +
// blockIdx.y.
// Split-K: workgroup z of S takes K tiles [z KT / S, (z + 1) KT / S) and, when
// S > 1, writes its fp32 partial tile to part[z][M][N] for split_reduce_kernel.
//
// Weight formats (FMT): INT4 reads the repacked tiles as above.  NF4 reads the
// canonical layout (row n: K / 2 bytes, element 2 j in the low nibble of byte
// j): for K tile t, lane l loads the 32 bytes holding inputs
// 128 t + 64 (l >> 5) .. + 63 of its column, one 64-element absmax block, and
// word j of them is the B operand of step j; the activation operand of step j
// is then chunk 8 (l >> 5) + j of the tile (the K order inside a tile is the
// same permutation on both sides).  Dequant: w = round16(L[c] * a'), a' =
// absmax_q * absmax_scale, L from LDS.  NF4 here needs K % 128 == 0.
// NF4R: NF4 with the codes re-laid once into the tiles of the integer
// formats' code layout (16 rows x 128 inputs, 1 KB, lane r holding bytes
// 64 t + 16 (r >> 4) .. + 15 of row r & 15): lane l's 32 bytes are then the
// 16-byte chunks of repacked lanes (l & 15) + 32 (l >> 5) and + 16.
enum { FMT_INT4 = 0, FMT_NF4 = 1, FMT_NF4R = 2 };
constexpr bool is_nf4_fmt(int fmt) { return fmt != FMT_INT4; }

// INT codes of BITS bits (3, 4 or 8; the Codes<BITS> forms of common.h): a
// column tile's K tile is 256 BITS bytes, repacked lane r's codes at 12 r
// (3 bits), 16 r (4 bits), or 16 r and 1024 + 16 r (8 bits).
template <int DT, int BM, bool TAIL, int FMT, int U, int BITS>
__global__ void __launch_bounds__(64 * PF_WAVES) __attribute__((amdgpu_waves_per_eu(1, 1)))
wq_prefill_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
                  const uint8_t* __restrict__ scales, const uint8_t* __restrict__ zeros,
                  uint32_t zx, Nf4Table L, uint16_t* __restrict__ out,
                  float* __restrict__ part, int M, int N, int K, int KT, int NP, int S,
                  int rb0) {
  typedef typename Op<DT>::vec vec;
  typedef Codes<is_nf4_fmt(FMT) ? 4 : BITS> CT;     // NF4: its 16-byte loads as Codes<4>
  constexpr int kTile = 256 * BITS;                 // INT: bytes per column tile, K tile
  constexpr int kZW = zero_field_bits(BITS);        // INT: zero field width
  constexpr int kZWords = U * kZW / 4;              // INT: zero dwords per column and run
  // NF4: the levels of every code byte, one entry per thread
  __shared__ float2 lut2[256];
  static_assert(64 * PF_WAVES == 256, "one thread per code byte");
  if (is_nf4_fmt(FMT)) lut2[threadIdx.x] = make_float2(L.v[threadIdx.x & 15u], L.v[threadIdx.x >> 4]);
  constexpr int PF_BM = BM;
  constexpr int PF_MT = BM / 32;
  constexpr int PF_STAGE = BM * PF_ROWB;
  constexpr int PF_ALD = BM * 16 / (64 * PF_WAVES);
  __shared__ __attribute__((aligned(16))) uint8_t As[2 * PF_STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = (rb0 + (int)blockIdx.y) * PF_BM;
  const int z = blockIdx.z;
  const int tb = (int)((int64_t)z * KT / S), te = (int)((int64_t)(z + 1) * KT / S);
  const int p = blockIdx.x * PF_WAVES + wave;  // this wave's 64-column panel
  const int KT8 = (KT + 7) >> 3;
  const int i16 = lane & 15, h = lane >> 5;

  // ---- activations: rows row0 .. row0 + vrows - 1 of x; rows past M read 0.
  // Instruction i of wave w fills the 1 KB LDS block 4 i + w (rows
  // 16 i + 4 w .. + 3), lane l writing position (l & 15) of row
  // 16 i + 4 w + (l >> 4), which holds chunk (l & 15) ^ (row & 15): the
  // swizzle is applied on the global side.
  const int vrows = min(PF_BM, M - row0);
  const rsrc_t rx = make_rsrc(x + (size_t)row0 * K, (uint32_t)vrows * (uint32_t)K * 2u);
  const uint32_t arow_bytes = (uint32_t)K * 2u;
  const int arow0 = 4 * wave + (lane >> 4);  // row & 15 of every instruction's row
  const uint32_t avoff = (uint32_t)arow0 * arow_bytes + (uint32_t)((i16 ^ arow0) << 4);
  const uint32_t astride = 16u * arow_bytes;

  // ---- weights of panel p (all loads return 0 for a panel past the last).
  // Column group g (32 columns): column tile 2 g + ((l & 31) >> 4), entry
  // l & 15 of its meta.
  const bool pv = p < NP;
  const size_t pp = pv ? (size_t)p : 0;
  rsrc_t rc, rs, rz;
  uint32_t vcode[2][2], vmeta[2], gblk[2];
  if constexpr (FMT == FMT_INT4) {
    rc = make_rsrc(codes + pp * KT * 4 * kTile, pv ? (uint32_t)KT * 4u * kTile : 0u);
    rs = make_rsrc(scales + pp * KT8 * 1024 * U, pv ? (uint32_t)KT8 * 1024u * U : 0u);
    rz = make_rsrc(zeros + pp * KT8 * 256 * kZWords,
                   pv && !zx ? (uint32_t)KT8 * 256u * kZWords : 0u);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int ct = 2 * g + ((lane & 31) >> 4);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        vcode[g][h2] =
            (uint32_t)(ct * kTile + (i16 + 16 * (2 * h2 + h)) * (BITS == 3 ? 12 : 16));
      vmeta[g] = (uint32_t)(ct * 16 + i16);
    }
  } else {
    // rows of this panel (N % 16 == 0; rows past N read 0 -> a' = 0)
    const int nrows = pv ? min(64, N - p * 64) : 0;
    const uint32_t Kb = (uint32_t)K / 2u, Kblk = (uint32_t)K / 64u;
    if constexpr (FMT == FMT_NF4R)
      rc = make_rsrc(codes + pp * 4 * KT * 1024, (uint32_t)(nrows / 16) * (uint32_t)KT * 1024u);
    else
      rc = make_rsrc(codes + pp * 64 * Kb, (uint32_t)nrows * Kb);
    rs = make_rsrc(scales + pp * 64 * Kblk, (uint32_t)nrows * Kblk);
    rz = make_rsrc(zeros, (uint32_t)(((int64_t)N * Kblk + 255) / 256 * 4));
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int c = 32 * g + (lane & 31);
      if constexpr (FMT == FMT_NF4R) {
        vcode[g][0] = (uint32_t)(((c >> 4) * KT * 64 + i16 + 32 * h) * 16);
        vcode[g][1] = vcode[g][0] + 256u;
      } else {
        vcode[g][0] = (uint32_t)c * Kb + 32u * (uint32_t)h;
        vcode[g][1] = vcode[g][0] + 16u;
      }
      vmeta[g] = (uint32_t)c * Kblk + (uint32_t)h;
      gblk[g] = (uint32_t)(pp * 64 + c) * Kblk + (uint32_t)h;
    }
  }
  // the weights and meta of K tile t for column group g.  INT: sa holds the U
  // scales of the tile (units (t & 7) U .. of the run, 2 U bytes), za the zero
  // dword holding their fields (XORed with zx where they are used, so that no
  // instruction needs a load's result before then).
  auto load_w = [&](int t, int g, CT (&w)[2], u32x2_t& sa, uint32_t& za) {
    if constexpr (FMT == FMT_INT4) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        if constexpr (BITS == 4) {
          w[h2].w = bld128(rc, vcode[g][h2], t * 4 * kTile);
        } else if constexpr (BITS == 3) {
          w[h2].w = bld96(rc, vcode[g][h2], t * 4 * kTile);
        } else {
          w[h2].lo = bld128(rc, vcode[g][h2], t * 4 * kTile);
          w[h2].hi = bld128(rc, vcode[g][h2] + 1024u, t * 4 * kTile);
        }
      }
      const int sb = (t >> 3) * 1024 * U + (t & 7) * 2 * U;
      if constexpr (U == 1) sa = u32x2_t{bld16(rs, vmeta[g] * 16u, sb), 0u};
      else if constexpr (U == 2) sa = u32x2_t{bld32(rs, vmeta[g] * 32u, sb), 0u};
      else sa = bld64(rs, vmeta[g] * 64u, sb);
      za = bld32(rz, vmeta[g] * 4u * kZWords,
                 (t >> 3) * 256 * kZWords + (((t & 7) * U * kZW) >> 5) * 4);
    } else {
      constexpr int kStep = FMT == FMT_NF4R ? 1024 : 64;  // bytes per K tile
      w[0].w = bld128(rc, vcode[g][0], t * kStep);
      w[1].w = bld128(rc, vcode[g][1], t * kStep);
      sa = u32x2_t{__builtin_amdgcn_raw_buffer_load_b8(rs, vmeta[g], 2 * t, 0), 0u};
      za = bld32(rz, ((gblk[g] + 2u * (uint32_t)t) >> 8) * 4u, 0);
    }
  };

  float16_t acc[PF_MT][2];
#pragma unroll
  for (int m = 0; m < PF_MT; ++m)
#pragma unroll
    for (int g = 0; g < 2; ++g) acc[m][g] = float16_t{};
  // FOLD (integer codes, one scale and zero per K tile, 32 rows): the B
  // operands are the codes alone (RawQ: o + q, o = 1024 in fp16, 128 in
  // bf16), summed over the tile into accT; accZ sums the products of the same
  // activations with the zero operand (o + z) of each column group.  At the
  // end of the tile
  //   acc += s (accT - accZ) = s sum_k x_k (q_k - z),
  // a subtract and a multiply-add per accumulator per tile in place of the
  // scale and zero in every operand: the dequant VALU per weight drops to the
  // insert.  The result differs from dequant-then-multiply by the rounding of
  // each weight to 16 bits, which this form never does (a one-hot row still
  // gives round16((q - z) s) exactly), and by the rounding of the two sums;
  // where every code of a column's tile equals its zero the two MFMA chains
  // see identical inputs and the tile adds exactly 0.
  constexpr bool FOLD = FMT == FMT_INT4 && U == 1 && BM == 32 && !(BITS == 8 && DT == DT_BF16);
  float16_t accT[FOLD ? PF_MT : 1][2], accZ[FOLD ? PF_MT : 1][2];
  const RawQ<DT> rq;

  // DEEP (32 rows): the weights of K tile t + 2 are in flight while
  // tile t is computed (two tiles of latency cover; with few rows a tile's
  // compute is short).  The weight registers are a ring of three slots, the
  // tile loop unrolled by three so that no in-flight register is copied.  The
  // activations of tile t + 1 are issued first, all at once (BM / 16 loads per
  // lane), then the weights of tile t + 2; the wait before each barrier
  // counts in issue order, so it leaves those kW loads pending (the barrier is
  // a plain s_barrier: __syncthreads would wait for every load).
  constexpr bool DEEP = BM == 32;
  constexpr int kW = 2 * ((is_nf4_fmt(FMT) ? 2 : (BITS == 8 ? 4 : 2)) + 2);  // loads per load_w pair
  CT cw[DEEP ? 3 : 2][2][2];
  u32x2_t sc[DEEP ? 3 : 2][2];
  uint32_t zz[DEEP ? 3 : 2][2];

  // ---- prologue: K tile tb (and, DEEP, the weights of tile tb + 1)
#pragma unroll
  for (int g = 0; g < 2; ++g) load_w(tb, g, cw[0][g], sc[0][g], zz[0][g]);
  if constexpr (DEEP) {
#pragma unroll
    for (int g = 0; g < 2; ++g) load_w(min(tb + 1, te - 1), g, cw[1][g], sc[1][g], zz[1][g]);
  }
#pragma unroll
  for (int i = 0; i < PF_ALD; ++i)
    lds_dma16(rx, As + (4 * i + wave) * 1024, TAIL ? avoff + (uint32_t)i * astride : avoff,
              TAIL ? tb * 256 : (int)((uint32_t)i * astride) + tb * 256);
  __syncthreads();

  // B operand of step s for column group g from the weight slot (cwx, scx,
  // zzx) of a K tile whose first meta unit is zero field zbx (NF4: a' = apx):
  // word j = s >> 1 of the tile, in meta unit j U / 4.  The unit's dequant
  // parameters are formed at the step (a few VALU instructions between MFMAs);
  // formed once per tile and held across it they made the small-M launches of
  // this kernel markedly slower.
  auto operand_of = [&](int s, int g, const CT (&cwx)[2][2], const u32x2_t (&scx)[2],
                        const uint32_t (&zzx)[2], int zbx, float apx) -> vec {
    if constexpr (FOLD) {
      return dequant_step<DT, false>(cwx[g][s & 1], s >> 1, rq);
    } else if constexpr (FMT == FMT_INT4) {
      const int u = (s >> 1) * U / 4;
      QParam<DT> q;
      q.template set<BITS == 4>((scx[g][u >> 1] >> (16 * (u & 1))) & 0xFFFFu,
                                ((zzx[g] ^ zx) >> (kZW * (zbx + u))) & ((1u << kZW) - 1u));
      return dequant_step<DT, false>(cwx[g][s & 1], s >> 1, q);
    } else {
      return nf4_pair_operand<DT>(cwx[g][s >> 2].w[s & 3], lut2, apx);
    }
  };
  auto zb_of = [&](int t) { return ((t & 7) * U) % (32 / kZW); };  // zero field of tile t's first unit
  auto ap_of = [&](const u32x2_t (&scx)[2], const uint32_t (&zzx)[2], int g) {
    return (float)(scx[g][0] & 0xFFu) * __builtin_bit_cast(float, zzx[g]);
  };
  // XPIPE (the two-stage tile loop): the step-0 B operands of tile t + 1 are
  // dequantized during step 7 of tile t, between its MFMAs, and carried across
  // the barrier in bcar, so a tile starts with its MFMAs instead of a dequant
  // that nothing overlaps (per-tile timestamps on MI355X, 256 rows: 0.5 of
  // 3.0 us went to that preamble).
  constexpr bool XPIPE = !DEEP;
  vec bcar[2];
  if constexpr (XPIPE) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
      bcar[g] = operand_of(0, g, cw[0], sc[0], zz[0], zb_of(tb),
                           is_nf4_fmt(FMT) ? ap_of(sc[0], zz[0], g) : 0.f);
  }

  // One K tile: compute tile t from the weight slot (cwc, scc, zzc) while the
  // weights of tile t + 1 (t + 2 when DEEP) are loaded into (cwn, scn, zzn).
  auto tile = [&](const int t, CT (&cwc)[2][2], u32x2_t (&scc)[2], uint32_t (&zzc)[2],
                  CT (&cwn)[2][2], u32x2_t (&scn)[2], uint32_t (&zzn)[2]) {
    // ---- issue K tile t + 1 (the last tile is re-read on the final pass);
    // its activations go to LDS stage (t - tb + 1) & 1, last read before the
    // previous barrier
    const int tn = min(t + 1, te - 1);
    uint8_t* sw = As + ((t - tb + 1) & 1) * PF_STAGE;
    auto issue_dma = [&](int i) {
      lds_dma16(rx, sw + (4 * i + wave) * 1024, TAIL ? avoff + (uint32_t)i * astride : avoff,
                TAIL ? tn * 256 : (int)((uint32_t)i * astride) + tn * 256);
    };
    if constexpr (DEEP) {
#pragma unroll
      for (int i = 0; i < PF_ALD; ++i) issue_dma(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 2; ++g) load_w(min(t + 2, te - 1), g, cwn[g], scn[g], zzn[g]);
    }
    // otherwise the weights of tile t + 1 are loaded in step 0 and its
    // activation loads spread over the first PF_DMA_STEPS steps of tile t, each
    // load between two MFMAs (a burst of them at the start of the tile stalls
    // the issuing wave behind the address queue while the matrix pipe idles)
    __builtin_amdgcn_sched_barrier(0);

    // ---- K tile t from LDS stage t & 1: 8 steps of 16 inputs.  Per step the
    // operand reads come first; the dequant of the next step's B operand is
    // spread between the step's MFMAs (each 32 x 32 x 16 MFMA keeps the matrix
    // pipe busy long enough to issue several VALU instructions behind it).
    float ap[2];  // NF4: a' of this lane's block
    const int zb = zb_of(t);
    if constexpr (is_nf4_fmt(FMT)) {
#pragma unroll
      for (int g = 0; g < 2; ++g) ap[g] = ap_of(scc, zzc, g);
    }
    vec bz[2];  // FOLD: the zero operand (o + z) of each column group
    if constexpr (FOLD) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
        bz[g] = rq.template zero_operand<BITS>(((zzc[g] ^ zx) >> (kZW * zb)) & ((1u << kZW) - 1u));
    }
    auto operand = [&](int s, int g) -> vec {
      return operand_of(s, g, cwc, scc, zzc, zb, is_nf4_fmt(FMT) ? ap[g] : 0.f);
    };
    const uint8_t* st = As + ((t - tb) & 1) * PF_STAGE;
    auto read_step = [&](int s, vec (&a)[PF_MT]) {
      // 8-element chunk of this lane's inputs in step s
      const int q = FMT == FMT_INT4 ? 2 * s + h : 8 * h + s;
#pragma unroll
      for (int m = 0; m < PF_MT; ++m)
        a[m] = *(const vec*)(st + (m * 32 + (lane & 31)) * PF_ROWB + ((q ^ i16) << 4));
    };
    vec b[2], a[PF_MT];
#pragma unroll
    for (int g = 0; g < 2; ++g) b[g] = XPIPE ? bcar[g] : operand(0, g);
    read_step(0, a);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      vec bn[2], an[PF_MT];
      // loads i with i * PF_DMA_STEPS / PF_ALD == s go out in step s
      const int i0 = (s * PF_ALD + PF_DMA_STEPS - 1) / PF_DMA_STEPS;
      const int i1 = ((s + 1) * PF_ALD + PF_DMA_STEPS - 1) / PF_DMA_STEPS;
      if constexpr (!DEEP) {
#pragma unroll
        for (int i = i0; i < i1 && i < PF_ALD; ++i) issue_dma(i);
        if (s == 0) {
#pragma unroll
          for (int g = 0; g < 2; ++g) load_w(tn, g, cwn[g], scn[g], zzn[g]);
        }
      }
      // memory loads of this step, one after each of the first MFMAs
      const int nvm = (i0 < PF_ALD ? min(i1, PF_ALD) - i0 : 0) + (!DEEP && s == 0 ? kW : 0);
      if (s < 7) {
        const int sn1 = s + 1;
        read_step(sn1, an);
#pragma unroll
        for (int g = 0; g < 2; ++g) bn[g] = operand(sn1, g);
      } else if constexpr (XPIPE) {
        // step 0 of tile t + 1 (on the last tile: a re-read of it, unused)
        const int zbn = zb_of(t + 1);
#pragma unroll
        for (int g = 0; g < 2; ++g)
          bn[g] = operand_of(0, g, cwn, scn, zzn, zbn, is_nf4_fmt(FMT) ? ap_of(scn, zzn, g) : 0.f);
      }
      if constexpr (FOLD) {
#pragma unroll
        for (int m = 0; m < PF_MT; ++m) {
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            accT[m][g] = mfma32x32x16<DT>(a[m], b[g], s == 0 ? float16_t{} : accT[m][g]);
            accZ[m][g] = mfma32x32x16<DT>(a[m], bz[g], s == 0 ? float16_t{} : accZ[m][g]);
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < PF_MT; ++m)
#pragma unroll
          for (int g = 0; g < 2; ++g) acc[m][g] = mfma32x32x16<DT>(a[m], b[g], acc[m][g]);
      }
      if (s < 7 || XPIPE) {
#pragma unroll
        for (int k = 0; k < (FOLD ? 4 : 2) * PF_MT; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          if (!DEEP && k < nvm)
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one memory load
          // the next step's operand reads early, 4 after each of the first
          // MFMAs, so they have landed when that step starts (one read per
          // MFMA left the last ones in flight there: whole calls at M = 2048
          // 1-3 % slower on MI355X)
          if (s < 7 && k < (PF_MT + 3) / 4) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // up to 4 VALU
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (s < 7) {
#pragma unroll
        for (int g = 0; g < 2; ++g) b[g] = bn[g];
#pragma unroll
        for (int m = 0; m < PF_MT; ++m) a[m] = an[m];
      } else if constexpr (XPIPE) {
#pragma unroll
        for (int g = 0; g < 2; ++g) bcar[g] = bn[g];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FOLD) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const float sf = (float)__builtin_bit_cast(_Float16, (uint16_t)(scc[g][0] & 0xFFFFu));
#pragma unroll
        for (int m = 0; m < PF_MT; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[m][g][r] = __builtin_fmaf(sf, accT[m][g][r] - accZ[m][g][r], acc[m][g][r]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DEEP) {
      // this wave's activation loads of tile t + 1 are complete (only the kW
      // weight loads of tile t + 2, issued after them, may be pending), then
      // every wave's; the memory clobber keeps LDS accesses on their side
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kW) : "memory");
    }
  };

  if constexpr (DEEP) {
    for (int t = tb; t < te; t += 3) {
      tile(t, cw[0], sc[0], zz[0], cw[2], sc[2], zz[2]);
      if (t + 1 < te) tile(t + 1, cw[1], sc[1], zz[1], cw[0], sc[0], zz[0]);
      if (t + 2 < te) tile(t + 2, cw[2], sc[2], zz[2], cw[1], sc[1], zz[1]);
    }
  } else {
    for (int t = tb; t < te; ++t) {
      tile(t, cw[0], sc[0], zz[0], cw[1], sc[1], zz[1]);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) cw[0][g][h2] = cw[1][g][h2];
        sc[0][g] = sc[1][g];
        zz[0][g] = zz[1][g];
      }
      __syncthreads();  // the LDS writes of tile t + 1 are complete (vmcnt) and visible
    }
  }

  // ---- epilogue: register r of lane l is row (r & 3) + 4 (l >> 5) + 8 (r >> 2),
  // column l & 31 of the 32 x 32 tile
  float* pz = part + (size_t)z * M * N;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int col = p * 64 + g * 32 + (lane & 31);
    if (col < N) {
#pragma unroll
      for (int m = 0; m < PF_MT; ++m) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + m * 32 + (r & 3) + 4 * h + 8 * (r >> 2);
          if (row < M) {
            if (S == 1)
              out[(size_t)row * N + col] = round16<DT>(acc[m][g][r]);
            else
              pz[(size_t)row * N + col] = acc[m][g][r];
          }
        }
      }
    }
  }
}

// out = round16(sum_z part[z]) over the S split-K partials, added in z order
// (bitwise reproducible); 4 consecutive outputs per thread.
template <int DT>
__global__ void __launch_bounds__(256)
split_reduce_kernel(const float* __restrict__ part, int S, int64_t MN, uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= MN) return;
  float4_t s = *(const float4_t*)(part + i);
  for (int z = 1; z < S; ++z) {
    const float4_t v = *(const float4_t*)(part + (size_t)z * MN + i);
    s[0] += v[0];
    s[1] += v[1];
    s[2] += v[2];
    s[3] += v[3];
  }
  const uint32_t lo = (uint32_t)round16<DT>(s[0]) | ((uint32_t)round16<DT>(s[1]) << 16);
  const uint32_t hi = (uint32_t)round16<DT>(s[2]) | ((uint32_t)round16<DT>(s[3]) << 16);
  *(uint2*)(out + i) = make_uint2(lo, hi);
}

template <int DT, int BM, int FMT, int U, int BITS>
static void launch_prefill_bm(const void* x, const void* codes_r, const void* scales_r,
                              const void* zeros_r, const Nf4Table& L, void* out, float* part,
                              int S, bool single, int64_t M, int64_t N, int64_t K,
                              hipStream_t stream) {
  const int64_t NP = ceil_div(N, 64);
  const int KT = (int)(K / 128);
  const unsigned gx = (unsigned)ceil_div(NP, PF_WAVES);
  // single: every row block in one launch of the ragged-tail form
  const int64_t full = single ? 0 : M / BM;
  const int64_t tail_rb0 = full, tail_blocks = single ? ceil_div(M, (int64_t)BM) : 1;
  // INT codes without zeros (symmetric): an empty zeros range over a valid
  // base, every zero field read as 0 ^ 2^(BITS-1)
  const uint32_t zx = (FMT == FMT_INT4 && !zeros_r) ? sym_zero_xor(BITS) : 0u;
  const uint8_t* zp = (const uint8_t*)(zeros_r ? zeros_r : scales_r);
  // the timing events (if set) go to the first launch
  if (full > 0)
    launch_timed(wq_prefill_kernel<DT, BM, false, FMT, U, BITS>,
                 dim3(gx, (unsigned)full, (unsigned)S), dim3(64 * PF_WAVES), 0, stream,
                 (const uint16_t*)x, (const uint8_t*)codes_r, (const uint8_t*)scales_r, zp, zx, L,
                 (uint16_t*)out, part, (int)M, (int)N, (int)K, KT, (int)NP, S, 0);
  if (single || M % BM)
    launch_timed(wq_prefill_kernel<DT, BM, true, FMT, U, BITS>,
                 dim3(gx, (unsigned)tail_blocks, (unsigned)S), dim3(64 * PF_WAVES), 0, stream,
                 (const uint16_t*)x, (const uint8_t*)codes_r, (const uint8_t*)scales_r, zp, zx, L,
                 (uint16_t*)out, part, (int)M, (int)N, (int)K, KT, (int)NP, S, (int)tail_rb0);
  if (S > 1) {
    const int64_t MN = M * N;
    hipLaunchKernelGGL(split_reduce_kernel<DT>, dim3((unsigned)ceil_div(MN / 4, (int64_t)256)),
                       dim3(256), 0, stream, (const float*)part, S, MN, (uint16_t*)out);
  }
}

template <int DT, int FMT, int U, int BITS>
static void launch_prefill_dt(const void* x, const void* codes_r, const void* scales_r,
                              const void* zeros_r, const Nf4Table& L, void* out, void* ws,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const PrefillPlan pl = plan_prefill(M, N, K, ws != nullptr);
  float* part = (float*)ws;
  if (pl.bm == 32)
    launch_prefill_bm<DT, 32, FMT, U, BITS>(x, codes_r, scales_r, zeros_r, L, out, part,
                                           pl.splits, pl.single, M, N, K, stream);
  else if (pl.bm == 64)
    launch_prefill_bm<DT, 64, FMT, U, BITS>(x, codes_r, scales_r, zeros_r, L, out, part,
                                           pl.splits, pl.single, M, N, K, stream);
  else if (pl.bm == 128)
    launch_prefill_bm<DT, 128, FMT, U, BITS>(x, codes_r, scales_r, zeros_r, L, out, part,
                                           pl.splits, pl.single, M, N, K, stream);
  else if (pl.bm == 192)
    launch_prefill_bm<DT, 192, FMT, U, BITS>(x, codes_r, scales_r, zeros_r, L, out, part,
                                           pl.splits, pl.single, M, N, K, stream);
  else
    launch_prefill_bm<DT, 256, FMT, U, BITS>(x, codes_r, scales_r, zeros_r, L, out, part,
                                           pl.splits, pl.single, M, N, K, stream);
}

template <int DT, int BITS>
static void launch_intb_prefill_dt(const void* x, const void* codes_r, const void* scales_r,
                                   const void* zeros_r, void* out, void* ws, int64_t M,
                                   int64_t N, int64_t K, int G, hipStream_t stream) {
  const Nf4Table none{};
  const int U = units_per_tile(G);
  if (U == 1)
    launch_prefill_dt<DT, FMT_INT4, 1, BITS>(x, codes_r, scales_r, zeros_r, none, out, ws, M, N,
                                             K, stream);
  else if (U == 2)
    launch_prefill_dt<DT, FMT_INT4, 2, BITS>(x, codes_r, scales_r, zeros_r, none, out, ws, M, N,
                                             K, stream);
  else
    launch_prefill_dt<DT, FMT_INT4, 4, BITS>(x, codes_r, scales_r, zeros_r, none, out, ws, M, N,
                                             K, stream);
}

// The large-M kernel for BITS-bit codes (instantiated once per width, each in
// its own translation unit).
template <int BITS>
void launch_intb_prefill(const void* x, const void* codes_r, const void* scales_r,
                         const void* zeros_r, void* out, void* ws, int64_t M, int64_t N,
                         int64_t K, int G, int dtype, hipStream_t stream) {
  if (dtype == DT_F16)
    launch_intb_prefill_dt<DT_F16, BITS>(x, codes_r, scales_r, zeros_r, out, ws, M, N, K, G,
                                         stream);
  else
    launch_intb_prefill_dt<DT_BF16, BITS>(x, codes_r, scales_r, zeros_r, out, ws, M, N, K, G,
                                          stream);
}
#define W4A16_PREFILL_ARGS \
  const void*, const void*, const void*, const void*, void*, void*, int64_t, int64_t, int64_t, \
      int, int, hipStream_t
extern template void launch_intb_prefill<3>(W4A16_PREFILL_ARGS);
extern template void launch_intb_prefill<4>(W4A16_PREFILL_ARGS);
extern template void launch_intb_prefill<8>(W4A16_PREFILL_ARGS);

}  // namespace w4a16

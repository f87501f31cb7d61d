// gemm.hip -- fused dequantize-and-multiply kernels (INT4 and NF4) for gfx950.
//
// The method is the fused kernel of [P5] "LLM量化技术深度对比..." "关键数据解读"
// item 1: the 4-bit weights are turned into 16-bit values in registers right
// before the multiply and are never written back to memory, so each call moves
// only the 4-bit codes plus their scales (decode time tracks weight bytes,
// item 3 of the same section).
//
// Skinny-M kernel (decode), memory bound:
//  * One workgroup of DW waves per 16-column MFMA tile (and per block of 16*MT
//    rows).  The waves split the K tiles of 128 between them in runs of 8
//    tiles (intra-workgroup split-K); each wave keeps fp32 accumulators in
//    registers and the partial tiles are added in wave order through LDS at
//    the end -- a fixed order, so results are bitwise reproducible and no
//    global reduction, atomic or fence is needed.
//  * The load pipe, not HBM, is what a naive version of this loop saturates:
//    every wave64 vector-memory instruction costs the CU's load path about
//    the same whatever its active lanes.  So per K tile a wave issues one
//    16-byte-per-lane load of codes (a contiguous, coalesced 1 KB tile), the
//    scales and zeros come once per run of 8 tiles (for G >= 128 one 16-byte
//    and one 4-byte load per lane), and for M <= 4 one 16-byte load per lane
//    carries the activations of all 4 MFMA steps of the tile (see "packed"
//    below).
//  * Each 32-bit code word becomes an 8-element MFMA operand, multiplied with
//    v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulation.  For M <= 4 (integer
//    codes) it is the codes alone, o + q, and each lane applies the scale and
//    zero of its column and MFMA step after the step's MFMA, with the step's
//    activation row sums from one more MFMA against ones: the same real
//    products without a 16-bit rounding of each weight, and far fewer VALU
//    instructions per code.  For 5..16 rows with G >= 128 the same is done
//    per K tile (FULLT mode, below); otherwise the code word is dequantized
//    exactly (the routine the dequant export uses).
//  * "Packed" activations (M <= 4): the 16 A-operand rows are 4 K-steps x 4
//    batch rows (row 4j + m holds step j of batch row m), so one load feeds
//    the 4 MFMAs of a tile; step j accumulates into its own tile acc[j], whose
//    rows 4j .. 4j+3 are the wanted products (the other rows mix steps and are
//    dropped).  At the end a cross-lane shuffle adds the 4 step tiles.
//  * Full rows (M > 4): 16 A-operand rows per row tile.  The MFMA layout puts
//    row l & 15 in lane l, so direct 16-byte loads touch 16 rows x 64 bytes
//    each; the FULLT mode instead loads whole 128-byte lines (lane l: chunk
//    l & 15 of row 4i + (l >> 4)) and transposes them through a swizzled
//    4 KB of LDS per wave and row tile.  Direct loads remain for at most 8
//    rows on layers of at most 4096 columns.
//  * Latency hiding: a ring of 8 tiles of codes (and of activations) is in
//    flight per wave.  All loads are buffer loads with per-lane offsets fixed
//    and the tile index in the wave-uniform offset, so the loop has no
//    divergent branch and no load result merges through a branch (either
//    would make the compiler drain every outstanding load per tile); rows
//    >= M read 0 through the descriptor range.
//  * Act-order permutation and AWQ input scales: for M <= 4 rows and a small
//    enough grid every workgroup stages the rows (with the permutation and/or
//    the scales) in LDS, divides them by the scales once and gathers
//    x[m][perm[k]] from there; otherwise a small preparation kernel writes
//    x[:, perm] / s into the workspace first and the GEMM streams contiguous
//    rows.
//  * Group sizes below 128 (U = 128 / G meta units per K tile) read U times the
//    scales and zeros per run; a symmetric weight reads no zeros at all.
#include "decode.h"

namespace w4a16 {

// Timing events for the next main-kernel launch on this host thread (set by
// w4a16_set_timing_events; consumed by one launch).
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

void set_timing_events(hipEvent_t a, hipEvent_t b) {
  t_ev_start = a;
  t_ev_stop = b;
}

// Activation preparation pass: x_p[m, k] = x[m, perm[k]] (perm may be null:
// identity), divided by the AWQ input scale s[perm[k]] when xsc is given (the
// same rounding as the fused loads).  One thread per 8 consecutive columns.
template <int DT>
__global__ void __launch_bounds__(256)
prep_x_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
              const uint16_t* __restrict__ xsc, uint16_t* __restrict__ xp, int M, int K) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = K >> 3;
  if (idx >= (int64_t)M * per_row) return;
  const int64_t m = idx / per_row;
  const int k = (int)(idx - m * per_row) * 8;
  const uint16_t* xr = x + m * K;
  int src[8];
  if (perm) {
    const int4* pp = (const int4*)(perm + k);
    const int4 p0 = pp[0], p1 = pp[1];
    src[0] = p0.x; src[1] = p0.y; src[2] = p0.z; src[3] = p0.w;
    src[4] = p1.x; src[5] = p1.y; src[6] = p1.z; src[7] = p1.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) src[e] = k + e;
  }
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = xr[src[e]];
    if (xsc) h[e] = div_scale1<DT>((uint16_t)h[e], xsc[src[e]]);
  }
  u32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = h[2 * i] | (h[2 * i + 1] << 16);
  *(u32x4_t*)(xp + m * K + k) = v;
}

// Workspace layout: the prepared activations (when they are permuted and/or
// divided by the AWQ input scales in a separate pass), then the large-M
// kernel's split-K partials (when it splits K).  The decode kernel gathers and
// scales M <= 4 rows itself when they fit on chip; other decode calls and the
// large-M kernel (whose activations go from memory straight into LDS) use the
// pass.
static int64_t xprep_bytes(int64_t M, int64_t N, int64_t K, bool perm, bool xs) {
  if (!perm && !xs) return 0;
  const int64_t bytes = ceil_div(M * K * 2, 256) * 256;
  if (use_prefill(M, N, K)) return bytes;
  int mt;
  return is_staged(pick_mode(M, N, K, perm, xs, &mt)) ? 0 : bytes;
}

int64_t int4_workspace_bytes(int64_t M, int64_t N, int64_t K, bool perm, bool xs) {
  return xprep_bytes(M, N, K, perm, xs) +
         (use_prefill(M, N, K) ? prefill_workspace_bytes(M, N, K) : 0);
}

hipError_t launch_int_gemm(const void* x, const void* xsc, const void* codes_r,
                           const void* scales_r, const void* zeros_r, const int32_t* perm,
                           void* out, int64_t M, int64_t N, int64_t K, int G, int bits,
                           int dtype, void* workspace, int64_t /*workspace_bytes*/,
                           hipStream_t stream) {
  int mt = 1;
  const bool pf = use_prefill(M, N, K);
  const int64_t xb = xprep_bytes(M, N, K, perm != nullptr, xsc != nullptr);
  const void* xa = x;
  if (xb > 0) {
    // the activations are prepared once into the workspace
    const int64_t n8 = M * (K / 8);
    const dim3 grid((unsigned)ceil_div(n8, 256));
    if (dtype == DT_F16)
      hipLaunchKernelGGL(prep_x_kernel<DT_F16>, grid, dim3(256), 0, stream, (const uint16_t*)x,
                         perm, (const uint16_t*)xsc, (uint16_t*)workspace, (int)M, (int)K);
    else
      hipLaunchKernelGGL(prep_x_kernel<DT_BF16>, grid, dim3(256), 0, stream, (const uint16_t*)x,
                         perm, (const uint16_t*)xsc, (uint16_t*)workspace, (int)M, (int)K);
    xa = workspace;
  }
  if (pf) {
    launch_int_prefill(xa, codes_r, scales_r, zeros_r, out, (uint8_t*)workspace + xb, M, N, K,
                       G, bits, dtype, stream);
    return hipGetLastError();
  }
  // what the decode kernel still has to do itself
  const bool gather = perm && xb == 0, scale = xsc && xb == 0;
  const int am = pick_mode(M, N, K, gather, scale, &mt);
  const DecodeArgs a{xa, scale ? xsc : nullptr, codes_r, scales_r, zeros_r,
                     gather ? perm : nullptr, out, M, N, K, stream};
  if (bits == 4) launch_intb_decode<4>(dtype, scale, am, mt, G, a);
  else if (bits == 3) launch_intb_decode<3>(dtype, scale, am, mt, G, a);
  else launch_intb_decode<8>(dtype, scale, am, mt, G, a);
  return hipGetLastError();
}

template <int DT, int MT, int AM, bool BATCH>
static void launch_nf4_v(const void* x, const uint8_t* q, const uint8_t* aq, const float* asc,
                         const Nf4Table& L, void* out, int64_t M, int64_t N, int64_t K,
                         hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(N, 16), (unsigned)ceil_div(M, 16 * MT));
  const size_t lds = AM == AM_FULLT ? xpose_bytes(MT) : 0;
  if (lds) allow_dynamic_lds((const void*)nf4_decode_kernel<DT, MT, AM, BATCH>);
  launch_timed(nf4_decode_kernel<DT, MT, AM, BATCH>, grid, dim3(64 * DW), lds, stream,
               (const uint16_t*)x, q, aq, asc, L, (uint16_t*)out, (int)M, (int)N, (int)K,
               (int)ceil_div(K, 128));
}

template <int DT, bool BATCH>
static void launch_nf4_dt(const void* x, const uint8_t* q, const uint8_t* aq, const float* asc,
                          const Nf4Table& L, void* out, int64_t M, int64_t N, int64_t K,
                          hipStream_t stream) {
  int mt;
  const int am = pick_mode(M, N, K, false, false, &mt);
  if (am == AM_PACKED)
    launch_nf4_v<DT, 1, AM_PACKED, BATCH>(x, q, aq, asc, L, out, M, N, K, stream);
  else if (am == AM_FULL)
    launch_nf4_v<DT, 1, AM_FULL, BATCH>(x, q, aq, asc, L, out, M, N, K, stream);
  else if (mt == 1)
    launch_nf4_v<DT, 1, AM_FULLT, BATCH>(x, q, aq, asc, L, out, M, N, K, stream);
  else if (mt == 2)
    launch_nf4_v<DT, 2, AM_FULLT, BATCH>(x, q, aq, asc, L, out, M, N, K, stream);
  else
    launch_nf4_v<DT, 4, AM_FULLT, BATCH>(x, q, aq, asc, L, out, M, N, K, stream);
}

int64_t nf4_workspace_bytes_for(int64_t M, int64_t N, int64_t K) {
  return nf4_use_prefill(M, N, K) ? prefill_workspace_bytes(M, N, K) : 0;
}

hipError_t launch_nf4_gemm(const void* x, const uint8_t* qweight, const uint8_t* absmax_q,
                           const float* absmax_scale, const Nf4Table& L, void* out, int64_t M,
                           int64_t N, int64_t K, int dtype, void* workspace,
                           int64_t /*workspace_bytes*/, hipStream_t stream) {
  if (nf4_use_prefill(M, N, K)) {
    launch_nf4_prefill(x, qweight, absmax_q, absmax_scale, L, out, workspace, M, N, K, dtype,
                       stream);
    return hipGetLastError();
  }
  const bool batch = K % 1024 == 0;
  if (dtype == DT_F16) {
    if (batch)
      launch_nf4_dt<DT_F16, true>(x, qweight, absmax_q, absmax_scale, L, out, M, N, K, stream);
    else
      launch_nf4_dt<DT_F16, false>(x, qweight, absmax_q, absmax_scale, L, out, M, N, K, stream);
  } else {
    if (batch)
      launch_nf4_dt<DT_BF16, true>(x, qweight, absmax_q, absmax_scale, L, out, M, N, K, stream);
    else
      launch_nf4_dt<DT_BF16, false>(x, qweight, absmax_q, absmax_scale, L, out, M, N, K, stream);
  }
  return hipGetLastError();
}

template void launch_intb_decode<4>(int, bool, int, int, int, const DecodeArgs&);

}  // namespace w4a16

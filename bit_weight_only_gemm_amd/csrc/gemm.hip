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
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "decode.h"

namespace w4a16 {

// Timing events for the next main-kernel launch on this host thread (set by
// w4a16_set_timing_events; consumed by one launch).
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

void set_timing_events(hipEvent_t a, hipEvent_t b) {
  t_ev_start = a;
  t_ev_stop = b;
}

// Activation preparation: x_p[m, k] = x[m, perm[k]] (perm may be null:
// identity), divided by the AWQ input scale s[perm[k]] when xsc is given (the
// same rounding as the fused loads).  gather8: the 8 consecutive prepared
// columns k .. k + 7 of row xr.
template <int DT>
__device__ __forceinline__ u32x4_t gather8(const uint16_t* __restrict__ xr,
                                           const int32_t* __restrict__ perm,
                                           const uint16_t* __restrict__ xsc, int k) {
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
  return v;
}

// The pass in row-major form (the packed decode modes and the large-M
// kernel): one thread per 8 consecutive columns of a row.
template <int DT>
__global__ void __launch_bounds__(256)
prep_x_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
              const uint16_t* __restrict__ xsc, uint16_t* __restrict__ xp, int M, int K) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = K >> 3;
  if (idx >= (int64_t)M * per_row) return;
  const int64_t m = idx / per_row;
  const int k = (int)(idx - m * per_row) * 8;
  *(u32x4_t*)(xp + m * K + k) = gather8<DT>(x + m * K, perm, xsc, k);
}

// The pass in the decode kernel's TILED operand layout, RT = ceil(M / 16) row
// tiles: the 16 bytes of chunk (t, R, j, l), at byte 16 (((t RT + R) 4 + j)
// 64 + l), are prepared columns 128 t + 32 j + 8 (l >> 4) .. + 7 of row
// 16 R + (l & 15) (the integer weights' lane order; zeros for rows >= M).
// One thread per chunk, so every store is part of one coalesced 1 KB run.
template <int DT>
__global__ void __launch_bounds__(256)
prep_tiled_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
                  const uint16_t* __restrict__ xsc, uint16_t* __restrict__ xp, int M, int K,
                  int RT) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)(K >> 7) * RT * 256) return;
  const int l = (int)(idx & 63), j = (int)((idx >> 6) & 3);
  const int64_t rest = idx >> 8;
  const int R = (int)(rest % RT), t = (int)(rest / RT);
  const int row = 16 * R + (l & 15);
  const int k = 128 * t + 32 * j + 8 * (l >> 4);
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (row < M) v = gather8<DT>(x + (int64_t)row * K, perm, xsc, k);
  *(u32x4_t*)(xp + idx * 8) = v;
}

// The pass with each row staged on chip, for K up to what LDS holds
// (prep_rows_fits): workgroup (s, r) takes row r and the 8-column chunk c =
// 256 s + thread.  The row (and the input scales) go into LDS by DMA while
// the thread's permutation entries load into registers, so the pass waits on
// memory once; the chunk is then gathered from LDS and stored, row-major
// (xp + r K + 8 c) or, TILED, at its operand slot (rows M .. 16 RT - 1 of
// the TILED layout are zeros).  One chunk per thread: the pass is latency
// bound, and more workgroups per row (each staging the row) run it on more
// CUs (measured on MI355X, 11008 inputs at M = 4 and 16, whole calls in a
// graph: 6 chunks per thread, one workgroup per row, 1.7 us slower).
constexpr int64_t kMaxPrepLds = 144 * 1024;
inline bool prep_rows_fits(int64_t K, bool xs) {
  const int64_t rowb = ceil_div(K * 2, 1024) * 1024;
  return rowb * (xs ? 2 : 1) <= kMaxPrepLds;
}

template <bool TILED>
__device__ __forceinline__ uint16_t* prep_slot(uint16_t* xp, int r, int c, int K, int RT) {
  if constexpr (TILED) {
    const int k0 = 8 * c, t = k0 >> 7, j = (k0 >> 5) & 3, b = (k0 >> 3) & 3;
    const int64_t idx = ((int64_t)(t * RT + (r >> 4)) * 4 + j) * 64 + (r & 15) + 16 * b;
    return xp + idx * 8;
  } else {
    return xp + (int64_t)r * K + 8 * c;
  }
}

template <int DT, bool TILED>
__global__ void __launch_bounds__(64 * DW)
prep_rows_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
                 const uint16_t* __restrict__ xsc, uint16_t* __restrict__ xp, int M, int K,
                 int RT) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int NT = 64 * DW, P = 1;
  const int r = blockIdx.y, nch = K >> 3, c0 = blockIdx.x * NT * P;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (r >= M) {  // padding rows of the TILED layout (workgroup-uniform)
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int c = c0 + (int)threadIdx.x + i * NT;
      if (c < nch) *(u32x4_t*)prep_slot<TILED>(xp, r, c, K, RT) = u32x4_t{0u, 0u, 0u, 0u};
    }
    return;
  }
  u32x4_t pr[P][2];
  if (perm) {
    const rsrc_t rp = make_rsrc(perm, (uint32_t)K * 4u);
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const uint32_t c = (uint32_t)(c0 + (int)threadIdx.x + i * NT);
      pr[i][0] = bld128(rp, c * 32u, 0);
      pr[i][1] = bld128(rp, c * 32u + 16u, 0);
    }
  }
  const uint32_t rowb = (uint32_t)ceil_div((int64_t)K * 2, 1024) * 1024u;
  stage_lds(x + (int64_t)r * K, (uint32_t)K * 2u, lds, wave, lane);
  if (xsc) stage_lds(xsc, (uint32_t)K * 2u, lds + rowb, wave, lane);
  lds_barrier();
  const uint16_t* row = (const uint16_t*)lds;
  const uint16_t* sl = (const uint16_t*)(lds + rowb);
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int c = c0 + (int)threadIdx.x + i * NT;
    if (c >= nch) break;
    uint32_t src[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      src[e] = perm ? (e < 4 ? pr[i][0][e] : pr[i][1][e - 4]) : (uint32_t)(8 * c + e);
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = row[src[e]];
      if (xsc) h[e] = div_scale1<DT>((uint16_t)h[e], sl[src[e]]);
    }
    *(u32x4_t*)prep_slot<TILED>(xp, r, c, K, RT) =
        u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }
}

template <int DT, bool TILED>
static void launch_prep_rows(const void* x, const int32_t* perm, const void* xsc, void* xp,
                             int64_t M, int64_t K, hipStream_t stream) {
  const int RT = (int)ceil_div(M, 16);
  const dim3 grid((unsigned)ceil_div(K / 8, (int64_t)64 * DW),
                  (unsigned)(TILED ? 16 * RT : M));
  const size_t lds = (size_t)ceil_div(K * 2, 1024) * 1024 * (xsc ? 2 : 1);
  allow_dynamic_lds((const void*)prep_rows_kernel<DT, TILED>);
  hipLaunchKernelGGL((prep_rows_kernel<DT, TILED>), grid, dim3(64 * DW), lds, stream,
                     (const uint16_t*)x, perm, (const uint16_t*)xsc, (uint16_t*)xp, (int)M, (int)K,
                     RT);
}

// Workspace layout: the prepared activations (when they are permuted and/or
// divided by the AWQ input scales in a separate pass), then the large-M
// kernel's split-K partials (when it splits K).  The decode kernel gathers and
// scales M <= 4 rows itself when they fit on chip; other decode calls and the
// large-M kernel (whose activations go from memory straight into LDS) use the
// pass.
static int64_t xprep_bytes(int64_t M, int64_t N, int64_t K, bool perm, bool xs) {
  if (!perm && !xs) return 0;
  if (use_prefill(M, N, K)) return ceil_div(M * K * 2, 256) * 256;
  int mt;
  if (is_staged(pick_mode(M, N, K, perm, xs, &mt))) return 0;
  // more than 4 rows: the TILED layout, in whole row tiles
  const int64_t rows = M > 4 ? ceil_div(M, 16) * 16 : M;
  return ceil_div(rows * K * 2, 256) * 256;
}

int64_t int4_workspace_bytes(int64_t M, int64_t N, int64_t K, bool perm, bool xs) {
  return xprep_bytes(M, N, K, perm, xs) +
         (use_prefill(M, N, K) ? prefill_workspace_bytes(M, N, K) : 0);
}

// The kernels of one call.  Without a workspace (ws == false) every call
// still runs, in the forms that need none: the large-M kernel without a split
// of K, and for a permutation or input scales the decode kernel gathers (and
// scales) the activations itself -- from the rows staged on chip where they
// fit (M <= 4), else element by element from global memory (GGATHER:
// correct at any M, not fast).
GemmPlan plan_int_gemm(int64_t M, int64_t N, int64_t K, int G, int bits, int dtype, bool perm,
                       bool xs, bool ws) {
  GemmPlan p;
  p.dtype = dtype;
  p.bits = bits;
  p.U = units_per_tile(G);
  // the large-M kernel takes its activations as stored: with a permutation or
  // input scales it needs the preparation pass, so without a workspace such a
  // call takes the decode kernel
  p.prefill = use_prefill(M, N, K) && (ws || (!perm && !xs));
  p.xprep = ws ? xprep_bytes(M, N, K, perm, xs) : 0;
  p.prep = p.xprep > 0;
  // (the rows of the row-staged pass are the grid's y dimension)
  p.prep_rows = p.prep && prep_rows_fits(K, xs) && ceil_div(M, 16) * 16 <= 65535;
  if (p.prefill) {
    const PrefillPlan pp = plan_prefill(M, N, K, ws);
    p.bm = pp.bm;
    p.splits = pp.splits;
    p.full = !pp.single && M / pp.bm > 0;
    p.tail = pp.single || M % pp.bm != 0;
    return p;
  }
  p.gather = perm && !p.prep;
  p.xs = xs && !p.prep;
  p.am = pick_mode(M, N, K, p.gather, p.xs, &p.mt);
  // prepared activations for more than 4 rows go into the operand layout
  if (p.prep && is_full(p.am)) p.am = AM_TILED;
  if ((p.gather || p.xs) && !is_staged(p.am)) {
    p.am = AM_GGATHER;
    p.mt = 1;
  }
  // the fold needs o + q exact in the operand type
  const bool fold = !(bits == 8 && dtype == DT_BF16);
  p.one = fold && M == 1 && is_packed(p.am);
  p.wide = fold && p.am == AM_PACKED && !p.xs && M >= 3 && N >= kWideMinN;
  return p;
}

GemmPlan plan_nf4_gemm(int64_t M, int64_t N, int64_t K, int dtype, bool ws, bool repacked) {
  GemmPlan p;
  p.nf4 = true;
  p.repacked = repacked;
  p.dtype = dtype;
  p.prefill = nf4_use_prefill(M, N, K);
  if (p.prefill) {
    // without a workspace the large-M kernel runs without a split of K
    const PrefillPlan pp = plan_prefill(M, N, K, ws);
    p.bm = pp.bm;
    p.splits = pp.splits;
    p.full = !pp.single && M / pp.bm > 0;
    p.tail = pp.single || M % pp.bm != 0;
    return p;
  }
  p.am = pick_mode(M, N, K, false, false, &p.mt);
  if (p.am != AM_FULLT) p.mt = 1;
  p.batch = K % 1024 == 0;
  return p;
}

namespace {
struct Names {
  char* out;
  int64_t n, len = 0;
  void add(const char* fmt, ...) __attribute__((format(printf, 2, 3))) {
    char buf[160];
    va_list ap;
    va_start(ap, fmt);
    const int k = vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    for (int i = 0; i < k; ++i, ++len)
      if (out && len + 1 < n) out[len] = buf[i];
    if (out && n > 0) out[std::min(len, n - 1)] = 0;
  }
};
const char* tf(bool b) { return b ? "true" : "false"; }
}  // namespace

int64_t plan_names(const GemmPlan& p, char* out, int64_t n) {
  Names o{out, n};
  if (out && n > 0) out[0] = 0;
  const bool tiled = !p.prefill && p.am == AM_TILED;
  if (p.prep_rows)
    o.add("w4a16::prep_rows_kernel<%d, %s> + ", p.dtype, tf(tiled));
  else if (p.prep)
    o.add("w4a16::%s<%d> + ", tiled ? "prep_tiled_kernel" : "prep_x_kernel", p.dtype);
  if (p.prefill) {
    const int fmt = p.nf4 ? (p.repacked ? 2 : 1) : 0, U = p.nf4 ? 1 : p.U, bits = p.nf4 ? 4 : p.bits;
    const char* sep = "";
    if (p.full) {
      o.add("w4a16::wq_prefill_kernel<%d, %d, false, %d, %d, %d>", p.dtype, p.bm, fmt, U, bits);
      sep = " + ";
    }
    if (p.tail)
      o.add("%sw4a16::wq_prefill_kernel<%d, %d, true, %d, %d, %d>", sep, p.dtype, p.bm, fmt, U,
            bits);
    if (p.splits > 1) o.add(" + w4a16::split_reduce_kernel<%d>", p.dtype);
  } else if (p.nf4) {
    o.add("w4a16::%s<%d, %d, %d, %s>", p.repacked ? "nf4r_decode_kernel" : "nf4_decode_kernel",
          p.dtype, p.mt, p.am, tf(p.batch));
  } else if (p.wide) {
    o.add("w4a16::intb_decode_wide_kernel<%d, %d, %d, 2, %d>", p.dtype, p.U, p.bits, RUN);
  } else {
    o.add("w4a16::intb_decode_kernel<%d, %d, %d, %d, %s, %d, %s>", p.dtype, p.mt, p.am, p.U,
          tf(p.xs), p.bits, tf(p.one));
  }
  return o.len;
}

hipError_t launch_int_gemm(const void* x, const void* xsc, const void* codes_r,
                           const void* scales_r, const void* zeros_r, const int32_t* perm,
                           void* out, int64_t M, int64_t N, int64_t K, int G, int bits,
                           int dtype, void* workspace, int64_t /*workspace_bytes*/,
                           hipStream_t stream) {
  const GemmPlan pl = plan_int_gemm(M, N, K, G, bits, dtype, perm != nullptr, xsc != nullptr,
                                    workspace != nullptr);
  const void* xa = x;
  if (pl.prep_rows) {
    const bool tiled = !pl.prefill && pl.am == AM_TILED;
    if (dtype == DT_F16) {
      if (tiled) launch_prep_rows<DT_F16, true>(x, perm, xsc, workspace, M, K, stream);
      else launch_prep_rows<DT_F16, false>(x, perm, xsc, workspace, M, K, stream);
    } else {
      if (tiled) launch_prep_rows<DT_BF16, true>(x, perm, xsc, workspace, M, K, stream);
      else launch_prep_rows<DT_BF16, false>(x, perm, xsc, workspace, M, K, stream);
    }
    xa = workspace;
  } else if (pl.prep && !pl.prefill && pl.am == AM_TILED) {
    // the activations are prepared once into the workspace, in the operand
    // layout of the TILED mode
    const int RT = (int)ceil_div(M, 16);
    const dim3 grid((unsigned)ceil_div((K / 128) * RT * 256, 256));
    if (dtype == DT_F16)
      hipLaunchKernelGGL(prep_tiled_kernel<DT_F16>, grid, dim3(256), 0, stream,
                         (const uint16_t*)x, perm, (const uint16_t*)xsc, (uint16_t*)workspace,
                         (int)M, (int)K, RT);
    else
      hipLaunchKernelGGL(prep_tiled_kernel<DT_BF16>, grid, dim3(256), 0, stream,
                         (const uint16_t*)x, perm, (const uint16_t*)xsc, (uint16_t*)workspace,
                         (int)M, (int)K, RT);
    xa = workspace;
  } else if (pl.prep) {
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
  // a timed call: the events bracket the GEMM kernel alone (the timing
  // events' contract)
  if (pl.prep && (t_ev_start || t_ev_stop)) {
    if (hipError_t e = hipStreamSynchronize(stream)) return e;
  }
  if (pl.prefill) {
    launch_int_prefill(xa, codes_r, scales_r, zeros_r, out,
                       workspace ? (uint8_t*)workspace + pl.xprep : nullptr, M, N, K, G, bits,
                       dtype, stream);
    return hipGetLastError();
  }
  // the row blocks of one launch: 16 MT rows each, at most 65536 of them (the
  // grid's y dimension), so the global gather (one row tile) takes calls of
  // more than 2^20 rows in several launches
  const int64_t rows = pl.am == AM_GGATHER ? (int64_t)16 << 16 : M;
  for (int64_t r0 = 0; r0 < M; r0 += rows) {
    const int64_t m = std::min(rows, M - r0);
    const DecodeArgs a{(const uint16_t*)xa + r0 * K, pl.xs ? xsc : nullptr, codes_r, scales_r,
                       zeros_r, pl.gather ? perm : nullptr, (uint16_t*)out + r0 * N, m, N, K,
                       stream, pl.one, pl.wide};
    if (bits == 4) launch_intb_decode<4>(dtype, pl.xs, pl.am, pl.mt, G, a);
    else if (bits == 3) launch_intb_decode<3>(dtype, pl.xs, pl.am, pl.mt, G, a);
    else launch_intb_decode<8>(dtype, pl.xs, pl.am, pl.mt, G, a);
  }
  return hipGetLastError();
}

// ---- the fixed scratch of w4a16_gemm_noalloc: a file-scope device array,
// allocated once per GPU when the library's code object is loaded there and
// held until the process ends.  Host code never uses the array's name as an
// address (in host code it is a host-side stand-in): the device address is
// taken once per GPU with hipGetSymbolAddress, with that GPU current, and
// kept.  Every call on one GPU shares its copy; each call writes every
// scratch byte it later reads (the prepared activations, the split-K
// partials), so nothing needs clearing between calls, but calls that overlap
// in time on one GPU (different streams) race.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t scratch_address(void** ptr) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

template <int DT, int MT, int AM, bool BATCH, bool RP>
static void launch_nf4_v(const void* x, const uint8_t* q, const uint8_t* aq, const float* asc,
                         const Nf4Table& L, void* out, int64_t M, int64_t N, int64_t K,
                         hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(N, 16), (unsigned)ceil_div(M, 16 * MT));
  const size_t lds = AM == AM_FULLT ? xpose_bytes(MT) : 0;
  auto kernel = RP ? nf4r_decode_kernel<DT, MT, AM, BATCH> : nf4_decode_kernel<DT, MT, AM, BATCH>;
  if (lds) allow_dynamic_lds((const void*)kernel);
  launch_timed(kernel, grid, dim3(64 * DW), lds, stream, (const uint16_t*)x, q, aq, asc, L,
               (uint16_t*)out, (int)M, (int)N, (int)K, (int)ceil_div(K, 128));
}

template <int DT, bool BATCH, bool RP>
static void launch_nf4_dt(const GemmPlan& pl, const void* x, const uint8_t* q, const uint8_t* aq,
                          const float* asc, const Nf4Table& L, void* out, int64_t M, int64_t N,
                          int64_t K, hipStream_t stream) {
  if (pl.am == AM_PACKED)
    launch_nf4_v<DT, 1, AM_PACKED, BATCH, RP>(x, q, aq, asc, L, out, M, N, K, stream);
  else if (pl.am == AM_FULL)
    launch_nf4_v<DT, 1, AM_FULL, BATCH, RP>(x, q, aq, asc, L, out, M, N, K, stream);
  else if (pl.mt == 1)
    launch_nf4_v<DT, 1, AM_FULLT, BATCH, RP>(x, q, aq, asc, L, out, M, N, K, stream);
  else if (pl.mt == 2)
    launch_nf4_v<DT, 2, AM_FULLT, BATCH, RP>(x, q, aq, asc, L, out, M, N, K, stream);
  else
    launch_nf4_v<DT, 4, AM_FULLT, BATCH, RP>(x, q, aq, asc, L, out, M, N, K, stream);
}

template <int DT, bool RP>
static void launch_nf4_dec(const GemmPlan& pl, const void* x, const uint8_t* q, const uint8_t* aq,
                           const float* asc, const Nf4Table& L, void* out, int64_t M, int64_t N,
                           int64_t K, hipStream_t stream) {
  if (pl.batch) launch_nf4_dt<DT, true, RP>(pl, x, q, aq, asc, L, out, M, N, K, stream);
  else launch_nf4_dt<DT, false, RP>(pl, x, q, aq, asc, L, out, M, N, K, stream);
}

int64_t nf4_workspace_bytes_for(int64_t M, int64_t N, int64_t K) {
  return nf4_use_prefill(M, N, K) ? prefill_workspace_bytes(M, N, K) : 0;
}

hipError_t launch_nf4_gemm(const void* x, const uint8_t* qweight, const uint8_t* absmax_q,
                           const float* absmax_scale, const Nf4Table& L, void* out, int64_t M,
                           int64_t N, int64_t K, int dtype, void* workspace,
                           int64_t /*workspace_bytes*/, bool repacked, hipStream_t stream) {
  const GemmPlan pl = plan_nf4_gemm(M, N, K, dtype, workspace != nullptr, repacked);
  if (pl.prefill) {
    launch_nf4_prefill(x, qweight, absmax_q, absmax_scale, L, out, workspace, M, N, K, dtype,
                       repacked, stream);
    return hipGetLastError();
  }
  if (dtype == DT_F16) {
    if (repacked) launch_nf4_dec<DT_F16, true>(pl, x, qweight, absmax_q, absmax_scale, L, out, M, N, K, stream);
    else launch_nf4_dec<DT_F16, false>(pl, x, qweight, absmax_q, absmax_scale, L, out, M, N, K, stream);
  } else {
    if (repacked) launch_nf4_dec<DT_BF16, true>(pl, x, qweight, absmax_q, absmax_scale, L, out, M, N, K, stream);
    else launch_nf4_dec<DT_BF16, false>(pl, x, qweight, absmax_q, absmax_scale, L, out, M, N, K, stream);
  }
  return hipGetLastError();
}

template void launch_intb_decode<4>(int, bool, int, int, int, const DecodeArgs&);

}  // namespace w4a16

/*
 * w4a16.h -- C ABI of the MI355X (gfx950) 4-bit weight-only GEMM library.
 *
 * Computes y = x * dequant(Wq)^T for fp16/bf16 activations x [M, K] and 4-bit
 * weights Wq [N, K] (row = output channel) with fp32 accumulation, in two
 * weight formats:
 *
 *   INT4  group-wise: per (column, group of G inputs along K) an fp16 scale
 *         and, for asymmetric codes, a 4-bit zero (symmetric codes have none
 *         and read as zero point 8); G = 128 by default, 32, 64, any multiple
 *         of 128 dividing K, or K itself (per-channel); optional act-order
 *         column map g_idx.
 *   NF4   block-wise normal-float: per 64-element block an absmax that is
 *         itself 8-bit quantized with one fp32 scale per 256 blocks.
 *
 * Sources (cited by page title and section):
 *  [P1] "GPTQ、AWQ与Bitsandbytes：大模型量化三大技术路径深度对比" (tqpw.cn/news/80721)
 *  [P2] "模型量化实践：GPTQ 与 AWQ 在生产环境的精度与速度权衡" (jsqmd.com/news/975148)
 *  [P3] "LLM 量化技术详解：GPTQ、AWQ 与 GGUF 的选型与实践"
 *       (cloud.tencent.com/developer/article/2726413)
 *  [P4] "GPTQ与bitsandbytes对比：谁是2024年大模型量化的终极选择？"
 *       (blog.csdn.net/gitblog_00436/article/details/141051550)
 *  [P5] "LLM量化技术深度对比:GPTQ vs AWQ vs bitsandbytes 2026基准全解析"
 *       (5ulink.com/archives/1952)
 *
 * Conventions for every entry point
 *  - Pointers named *_host are host memory; every other pointer is device
 *    memory owned by the caller.  The library never allocates or frees caller
 *    memory and never calls hipMalloc/hipFree.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Launches are asynchronous on it unless the entry point says it blocks.
 *  - Arguments are validated on the host before anything is launched; a
 *    non-zero status means nothing was launched.  Device-side faults surface
 *    at the caller's next stream synchronization, not in the return value.
 *    Nothing throws or aborts across the ABI: a failed host allocation (or
 *    any other C++ exception inside the library) returns W4A16_ERR_HOST.
 *  - An entry point that launches work first clears (consumes) any HIP error
 *    an earlier runtime call left pending on the calling thread, so that
 *    W4A16_ERR_HIP reports only this call's own launch failures.
 *  - Size limits (W4A16_ERR_UNSUPPORTED beyond them): K <= 2^22, N <= 2^28,
 *    N*K <= 2^37, M <= 2^21, M*K <= 2^36 and M*N <= 2^36.  They keep every
 *    32-bit buffer range and offset the kernels use below 2^31.
 *  - All device pointers must be 16-byte aligned (W4A16_ERR_MISALIGNED).
 *  - 16-bit floats are passed as their bit patterns (uint16_t / void*).
 *  - Rounding: every conversion to fp16/bf16 is round-to-nearest-even;
 *    subnormals are kept (no flush to zero).
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_INVALID_ARG = 1,   /* bad size, NULL required pointer, unknown dtype */
  W4A16_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement */
  W4A16_ERR_MISALIGNED = 3,    /* a device pointer is not 16-byte aligned        */
  W4A16_ERR_BAD_GIDX = 4,      /* g_idx out of range or a group not of size G     */
  W4A16_ERR_WORKSPACE = 5,     /* workspace given but smaller than required       */
  W4A16_ERR_HIP = 6,           /* a HIP runtime call or kernel launch failed      */
  W4A16_ERR_HOST = 7           /* host-side failure (host memory allocation)      */
} w4a16_status_t;

typedef enum { W4A16_F16 = 0, W4A16_BF16 = 1 } w4a16_dtype_t;

/* Which array w4a16_repacked_bytes sizes. */
typedef enum { W4A16_CODES = 0, W4A16_SCALES = 1, W4A16_ZEROS = 2 } w4a16_array_t;

/* Human-readable name of a status code (static storage; never NULL). */
const char* w4a16_status_string(int status);

/* ABI version; bumped on any incompatible change (2: NULL workspace legal on
 * every GEMM call, W4A16_ERR_HOST, the plan queries). */
int w4a16_version(void);

/*
 * Kernel timing (for benchmarks): attach two HIP events (hipEvent_t, created
 * by the caller) to the NEXT main GEMM kernel that w4a16_gemm or nf4_gemm
 * launches from the calling host thread.  The events are recorded by the
 * kernel's own dispatch (hipExtLaunchKernel), so hipEventElapsedTime between
 * them is that kernel's execution time.  One-shot: cleared by that launch.
 * A call whose activations go through a preparation pass first (the
 * permutation, the AWQ input scales) then waits on the host for that pass to
 * finish (hipStreamSynchronize) before it launches the timed kernel, so that
 * the start event does not take in the pass's tail.  Passing NULLs clears a
 * pending request.  Do not use under graph capture.
 */
int w4a16_set_timing_events(void* start_event, void* stop_event);

/*
 * Measurement export (not part of the GEMM): a plain streaming read of
 * `bytes` bytes of device memory by `workgroups` workgroups of 256 lanes,
 * 16-byte loads, eight in flight per lane; each workgroup reads one
 * contiguous chunk.  Its time is the practical HBM read ceiling for a weight
 * stream of that size, against which the decode calls are reported ([P5]
 * "关键数据解读" item 3: decode time follows the weight bytes moved).
 *   buf   device, bytes readable (16-byte aligned).
 *   out   uint32 [workgroups * 256] device, written (each lane's xor of what
 *         it read).
 * Constraints: 0 < bytes <= 2^40, 0 < workgroups <= 2^20, at most 2^30 bytes
 * per workgroup.  Async; honours w4a16_set_timing_events.
 */
int w4a16_stream_read(const void* buf, int64_t bytes, int32_t workgroups, uint32_t* out,
                      void* stream);

/* ------------------------------------------------------------------ INT4 --- */

/*
 * Group sizes (every INT4 entry point): group_size G in {32, 64}, or a
 * multiple of 128 that divides K; -1 means per-channel (G = K, [P3] §2.2),
 * as does G == K.  Smaller groups trade bytes for accuracy ([P3] §7.1,
 * [P1] §3.1 node 3).  K % 128 == 0 and N % 8 == 0 always.  An unsupported G
 * gives W4A16_ERR_UNSUPPORTED, a G that does not divide K
 * W4A16_ERR_INVALID_ARG.
 *
 * Bytes of one array of the repacked INT4 layout for a [N, K] weight
 * (-1 on bad input; a symmetric weight has no zeros array).
 *
 * Repacked layout (KT = K/128 tiles of 128 inputs, NP = ceil(N/64) panels of
 * 64 columns, U = 128/G meta units per tile for G < 128, else U = 1):
 *   codes  uint8 [NP][KT][4][64][16]: output column n = 64p + 16c + i and
 *          (permuted) input column k = 128t + 32j + 8b + e are stored in lane
 *          l = i + 16b, 32-bit little-endian word j of that lane's 16 bytes,
 *          nibble slot (e >> 1) + 4*(e & 1).  Padding columns are zero.
 *   Meta unit v = tU + u of a column: for G < 128 the group (128t + uG)/G
 *          (word j of a lane lies in unit tU + jU/4); for G >= 128 the group
 *          holding tile t (repeated on each tile of a group).
 *   scales fp16  [NP][KT8][4][16][8U] (KT8 = ceil(KT/8)): entry [p][g][c][i][r]
 *          = scale(64p+16c+i, unit 8Ug+r); zero for padding columns/units.
 *   zeros  uint32 [NP][KT8][4][16][U]: bits [4e, 4e+4) of word w =
 *          zero(64p+16c+i, unit 8Ug+8w+e).
 *   (Runs of 8 tiles let a decode wave fetch a run's scales in U 16-byte
 *   loads and its zeros in one load of U dwords.)
 */
int64_t w4a16_repacked_bytes(int64_t K, int64_t N, int32_t group_size, int32_t which);

/*
 * Canonical act-order permutation from a group map ([P2] §三 3.1 desc_act;
 * [P4] "技术原理" --act-order): perm = stable argsort(g_idx), so permuted
 * column k' is original column perm[k'] and each run of G permuted columns is
 * one whole group.
 *   g_idx      int32 [K] device: group of each original input column.
 *   perm       int32 [K] device, written.
 *   nontrivial_host  int32 host, written: 0 if g_idx == k/G for all k.
 * Validates that every value is in [0, K/G) and every group has exactly G
 * members (W4A16_ERR_BAD_GIDX otherwise).  BLOCKS: copies g_idx to the host
 * and synchronizes `stream`.
 */
int w4a16_make_perm(const int32_t* g_idx, int64_t K, int32_t group_size, int32_t* perm,
                    int32_t* nontrivial_host, void* stream);

/*
 * Round-to-nearest group quantizer ([P4] "技术原理": RTN is the baseline GPTQ
 * improves on; [P3] §2.1 asymmetric with a zero point, or symmetric with the
 * zero point fixed; [P3] §2.2 group-wise).
 * Per output row n and group g (the columns {perm[gG .. gG+G-1]} when perm is
 * given, else G consecutive columns):
 *   asymmetric (qzeros given): s = fp16(fp32(max - min) / 15),
 *     z = clip(rint(-min / s), 0, 15),  q = clip(rint(w / s) + z, 0, 15);
 *   symmetric (qzeros NULL): s = fp16(fp32(max |w|) / 7),
 *     q = clip(rint(w / s), -8, 7) + 8  (stored offset by 8; dequantized as
 *     (q - 8) s, so +-max|w| map to +-7);
 * s = 1 where the fp16 scale rounds to 0; all decisions in fp32, rint = half
 * to even.
 *   W        fp32 [N, K] device (finite values).
 *   g_idx    int32 [K] or NULL; perm int32 [K] (from w4a16_make_perm) iff g_idx.
 *   qweight  int32 [K/8, N]: bits [4j,4j+4) of (i, n) = q(n, 8i+j), original order.
 *   scales   fp16 [K/G, N];  qzeros int32 [K/G, N/8] or NULL (symmetric):
 *            bits [4j,4j+4) of (g, i) = z(g, 8i+j).
 * Constraints: the group sizes above.
 */
int w4a16_quantize_rtn(const float* W, const int32_t* g_idx, const int32_t* perm,
                       int64_t N, int64_t K, int32_t group_size, int32_t* qweight,
                       uint16_t* scales, int32_t* qzeros, void* stream);

/*
 * Offline repack of canonical GPTQ-style tensors into the tile layout above
 * (pay the layout translation once, not per call: [P5] "关键数据解读" item 4).
 *   qweight int32 [K/8, N]; scales fp16 [K/G, N]; qzeros int32 [K/G, N/8],
 *           or NULL for a symmetric weight (then zeros_r must be NULL too).
 *   g_idx   int32 [K] or NULL.  When given, `perm` (int32 [K], required then)
 *           receives w4a16_make_perm's permutation (the identity for the
 *           trivial k/G map).  If g_idx is non-trivial the codes are stored in
 *           perm order and *perm_used_host is set to 1: pass `perm` to
 *           w4a16_gemm.  Otherwise *perm_used_host = 0: pass NULL.
 *   codes_r / scales_r / zeros_r: sized by w4a16_repacked_bytes.
 * W4A16_ERR_INVALID_ARG when exactly one of qzeros, zeros_r is NULL.
 * BLOCKS when g_idx is non-NULL (host validation of g_idx); otherwise async.
 */
int w4a16_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                 const int32_t* g_idx, int64_t K, int64_t N, int32_t group_size,
                 void* codes_r, void* scales_r, void* zeros_r, int32_t* perm,
                 int32_t* perm_used_host, void* stream);

/*
 * Workspace bytes w4a16_gemm and w4a16_gemm_xscale use at this shape
 * (covering calls with a column permutation and with input scales): room for
 * the prepared activations M*K*2 where a separate pass writes x[:, perm]
 * and/or x / s, plus the fp32 partials S*M*N*4 of the large-M kernel (M >= 32;
 * M >= 5 on layers of 100 Mi weights and more; M >= 17 on layers of 24 Mi
 * weights and more with N < 5120) when it splits K over S workgroups.  A
 * given call may need less, or nothing: no pass runs where
 * the decode kernel gathers x[:, perm] and/or divides by s itself (M <= 4,
 * the rows, the permutation and the scales staged on chip: at most 152 KB per
 * workgroup on grids of at most 256 workgroups, else 72 KB, and 40 MiB over
 * its grid of N/16 workgroups).
 * A workspace is optional on every call (see w4a16_gemm).  -1 on bad input.
 * Calls that overlap in time must not share a workspace.
 */
int64_t w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group_size);

/*
 * Host-only plan query (no device needed): the kernels w4a16_gemm_bits would
 * launch for this call, in launch order, as the profiler names their
 * instantiations, e.g. "w4a16::prep_x_kernel<0> +
 * w4a16::intb_decode_kernel<0, 1, 4, 1, false, 4, false>".  has_perm,
 * has_x_scale, has_workspace: whether the call passes a permutation, input
 * scales and a workspace (non-zero = yes).
 *   names_host   char[names_bytes] host, written NUL-terminated (truncated to
 *                fit; may be NULL when names_bytes == 0).
 *   names_len_host  int64 host or NULL: the full length without the NUL.
 * Errors as for w4a16_gemm_bits' shape, bits and dtype checks.
 */
int w4a16_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t bits,
                    int32_t dtype, int32_t has_perm, int32_t has_x_scale, int32_t has_workspace,
                    char* names_host, int64_t names_bytes, int64_t* names_len_host);

/*
 * Fused dequantize-and-multiply, the method of [P5] "关键数据解读" item 1
 * (weights are never written back as 16-bit values):
 *   y[m, n] = sum_k x[m, perm[k]] * w[n, k],
 *   w[n, k] = round_dtype(fp32(q - z) * fp32(s))  (q, z, s of column n and the
 *             group of permuted column k; z = 8 when zeros_r is NULL),
 * with fp32 accumulation and one round-to-nearest-even to the output dtype.
 * Paths that apply s and z after a K tile's sum (M <= 4; 9..16 rows, or
 * 5..16 on layers of more than 4096 columns or with prepared activations,
 * with group_size >= 128 in the decode kernel; the large-M kernel's 32-row
 * tiles with group_size >= 128; never 8-bit codes in bf16) compute
 * s * (T - Z) per tile, column and group, T = sum x (o + q) and
 * Z = sum x (o + z) (o = 1024 in fp16, or 64 for the high nibble of each byte
 * of 4-bit codes; 128 in bf16) from two MFMA chains over the same
 * activations, without rounding w to
 * 16 bits first.  Each product is exact in fp32; with each addition of a
 * chain of n products rounded to fp32 (to nearest or toward zero), the
 * tile's error is at most |s| * 2 n u (2 o + 30) * sum |x| (u = 2^-23; n = 32
 * for M <= 4, 128 otherwise), where dequant-then-multiply errs by up to
 * |s| * 15 * 2^-11 * sum |x| (fp16; 2^-8 in bf16) from the rounding of w
 * alone.  Exact on every path: a
 * group whose codes all equal its zero adds exactly 0 (the two chains see
 * identical inputs); a row with one nonzero x, a power of two, gives
 * round_dtype(w).
 *   x      [M, K] row-major, dtype;  out [M, N] row-major, dtype.
 *   perm   int32 [K] from w4a16_repack (or NULL for identity): a
 *          permutation of 0 .. K-1; other entries give unspecified outputs.
 *   codes_r, scales_r, zeros_r from w4a16_repack with the same group_size
 *          (zeros_r NULL: a symmetric weight).
 *   dtype  W4A16_F16 or W4A16_BF16 (activations and output).
 *   workspace / workspace_bytes: optional.  NULL is always legal: the call
 *          then runs in forms that need none (the large-M kernel without a
 *          split of K; the decode kernel gathering x[m][perm[k]], and
 *          dividing by s, itself -- element by element from global memory
 *          where the rows cannot be staged on chip; correct, slower).  A
 *          workspace given must hold w4a16_workspace_bytes(M, N, K,
 *          group_size) bytes (W4A16_ERR_WORKSPACE when smaller); its contents
 *          need not be initialized.
 * Constraints: M >= 1 and the group sizes above.
 * Async on `stream`.  Results are bitwise reproducible run to run for a given
 * shape and workspace choice (every split of K is reduced in a fixed order).
 */
int w4a16_gemm(const void* x, const void* codes_r, const void* scales_r, const void* zeros_r,
               const int32_t* perm, int32_t group_size, void* out, int64_t M, int64_t N,
               int64_t K, int32_t dtype, void* workspace, int64_t workspace_bytes,
               void* stream);

/*
 * w4a16_gemm_bits without any allocation or workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the call runs exactly as
 * w4a16_gemm_bits with a workspace -- the same kernels, bitwise the same
 * output -- but the workspace is a fixed scratch array of
 * W4A16_NOALLOC_SCRATCH_BYTES in device memory that the library holds on
 * each GPU from the first such call until the process ends.  The library
 * calls no hipMalloc, hipFree or allocating routine here.
 *   Arguments: as w4a16_gemm_bits (x_scale NULL: no input scales; bits 3, 4
 *   or 8), on the current GPU's stream.
 *   Calls whose workspace need (w4a16_workspace_bytes) exceeds the scratch
 *   return W4A16_ERR_WORKSPACE (nothing launched); w4a16_gemm_bits with
 *   workspace = NULL also allocates nothing and has no size limit.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in
 * time on one GPU (different streams, or threads) race and must be ordered
 * by the caller.  Each call writes every scratch byte it reads, so no
 * clearing is needed between calls.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES ((int64_t)32 << 20)
int w4a16_gemm_noalloc(const void* x, const void* x_scale, const void* codes_r,
                       const void* scales_r, const void* zeros_r, const int32_t* perm,
                       int32_t group_size, int32_t bits, void* out, int64_t M, int64_t N,
                       int64_t K, int32_t dtype, void* stream);

/*
 * w4a16_gemm with AWQ input scales ([P3] §4.1: the weights of salient input
 * channels are scaled up by s_k before quantization and the activations
 * divided by s_k; here the division is applied by the GEMM, so callers pass
 * the raw activations):
 *   y[m, n] = sum_k (x[m, perm[k]] / s[perm[k]]) * w[n, k].
 *   x_scale  s [K] in the activation dtype (finite, non-zero), indexed by
 *            original input channel; NULL makes the call w4a16_gemm.
 * Each x / s is formed as x * (fp32 reciprocal of s, within 1 ulp) and rounded
 * once to the activation dtype before the multiply.  For M <= 4 rows that the
 * decode kernel stages on chip (see w4a16_workspace_bytes) every workgroup
 * divides its staged copy once; otherwise a preparation pass writes x / s
 * (permuted) into the workspace first, or, without a workspace, the decode
 * kernel divides each gathered element itself.  Other arguments, constraints
 * and the workspace rule as for w4a16_gemm (w4a16_workspace_bytes covers
 * these calls too).
 */
int w4a16_gemm_xscale(const void* x, const void* x_scale, const void* codes_r,
                      const void* scales_r, const void* zeros_r, const int32_t* perm,
                      int32_t group_size, void* out, int64_t M, int64_t N, int64_t K,
                      int32_t dtype, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Test/debug export: the dequantized weight matrix w [N, K] (dtype), in the
 * permuted column order of the repacked codes, computed by the same device
 * routine the GEMM uses.  Async on `stream`.
 */
int w4a16_dequant(const void* codes_r, const void* scales_r, const void* zeros_r, int64_t K,
                  int64_t N, int32_t group_size, int32_t dtype, void* w_out, void* stream);

/* ------------------------------------------------- 3- and 8-bit integers --- */

/*
 * The INT4 entry points above for b-bit integer codes, b = `bits` in
 * {3, 4, 8} (b = 4 is the entry point without the suffix): weight-only
 * quantization at 8 bits trades little accuracy for half the 4-bit saving,
 * at 3 bits more saving for visible loss ([P3] §2.3; the GPTQ-3bit and
 * AWQ-3bit rows of [P1] §4.1; [P4] "量化效果PK", 3-bit codes with groups of
 * 128, and "部署实战", the bit-width option).  Everything else -- group
 * sizes, symmetric codes (implicit zero 2^(b-1)), act-order, AWQ input
 * scales, workspace, dtypes, errors -- is as for 4 bits.  bits outside
 * {3, 4, 8}: W4A16_ERR_UNSUPPORTED.
 *
 * Canonical tensors (GPTQ style, original column order): codes in
 * [0, 2^b - 1]; qweight int32 [K b / 32, N], qzeros int32 [K/G, N b / 32]
 * (asymmetric only).  Each run of 32 consecutive codes along K (qweight) or
 * N (qzeros) is a little-endian bit stream of b words, code e at bits
 * [b e, b e + b); at b = 3 codes 10 and 21 of a run straddle words, and a
 * call that reads or writes 3-bit qzeros needs N % 32 == 0
 * (W4A16_ERR_INVALID_ARG).  RTN as above with 2^b - 1 levels: s =
 * fp16(fp32(max - min) / (2^b - 1)), or s = fp16(fp32(max |w|) /
 * (2^(b-1) - 1)) for symmetric codes.
 *
 * Repacked layout: the tiles of the INT4 layout with each lane's 32 codes in
 * b-bit form (a column tile's K tile is 256 b bytes):
 *   b = 8  uint8 [NP][KT][4][2][64][16]: code (j, e) of lane l in half j >> 1,
 *          dword 2 (j & 1) + (e >> 2) of the lane's 16 bytes, byte slot
 *          ((e & 3) >> 1) + 2 (e & 1).
 *   b = 3  uint8 [NP][KT][4][64][12]: the low 2 bits of code (j, e) at bit
 *          16 (e & 1) + 2 (4 (j & 1) + (e >> 1)) of dword j >> 1, its high
 *          bit at bit 16 (e & 1) + 4 j + (e >> 1) of dword 2.
 *   scales as for 4 bits; zeros in 4-bit fields for b = 3 (as for 4 bits) and
 *   8-bit fields for b = 8 (uint32 [NP][KT8][4][16][2U], unit r of a run at
 *   byte r).
 */
int64_t w4a16_repacked_bytes_bits(int64_t K, int64_t N, int32_t group_size, int32_t bits,
                                  int32_t which);
int w4a16_quantize_rtn_bits(const float* W, const int32_t* g_idx, const int32_t* perm,
                            int64_t N, int64_t K, int32_t group_size, int32_t bits,
                            int32_t* qweight, uint16_t* scales, int32_t* qzeros, void* stream);
int w4a16_repack_bits(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                      const int32_t* g_idx, int64_t K, int64_t N, int32_t group_size,
                      int32_t bits, void* codes_r, void* scales_r, void* zeros_r, int32_t* perm,
                      int32_t* perm_used_host, void* stream);
int w4a16_gemm_bits(const void* x, const void* x_scale, const void* codes_r,
                    const void* scales_r, const void* zeros_r, const int32_t* perm,
                    int32_t group_size, int32_t bits, void* out, int64_t M, int64_t N,
                    int64_t K, int32_t dtype, void* workspace, int64_t workspace_bytes,
                    void* stream);
int w4a16_dequant_bits(const void* codes_r, const void* scales_r, const void* zeros_r, int64_t K,
                       int64_t N, int32_t group_size, int32_t bits, int32_t dtype, void* w_out,
                       void* stream);

/* ------------------------------------------------------------------- NF4 --- */

/*
 * The library's 16 NF4 levels as fp32 (ascending; L[0] = -1, L[7] = 0,
 * L[15] = 1): normal quantiles at 8 equal steps from 1/2 to delta on the
 * positive side and 7 on the negative side, divided by the largest, with
 * delta = ((1 - 1/30) + (1 - 1/32)) / 2 ([P1] §2.3 and §3.3: levels at
 * quantiles of N(0,1); [P5] "关键数据解读" item 2: levels crowd near zero).
 *   out16_host  float[16] host, written.
 */
int nf4_codebook(float* out16_host);

/*
 * On-device NF4 block quantizer with double quantization (calibration-free,
 * done at load time: [P5] "2026 年选型建议" item 4; [P4] "技术原理"):
 *   per block b of `blocksize` consecutive elements of row-major W:
 *   absmax_b = max|w|;  code = argmin_i |w/absmax_b - L_i| (fp32, ties to the
 *   lower index; an all-zero block gives code 7);
 *   per group of 256 consecutive blocks: absmax_scale = fp32(max absmax / 255),
 *   absmax_q = clip(rint(absmax / absmax_scale), 0, 255) (0 if the scale is 0).
 *   W            fp32 [N, K] device (finite values).
 *   qweight      uint8 [N, K/2]: element 2j in the low nibble of byte j.
 *   absmax_q     uint8 [N*K/blocksize];  absmax_scale fp32 [ceil(N*K/blocksize/256)].
 * Constraints: blocksize == 64, K % 64 == 0.
 */
int nf4_quantize(const float* W, int64_t N, int64_t K, int32_t blocksize, uint8_t* qweight,
                 uint8_t* absmax_q, float* absmax_scale, void* stream);

/*
 * Workspace bytes nf4_gemm uses at this shape: the fp32 split-K partials of
 * the large-M kernel (K % 128 == 0 and M >= 64; M >= 33 on layers of 24 Mi
 * weights and more) when it splits K; 0 otherwise.  -1 on bad input.
 */
int64_t nf4_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t blocksize);

/* Host-only plan query for nf4_gemm, as w4a16_gemm_plan. */
int nf4_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t blocksize, int32_t dtype,
                  int32_t has_workspace, char* names_host, int64_t names_bytes,
                  int64_t* names_len_host);

/*
 * Fused NF4 dequantize-and-multiply (bitsandbytes' 4-bit format, dequantized
 * on every forward in its own kernels: [P5] "关键数据解读" item 2; here fused):
 *   y[m, n] = sum_k x[m, k] * w[n, k],
 *   w[n, k] = round_dtype(fp32(L[c] * a')),  a' = fp32(fp32(absmax_q[b]) *
 *   absmax_scale[b / 256]),  b = (n*K + k) / blocksize.
 *   x [M, K] and out [M, N] row-major in dtype; qweight/absmax as nf4_quantize.
 * Constraints: M >= 1, blocksize == 64, K % 64 == 0, N % 16 == 0.
 * workspace: optional; NULL is legal (the large-M kernel then does not split
 * K).  A workspace given must hold nf4_workspace_bytes(M, N, K, 64) bytes
 * (W4A16_ERR_WORKSPACE when smaller).  Async.
 */
int nf4_gemm(const void* x, const uint8_t* qweight, const uint8_t* absmax_q,
             const float* absmax_scale, int32_t blocksize, void* out, int64_t M, int64_t N,
             int64_t K, int32_t dtype, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * NF4 codes re-laid once, offline, into the 1 KB tiles the decode and large-M
 * kernels read contiguously ([P5] "关键数据解读" item 4: a layout is translated
 * once, not on every run): tiles of 16 output rows x 128 inputs, tile (c, t)
 * at byte 1024 (c ceil(K/128) + t), its 16-byte chunk l holding bytes
 * 64 t + 16 (l >> 4) .. + 15 of canonical row 16 c + (l & 15) (the codes of
 * inputs 128 t + 32 (l >> 4) .. + 31, low nibble first), zeros past the row's
 * K / 2 bytes.  The absmax codes and scales stay as nf4_quantize writes them.
 *   nf4_repacked_bytes: N / 16 * ceil(K / 128) * 1024, or -1 on bad input
 *   (N % 16 != 0, or the shape rules of nf4_gemm).
 *   nf4_repack: qweight uint8 [N, K/2] (device, canonical) -> qweight_r
 *   (device, nf4_repacked_bytes); the two must not overlap.  Async; errors as
 *   for nf4_gemm's shape and pointer checks.
 */
int64_t nf4_repacked_bytes(int64_t N, int64_t K, int32_t blocksize);
int nf4_repack(const uint8_t* qweight, int64_t N, int64_t K, int32_t blocksize,
               uint8_t* qweight_r, void* stream);

/*
 * nf4_gemm on repacked codes (nf4_repack): the same product, the same
 * kernels' arithmetic in the same order -- bitwise the same output as
 * nf4_gemm on the canonical codes -- reading each tile of codes as one
 * contiguous block.  Arguments, constraints, workspace and errors as for
 * nf4_gemm (nf4_workspace_bytes covers these calls too).
 */
int nf4_gemm_repacked(const void* x, const uint8_t* qweight_r, const uint8_t* absmax_q,
                      const float* absmax_scale, int32_t blocksize, void* out, int64_t M,
                      int64_t N, int64_t K, int32_t dtype, void* workspace,
                      int64_t workspace_bytes, void* stream);
/* Host-only plan query for nf4_gemm_repacked, as w4a16_gemm_plan. */
int nf4_gemm_repacked_plan(int64_t M, int64_t N, int64_t K, int32_t blocksize, int32_t dtype,
                           int32_t has_workspace, char* names_host, int64_t names_bytes,
                           int64_t* names_len_host);

/* Test/debug export: dequantized NF4 weights w [N, K] in dtype.  Async. */
int nf4_dequant(const uint8_t* qweight, const uint8_t* absmax_q, const float* absmax_scale,
                int64_t N, int64_t K, int32_t blocksize, int32_t dtype, void* w_out,
                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */

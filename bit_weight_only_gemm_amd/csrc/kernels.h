// kernels.h -- host-side launch entry points of the device kernels.  Every
// launcher assumes arguments were validated by the C-ABI layer (api.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace w4a16 {

// NF4 levels passed by value as a kernel argument (64 bytes).
struct Nf4Table {
  float v[16];
};

// INT4 group sizes: G in {32, 64} or a multiple of 128 dividing K (G = K is
// per-channel).  The repacked scales and zeros come in "units", U per K tile
// of 128 inputs: for G < 128 unit u of tile t is group (128 t + u G) / G and
// word j of a repacked lane (inputs 128 t + 32 j + ...) lies in unit j U / 4;
// for G >= 128 the single unit of tile t repeats the scale and zero of the
// group that holds the tile.
__host__ __device__ constexpr int units_per_tile(int G) { return G < 128 ? 128 / G : 1; }

// Workspace bytes the INT4 GEMM needs at this shape, with or without a column
// permutation and AWQ input scales: room for the prepared activations (when
// they are permuted and/or scaled in a separate pass) and for the prefill
// kernel's split-K partials.
int64_t int4_workspace_bytes(int64_t M, int64_t N, int64_t K, bool perm, bool xs);
// Bytes of the prefill kernel's split-K partials at this shape (0: no split).
int64_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K);

// Attach HIP timing events to the next main GEMM kernel launched by the
// calling host thread (hipExtLaunchKernel start/stop events).
void set_timing_events(hipEvent_t start, hipEvent_t stop);

// bits-bit RTN codes (3, 4 or 8) in the canonical packing; qzeros == nullptr:
// symmetric codes (no zeros).
hipError_t launch_rtn_int(const float* W, const int32_t* perm, int64_t N, int64_t K, int G,
                          int bits, int32_t* qweight, uint16_t* scales, int32_t* qzeros,
                          hipStream_t stream);
hipError_t launch_nf4_quant(const float* W, int64_t N, int64_t K, const Nf4Table& L,
                            uint8_t* qweight, uint8_t* absmax_q, float* absmax_scale,
                            hipStream_t stream);
// In the repack, dequant and GEMM launchers zeros == nullptr (qzeros,
// zeros_r) is a symmetric weight.
hipError_t launch_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                         const int32_t* perm, int64_t K, int64_t N, int G, int bits,
                         void* codes_r, void* scales_r, void* zeros_r, hipStream_t stream);
hipError_t launch_dequant_int(const void* codes_r, const void* scales_r, const void* zeros_r,
                              int64_t K, int64_t N, int G, int bits, int dtype, void* w_out,
                              hipStream_t stream);
hipError_t launch_dequant_nf4(const uint8_t* qweight, const uint8_t* absmax_q,
                              const float* absmax_scale, int64_t N, int64_t K, int dtype,
                              const Nf4Table& L, void* w_out, hipStream_t stream);

// Rows per workgroup of the large-M kernel for M, and the split of K that
// fills the GPU best: a simple model of the call time (rounds of workgroups on
// 256 CUs x K tiles per workgroup x per-tile MFMA time, plus the partials'
// round trip through HBM).  split_ok = false: no workspace for partials, one
// workgroup per output tile.
struct PrefillPlan {
  int bm, splits;
  bool single;  // one launch of the ragged-tail form covers every row block
};
PrefillPlan plan_prefill(int64_t M, int64_t N, int64_t K, bool split_ok = true);

// How one GEMM call runs: the kernels it launches, in order.  The launchers
// follow the plan, and plan_names reports it (the kernel instantiations as
// the profiler names them), so a report cannot drift from the dispatch.
struct GemmPlan {
  bool nf4 = false;
  int dtype = 0, bits = 4, U = 1;
  bool prep = false;        // a pass writes x[:, perm] / s into the workspace first
  bool prep_rows = false;   // ... prep_rows_kernel (each row staged on chip)
  int64_t xprep = 0;        // its workspace bytes
  bool prefill = false;     // the large-M kernel (else the decode kernel)
  int bm = 0, splits = 1;   // large-M: rows per workgroup, split of K
  bool full = false, tail = false;  // large-M: launches over whole and partial row blocks
  int am = 0, mt = 1;       // decode: activation mode, row tiles per workgroup
  bool xs = false;          // decode: the kernel divides by the input scales itself
  bool gather = false;      // decode: the kernel applies the permutation itself
  bool one = false;         // decode: the one-row form of the packed fold
  bool wide = false;        // decode: the wide packed kernel (2 column tiles per wave)
  bool batch = false;       // NF4 decode: absmax codes of a run in one load
  bool repacked = false;    // NF4: the codes in the tile layout (nf4_repack)
};
// ws: whether the call has a workspace (of at least int4_workspace_bytes).
GemmPlan plan_int_gemm(int64_t M, int64_t N, int64_t K, int G, int bits, int dtype, bool perm,
                       bool xs, bool ws);
GemmPlan plan_nf4_gemm(int64_t M, int64_t N, int64_t K, int dtype, bool ws, bool repacked = false);
// "w4a16::kernel<args> + ..." in launch order (at most n bytes with the NUL);
// returns the full length.
int64_t plan_names(const GemmPlan& p, char* out, int64_t n);

// Bytes of the fixed device scratch that w4a16_gemm_noalloc uses in place of
// a workspace, and its device address on the current GPU (taken once per GPU).
constexpr int64_t kScratchBytes = (int64_t)32 << 20;
hipError_t scratch_address(void** ptr);

// xsc: AWQ input scales s [K] (activation dtype) or nullptr; bits: 3, 4 or 8.
hipError_t launch_int_gemm(const void* x, const void* xsc, const void* codes_r,
                           const void* scales_r, const void* zeros_r, const int32_t* perm,
                           void* out, int64_t M, int64_t N, int64_t K, int G, int bits,
                           int dtype, void* workspace,
                            int64_t workspace_bytes, hipStream_t stream);
// Whether w4a16_gemm runs the LDS-staged large-M kernel (activations shared
// by a workgroup's 256 columns through LDS) rather than the skinny decode
// kernel.  The decode kernel's time grows with every 16 rows; the large-M
// kernel's hardly changes with M below 32 rows but carries the fixed cost of
// its split-K reduction launch.  Measured whole-call crossovers on MI355X
// (HIP graphs of calls over weight sets larger than the caches): from 5 rows
// on layers of 100 Mi weights and more (5120 x 55296 at M = 5: 45.4 us against
// 52.3), from 17 rows on layers of 24 Mi weights and more with N < 5120
// (11008 x 4096, act-order: 16.8 us against 21.8 at M = 16, 22.1 against 21.5
// at M = 20, where the decode kernel takes 32-row tiles on a grid of one
// workgroup per CU), and from 32 rows otherwise (4096 x 11008, act-order, at
// M = 24: 17.8 against 19.5; 5120 x 5120 at M = 24: 14.4 against 14.7).
inline bool use_prefill(int64_t M, int64_t N, int64_t K) {
  if (M >= 32) return true;
  const int64_t w = N * K;
  if (w >= (int64_t)100 << 20) return M >= 5;
  if (w >= (int64_t)24 << 20 && N < 5120) return M >= 17;
  return false;
}
void launch_int_prefill(const void* x, const void* codes_r, const void* scales_r,
                        const void* zeros_r, void* out, void* ws, int64_t M, int64_t N,
                        int64_t K, int G, int bits, int dtype, hipStream_t stream);

// repacked: the NF4 codes in the tile layout of launch_nf4_repack
void launch_nf4_prefill(const void* x, const uint8_t* qweight, const uint8_t* absmax_q,
                        const float* absmax_scale, const Nf4Table& L, void* out, void* ws,
                        int64_t M, int64_t N, int64_t K, int dtype, bool repacked,
                        hipStream_t stream);
// Whether nf4_gemm runs the large-M kernel at this shape, and the workspace
// bytes it then needs.  Its codebook dequant costs about twice the INT4 one,
// so the crossovers (measured in bf16) are later than INT4's: past the
// decode kernel's 32-row tiles on layers of 24 Mi weights and more (28672 x
// 8192: 77.0 us against 80.8 at M = 32, 143.5 against 119.7 at M = 48; 4096 x
// 11008: 18.9 against 24.8 at M = 32), from 64 rows otherwise.
inline bool nf4_use_prefill(int64_t M, int64_t N, int64_t K) {
  const int64_t w = N * K;
  return K % 128 == 0 && (M >= 64 || (w >= (int64_t)24 << 20 && M > 32));
}
int64_t nf4_workspace_bytes_for(int64_t M, int64_t N, int64_t K);

hipError_t launch_nf4_gemm(const void* x, const uint8_t* qweight, const uint8_t* absmax_q,
                           const float* absmax_scale, const Nf4Table& L, void* out, int64_t M,
                           int64_t N, int64_t K, int dtype, void* workspace,
                           int64_t workspace_bytes, bool repacked, hipStream_t stream);
// NF4 codes re-laid into tiles of 16 rows x 128 inputs (1 KB; lane r of tile
// (c, t) holds bytes 64 t + 16 (r >> 4) .. + 15 of row 16 c + (r & 15), zeros
// past the row): N / 16 x ceil(K / 128) KB.
inline int64_t nf4_repacked_bytes_for(int64_t N, int64_t K) { return N / 16 * ((K + 127) / 128) * 1024; }
hipError_t launch_nf4_repack(const uint8_t* qweight, int64_t N, int64_t K, uint8_t* qweight_r,
                             hipStream_t stream);

// A plain streaming read of `bytes` by `workgroups` workgroups of 256 lanes
// (the practical HBM read ceiling); out: uint32 [workgroups * 256].
hipError_t launch_stream_read(const void* buf, int64_t bytes, int workgroups, uint32_t* out,
                              hipStream_t stream);

}  // namespace w4a16

// api.hip -- the C ABI declared in include/w4a16.h: host-side validation,
// the act-order permutation, the NF4 codebook, and dispatch to the kernels.
//
// Every entry point validates all arguments on the host before launching
// anything and returns a status code; nothing throws across the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/w4a16.h"
#include "common.h"
#include "kernels.h"

using namespace w4a16;

static_assert(kScratchBytes == W4A16_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");

namespace {

constexpr int64_t kMaxM = (int64_t)1 << 21;  // keeps every row-block grid dimension < 65536

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_ptrs(std::initializer_list<const void*> required) {
  for (const void* p : required) {
    if (!p) return W4A16_ERR_INVALID_ARG;
  }
  for (const void* p : required) {
    if (!aligned16(p)) return W4A16_ERR_MISALIGNED;
  }
  return W4A16_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP; }

// The launchers report hipGetLastError() after their launches; an error an
// earlier runtime call of the caller left pending is cleared (consumed) first
// so that it is not reported as this call's failure.
void clear_pending_error() { (void)hipGetLastError(); }

// Runs an entry point's body so that no C++ exception crosses the C ABI: a
// failed host allocation (std::bad_alloc) or any other exception becomes
// W4A16_ERR_HOST.
template <class F>
int guarded(F&& f) noexcept {
  try {
    return f();
  } catch (...) {
    return W4A16_ERR_HOST;
  }
}

// ---- NF4 codebook, computed here from its closed form (independent of any
// table elsewhere): Phi^-1 by Newton iteration on erfc in double precision.
double norm_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double norm_ppf(double p) {
  double x = 0.0;
  for (int it = 0; it < 100; ++it) {
    const double pdf = std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
    const double dx = (norm_cdf(x) - p) / pdf;
    x -= dx;
    if (std::fabs(dx) <= 1e-17 * std::fmax(1.0, std::fabs(x))) break;
  }
  return x;
}

struct Codebook {
  Nf4Table t;
  Codebook() {
    const double d = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
    std::vector<double> v;
    // equal probability steps from d down to 1/2 (the 1/2 end, level 0, dropped)
    const double step9 = (0.5 - d) / 8.0, step8 = (0.5 - d) / 7.0;
    for (int i = 0; i < 8; ++i) v.push_back(norm_ppf((double)i * step9 + d));
    for (int i = 0; i < 7; ++i) v.push_back(-norm_ppf((double)i * step8 + d));
    v.push_back(0.0);
    std::sort(v.begin(), v.end());
    const double top = norm_ppf(d);
    for (int i = 0; i < 16; ++i) t.v[i] = (float)(v[i] / top);
  }
};

const Nf4Table& codebook() {
  static const Codebook cb;
  return cb.t;
}

// Group size G: 32, 64 or a multiple of 128 that divides K; -1 (or K) is
// per-channel.  K is a whole number of 128-input tiles in every case.
int64_t resolve_group(int64_t K, int32_t group_size) {
  return group_size == -1 ? K : (int64_t)group_size;
}

// Size limits.  The kernels address each buffer through 32-bit descriptor
// ranges and offsets relative to a per-panel or per-row-block base: a row
// block of up to 256 activation rows (256 * K * 2 bytes), one 64-column panel
// of codes (64 * K bytes at 8 bits), NF4 block indices n * K / 64 for the
// whole weight.  K <= 2^22, N <= 2^28, N * K <= 2^37 and M * K, M * N <= 2^36
// keep every such range and offset below 2^31 (and every grid dimension in
// range); larger shapes are W4A16_ERR_UNSUPPORTED.
constexpr int64_t kMaxK = (int64_t)1 << 22, kMaxN = (int64_t)1 << 28;
constexpr int64_t kMaxNK = (int64_t)1 << 37, kMaxMX = (int64_t)1 << 36;

bool too_big(int64_t N, int64_t K) { return K > kMaxK || N > kMaxN || N * K > kMaxNK; }
bool too_big_m(int64_t M, int64_t N, int64_t K) {
  return M > kMaxM || M * K > kMaxMX || M * N > kMaxMX;
}

int validate_int4_shape(int64_t K, int64_t N, int32_t group_size) {
  if (K <= 0 || N <= 0) return W4A16_ERR_INVALID_ARG;
  if (K % 128 != 0 || N % 8 != 0) return W4A16_ERR_INVALID_ARG;
  if (too_big(N, K)) return W4A16_ERR_UNSUPPORTED;
  const int64_t G = resolve_group(K, group_size);
  if (G == 32 || G == 64) return W4A16_OK;
  if (G <= 0 || G % 128 != 0) return W4A16_ERR_UNSUPPORTED;
  if (K % G != 0) return W4A16_ERR_INVALID_ARG;
  return W4A16_OK;
}

// Code widths: 3, 4 or 8 bits.  3-bit zeros pack in runs of 32 columns, so a
// call that reads or writes canonical 3-bit zeros needs N % 32 == 0.
int validate_bits(int32_t bits) {
  return (bits == 3 || bits == 4 || bits == 8) ? W4A16_OK : W4A16_ERR_UNSUPPORTED;
}
int validate_zero_rows(int64_t N, int32_t bits, bool zeros) {
  return (zeros && bits == 3 && N % 32 != 0) ? W4A16_ERR_INVALID_ARG : W4A16_OK;
}

int validate_dtype(int32_t dtype) {
  return (dtype == W4A16_F16 || dtype == W4A16_BF16) ? W4A16_OK : W4A16_ERR_INVALID_ARG;
}

}  // namespace

extern "C" {

const char* w4a16_status_string(int status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_INVALID_ARG: return "invalid argument";
    case W4A16_ERR_UNSUPPORTED: return "unsupported configuration";
    case W4A16_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case W4A16_ERR_BAD_GIDX: return "malformed g_idx (value out of range or group size != G)";
    case W4A16_ERR_WORKSPACE: return "workspace smaller than required";
    case W4A16_ERR_HIP: return "HIP runtime error";
    case W4A16_ERR_HOST: return "host-side failure (host memory allocation)";
    default: return "unknown status";
  }
}

int w4a16_version(void) { return 2; }

int64_t w4a16_repacked_bytes_bits(int64_t K, int64_t N, int32_t group_size, int32_t bits,
                                  int32_t which) {
  if (validate_int4_shape(K, N, group_size) != W4A16_OK || validate_bits(bits) != W4A16_OK)
    return -1;
  const int64_t U = units_per_tile((int)resolve_group(K, group_size));
  const int64_t NP = ceil_div(N, 64), KT = K / 128, KT8 = ceil_div(KT, 8);
  switch (which) {
    case W4A16_CODES: return NP * KT * 4 * 256 * bits;
    case W4A16_SCALES: return NP * KT8 * 1024 * U;
    case W4A16_ZEROS: return NP * KT8 * 256 * U * (zero_field_bits(bits) / 4);
    default: return -1;
  }
}

int64_t w4a16_repacked_bytes(int64_t K, int64_t N, int32_t group_size, int32_t which) {
  return w4a16_repacked_bytes_bits(K, N, group_size, 4, which);
}

int w4a16_make_perm(const int32_t* g_idx, int64_t K, int32_t group_size, int32_t* perm,
                    int32_t* nontrivial_host, void* stream) {
  return guarded([&]() -> int {
    if (!nontrivial_host) return W4A16_ERR_INVALID_ARG;
    if (int s = validate_int4_shape(K, 8, group_size)) return s;
    if (int s = check_ptrs({g_idx, perm})) return s;
    const int64_t G = resolve_group(K, group_size);
    hipStream_t st = (hipStream_t)stream;
    std::vector<int32_t> g((size_t)K);
    if (hipMemcpyAsync(g.data(), g_idx, (size_t)K * 4, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return W4A16_ERR_HIP;
    const int64_t ng = K / G;
    std::vector<int64_t> count((size_t)ng, 0);
    bool trivial = true;
    for (int64_t k = 0; k < K; ++k) {
      if (g[k] < 0 || g[k] >= ng) return W4A16_ERR_BAD_GIDX;
      ++count[g[k]];
      if (g[k] != k / G) trivial = false;
    }
    for (int64_t c : count)
      if (c != G) return W4A16_ERR_BAD_GIDX;
    // stable counting sort: columns of group 0 in original order, then group 1, ...
    std::vector<int32_t> p((size_t)K);
    std::vector<int64_t> next((size_t)ng);
    for (int64_t i = 0; i < ng; ++i) next[i] = i * G;
    for (int64_t k = 0; k < K; ++k) p[next[g[k]]++] = (int32_t)k;
    if (hipMemcpyAsync(perm, p.data(), (size_t)K * 4, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return W4A16_ERR_HIP;
    *nontrivial_host = trivial ? 0 : 1;
    return W4A16_OK;
  });
}

int w4a16_quantize_rtn_bits(const float* W, const int32_t* g_idx, const int32_t* perm,
                            int64_t N, int64_t K, int32_t group_size, int32_t bits,
                            int32_t* qweight, uint16_t* scales, int32_t* qzeros, void* stream) {
  return guarded([&]() -> int {
    if (int s = validate_int4_shape(K, N, group_size)) return s;
    if (int s = validate_bits(bits)) return s;
    if (int s = validate_zero_rows(N, bits, qzeros != nullptr)) return s;
    if ((g_idx == nullptr) != (perm == nullptr)) return W4A16_ERR_INVALID_ARG;
    if (int s = check_ptrs({W, qweight, scales})) return s;
    if (perm && !aligned16(perm)) return W4A16_ERR_MISALIGNED;
    if (qzeros && !aligned16(qzeros)) return W4A16_ERR_MISALIGNED;
    clear_pending_error();
    return hip_status(launch_rtn_int(W, perm, N, K, (int)resolve_group(K, group_size), bits,
                                     qweight, scales, qzeros, (hipStream_t)stream));
  });
}

int w4a16_quantize_rtn(const float* W, const int32_t* g_idx, const int32_t* perm, int64_t N,
                       int64_t K, int32_t group_size, int32_t* qweight, uint16_t* scales,
                       int32_t* qzeros, void* stream) {
  return w4a16_quantize_rtn_bits(W, g_idx, perm, N, K, group_size, 4, qweight, scales, qzeros,
                                 stream);
}

int w4a16_repack_bits(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                      const int32_t* g_idx, int64_t K, int64_t N, int32_t group_size,
                      int32_t bits, void* codes_r, void* scales_r, void* zeros_r, int32_t* perm,
                      int32_t* perm_used_host, void* stream) {
  return guarded([&]() -> int {
    if (int s = validate_int4_shape(K, N, group_size)) return s;
    if (int s = validate_bits(bits)) return s;
    if (int s = validate_zero_rows(N, bits, qzeros != nullptr)) return s;
    if (!perm_used_host) return W4A16_ERR_INVALID_ARG;
    // a symmetric weight has neither zeros nor repacked zeros
    if ((qzeros == nullptr) != (zeros_r == nullptr)) return W4A16_ERR_INVALID_ARG;
    if (int s = check_ptrs({qweight, scales, codes_r, scales_r})) return s;
    if (qzeros && (!aligned16(qzeros) || !aligned16(zeros_r))) return W4A16_ERR_MISALIGNED;
    int32_t used = 0;
    if (g_idx) {
      if (!perm) return W4A16_ERR_INVALID_ARG;
      if (int s = w4a16_make_perm(g_idx, K, group_size, perm, &used, stream)) return s;
    }
    clear_pending_error();
    if (int s = hip_status(launch_repack(qweight, scales, qzeros, used ? perm : nullptr, K, N,
                                         (int)resolve_group(K, group_size), bits, codes_r,
                                         scales_r, zeros_r, (hipStream_t)stream)))
      return s;
    *perm_used_host = used;
    return W4A16_OK;
  });
}

int w4a16_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                 const int32_t* g_idx, int64_t K, int64_t N, int32_t group_size, void* codes_r,
                 void* scales_r, void* zeros_r, int32_t* perm, int32_t* perm_used_host,
                 void* stream) {
  return w4a16_repack_bits(qweight, scales, qzeros, g_idx, K, N, group_size, 4, codes_r,
                           scales_r, zeros_r, perm, perm_used_host, stream);
}

int64_t w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group_size) {
  if (M <= 0 || validate_int4_shape(K, N, group_size) != W4A16_OK || too_big_m(M, N, K))
    return -1;
  return int4_workspace_bytes(M, N, K, true, true);
}

int w4a16_set_timing_events(void* start_event, void* stop_event) {
  set_timing_events((hipEvent_t)start_event, (hipEvent_t)stop_event);
  return W4A16_OK;
}

int w4a16_stream_read(const void* buf, int64_t bytes, int32_t workgroups, uint32_t* out,
                      void* stream) {
  return guarded([&]() -> int {
    if (bytes <= 0 || bytes > ((int64_t)1 << 40) || workgroups <= 0 ||
        workgroups > (1 << 20))
      return W4A16_ERR_INVALID_ARG;
    if (ceil_div(bytes, (int64_t)workgroups) > ((int64_t)1 << 30)) return W4A16_ERR_UNSUPPORTED;
    if (int s = check_ptrs({buf, out})) return s;
    clear_pending_error();
    return hip_status(launch_stream_read(buf, bytes, workgroups, out, (hipStream_t)stream));
  });
}

int w4a16_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t bits,
                    int32_t dtype, int32_t has_perm, int32_t has_x_scale, int32_t has_workspace,
                    char* names_host, int64_t names_bytes, int64_t* names_len_host) {
  return guarded([&]() -> int {
    if (M <= 0) return W4A16_ERR_INVALID_ARG;
    if (int s = validate_int4_shape(K, N, group_size)) return s;
    if (too_big_m(M, N, K)) return W4A16_ERR_UNSUPPORTED;
    if (int s = validate_bits(bits)) return s;
    if (int s = validate_dtype(dtype)) return s;
    if (names_bytes < 0 || (names_bytes > 0 && !names_host)) return W4A16_ERR_INVALID_ARG;
    const GemmPlan pl = plan_int_gemm(M, N, K, (int)resolve_group(K, group_size), bits, dtype,
                                      has_perm != 0, has_x_scale != 0, has_workspace != 0);
    const int64_t len = plan_names(pl, names_host, names_bytes);
    if (names_len_host) *names_len_host = len;
    return W4A16_OK;
  });
}

int w4a16_gemm_bits(const void* x, const void* x_scale, const void* codes_r,
                    const void* scales_r, const void* zeros_r, const int32_t* perm,
                    int32_t group_size, int32_t bits, void* out, int64_t M, int64_t N,
                    int64_t K, int32_t dtype, void* workspace, int64_t workspace_bytes,
                    void* stream) {
  return guarded([&]() -> int {
    if (M <= 0) return W4A16_ERR_INVALID_ARG;
    if (int s = validate_int4_shape(K, N, group_size)) return s;
    if (too_big_m(M, N, K)) return W4A16_ERR_UNSUPPORTED;
    if (int s = validate_bits(bits)) return s;
    if (int s = validate_dtype(dtype)) return s;
    if (int s = check_ptrs({x, codes_r, scales_r, out})) return s;
    if (zeros_r && !aligned16(zeros_r)) return W4A16_ERR_MISALIGNED;
    if (x_scale && !aligned16(x_scale)) return W4A16_ERR_MISALIGNED;
    if (perm && !aligned16(perm)) return W4A16_ERR_MISALIGNED;
    if (workspace && !aligned16(workspace)) return W4A16_ERR_MISALIGNED;
    // NULL workspace: legal, the call takes the forms that need none
    if (workspace &&
        workspace_bytes < int4_workspace_bytes(M, N, K, perm != nullptr, x_scale != nullptr))
      return W4A16_ERR_WORKSPACE;
    clear_pending_error();
    return hip_status(launch_int_gemm(x, x_scale, codes_r, scales_r, zeros_r, perm, out, M, N,
                                      K, (int)resolve_group(K, group_size), bits, dtype,
                                      workspace, workspace_bytes, (hipStream_t)stream));
  });
}

int w4a16_gemm_noalloc(const void* x, const void* x_scale, const void* codes_r,
                       const void* scales_r, const void* zeros_r, const int32_t* perm,
                       int32_t group_size, int32_t bits, void* out, int64_t M, int64_t N,
                       int64_t K, int32_t dtype, void* stream) {
  return guarded([&]() -> int {
    if (M <= 0) return W4A16_ERR_INVALID_ARG;
    if (int s = validate_int4_shape(K, N, group_size)) return s;
    if (too_big_m(M, N, K)) return W4A16_ERR_UNSUPPORTED;
    if (int s = validate_bits(bits)) return s;
    if (int s = validate_dtype(dtype)) return s;
    if (int s = check_ptrs({x, codes_r, scales_r, out})) return s;
    if (zeros_r && !aligned16(zeros_r)) return W4A16_ERR_MISALIGNED;
    if (x_scale && !aligned16(x_scale)) return W4A16_ERR_MISALIGNED;
    if (perm && !aligned16(perm)) return W4A16_ERR_MISALIGNED;
    const int64_t need = int4_workspace_bytes(M, N, K, perm != nullptr, x_scale != nullptr);
    if (need > kScratchBytes) return W4A16_ERR_WORKSPACE;
    clear_pending_error();
    void* ws = nullptr;
    if (int s = hip_status(scratch_address(&ws))) return s;
    return hip_status(launch_int_gemm(x, x_scale, codes_r, scales_r, zeros_r, perm, out, M, N,
                                      K, (int)resolve_group(K, group_size), bits, dtype, ws,
                                      kScratchBytes, (hipStream_t)stream));
  });
}

int w4a16_gemm_xscale(const void* x, const void* x_scale, const void* codes_r,
                      const void* scales_r, const void* zeros_r, const int32_t* perm,
                      int32_t group_size, void* out, int64_t M, int64_t N, int64_t K,
                      int32_t dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  return w4a16_gemm_bits(x, x_scale, codes_r, scales_r, zeros_r, perm, group_size, 4, out, M, N,
                         K, dtype, workspace, workspace_bytes, stream);
}

int w4a16_gemm(const void* x, const void* codes_r, const void* scales_r, const void* zeros_r,
               const int32_t* perm, int32_t group_size, void* out, int64_t M, int64_t N,
               int64_t K, int32_t dtype, void* workspace, int64_t workspace_bytes,
               void* stream) {
  return w4a16_gemm_bits(x, nullptr, codes_r, scales_r, zeros_r, perm, group_size, 4, out, M, N,
                         K, dtype, workspace, workspace_bytes, stream);
}

int w4a16_dequant_bits(const void* codes_r, const void* scales_r, const void* zeros_r, int64_t K,
                       int64_t N, int32_t group_size, int32_t bits, int32_t dtype, void* w_out,
                       void* stream) {
  return guarded([&]() -> int {
    if (int s = validate_int4_shape(K, N, group_size)) return s;
    if (int s = validate_bits(bits)) return s;
    if (int s = validate_dtype(dtype)) return s;
    if (int s = check_ptrs({codes_r, scales_r, w_out})) return s;
    if (zeros_r && !aligned16(zeros_r)) return W4A16_ERR_MISALIGNED;
    clear_pending_error();
    return hip_status(launch_dequant_int(codes_r, scales_r, zeros_r, K, N,
                                         (int)resolve_group(K, group_size), bits, dtype, w_out,
                                         (hipStream_t)stream));
  });
}

int w4a16_dequant(const void* codes_r, const void* scales_r, const void* zeros_r, int64_t K,
                  int64_t N, int32_t group_size, int32_t dtype, void* w_out, void* stream) {
  return w4a16_dequant_bits(codes_r, scales_r, zeros_r, K, N, group_size, 4, dtype, w_out,
                            stream);
}

int nf4_codebook(float* out16_host) {
  return guarded([&]() -> int {
    if (!out16_host) return W4A16_ERR_INVALID_ARG;
    std::memcpy(out16_host, codebook().v, sizeof(float) * 16);
    return W4A16_OK;
  });
}

static int validate_nf4_shape(int64_t N, int64_t K, int32_t blocksize) {
  if (N <= 0 || K <= 0) return W4A16_ERR_INVALID_ARG;
  if (blocksize != 64) return W4A16_ERR_UNSUPPORTED;
  if (K % 64 != 0) return W4A16_ERR_INVALID_ARG;
  if (too_big(N, K)) return W4A16_ERR_UNSUPPORTED;
  return W4A16_OK;
}

int nf4_quantize(const float* W, int64_t N, int64_t K, int32_t blocksize, uint8_t* qweight,
                 uint8_t* absmax_q, float* absmax_scale, void* stream) {
  return guarded([&]() -> int {
    if (int s = validate_nf4_shape(N, K, blocksize)) return s;
    if (int s = check_ptrs({W, qweight, absmax_q, absmax_scale})) return s;
    clear_pending_error();
    return hip_status(launch_nf4_quant(W, N, K, codebook(), qweight, absmax_q, absmax_scale,
                                       (hipStream_t)stream));
  });
}

int64_t nf4_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t blocksize) {
  if (M <= 0 || validate_nf4_shape(N, K, blocksize) != W4A16_OK || too_big_m(M, N, K))
    return -1;
  return nf4_workspace_bytes_for(M, N, K);
}

static int nf4_plan(int64_t M, int64_t N, int64_t K, int32_t blocksize, int32_t dtype,
                    int32_t has_workspace, char* names_host, int64_t names_bytes,
                    int64_t* names_len_host, bool repacked) {
  return guarded([&]() -> int {
    if (M <= 0) return W4A16_ERR_INVALID_ARG;
    if (int s = validate_nf4_shape(N, K, blocksize)) return s;
    if (N % 16 != 0) return W4A16_ERR_INVALID_ARG;
    if (too_big_m(M, N, K)) return W4A16_ERR_UNSUPPORTED;
    if (int s = validate_dtype(dtype)) return s;
    if (names_bytes < 0 || (names_bytes > 0 && !names_host)) return W4A16_ERR_INVALID_ARG;
    const int64_t len = plan_names(plan_nf4_gemm(M, N, K, dtype, has_workspace != 0, repacked),
                                   names_host, names_bytes);
    if (names_len_host) *names_len_host = len;
    return W4A16_OK;
  });
}

int nf4_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t blocksize, int32_t dtype,
                  int32_t has_workspace, char* names_host, int64_t names_bytes,
                  int64_t* names_len_host) {
  return nf4_plan(M, N, K, blocksize, dtype, has_workspace, names_host, names_bytes,
                  names_len_host, false);
}

int nf4_gemm_repacked_plan(int64_t M, int64_t N, int64_t K, int32_t blocksize, int32_t dtype,
                           int32_t has_workspace, char* names_host, int64_t names_bytes,
                           int64_t* names_len_host) {
  return nf4_plan(M, N, K, blocksize, dtype, has_workspace, names_host, names_bytes,
                  names_len_host, true);
}

int64_t nf4_repacked_bytes(int64_t N, int64_t K, int32_t blocksize) {
  if (validate_nf4_shape(N, K, blocksize) != W4A16_OK || N % 16 != 0) return -1;
  return nf4_repacked_bytes_for(N, K);
}

int nf4_repack(const uint8_t* qweight, int64_t N, int64_t K, int32_t blocksize,
               uint8_t* qweight_r, void* stream) {
  return guarded([&]() -> int {
    if (int s = validate_nf4_shape(N, K, blocksize)) return s;
    if (N % 16 != 0) return W4A16_ERR_INVALID_ARG;
    if (int s = check_ptrs({qweight, qweight_r})) return s;
    clear_pending_error();
    return hip_status(launch_nf4_repack(qweight, N, K, qweight_r, (hipStream_t)stream));
  });
}

static int nf4_gemm_any(const void* x, const uint8_t* qweight, const uint8_t* absmax_q,
                        const float* absmax_scale, int32_t blocksize, void* out, int64_t M,
                        int64_t N, int64_t K, int32_t dtype, void* workspace,
                        int64_t workspace_bytes, void* stream, bool repacked) {
  return guarded([&]() -> int {
    if (M <= 0) return W4A16_ERR_INVALID_ARG;
    if (int s = validate_nf4_shape(N, K, blocksize)) return s;
    if (N % 16 != 0) return W4A16_ERR_INVALID_ARG;
    if (too_big_m(M, N, K)) return W4A16_ERR_UNSUPPORTED;
    if (int s = validate_dtype(dtype)) return s;
    if (int s = check_ptrs({x, qweight, absmax_q, absmax_scale, out})) return s;
    if (workspace && !aligned16(workspace)) return W4A16_ERR_MISALIGNED;
    // NULL workspace: legal, the large-M kernel then does not split K
    if (workspace && workspace_bytes < nf4_workspace_bytes_for(M, N, K))
      return W4A16_ERR_WORKSPACE;
    clear_pending_error();
    return hip_status(launch_nf4_gemm(x, qweight, absmax_q, absmax_scale, codebook(), out, M, N,
                                      K, dtype, workspace, workspace_bytes, repacked,
                                      (hipStream_t)stream));
  });
}

int nf4_gemm(const void* x, const uint8_t* qweight, const uint8_t* absmax_q,
             const float* absmax_scale, int32_t blocksize, void* out, int64_t M, int64_t N,
             int64_t K, int32_t dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  return nf4_gemm_any(x, qweight, absmax_q, absmax_scale, blocksize, out, M, N, K, dtype,
                      workspace, workspace_bytes, stream, false);
}

int nf4_gemm_repacked(const void* x, const uint8_t* qweight_r, const uint8_t* absmax_q,
                      const float* absmax_scale, int32_t blocksize, void* out, int64_t M,
                      int64_t N, int64_t K, int32_t dtype, void* workspace,
                      int64_t workspace_bytes, void* stream) {
  return nf4_gemm_any(x, qweight_r, absmax_q, absmax_scale, blocksize, out, M, N, K, dtype,
                      workspace, workspace_bytes, stream, true);
}

int nf4_dequant(const uint8_t* qweight, const uint8_t* absmax_q, const float* absmax_scale,
                int64_t N, int64_t K, int32_t blocksize, int32_t dtype, void* w_out,
                void* stream) {
  return guarded([&]() -> int {
    if (int s = validate_nf4_shape(N, K, blocksize)) return s;
    if (int s = validate_dtype(dtype)) return s;
    if (int s = check_ptrs({qweight, absmax_q, absmax_scale, w_out})) return s;
    clear_pending_error();
    return hip_status(launch_dequant_nf4(qweight, absmax_q, absmax_scale, N, K, dtype,
                                         codebook(), w_out, (hipStream_t)stream));
  });
}

}  // extern "C"

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

// Split-K plan shared by the GEMM launchers and the workspace-size query.
struct SplitPlan {
  int mt;          // 16-row MFMA tiles per workgroup row block (1, 2 or 4)
  int64_t nrb;     // row blocks of 16 * mt rows
  int64_t ncb;     // column blocks (4 panels of 64 columns each)
  int64_t kt;      // K tiles of 128
  int64_t kt_per;  // K tiles per workgroup
  int64_t nsplit;  // workgroups along K per output tile
  int64_t ws_bytes;
};

SplitPlan plan_int4(int64_t M, int64_t N, int64_t K, bool have_workspace);
SplitPlan plan_nf4(int64_t M, int64_t N, int64_t K, bool have_workspace);

hipError_t launch_rtn_int4(const float* W, const int32_t* perm, int64_t N, int64_t K,
                           int32_t* qweight, uint16_t* scales, int32_t* qzeros,
                           hipStream_t stream);
hipError_t launch_nf4_quant(const float* W, int64_t N, int64_t K, const Nf4Table& L,
                            uint8_t* qweight, uint8_t* absmax_q, float* absmax_scale,
                            hipStream_t stream);
hipError_t launch_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                         const int32_t* perm, int64_t K, int64_t N, void* codes_r,
                         void* scales_r, void* zeros_r, hipStream_t stream);
hipError_t launch_dequant_int4(const void* codes_r, const void* scales_r, const void* zeros_r,
                               int64_t K, int64_t N, int dtype, void* w_out, hipStream_t stream);
hipError_t launch_dequant_nf4(const uint8_t* qweight, const uint8_t* absmax_q,
                              const float* absmax_scale, int64_t N, int64_t K, int dtype,
                              const Nf4Table& L, void* w_out, hipStream_t stream);

hipError_t launch_int4_gemm(const void* x, const void* codes_r, const void* scales_r,
                            const void* zeros_r, const int32_t* perm, void* out, int64_t M,
                            int64_t N, int64_t K, int dtype, void* workspace,
                            int64_t workspace_bytes, hipStream_t stream);
hipError_t launch_nf4_gemm(const void* x, const uint8_t* qweight, const uint8_t* absmax_q,
                           const float* absmax_scale, const Nf4Table& L, void* out, int64_t M,
                           int64_t N, int64_t K, int dtype, void* workspace,
                           int64_t workspace_bytes, hipStream_t stream);

}  // namespace w4a16

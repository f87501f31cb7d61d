// measure.hip -- a plain streaming read of device memory, the practical HBM
// read ceiling the GEMM kernels are measured against ([P5] "关键数据解读"
// item 3: a decode step's time follows the weight bytes it moves, so the
// fastest way to move those bytes bounds the step).  Not on the GEMM path.
//
// Workgroup w of G reads its chunk of the buffer (the bytes split into G
// chunks of whole 4 KB steps): 256 lanes x 16 bytes per step, eight steps in
// flight per lane, buffer loads whose range ends at the buffer's end.  Each
// lane's xor of what it read is stored, so no load can be dropped.
#include "common.h"
#include "kernels.h"
#include "launch.h"

namespace w4a16 {

__global__ void __launch_bounds__(256)
stream_read_kernel(const uint8_t* __restrict__ buf, int64_t bytes, int64_t per,
                   uint32_t* __restrict__ out) {
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t len = b0 < bytes ? (bytes - b0 < per ? bytes - b0 : per) : 0;
  const rsrc_t r = make_rsrc(buf + (b0 < bytes ? b0 : 0), (uint32_t)len);
  const uint32_t voff = threadIdx.x * 16u;
  const int steps = (int)(per / 4096);
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int i = 0; i < steps; i += 8) {
    u32x4_t v[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) v[s] = bld128(r, voff, (i + s) * 4096);
#pragma unroll
    for (int s = 0; s < 8; ++s) acc ^= v[s];
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, int workgroups, uint32_t* out,
                              hipStream_t stream) {
  // whole groups of 8 steps of 4 KB per workgroup
  const int64_t per = ceil_div(ceil_div(bytes, (int64_t)workgroups), (int64_t)32768) * 32768;
  launch_timed(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream,
               (const uint8_t*)buf, bytes, per, out);
  return hipGetLastError();
}

}  // namespace w4a16

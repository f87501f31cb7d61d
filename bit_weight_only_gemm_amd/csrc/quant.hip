// quant.hip -- on-device quantizers (load-time input preparation), the
// offline INT4 repack, and the dequantization export kernels.
//
// None of these is on the per-call GEMM path; they are memory-bound elementwise
// or per-group kernels written for clarity: one wave per quantization group
// (INT4) or per 64-element block (NF4), wave64 shuffles for reductions.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

// ---------------------------------------------------------------- RTN INT4 --
// One wave per (row n, group g of G members); lane holds members u = lane +
// 64 h, read twice (range, then codes).  Codes are OR-ed into the zero-filled
// canonical qweight / qzeros words.  Asymmetric: s = fp16(fp32(max - min) / 15),
// z = clip(rint(-min / s), 0, 15), q = clip(rint(w / s) + z, 0, 15).
// Symmetric (qzeros == nullptr): s = fp16(fp32(max |w|) / 7),
// q = clip(rint(w / s), -8, 7) + 8.  A group whose fp16 scale is 0 uses s = 1.
__global__ void __launch_bounds__(256)
rtn_int4_kernel(const float* __restrict__ W, const int32_t* __restrict__ perm, int64_t N,
                int64_t K, int G, uint32_t* __restrict__ qweight, uint16_t* __restrict__ scales,
                uint32_t* __restrict__ qzeros) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t ng = K / G;
  if (item >= N * ng) return;
  const int64_t g = item / N, n = item % N;  // n fastest across waves
  const bool sym = qzeros == nullptr;
  auto col = [&](int u) -> int64_t {
    const int64_t k = g * G + u;
    return perm ? (int64_t)perm[k] : k;
  };
  float mn = INFINITY, mx = -INFINITY;
  for (int u = lane; u < G; u += 64) {
    const float w = W[n * K + col(u)];
    mn = fminf(mn, w);
    mx = fmaxf(mx, sym ? fabsf(w) : w);
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  _Float16 s16 = sym ? (_Float16)(mx / 7.0f)             // correctly rounded fp32 div, RNE
                     : (_Float16)((mx - mn) / 15.0f);    // fp32 sub + div, RNE
  if (s16 == (_Float16)0.0f) s16 = (_Float16)1.0f;
  const float sf = (float)s16;
  // symmetric: clip(rint(w / s), -8, 7) + 8 is the asymmetric formula with z = 8
  const float z = sym ? 8.0f : fminf(fmaxf(rintf(-mn / sf), 0.0f), 15.0f);
  for (int u = lane; u < G; u += 64) {
    const int64_t k = col(u);
    const float w = W[n * K + k];
    const float q = fminf(fmaxf(rintf(w / sf) + z, 0.0f), 15.0f);
    const uint32_t qi = (uint32_t)q;
    if (qi) atomicOr(&qweight[(k >> 3) * N + n], qi << (4 * (k & 7)));
  }
  if (lane == 0) {
    scales[g * N + n] = __builtin_bit_cast(uint16_t, s16);
    const uint32_t zi = (uint32_t)z;
    if (!sym && zi) atomicOr(&qzeros[g * (N >> 3) + (n >> 3)], zi << (4 * (n & 7)));
  }
}

hipError_t launch_rtn_int4(const float* W, const int32_t* perm, int64_t N, int64_t K, int G,
                           int32_t* qweight, uint16_t* scales, int32_t* qzeros,
                           hipStream_t stream) {
  const int64_t nw = (K / 8) * N, nz = (K / G) * (N / 8);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(nw, 256), 65535)),
                     dim3(256), 0, stream, (uint32_t*)qweight, nw, 0u);
  if (qzeros)
    hipLaunchKernelGGL(fill_u32_kernel,
                       dim3((unsigned)std::min<int64_t>(ceil_div(nz, 256), 65535)), dim3(256), 0,
                       stream, (uint32_t*)qzeros, nz, 0u);
  const int64_t items = N * (K / G);
  hipLaunchKernelGGL(rtn_int4_kernel, dim3((unsigned)ceil_div(items, 4)), dim3(256), 0, stream,
                     W, perm, N, K, G, (uint32_t*)qweight, scales, (uint32_t*)qzeros);
  return hipGetLastError();
}

// -------------------------------------------------------------- NF4 quantizer --
// One workgroup (4 waves) per double-quant group of 256 blocks of 64 elements.
// Each wave walks 64 blocks: lane = element, wave max -> absmax, 16-way argmin
// in fp32 (first minimum), nibble pairs combined with a shuffle.  The block
// absmax values stay in LDS for the group's 8-bit double quantization.
__global__ void __launch_bounds__(256)
nf4_quant_kernel(const float* __restrict__ W, int64_t nblocks, Nf4Table L,
                 uint8_t* __restrict__ qweight, uint8_t* __restrict__ absmax_q,
                 float* __restrict__ absmax_scale) {
  __shared__ float am[256];
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t b0 = (int64_t)blockIdx.x * 256;
  float wmax = 0.0f;
  for (int bi = wave; bi < 256; bi += 4) {
    const int64_t b = b0 + bi;
    if (b >= nblocks) break;
    const float w = W[b * 64 + lane];
    const float a = wave_max(fabsf(w));
    const float v = (a == 0.0f) ? 0.0f : w / a;
    int best = 0;
    float bd = fabsf(v - L.v[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      const float d = fabsf(v - L.v[i]);
      if (d < bd) { bd = d; best = i; }
    }
    const int other = __shfl_xor(best, 1, 64);
    if ((lane & 1) == 0) qweight[b * 32 + (lane >> 1)] = (uint8_t)(best | (other << 4));
    if (lane == 0) am[bi] = a;
    wmax = fmaxf(wmax, a);
  }
  if (lane == 0) red[wave] = wmax;
  __syncthreads();
  const float gmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = gmax / 255.0f;
  const int64_t b = b0 + threadIdx.x;
  if (b < nblocks) {
    const float qv = (sc > 0.0f) ? fminf(fmaxf(rintf(am[threadIdx.x] / sc), 0.0f), 255.0f) : 0.0f;
    absmax_q[b] = (uint8_t)qv;
  }
  if (threadIdx.x == 0) absmax_scale[blockIdx.x] = sc;
}

hipError_t launch_nf4_quant(const float* W, int64_t N, int64_t K, const Nf4Table& L,
                            uint8_t* qweight, uint8_t* absmax_q, float* absmax_scale,
                            hipStream_t stream) {
  const int64_t nblocks = N * K / 64;
  hipLaunchKernelGGL(nf4_quant_kernel, dim3((unsigned)ceil_div(nblocks, 256)), dim3(256), 0,
                     stream, W, nblocks, L, qweight, absmax_q, absmax_scale);
  return hipGetLastError();
}

// --------------------------------------------------------------------- repack --
// One thread per 32-bit output word of the code tiles (coalesced writes).
__global__ void __launch_bounds__(256)
repack_codes_kernel(const uint32_t* __restrict__ qweight, const int32_t* __restrict__ perm,
                    int64_t K, int64_t N, int64_t NP, uint32_t* __restrict__ codes_r) {
  const int64_t KT = K / 128;
  const int64_t total = NP * KT * 4 * 64 * 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int j = (int)(idx & 3);
  const int lane = (int)((idx >> 2) & 63);
  const int c = (int)((idx >> 8) & 3);
  const int64_t pt = idx >> 10;  // p * KT + t
  const int64_t t = pt % KT, p = pt / KT;
  const int64_t n = p * 64 + c * 16 + (lane & 15);
  uint32_t word = 0;
  if (n < N) {
    const int64_t kb = t * 128 + j * 32 + (lane >> 4) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t k = perm ? (int64_t)perm[kb + e] : kb + e;
      const uint32_t q = (qweight[(k >> 3) * N + n] >> (4 * (k & 7))) & 0xFu;
      word |= q << (4 * ((e >> 1) + 4 * (e & 1)));
    }
  }
  codes_r[idx] = word;
}

// One thread per (panel p, run g of 8 K tiles, column tile c, column i): the
// 8 U scales (16 U bytes) and 8 U zero nibbles (U words) of that column, unit
// r of the run being tile 8 g + r / U, unit r % U.
__global__ void __launch_bounds__(256)
repack_meta_kernel(const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros,
                   int64_t K, int64_t N, int64_t NP, int G, uint16_t* __restrict__ scales_r,
                   uint32_t* __restrict__ zeros_r) {
  const int64_t KT = K / 128, KT8 = ceil_div(KT, 8);
  const int U = units_per_tile(G), span = G < 128 ? G : 128;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= NP * KT8 * 64) return;
  const int i = (int)(idx & 15);
  const int c = (int)((idx >> 4) & 3);
  const int64_t pg = idx >> 6;
  const int64_t g = pg % KT8, p = pg / KT8;
  const int64_t n = p * 64 + c * 16 + i;
  for (int w = 0; w < U; ++w) {
    uint32_t zw = 0;
    u32x4_t sv = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t v = g * 8 * U + 8 * w + e;  // unit index
      const int64_t t = v / U;
      uint32_t sb = 0, z = 0;
      if (n < N && t < KT) {
        const int64_t grp = (128 * t + (v % U) * span) / G;
        sb = scales[grp * N + n];
        if (qzeros) z = (qzeros[grp * (N >> 3) + (n >> 3)] >> (4 * (n & 7))) & 0xFu;
      }
      sv[e >> 1] |= sb << (16 * (e & 1));
      zw |= z << (4 * e);
    }
    *(u32x4_t*)(scales_r + (idx * U + w) * 8) = sv;
    if (zeros_r) zeros_r[idx * U + w] = zw;
  }
}

hipError_t launch_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                         const int32_t* perm, int64_t K, int64_t N, int G, void* codes_r,
                         void* scales_r, void* zeros_r, hipStream_t stream) {
  const int64_t NP = ceil_div(N, 64), KT = K / 128;
  const int64_t words = NP * KT * 1024;
  hipLaunchKernelGGL(repack_codes_kernel, dim3((unsigned)ceil_div(words, 256)), dim3(256), 0,
                     stream, (const uint32_t*)qweight, perm, K, N, NP, (uint32_t*)codes_r);
  const int64_t metas = NP * ceil_div(KT, 8) * 64;
  hipLaunchKernelGGL(repack_meta_kernel, dim3((unsigned)ceil_div(metas, 256)), dim3(256), 0,
                     stream, scales, (const uint32_t*)qzeros, K, N, NP, G, (uint16_t*)scales_r,
                     (uint32_t*)zeros_r);
  return hipGetLastError();
}

// ------------------------------------------------------------ dequant exports --
// INT4: one thread per repacked word, through the same dequant_word routine
// the GEMM kernels use; writes 8 consecutive elements (16 bytes) of w [N, K].
template <int DT>
__global__ void __launch_bounds__(256)
dequant_int4_kernel(const uint32_t* __restrict__ codes_r, const uint16_t* __restrict__ scales_r,
                    const uint32_t* __restrict__ zeros_r, int64_t K, int64_t N, int64_t NP,
                    int G, uint16_t* __restrict__ w_out) {
  const int64_t KT = K / 128, KT8 = ceil_div(KT, 8);
  const int U = units_per_tile(G);
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= NP * KT * 1024) return;
  const int j = (int)(idx & 3);
  const int lane = (int)((idx >> 2) & 63);
  const int c = (int)((idx >> 8) & 3);
  const int64_t pt = idx >> 10;
  const int64_t t = pt % KT, p = pt / KT;
  const int i = lane & 15;
  const int64_t n = p * 64 + c * 16 + i;
  if (n >= N) return;
  const int64_t meta = ((p * KT8 + (t >> 3)) * 4 + c) * 16 + i;
  const int r = (int)(t & 7) * U + j * U / 4;  // unit of word j within the run
  const uint32_t z = zeros_r ? (zeros_r[meta * U + (r >> 3)] >> (4 * (r & 7))) & 0xFu : 8u;
  QParam<DT> qp;
  qp.set(scales_r[meta * 8 * U + r], z);
  const auto v = dequant_word(codes_r[idx], qp);
  const int64_t k = t * 128 + j * 32 + (lane >> 4) * 8;
  *(u32x4_t*)(w_out + n * K + k) = __builtin_bit_cast(u32x4_t, v);
}

hipError_t launch_dequant_int4(const void* codes_r, const void* scales_r, const void* zeros_r,
                               int64_t K, int64_t N, int G, int dtype, void* w_out,
                               hipStream_t stream) {
  const int64_t NP = ceil_div(N, 64), KT = K / 128;
  const dim3 grid((unsigned)ceil_div(NP * KT * 1024, 256));
  if (dtype == DT_F16)
    hipLaunchKernelGGL(dequant_int4_kernel<DT_F16>, grid, dim3(256), 0, stream,
                       (const uint32_t*)codes_r, (const uint16_t*)scales_r,
                       (const uint32_t*)zeros_r, K, N, NP, G, (uint16_t*)w_out);
  else
    hipLaunchKernelGGL(dequant_int4_kernel<DT_BF16>, grid, dim3(256), 0, stream,
                       (const uint32_t*)codes_r, (const uint16_t*)scales_r,
                       (const uint32_t*)zeros_r, K, N, NP, G, (uint16_t*)w_out);
  return hipGetLastError();
}

// NF4: one thread per 8 elements (one 32-bit word of packed codes).
template <int DT>
__global__ void __launch_bounds__(256)
dequant_nf4_kernel(const uint32_t* __restrict__ qweight, const uint8_t* __restrict__ absmax_q,
                   const float* __restrict__ absmax_scale, int64_t total_words, Nf4Table L,
                   uint16_t* __restrict__ w_out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total_words) return;
  const int64_t b = idx >> 3;  // 8 words of 8 elements per 64-element block
  const float a = (float)absmax_q[b] * absmax_scale[b >> 8];
  const uint32_t w = qweight[idx];
  uint16_t o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = round16<DT>(L.v[(w >> (4 * e)) & 0xFu] * a);
  u32x4_t v;
#pragma unroll
  for (int h = 0; h < 4; ++h) v[h] = (uint32_t)o[2 * h] | ((uint32_t)o[2 * h + 1] << 16);
  *(u32x4_t*)(w_out + idx * 8) = v;
}

hipError_t launch_dequant_nf4(const uint8_t* qweight, const uint8_t* absmax_q,
                              const float* absmax_scale, int64_t N, int64_t K, int dtype,
                              const Nf4Table& L, void* w_out, hipStream_t stream) {
  const int64_t words = N * K / 8;
  const dim3 grid((unsigned)ceil_div(words, 256));
  if (dtype == DT_F16)
    hipLaunchKernelGGL(dequant_nf4_kernel<DT_F16>, grid, dim3(256), 0, stream,
                       (const uint32_t*)qweight, absmax_q, absmax_scale, words, L,
                       (uint16_t*)w_out);
  else
    hipLaunchKernelGGL(dequant_nf4_kernel<DT_BF16>, grid, dim3(256), 0, stream,
                       (const uint32_t*)qweight, absmax_q, absmax_scale, words, L,
                       (uint16_t*)w_out);
  return hipGetLastError();
}

}  // namespace w4a16

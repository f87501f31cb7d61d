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

// ------------------------------------------------- canonical b-bit packing --
// GPTQ style: each run of L = 32 / gcd(b, 32) consecutive codes (8 at 4 bits,
// 4 at 8 bits, 32 at 3 bits) is a little-endian bit stream of L b / 32 words,
// code e at bits [b e, b e + b); qweight runs along K (word row = run word,
// column n), qzeros runs along N within each group row.
__host__ __device__ constexpr int run_codes(int bits) { return bits == 3 ? 32 : 32 / bits; }

struct BitPos {
  int64_t word;  // run word index along the packed dimension
  int sh;        // bit position in that word (the code continues in word + 1 when sh + b > 32)
};
__device__ __forceinline__ BitPos bit_pos(int64_t i, int bits) {
  const int L = run_codes(bits), nw = L * bits / 32;
  const int pos = bits * (int)(i % L);
  return BitPos{(i / L) * nw + pos / 32, pos % 32};
}

// code (n, k) of a canonical qweight [K b / 32, N]
__device__ __forceinline__ uint32_t canon_code(const uint32_t* __restrict__ qw, int64_t N,
                                               int64_t n, int64_t k, int bits) {
  const BitPos bp = bit_pos(k, bits);
  uint32_t v = qw[bp.word * N + n] >> bp.sh;
  if (bp.sh + bits > 32) v |= qw[(bp.word + 1) * N + n] << (32 - bp.sh);
  return v & ((1u << bits) - 1u);
}

// zero (g, n) of a canonical qzeros [K/G, N b / 32]
__device__ __forceinline__ uint32_t canon_zero(const uint32_t* __restrict__ qz, int64_t N,
                                               int64_t g, int64_t n, int bits) {
  const BitPos bp = bit_pos(n, bits);
  const uint32_t* row = qz + g * (N * bits / 32);
  uint32_t v = row[bp.word] >> bp.sh;
  if (bp.sh + bits > 32) v |= row[bp.word + 1] << (32 - bp.sh);
  return v & ((1u << bits) - 1u);
}

// OR a code into a canonical packed array (its word row stride is `stride`).
__device__ __forceinline__ void canon_or(uint32_t* __restrict__ base, int64_t stride,
                                         int64_t col, int64_t i, uint32_t q, int bits) {
  if (!q) return;
  const BitPos bp = bit_pos(i, bits);
  atomicOr(&base[bp.word * stride + col], q << bp.sh);
  if (bp.sh + bits > 32) atomicOr(&base[(bp.word + 1) * stride + col], q >> (32 - bp.sh));
}

// ------------------------------------------------------------------ RTN INT --
// One wave per (row n, group g of G members); lane holds members u = lane +
// 64 h, read twice (range, then codes).  Codes are OR-ed into the zero-filled
// canonical qweight / qzeros words.  With qmax = 2^b - 1:
// asymmetric: s = fp16(fp32(max - min) / qmax), z = clip(rint(-min / s), 0, qmax),
// q = clip(rint(w / s) + z, 0, qmax).  Symmetric (qzeros == nullptr): s =
// fp16(fp32(max |w|) / (2^(b-1) - 1)), q = clip(rint(w / s), -2^(b-1),
// 2^(b-1) - 1) + 2^(b-1).  A group whose fp16 scale is 0 uses s = 1.
__global__ void __launch_bounds__(256)
rtn_int_kernel(const float* __restrict__ W, const int32_t* __restrict__ perm, int64_t N,
               int64_t K, int G, int bits, uint32_t* __restrict__ qweight,
               uint16_t* __restrict__ scales, uint32_t* __restrict__ qzeros) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t ng = K / G;
  if (item >= N * ng) return;
  const int64_t g = item / N, n = item % N;  // n fastest across waves
  const bool sym = qzeros == nullptr;
  const float qmax = (float)((1 << bits) - 1), half = (float)(1 << (bits - 1));
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
  _Float16 s16 = sym ? (_Float16)(mx / (half - 1.0f))   // correctly rounded fp32 div, RNE
                     : (_Float16)((mx - mn) / qmax);    // fp32 sub + div, RNE
  if (s16 == (_Float16)0.0f) s16 = (_Float16)1.0f;
  const float sf = (float)s16;
  // symmetric: clip(rint(w / s), -h, h - 1) + h is the asymmetric formula with z = h
  const float z = sym ? half : fminf(fmaxf(rintf(-mn / sf), 0.0f), qmax);
  for (int u = lane; u < G; u += 64) {
    const int64_t k = col(u);
    const float w = W[n * K + k];
    const float q = fminf(fmaxf(rintf(w / sf) + z, 0.0f), qmax);
    canon_or(qweight, N, n, k, (uint32_t)q, bits);
  }
  if (lane == 0) {
    scales[g * N + n] = __builtin_bit_cast(uint16_t, s16);
    if (!sym) canon_or(qzeros + g * (N * bits / 32), 1, 0, n, (uint32_t)z, bits);
  }
}

hipError_t launch_rtn_int(const float* W, const int32_t* perm, int64_t N, int64_t K, int G,
                          int bits, int32_t* qweight, uint16_t* scales, int32_t* qzeros,
                          hipStream_t stream) {
  const int64_t nw = (K * bits / 32) * N, nz = (K / G) * (N * bits / 32);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(nw, 256), 65535)),
                     dim3(256), 0, stream, (uint32_t*)qweight, nw, 0u);
  if (qzeros)
    hipLaunchKernelGGL(fill_u32_kernel,
                       dim3((unsigned)std::min<int64_t>(ceil_div(nz, 256), 65535)), dim3(256), 0,
                       stream, (uint32_t*)qzeros, nz, 0u);
  const int64_t items = N * (K / G);
  hipLaunchKernelGGL(rtn_int_kernel, dim3((unsigned)ceil_div(items, 4)), dim3(256), 0, stream,
                     W, perm, N, K, G, bits, (uint32_t*)qweight, scales, (uint32_t*)qzeros);
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
// Dwords per lane of one repacked tile (16 columns x 128 inputs) at b bits.
__host__ __device__ constexpr int tile_lane_dwords(int bits) { return bits == 3 ? 3 : bits == 4 ? 4 : 8; }

// One thread per 32-bit output word of the code tiles (coalesced writes).
// Tile (p, t, c) holds 64 lanes x D dwords: [64][D] at 3 and 4 bits,
// [2 halves][64][4] at 8 bits; lane l = i + 16 b of column 64p + 16c + i.
// The codes of each lane dword (Codes<b> forms of common.h) are read from
// the canonical array through the permutation.
__global__ void __launch_bounds__(256)
repack_codes_kernel(const uint32_t* __restrict__ qweight, const int32_t* __restrict__ perm,
                    int64_t K, int64_t N, int64_t NP, int bits, uint32_t* __restrict__ codes_r) {
  const int64_t KT = K / 128;
  const int D = tile_lane_dwords(bits);
  const int64_t per_tile = 64 * D;
  const int64_t total = NP * KT * 4 * per_tile;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int w = (int)(idx % per_tile);
  const int c = (int)((idx / per_tile) & 3);
  const int64_t pt = idx / per_tile / 4;  // p * KT + t
  const int64_t t = pt % KT, p = pt / KT;
  int lane, d;
  if (bits == 8) {
    lane = (w >> 2) & 63;
    d = 4 * (w >> 8) + (w & 3);
  } else {
    lane = w / D;
    d = w % D;
  }
  const int64_t n = p * 64 + c * 16 + (lane & 15);
  const int b = lane >> 4;
  uint32_t word = 0;
  if (n < N) {
    auto code = [&](int j, int e) -> uint32_t {
      const int64_t kp = t * 128 + 32 * j + 8 * b + e;  // permuted input
      return canon_code(qweight, N, n, perm ? (int64_t)perm[kp] : kp, bits);
    };
    if (bits == 4) {
      for (int e = 0; e < 8; ++e) word |= code(d, e) << (4 * ((e >> 1) + 4 * (e & 1)));
    } else if (bits == 8) {
      const int h = d >> 2, dd = d & 3;
      const int j = 2 * h + (dd >> 1);
      for (int e4 = 0; e4 < 4; ++e4)
        word |= code(j, 4 * (dd & 1) + e4) << (8 * ((e4 >> 1) + 2 * (e4 & 1)));
    } else if (d < 2) {  // 3 bits: low 2 bits of steps 2d, 2d + 1
      for (int jj = 0; jj < 2; ++jj)
        for (int e = 0; e < 8; ++e)
          word |= (code(2 * d + jj, e) & 3u) << (16 * (e & 1) + 2 * (4 * jj + (e >> 1)));
    } else {             // 3 bits: high bits of all 4 steps
      for (int j = 0; j < 4; ++j)
        for (int e = 0; e < 8; ++e)
          word |= (code(j, e) >> 2) << (16 * (e & 1) + 4 * j + (e >> 1));
    }
  }
  codes_r[idx] = word;
}

// One thread per (panel p, run g of 8 K tiles, column tile c, column i): the
// 8 U scales (16 U bytes) and 8 U zero fields of that column, unit r of the
// run being tile 8 g + r / U, unit r % U.  Zero fields are 4 bits wide (8 at
// 8 bits): U or 2U dwords.
__global__ void __launch_bounds__(256)
repack_meta_kernel(const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros,
                   int64_t K, int64_t N, int64_t NP, int G, int bits,
                   uint16_t* __restrict__ scales_r, uint32_t* __restrict__ zeros_r) {
  const int64_t KT = K / 128, KT8 = ceil_div(KT, 8);
  const int U = units_per_tile(G), span = G < 128 ? G : 128;
  const int zw = zero_field_bits(bits), per = 32 / zw, nzw = 8 * U / per;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= NP * KT8 * 64) return;
  const int i = (int)(idx & 15);
  const int c = (int)((idx >> 4) & 3);
  const int64_t pg = idx >> 6;
  const int64_t g = pg % KT8, p = pg / KT8;
  const int64_t n = p * 64 + c * 16 + i;
  for (int w = 0; w < U; ++w) {
    u32x4_t sv = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t v = g * 8 * U + 8 * w + e;  // unit index
      const int64_t t = v / U;
      uint32_t sb = 0;
      if (n < N && t < KT) sb = scales[((128 * t + (v % U) * span) / G) * N + n];
      sv[e >> 1] |= sb << (16 * (e & 1));
    }
    *(u32x4_t*)(scales_r + (idx * U + w) * 8) = sv;
  }
  if (!zeros_r) return;
  for (int w = 0; w < nzw; ++w) {
    uint32_t zv = 0;
    for (int f = 0; f < per; ++f) {
      const int64_t v = g * 8 * U + per * w + f;
      const int64_t t = v / U;
      if (n < N && t < KT)
        zv |= canon_zero(qzeros, N, (128 * t + (v % U) * span) / G, n, bits) << (zw * f);
    }
    zeros_r[idx * nzw + w] = zv;
  }
}

hipError_t launch_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                         const int32_t* perm, int64_t K, int64_t N, int G, int bits,
                         void* codes_r, void* scales_r, void* zeros_r, hipStream_t stream) {
  const int64_t NP = ceil_div(N, 64), KT = K / 128;
  const int64_t words = NP * KT * 4 * 64 * tile_lane_dwords(bits);
  hipLaunchKernelGGL(repack_codes_kernel, dim3((unsigned)ceil_div(words, 256)), dim3(256), 0,
                     stream, (const uint32_t*)qweight, perm, K, N, NP, bits,
                     (uint32_t*)codes_r);
  const int64_t metas = NP * ceil_div(KT, 8) * 64;
  hipLaunchKernelGGL(repack_meta_kernel, dim3((unsigned)ceil_div(metas, 256)), dim3(256), 0,
                     stream, scales, (const uint32_t*)qzeros, K, N, NP, G, bits,
                     (uint16_t*)scales_r, (uint32_t*)zeros_r);
  return hipGetLastError();
}

// ------------------------------------------------------------ dequant exports --
// b-bit integer codes: one thread per (tile, lane, step j): the lane's codes
// and the unit's scale and zero through the same dequant_step routine the
// GEMM kernels use; writes 8 consecutive elements (16 bytes) of w [N, K].
template <int DT, int BITS>
__global__ void __launch_bounds__(256)
dequant_int_kernel(const uint8_t* __restrict__ codes_r, const uint16_t* __restrict__ scales_r,
                   const uint32_t* __restrict__ zeros_r, int64_t K, int64_t N, int64_t NP,
                   int G, uint16_t* __restrict__ w_out) {
  constexpr int kTile = 256 * BITS, kZW = zero_field_bits(BITS), per = 32 / kZW;
  const int64_t KT = K / 128, KT8 = ceil_div(KT, 8);
  const int U = units_per_tile(G), nzw = 8 * U / per;
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
  const uint8_t* tile = codes_r + (pt * 4 + c) * kTile;
  Codes<BITS> w;
  if constexpr (BITS == 4) {
    w.w = *(const u32x4_t*)(tile + lane * 16);
  } else if constexpr (BITS == 3) {
    const uint32_t* q = (const uint32_t*)(tile + lane * 12);
    w.w = u32x3_t{q[0], q[1], q[2]};
  } else {
    w.lo = *(const u32x4_t*)(tile + lane * 16);
    w.hi = *(const u32x4_t*)(tile + 1024 + lane * 16);
  }
  const int64_t meta = ((p * KT8 + (t >> 3)) * 4 + c) * 16 + i;
  const int r = (int)(t & 7) * U + j * U / 4;  // unit of step j within the run
  const uint32_t z = zeros_r ? (zeros_r[meta * nzw + r / per] >> (kZW * (r % per))) &
                                   ((1u << kZW) - 1u)
                             : (1u << (BITS - 1));
  QParam<DT> qp;
  qp.template set<BITS == 4>(scales_r[meta * 8 * U + r], z);
  const auto v = dequant_step<DT>(w, j, qp);
  const int64_t k = t * 128 + j * 32 + (lane >> 4) * 8;
  *(u32x4_t*)(w_out + n * K + k) = __builtin_bit_cast(u32x4_t, v);
}

template <int DT>
static void launch_dequant_int_dt(const void* codes_r, const void* scales_r, const void* zeros_r,
                                  int64_t K, int64_t N, int G, int bits, void* w_out,
                                  hipStream_t stream) {
  const int64_t NP = ceil_div(N, 64), KT = K / 128;
  const dim3 grid((unsigned)ceil_div(NP * KT * 1024, 256));
  auto args = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, (const uint8_t*)codes_r,
                       (const uint16_t*)scales_r, (const uint32_t*)zeros_r, K, N, NP, G,
                       (uint16_t*)w_out);
  };
  if (bits == 4) args(dequant_int_kernel<DT, 4>);
  else if (bits == 3) args(dequant_int_kernel<DT, 3>);
  else args(dequant_int_kernel<DT, 8>);
}

hipError_t launch_dequant_int(const void* codes_r, const void* scales_r, const void* zeros_r,
                              int64_t K, int64_t N, int G, int bits, int dtype, void* w_out,
                              hipStream_t stream) {
  if (dtype == DT_F16)
    launch_dequant_int_dt<DT_F16>(codes_r, scales_r, zeros_r, K, N, G, bits, w_out, stream);
  else
    launch_dequant_int_dt<DT_BF16>(codes_r, scales_r, zeros_r, K, N, G, bits, w_out, stream);
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

// NF4 codes into tiles of 16 rows x 128 inputs: one thread per 16-byte chunk
// (c, t, l) of the output, at byte 16 ((c KT + t) 64 + l), holding bytes
// 64 t + 16 (l >> 4) .. + 15 of row 16 c + (l & 15) (rows are K / 2 bytes,
// a multiple of 32, so a chunk lies wholly inside the row or wholly past it:
// then zeros).
__global__ void __launch_bounds__(256)
nf4_repack_kernel(const uint8_t* __restrict__ qweight, int64_t rowb, int KT, int64_t chunks,
                  uint8_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= chunks) return;
  const int l = (int)(idx & 63);
  const int64_t ct = (idx >> 6) / KT;
  const int t = (int)((idx >> 6) - ct * KT);
  const int64_t b0 = 64 * (int64_t)t + 16 * (l >> 4);
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (b0 < rowb) v = *(const u32x4_t*)(qweight + (16 * ct + (l & 15)) * rowb + b0);
  *(u32x4_t*)(out + idx * 16) = v;
}

hipError_t launch_nf4_repack(const uint8_t* qweight, int64_t N, int64_t K, uint8_t* qweight_r,
                             hipStream_t stream) {
  const int KT = (int)((K + 127) / 128);
  const int64_t chunks = N / 16 * KT * 64;
  hipLaunchKernelGGL(nf4_repack_kernel, dim3((unsigned)ceil_div(chunks, (int64_t)256)),
                     dim3(256), 0, stream, qweight, K / 2, KT, chunks, qweight_r);
  return hipGetLastError();
}

}  // namespace w4a16

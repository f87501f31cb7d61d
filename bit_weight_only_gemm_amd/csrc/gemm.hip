// gemm.hip -- fused dequantize-and-multiply kernels (INT4 and NF4) for gfx950.
//
// The method is the fused kernel of [P5] "LLM量化技术深度对比..." "关键数据解读"
// item 1: the 4-bit weights are turned into 16-bit values in registers right
// before the multiply and are never written back to memory, so each call moves
// only the 4-bit codes plus their scales (decode time tracks weight bytes,
// item 3 of the same section).
//
// Work decomposition (skinny M, memory bound):
//  * A workgroup is 4 waves.  Wave w owns one 64-column panel (4 MFMA column
//    tiles of 16) of a 256-column block and a range of K tiles of 128; the 4
//    waves share the same K range, so the activation slice for that range is
//    staged in LDS once per workgroup, already in MFMA operand order.  For an
//    act-order weight the staging gathers x[:, perm[k]] here, fused into the
//    load (no separate permutation pass).
//  * Per K tile a lane issues four 16-byte loads (one per column tile) of
//    consecutive, fully coalesced 1 KB code tiles, dequantizes each 32-bit word
//    into an 8-element MFMA operand and issues v_mfma_f32_16x16x32_{f16,bf16}
//    with the M rows padded to 16 (x rows >= M are zero in LDS).
//  * Split-K: when a workspace is given, the K range is split over several
//    workgroups; each writes fp32 partial sums, and the last workgroup to
//    arrive (device-scope atomic counter) adds them in split order and writes
//    the rounded output, then re-arms the counter.  The reduction order is
//    fixed, so results are bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

// LDS activation staging capacity: 8 units of (one K tile x one 16-row tile)
// of 4 KB each = 32 KB per workgroup.
constexpr int XS_UNITS = 8;

// --------------------------------------------------------------- INT4 policy --
// Tile (panel p, group t): 4 column tiles x 64 lanes x 16 bytes of codes,
// 16 x 4 fp16 scales, 16 packed zero nibble quads.  Word j of a lane covers
// K = 32j + 8(lane >> 4) + e of the tile, which fixes the x staging order.
template <int DT>
struct Int4W {
  const u32x4_t* codes;
  const uint2* scales;
  const uint16_t* zeros;
  int KT;
  u32x4_t cw[4];
  uint2 sc;
  uint32_t zz;
  __device__ __forceinline__ void load(int panel, int t, int lane, int /*N*/, int /*K*/) {
    const size_t tile = (size_t)panel * KT + t;
#pragma unroll
    for (int c = 0; c < 4; ++c) cw[c] = codes[tile * 256 + c * 64 + lane];
    sc = scales[tile * 16 + (lane & 15)];
    zz = zeros[tile * 16 + (lane & 15)];
  }
  // operand for column tile c, MFMA step j
  __device__ __forceinline__ void operands(int c, typename Op<DT>::vec b[4]) const {
    QParam<DT> qp;
    const uint32_t sbits = ((c < 2 ? sc.x : sc.y) >> (16 * (c & 1))) & 0xFFFFu;
    qp.set(sbits, (zz >> (4 * c)) & 0xFu);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = dequant_word(cw[c][j], qp);
  }
  // K offset (within the 128-wide tile) of the 8 x values lane-group b feeds in step j
  __device__ static __forceinline__ int xk(int j, int b) { return 32 * j + 8 * b; }
};

// ---------------------------------------------------------------- NF4 policy --
// Raw bitsandbytes-style layout: row n of qweight holds K/2 bytes, element 2j
// in the low nibble of byte j.  Lane (column i = lane & 15, group b = lane >> 4)
// loads 16 bytes = 32 consecutive elements k0 + 32b .. k0 + 32b + 31 of its
// column, all inside one 64-element absmax block; word j of the load feeds MFMA
// step j.  Dequant follows the definition exactly: a' = fp32(absmax_q) * scale,
// w = round16(fp32(L[c] * a')).
template <int DT>
struct Nf4W {
  const uint8_t* q;
  const uint8_t* aq;
  const float* asc;
  const float* lut;  // 16 fp32 levels in LDS
  u32x4_t cw[4];
  float a[4];
  __device__ __forceinline__ void load(int panel, int t, int lane, int N, int K) {
    const int b = lane >> 4;
    const int k = t * 128 + 32 * b;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int n = panel * 64 + c * 16 + (lane & 15);
      if (n < N && k < K) {
        cw[c] = *(const u32x4_t*)(q + (size_t)n * (K >> 1) + (k >> 1));
        const size_t blk = ((size_t)n * K + k) >> 6;
        a[c] = (float)aq[blk] * asc[blk >> 8];
      } else {
        cw[c] = u32x4_t{0, 0, 0, 0};
        a[c] = 0.0f;
      }
    }
  }
  __device__ __forceinline__ void operands(int c, typename Op<DT>::vec b[4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = cw[c][j];
      typename Op<DT>::vec v;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = lut[(w >> (4 * e)) & 0xFu] * a[c];
        if constexpr (DT == DT_F16) v[e] = (_Float16)f;
        else v[e] = (__bf16)f;
      }
      b[j] = v;
    }
  }
  __device__ static __forceinline__ int xk(int j, int b) { return 32 * b + 8 * j; }
};

template <int DT, int MT, bool PERM, class WP>
__device__ __forceinline__ void gemm_body(const uint16_t* __restrict__ x,
                                          const int32_t* __restrict__ perm, WP& wp,
                                          uint16_t* __restrict__ out, uint32_t* __restrict__ cnt,
                                          float* __restrict__ part, int M, int N, int K, int NP,
                                          int KT, int kt_per, int nsplit, u32x4_t* xs) {
  __shared__ uint32_t s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cb = blockIdx.x, sp = blockIdx.y, rb = blockIdx.z;
  const int row0 = rb * 16 * MT;
  const int panel = cb * 4 + wave;
  const bool active = panel < NP;
  const int kt0 = sp * kt_per;
  const int kt1 = min(KT, kt0 + kt_per);
  constexpr int CH = XS_UNITS / MT;  // K tiles per staged chunk

  float4_t acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[m][c] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int c0 = kt0; c0 < kt1; c0 += CH) {
    const int nct = min(CH, kt1 - c0);
    if (active) wp.load(panel, c0, lane, N, K);  // first tile's weights in flight
    __syncthreads();                             // previous chunk fully consumed
    // ---- stage x[row0 .. row0+16MT, K chunk] in MFMA A-operand order
    const int units = nct * MT * 256;
    for (int idx = tid; idx < units; idx += 256) {
      const int l = idx & 63, j = (idx >> 6) & 3, r = idx >> 8;
      const int mt = r % MT, t = r / MT;
      const int row = row0 + mt * 16 + (l & 15);
      const int kp = (c0 + t) * 128 + WP::xk(j, l >> 4);
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row < M && kp < K) {
        const uint16_t* xr = x + (size_t)row * K;
        if constexpr (!PERM) {
          v = *(const u32x4_t*)(xr + kp);
        } else {
#pragma unroll
          for (int h = 0; h < 4; ++h)
            v[h] = (uint32_t)xr[perm[kp + 2 * h]] | ((uint32_t)xr[perm[kp + 2 * h + 1]] << 16);
        }
      }
      xs[idx] = v;
    }
    __syncthreads();
    if (active) {
      for (int t = 0; t < nct; ++t) {
        WP cur = wp;
        if (t + 1 < nct) wp.load(panel, c0 + t + 1, lane, N, K);  // prefetch next tile
        typename Op<DT>::vec a[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            a[m][j] = __builtin_bit_cast(typename Op<DT>::vec, xs[((t * MT + m) * 4 + j) * 64 + lane]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          typename Op<DT>::vec b[4];
          cur.operands(c, b);
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m][c] = mfma16x16x32<DT>(a[m][j], b[j], acc[m][c]);
        }
      }
    }
  }

  // ---- epilogue.  v_mfma_f32_16x16x32 result layout: element i of lane l is
  // row 4 * (l >> 4) + i, column l & 15 of the 16x16 tile.
  const int rsub = 4 * (lane >> 4);
  if (nsplit == 1) {
    if (!active) return;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = panel * 64 + c * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = row0 + m * 16 + rsub + i;
          if (row < M && col < N) out[(size_t)row * N + col] = round16<DT>(acc[m][c][i]);
        }
      }
    return;
  }
  const int Np = NP * 64;
  if (active) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = panel * 64 + c * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = row0 + m * 16 + rsub + i;
          if (row < M) part[((size_t)sp * M + row) * Np + col] = acc[m][c][i];
        }
      }
  }
  __threadfence();
  __syncthreads();
  uint32_t* ctr = cnt + (size_t)rb * gridDim.x + cb;
  if (tid == 0) s_last = (atomicAdd(ctr, 1u) == (uint32_t)(nsplit - 1)) ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int col = cb * 256 + tid;
  if (col < N) {
    for (int r = 0; r < 16 * MT; ++r) {
      const int row = row0 + r;
      if (row >= M) break;
      float s = 0.0f;
      for (int q = 0; q < nsplit; ++q) s += part[((size_t)q * M + row) * Np + col];
      out[(size_t)row * N + col] = round16<DT>(s);
    }
  }
  if (tid == 0) *ctr = 0u;  // re-arm for the next call
}

template <int DT, int MT, bool PERM>
__global__ void __launch_bounds__(256)
int4_gemm_kernel(const uint16_t* __restrict__ x, const u32x4_t* __restrict__ codes,
                 const uint2* __restrict__ scales, const uint16_t* __restrict__ zeros,
                 const int32_t* __restrict__ perm, uint16_t* __restrict__ out,
                 uint32_t* __restrict__ cnt, float* __restrict__ part, int M, int N, int K,
                 int NP, int KT, int kt_per, int nsplit) {
  __shared__ u32x4_t xs[XS_UNITS * 256];
  Int4W<DT> wp;
  wp.codes = codes;
  wp.scales = scales;
  wp.zeros = zeros;
  wp.KT = KT;
  gemm_body<DT, MT, PERM>(x, perm, wp, out, cnt, part, M, N, K, NP, KT, kt_per, nsplit, xs);
}

template <int DT, int MT>
__global__ void __launch_bounds__(256)
nf4_gemm_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q,
                const uint8_t* __restrict__ aq, const float* __restrict__ asc, Nf4Table L,
                uint16_t* __restrict__ out, uint32_t* __restrict__ cnt,
                float* __restrict__ part, int M, int N, int K, int NP, int KT, int kt_per,
                int nsplit) {
  __shared__ u32x4_t xs[XS_UNITS * 256];
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = L.v[threadIdx.x];
  Nf4W<DT> wp;
  wp.q = q;
  wp.aq = aq;
  wp.asc = asc;
  wp.lut = lut;
  __syncthreads();
  gemm_body<DT, MT, false>(x, nullptr, wp, out, cnt, part, M, N, K, NP, KT, kt_per, nsplit, xs);
}

// ---------------------------------------------------------------- planning --
static int g_target_wgs = 512;

SplitPlan plan_common(int64_t M, int64_t N, int64_t K, bool have_ws) {
  SplitPlan p;
  p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.nrb = ceil_div(M, 16 * p.mt);
  const int64_t NP = ceil_div(N, 64);
  p.ncb = ceil_div(NP, 4);
  p.kt = ceil_div(K, 128);
  p.nsplit = 1;
  if (have_ws) {
    const int64_t base = p.ncb * p.nrb;
    p.nsplit = std::max<int64_t>(1, std::min<int64_t>(p.kt, ceil_div(g_target_wgs, base)));
  }
  p.kt_per = ceil_div(p.kt, p.nsplit);
  p.nsplit = ceil_div(p.kt, p.kt_per);
  p.ws_bytes = 0;
  if (p.nsplit > 1) {
    const int64_t cnt_bytes = ceil_div(p.nrb * p.ncb * 4, 256) * 256;
    p.ws_bytes = cnt_bytes + p.nsplit * M * NP * 64 * 4;
  }
  return p;
}

SplitPlan plan_int4(int64_t M, int64_t N, int64_t K, bool have_ws) {
  return plan_common(M, N, K, have_ws);
}
SplitPlan plan_nf4(int64_t M, int64_t N, int64_t K, bool have_ws) {
  return plan_common(M, N, K, have_ws);
}

void set_target_wgs(int v) { g_target_wgs = v > 0 ? v : 512; }

template <int DT, int MT>
static void launch_int4_mt(const void* x, const void* codes_r, const void* scales_r,
                           const void* zeros_r, const int32_t* perm, void* out, int64_t M,
                           int64_t N, int64_t K, const SplitPlan& p, uint32_t* cnt, float* part,
                           hipStream_t stream) {
  const dim3 grid((unsigned)p.ncb, (unsigned)p.nsplit, (unsigned)p.nrb);
  const int NP = (int)ceil_div(N, 64);
  if (perm)
    hipLaunchKernelGGL((int4_gemm_kernel<DT, MT, true>), grid, dim3(256), 0, stream,
                       (const uint16_t*)x, (const u32x4_t*)codes_r, (const uint2*)scales_r,
                       (const uint16_t*)zeros_r, perm, (uint16_t*)out, cnt, part, (int)M,
                       (int)N, (int)K, NP, (int)p.kt, (int)p.kt_per, (int)p.nsplit);
  else
    hipLaunchKernelGGL((int4_gemm_kernel<DT, MT, false>), grid, dim3(256), 0, stream,
                       (const uint16_t*)x, (const u32x4_t*)codes_r, (const uint2*)scales_r,
                       (const uint16_t*)zeros_r, perm, (uint16_t*)out, cnt, part, (int)M,
                       (int)N, (int)K, NP, (int)p.kt, (int)p.kt_per, (int)p.nsplit);
}

static void split_ws(const SplitPlan& p, void* ws, uint32_t** cnt, float** part) {
  *cnt = nullptr;
  *part = nullptr;
  if (p.nsplit > 1) {
    *cnt = (uint32_t*)ws;
    *part = (float*)((char*)ws + ceil_div(p.nrb * p.ncb * 4, 256) * 256);
  }
}

hipError_t launch_int4_gemm(const void* x, const void* codes_r, const void* scales_r,
                            const void* zeros_r, const int32_t* perm, void* out, int64_t M,
                            int64_t N, int64_t K, int dtype, void* workspace,
                            int64_t /*workspace_bytes*/, hipStream_t stream) {
  const SplitPlan p = plan_int4(M, N, K, workspace != nullptr);
  uint32_t* cnt;
  float* part;
  split_ws(p, workspace, &cnt, &part);
#define W4_LAUNCH(DTV, MTV) \
  launch_int4_mt<DTV, MTV>(x, codes_r, scales_r, zeros_r, perm, out, M, N, K, p, cnt, part, stream)
  if (dtype == DT_F16) {
    if (p.mt == 1) W4_LAUNCH(DT_F16, 1);
    else if (p.mt == 2) W4_LAUNCH(DT_F16, 2);
    else W4_LAUNCH(DT_F16, 4);
  } else {
    if (p.mt == 1) W4_LAUNCH(DT_BF16, 1);
    else if (p.mt == 2) W4_LAUNCH(DT_BF16, 2);
    else W4_LAUNCH(DT_BF16, 4);
  }
#undef W4_LAUNCH
  return hipGetLastError();
}

template <int DT, int MT>
static void launch_nf4_mt(const void* x, const uint8_t* q, const uint8_t* aq, const float* asc,
                          const Nf4Table& L, void* out, int64_t M, int64_t N, int64_t K,
                          const SplitPlan& p, uint32_t* cnt, float* part, hipStream_t stream) {
  const dim3 grid((unsigned)p.ncb, (unsigned)p.nsplit, (unsigned)p.nrb);
  hipLaunchKernelGGL((nf4_gemm_kernel<DT, MT>), grid, dim3(256), 0, stream, (const uint16_t*)x, q,
                     aq, asc, L, (uint16_t*)out, cnt, part, (int)M, (int)N, (int)K,
                     (int)ceil_div(N, 64), (int)p.kt, (int)p.kt_per, (int)p.nsplit);
}

hipError_t launch_nf4_gemm(const void* x, const uint8_t* qweight, const uint8_t* absmax_q,
                           const float* absmax_scale, const Nf4Table& L, void* out, int64_t M,
                           int64_t N, int64_t K, int dtype, void* workspace,
                           int64_t /*workspace_bytes*/, hipStream_t stream) {
  const SplitPlan p = plan_nf4(M, N, K, workspace != nullptr);
  uint32_t* cnt;
  float* part;
  split_ws(p, workspace, &cnt, &part);
#define NF_LAUNCH(DTV, MTV) \
  launch_nf4_mt<DTV, MTV>(x, qweight, absmax_q, absmax_scale, L, out, M, N, K, p, cnt, part, stream)
  if (dtype == DT_F16) {
    if (p.mt == 1) NF_LAUNCH(DT_F16, 1);
    else if (p.mt == 2) NF_LAUNCH(DT_F16, 2);
    else NF_LAUNCH(DT_F16, 4);
  } else {
    if (p.mt == 1) NF_LAUNCH(DT_BF16, 1);
    else if (p.mt == 2) NF_LAUNCH(DT_BF16, 2);
    else NF_LAUNCH(DT_BF16, 4);
  }
#undef NF_LAUNCH
  return hipGetLastError();
}

}  // namespace w4a16

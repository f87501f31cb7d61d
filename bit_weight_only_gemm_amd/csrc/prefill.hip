// prefill.hip -- large-M fused dequantize-and-multiply for INT4 weights.
//
// Same product as the decode kernel ([P5] "LLM量化技术深度对比..." "关键数据解读"
// item 1: the 4-bit weights are expanded in registers, never in memory), for
// M large enough that the multiply, not the weight stream, bounds the call.
//
//  * One workgroup computes a 256 x 256 output tile with 4 waves; wave w owns
//    the 64-column panel 4 bx + w for all 256 rows (16 x 4 MFMA tiles of
//    16 x 16, fp32 accumulators).
//  * Activations: each K tile (128 inputs) of the 256 rows is loaded once per
//    workgroup, 16 bytes per lane, and staged in LDS (64 KB per stage, two
//    stages); the 16-byte chunk q of row r sits at chunk position q ^ (r & 15)
//    of its 256-byte LDS row, so the MFMA operand reads (16 rows, one chunk
//    each) hit distinct banks.
//  * Weights: the repacked code tile is already the B operand layout of
//    v_mfma_f32_16x16x32, so each wave loads its 4 column tiles straight into
//    registers (one 16-byte load per lane each) and dequantizes them exactly
//    with the routine of the dequant export.  Each weight is therefore read
//    and dequantized once per workgroup, and B never passes through LDS.
//  * The loads of K tile t + 1 are issued before the MFMAs of tile t and land
//    in the other LDS stage after them; one barrier per K tile.
#include "common.h"
#include "kernels.h"
#include "launch.h"

namespace w4a16 {

constexpr int PF_WAVES = 4;                  // waves per workgroup
constexpr int PF_BM = 256;                   // rows per workgroup
constexpr int PF_MT = PF_BM / 16;            // 16-row MFMA tiles per wave
constexpr int PF_ROWB = 256;                 // LDS bytes of one row of a K tile
constexpr int PF_STAGE = PF_BM * PF_ROWB;    // 64 KB
constexpr int PF_ALD = PF_BM * 16 / (64 * PF_WAVES);  // 16-byte A chunks per thread

template <int DT>
__global__ void __launch_bounds__(64 * PF_WAVES) __attribute__((amdgpu_waves_per_eu(1, 1)))
int4_prefill_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
                    const uint8_t* __restrict__ scales, const uint8_t* __restrict__ zeros,
                    uint16_t* __restrict__ out, int M, int N, int K, int KT, int NP) {
  typedef typename Op<DT>::vec vec;
  __shared__ __attribute__((aligned(16))) uint8_t As[2 * PF_STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = blockIdx.y * PF_BM;
  const int p = blockIdx.x * PF_WAVES + wave;  // this wave's 64-column panel
  const int KT8 = (KT + 7) >> 3;

  // ---- activations: rows row0 .. row0 + vrows - 1 of x; rows past M read 0
  const int vrows = min(PF_BM, M - row0);
  const rsrc_t rx = make_rsrc(x + (size_t)row0 * K, (uint32_t)vrows * (uint32_t)K * 2u);
  // thread's chunks: row i * 16 + ar, chunk aq (i = 0 .. PF_ALD - 1)
  const int aq = tid & 15, ar = tid >> 4;
  const uint32_t arow_bytes = (uint32_t)K * 2u;
  const uint32_t avoff = (uint32_t)ar * arow_bytes + (uint32_t)aq * 16u;
  const uint32_t astride = 16u * arow_bytes;
  const int aw = ar * PF_ROWB + ((aq ^ ar) << 4);  // (i * 16 + ar) & 15 == ar

  // ---- weights of panel p (all loads return 0 for a panel past the last)
  const bool pv = p < NP;
  const size_t pp = pv ? (size_t)p : 0;
  const rsrc_t rc = make_rsrc(codes + pp * KT * 4096, pv ? (uint32_t)KT * 4096u : 0u);
  const rsrc_t rs = make_rsrc(scales + pp * KT8 * 1024, pv ? (uint32_t)KT8 * 1024u : 0u);
  const rsrc_t rz = make_rsrc(zeros + pp * KT8 * 256, pv ? (uint32_t)KT8 * 256u : 0u);
  const int i16 = lane & 15;

  float4_t acc[PF_MT][4];
#pragma unroll
  for (int m = 0; m < PF_MT; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[m][c] = float4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ast[PF_ALD];
  u32x4_t cw[4], cn[4];
  uint32_t sc[4], zz[4], sn[4], zn[4];

  // ---- prologue: K tile 0
#pragma unroll
  for (int i = 0; i < PF_ALD; ++i) ast[i] = bld128(rx, avoff + (uint32_t)i * astride, 0);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    cw[c] = bld128(rc, (uint32_t)(c * 1024 + lane * 16), 0);
    sc[c] = bld16(rs, (uint32_t)((c * 16 + i16) * 16), 0);
    zz[c] = bld32(rz, (uint32_t)((c * 16 + i16) * 4), 0);
  }
#pragma unroll
  for (int i = 0; i < PF_ALD; ++i) *(u32x4_t*)(As + aw + i * 16 * PF_ROWB) = ast[i];
  __syncthreads();

  for (int t = 0; t < KT; ++t) {
    // ---- issue K tile t + 1 (the last tile is re-read on the final pass)
    const int tn = min(t + 1, KT - 1);
#pragma unroll
    for (int i = 0; i < PF_ALD; ++i)
      ast[i] = bld128(rx, avoff + (uint32_t)i * astride, tn * 256);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      cn[c] = bld128(rc, (uint32_t)(c * 1024 + lane * 16), tn * 4096);
      sn[c] = bld16(rs, (uint32_t)((c * 16 + i16) * 16), (tn >> 3) * 1024 + (tn & 7) * 2);
      zn[c] = bld32(rz, (uint32_t)((c * 16 + i16) * 4), (tn >> 3) * 256);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- K tile t from LDS stage t & 1
    QParam<DT> qp[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) qp[c].set(sc[c] & 0xFFFFu, (zz[c] >> (4 * (t & 7))) & 0xFu);
    const uint8_t* st = As + (t & 1) * PF_STAGE;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vec b[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) b[c] = dequant_word(cw[c][j], qp[c]);
      const int q = 4 * j + (lane >> 4);  // chunk of step j for this lane's K group
#pragma unroll
      for (int m = 0; m < PF_MT; ++m) {
        const vec a = *(const vec*)(st + (m * 16 + i16) * PF_ROWB + ((q ^ i16) << 4));
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[m][c] = mfma16x16x32<DT>(a, b[c], acc[m][c]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- stage K tile t + 1 (stage (t + 1) & 1 was last read before the
    // previous barrier)
    uint8_t* sw = As + ((t + 1) & 1) * PF_STAGE;
#pragma unroll
    for (int i = 0; i < PF_ALD; ++i) *(u32x4_t*)(sw + aw + i * 16 * PF_ROWB) = ast[i];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      cw[c] = cn[c];
      sc[c] = sn[c];
      zz[c] = zn[c];
    }
    __syncthreads();
  }

  // ---- epilogue: element e of lane l is row 4 (l >> 4) + e, column l & 15
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int col = p * 64 + c * 16 + i16;
    if (col < N) {
#pragma unroll
      for (int m = 0; m < PF_MT; ++m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = row0 + m * 16 + 4 * (lane >> 4) + e;
          if (row < M) out[(size_t)row * N + col] = round16<DT>(acc[m][c][e]);
        }
      }
    }
  }
}

void launch_int4_prefill(const void* x, const void* codes_r, const void* scales_r,
                         const void* zeros_r, void* out, int64_t M, int64_t N, int64_t K,
                         int dtype, hipStream_t stream) {
  const int64_t NP = ceil_div(N, 64);
  const dim3 grid((unsigned)ceil_div(NP, PF_WAVES), (unsigned)ceil_div(M, PF_BM));
  const int KT = (int)(K / 128);
  if (dtype == DT_F16)
    launch_timed(int4_prefill_kernel<DT_F16>, grid, dim3(64 * PF_WAVES), 0, stream,
                 (const uint16_t*)x, (const uint8_t*)codes_r, (const uint8_t*)scales_r,
                 (const uint8_t*)zeros_r, (uint16_t*)out, (int)M, (int)N, (int)K, KT, (int)NP);
  else
    launch_timed(int4_prefill_kernel<DT_BF16>, grid, dim3(64 * PF_WAVES), 0, stream,
                 (const uint16_t*)x, (const uint8_t*)codes_r, (const uint8_t*)scales_r,
                 (const uint8_t*)zeros_r, (uint16_t*)out, (int)M, (int)N, (int)K, KT, (int)NP);
}

}  // namespace w4a16

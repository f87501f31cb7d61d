// prefill.hip -- large-M fused dequantize-and-multiply (integer codes of 3, 4
// or 8 bits, and NF4): planning, dispatch and the 4-bit and NF4
// instantiations of the kernel in prefill.h.
//
// Same product as the decode kernel ([P5] "LLM量化技术深度对比..." "关键数据解读"
// item 1: the 4-bit weights are expanded in registers, never in memory), for
// M large enough that the multiply, not the weight stream, bounds the call.
//
//  * One workgroup computes a 256 x 256 output tile with 4 waves; wave w owns
//    the 64-column panel 4 bx + w for all 256 rows: 8 x 2 tiles of 32 x 32 on
//    v_mfma_f32_32x32x16_{f16,bf16} (on gfx950 this shape sustains a much
//    higher fraction of the matrix peak than 16x16x32), fp32 accumulators.
//  * Activations: each K tile (128 inputs) of the 256 rows is loaded once per
//    workgroup straight from HBM into LDS (buffer loads with an LDS
//    destination, 16 bytes per lane; 64 KB per stage, two stages).  The
//    16-byte chunk q of row r sits at chunk position q ^ (r & 15) of its
//    256-byte LDS row, so the operand reads (32 rows x 2 chunks) hit distinct
//    banks.
//  * Weights: the repacked code tiles (16 columns x 128 inputs; 1 KB at 4
//    bits, 768 B at 3, 2 KB at 8) are read straight into registers.  The B operand of a 32 x 32 x 16 step is 8
//    codes (one 32-bit word) per lane: column l & 31, inputs 8 (l >> 5) + e
//    of the step.  Lane l therefore loads the 16 bytes that repacked lane
//    (l & 15) + 16 (2 h2 + (l >> 5)) of column tile 2 g + ((l & 31) >> 4)
//    holds, for h2 = 0 (even steps) and 1 (odd steps): word j of those is the
//    operand of step 2 j + h2.  Each weight is read and dequantized exactly
//    (the routine of the dequant export) once per workgroup; B never passes
//    through LDS.
//  * The loads of K tile t + 1 go out during tile t, each between two MFMAs
//    (its weights in step 0, its activations, into the other LDS stage, over
//    the first steps), and the step-0 B operands of tile t + 1 are dequantized
//    during step 7 of tile t, so a tile starts with its MFMAs; one barrier per
//    K tile.  Per-tile timestamps (MI355X, 256 rows, 5120 x 7168 at M = 2048):
//    0.49 us of a 2.96 us tile went to the preamble before the first MFMA;
//    0.16 us now (whole calls 2-6 % faster on the four Qwen2.5-32B-shaped
//    layers).
//  * Up to 32 rows (BM = 32) the call is bound by the dequant and by latency,
//    not by the multiply: the integer codes enter the MFMAs alone (o + q) and
//    the scale and zero are applied once per K tile after the sum, and the
//    weights of tile t + 2 stay in flight across the barrier that ends tile t
//    (see prefill.h).
#include "prefill.h"

namespace w4a16 {

// ---------------------------------------------------------------- planning --
// Rows per workgroup for M, and the split of K that fills the GPU best: a
// simple model of the call time (rounds of workgroups on 256 CUs x K tiles per
// workgroup x per-tile MFMA time, plus the partials' round trip through HBM).
// Whole row blocks and a partial last one are separate launches (the partial
// one puts its row in the per-lane offset), so they count as separate rounds.
//
// For M > 128, when 256-row tiles need no split of K, 192-row tiles are taken
// instead if they finish in fewer tile-times: a 192-row workgroup takes about
// 0.83 of a 256-row one per K tile (measured on MI355X), and the smaller tile
// can fill a round that 256-row tiles leave partly idle.
PrefillPlan plan_prefill(int64_t M, int64_t N, int64_t K, bool split_ok) {
  const int64_t cols = ceil_div(ceil_div(N, 64), (int64_t)PF_WAVES);
  const int64_t KT = K / 128;
  // Rounds of the grid over 256 CUs (one workgroup each): whole row blocks
  // and a ragged last one in launches of their own (each a round of its
  // own), or every row block in one launch of the ragged-tail form.
  auto rounds = [&](int64_t bm, int64_t S, bool single) {
    if (single) return (double)ceil_div(ceil_div(M, bm) * cols * S, (int64_t)256);
    const int64_t full = M / bm;
    return (double)(ceil_div(full * cols * S, (int64_t)256) +
                    (M % bm ? ceil_div(cols * S, (int64_t)256) : 0));
  };
  // Time of one K tile of a workgroup: 3.4 us with 256 rows (measured on
  // MI355X); 192 rows take 0.874 of that (their dequantized weights serve
  // fewer rows), smaller blocks their share of rows; the ragged-tail form
  // about 2 % more.  A split of K adds its partials' write and read.
  auto cost = [&](int bm, int64_t S, bool single) {
    const double t_tile = 3.4e-6 * (bm == 192 ? 0.874 : bm / 256.0) * (single ? 1.02 : 1.0);
    double t = rounds(bm, S, single) * (double)ceil_div(KT, S) * t_tile;
    if (S > 1) t += (double)(S * 4 + 2) * M * N / 4.0e12 + 2e-6;
    return t;
  };
  PrefillPlan pl;
  pl.bm = M <= 32 ? 32 : M <= 64 ? 64 : (M <= 128 ? 128 : 256);
  pl.splits = 1;
  pl.single = false;
  double best = cost(pl.bm, 1, false);
  // other forms must save 3 %: 256-row blocks (large M), splits of K, the
  // single ragged-tail launch, 192-row blocks
  const int bms[2] = {pl.bm, 192};
  for (int bi = 0; bi < (pl.bm == 256 ? 2 : 1); ++bi) {
    const int bm = bms[bi];
    for (int single = 0; single < (M % bm ? 2 : 1); ++single)
      for (int S = 1; S <= (split_ok ? 16 : 1) && S <= KT; ++S) {
        const double t = cost(bm, S, single != 0);
        if (t < best * 0.97) {
          best = t;
          pl.bm = bm;
          pl.splits = S;
          pl.single = single != 0;
        }
      }
  }
  return pl;
}

int64_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const PrefillPlan pl = plan_prefill(M, N, K);
  return pl.splits > 1 ? ceil_div((int64_t)pl.splits * M * N * 4, 256) * 256 : 0;
}

void launch_int_prefill(const void* x, const void* codes_r, const void* scales_r,
                        const void* zeros_r, void* out, void* ws, int64_t M, int64_t N,
                        int64_t K, int G, int bits, int dtype, hipStream_t stream) {
  if (bits == 4)
    launch_intb_prefill<4>(x, codes_r, scales_r, zeros_r, out, ws, M, N, K, G, dtype, stream);
  else if (bits == 3)
    launch_intb_prefill<3>(x, codes_r, scales_r, zeros_r, out, ws, M, N, K, G, dtype, stream);
  else
    launch_intb_prefill<8>(x, codes_r, scales_r, zeros_r, out, ws, M, N, K, G, dtype, stream);
}

void launch_nf4_prefill(const void* x, const uint8_t* qweight, const uint8_t* absmax_q,
                        const float* absmax_scale, const Nf4Table& L, void* out, void* ws,
                        int64_t M, int64_t N, int64_t K, int dtype, bool repacked,
                        hipStream_t stream) {
  if (repacked) {
    if (dtype == DT_F16)
      launch_prefill_dt<DT_F16, FMT_NF4R, 1, 4>(x, qweight, absmax_q, absmax_scale, L, out, ws,
                                                M, N, K, stream);
    else
      launch_prefill_dt<DT_BF16, FMT_NF4R, 1, 4>(x, qweight, absmax_q, absmax_scale, L, out, ws,
                                                 M, N, K, stream);
  } else if (dtype == DT_F16) {
    launch_prefill_dt<DT_F16, FMT_NF4, 1, 4>(x, qweight, absmax_q, absmax_scale, L, out, ws, M,
                                             N, K, stream);
  } else {
    launch_prefill_dt<DT_BF16, FMT_NF4, 1, 4>(x, qweight, absmax_q, absmax_scale, L, out, ws, M,
                                              N, K, stream);
  }
}

template void launch_intb_prefill<4>(W4A16_PREFILL_ARGS);

}  // namespace w4a16

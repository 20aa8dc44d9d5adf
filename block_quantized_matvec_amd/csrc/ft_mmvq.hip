// ft_mmvq.hip -- quantized matvec entry: launch plan, the dot4 instantiations for
// Q4_0 / Q8_0 / Q4_K (kernels in ft_mmvq_kernels.h), routing between the dot4 and
// the int8 MFMA kernels (ft_mmvq_mfma.hip).
#include "ft_mmvq_kernels.h"

// Launch plan: lanes per row (LR) and units per lane (P) cover a row with the
// fewest idle lanes, at most 16 unit-token activation sets per lane; a tile is
// as many whole rows as fit in CPL * 4 KiB and must give every row group a row;
// the grid is a few workgroups per CU, each owning an equal share of rows.
// Per-wave ring: units per lane cover the row in 64-unit segments.  Measured on
// the 14336 x 4096 and 4096 x 14336 Q4_K / Q8_0 matrices at 1, 2 and 4 tokens
// (grid of 1..4 workgroups per CU x 2..4 stages, contiguous or interleaved rows):
// rows of one or two segments run best with the rows interleaved over all waves
// (the waves' requests then stay inside one band of the matrix) once every wave
// gets at least 4 rows, with 3 workgroups per CU and 2 stages for 1 token (Q4_K
// 7.25 us), 2 and 3 for 2 tokens (8.84 -> 8.59 us) and 2 and 2 for 4 token slots
// (11.43 -> 10.80 us: more activation registers per lane), else with 2
// workgroups per CU and contiguous shares.  Rows of 8 segments (Q8_0, K = 14336)
// take 1 workgroup per CU, 4 stages, interleaved (12.01 -> 11.64 us); 4 segments
// (Q4_K, K = 14336) 1 workgroup per CU, 4 stages, contiguous, except 1 token: 2
// workgroups per CU, 2 stages (9.17 -> 8.84 us).  More waves or deeper rings
// beyond these only add requests in flight.
static int mmvq_plan_wave(int units_per_row, int tslot, int row_bytes, int64_t n, MmvqPlan* out) {
  int P = 1;
  while (P * 64 < units_per_row) P *= 2;
  if (P > 8 || P * 64 < units_per_row || P * tslot > 16) return 0;
  int wpc, stages, il;
  if (P >= 8) {
    wpc = 1; stages = 4; il = 1;
  } else if (P >= 4) {
    const bool one = tslot == 1;
    wpc = one ? 2 : 1; stages = one ? 2 : 4; il = 0;
  } else {
    wpc = tslot == 1 ? 3 : 2; stages = tslot == 2 ? 3 : 2; il = 1;
  }
  // interleave only when every wave gets at least 4 rows; short-row matrices
  // that small take 2 workgroups per CU, 2 stages, contiguous shares
  if (n < (int64_t)ftk::num_cus() * wpc * 4 * 4) {
    il = 0;
    if (P <= 2) { wpc = 2; stages = 2; }
  }
  const int64_t waves = (int64_t)ftk::num_cus() * wpc * 4;
  int64_t rpw = (n + waves - 1) / waves;
  if (rpw < 1) rpw = 1;
  MmvqPlan pl{};
  pl.wave = 1;
  pl.stages = stages;
  pl.tslot = tslot;
  pl.p = P;
  pl.rows_per_wg = (int)rpw;   // rows per wave
  int64_t nwaves = (n + rpw - 1) / rpw;
  pl.row_stride = 1;
  if (il) {   // interleaved rows over all waves
    nwaves = waves < n ? waves : n;
    pl.row_stride = nwaves;
  }
  pl.grid = (int)((nwaves + 3) / 4);
  *out = pl;
  return 1;
}

int ftk_mmvq_plan(int units_per_row, int tslot, int row_bytes, int64_t n, MmvqPlan* out) {
  MmvqPlan best{};
  double best_cost = 1e30;
  // per-wave rings first; workgroup LDS tiles for what they cannot hold
  if (mmvq_plan_wave(units_per_row, tslot, row_bytes, n, out)) return 1;
  for (int cpl = 4; cpl <= 8; cpl += 4) {
    const int rt = (cpl * 4096 - 15) / row_bytes;
    if (rt < 1) continue;
    for (int L = 64; L <= 256; L *= 2) {
      const int G = ftk::MMVQ_THREADS / L;
      if (G > rt) continue;
      for (int P = 1; P <= 8; P *= 2) {
        if (P * L < units_per_row || P * tslot > 16) continue;
        const double waste = (double)(P * L - units_per_row) / (P * L);
        const int rows_per_group = rt / G;
        const double idle_groups = (double)(rt % G) / rt;
        double cost = waste + 0.5 * idle_groups + 0.04 * (L / 64 - 1) + (P * tslot > 8 ? 0.3 : 0.0);
        cost += rows_per_group < 2 ? 0.05 : 0.0;
        cost += cpl == 8 ? 0.02 : 0.0;
        if (cost < best_cost) {
          best_cost = cost;
          best.lr = L;
          best.p = P;
          best.cpl = cpl;
          best.rows_per_tile = rt;
        }
      }
    }
  }
  if (!best.lr) return 0;
  best.tslot = tslot;
  best.stages = best.cpl == 8 ? 2 : 4;
  const int wgs_per_cu = 2;
  const int64_t slots = (int64_t)ftk::num_cus() * wgs_per_cu;
  const int64_t tiles = (n + best.rows_per_tile - 1) / best.rows_per_tile;
  const int64_t grid = tiles < slots ? tiles : slots;
  best.rows_per_wg = (int)((n + grid - 1) / grid);
  best.grid = (int)((n + best.rows_per_wg - 1) / best.rows_per_wg);
  *out = best;
  return 1;
}


// compute units of the current device (cached; every device of one node is the same part)
int ftk_num_cus() {
  static int cached = 0;
  if (cached > 0) return cached;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
    cached = cus;
  else
    cached = 256;
  return cached;
}

// Several tokens go to the int8 MFMA kernels (ft_mmvq_mfma.hip) when K is a whole
// number of chunks: from 5 tokens on for rows of at most 128 units, and on longer
// rows from 2 tokens on (Q4_0 / Q4_K / Q6_K / MXFP4) or 3 (Q8_0 / Q5_K).  The rest
// stay on the per-wave dot4 ring.  With every weight copy out of the last-level
// cache, 4 tokens on 14336 x 4096 take (dot4 vs MFMA, us) Q4_K 10.9 / 12.6, Q4_0
// 12.0 / 12.6, MXFP4 13.9 / 15.2, Q6_K 19.2 / 19.6.  Earlier measurements
// (dot4 vs MFMA, us): 2 tokens, 14336 x 4096: Q8_0 12.0 / 14.9, Q4_K 8.7 / 10.4,
// Q4_0 9.4 / 10.4; 4096 x 14336: Q8_0 13.2 / 13.7, Q4_K 11.3 / 9.7, Q4_0 12.7 /
// 10.1.  4 tokens, 14336 x 4096: Q8_0 13.1 / 15.2, Q4_K 10.8 / 10.4, Q4_0 12.1 /
// 11.5, Q5_K 12.2 / 13.8, MXFP4 13.8 / 14.0; 4096 x 14336: Q4_K 16.2 / 9.8.  8 tokens
// are faster on MFMA throughout (Q5_K 25.6 / 16.6, Q6_K 59.5 / 20.7, MXFP4 24.5 /
// 16.5); Q6_K 4096 x 14336 at 2 tokens 21.7 / 18.0.  Q2_K / Q3_K from 5 tokens on
// (14336 x 4096, 4 tokens 12.7 / 14.7 and 15.3 / 22.4, 8 tokens 27.9 / 21.5 and
// 30.4 / 23.5: their few bytes per chunk leave the MFMA kernel bound by its
// per-block unpack and combine), and so do Q4_1 / Q5_0 / Q5_1 (4 tokens 12.4 / 13.4,
// 13.1 / 14.8, 13.5 / 21.1; 8 tokens 24.6 / 15.4, 26.7 / 16.3, 27.0 / 22.9 before
// Q5_1's slot pad).

static int64_t units_of(int w, int64_t k) {
  switch (w) {
    case FT_Q4_0: return ftk::units_in_row<FT_Q4_0>(k);
    case FT_Q8_0: return ftk::units_in_row<FT_Q8_0>(k);
    case FT_Q4_K: return ftk::units_in_row<FT_Q4_K>(k);
    case FT_Q5_K: return ftk::units_in_row<FT_Q5_K>(k);
    case FT_Q6_K: return ftk::units_in_row<FT_Q6_K>(k);
    case FT_MXFP4: return ftk::units_in_row<FT_MXFP4>(k);
    case FT_Q2_K: return ftk::units_in_row<FT_Q2_K>(k);
    case FT_Q3_K: return ftk::units_in_row<FT_Q3_K>(k);
    case FT_Q4_1: return ftk::units_in_row<FT_Q4_1>(k);
    case FT_Q5_0: return ftk::units_in_row<FT_Q5_0>(k);
    case FT_Q5_1: return ftk::units_in_row<FT_Q5_1>(k);
    default: return 0;
  }
}

hipError_t ftk_launch_mmvq(const MmvqArgs& a, int64_t k, hipStream_t st) {
  using namespace ftk;
  if (a.act == FT_Q8_K) return ftk_launch_mmvq_q8k(a, k, st);
  const bool lng = units_of(a.w, k) > 128;
  const bool late = a.w == FT_Q2_K || a.w == FT_Q3_K || a.w == FT_Q4_1 || a.w == FT_Q5_0 || a.w == FT_Q5_1;
  const bool mfma = late || !lng ? a.t >= 5 : (a.w == FT_Q8_0 || a.w == FT_Q5_K ? a.t >= 3 : a.t >= 2);
  if (mfma && ftk_mmvq_mfma_ok(a.w, a.act, k, a.t)) return ftk_launch_mmvq_mfma(a, k, st);
  if (a.act == FT_Q8_1) {
    switch (a.w) {
      case FT_Q4_0: return launch_fa<FT_Q4_0, FT_Q8_1>(a, k, st);
      case FT_Q8_0: return launch_fa<FT_Q8_0, FT_Q8_1>(a, k, st);
      case FT_Q4_K: return launch_fa<FT_Q4_K, FT_Q8_1>(a, k, st);
      default: break;
    }
  }
  return ftk_launch_mmvq_kq(a, k, st);   // the other formats (ft_mmvq_kq.hip)
}

// ft_mmvq_kernels.h -- the dot4 quantized matvec kernels y[t][n] = W[n][:] . xhat[t][:]
// and their launch templates, instantiated per weight format by ft_mmvq.hip (Q4_0,
// Q8_0, Q4_K) and ft_mmvq_kq.hip (Q5_K, Q6_K, MXFP4), so that the two compile in
// parallel.
//
// The operation is the int8-dot matvec of FreeToken PR #136 (Summary: production
// matvec with quantized activations) and the non-grouped keep-quant op of
// vllm.cpp PR #523 (What changed).  Design for MI355X:
//  * Each lane owns fixed 32-weight units of a row (64 for Q4_K / Q5_K) and keeps
//    the matching activation codes and scales in VGPRs for the whole kernel, so
//    LDS carries only weight bytes.  Nibble / 6-bit / high-bit unpack happens in
//    registers; dots use v_dot4_i32_i8.  Any block size or alignment works because
//    lanes read their units back from LDS at byte granularity.
//  * mmvq_wave_kernel (the default): every wave streams its own rows through its
//    own LDS ring of global_load_lds_dwordx4 stages and waits only on its own
//    vmcnt; mmvq_kernel (rows over 512 units, or more token slots than the
//    per-wave ring holds in registers): each workgroup walks its contiguous share
//    of rows in tiles of whole rows through a workgroup-wide LDS ring.
//  * Rows are reduced over their lanes with a multi-value butterfly (M values cost
//    M-1 + log2(L/M) shuffles instead of M*log2(L)).
#pragma once

#include <stdlib.h>

#include "ft_device.h"
#include "ft_internal.h"

namespace ftk {

constexpr int MMVQ_THREADS = 256;

// LDS ring per workgroup: S stages of one tile (CPL 16-byte chunks per thread),
// at most MMVQ_RING_CHUNKS chunks per thread (64 KiB).
constexpr int MMVQ_RING_CHUNKS = 16;
constexpr size_t mmvq_lds_bytes(int cpl, int s) {
  return (size_t)cpl * s * 256 * 16 + 16 + 2 * (256 / 64) * 64 * sizeof(float);
}

// LR: lanes per row (64, 128 or 256); P: units per lane; T: token slots;
// CPL: 16-byte chunks per lane per tile (tile <= CPL * 4 KiB); S: ring stages.
template <int F, int A, int T, int LR, int P, int CPL, int S>
__global__ void __launch_bounds__(MMVQ_THREADS)
mmvq_kernel(const uint8_t* __restrict__ W, int64_t n, int row_bytes, int units_per_row, int rows_per_wg,
            int rows_per_tile, const uint8_t* __restrict__ xq, int xrow_bytes, int t_real,
            float* __restrict__ y, int64_t ldy) {
  using FT = Fmt<F>;
  constexpr int G = MMVQ_THREADS / LR;        // row groups in the workgroup
  constexpr int RA = T >= 2 ? 1 : 2;          // rows per group per reduction step
  constexpr int M = RA * T;                   // values reduced per step
  constexpr int WPR = LR / 64;                // waves per row
  constexpr int TB = CPL * MMVQ_THREADS * 16; // bytes per stage
  static_assert(S >= 2 && S * CPL <= MMVQ_RING_CHUNKS, "");
  extern __shared__ u32x4 smem4[];
  uint8_t* ring = (uint8_t*)smem4;
  float* red = (float*)(ring + S * TB + 16);   // 16 bytes of slack for reads past a row

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = tid / LR, gl = tid % LR;

  const int64_t wr0 = (int64_t)blockIdx.x * rows_per_wg;
  if (wr0 >= n) return;
  const int wrows = (int)min<int64_t>(rows_per_wg, n - wr0);
  const int ntiles = (wrows + rows_per_tile - 1) / rows_per_tile;

  // tile -> ring stage tile % S, chunk c at byte 16c of the stage.  Every wave
  // issues exactly CPL loads per tile (chunks past the tile re-read its last
  // chunk into unused bytes), so the vmcnt arithmetic of wait_tiles holds.  The
  // prologue fills all S stages; a stage past the last tile (never read) takes
  // one 16-byte chunk.
  auto issue = [&](int tile) {
    const bool real = tile < ntiles;
    const int64_t r0 = wr0 + (int64_t)(real ? tile : ntiles - 1) * rows_per_tile;
    const int nr = min(rows_per_tile, (int)(wr0 + wrows - r0));
    const int64_t start = r0 * row_bytes, a0 = start & ~(int64_t)15;
    const int nch = real ? (int)((start + (int64_t)nr * row_bytes - a0 + 15) >> 4) : 1;
    const uint8_t* src = W + a0;
    uint8_t* dst = ring + (tile % S) * TB + 1024 * wave;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = min(i * MMVQ_THREADS + tid, nch - 1);
      lds_dma16(src + 16 * (int64_t)c, dst + 4096 * i);
    }
  };
  issue(0);
  asm volatile("" ::: "memory");   // keep the activation loads between the two

  // activations of this lane's units (VGPR-resident for the whole kernel): loaded
  // unconditionally (idle lanes and token slots read a real unit and are zeroed
  // afterwards) between the first tile and the rest of the ring, so that waiting
  // for them does not wait for the ring
  ActUnit<F> act[P][T];
  uint32_t ub[P];
  int uu[P];
  bool uv[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int u0 = gl + p * LR;
    uv[p] = u0 < units_per_row;
    const int u = uv[p] ? u0 : 0;
    ub[p] = (uint32_t)(u / FT::UPB) * FT::BB;
    uu[p] = u % FT::UPB;
#pragma unroll
    for (int t = 0; t < T; ++t)
      load_act_raw<F, A>(xq + (size_t)(t < t_real ? t : 0) * xrow_bytes, u / FT::UPB, uu[p], act[p][t]);
  }
  asm volatile("" ::: "memory");
  int issued = S - 1;   // last tile in flight
#pragma unroll
  for (int i = 1; i < S; ++i) issue(i);
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<(S - 1) * CPL>();   // the activations (and the first tile) have arrived
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int t = 0; t < T; ++t) finish_act_unit<F, A>(act[p][t], uv[p] && t < t_real);

  const Reader<const uint32_t*> rd{(const uint32_t*)ring};
  int parity = 0;
  int tile = 0;
  do {   // ntiles >= 1
    wait_tiles<CPL, S>(issued - tile);
    lds_barrier();   // the whole tile has landed; every wave is done with the previous one
    if (tile >= 1 && tile + S - 1 < ntiles) {
      issue(tile + S - 1);   // into the previous tile's stage
      issued = tile + S - 1;
    }
    const int64_t r0 = wr0 + (int64_t)tile * rows_per_tile;
    const int nr = min(rows_per_tile, (int)(wr0 + wrows - r0));
    const uint32_t shift = (uint32_t)((tile % S) * TB) + (uint32_t)((r0 * row_bytes) & 15);

    for (int rb = 0; rb < nr; rb += G * RA) {
      float v[M];
#pragma unroll
      for (int i = 0; i < M; ++i) v[i] = 0.0f;
#pragma unroll
      for (int ra = 0; ra < RA; ++ra) {
        const int r = rb + ra * G + grp;
        if (r < nr) {
          const uint32_t rowoff = shift + (uint32_t)r * row_bytes;
#pragma unroll
          for (int p = 0; p < P; ++p) {
            Unit<F> un;
            unpack_unit<F, (F == FT_Q4_K || F == FT_Q5_K)>(rd, rowoff + ub[p], uu[p], un);
#pragma unroll
            for (int t = 0; t < T; ++t) v[ra * T + t] = unit_combine<F>(un, act[p][t], v[ra * T + t]);
          }
        }
      }
      group_reduce_multi<M, (LR < 64 ? LR : 64)>(v, LR < 64 ? gl : lane);
      constexpr int L = LR < 64 ? LR : 64;
      const int idx = (LR < 64 ? gl : lane) / (L / M);
      const bool leader = ((LR < 64 ? gl : lane) % (L / M)) == 0;
      if (WPR <= 1) {
        if (leader) {
          const int ra = idx / T, t = idx % T;
          const int r = rb + ra * G + grp;
          if (r < nr && t < t_real) y[(int64_t)t * ldy + r0 + r] = v[0];
        }
      } else {
        float* rp = red + parity * (MMVQ_THREADS / 64) * M;
        if (leader) rp[wave * M + idx] = v[0];
        lds_barrier();
        if (gl < M) {
          const int ra = gl / T, t = gl % T;
          const int r = rb + ra * G + grp;
          float s = 0.0f;
#pragma unroll
          for (int w = 0; w < WPR; ++w) s += rp[(grp * WPR + w) * M + gl];
          if (r < nr && t < t_real) y[(int64_t)t * ldy + r0 + r] = s;
        }
        parity ^= 1;
      }
    }
  } while (++tile < ntiles);
}

// ---------------------------------------------------------------------------
// Per-wave ring: every wave owns a contiguous share of the rows and streams it
// through its own LDS ring of S stages, one 64-unit segment of a row per stage
// (lane l takes unit l of the segment), waiting only on its own vmcnt: no
// workgroup barriers, so a wave computes a segment as soon as its bytes have
// landed and the work left after the last byte arrives is one segment.
// ---------------------------------------------------------------------------
template <int F, int S>
constexpr size_t mmvq_wave_lds_bytes() {
  return (size_t)(MMVQ_THREADS / 64) * (S * SegGeo<F>::CPW * 1024 + 16);
}

template <int F, int A, int T, int P, int S>
__global__ void __launch_bounds__(MMVQ_THREADS)
mmvq_wave_kernel(const uint8_t* __restrict__ W, int64_t n, int row_bytes, int units_per_row, int rows_per_wave,
                 int64_t row_stride, const uint8_t* __restrict__ xq, int xrow_bytes, int t_real,
                 float* __restrict__ y, int64_t ldy) {
  using FT = Fmt<F>;
  constexpr int SEG = SegGeo<F>::BYTES;
  constexpr int CPW = SegGeo<F>::CPW;
  constexpr int SB = CPW * 1024;              // bytes per stage
  constexpr int RA = T >= 2 ? 1 : 2;          // rows per reduction step
  constexpr int M = RA * T;                   // values reduced per step
  extern __shared__ u32x4 smem4[];
  const int lane = threadIdx.x & 63, wave = wave_id();
  uint8_t* ring = (uint8_t*)smem4 + wave * (S * SB + 16);   // 16 bytes of slack past each ring

  // the wave's rows: r0 + i * row_stride, i < nrows (a contiguous share when
  // row_stride is 1, every row_stride-th row from the wave's index otherwise)
  const int64_t gw = (int64_t)blockIdx.x * (MMVQ_THREADS / 64) + wave;
  const int64_t r0 = row_stride == 1 ? gw * rows_per_wave : gw;
  if (r0 >= n) return;   // whole wave; there are no workgroup barriers
  const int nrows = row_stride == 1 ? (int)min<int64_t>(rows_per_wave, n - r0)
                                    : (int)((n - r0 + row_stride - 1) / row_stride);
  const int nseg = (units_per_row + 63) >> 6;   // segments per row, <= P
  const int ntiles = nrows * nseg;

  // tile j = segment (j % nseg) of row (j / nseg), in ring stage j % S.  Every
  // tile is CPW loads per lane (chunks past the segment re-read its last chunk
  // into unused bytes; tiles past the share re-read the first chunk of the share),
  // so the vmcnt arithmetic of wait_tiles holds.  The bookkeeping is wave-uniform
  // (scalar): running byte offsets, no multiplies per tile.
  const int64_t row_step = row_stride * (int64_t)row_bytes;
  const int64_t first_a0 = (r0 * (int64_t)row_bytes) & ~(int64_t)15;
  const int last_len = row_bytes - (nseg - 1) * SEG;   // bytes of a row's last segment
  int64_t is_base = r0 * (int64_t)row_bytes;            // row of the next tile to issue
  int issued = 0, is_seg = 0, is_stage = 0;
  int c_nch = -1;          // chunk count the lane offsets below were made for
  uint32_t c_off[CPW];     // byte offset of this lane's chunk i: 16 * min(lane + 64 i, nch - 1)
  auto issue_next = [&]() {
    const bool real = issued < ntiles;
    const int64_t start = is_base + is_seg * SEG;
    const int64_t a0 = real ? start & ~(int64_t)15 : first_a0;
    const int nch = real ? ((int)(start & 15) + (is_seg == nseg - 1 ? last_len : SEG) + 15) >> 4 : 1;
    if (nch != c_nch) {    // uniform; rows of 16-byte multiples keep one count
      c_nch = nch;
#pragma unroll
      for (int i = 0; i < CPW; ++i) c_off[i] = 16u * (uint32_t)min(lane + 64 * i, nch - 1);
    }
    uint8_t* dst = ring + is_stage * SB;
    const uint8_t* src = W + a0;   // uniform base, 32-bit lane offsets
#pragma unroll
    for (int i = 0; i < CPW; ++i) lds_dma16(src + c_off[i], dst + 1024 * i);
    ++issued;
    is_stage = is_stage + 1 == S ? 0 : is_stage + 1;
    if (++is_seg == nseg) { is_seg = 0; is_base += row_step; }
  };
  issue_next();
  asm volatile("" ::: "memory");   // keep the activation loads between the first tile and the rest

  // activations of this lane's units (VGPR-resident for the whole kernel);
  // idle lanes read the segment's first unit against zero activations
  ActUnit<F> act[P][T];
  const uint32_t ub = (uint32_t)(lane / FT::UPB) * FT::BB;   // unit offset in a full segment
  const int uu = lane % FT::UPB;
  bool uv[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int u0 = 64 * p + lane;
    uv[p] = u0 < units_per_row;
    const int u = uv[p] ? u0 : 0;
#pragma unroll
    for (int t = 0; t < T; ++t)
      load_act_raw<F, A>(xq + (size_t)(t < t_real ? t : 0) * xrow_bytes, u / FT::UPB, u % FT::UPB, act[p][t]);
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 1; i < S; ++i) issue_next();
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<(S - 1) * CPW>();   // the activations (and the first tile) have arrived
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int t = 0; t < T; ++t) finish_act_unit<F, A>(act[p][t], uv[p] && t < t_real);

  const Reader<const uint32_t*> rd{(const uint32_t*)ring};
  int cur = 0, cs_stage = 0;                             // tiles consumed, stage of the next one
  uint32_t cs_off = (uint32_t)(r0 * (int64_t)row_bytes);   // low bits of the consumed row's offset
  for (int rp = 0; rp < nrows; rp += RA) {
    float v[M];
#pragma unroll
    for (int i = 0; i < M; ++i) v[i] = 0.0f;
#pragma unroll
    for (int ra = 0; ra < RA; ++ra) {
      if (rp + ra < nrows) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          if (p < nseg) {
            wait_tiles<CPW, S>(issued - 1 - cur);
            const uint32_t so = (uint32_t)(cs_stage * SB) + ((cs_off + (uint32_t)(p * SEG)) & 15u);
            Unit<F> un;
            unpack_unit<F, (F == FT_Q4_K || F == FT_Q5_K)>(rd, so + (uv[p] ? ub : 0u), uv[p] ? uu : 0, un);
#pragma unroll
            for (int t = 0; t < T; ++t) v[ra * T + t] = unit_combine<F>(un, act[p][t], v[ra * T + t]);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0): the stage is read
            issue_next();   // refill the stage just read
            ++cur;
            cs_stage = cs_stage + 1 == S ? 0 : cs_stage + 1;
          }
        }
        cs_off += (uint32_t)row_step;
      }
    }
    group_reduce_multi<M, 64>(v, lane);
    const int idx = lane / (64 / M);
    if ((lane % (64 / M)) == 0) {
      const int ra = idx / T, t = idx % T;
      if (rp + ra < nrows && t < t_real) y[(int64_t)t * ldy + r0 + (rp + ra) * row_stride] = v[0];
    }
  }
}

// host side -------------------------------------------------------------------

static int num_cus() { return ftk_num_cus(); }

template <int F, int A, int T, int LR, int P, int CPL, int S>
static hipError_t launch_mmvq_t(const MmvqArgs& a, const MmvqPlan& pl, hipStream_t st) {
  constexpr size_t lds = mmvq_lds_bytes(CPL, S);
  static const bool attr = hipFuncSetAttribute((const void*)mmvq_kernel<F, A, T, LR, P, CPL, S>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess;
  if (!attr) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((mmvq_kernel<F, A, T, LR, P, CPL, S>), dim3((unsigned)pl.grid), dim3(MMVQ_THREADS), lds, st,
                     (const uint8_t*)a.W, a.n, a.row_bytes, a.units_per_row, pl.rows_per_wg, pl.rows_per_tile,
                     (const uint8_t*)a.xq, a.xrow_bytes, a.t, a.y, a.ldy);
  return hipGetLastError();
}

template <int F, int A, int T, int P, int S>
static hipError_t launch_wave_t(const MmvqArgs& a, const MmvqPlan& pl, hipStream_t st) {
  constexpr size_t lds = mmvq_wave_lds_bytes<F, S>();
  static const bool attr = hipFuncSetAttribute((const void*)mmvq_wave_kernel<F, A, T, P, S>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess;
  if (!attr) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((mmvq_wave_kernel<F, A, T, P, S>), dim3((unsigned)pl.grid), dim3(MMVQ_THREADS), lds, st,
                     (const uint8_t*)a.W, a.n, a.row_bytes, a.units_per_row, pl.rows_per_wg, pl.row_stride,
                     (const uint8_t*)a.xq, a.xrow_bytes, a.t, a.y, a.ldy);
  return hipGetLastError();
}

template <int F, int A, int T>
static hipError_t dispatch_wave(const MmvqArgs& a, const MmvqPlan& pl, hipStream_t st) {
#define FT_WV(PV) \
  if constexpr (PV * T <= 16) {                                              \
    if (pl.p == PV && pl.stages == 2) return launch_wave_t<F, A, T, PV, 2>(a, pl, st); \
    if (pl.p == PV && pl.stages == 3) return launch_wave_t<F, A, T, PV, 3>(a, pl, st); \
    if (pl.p == PV && pl.stages == 4) return launch_wave_t<F, A, T, PV, 4>(a, pl, st); \
  }
  FT_WV(1) FT_WV(2) FT_WV(4) FT_WV(8)
#undef FT_WV
  return hipErrorInvalidValue;
}

template <int F, int A, int T, int CPL, int S>
static hipError_t dispatch_lp(const MmvqArgs& a, const MmvqPlan& pl, hipStream_t st) {
#define FT_LP(LRV, PV)                                                             \
  if constexpr (PV * T <= 16)                                                     \
    if (pl.lr == LRV && pl.p == PV) return launch_mmvq_t<F, A, T, LRV, PV, CPL, S>(a, pl, st);
  FT_LP(64, 1) FT_LP(64, 2) FT_LP(64, 4) FT_LP(64, 8)
  FT_LP(128, 1) FT_LP(128, 2) FT_LP(128, 4) FT_LP(128, 8)
  FT_LP(256, 1) FT_LP(256, 2) FT_LP(256, 4) FT_LP(256, 8)
#undef FT_LP
  return hipErrorInvalidValue;
}

template <int F, int A, int T>
static hipError_t dispatch_c(const MmvqArgs& a, const MmvqPlan& pl, hipStream_t st) {
  if (pl.wave) return dispatch_wave<F, A, T>(a, pl, st);
  if (pl.cpl == 4 && pl.stages == 2) return dispatch_lp<F, A, T, 4, 2>(a, pl, st);
  if (pl.cpl == 4 && pl.stages == 4) return dispatch_lp<F, A, T, 4, 4>(a, pl, st);
  if (pl.cpl == 8 && pl.stages == 2) return dispatch_lp<F, A, T, 8, 2>(a, pl, st);
  return hipErrorInvalidValue;
}

template <int F, int A>
static hipError_t dispatch_t(const MmvqArgs& a, const MmvqPlan& pl, hipStream_t st) {
  switch (pl.tslot) {
    case 1: return dispatch_c<F, A, 1>(a, pl, st);
    case 2: return dispatch_c<F, A, 2>(a, pl, st);
    case 4: return dispatch_c<F, A, 4>(a, pl, st);
    case 8: return dispatch_c<F, A, 8>(a, pl, st);
  }
  return hipErrorInvalidValue;
}


template <int F, int A>
static hipError_t launch_fa(MmvqArgs a, int64_t k, hipStream_t st) {
  const int tslot = a.t <= 1 ? 1 : a.t <= 2 ? 2 : a.t <= 4 ? 4 : 8;
  a.units_per_row = (int)units_in_row<F>(k);
  MmvqPlan pl;
  if (!ftk_mmvq_plan(a.units_per_row, tslot, a.row_bytes, a.n, &pl))
    return hipErrorInvalidValue;
  return dispatch_t<F, A>(a, pl, st);
}

}  // namespace ftk

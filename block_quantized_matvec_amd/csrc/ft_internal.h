// ft_internal.h -- host-side launcher interface between the C ABI (ft_api.cpp)
// and the kernel translation units.  Launchers assume validated arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ft.h"

int ftk_num_cus();   // compute units of the current device

struct MmvqArgs {
  int w, act;
  const void* W;
  int64_t n;
  int row_bytes, units_per_row;  // units_per_row is set by the launcher
  const void* xq;
  int xrow_bytes;
  int t;  // 1..8
  float* y;
  int64_t ldy;
};

struct MmvqPlan {
  int wave;           // 1: per-wave LDS ring, rows_per_wg = rows per wave
  int64_t row_stride; // per-wave ring: 1 = contiguous shares, else rows interleaved over the waves
  int tslot;          // token slots of the kernel (1, 2, 4, 8)
  int lr, p;          // lanes per row, units per lane
  int cpl;            // 16-byte chunks per lane per tile (LDS variant)
  int stages;         // tiles in the LDS ring (LDS variant; cpl * stages <= 16)
  int rows_per_tile, rows_per_wg, grid;
};
int ftk_mmvq_plan(int units_per_row, int tslot, int row_bytes, int64_t n, MmvqPlan* out);
// dot4 matvec of Q5_K / Q6_K / MXFP4 x Q8_1 (ft_mmvq_kq.hip)
hipError_t ftk_launch_mmvq_kq(const MmvqArgs& a, int64_t k, hipStream_t st);
hipError_t ftk_launch_mmvq_dot4_mxfp4(const MmvqArgs& a, int64_t k, hipStream_t st);
hipError_t ftk_launch_mmvq_dot4_q2_k(const MmvqArgs& a, int64_t k, hipStream_t st);
hipError_t ftk_launch_mmvq_dot4_q3_k(const MmvqArgs& a, int64_t k, hipStream_t st);
hipError_t ftk_launch_mmvq_dot4_q4_1(const MmvqArgs& a, int64_t k, hipStream_t st);
hipError_t ftk_launch_mmvq_dot4_q5_0(const MmvqArgs& a, int64_t k, hipStream_t st);
hipError_t ftk_launch_mmvq_dot4_q5_1(const MmvqArgs& a, int64_t k, hipStream_t st);
hipError_t ftk_launch_mmvq(const MmvqArgs& a, int64_t k, hipStream_t st);
// int8-MFMA matvec for 2..8 tokens (K % 256 == 0; Q4_0, Q8_0, Q4_K x Q8_1)
bool ftk_mmvq_mfma_ok(int w, int act, int64_t k, int t);
hipError_t ftk_launch_mmvq_mfma(const MmvqArgs& a, int64_t k, hipStream_t st);

// measurement microkernels (ft_probe.hip): 0 streaming read, 1 int8 MFMA, 2 dot4
hipError_t ftk_launch_probe(int which, const void* buf, int64_t bytes, int64_t iters, uint32_t* out, hipStream_t st);
hipError_t ftk_launch_quantize(int act, const float* x, int64_t rows, int64_t k, int64_t ldx, void* xq,
                               hipStream_t st);
// Q8_0 activation blocks -> the Q8_1 layout (same d and codes), nblocks blocks
hipError_t ftk_launch_repack_q8_0(const void* src, int64_t nblocks, void* dst, hipStream_t st);
// dot4 matvec of Q4_K / Q5_K / Q6_K / MXFP4 x Q8_K (ft_mmvq_q8k.hip)
hipError_t ftk_launch_mmvq_q8k(const MmvqArgs& a, int64_t k, hipStream_t st);
// Q8_K rows [rows][k/256] -> FP8 halves for the FP4 MFMA, 512 bytes per superblock
hipError_t ftk_launch_fp8_split(const void* xq, int64_t rows, int64_t k, void* out, hipStream_t st);
hipError_t ftk_launch_dequant(int w, const void* blocks, int64_t rows, int64_t k, float* out,
                              hipStream_t st);
hipError_t ftk_launch_block_dots(int w, const void* W, int64_t n, int64_t k, int act, const void* xq,
                                 int64_t t, int32_t* partials, hipStream_t st);

hipError_t ftk_launch_route(const float* logits, int64_t t, int64_t n_expert, int topk, int32_t* ids,
                            float* w, hipStream_t st);
hipError_t ftk_launch_sort(const int32_t* ids, int64_t t, int topk, int64_t n_expert, int32_t* counts,
                           int32_t* offsets, int32_t* pairs, hipStream_t st);

// routed-MoE vector path (direct route): per-stage launchers
struct MoeArgs {
  int w, act;
  const void *w_gate, *w_up, *w_down;
  int64_t n_expert, hidden, inter;
  int64_t t;
  int topk;
  const int32_t* ids;
  const float* ew;
  const float* logits;   // nullable: the fused layer routes from these itself (ids / ew unused)
  int32_t* ids_out;      // nullable: that routing
  float* w_out;
  const float* x;      // [t][hidden] fp32 (the direct route quantizes it in its gate/up prologue)
  const void* xq;      // quantized x [t][hidden/blk_a] (sorted-tile route)
  float* h;            // [t*topk][inter]
  float* g_tap;        // nullable
  float* u_tap;        // nullable
  void* hq;            // quantized h [t*topk][inter/blk_a] (sorted-tile route)
  void* hq_tap;        // nullable: the direct route writes quantized h here
  const void* in_hq;   // nullable: the direct route's down stage reads these blocks instead
  float* dpair;        // [t*topk][hidden] per-pair down projections
  float* d_tap;        // nullable: the caller's tap for dpair (the fused layer writes no dpair otherwise)
  float* h_tap;        // nullable: the caller's tap for h (the fused layer writes no h otherwise)
  float* y;            // [t][hidden]
};
// the whole Q4_K x Q8_1 layer in two launches per 4-token chunk (ft_moe_fused.hip):
// shapes it takes, and the launch; table: ftk_moe_fused_table_bytes() of scratch
// the first launch hands the routing to the second in
size_t ftk_moe_fused_table_bytes();
bool ftk_moe_fused_ok(int w, int act, int64_t hidden, int64_t inter, int topk);
bool ftk_moe_fused_routes(int64_t n_expert);   // the fused layer can route this many experts itself
hipError_t ftk_launch_moe_fused(const MoeArgs& a, void* table, hipStream_t st);
hipError_t ftk_launch_moe_gate_up(const MoeArgs& a, hipStream_t st);
hipError_t ftk_launch_moe_down(const MoeArgs& a, hipStream_t st);
// MXFP4 x Q8_K direct-route stages on the FP4 MFMA (hidden, inter multiples of 256)
hipError_t ftk_launch_moe_fp4_gate_up(const MoeArgs& a, hipStream_t st);
hipError_t ftk_launch_moe_fp4_down(const MoeArgs& a, hipStream_t st);
// one token: MXFP4 down and the slot-order combine in one launch (y written; d only to d_tap)
bool ftk_moe_fp4_down_combine_ok(const MoeArgs& a);
hipError_t ftk_launch_moe_fp4_down_combine(const MoeArgs& a, hipStream_t st);
// y from the per-pair rows in dpair, slot order
hipError_t ftk_launch_moe_combine(const MoeArgs& a, hipStream_t st);

// grouped GEMM over expert-sorted pairs.  With W2 set W and W2 are
// the gate and up banks and y receives silu(g) * u.
struct GroupedArgs {
  int w, act;
  const void* W;
  const void* W2;          // nullable
  float* g_tap;            // nullable (W2 form)
  float* u_tap;            // nullable (W2 form)
  int64_t n_expert, n, k;
  const void* xq;
  const void* xf8;         // MXFP4: FP8 halves of xq (ftk_launch_fp8_split), 512 B per superblock
  int x_per_pair;
  int64_t t;
  int topk;
  const int32_t* counts;   // [E]   (device, from the sort)
  const int32_t* offsets;  // [E+1]
  const int32_t* pairs;    // [t*topk]
  float* y;                // [t*topk][n]
};
hipError_t ftk_launch_grouped(const GroupedArgs& a, hipStream_t st);

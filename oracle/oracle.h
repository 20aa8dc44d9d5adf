/*
 * oracle.h -- plain, slow CPU oracle for block-quantized matvec / routed MoE.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this library; only the tests, the smoke check and the bench's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * GPU library: every layout, table and formula below is written out again here.
 *
 * What it computes (the pages name the operations, not their arithmetic):
 *  - block layouts of Q4_0, Q8_0, Q4_K, Q5_K, Q6_K, MXFP4 weights and Q8_1 / Q8_K
 *    activations follow the public GGUF (ggml) block formats.  The pages only
 *    name the formats: FreeToken PR #136 "enable native GGUF kernels on ROCm"
 *    (Summary: Q4_0 dequantization), FreeToken PR #260 (Summary: packed Q4_K,
 *    Q5_K, Q6_K, Q8_0), vllm.cpp PR #523 "grouped + non-grouped keep-quant expert
 *    GEMM" (What changed: formats, Q8_0/Q8_K quantizers, DotQ* superblocks) and
 *    ds4 PR #656 "Add ROCm MXFP4 routed expert kernels" (Summary: MXFP4 x Q8_K).
 *  - the matvec is its plain definition: y = sum_k w_k * xhat_k with w and xhat
 *    the exact dequantized values, accumulated in fp64 and rounded once.
 *  - a second matvec follows the keep-quant method (integer block dots, then a
 *    scale combine) in fp64, so the two can be pinned against each other.
 *
 * Format codes are this library's own; callers map names to codes.
 * Parity vs real GGUF files: unpinned (no GGUF file is available); the layouts
 * are pinned by hand-built one-hot blocks against the written layout.
 */
#ifndef BQM_ORACLE_H
#define BQM_ORACLE_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* oracle format codes */
enum {
  OR_Q4_0 = 0, OR_Q8_0 = 1, OR_Q4_K = 2, OR_Q5_K = 3, OR_Q6_K = 4, OR_MXFP4 = 5,
  OR_Q8_1 = 6, OR_Q8_K = 7, OR_Q2_K = 8, OR_Q3_K = 9, OR_Q4_1 = 10, OR_Q5_0 = 11, OR_Q5_1 = 12
};

int    or_block_elems(int fmt);            /* 32 or 256, 0 for unknown */
int    or_block_bytes(int fmt);            /* bytes per block, 0 for unknown */
int    or_sub_elems(int wfmt);             /* elements per integer partial: 16 for Q2_K, Q3_K, Q6_K, else 32 */
int    or_threads(void);                   /* OpenMP threads the oracle will use */
void   or_set_threads(int n);              /* use n OpenMP threads from now on (n > 0) */

/* IEEE binary16 <-> binary32, written by hand (round to nearest even). */
float    or_f16_to_f32(uint16_t h);
uint16_t or_f32_to_f16(float f);
/* convert `count` consecutive fp32 bit patterns starting at `first` (wrapping
   is not allowed) -- used for the exhaustive check against a library routine */
void     or_f32_to_f16_range(uint32_t first, uint32_t count, uint16_t* out);

/* exact value of element e (0 <= e < block elems) of one block, in fp64 */
double or_elem(int fmt, const uint8_t* block, int e);

/* dequantize rows x k elements (rows*(k/blk) blocks, row-major) to fp32 */
void or_dequant_f32(int fmt, const uint8_t* blocks, int64_t rows, int64_t k, float* out);

/* activation quantizers: x [rows][k] fp32 (row stride ldx) -> rows*(k/blk) blocks */
void or_quantize(int afmt, const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* out);

/* integer partial per (token, row, sub-block): sum over the sub-block of the
   weight's integer code times the activation's int8 code.
   partials: [t][n][k/sub] int32.  Returns 0, or -1 for an unsupported pair. */
int or_block_dots(int wfmt, const uint8_t* W, int64_t n, int64_t k,
                  int afmt, const uint8_t* xq, int64_t t, int32_t* partials);

/* plain definition: y[t][n] = sum_k w[n][k] * xhat[t][k] in fp64, rounded once.
   ldy >= n.  Returns 0, or -1 if k is not a multiple of both block sizes. */
int or_matvec(int wfmt, const uint8_t* W, int64_t n, int64_t k,
              int afmt, const uint8_t* xq, int64_t t, float* y, int64_t ldy);

/* keep-quant method: integer block dots + per-block scale combine, in fp64. */
int or_matvec_keepquant(int wfmt, const uint8_t* W, int64_t n, int64_t k,
                        int afmt, const uint8_t* xq, int64_t t, double* y);

/* routing: top-k of logits [t][E] (ties toward the lower expert index, slot 0 the
   largest), weights = softmax over the selected logits (fp64 -> fp32). */
int or_route(const float* logits, int64_t t, int64_t n_expert, int topk,
             int32_t* ids, float* w);

/* stable token->expert sort of the t*topk (token, slot) pairs by expert id.
   counts [E], offsets [E+1], pairs [t*topk] (pair index = token*topk + slot). */
int or_sort_pairs(const int32_t* ids, int64_t t, int topk, int64_t n_expert,
                  int32_t* counts, int32_t* offsets, int32_t* pairs);

/* routed MoE, stage by stage.
   gate/up: g,u,h [t*topk][inter]; g = Wg[e].xhat_t, u = Wu[e].xhat_t, h = silu(g)*u.
   Weight banks [E][inter][hidden/blk]. */
int or_moe_gate_up(int wfmt, const uint8_t* w_gate, const uint8_t* w_up,
                   int64_t n_expert, int64_t hidden, int64_t inter,
                   int afmt, const uint8_t* xq, int64_t t,
                   const int32_t* ids, int topk, float* g, float* u, float* h);
/* down: d [t*topk][hidden] = Wd[e] . hq[pair]; Wd bank [E][hidden][inter/blk] */
int or_moe_down(int wfmt, const uint8_t* w_down, int64_t n_expert, int64_t hidden,
                int64_t inter, int afmt, const uint8_t* hq, int64_t t,
                const int32_t* ids, int topk, float* d);
/* combine: y[t][hidden] = sum_k w[t][k] * d[t*topk+k][:] (fp64, rounded once) */
void or_moe_combine(const float* d, const float* w, int64_t t, int topk,
                    int64_t hidden, float* y);

/* grouped keep-quant GEMM:
   y[p][:] = W[ids[p]] . xhat_row, p = token*topk + slot, row = p if x_per_pair else token.
   W bank [E][n][k/blk]; y [t*topk][n]. */
int or_grouped(int wfmt, const uint8_t* W, int64_t n_expert, int64_t n, int64_t k,
               int afmt, const uint8_t* xq, int x_per_pair,
               const int32_t* ids, int64_t t, int topk, float* y);

#ifdef __cplusplus
}
#endif
#endif

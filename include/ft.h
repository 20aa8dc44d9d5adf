/*
 * ft.h -- C ABI of libft.so: block-quantized matvec, routed-MoE vector path and
 * grouped keep-quant expert GEMM on AMD Instinct MI355X (gfx950).
 *
 * Sources the operations come from (cited by page title and section):
 *  [P1] FreeToken PR #136 "enable native GGUF kernels on ROCm (validated on RDNA4)",
 *       Summary: Q4_0 dequantization, the int8-dot matvec (mul_mat_vec with
 *       quantized activations) and the routed MoE vector kernel.
 *  [P2] FreeToken PR #260 "validate native gfx1151 serving on Strix Halo",
 *       Summary: packed Q4_K, Q5_K, Q6_K and Q8_0 weights kept quantized.
 *  [P3] vllm.cpp PR #523 "grouped + non-grouped keep-quant expert GEMM",
 *       What changed: Y = X.W^T with keep-quant W (non-grouped op) and the same
 *       grouped over expert_ids; Q8_0/Q8_K activation quantizers; per-superblock
 *       integer dots.  Review and rework: a per-format availability query in place
 *       of a boolean, refusal before the first forward, a grow-only per-stream
 *       scratch pool with no per-call malloc, free or synchronize.
 *  [P4] ds4 PR #656 "Add ROCm MXFP4 routed expert kernels", Summary: MXFP4 x Q8_K
 *       routed gate/up and down, SwiGLU between them, tiny batches (2-4 tokens)
 *       on direct kernels and larger ones on expert-sorted tiles.
 * Block byte layouts are the public GGUF (ggml) formats; the pages name the
 * formats but do not print them.
 *
 * Conventions for every call:
 *  - Pointers are device pointers unless stated.  The caller owns every input
 *    and output buffer; the library owns only its scratch pool.
 *  - Layouts are row-major, little-endian.  Weights are [rows][k/blk] blocks
 *    with rows the outputs (y = W.x).  Activations are [tokens][k/blk_a] blocks.
 *  - Weight, block and activation base pointers must be 16-byte aligned
 *    (FT_ERR_ALIGNMENT otherwise).  Kernels may read up to 15 bytes past the end
 *    of a weight buffer whose size is not a multiple of 16; such reads never
 *    cross a 4 KiB page.
 *  - Work is enqueued on `stream` (0 = the null stream) and the call returns.
 *    No call synchronizes.  After ft_scratch_reserve() has sized the pool, no
 *    call allocates, so the calls may be captured in a HIP graph.
 *  - Errors are returned as ft_status, nothing throws.  Host-checkable
 *    conditions (NULL, shapes, unsupported pairs) are refused before any work
 *    is enqueued.  Out-of-range expert ids and non-finite inputs are outside
 *    the contract (results undefined, never a memory fault: ids are clamped).
 *  - Calls on different streams may run concurrently; calls that share a
 *    stream's scratch pool are ordered by that stream.
 */
#ifndef FT_H
#define FT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* ft_stream_t; /* a hipStream_t */

/* block formats */
typedef enum {
  FT_Q4_0 = 0,  /* 32 weights: fp16 d, 16 B nibbles; w = d*(n-8)            18 B */
  FT_Q8_0 = 1,  /* 32 weights (or activations): fp16 d, 32 int8; w = d*q     34 B */
  FT_Q4_K = 2,  /* 256: fp16 d, fp16 dmin, 12 B of 6-bit scales/mins, 128 B nibbles;
                   w = d*sc_j*n - dmin*m_j per 32-element sub-block j       144 B */
  FT_Q5_K = 3,  /* 256: as Q4_K plus 32 B of fifth bits                     176 B */
  FT_Q6_K = 4,  /* 256: 128 B low nibbles, 64 B high 2-bit pairs, 16 int8 scales,
                   fp16 d; w = d*sc*(q6-32) per 16-element sub-block         210 B */
  FT_MXFP4 = 5, /* 32: E8M0 exponent e, 16 B E2M1 codes; w = E2M1*2^(e-127)   17 B */
  FT_Q8_1 = 6,  /* activation, 32: fp16 d, fp16 s = d*sum(q), 32 int8         36 B */
  FT_Q8_K = 7,  /* activation, 256: fp32 d, 256 int8, 16 int16 group sums   292 B */
  FT_Q2_K = 8,  /* 256: 16 B of 4-bit scale|min pairs, 64 B of 2-bit codes, fp16 d,
                   fp16 dmin; w = d*sc*q - dmin*m per 16 elements              84 B */
  FT_Q3_K = 9,  /* 256: 32 B third bits, 64 B of 2-bit codes, 12 B of 6-bit
                   scales (+32), fp16 d; w = d*(sc-32)*(q-4) per 16 elements 110 B */
  FT_Q4_1 = 10, /* 32: fp16 d, fp16 m, 16 B nibbles; w = d*n + m              20 B */
  FT_Q5_0 = 11, /* 32: fp16 d, 4 B fifth bits, 16 B nibbles; w = d*(q-16)     22 B */
  FT_Q5_1 = 12  /* 32: fp16 d, fp16 m, 4 B fifth bits, 16 B nibbles; w = d*q + m
                                                                            24 B */
} ft_type;

typedef enum {
  FT_OK = 0,
  FT_ERR_INVALID_ARG = 1, /* NULL pointer, negative size, bad option */
  FT_ERR_UNSUPPORTED = 2, /* (op, weight, activation) combination not provided */
  FT_ERR_SHAPE = 3,       /* k not a multiple of the block sizes, topk out of range */
  FT_ERR_ALIGNMENT = 4,   /* a base pointer is not 16-byte aligned */
  FT_ERR_NO_SCRATCH = 5,  /* the pool is too small and the stream is capturing */
  FT_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed */
} ft_status;

typedef enum {
  FT_OP_QUANTIZE = 0, FT_OP_DEQUANT = 1, FT_OP_MMVQ = 2, FT_OP_MOE_VEC = 3,
  FT_OP_GROUPED = 4, FT_OP_BLOCK_DOTS = 5
} ft_op;

/* Elements per block (32 or 256) and bytes per block; 0 for an unknown type. */
int ft_block_elems(ft_type type);
size_t ft_block_bytes(ft_type type);

/* Per-format availability, answered on the host before any data exists [P3,
   review: a per-dtype query instead of a boolean].  Returns 1 if `op` runs for
   (w, act); act is ignored for FT_OP_DEQUANT and w for FT_OP_QUANTIZE.
   Every combination reported 0 makes the op return FT_ERR_UNSUPPORTED. */
int ft_supported(ft_op op, ft_type w, ft_type act);

/* Human-readable status. */
const char* ft_status_str(ft_status status);

/* Library version string (static storage). */
const char* ft_version(void);

/* Activation quantizer [P3 What changed: Q8_0/Q8_K quantizers; P4: Q8 prequant].
   x: [rows][k] fp32 with row stride ldx (elements) >= k.  xq: [rows][k/blk] blocks
   of `act` (FT_Q8_1, FT_Q8_0 or FT_Q8_K), written in full.
   Q8_1 per 32-block: d = fp16(amax/127); q = clamp(round_half_away(x/d), -127, 127)
   against the stored d (q = 0 when d is 0); s = fp16(d * sum q).
   Q8_0 per 32-block: d and q as Q8_1, no s (fp16 d at byte 0, codes from byte 2).
   Q8_K per 256-block: d = amax/127 in fp32; q as above; bsums[g] = sum of q over
   elements 16g..16g+15. */
ft_status ft_quantize_act(ft_type act, const float* x, int64_t rows, int64_t k, int64_t ldx,
                          void* xq, ft_stream_t stream);

/* Dequantization [P1 Summary: Q4_0 dequantization; P2: packed K-quants].
   blocks: [rows][k/blk] of weight type w.  out: [rows][k] fp32 -- each value is
   the exact weight rounded once to fp32 (exact for every format but the Q4_K /
   Q5_K / Q2_K difference d*sc*n - dmin*m and the Q4_1 / Q5_1 sum d*q + m, which
   round once). */
ft_status ft_dequant(ft_type w, const void* blocks, int64_t rows, int64_t k, float* out,
                     ft_stream_t stream);

/* Quantized matvec [P1 Summary: int8-dot matvec; P3 What changed: non-grouped op].
   W: [n][k/blk] blocks of w; xq: [t][k/blk_a] blocks of act;
   y: [t][ldy] fp32, ldy >= n, y[i][r] = sum_k w[r][k] * xhat[i][k], computed as exact
   integer dots per block followed by an fp32 scale combine.  Any t >= 0 (t = 0 is a
   no-op); batches beyond 8 tokens are processed 8 at a time.  Supported (w, act):
   every weight type x FT_Q8_1 and x FT_Q8_0; (Q4_K, Q5_K, Q6_K, MXFP4) x FT_Q8_K
   [P3 What changed: the non-grouped op with Q8_0 / Q8_K activations].  With
   FT_Q8_1 or FT_Q8_0, from 2-5 tokens on (the threshold depends on the format and
   on k) every format runs on the int8 matrix cores when k is a multiple of 256 (512
   for MXFP4); the result is the same integer dots either way.  FT_Q8_0 activations
   are first copied into the Q8_1 block layout (same d and codes) in the stream's
   scratch pool, so under graph capture the pool must hold t*(k/32)*36 bytes
   (FT_ERR_NO_SCRATCH otherwise).  FT_Q8_K runs on the dot4 kernels at every t. */
ft_status ft_mul_mat_vec_q(ft_type w, const void* W, int64_t n, int64_t k,
                           ft_type act, const void* xq, int64_t t,
                           float* y, int64_t ldy, ft_stream_t stream);

/* Router [P4 Summary; routing semantics as read from the pages]:
   logits [t][n_expert] fp32 -> ids [t][topk] int32 (the topk largest logits, ties
   toward the lower expert index, slot 0 the largest) and w [t][topk] fp32 = softmax
   over the selected logits.  1 <= topk <= min(8, n_expert), n_expert <= 1024. */
ft_status ft_moe_route(const float* logits, int64_t t, int64_t n_expert, int topk,
                       int32_t* ids, float* w, ft_stream_t stream);

/* Stable token->expert sort of the t*topk (token, slot) pairs [P4: expert-sorted
   tiles].  counts [n_expert], offsets [n_expert+1] (exclusive prefix sum), pairs
   [t*topk] = pair indices (token*topk + slot) ordered by expert, ascending pair index
   within an expert.  All int32. */
ft_status ft_moe_sort(const int32_t* ids, int64_t t, int topk, int64_t n_expert,
                      int32_t* counts, int32_t* offsets, int32_t* pairs, ft_stream_t stream);

/* Options of ft_moe_q_vec; pass NULL for defaults. */
typedef struct {
  int route;          /* 0 auto, 1 force the direct route ((Q4_K, Q8_1) and (MXFP4,
                         Q8_K) only), 2 force sorted tiles (every (w, Q8_K) pair);
                         a route the pair lacks gives FT_ERR_UNSUPPORTED */
  int direct_max_t;   /* auto route: direct for t <= direct_max_t (0 = default 8),
                         sorted tiles above it where supported; pairs without a
                         direct route take the tiles at every t */
  float* tap_g;       /* nullable [t*topk][inter] fp32: gate projections */
  float* tap_u;       /* nullable [t*topk][inter] fp32: up projections */
  float* tap_h;       /* nullable [t*topk][inter] fp32: silu(g)*u */
  void* tap_hq;       /* nullable [t*topk][inter/blk_a] blocks: quantized h */
  float* tap_down;    /* nullable [t*topk][hidden] fp32: per-pair down projections */
  const void* in_hq;  /* nullable: use these quantized h blocks for the down stage */
  const float* logits;/* nullable [t][n_expert] router logits (n_expert <= 1024): the layer
                         routes each token itself, as ft_moe_route, and expert_ids /
                         expert_w are not read (they may be NULL) */
  int32_t* ids_out;   /* nullable [t][topk]: receives that routing's ids ... */
  float* w_out;       /* nullable [t][topk]: ... and weights */
} ft_moe_opts;

/* Routed-MoE layer [P1: routed MoE vector kernel; P4: gate/up, SwiGLU, down].
   w_gate, w_up: [n_expert][inter][hidden/blk]; w_down: [n_expert][hidden][inter/blk],
   all of weight type w.  x: [t][hidden] fp32.  expert_ids, expert_w: [t][topk].
   For every token i and slot s with e = expert_ids[i][s]:
     g = W_gate[e].xhat_i, u = W_up[e].xhat_i (xhat = act-quantized x_i),
     h = silu(g)*u, hhat = act-quantized h, d = W_down[e].hhat,
   and y[i] = sum over s (in slot order) of expert_w[i][s] * d.  y: [t][hidden] fp32.
   The topk ids of one token must be distinct (as top-k routing makes them).
   Supported (w, act): (Q4_K, Q8_1) and (MXFP4, Q8_K) on both routes; (Q4_K, Q8_K),
   (Q5_K, Q8_K), (Q6_K, Q8_K) on the sorted tiles.  topk 1..8; n_expert <= 8192 on
   the sorted tiles.
   Routes [P4 Summary: tiny batches direct, larger ones on expert-sorted tiles;
   P3 What changed: the grouped keep-quant op over expert_ids]:
   direct = the selected experts' rows streamed once per chunk of tokens, every token
   that picked an expert served from the same bytes: for (Q4_K, Q8_1) with hidden
   and inter multiples of 256 up to 4096 (inter up to about 1536), two launches per
   4-token chunk (routing from the logits, x quantize, gate/up + SwiGLU, h quantize;
   then down and the slot-order combine), otherwise one workgroup per selected
   expert and row tile per stage, then a combine; for (MXFP4, Q8_K) the gate/up
   launch routes 1-2 tokens from the logits itself, and at 1-2 tokens down and the
   combine are one launch whose workgroups each take one token's rows (an expert
   both tokens picked is read once per token there);
   sorted tiles = token->expert sort, one fused gate/up + SwiGLU grouped MFMA GEMM,
   h quantize, grouped down GEMM, slot-order combine.  Both give the same result
   up to fp32 rounding order. */
ft_status ft_moe_q_vec(ft_type w, const void* w_gate, const void* w_up, const void* w_down,
                       int64_t n_expert, int64_t hidden, int64_t inter,
                       ft_type act, const float* x, int64_t t,
                       const int32_t* expert_ids, const float* expert_w, int topk,
                       float* y, const ft_moe_opts* opts, ft_stream_t stream);

/* The same layer for callers that cannot allocate device memory (code under HIP
   graph capture, serving loops that must not call hipMalloc, harnesses that forbid
   it).  Arguments, routes, results and errors as ft_moe_q_vec; its scratch is a
   fixed device array of FT_NOALLOC_SCRATCH_BYTES per GPU, held by the library until
   the process ends, instead of the stream's pool.  A problem whose scratch
   (ft_moe_scratch_bytes) exceeds that size is refused with FT_ERR_SHAPE before
   anything is enqueued.  Calls on one GPU share that array: calls that may overlap
   on one GPU (different streams) race and must be ordered by the caller.  Nothing
   in the array needs to start at zero.  The first call on a device looks the
   array's address up (hipGetSymbolAddress) and keeps it. */
#define FT_NOALLOC_SCRATCH_BYTES (32u << 20)
ft_status ft_moe_q_vec_noalloc(ft_type w, const void* w_gate, const void* w_up, const void* w_down,
                               int64_t n_expert, int64_t hidden, int64_t inter,
                               ft_type act, const float* x, int64_t t,
                               const int32_t* expert_ids, const float* expert_w, int topk,
                               float* y, const ft_moe_opts* opts, ft_stream_t stream);

/* Grouped keep-quant expert GEMM [P3 What changed: grouped over expert_ids].
   W: [n_expert][n][k/blk] blocks; xq: act blocks, [t][k/blk_a] when x_per_pair = 0
   (every slot of a token reads its token's row) or [t*topk][k/blk_a] when 1.
   y: [t*topk][n] fp32 in (token, slot) order: y[p] = W[ids[p]] . xhat_row(p).
   Supported (w, act): (Q5_K, Q8_K), (Q6_K, Q8_K), (MXFP4, Q8_K), (Q4_K, Q8_K). */
ft_status ft_grouped_gemm_q(ft_type w, const void* W, int64_t n_expert, int64_t n, int64_t k,
                            ft_type act, const void* xq, int x_per_pair,
                            const int32_t* expert_ids, int64_t t, int topk,
                            float* y, ft_stream_t stream);

/* Integer partials of the block dots (debug tap; [P3 What changed: bit-identical
   integer core]).  partials: [t][n][k/sub] int32, sub = 16 for Q2_K, Q3_K and Q6_K
   and 32 otherwise: the sum over each sub-block of the weight's integer code (n-8 for
   Q4_0, q for Q8_0, the 4/5-bit n for Q4_K/Q5_K, q6-32 for Q6_K, twice the E2M1 value
   for MXFP4, the 2-bit q for Q2_K, the 3-bit q-4 for Q3_K) times the activation's
   int8 code (act: FT_Q8_1, FT_Q8_0 -- through its Q8_1 layout, as the matvec --
   or FT_Q8_K).  Computed with the unpack and v_dot4 core of the dot4 matvec kernels
   (one and two tokens); the int8-MFMA matvec, the grouped GEMM and the FP4-MFMA
   MoE kernels form the same integers on the matrix cores and are checked for
   them through exactly representable outputs instead. */
ft_status ft_debug_block_dots(ft_type w, const void* W, int64_t n, int64_t k,
                              ft_type act, const void* xq, int64_t t,
                              int32_t* partials, ft_stream_t stream);

/* Measurement microkernels (not part of the method): the ceilings the hot path is
   held against, measured on the part next to its published peaks.
   which = 0: streaming read of `bytes` bytes at `buf` (device, 16-byte aligned,
   bytes a multiple of 16) with 16-byte loads; which = 1: `iters` rounds of eight
   independent int8 MFMA chains (v_mfma_i32_16x16x32_i8, 16384 ops each) per wave;
   which = 2: `iters` rounds of eight independent v_dot4_i32_i8 chains per lane
   (8 ops per lane each); which = 3: as 1 with v_mfma_i32_16x16x64_i8 (32768 ops
   each).  1-3 run 8 workgroups of 256 threads per CU and ignore buf/bytes.  out: one device uint32 that receives nothing in practice (it keeps
   the work live).  The caller times the call. */
ft_status ft_debug_ceiling(int which, const void* buf, int64_t bytes, int64_t iters, void* out,
                           ft_stream_t stream);

/* Grow the stream's scratch pool to at least `bytes` [P3 review: grow-only
   per-stream pool].  Call before capturing a graph.  The pool is never shrunk;
   retired buffers are released by ft_shutdown(). */
ft_status ft_scratch_reserve(ft_stream_t stream, size_t bytes);

/* Scratch bytes ft_moe_q_vec / ft_grouped_gemm_q need for a problem size. */
size_t ft_moe_scratch_bytes(ft_type w, ft_type act, int64_t n_expert, int64_t hidden,
                            int64_t inter, int64_t t, int topk);
size_t ft_grouped_scratch_bytes(ft_type w, int64_t n_expert, int64_t k, int64_t t, int topk, int x_per_pair);

/* Release every scratch buffer.  No call may be in flight. */
void ft_shutdown(void);

#ifdef __cplusplus
}
#endif
#endif /* FT_H */

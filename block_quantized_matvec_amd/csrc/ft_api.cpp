// ft_api.cpp -- the C ABI of libft.so: argument validation, the per-format
// capability table, the per-stream grow-only scratch pool and dispatch.
//
// Refusal happens on the host before anything is enqueued, and the capability
// table is the one the dispatcher uses (vllm.cpp PR #523, review and rework:
// per-dtype availability instead of a boolean; refuse before the first
// forward).  Scratch comes from a per-stream pool that only grows and retires
// buffers instead of freeing them while work may be in flight (same PR: a
// grow-only per-stream pool, no per-call malloc/free/synchronize).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "ft.h"
#include "ft_internal.h"

namespace {

constexpr int kTypes = 13;
constexpr int kElems[kTypes] = {32, 32, 256, 256, 256, 32, 32, 256, 256, 256, 32, 32, 32};
constexpr int kBytes[kTypes] = {18, 34, 144, 176, 210, 17, 36, 292, 84, 110, 20, 22, 24};

bool is_weight(int t) { return (t >= FT_Q4_0 && t <= FT_MXFP4) || (t >= FT_Q2_K && t <= FT_Q5_1); }
// Q8_0 is a weight format and, with the same block layout, an activation format
bool is_act(int t) { return t == FT_Q8_1 || t == FT_Q8_K || t == FT_Q8_0; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
int64_t row_bytes_of(int type, int64_t k) { return k / kElems[type] * kBytes[type]; }

hipStream_t hs(ft_stream_t s) { return (hipStream_t)s; }

ft_status hip_status(hipError_t e) { return e == hipSuccess ? FT_OK : FT_ERR_HIP; }

// --------------------------------------------------------------------------
// scratch pool
// --------------------------------------------------------------------------
struct Pool {
  void* ptr = nullptr;
  size_t size = 0;
  std::vector<void*> retired;
};
std::mutex g_pool_mu;
std::unordered_map<hipStream_t, Pool> g_pools;

ft_status pool_get(hipStream_t st, size_t bytes, void** out) {
  std::lock_guard<std::mutex> lk(g_pool_mu);
  Pool& p = g_pools[st];
  if (p.size >= bytes) {
    *out = p.ptr;
    return FT_OK;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return FT_ERR_HIP;
  if (cs != hipStreamCaptureStatusNone) return FT_ERR_NO_SCRATCH;
  size_t want = std::max(bytes, 2 * p.size);
  want = (want + ((size_t)1 << 20) - 1) & ~(((size_t)1 << 20) - 1);
  void* np = nullptr;
  if (hipMalloc(&np, want) != hipSuccess) return FT_ERR_HIP;
  if (p.ptr) p.retired.push_back(p.ptr);  // work already enqueued may still use it
  p.ptr = np;
  p.size = want;
  *out = np;
  return FT_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// scratch layout of ft_moe_q_vec
struct MoeScratch {
  size_t xq, h, hq, d, ids, w, tab, total;
};
MoeScratch moe_layout(int w, int act, int64_t hidden, int64_t inter, int64_t t, int topk) {
  (void)w;
  MoeScratch s;
  size_t off = 0;
  s.xq = off;
  off += align256((size_t)t * row_bytes_of(act, hidden));
  s.h = off;
  off += align256((size_t)t * topk * inter * sizeof(float));
  s.hq = off;
  off += align256((size_t)t * topk * row_bytes_of(act, inter));
  s.d = off;
  off += align256((size_t)t * topk * hidden * sizeof(float));
  s.ids = off;   // the routing when the layer routes from logits
  off += align256((size_t)t * topk * 4);
  s.w = off;
  off += align256((size_t)t * topk * 4);
  s.tab = off;   // the fused Q4_K layer's routing table (its first launch -> its second)
  off += align256(ftk_moe_fused_table_bytes());
  s.total = off;
  return s;
}

// scratch layout of the grouped GEMM: the sort, then (MXFP4) the FP8 halves of
// the activation rows (512 bytes per row and superblock)
struct SortScratch {
  size_t counts, offsets, pairs, xf8, total;
};
SortScratch sort_layout(int64_t n_expert, int64_t t, int topk, size_t xf8_bytes = 0) {
  SortScratch s;
  size_t off = 0;
  s.counts = off;
  off += align256((size_t)n_expert * 4);
  s.offsets = off;
  off += align256((size_t)(n_expert + 1) * 4);
  s.pairs = off;
  off += align256((size_t)t * topk * 4);
  s.xf8 = off;
  off += align256(xf8_bytes);
  s.total = off;
  return s;
}
size_t xf8_bytes_of(int w, int64_t rows, int64_t k) { return w == FT_MXFP4 ? (size_t)rows * (k / 256) * 512 : 0; }

// every weight format x Q8_1 or Q8_0; the grouped-GEMM formats x Q8_K
bool mmvq_pair(int w, int a) {
  return ((a == FT_Q8_1 || a == FT_Q8_0) && is_weight(w)) ||
         (a == FT_Q8_K && (w == FT_Q4_K || w == FT_Q5_K || w == FT_Q6_K || w == FT_MXFP4));
}
// the direct route: Q4_K x Q8_1 on dot4, MXFP4 x Q8_K on the FP4 MFMA; the sorted
// tiles: every grouped-GEMM format x Q8_K
bool moe_direct_pair(int w, int a) { return (w == FT_Q4_K && a == FT_Q8_1) || (w == FT_MXFP4 && a == FT_Q8_K); }
bool moe_tile_pair(int w, int a) {
  return a == FT_Q8_K && (w == FT_Q4_K || w == FT_Q5_K || w == FT_Q6_K || w == FT_MXFP4);
}
bool moe_pair(int w, int a) { return moe_direct_pair(w, a) || moe_tile_pair(w, a); }
// the tile route splits x, then h, into FP8 halves in one buffer
size_t moe_xf8_bytes(int w, int64_t hidden, int64_t inter, int64_t t, int topk) {
  const size_t a = xf8_bytes_of(w, t, hidden), b = xf8_bytes_of(w, t * topk, inter);
  return a > b ? a : b;
}
bool grouped_pair(int w, int a) {
  return a == FT_Q8_K && (w == FT_Q4_K || w == FT_Q5_K || w == FT_Q6_K || w == FT_MXFP4);
}

}  // namespace

extern "C" {

int ft_block_elems(ft_type t) { return ((int)t >= 0 && (int)t < kTypes) ? kElems[t] : 0; }
size_t ft_block_bytes(ft_type t) { return ((int)t >= 0 && (int)t < kTypes) ? (size_t)kBytes[t] : 0; }

const char* ft_version(void) { return "ft 0.1 (gfx950)"; }

int ft_supported(ft_op op, ft_type w, ft_type act) {
  switch (op) {
    case FT_OP_QUANTIZE: return is_act(act);
    case FT_OP_DEQUANT: return is_weight(w);
    case FT_OP_MMVQ: return mmvq_pair(w, act);
    case FT_OP_MOE_VEC: return moe_pair(w, act);
    case FT_OP_GROUPED: return grouped_pair(w, act);
    case FT_OP_BLOCK_DOTS: return is_weight(w) && is_act(act);
  }
  return 0;
}

const char* ft_status_str(ft_status s) {
  switch (s) {
    case FT_OK: return "ok";
    case FT_ERR_INVALID_ARG: return "invalid argument";
    case FT_ERR_UNSUPPORTED: return "unsupported format combination";
    case FT_ERR_SHAPE: return "shape not supported (block multiple, topk or size limit)";
    case FT_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case FT_ERR_NO_SCRATCH: return "scratch pool too small while capturing";
    case FT_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

ft_status ft_quantize_act(ft_type act, const float* x, int64_t rows, int64_t k, int64_t ldx, void* xq,
                          ft_stream_t stream) {
  if (!is_act(act)) return FT_ERR_UNSUPPORTED;
  if (rows < 0 || k < 0 || ldx < k) return FT_ERR_INVALID_ARG;
  if (k % kElems[act]) return FT_ERR_SHAPE;
  if (rows == 0 || k == 0) return FT_OK;
  if (!x || !xq) return FT_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(xq)) return FT_ERR_ALIGNMENT;
  return hip_status(ftk_launch_quantize(act, x, rows, k, ldx, xq, hs(stream)));
}

ft_status ft_dequant(ft_type w, const void* blocks, int64_t rows, int64_t k, float* out, ft_stream_t stream) {
  if (!is_weight(w)) return FT_ERR_UNSUPPORTED;
  if (rows < 0 || k < 0) return FT_ERR_INVALID_ARG;
  if (k % kElems[w]) return FT_ERR_SHAPE;
  if (rows == 0 || k == 0) return FT_OK;
  if (!blocks || !out) return FT_ERR_INVALID_ARG;
  if (!aligned16(blocks) || !aligned16(out)) return FT_ERR_ALIGNMENT;
  return hip_status(ftk_launch_dequant(w, blocks, rows, k, out, hs(stream)));
}

ft_status ft_mul_mat_vec_q(ft_type w, const void* W, int64_t n, int64_t k, ft_type act, const void* xq, int64_t t,
                           float* y, int64_t ldy, ft_stream_t stream) {
  if (!is_weight(w) || !is_act(act) || !mmvq_pair(w, act)) return FT_ERR_UNSUPPORTED;
  if (n < 0 || k < 0 || t < 0 || ldy < n) return FT_ERR_INVALID_ARG;
  if (k % kElems[w] || k % kElems[act]) return FT_ERR_SHAPE;
  if (k > 32768 || n > ((int64_t)1 << 31) / 2) return FT_ERR_SHAPE;
  if (n == 0 || t == 0) return FT_OK;
  if (!W || !xq || !y) return FT_ERR_INVALID_ARG;
  if (k == 0) return FT_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(xq) || !aligned16(y)) return FT_ERR_ALIGNMENT;
  if (act == FT_Q8_0) {   // the Q8_1 layout of the same blocks, in the stream's pool
    void* rp = nullptr;
    const int64_t nblk = t * (k / 32);
    const ft_status ps = pool_get(hs(stream), align256((size_t)nblk * 36), &rp);
    if (ps != FT_OK) return ps;
    const hipError_t e = ftk_launch_repack_q8_0(xq, nblk, rp, hs(stream));
    if (e != hipSuccess) return FT_ERR_HIP;
    xq = rp;
    act = FT_Q8_1;
  }
  MmvqArgs a;
  a.w = w;
  a.act = act;
  a.W = W;
  a.n = n;
  a.row_bytes = (int)row_bytes_of(w, k);
  a.units_per_row = 0;
  a.xrow_bytes = (int)row_bytes_of(act, k);
  a.ldy = ldy;
  for (int64_t t0 = 0; t0 < t; t0 += 8) {
    a.t = (int)std::min<int64_t>(8, t - t0);
    a.xq = (const uint8_t*)xq + t0 * a.xrow_bytes;
    a.y = y + t0 * ldy;
    const hipError_t e = ftk_launch_mmvq(a, k, hs(stream));
    if (e != hipSuccess) return FT_ERR_HIP;
  }
  return FT_OK;
}

ft_status ft_moe_route(const float* logits, int64_t t, int64_t n_expert, int topk, int32_t* ids, float* w,
                       ft_stream_t stream) {
  if (t < 0 || n_expert < 1 || n_expert > 1024) return FT_ERR_SHAPE;
  if (topk < 1 || topk > 8 || topk > n_expert) return FT_ERR_SHAPE;
  if (t == 0) return FT_OK;
  if (!logits || !ids || !w) return FT_ERR_INVALID_ARG;
  return hip_status(ftk_launch_route(logits, t, n_expert, topk, ids, w, hs(stream)));
}

ft_status ft_moe_sort(const int32_t* ids, int64_t t, int topk, int64_t n_expert, int32_t* counts, int32_t* offsets,
                      int32_t* pairs, ft_stream_t stream) {
  if (t < 0 || n_expert < 1 || n_expert > 8192 || topk < 1 || topk > 8) return FT_ERR_SHAPE;
  if (!counts || !offsets || (t > 0 && (!ids || !pairs))) return FT_ERR_INVALID_ARG;
  return hip_status(ftk_launch_sort(ids, t, topk, n_expert, counts, offsets, pairs, hs(stream)));
}

size_t ft_moe_scratch_bytes(ft_type w, ft_type act, int64_t n_expert, int64_t hidden, int64_t inter, int64_t t,
                            int topk) {
  if (!is_act(act) || t < 0 || topk < 0 || n_expert < 1) return 0;
  // the sorted-tile route also needs the sort's buffers
  return moe_layout(w, act, hidden, inter, t, topk).total +
         (moe_tile_pair(w, act) ? sort_layout(n_expert, t, topk, moe_xf8_bytes(w, hidden, inter, t, topk)).total : 0);
}

size_t ft_grouped_scratch_bytes(ft_type w, int64_t n_expert, int64_t k, int64_t t, int topk, int x_per_pair) {
  if (n_expert < 1 || k < 0 || t < 0 || topk < 1) return 0;
  return sort_layout(n_expert, t, topk, xf8_bytes_of(w, x_per_pair ? t * topk : t, k)).total;
}

}  // extern "C"

namespace {

// Host-side checks of ft_moe_q_vec; on FT_OK, *tiles says which route runs and
// *need the scratch bytes it takes.
ft_status moe_check(ft_type w, const void* w_gate, const void* w_up, const void* w_down, int64_t n_expert,
                    int64_t hidden, int64_t inter, ft_type act, const float* x, int64_t t,
                    const int32_t* expert_ids, const float* expert_w, int topk, float* y, const ft_moe_opts& o,
                    bool* tiles, size_t* need) {
  if (!is_weight(w) || !is_act(act) || !moe_pair(w, act)) return FT_ERR_UNSUPPORTED;
  if (n_expert < 1 || hidden < 0 || inter < 0 || t < 0) return FT_ERR_INVALID_ARG;
  if (topk < 1 || topk > 8 || topk > n_expert) return FT_ERR_SHAPE;
  if (hidden % kElems[w] || hidden % kElems[act] || inter % kElems[w] || inter % kElems[act]) return FT_ERR_SHAPE;
  if (hidden == 0 || inter == 0 || hidden > 16384 || inter > 16384) return FT_ERR_SHAPE;
  if (o.route < 0 || o.route > 2 || o.direct_max_t < 0) return FT_ERR_INVALID_ARG;
  const bool tile_ok = moe_tile_pair(w, act), direct_ok = moe_direct_pair(w, act);
  if ((o.route == 2 && !tile_ok) || (o.route == 1 && !direct_ok)) return FT_ERR_UNSUPPORTED;
  // default threshold: up to 8 tokens (one launch chunk of the direct MXFP4 kernels)
  // the direct route wins on MI355X (measured per layer: t = 8: 284 vs 290 us; t = 9:
  // 317 vs 298 us for the sorted tiles); pairs with no direct kernels take the tiles
  const int64_t dmax = o.direct_max_t > 0 ? o.direct_max_t : 8;
  *tiles = o.route == 2 || (o.route == 0 && (!direct_ok || (tile_ok && t > dmax)));
  // the sort behind the tiles holds one counter per expert in LDS
  if (*tiles && n_expert > 8192) return FT_ERR_SHAPE;
  if (o.logits && n_expert > 1024) return FT_ERR_SHAPE;   // the router's limit
  if (t == 0) return FT_OK;
  if (!w_gate || !w_up || !w_down || !x || !y) return FT_ERR_INVALID_ARG;
  if (!o.logits && (!expert_ids || !expert_w)) return FT_ERR_INVALID_ARG;
  if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(x) || !aligned16(y))
    return FT_ERR_ALIGNMENT;
  if ((o.tap_g && !aligned16(o.tap_g)) || (o.tap_u && !aligned16(o.tap_u)) || (o.tap_h && !aligned16(o.tap_h)) ||
      (o.tap_hq && !aligned16(o.tap_hq)) || (o.tap_down && !aligned16(o.tap_down)) ||
      (o.in_hq && !aligned16(o.in_hq)))
    return FT_ERR_ALIGNMENT;
  *need = moe_layout(w, act, hidden, inter, t, topk).total +
          (*tiles ? sort_layout(n_expert, t, topk, moe_xf8_bytes(w, hidden, inter, t, topk)).total : 0);
  return FT_OK;
}

// The layer on checked arguments, its scratch at b (moe_check's `need` bytes).
ft_status moe_run(ft_type w, const void* w_gate, const void* w_up, const void* w_down, int64_t n_expert,
                  int64_t hidden, int64_t inter, ft_type act, const float* x, int64_t t,
                  const int32_t* expert_ids, const float* expert_w, int topk, float* y, const ft_moe_opts& o,
                  bool tiles, uint8_t* b, hipStream_t st) {
  const MoeScratch L = moe_layout(w, act, hidden, inter, t, topk);
  const SortScratch S = sort_layout(n_expert, t, topk, moe_xf8_bytes(w, hidden, inter, t, topk));
  MoeArgs a = {};
  a.w = w;
  a.act = act;
  a.w_gate = w_gate;
  a.w_up = w_up;
  a.w_down = w_down;
  a.n_expert = n_expert;
  a.hidden = hidden;
  a.inter = inter;
  a.t = t;
  a.topk = topk;
  a.ids = expert_ids;
  a.ew = expert_w;
  a.x = x;
  a.xq = b + L.xq;
  a.h = o.tap_h ? o.tap_h : (float*)(b + L.h);
  a.g_tap = o.tap_g;
  a.u_tap = o.tap_u;
  a.hq = o.in_hq ? const_cast<void*>(o.in_hq) : (o.tap_hq ? o.tap_hq : (void*)(b + L.hq));
  a.hq_tap = o.tap_hq;
  a.in_hq = o.in_hq;
  a.dpair = o.tap_down ? o.tap_down : (float*)(b + L.d);
  a.d_tap = o.tap_down;
  a.h_tap = o.tap_h;
  a.y = y;

  hipError_t e = hipSuccess;
  a.logits = nullptr;
  a.ids_out = o.ids_out;
  a.w_out = o.w_out;
  const bool fused = !tiles && ftk_moe_fused_ok(w, act, hidden, inter, topk);
  if (o.logits && fused && ftk_moe_fused_routes(n_expert)) {
    a.logits = o.logits;   // the fused layer routes itself
    a.ids = nullptr;
    a.ew = nullptr;
  } else if (o.logits && !tiles && w == FT_MXFP4 && act == FT_Q8_K && n_expert <= 256 && t <= 2) {
    // the MXFP4 direct gate/up launch routes the tokens itself (the router's
    // selection and weights) and leaves the routing here for the later stages
    // (1-2 tokens: 1.2-1.5 us less per layer; from 4 tokens on, every workgroup
    // routing its chunk costs more than the router's launch)
    a.logits = o.logits;
    a.ids = o.ids_out ? o.ids_out : (int32_t*)(b + L.ids);
    a.ew = o.w_out ? o.w_out : (float*)(b + L.w);
    expert_ids = a.ids;
  } else if (o.logits) {   // route first, into the caller's outputs or scratch
    int32_t* ri = o.ids_out ? o.ids_out : (int32_t*)(b + L.ids);
    float* rw = o.w_out ? o.w_out : (float*)(b + L.w);
    e = ftk_launch_route(o.logits, t, n_expert, topk, ri, rw, st);
    if (e != hipSuccess) return FT_ERR_HIP;
    a.ids = ri;
    a.ew = rw;
    expert_ids = ri;
  }
  if (tiles) {
    e = ftk_launch_quantize(act, x, t, hidden, hidden, (void*)a.xq, st);
    uint8_t* sb = b + L.total;
    int32_t* counts = (int32_t*)(sb + S.counts);
    int32_t* offsets = (int32_t*)(sb + S.offsets);
    int32_t* pairs = (int32_t*)(sb + S.pairs);
    void* xf8 = sb + S.xf8;
    if (e == hipSuccess) e = ftk_launch_sort(expert_ids, t, topk, n_expert, counts, offsets, pairs, st);
    if (e == hipSuccess && w == FT_MXFP4) e = ftk_launch_fp8_split(a.xq, t, hidden, xf8, st);
    GroupedArgs gu = {};
    gu.w = w;
    gu.act = act;
    gu.W = w_gate;
    gu.W2 = w_up;
    gu.g_tap = o.tap_g;
    gu.u_tap = o.tap_u;
    gu.n_expert = n_expert;
    gu.n = inter;
    gu.k = hidden;
    gu.xq = a.xq;
    gu.xf8 = w == FT_MXFP4 ? xf8 : nullptr;
    gu.x_per_pair = 0;
    gu.t = t;
    gu.topk = topk;
    gu.counts = counts;
    gu.offsets = offsets;
    gu.pairs = pairs;
    gu.y = a.h;
    if (e == hipSuccess) e = ftk_launch_grouped(gu, st);
    if (e == hipSuccess && !o.in_hq) e = ftk_launch_quantize(act, a.h, t * topk, inter, inter, a.hq, st);
    if (e == hipSuccess && o.in_hq && o.tap_hq)
      e = hipMemcpyAsync(o.tap_hq, o.in_hq, (size_t)t * topk * row_bytes_of(act, inter), hipMemcpyDeviceToDevice,
                         st);
    if (e == hipSuccess && w == FT_MXFP4) e = ftk_launch_fp8_split(a.hq, t * topk, inter, xf8, st);
    GroupedArgs dn = gu;
    dn.W = w_down;
    dn.W2 = nullptr;
    dn.g_tap = dn.u_tap = nullptr;
    dn.n = hidden;
    dn.k = inter;
    dn.xq = a.hq;
    dn.xf8 = w == FT_MXFP4 ? xf8 : nullptr;
    dn.x_per_pair = 1;
    dn.y = a.dpair;
    if (e == hipSuccess) e = ftk_launch_grouped(dn, st);
    if (e == hipSuccess) e = ftk_launch_moe_combine(a, st);
    return hip_status(e);
  }
  // direct route, Q4_K x Q8_1 shapes that fit: the whole layer in two launches per 4-token chunk
  if (fused) return hip_status(ftk_launch_moe_fused(a, b + L.tab, st));
  // otherwise gate/up (quantizes x itself), down (quantizes each expert's h rows
  // itself, or reads in_hq), slot-order combine
  e = ftk_launch_moe_gate_up(a, st);
  if (e == hipSuccess && w == FT_MXFP4 && ftk_moe_fp4_down_combine_ok(a))
    return hip_status(ftk_launch_moe_fp4_down_combine(a, st));   // 1-2 tokens: down + combine
  if (e == hipSuccess) e = ftk_launch_moe_down(a, st);
  if (e == hipSuccess) e = ftk_launch_moe_combine(a, st);
  return hip_status(e);
}

// --------------------------------------------------------------------------
// fixed scratch of ft_moe_q_vec_noalloc: a device array of every GPU the library
// runs on, held until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is a stand-in, not a device address): the address
// comes from hipGetSymbolAddress once per device and is kept here.
// --------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[FT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};

ft_status static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FT_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FT_ERR_HIP;
    g_static_ptr[dev] = p;
  }
  *out = g_static_ptr[dev];
  return FT_OK;
}

}  // namespace

extern "C" {

ft_status ft_moe_q_vec(ft_type w, const void* w_gate, const void* w_up, const void* w_down, int64_t n_expert,
                       int64_t hidden, int64_t inter, ft_type act, const float* x, int64_t t,
                       const int32_t* expert_ids, const float* expert_w, int topk, float* y, const ft_moe_opts* opts,
                       ft_stream_t stream) {
  ft_moe_opts o = {};
  if (opts) o = *opts;
  bool tiles = false;
  size_t need = 0;
  ft_status s = moe_check(w, w_gate, w_up, w_down, n_expert, hidden, inter, act, x, t, expert_ids, expert_w, topk,
                          y, o, &tiles, &need);
  if (s != FT_OK || t == 0) return s;
  hipStream_t st = hs(stream);
  void* base = nullptr;
  s = pool_get(st, need, &base);
  if (s != FT_OK) return s;
  return moe_run(w, w_gate, w_up, w_down, n_expert, hidden, inter, act, x, t, expert_ids, expert_w, topk, y, o,
                 tiles, (uint8_t*)base, st);
}

ft_status ft_moe_q_vec_noalloc(ft_type w, const void* w_gate, const void* w_up, const void* w_down,
                               int64_t n_expert, int64_t hidden, int64_t inter, ft_type act, const float* x,
                               int64_t t, const int32_t* expert_ids, const float* expert_w, int topk, float* y,
                               const ft_moe_opts* opts, ft_stream_t stream) {
  ft_moe_opts o = {};
  if (opts) o = *opts;
  bool tiles = false;
  size_t need = 0;
  ft_status s = moe_check(w, w_gate, w_up, w_down, n_expert, hidden, inter, act, x, t, expert_ids, expert_w, topk,
                          y, o, &tiles, &need);
  if (s != FT_OK || t == 0) return s;
  if (need > (size_t)FT_NOALLOC_SCRATCH_BYTES) return FT_ERR_SHAPE;
  void* base = nullptr;
  s = static_scratch(&base);
  if (s != FT_OK) return s;
  return moe_run(w, w_gate, w_up, w_down, n_expert, hidden, inter, act, x, t, expert_ids, expert_w, topk, y, o,
                 tiles, (uint8_t*)base, hs(stream));
}

ft_status ft_grouped_gemm_q(ft_type w, const void* W, int64_t n_expert, int64_t n, int64_t k, ft_type act,
                            const void* xq, int x_per_pair, const int32_t* expert_ids, int64_t t, int topk, float* y,
                            ft_stream_t stream) {
  if (!is_weight(w) || !is_act(act) || !grouped_pair(w, act)) return FT_ERR_UNSUPPORTED;
  if (n_expert < 1 || n < 0 || k < 0 || t < 0) return FT_ERR_INVALID_ARG;
  if (topk < 1 || topk > 8 || topk > n_expert || n_expert > 8192) return FT_ERR_SHAPE;
  if (k % kElems[w] || k % kElems[act] || k == 0 || k > 16384) return FT_ERR_SHAPE;
  if (n == 0 || t == 0) return FT_OK;
  if (!W || !xq || !expert_ids || !y) return FT_ERR_INVALID_ARG;
  if (!aligned16(W) || !aligned16(xq) || !aligned16(y)) return FT_ERR_ALIGNMENT;
  hipStream_t st = hs(stream);
  const SortScratch L = sort_layout(n_expert, t, topk, xf8_bytes_of(w, x_per_pair ? t * topk : t, k));
  void* base = nullptr;
  ft_status s = pool_get(st, L.total, &base);
  if (s != FT_OK) return s;
  uint8_t* b = (uint8_t*)base;
  GroupedArgs a = {};
  a.w = w;
  a.act = act;
  a.W = W;
  a.n_expert = n_expert;
  a.n = n;
  a.k = k;
  a.xq = xq;
  a.x_per_pair = x_per_pair ? 1 : 0;
  a.t = t;
  a.topk = topk;
  a.counts = (const int32_t*)(b + L.counts);
  a.offsets = (const int32_t*)(b + L.offsets);
  a.pairs = (const int32_t*)(b + L.pairs);
  a.y = y;
  a.xf8 = w == FT_MXFP4 ? (const void*)(b + L.xf8) : nullptr;
  hipError_t e = ftk_launch_sort(expert_ids, t, topk, n_expert, (int32_t*)(b + L.counts), (int32_t*)(b + L.offsets),
                                 (int32_t*)(b + L.pairs), st);
  if (e == hipSuccess && w == FT_MXFP4) e = ftk_launch_fp8_split(xq, x_per_pair ? t * topk : t, k, b + L.xf8, st);
  if (e == hipSuccess) e = ftk_launch_grouped(a, st);
  return hip_status(e);
}

ft_status ft_debug_block_dots(ft_type w, const void* W, int64_t n, int64_t k, ft_type act, const void* xq, int64_t t,
                              int32_t* partials, ft_stream_t stream) {
  if (!is_weight(w) || !is_act(act)) return FT_ERR_UNSUPPORTED;
  if (n < 0 || k < 0 || t < 0) return FT_ERR_INVALID_ARG;
  if (k % kElems[w] || k % kElems[act]) return FT_ERR_SHAPE;
  if (n == 0 || t == 0 || k == 0) return FT_OK;
  if (!W || !xq || !partials) return FT_ERR_INVALID_ARG;
  if (!aligned16(W) || !aligned16(xq)) return FT_ERR_ALIGNMENT;
  if (act == FT_Q8_0) {   // as the matvec: the Q8_1 layout of the same blocks
    void* rp = nullptr;
    const int64_t nblk = t * (k / 32);
    const ft_status ps = pool_get(hs(stream), align256((size_t)nblk * 36), &rp);
    if (ps != FT_OK) return ps;
    const hipError_t e = ftk_launch_repack_q8_0(xq, nblk, rp, hs(stream));
    if (e != hipSuccess) return FT_ERR_HIP;
    xq = rp;
    act = FT_Q8_1;
  }
  return hip_status(ftk_launch_block_dots(w, W, n, k, act, xq, t, partials, hs(stream)));
}

ft_status ft_debug_ceiling(int which, const void* buf, int64_t bytes, int64_t iters, void* out,
                           ft_stream_t stream) {
  if (which < 0 || which > 3 || !out || iters < 0) return FT_ERR_INVALID_ARG;
  if (which == 0) {
    if (!buf || bytes < 0 || bytes % 16) return FT_ERR_INVALID_ARG;
    if (!aligned16(buf)) return FT_ERR_ALIGNMENT;
    if (bytes == 0) return FT_OK;
  }
  return hip_status(ftk_launch_probe(which, buf, bytes, iters, (uint32_t*)out, hs(stream)));
}

ft_status ft_scratch_reserve(ft_stream_t stream, size_t bytes) {
  void* p = nullptr;
  return pool_get(hs(stream), bytes, &p);
}

void ft_shutdown(void) {
  std::lock_guard<std::mutex> lk(g_pool_mu);
  for (auto& kv : g_pools) {
    if (kv.second.ptr) (void)hipFree(kv.second.ptr);
    for (void* r : kv.second.retired) (void)hipFree(r);
  }
  g_pools.clear();
}

}  // extern "C"

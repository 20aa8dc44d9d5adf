// ft_moe.hip -- routed-MoE vector path: router, token->expert sort, the slot-order
// combine, and the direct-route dot4 expert kernels (gate/up + SwiGLU, down) used
// for Q4_K x Q8_1 (MXFP4 x Q8_K has its own, on the FP4 MFMA: ft_moe_fp4.hip).
//
// ds4 PR #656 "Add ROCm MXFP4 routed expert kernels" (Summary): routed gate/up and
// down kernels with SwiGLU between them, coalesced weight reads with register
// unpack, and tiny batches sent through direct kernels instead of partly filled
// expert-sorted tiles.  FreeToken PR #136 (Summary): the routed MoE vector kernel.
// MI355X design:
//  * one workgroup per (distinct selected expert, share of its output rows); the
//    share is streamed through LDS in tiles of whole rows with 16-byte loads (the
//    next tile into VGPRs while the current one is computed) and applied to every
//    token that selected the expert (duplicates across tokens are read once; the
//    first slot naming an expert owns it);
//  * the chunk's expert ids are read once, one pair per lane, and the ownership
//    and token masks come from ballots;
//  * each workgroup quantizes the activation rows it needs itself, with all loads
//    of a batch in flight before any block is reduced;
//  * activation codes of all tokens sit in VGPRs; a wave-uniform token mask skips
//    tokens that did not pick the expert;
//  * gate and up share the activations; SwiGLU is applied right after the 64-lane
//    reduction, before h leaves registers.
#include <stdlib.h>

#include <string.h>

#include "ft_device.h"
#include "ft_internal.h"

namespace ftk {

constexpr int MOE_THREADS = 256;

// ---------------------------------------------------------------------------
// router: one wave per token (route_token, ft_device.h)
// ---------------------------------------------------------------------------
template <int MAXE>   // logits per lane (n_expert <= 64 * MAXE)
__global__ void __launch_bounds__(256)
route_kernel(const float* __restrict__ logits, int64_t t, int n_expert, int topk, int32_t* __restrict__ ids,
             float* __restrict__ w) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + wave;
  if (tok >= t) return;
  route_token<MAXE>(logits + tok * n_expert, n_expert, topk, lane, ids + tok * topk, w + tok * topk);
}

// ---------------------------------------------------------------------------
// stable counting sort of (token, slot) pairs by expert: one workgroup of 1024
//  1. histogram of all pairs (LDS atomics) and a block-wide exclusive scan ->
//     offsets; counts[] serves as the per-expert insert cursor until the end;
//  2. pairs are taken in chunks of at most `chunk` in pair order; a chunk is
//     histogrammed again (two 16-bit counters per LDS word), scanned, and its pairs
//     dropped into their expert's segment of an LDS list with atomics (any order);
//     each pair then counts the smaller pair indices in its own segment, which is
//     its stable rank, and lands at cursor[e] + rank;
//  3. counts[] = offsets[e+1] - offsets[e].
// Work per pair is O(its expert's share of the chunk); LDS use is
// 4*E + 4*chunk bytes.
// ---------------------------------------------------------------------------
constexpr int SORT_THREADS = 1024;

__device__ __forceinline__ int clamp_e(int e, int n_expert) {
  return e < 0 ? 0 : (e >= n_expert ? n_expert - 1 : e);
}

// Exclusive scan over n values get(i) in index order; put(i, prefix) for each i.
// Returns the total in every thread.  Needs wsum[SORT_THREADS / 64 + 1] in LDS.
template <typename G, typename P>
__device__ __forceinline__ int block_exclusive_scan(int n, int* wsum, G get, P put) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  constexpr int NW = SORT_THREADS / 64;
  const int per = (n + SORT_THREADS - 1) / SORT_THREADS;
  const int i0 = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (i0 + i < n) local += get(i0 + i);
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int v = lane < NW ? wsum[lane] : 0;
    int sc = v;
#pragma unroll
    for (int d = 1; d < NW; d <<= 1) {
      const int u = __shfl_up(sc, d, 64);
      if (lane >= d) sc += u;
    }
    if (lane < NW) wsum[lane] = sc - v;
    if (lane == NW - 1) wsum[NW] = sc;
  }
  __syncthreads();
  int run = wsum[wave] + incl - local;
  for (int i = 0; i < per; ++i)
    if (i0 + i < n) {
      const int c = get(i0 + i);
      put(i0 + i, run);
      run += c;
    }
  const int total = wsum[NW];
  __syncthreads();
  return total;
}

__global__ void __launch_bounds__(SORT_THREADS)
sort_kernel(const int32_t* __restrict__ ids, int npairs, int n_expert, int chunk, int32_t* __restrict__ counts,
            int32_t* __restrict__ offsets, int32_t* __restrict__ pairs) {
  extern __shared__ int32_t sh[];
  __shared__ int wsum[SORT_THREADS / 64 + 1];
  const int tid = threadIdx.x;
  const int E = n_expert;

  // 1. global histogram and offsets
  int32_t* hist = sh;   // [E]
  for (int e = tid; e < E; e += SORT_THREADS) hist[e] = 0;
  __syncthreads();
  for (int p = tid; p < npairs; p += SORT_THREADS) atomicAdd(&hist[clamp_e(ids[p], E)], 1);
  __syncthreads();
  const int total = block_exclusive_scan(
      E, wsum, [&](int e) { return hist[e]; },
      [&](int e, int v) {
        offsets[e] = v;
        counts[e] = v;   // insert cursor
      });
  if (tid == 0) offsets[E] = total;

  // 2. chunks in pair order
  uint32_t* lc = (uint32_t*)sh;                 // [(E+1)/2] packed 16-bit counts, then cursors
  uint16_t* lo = (uint16_t*)(lc + (E + 1) / 2);  // [E+1] chunk-local offsets
  int32_t* lst = (int32_t*)(lc + (E + 1) / 2 + (E + 2) / 2);  // [chunk]
  for (int c0 = 0; c0 < npairs; c0 += chunk) {
    const int cn = min(chunk, npairs - c0);
    for (int i = tid; i < (E + 1) / 2; i += SORT_THREADS) lc[i] = 0;
    __syncthreads();
    for (int p = c0 + tid; p < c0 + cn; p += SORT_THREADS) {
      const int e = clamp_e(ids[p], E);
      atomicAdd(&lc[e >> 1], 1u << (16 * (e & 1)));
    }
    __syncthreads();
    block_exclusive_scan(
        E, wsum, [&](int e) { return (int)((lc[e >> 1] >> (16 * (e & 1))) & 0xFFFFu); },
        [&](int e, int v) { lo[e] = (uint16_t)v; });
    if (tid == 0) lo[E] = (uint16_t)cn;
    __syncthreads();
    // cursors start at the chunk-local offsets (each thread rewrites whole words)
    for (int i = tid; i < (E + 1) / 2; i += SORT_THREADS) {
      const uint32_t a = lo[2 * i], b = 2 * i + 1 < E ? lo[2 * i + 1] : 0u;
      lc[i] = a | (b << 16);
    }
    __syncthreads();
    for (int p = c0 + tid; p < c0 + cn; p += SORT_THREADS) {
      const int e = clamp_e(ids[p], E);
      const uint32_t old = atomicAdd(&lc[e >> 1], 1u << (16 * (e & 1)));
      lst[(old >> (16 * (e & 1))) & 0xFFFFu] = p;
    }
    __syncthreads();
    for (int s = tid; s < cn; s += SORT_THREADS) {
      const int p = lst[s];
      const int e = clamp_e(ids[p], E);
      const int b0 = lo[e], b1 = lo[e + 1];
      int rank = 0;
      for (int s2 = b0; s2 < b1; ++s2) rank += lst[s2] < p;
      pairs[counts[e] + rank] = p;
    }
    __syncthreads();
    for (int e = tid; e < E; e += SORT_THREADS) counts[e] += lo[e + 1] - lo[e];
    __syncthreads();
  }

  // 3. counts
  __syncthreads();
  for (int e = tid; e < E; e += SORT_THREADS) counts[e] = offsets[e + 1] - offsets[e];
}

// The same stable sort for at most 16384 pairs and 512 experts, without the
// per-pair count over its segment.  Wave w owns the consecutive pairs
// [w * per, (w + 1) * per), 64 per round in pair order.  In a round the lanes that
// hold the same expert find each other with one ballot per bit of the expert
// index; a pair's rank among its wave's earlier pairs of that expert is the
// wave's running count for it (one LDS row of E counters per wave) plus the
// group's lanes below it, and the group's highest lane advances the count (the
// wave's LDS read precedes its write).  Then each expert's per-wave counts become
// starts in wave order, the totals are scanned into the offsets, and every pair
// lands at offsets[e] + its wave's start + its rank.
constexpr int SORTF_MAXE = 512;
constexpr int SORTF_MAXR = 16;   // rounds per wave: 16 waves x 64 lanes x 16 = 16384 pairs

__global__ void __launch_bounds__(SORT_THREADS)
sort_fast_kernel(const int32_t* __restrict__ ids, int npairs, int n_expert, int nbits, int per,
                 int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ pairs) {
  constexpr int NW = SORT_THREADS / 64;
  __shared__ int32_t cnt[NW * SORTF_MAXE];
  __shared__ int32_t base[SORTF_MAXE];
  __shared__ int wsum[NW + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int E = n_expert;
  int32_t* my = cnt + wave * E;
  for (int e = lane; e < E; e += 64) my[e] = 0;
  __builtin_amdgcn_wave_barrier();
  const int p0 = wave * per;
  const uint64_t below = (1ull << lane) - 1ull;
  int er[SORTF_MAXR], rk[SORTF_MAXR];
#pragma unroll
  for (int r = 0; r < SORTF_MAXR; ++r) {
    er[r] = -1;
    rk[r] = 0;
    if (r * 64 < per) {
      const int p = p0 + r * 64 + lane;
      const bool v = p < npairs;
      const int e = v ? clamp_e(ids[p], E) : 0;
      uint64_t m = __ballot(v);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(v && bit);
        m &= bit ? bb : ~bb;
      }
      if (v) {
        const int prev = my[e];
        er[r] = e;
        rk[r] = prev + __popcll(m & below);
        if ((m >> lane) == 1ull) my[e] = prev + __popcll(m);   // highest lane of the group
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += SORT_THREADS) {
    int run = 0;
    for (int w = 0; w < NW; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += c;
    }
    base[e] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan(
      E, wsum, [&](int e) { return base[e]; },
      [&](int e, int v) {
        counts[e] = base[e];
        offsets[e] = v;
        base[e] = v;
      });
  if (tid == 0) offsets[E] = total;
#pragma unroll
  for (int r = 0; r < SORTF_MAXR; ++r) {
    if (er[r] >= 0) {
      const int d = base[er[r]] + cnt[wave * E + er[r]] + rk[r];
      if (d < npairs) pairs[d] = p0 + r * 64 + lane;
    }
  }
}

// ---------------------------------------------------------------------------
// helpers shared by the expert kernels
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Direct-route expert kernels.  Each workgroup streams whole weight rows through
// LDS in tiles: tile i+1 is fetched into VGPRs with 16-byte loads while tile i is
// computed from LDS (as the matvec does).  The activation rows a workgroup needs
// are quantized by the workgroup itself into LDS first (x for gate/up, the
// selected experts' h rows for down), with the arithmetic of ft_quantize_act.
// ---------------------------------------------------------------------------
template <int CPL>
struct TileFetch {
  u32x4 pre[CPL];
  int nch;
  __device__ __forceinline__ uint32_t fetch(const uint8_t* src, int64_t nbytes, int tid) {
    const uintptr_t a = (uintptr_t)src;
    const uint32_t shift = (uint32_t)(a & 15);
    nch = (int)((shift + nbytes + 15) >> 4);
    const u32x4* s4 = (const u32x4*)(src - shift);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = i * MOE_THREADS + tid;
      if (c < nch) pre[i] = __builtin_nontemporal_load(s4 + c);
    }
    return shift;
  }
  __device__ __forceinline__ void commit(u32x4* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = i * MOE_THREADS + tid;
      if (c < nch) dst[c] = pre[i];
    }
  }
};

// Quantize `rows` fp32 rows of k elements with the whole workgroup: src(r) is row
// r's data (16-byte aligned), dst(r) its first activation block.  A thread takes 8
// (Q8_1) or 16 (Q8_K) consecutive elements, so a block is 4 or 16 aligned lanes;
// the loads of up to 32 elements per thread are all issued before any block is
// reduced, so a workgroup pays one memory latency per 8192 elements.
template <int A, typename S, typename D>
__device__ __forceinline__ void quantize_rows(int rows, int k, S src, D dst, int tid) {
  constexpr int EPT = A == FT_Q8_1 ? 8 : 16;
  constexpr int BATCH = 32 / EPT;
  const int per_row = k / EPT;
  const int total = rows * per_row;
  for (int base = 0; base < total; base += MOE_THREADS * BATCH) {
    float v[BATCH][EPT];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int idx = base + b * MOE_THREADS + tid;
      if (idx < total) {
        const int r = idx / per_row, c = (idx - r * per_row) * EPT;
        const float4* p = (const float4*)(src(r) + c);
#pragma unroll
        for (int q = 0; q < EPT / 4; ++q) {
          const float4 f = p[q];
          v[b][4 * q] = f.x;
          v[b][4 * q + 1] = f.y;
          v[b][4 * q + 2] = f.z;
          v[b][4 * q + 3] = f.w;
        }
      }
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int idx = base + b * MOE_THREADS + tid;
      if (idx < total) {   // the same for all lanes of a block: k is a whole number of blocks
        const int r = idx / per_row, c = (idx - r * per_row) * EPT;
        uint8_t* ob = dst(r) + (c / Act<A>::BLK) * Act<A>::BB;
        if constexpr (A == FT_Q8_1) q8_1_part(v[b], tid & 3, ob);
        else q8_k_part(v[b], tid & 15, ob);
      }
    }
  }
}

// gate/up + SwiGLU: h[pair][r] = silu(g) * u for the rows of this workgroup's share
template <int F, int A, int T, int LR, int P, int CPL>
__global__ void __launch_bounds__(MOE_THREADS)
moe_gate_up_kernel(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu, int64_t n_expert,
                   int64_t inter, int row_bytes, int units_per_row, int rows_per_wg, int rows_per_tile,
                   const float* __restrict__ x, int64_t hidden, int t_real, const int32_t* __restrict__ ids,
                   int topk, float* __restrict__ h, float* __restrict__ gtap, float* __restrict__ utap) {
  using FT = Fmt<F>;
  constexpr int G = MOE_THREADS / LR;
  constexpr int M = 2 * T;   // g values then u values of one row per group
  static_assert(M <= LR, "");
  extern __shared__ u32x4 smem4[];
  const int tid = threadIdx.x, grp = tid / LR, gl = tid % LR;

  int e;
  uint32_t mask;
  uint64_t smask;
  if (!expert_tokens(ids, blockIdx.y, t_real, topk, n_expert, e, mask, smask)) return;
  const int64_t wr0 = (int64_t)blockIdx.x * rows_per_wg;
  if (wr0 >= inter) return;
  const int wrows = (int)min<int64_t>(rows_per_wg, inter - wr0);
  const int ntiles = (wrows + rows_per_tile - 1) / rows_per_tile;
  const uint8_t* gbase = wg + ((int64_t)e * inter + wr0) * row_bytes;
  const uint8_t* ubase = wu + ((int64_t)e * inter + wr0) * row_bytes;

  u32x4* tg = smem4;
  u32x4* tu = smem4 + CPL * MOE_THREADS + 1;
  uint8_t* xql = (uint8_t*)(smem4 + 2 * (CPL * MOE_THREADS + 1));
  const int xrb = (int)(hidden / Act<A>::BLK * Act<A>::BB);

  TileFetch<CPL> fg, fu;
  auto tile_rows = [&](int tile) { return min(rows_per_tile, wrows - tile * rows_per_tile); };
  uint32_t sg = fg.fetch(gbase, (int64_t)tile_rows(0) * row_bytes, tid);
  uint32_t su = fu.fetch(ubase, (int64_t)tile_rows(0) * row_bytes, tid);

  quantize_rows<A>(
      t_real, (int)hidden, [&](int r) { return x + (int64_t)r * hidden; }, [&](int r) { return xql + r * xrb; }, tid);
  __syncthreads();
  ActUnit<F> act[P][T];
  int ub[P], uu[P];
  bool uv[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int u0 = gl + p * LR;
    uv[p] = u0 < units_per_row;
    const int u = uv[p] ? u0 : 0;
    ub[p] = u / FT::UPB;
    uu[p] = u % FT::UPB;
#pragma unroll
    for (int i = 0; i < T; ++i) {
      if (uv[p] && ((mask >> i) & 1)) load_act_unit<F, A>(xql + i * xrb, ub[p], uu[p], act[p][i]);
      else zero_act_unit<F>(act[p][i]);
    }
  }
  fg.commit(tg, tid);
  fu.commit(tu, tid);
  __syncthreads();

  const Reader<const uint32_t*> rg{(const uint32_t*)tg}, ru{(const uint32_t*)tu};
  for (int tile = 0; tile < ntiles; ++tile) {
    const int nr = tile_rows(tile);
    const uint32_t cg = sg, cu = su;
    if (tile + 1 < ntiles) {
      const int64_t off = (int64_t)(tile + 1) * rows_per_tile * row_bytes;
      sg = fg.fetch(gbase + off, (int64_t)tile_rows(tile + 1) * row_bytes, tid);
      su = fu.fetch(ubase + off, (int64_t)tile_rows(tile + 1) * row_bytes, tid);
    }
    for (int rb = 0; rb < nr; rb += G) {
      float v[M];
#pragma unroll
      for (int i = 0; i < M; ++i) v[i] = 0.0f;
      const int r = rb + grp;
      if (r < nr) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const uint32_t off = (uint32_t)r * row_bytes + (uint32_t)ub[p] * FT::BB;
          Unit<F> ug, uup;
          unpack_unit<F, (F == FT_Q4_K || F == FT_Q5_K)>(rg, cg + off, uu[p], ug);
          unpack_unit<F, (F == FT_Q4_K || F == FT_Q5_K)>(ru, cu + off, uu[p], uup);
#pragma unroll
          for (int i = 0; i < T; ++i) {
            if ((mask >> i) & 1) {
              v[i] = unit_combine<F>(ug, act[p][i], v[i]);
              v[T + i] = unit_combine<F>(uup, act[p][i], v[T + i]);
            }
          }
        }
      }
      group_reduce_multi<M, LR>(v, gl);
      const int idx = gl / (LR / M);
      const bool leader = (gl % (LR / M)) == 0;
      const float other = __shfl_xor(v[0], LR / 2, 64);   // the u value of the same token
      if (leader && idx < T) {
        const int i = idx;
        if (r < nr && ((mask >> i) & 1)) {
          const float g = v[0], u = other, hv = g / (1.0f + expf(-g)) * u;
          const int64_t row = wr0 + (int64_t)tile * rows_per_tile + r;
          for (int k = 0; k < topk; ++k) {   // every slot of token i that names e
            if ((smask >> (8 * i + k)) & 1) {
              const int64_t o = (int64_t)(i * topk + k) * inter + row;
              h[o] = hv;
              if (gtap) gtap[o] = g;
              if (utap) utap[o] = u;
            }
          }
        }
      }
    }
    if (tile + 1 < ntiles) {
      __syncthreads();   // every wave is done reading the tile
      fg.commit(tg, tid);
      fu.commit(tu, tid);
      __syncthreads();
    }
  }
}

// Down projection: d[pair][r] = W_down[e][r] . hhat(pair) for this workgroup's
// share of rows of its expert; hhat of the expert's tokens is quantized here (or
// read from in_hq), and the first workgroup of the slot writes it to hq_tap.
// Slots that repeat an expert within a token share the first slot's h and d.
template <int F, int A, int T, int LR, int P, int CPL>
__global__ void __launch_bounds__(MOE_THREADS)
moe_down_kernel(const uint8_t* __restrict__ wd, int64_t n_expert, int64_t hidden, int row_bytes,
                int units_per_row, int rows_per_wg, int rows_per_tile, const float* __restrict__ h,
                const uint8_t* __restrict__ in_hq, uint8_t* __restrict__ hq_tap, int64_t inter, int t_real,
                const int32_t* __restrict__ ids, int topk, float* __restrict__ dpair) {
  using FT = Fmt<F>;
  constexpr int G = MOE_THREADS / LR;
  constexpr int M = T;
  static_assert(M <= LR, "");
  extern __shared__ u32x4 smem4[];
  const int tid = threadIdx.x, grp = tid / LR, gl = tid % LR;

  int e;
  uint32_t mask;
  uint64_t smask;
  if (!expert_tokens(ids, blockIdx.y, t_real, topk, n_expert, e, mask, smask)) return;
  const int64_t wr0 = (int64_t)blockIdx.x * rows_per_wg;
  if (wr0 >= hidden) return;
  const int wrows = (int)min<int64_t>(rows_per_wg, hidden - wr0);
  const int ntiles = (wrows + rows_per_tile - 1) / rows_per_tile;
  const uint8_t* dbase = wd + ((int64_t)e * hidden + wr0) * row_bytes;

  u32x4* td = smem4;
  uint8_t* hql = (uint8_t*)(smem4 + CPL * MOE_THREADS + 1);
  const int hrb = (int)(inter / Act<A>::BLK * Act<A>::BB);

  TileFetch<CPL> fd;
  auto tile_rows = [&](int tile) { return min(rows_per_tile, wrows - tile * rows_per_tile); };
  uint32_t sd = fd.fetch(dbase, (int64_t)tile_rows(0) * row_bytes, tid);

  // hhat of the expert's tokens (token i -> LDS row i), from the first slot of
  // token i that names e
  const int ntok = __popc(mask);
  auto first_pair = [&](int i) { return i * topk + __ffs((unsigned)(smask >> (8 * i)) & 0xFFu) - 1; };
  if (in_hq) {
    for (int c = tid; c < ntok * (hrb >> 2); c += MOE_THREADS) {
      const int j = c / (hrb >> 2), w = c - j * (hrb >> 2), i = nth_bit(mask, j);
      ((uint32_t*)(hql + i * hrb))[w] = ((const uint32_t*)(in_hq + (int64_t)first_pair(i) * hrb))[w];
    }
  } else {
    quantize_rows<A>(
        ntok, (int)inter, [&](int j) { return h + (int64_t)first_pair(nth_bit(mask, j)) * inter; },
        [&](int j) { return hql + nth_bit(mask, j) * hrb; }, tid);
  }
  __syncthreads();
  if (hq_tap && blockIdx.x == 0) {
    for (int i = 0; i < T; ++i)
      for (int k = 0; k < topk; ++k)
        if ((smask >> (8 * i + k)) & 1)
          for (int c = tid; c < (hrb >> 2); c += MOE_THREADS)
            ((uint32_t*)(hq_tap + (int64_t)(i * topk + k) * hrb))[c] = ((const uint32_t*)(hql + i * hrb))[c];
  }

  ActUnit<F> act[P][T];
  int ub[P], uu[P];
  bool uv[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int u0 = gl + p * LR;
    uv[p] = u0 < units_per_row;
    const int u = uv[p] ? u0 : 0;
    ub[p] = u / FT::UPB;
    uu[p] = u % FT::UPB;
#pragma unroll
    for (int i = 0; i < T; ++i) {
      if (uv[p] && ((mask >> i) & 1)) load_act_unit<F, A>(hql + i * hrb, ub[p], uu[p], act[p][i]);
      else zero_act_unit<F>(act[p][i]);
    }
  }
  fd.commit(td, tid);
  __syncthreads();

  const Reader<const uint32_t*> rd{(const uint32_t*)td};
  for (int tile = 0; tile < ntiles; ++tile) {
    const int nr = tile_rows(tile);
    const uint32_t cd = sd;
    if (tile + 1 < ntiles)
      sd = fd.fetch(dbase + (int64_t)(tile + 1) * rows_per_tile * row_bytes, (int64_t)tile_rows(tile + 1) * row_bytes,
                    tid);
    for (int rb = 0; rb < nr; rb += G) {
      float v[M];
#pragma unroll
      for (int i = 0; i < M; ++i) v[i] = 0.0f;
      const int r = rb + grp;
      if (r < nr) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          Unit<F> un;
          unpack_unit<F, (F == FT_Q4_K || F == FT_Q5_K)>(rd, cd + (uint32_t)r * row_bytes + (uint32_t)ub[p] * FT::BB,
                                                         uu[p], un);
#pragma unroll
          for (int i = 0; i < T; ++i)
            if ((mask >> i) & 1) v[i] = unit_combine<F>(un, act[p][i], v[i]);
        }
      }
      group_reduce_multi<M, LR>(v, gl);
      const int i = gl / (LR / M);
      if ((gl % (LR / M)) == 0 && r < nr && ((mask >> i) & 1)) {
        const int64_t row = wr0 + (int64_t)tile * rows_per_tile + r;
        for (int k = 0; k < topk; ++k)
          if ((smask >> (8 * i + k)) & 1) dpair[(int64_t)(i * topk + k) * hidden + row] = v[0];
      }
    }
    if (tile + 1 < ntiles) {
      __syncthreads();
      fd.commit(td, tid);
      __syncthreads();
    }
  }
}

// y[t][c] = sum_k w[t][k] * d[t*topk+k][c], slot order
__global__ void __launch_bounds__(256)
moe_combine_kernel(const float* __restrict__ d, const float* __restrict__ w, int64_t t, int topk, int64_t hidden,
                   float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= t * hidden) return;
  const int64_t tok = i / hidden, c = i % hidden;
  float s = 0.0f;
  for (int k = 0; k < topk; ++k) s = fmaf(w[tok * topk + k], d[(tok * topk + k) * hidden + c], s);
  y[i] = s;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// The same sums, four consecutive columns per thread with 16-byte loads (hidden a
// multiple of 4): workgroup b takes token b / bpt, columns 1024 * (b % bpt) ..;
// every slot's load is in flight before the first multiply-add, and each column
// is summed in slot order as above, so the results are the same bits.
__global__ void __launch_bounds__(256)
moe_combine4_kernel(const float* __restrict__ d, const float* __restrict__ w, int topk, int64_t hidden, int bpt,
                    float* __restrict__ y) {
  const int64_t tok = blockIdx.x / bpt;
  const int64_t c = ((int64_t)(blockIdx.x % bpt) * 256 + threadIdx.x) * 4;
  if (c >= hidden) return;
  const float* dt = d + tok * topk * hidden + c;
  const float* wt = w + tok * topk;
  f32x4 v[8];
  float wk[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < topk) {
      v[k] = *(const f32x4*)(dt + k * hidden);
      wk[k] = wt[k];
    }
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < topk) {
      s[0] = fmaf(wk[k], v[k][0], s[0]);
      s[1] = fmaf(wk[k], v[k][1], s[1]);
      s[2] = fmaf(wk[k], v[k][2], s[2]);
      s[3] = fmaf(wk[k], v[k][3], s[3]);
    }
  *(f32x4*)(y + tok * hidden + c) = s;
}

// ---------------------------------------------------------------------------
// launch planning: lanes per row / units per lane as for the matvec (LR <= 64),
// tiles of whole rows in 16 KiB, and about two workgroups per CU over all slots,
// each owning an equal share of its expert's rows.
// ---------------------------------------------------------------------------
constexpr int MOE_CPL = 4;
struct MoePlan { int lr, p, rows_per_tile, rows_per_wg, wgs; };

static bool moe_plan(int units_per_row, int row_bytes, int64_t rows, int slots, MoePlan& pl) {
  if (units_per_row <= 64) {
    pl.p = 1;
    pl.lr = 16;
    while (pl.lr < units_per_row) pl.lr *= 2;
  } else {
    pl.lr = 64;
    pl.p = 1;
    while (pl.p * 64 < units_per_row) pl.p *= 2;
  }
  if (pl.p > 8) return false;
  pl.rows_per_tile = (MOE_CPL * 4096 - 15) / row_bytes;
  if (pl.rows_per_tile < 1) return false;
  const int wpc = 2;
  const int64_t target = (int64_t)wpc * ftk_num_cus();
  int64_t x = (target + slots - 1) / slots;
  if (x < 1) x = 1;
  int64_t rpw = (rows + x - 1) / x;
  if (rpw < 1) rpw = 1;
  pl.rows_per_wg = (int)rpw;
  pl.wgs = (int)((rows + rpw - 1) / rpw);
  return true;
}

template <int F, int A, int T, int LR, int P>
static hipError_t launch_gate_up_t(const MoeArgs& a, const MoePlan& pl, int row_bytes, int units, int chunk0,
                                   int tchunk, hipStream_t st) {
  const int xrb = (int)(a.hidden / Act<A>::BLK * Act<A>::BB);
  const size_t lds = 2 * (size_t)(MOE_CPL * MOE_THREADS + 1) * 16 + (size_t)T * xrb;
  const dim3 grid((unsigned)pl.wgs, (unsigned)(tchunk * a.topk));
  hipLaunchKernelGGL((moe_gate_up_kernel<F, A, T, LR, P, MOE_CPL>), grid, dim3(MOE_THREADS), lds, st,
                     (const uint8_t*)a.w_gate, (const uint8_t*)a.w_up, a.n_expert, a.inter, row_bytes, units,
                     pl.rows_per_wg, pl.rows_per_tile, a.x + (size_t)chunk0 * a.hidden, a.hidden, tchunk,
                     a.ids + (size_t)chunk0 * a.topk, a.topk, a.h + (size_t)chunk0 * a.topk * a.inter,
                     a.g_tap ? a.g_tap + (size_t)chunk0 * a.topk * a.inter : nullptr,
                     a.u_tap ? a.u_tap + (size_t)chunk0 * a.topk * a.inter : nullptr);
  return hipGetLastError();
}

template <int F, int A, int T, int LR, int P>
static hipError_t launch_down_t(const MoeArgs& a, const MoePlan& pl, int row_bytes, int units, int chunk0,
                                int tchunk, hipStream_t st) {
  const int hrb = (int)(a.inter / Act<A>::BLK * Act<A>::BB);
  const size_t lds = (size_t)(MOE_CPL * MOE_THREADS + 1) * 16 + (size_t)T * hrb;
  const dim3 grid((unsigned)pl.wgs, (unsigned)(tchunk * a.topk));
  // pair indices inside the chunk are relative to the chunk's first pair
  const size_t p0 = (size_t)chunk0 * a.topk;
  hipLaunchKernelGGL((moe_down_kernel<F, A, T, LR, P, MOE_CPL>), grid, dim3(MOE_THREADS), lds, st,
                     (const uint8_t*)a.w_down, a.n_expert, a.hidden, row_bytes, units, pl.rows_per_wg,
                     pl.rows_per_tile, a.h + p0 * a.inter, a.in_hq ? (const uint8_t*)a.in_hq + p0 * hrb : nullptr,
                     a.hq_tap ? (uint8_t*)a.hq_tap + p0 * hrb : nullptr, a.inter, tchunk, a.ids + p0,
                     a.topk, a.dpair + p0 * a.hidden);
  return hipGetLastError();
}

template <int F, int A, int T>
static hipError_t gate_up_lp(const MoeArgs& a, const MoePlan& pl, int rb, int units, int c0, int tc,
                             hipStream_t st) {
#define FT_GU(LRV, PV) \
  if (pl.lr == LRV && pl.p == PV) return launch_gate_up_t<F, A, T, LRV, PV>(a, pl, rb, units, c0, tc, st);
  if constexpr (2 * T <= 16) { FT_GU(16, 1) }
  FT_GU(32, 1) FT_GU(64, 1) FT_GU(64, 2) FT_GU(64, 4)
  if constexpr (T <= 2) { FT_GU(64, 8) }
#undef FT_GU
  return hipErrorInvalidValue;
}

template <int F, int A, int T>
static hipError_t down_lp(const MoeArgs& a, const MoePlan& pl, int rb, int units, int c0, int tc, hipStream_t st) {
#define FT_DN(LRV, PV) \
  if (pl.lr == LRV && pl.p == PV) return launch_down_t<F, A, T, LRV, PV>(a, pl, rb, units, c0, tc, st);
  FT_DN(16, 1) FT_DN(32, 1) FT_DN(64, 1) FT_DN(64, 2) FT_DN(64, 4)
  if constexpr (T <= 2) { FT_DN(64, 8) }
#undef FT_DN
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Direct-route expert kernels on per-wave LDS-DMA rings (rows of at most 64
// units).  As in the dense 1-2 token matvec, every wave streams its own rows
// through an S-stage ring with global_load_lds_dwordx4 and waits only on its own
// vmcnt; the one workgroup barrier follows the activation quantize prologue.  A
// stage holds a group of G = 64 / LR consecutive rows of one matrix (LR lanes per
// row: lane = (row in group, unit)), so that short rows still fill the wave; the
// gate/up kernel streams a group's gate rows and then its up rows, and the SwiGLU
// pair meets in one reduction.  Groups are dealt to the slot's waves in turn
// (group_stride > 1) or in contiguous shares.  Every tile is CPW loads per lane
// (chunks past the group re-read its last chunk; tiles past the share re-read the
// share's first chunk), so the vmcnt arithmetic of wait_tiles holds.
// ---------------------------------------------------------------------------
struct RingShare {
  int64_t g0;   // first group of the wave
  int ng;       // groups of the wave
};
__device__ __forceinline__ RingShare ring_share(int64_t ngroups, int groups_per_wave, int64_t group_stride,
                                                int wave) {
  const int64_t gw = (int64_t)blockIdx.x * (MOE_THREADS / 64) + wave;
  RingShare r;
  r.g0 = group_stride == 1 ? gw * groups_per_wave : gw;
  r.ng = r.g0 >= ngroups ? 0
         : group_stride == 1 ? (int)min<int64_t>(groups_per_wave, ngroups - r.g0)
                             : (int)((ngroups - r.g0 + group_stride - 1) / group_stride);
  return r;
}

// NM matrices of one expert (gate and up, or down) streamed group by group: tile j
// is group j / NM of the share in matrix j % NM.
template <int F, int NM, int S>
struct ExpertRing {
  static constexpr int CPW = SegGeo<F>::CPW;
  static constexpr int SB = CPW * 1024;
  const uint8_t* mat[NM];   // the expert's matrices
  uint8_t* ring;
  int64_t rows, row_bytes, gbytes, gstep;   // end row of the expert in the bank, bytes per row / group / step
  int64_t first_a0;
  int ntiles, issued = 0, is_mat = 0, is_stage = 0, c_nch = -1, lane;
  int64_t is_off, is_row;                   // the next tile's group: byte offset and first row
  uint32_t c_off[CPW];
  __device__ __forceinline__ void issue_next() {
    const bool real = issued < ntiles;
    const int64_t a0 = real ? is_off & ~(int64_t)15 : first_a0;
    const int64_t nb = min<int64_t>(gbytes, (rows - is_row) * row_bytes);
    const int nch = real ? (int)(((is_off & 15) + nb + 15) >> 4) : 1;
    if (nch != c_nch) {   // uniform; whole groups of 16-byte rows keep one count
      c_nch = nch;
#pragma unroll
      for (int i = 0; i < CPW; ++i) c_off[i] = 16u * (uint32_t)min(lane + 64 * i, nch - 1);
    }
    const uint8_t* src = mat[NM == 1 ? 0 : is_mat] + a0;
    uint8_t* dst = ring + is_stage * SB;
#pragma unroll
    for (int i = 0; i < CPW; ++i) lds_dma16(src + c_off[i], dst + 1024 * i);
    ++issued;
    is_stage = is_stage + 1 == S ? 0 : is_stage + 1;
    if (++is_mat == NM) {
      is_mat = 0;
      is_off += gstep;
      is_row += gstep / row_bytes;
    }
  }
};

// gate/up + SwiGLU on the ring: h[pair][r] = silu(g) * u
template <int F, int A, int T, int LR, int S>
__global__ void __launch_bounds__(MOE_THREADS)
moe_ring_gate_up_kernel(const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu, int64_t n_expert,
                        int64_t inter, int row_bytes, int units_per_row, int groups_per_wave, int64_t group_stride,
                        const float* __restrict__ x, int64_t hidden, int t_real, const int32_t* __restrict__ ids,
                        int topk, float* __restrict__ h, float* __restrict__ gtap, float* __restrict__ utap) {
  using FT = Fmt<F>;
  using RG = ExpertRing<F, 2, S>;
  constexpr int G = 64 / LR;   // rows per group
  constexpr int M = 2 * T;     // g values then u values of one row per lane group
  static_assert(M <= LR, "");
  extern __shared__ u32x4 smem4[];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int xrb = (int)(hidden / Act<A>::BLK * Act<A>::BB);
  uint8_t* xql = (uint8_t*)smem4;
  uint8_t* ring = xql + ((T * xrb + 15) & ~15) + wave * (S * RG::SB + 16);

  int e;
  uint32_t mask;
  uint64_t smask;
  if (!expert_tokens(ids, blockIdx.y, t_real, topk, n_expert, e, mask, smask)) return;
  const int64_t ngroups = (inter + G - 1) / G;
  const RingShare sh = ring_share(ngroups, groups_per_wave, group_stride, wave);
  // offsets from the 16-byte aligned bank bases, so that a0 is an aligned address
  const int64_t ebase = (int64_t)e * inter * row_bytes;
  RG rg;
  rg.mat[0] = wg;
  rg.mat[1] = wu;
  rg.ring = ring;
  rg.rows = (int64_t)(e + 1) * inter;
  rg.row_bytes = row_bytes;
  rg.gbytes = (int64_t)G * row_bytes;
  rg.gstep = group_stride * rg.gbytes;
  rg.is_off = ebase + sh.g0 * rg.gbytes;
  rg.is_row = (int64_t)e * inter + sh.g0 * G;
  rg.first_a0 = rg.is_off & ~(int64_t)15;
  rg.ntiles = 2 * sh.ng;
  rg.lane = lane;
  if (sh.ng > 0) {
#pragma unroll
    for (int i = 0; i < S; ++i) rg.issue_next();
  }
  quantize_rows<A>(
      t_real, (int)hidden, [&](int r) { return x + (int64_t)r * hidden; }, [&](int r) { return xql + r * xrb; }, tid);
  lds_barrier();
  if (sh.ng == 0) return;   // whole wave, after the only barrier

  const int gl = lane % LR, rig = lane / LR;   // unit, row in the group
  const bool uv = gl < units_per_row;
  const int u = uv ? gl : 0;
  ActUnit<F> act[T];
#pragma unroll
  for (int i = 0; i < T; ++i) {
    if (uv && ((mask >> i) & 1)) load_act_unit<F, A>(xql + i * xrb, u / FT::UPB, u % FT::UPB, act[i]);
    else zero_act_unit<F>(act[i]);
  }
  const uint32_t lane_off = (uint32_t)(rig * row_bytes + (u / FT::UPB) * FT::BB);

  const Reader<const uint32_t*> rd{(const uint32_t*)ring};
  int cur = 0, cs_stage = 0;
  int64_t cs_off = ebase + sh.g0 * rg.gbytes, cs_row = sh.g0 * G;
  for (int gi = 0; gi < sh.ng; ++gi) {
    float v[M];
#pragma unroll
    for (int i = 0; i < M; ++i) v[i] = 0.0f;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      wait_tiles<RG::CPW, S>(rg.issued - 1 - cur);
      const uint32_t so = (uint32_t)(cs_stage * RG::SB) + (uint32_t)(cs_off & 15) + lane_off;
      Unit<F> un;
      unpack_unit<F, (F == FT_Q4_K || F == FT_Q5_K)>(rd, so, u % FT::UPB, un);
#pragma unroll
      for (int i = 0; i < T; ++i) v[m * T + i] = unit_combine<F>(un, act[i], v[m * T + i]);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0): the stage is read
      rg.issue_next();
      ++cur;
      cs_stage = cs_stage + 1 == S ? 0 : cs_stage + 1;
    }
    group_reduce_multi<M, LR>(v, gl);
    const int idx = gl / (LR / M);
    const bool leader = (gl % (LR / M)) == 0;
    const float other = __shfl_xor(v[0], LR / 2, 64);   // the u value of the same token
    const int64_t row = cs_row + rig;
    if (leader && idx < T && row < inter && ((mask >> idx) & 1)) {
      const float g = v[0], uu = other, hv = g / (1.0f + expf(-g)) * uu;
      for (int k = 0; k < topk; ++k) {   // every slot of token idx that names e
        if ((smask >> (8 * idx + k)) & 1) {
          const int64_t o = (int64_t)(idx * topk + k) * inter + row;
          h[o] = hv;
          if (gtap) gtap[o] = g;
          if (utap) utap[o] = uu;
        }
      }
    }
    cs_off += rg.gstep;
    cs_row += group_stride * G;
  }
}

// down projection on the ring: d[pair][r] = W_down[e][r] . hhat(pair); hhat of the
// expert's tokens is quantized here (or read from in_hq), and the first workgroup
// of the slot writes it to hq_tap
template <int F, int A, int T, int LR, int S>
__global__ void __launch_bounds__(MOE_THREADS)
moe_ring_down_kernel(const uint8_t* __restrict__ wd, int64_t n_expert, int64_t hidden, int row_bytes,
                     int units_per_row, int groups_per_wave, int64_t group_stride, const float* __restrict__ h,
                     const uint8_t* __restrict__ in_hq, uint8_t* __restrict__ hq_tap, int64_t inter, int t_real,
                     const int32_t* __restrict__ ids, int topk, float* __restrict__ dpair) {
  using FT = Fmt<F>;
  using RG = ExpertRing<F, 1, S>;
  constexpr int G = 64 / LR;
  constexpr int M = T;
  static_assert(M <= LR, "");
  extern __shared__ u32x4 smem4[];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int hrb = (int)(inter / Act<A>::BLK * Act<A>::BB);
  uint8_t* hql = (uint8_t*)smem4;
  uint8_t* ring = hql + ((T * hrb + 15) & ~15) + wave * (S * RG::SB + 16);

  int e;
  uint32_t mask;
  uint64_t smask;
  if (!expert_tokens(ids, blockIdx.y, t_real, topk, n_expert, e, mask, smask)) return;
  const int64_t ngroups = (hidden + G - 1) / G;
  const RingShare sh = ring_share(ngroups, groups_per_wave, group_stride, wave);
  const int64_t ebase = (int64_t)e * hidden * row_bytes;   // from the aligned bank base
  RG rg;
  rg.mat[0] = wd;
  rg.ring = ring;
  rg.rows = (int64_t)(e + 1) * hidden;
  rg.row_bytes = row_bytes;
  rg.gbytes = (int64_t)G * row_bytes;
  rg.gstep = group_stride * rg.gbytes;
  rg.is_off = ebase + sh.g0 * rg.gbytes;
  rg.is_row = (int64_t)e * hidden + sh.g0 * G;
  rg.first_a0 = rg.is_off & ~(int64_t)15;
  rg.ntiles = sh.ng;
  rg.lane = lane;
  if (sh.ng > 0) {
#pragma unroll
    for (int i = 0; i < S; ++i) rg.issue_next();
  }
  // hhat of the expert's tokens (token i -> LDS row i), from the first slot of
  // token i that names e
  const int ntok = __popc(mask);
  auto first_pair = [&](int i) { return i * topk + __ffs((unsigned)(smask >> (8 * i)) & 0xFFu) - 1; };
  if (in_hq) {
    for (int c = tid; c < ntok * (hrb >> 2); c += MOE_THREADS) {
      const int j = c / (hrb >> 2), w = c - j * (hrb >> 2), i = nth_bit(mask, j);
      ((uint32_t*)(hql + i * hrb))[w] = ((const uint32_t*)(in_hq + (int64_t)first_pair(i) * hrb))[w];
    }
  } else {
    quantize_rows<A>(
        ntok, (int)inter, [&](int j) { return h + (int64_t)first_pair(nth_bit(mask, j)) * inter; },
        [&](int j) { return hql + nth_bit(mask, j) * hrb; }, tid);
  }
  lds_barrier();
  if (hq_tap && blockIdx.x == 0) {
    for (int i = 0; i < T; ++i)
      for (int k = 0; k < topk; ++k)
        if ((smask >> (8 * i + k)) & 1)
          for (int c = tid; c < (hrb >> 2); c += MOE_THREADS)
            ((uint32_t*)(hq_tap + (int64_t)(i * topk + k) * hrb))[c] = ((const uint32_t*)(hql + i * hrb))[c];
  }
  if (sh.ng == 0) return;   // whole wave, after the only barrier

  const int gl = lane % LR, rig = lane / LR;
  const bool uv = gl < units_per_row;
  const int u = uv ? gl : 0;
  ActUnit<F> act[T];
#pragma unroll
  for (int i = 0; i < T; ++i) {
    if (uv && ((mask >> i) & 1)) load_act_unit<F, A>(hql + i * hrb, u / FT::UPB, u % FT::UPB, act[i]);
    else zero_act_unit<F>(act[i]);
  }
  const uint32_t lane_off = (uint32_t)(rig * row_bytes + (u / FT::UPB) * FT::BB);

  const Reader<const uint32_t*> rd{(const uint32_t*)ring};
  int cur = 0, cs_stage = 0;
  int64_t cs_off = ebase + sh.g0 * rg.gbytes, cs_row = sh.g0 * G;
  for (int gi = 0; gi < sh.ng; ++gi) {
    float v[M];
#pragma unroll
    for (int i = 0; i < M; ++i) v[i] = 0.0f;
    wait_tiles<RG::CPW, S>(rg.issued - 1 - cur);
    const uint32_t so = (uint32_t)(cs_stage * RG::SB) + (uint32_t)(cs_off & 15) + lane_off;
    Unit<F> un;
    unpack_unit<F, (F == FT_Q4_K || F == FT_Q5_K)>(rd, so, u % FT::UPB, un);
#pragma unroll
    for (int i = 0; i < T; ++i) v[i] = unit_combine<F>(un, act[i], v[i]);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0): the stage is read
    rg.issue_next();
    ++cur;
    cs_stage = cs_stage + 1 == S ? 0 : cs_stage + 1;
    group_reduce_multi<M, LR>(v, gl);
    const int idx = gl / (LR / M);
    const int64_t row = cs_row + rig;
    if ((gl % (LR / M)) == 0 && idx < T && row < hidden && ((mask >> idx) & 1)) {
      for (int k = 0; k < topk; ++k)
        if ((smask >> (8 * idx + k)) & 1) dpair[(int64_t)(idx * topk + k) * hidden + row] = v[0];
    }
    cs_off += rg.gstep;
    cs_row += group_stride * G;
  }
}

// Ring plan for rows of at most 64 units: LR lanes per row (16, 32 or 64), about
// wpc workgroups per CU over all the launch's slots, S ring stages, row groups dealt
// to the slot's waves in contiguous shares or in turn.  Measured on the Q4_K layer
// (2048 hidden, 768 intermediate, 128 experts, top-8; layer us, old workgroup-tile
// kernels -> rings): 1 token 22.1 -> 22.1, 2 tokens 30.5 -> 29.5 (2 workgroups per
// CU, 2 stages, contiguous), 3 tokens 46.7 -> 40.5 and 4 tokens 48.2 -> 47.9 (3 per
// CU, 2 stages, interleaved); 3 stages were slower throughout.  The direct kernels
// are bound by latency (expert ids, then the first weight bytes), not by the
// stream.
struct RingPlan { int lr, stages, groups_per_wave, wgs; int64_t group_stride; };

static bool moe_ring_plan(int units, int64_t rows, int slots, int tslot, RingPlan& pl) {
  if (units > 64) return false;
  const int wpc = tslot >= 4 ? 3 : 2, st = 2, il = tslot >= 4 ? 1 : 0;
  pl.lr = 16;
  while (pl.lr < units) pl.lr *= 2;
  pl.stages = st;
  const int64_t ngroups = (rows + 64 / pl.lr - 1) / (64 / pl.lr);
  const int64_t per_slot = ((int64_t)wpc * ftk_num_cus() + slots - 1) / slots;   // workgroups
  int64_t waves = per_slot * (MOE_THREADS / 64);
  if (waves > ngroups) waves = ngroups;
  if (il) {
    pl.group_stride = waves;
    pl.groups_per_wave = 0;
  } else {
    pl.group_stride = 1;
    pl.groups_per_wave = (int)((ngroups + waves - 1) / waves);
    waves = (ngroups + pl.groups_per_wave - 1) / pl.groups_per_wave;
  }
  pl.wgs = (int)((waves + MOE_THREADS / 64 - 1) / (MOE_THREADS / 64));
  return true;
}

template <int F, int A, int T, int LR, int S>
static hipError_t launch_ring(const MoeArgs& a, bool gate, const RingPlan& pl, int row_bytes, int units, int c0,
                              int tc, hipStream_t st) {
  const int64_t k = gate ? a.hidden : a.inter;
  const size_t arb = (size_t)(k / Act<A>::BLK * Act<A>::BB);
  const size_t lds = ((T * arb + 15) & ~(size_t)15) + (size_t)(MOE_THREADS / 64) * (S * SegGeo<F>::CPW * 1024 + 16);
  const dim3 grid((unsigned)pl.wgs, (unsigned)(tc * a.topk));
  const size_t p0 = (size_t)c0 * a.topk;
  // more than 64 KiB of LDS needs the opt-in (rows of 64 units, 4 stages, 4 tokens)
  static const bool attr_g = hipFuncSetAttribute((const void*)moe_ring_gate_up_kernel<F, A, T, LR, S>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
  static const bool attr_d = hipFuncSetAttribute((const void*)moe_ring_down_kernel<F, A, T, LR, S>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
  if (lds > 65536 && !(gate ? attr_g : attr_d)) return hipErrorInvalidConfiguration;
  if (gate) {
    hipLaunchKernelGGL((moe_ring_gate_up_kernel<F, A, T, LR, S>), grid, dim3(MOE_THREADS), lds, st,
                       (const uint8_t*)a.w_gate, (const uint8_t*)a.w_up, a.n_expert, a.inter, row_bytes, units,
                       pl.groups_per_wave, pl.group_stride, a.x + (size_t)c0 * a.hidden, a.hidden, tc,
                       a.ids + p0, a.topk, a.h + p0 * a.inter, a.g_tap ? a.g_tap + p0 * a.inter : nullptr,
                       a.u_tap ? a.u_tap + p0 * a.inter : nullptr);
  } else {
    const size_t hrb = arb;
    hipLaunchKernelGGL((moe_ring_down_kernel<F, A, T, LR, S>), grid, dim3(MOE_THREADS), lds, st,
                       (const uint8_t*)a.w_down, a.n_expert, a.hidden, row_bytes, units, pl.groups_per_wave,
                       pl.group_stride, a.h + p0 * a.inter, a.in_hq ? (const uint8_t*)a.in_hq + p0 * hrb : nullptr,
                       a.hq_tap ? (uint8_t*)a.hq_tap + p0 * hrb : nullptr, a.inter, tc, a.ids + p0, a.topk,
                       a.dpair + p0 * a.hidden);
  }
  return hipGetLastError();
}

template <int F, int A, int T>
static hipError_t ring_lp(const MoeArgs& a, bool gate, const RingPlan& pl, int rb, int units, int c0, int tc,
                          hipStream_t st) {
#define FT_RG(LRV, SV) \
  if (pl.lr == LRV && pl.stages == SV) return launch_ring<F, A, T, LRV, SV>(a, gate, pl, rb, units, c0, tc, st);
  FT_RG(16, 2) FT_RG(16, 3) FT_RG(16, 4) FT_RG(32, 2) FT_RG(32, 3) FT_RG(32, 4)
  FT_RG(64, 2) FT_RG(64, 3) FT_RG(64, 4)
#undef FT_RG
  return hipErrorInvalidValue;
}

// tokens are taken in chunks of up to 4 (fewer when the stage's LDS would not fit
// in 64 KiB)
template <int F, int A>
static hipError_t moe_stage(const MoeArgs& a, bool gate, hipStream_t st) {
  const int64_t k = gate ? a.hidden : a.inter;
  const int64_t rows = gate ? a.inter : a.hidden;
  const int row_bytes = (int)(k / Fmt<F>::BLK * Fmt<F>::BB);
  const int units = (int)units_in_row<F>(k);
  const size_t arb = (size_t)(k / Act<A>::BLK * Act<A>::BB);   // quantized activation row
  const size_t tile = (size_t)(MOE_CPL * MOE_THREADS + 1) * 16 * (gate ? 2 : 1);
  int cs = 4;
  while (cs > 1 && tile + (size_t)cs * arb > 65536) cs /= 2;
  if (tile + (size_t)cs * arb > 65536) return hipErrorInvalidValue;
  for (int64_t c0 = 0; c0 < a.t; c0 += cs) {
    const int tc = (int)(a.t - c0 < cs ? a.t - c0 : cs);
    const int tslot = tc <= 1 ? 1 : tc <= 2 ? 2 : 4;
    RingPlan rp;
    if (moe_ring_plan(units, rows, tc * a.topk, tslot, rp)) {
      hipError_t err;
      if (tslot == 1) err = ring_lp<F, A, 1>(a, gate, rp, row_bytes, units, (int)c0, tc, st);
      else if (tslot == 2) err = ring_lp<F, A, 2>(a, gate, rp, row_bytes, units, (int)c0, tc, st);
      else err = ring_lp<F, A, 4>(a, gate, rp, row_bytes, units, (int)c0, tc, st);
      if (err != hipSuccess) return err;
      continue;
    }
    MoePlan pl;
    if (!moe_plan(units, row_bytes, rows, tc * a.topk, pl)) return hipErrorInvalidValue;
    const MoeArgs& ac = a;
    hipError_t err = hipErrorInvalidValue;
    if (gate) {
      if (tslot == 1) err = gate_up_lp<F, A, 1>(ac, pl, row_bytes, units, (int)c0, tc, st);
      else if (tslot == 2) err = gate_up_lp<F, A, 2>(ac, pl, row_bytes, units, (int)c0, tc, st);
      else err = gate_up_lp<F, A, 4>(ac, pl, row_bytes, units, (int)c0, tc, st);
    } else {
      if (tslot == 1) err = down_lp<F, A, 1>(ac, pl, row_bytes, units, (int)c0, tc, st);
      else if (tslot == 2) err = down_lp<F, A, 2>(ac, pl, row_bytes, units, (int)c0, tc, st);
      else err = down_lp<F, A, 4>(ac, pl, row_bytes, units, (int)c0, tc, st);
    }
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace ftk

using namespace ftk;

hipError_t ftk_launch_route(const float* logits, int64_t t, int64_t n_expert, int topk, int32_t* ids, float* w,
                            hipStream_t st) {
  const dim3 grid((unsigned)((t + 3) / 4));
#define FT_RT(ME)                                                                                          \
  if (n_expert <= 64 * ME) {                                                                               \
    hipLaunchKernelGGL(route_kernel<ME>, grid, dim3(256), 0, st, logits, t, (int)n_expert, topk, ids, w); \
    return hipGetLastError();                                                                              \
  }
  FT_RT(1) FT_RT(2) FT_RT(4) FT_RT(8) FT_RT(16)
#undef FT_RT
  return hipErrorInvalidValue;
}

hipError_t ftk_launch_sort(const int32_t* ids, int64_t t, int topk, int64_t n_expert, int32_t* counts,
                           int32_t* offsets, int32_t* pairs, hipStream_t st) {
  // LDS: max(4E, 2*ceil(E/2) + 2*(E+2) + 4*chunk) bytes, kept within 64 KiB
  const int64_t npairs = t * topk;
  if (npairs >= 1 && npairs <= 16 * 64 * SORTF_MAXR && n_expert <= SORTF_MAXE) {
    const int per = (int)(((npairs + 15) / 16 + 63) / 64 * 64);
    int nbits = 0;
    while ((1 << nbits) < n_expert) ++nbits;
    hipLaunchKernelGGL(sort_fast_kernel, dim3(1), dim3(SORT_THREADS), 0, st, ids, (int)npairs, (int)n_expert, nbits,
                       per, counts, offsets, pairs);
    return hipGetLastError();
  }
  const int64_t fixed = 4 * ((n_expert + 1) / 2) + 4 * ((n_expert + 2) / 2);
  int64_t chunk = (65536 - fixed) / 4;
  if (chunk > 65535) chunk = 65535;
  if (chunk < 1024 || npairs > INT32_MAX) return hipErrorInvalidValue;
  if (chunk > npairs) chunk = npairs < 1 ? 1 : npairs;
  size_t lds = (size_t)(fixed + 4 * chunk);
  if (lds < (size_t)(4 * n_expert)) lds = (size_t)(4 * n_expert);
  hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(SORT_THREADS), lds, st, ids, (int)npairs, (int)n_expert, (int)chunk,
                     counts, offsets, pairs);
  return hipGetLastError();
}

// MXFP4 x Q8_K runs on the FP4 matrix cores (ft_moe_fp4.hip)
hipError_t ftk_launch_moe_gate_up(const MoeArgs& a, hipStream_t st) {
  if (a.w == FT_Q4_K && a.act == FT_Q8_1) return moe_stage<FT_Q4_K, FT_Q8_1>(a, true, st);
  if (a.w == FT_MXFP4 && a.act == FT_Q8_K) return ftk_launch_moe_fp4_gate_up(a, st);
  return hipErrorInvalidValue;
}

hipError_t ftk_launch_moe_down(const MoeArgs& a, hipStream_t st) {
  if (a.w == FT_Q4_K && a.act == FT_Q8_1) return moe_stage<FT_Q4_K, FT_Q8_1>(a, false, st);
  if (a.w == FT_MXFP4 && a.act == FT_Q8_K) return ftk_launch_moe_fp4_down(a, st);
  return hipErrorInvalidValue;
}

hipError_t ftk_launch_moe_combine(const MoeArgs& a, hipStream_t st) {
  const int64_t n = a.t * a.hidden;
  if (n == 0) return hipSuccess;
  if (a.hidden % 4 == 0 && a.topk <= 8) {
    const int bpt = (int)((a.hidden + 1023) / 1024);
    hipLaunchKernelGGL(moe_combine4_kernel, dim3((unsigned)(a.t * bpt)), dim3(256), 0, st, a.dpair, a.ew, a.topk,
                       a.hidden, bpt, a.y);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.dpair, a.ew, a.t,
                     a.topk, a.hidden, a.y);
  return hipGetLastError();
}

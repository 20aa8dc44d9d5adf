// ft_moe_fused.hip -- the routed-MoE layer for Q4_K experts x Q8_1 activations in
// two launches: (1) routing, quantize x, gate/up + SwiGLU and the Q8_1 blocks of
// h; (2) down and the weighted combine (ds4 PR #656 "Add ROCm MXFP4 routed expert
// kernels", Summary: routed gate/up and down with SwiGLU between them, coalesced
// weight reads, register unpack, tiny batches on direct kernels; FreeToken PR
// #136, Summary: the routed MoE vector kernel).
//
// Why this split.  At 1-4 tokens the layer reads 21-77 MB of expert weights, a
// few microseconds of HBM time, and latency decides: each launch pays its start,
// the latency of the first weight bytes and a tail.  Separate route, gate/up,
// down and combine launches paid that four times.  Here:
//   K1  every workgroup routes the chunk's tokens itself from the logits (the
//       whole workgroup ranks the keys in parallel: a wave-serial top-k costs
//       microseconds of dependent instructions) or reads the given ids, and
//       builds the table of unique experts.  It takes (expert, 32-row block) tasks of the
//       gate and up banks; each wave streams its rows through its own LDS-DMA
//       ring, SwiGLU follows the 64-lane reduction, the block's 32 h values per
//       token meet in LDS and are quantized to one Q8_1 block there (h itself
//       never goes out unless tapped).  (Reading the down rows K2 streams first
//       at the end of K1, to have them cached, was measured: it made the layer
//       0.6-0.9 us slower, the K1 tail longer than what K2 saved.)
//   K2  a workgroup owns blocks of output rows for every selected expert; each
//       wave takes some of the experts; the (token, slot) down values meet in LDS
//       and the combine is summed there in slot order, so no per-pair rows go out
//       and no combine launch runs.
// A single launch with a grid-wide barrier between the phases was built and
// measured first: on this part the barrier (release, arrival flags, polling,
// acquire) cost 3.5-6 us after the last arrival against ~1.7 us for a kernel
// boundary, so the layer is two ordinary launches with no cross-workgroup waits.
#include <math.h>

#include "ft_device.h"
#include "ft_internal.h"

namespace ftk {

constexpr int FU_WAVES = 8;
constexpr int FU_THREADS = 64 * FU_WAVES;
constexpr int FU_S = 4;                    // ring stages per wave
constexpr int FU_MAXU = 32;                // unique experts of a 4-token chunk at top-8
constexpr int FU_MAXE = 256;               // experts the in-kernel router takes
constexpr int FU_STG = 8;                  // tasks (K1) / row blocks (K2) staged in LDS between stores
constexpr int FU_TAB = 4240;               // LDS bytes: expert table, routing, h and down values, staging

// the chunk's routing and unique-expert table as K1 hands it to K2 (global scratch)
struct FuTable {
  int nu;
  int pad[3];
  int ue[FU_MAXU];          // expert of unique u
  uint32_t um[FU_MAXU];     // tokens of u
  uint64_t us[FU_MAXU];     // (token, slot) pairs of u: bit 8i + k
  int32_t ids[4 * 8];       // [t][topk] routing
  float w[4 * 8];
};

struct FusedArgs {
  const uint8_t* wg;
  const uint8_t* wu;
  const uint8_t* wd;
  int64_t n_expert, hidden, inter;
  const float* x;        // [t][hidden] (this chunk)
  const int32_t* ids;    // [t][topk] (unless routed here)
  const float* ew;       // [t][topk] (unless routed here)
  const float* logits;   // nullable [t][n_expert]: route here (n_expert <= FU_MAXE)
  int rc;                // router: threads per (token, expert) key (1, 2, 4 or 8; t * n_expert * rc <= 512)
  int32_t* ids_out;      // nullable [t][topk]: the routing, written by workgroup 0
  float* w_out;          // nullable [t][topk]
  int t, topk;
  float* h_tap;          // nullable [t*topk][inter]
  float* g_tap;          // nullable
  float* u_tap;          // nullable
  uint8_t* hq;           // [t*topk][inter/32] Q8_1 blocks (written unless in_hq)
  const uint8_t* in_hq;  // nullable: use these blocks instead of quantizing h
  uint8_t* hq_tap;       // nullable: receives in_hq
  float* d_tap;          // nullable [t*topk][hidden]
  float* y;              // [t][hidden]
  FuTable* table;        // scratch: K1 -> K2
};

// LDS layout shared by both kernels: [x-hat or h-hat region][table][rings]
struct FuLds {
  uint8_t* xreg;
  int* s_ue;
  uint32_t* s_um;
  uint64_t* s_us;
  int* s_misc;       // [0] unique count
  float* s_h;        // [2][T][32] (two tasks in turn)
  float* s_d;        // [2][T][8][GB] (two row blocks in turn)
  int32_t* s_ids;    // [4][8]
  float* s_w;        // [4][8]
  uint8_t* stg;      // K1: [FU_STG][T] Q8_1 blocks of h; K2: [FU_STG][T][GB] outputs
  uint32_t* s_selk;  // [4][8] router: the winners' keys
  int32_t* s_ep;     // [32] the experts of the chunk's pairs
  uint8_t* rings;    // the ring area (K1's router keys before the rings start)
  uint8_t* ring;     // this wave's
};
__device__ __forceinline__ FuLds fu_lds(int xbytes, int wave, int sb) {
  extern __shared__ u32x4 smem4[];
  FuLds L;
  L.xreg = (uint8_t*)smem4;
  uint8_t* tab = L.xreg + ((xbytes + 15) & ~15);
  L.s_ue = (int*)tab;
  L.s_um = (uint32_t*)(tab + 128);
  L.s_us = (uint64_t*)(tab + 256);
  L.s_misc = (int*)(tab + 512);
  L.s_h = (float*)(tab + 528);
  L.s_d = (float*)(tab + 1552);
  L.s_ids = (int32_t*)(tab + 2576);
  L.s_w = (float*)(tab + 2704);
  L.stg = tab + 2832;                      // 1152 bytes
  L.s_selk = (uint32_t*)(tab + 3984);
  L.s_ep = (int32_t*)(tab + 4112);
  L.rings = tab + FU_TAB;
  L.ring = L.rings + wave * (FU_S * sb + 16);
  return L;
}

// One ring stage: `nbytes` (<= CPW KiB) from src (16-byte aligned) into dst, CPW
// 16-byte loads per lane (lanes past the end re-read the last chunk), so every
// stage is exactly CPW loads of this wave.  Default cache policy: against the
// streaming hint the layer measured 0.1-0.4 us shorter at 1 and 3 tokens.
template <int CPW>
__device__ __forceinline__ void fu_issue(const uint8_t* src, int nbytes, uint8_t* dst, int lane) {
  const int nch = (nbytes + 15) >> 4;
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int ch = lane + 64 * c < nch ? lane + 64 * c : nch - 1;
    lds_dma16_cached(src + 16 * ch, dst + 1024 * c);
  }
}

// wait until at most k ring stages (CPW loads each) of this wave are in flight,
// 0 <= k <= FU_S
template <int CPW>
__device__ __forceinline__ void wait_stages(int k) {
  static_assert(FU_S == 4 && 4 * CPW < 64, "");
  if (k >= 4) wait_vm<4 * CPW>();
  else if (k == 3) wait_vm<3 * CPW>();
  else if (k == 2) wait_vm<2 * CPW>();
  else if (k == 1) wait_vm<CPW>();
  else wait_vm<0>();
}

// Global stores and loads share one in-order counter on this part: a store issued
// between ring stages makes every later wait for a stage wait for the store too.
// So neither kernel stores inside its ring loop; results are staged in LDS and
// written out after the loop (or when the staging area is full).

// K1: routing, unique experts, gate/up + SwiGLU, Q8_1 blocks of h.
// T: token slots (1, 2, 4); LRA: lanes per gate/up row (a power of two >= the
// row's 64-element units, at most 64).
template <int T, int LRA>
__global__ void __launch_bounds__(FU_THREADS)
moe_q4k_gate_up_kernel(FusedArgs a) {
  using FT = Fmt<FT_Q4_K>;
  constexpr int CPW = SegGeo<FT_Q4_K>::CPW;   // 16-byte DMA chunks per lane per stage
  constexpr int SB = CPW * 1024;              // bytes per ring stage
  constexpr int GA = 64 / LRA;                // rows per stage
  constexpr int GPW = 32 / GA / FU_WAVES;     // groups per wave in a 32-row task
  constexpr int NTT = 2 * GPW;                // tiles per wave and task (gate, up)
  constexpr int MA = 2 * T;
  static_assert(MA <= LRA && GPW >= 1 && FU_STG * T * 36 <= 1152, "");
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int P = (int)gridDim.x;
  const int64_t H = a.hidden, I = a.inter;
  const int xrb = (int)(H / 32 * 36), hrb = (int)(I / 32 * 36);
  const int rba = (int)(H / 256 * 144);       // row bytes (a multiple of 16)
  const int npairs = a.t * a.topk;
  const int nblk = (int)(I / 32);
  const FuLds L = fu_lds(T * xrb, wave, SB);
  const Reader<const uint32_t*> rr{(const uint32_t*)L.ring};

  // the given routing (wave 0, lane p: pair p), then x, then the router logits
  // (element q = tid + FU_THREADS * k of the chunk's [t][n_expert]): every load is
  // in flight before the first use
  int id_in = 0;
  float w_in = 0.0f;
  if (!a.logits && wave == 0 && lane < npairs) {
    id_in = a.ids[lane];
    w_in = a.ew[lane];
  }
  // x in groups of 8 elements: group p of the chunk (token p / xg) on thread
  // p mod FU_THREADS, so all waves share the quantization (xg is a multiple of 4:
  // a block's four groups stay on four aligned lanes)
  const int xg = (int)(H / 8), nxg = a.t * xg;   // xg <= FU_THREADS
  float xv[T][8];
  int xo[T];                                       // LDS offset of the group's block part
#pragma unroll
  for (int k = 0; k < T; ++k) {
    const int p = tid + FU_THREADS * k;
    xo[k] = -1;
    if (p < nxg) {
      const int i = p / xg, gi = p - i * xg;
      xo[k] = i * xrb + (gi >> 2) * 36;
      const float4* src = (const float4*)(a.x + (int64_t)i * H + 8 * gi);
      const float4 f0 = src[0], f1 = src[1];
      xv[k][0] = f0.x; xv[k][1] = f0.y; xv[k][2] = f0.z; xv[k][3] = f0.w;
      xv[k][4] = f1.x; xv[k][5] = f1.y; xv[k][6] = f1.z; xv[k][7] = f1.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) xv[k][q] = 0.0f;
    }
  }
  const int E = (int)a.n_expert, ne = a.logits ? a.t * E : 0;   // ne <= 4 * FU_MAXE
  constexpr int RK = 4 * FU_MAXE / FU_THREADS;
  float lr[RK];
#pragma unroll
  for (int k = 0; k < RK; ++k) {
    const int q = tid + FU_THREADS * k;
    lr[k] = q < ne ? a.logits[q] : 0.0f;
  }

  // quantize x into LDS (Q8_1), the arithmetic of ft_quantize_act, while the
  // logits arrive
#pragma unroll
  for (int k = 0; k < T; ++k)
    if (xo[k] >= 0) q8_1_part(xv[k], tid & 3, L.xreg + xo[k]);

  // the router (same selection and weights as ft_moe_route), spread over the
  // workgroup: each (token, expert) gets the 64-bit key (order-preserving logit
  // key, then the complement of the expert index), so keys are distinct and
  // "greater" means larger logit, or equal logit and lower index; an expert's
  // slot is the number of its token's keys above its own (rc threads per expert
  // count a share each), and slots below k are the winners
  if (a.logits)
    wg_route_rank<FU_THREADS, RK>(lr, ne, E, a.topk, a.rc, (uint64_t*)L.rings, (uint32_t*)(L.rings + 8 * 4 * FU_MAXE),
                                  L.s_ids, L.s_selk);
  lds_barrier();

  // wave 0: the routing weights (logits) and the chunk's unique experts, each with
  // its tokens and (token, slot) pairs (lane p holds pair p; its first occurrence
  // owns the expert).  One token routed here: its slots are already the unique
  // experts (top-k picks distinct ones), so every workgroup but the one that
  // writes the table for K2 takes them straight from the routing (1 token
  // 16.2-16.4 -> 15.7-15.8 us per layer).
  const bool fast1 = T == 1 && a.logits != nullptr && blockIdx.x != 0;
  if (fast1) {
    if (tid < a.topk) {
      L.s_ue[tid] = L.s_ids[tid];
      L.s_um[tid] = 1u;
      L.s_us[tid] = 1ull << tid;
    }
    if (tid == 0) L.s_misc[0] = a.topk;
  }
  if (wave == 0 && !fast1) {
    const bool pv = lane < npairs;
    int ep = 0;
    float wv = 0.0f;
    if (a.logits) {
      route_pair_weights(L.s_ids, L.s_selk, (float*)L.rings, a.t, a.topk, lane, ep, wv);
    } else if (pv) {
      ep = clamp_id(id_in, a.n_expert);
      wv = w_in;
    }
    if (lane < 32) L.s_ep[lane] = pv ? ep : -1 - lane;   // no two idle entries match
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    uint64_t same = 0;   // pairs naming the same expert as this lane's (all 32 entries, 4 per read)
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
      const int4 q = *(const int4*)(L.s_ep + j);
      same |= ((uint64_t)(q.x == ep) << j) | ((uint64_t)(q.y == ep) << (j + 1)) | ((uint64_t)(q.z == ep) << (j + 2)) |
              ((uint64_t)(q.w == ep) << (j + 3));
    }
    if (!pv) same = 0;
    const bool first = pv && (same & ((1ull << lane) - 1)) == 0;
    const uint64_t firsts = __ballot(first);
    const int nu = __popcll(firsts);
    if (first) {
      const int u = __popcll(firsts & ((1ull << lane) - 1));
      uint32_t m = 0;
      uint64_t sm = 0;
      for (int i = 0; i < a.t; ++i) {
        const uint64_t b = (same >> (i * a.topk)) & ((1ull << a.topk) - 1);
        sm |= b << (8 * i);
        if (b) m |= 1u << i;
      }
      L.s_ue[u] = ep;
      L.s_um[u] = m;
      L.s_us[u] = sm;
      if (blockIdx.x == 0) {   // the table for K2
        a.table->ue[u] = ep;
        a.table->um[u] = m;
        a.table->us[u] = sm;
      }
    }
    if (lane == 0) L.s_misc[0] = nu;
    if (blockIdx.x == 0) {
      if (lane == 0) a.table->nu = nu;
      if (pv) {   // the routing for K2 and the caller
        a.table->ids[lane] = ep;
        a.table->w[lane] = wv;
        if (a.logits && a.ids_out) a.ids_out[lane] = ep;
        if (a.logits && a.w_out) a.w_out[lane] = wv;
      }
    }
  }
  lds_barrier();
  const int nu = __builtin_amdgcn_readfirstlane(L.s_misc[0]);

  // tasks (u, 32-row block) = blockIdx.x + j * P; in a task, wave v takes the
  // groups v*GPW .. v*GPW + GPW - 1 of GA rows, each as a gate tile and an up tile
  const int ntask = nu * nblk;
  const int my_tasks = (int)blockIdx.x < ntask ? (ntask - (int)blockIdx.x + P - 1) / P : 0;
  const int ntiles_a = my_tasks * NTT;
  int issued = 0, stage_i = 0;
  auto issue_a = [&](int jt) {
    const int task = (int)blockIdx.x + (jt / NTT) * P;
    const int q2 = jt % NTT;
    const int u = task / nblk, blk = task - u * nblk;
    const int e = __builtin_amdgcn_readfirstlane(L.s_ue[u]);
    const int64_t r0 = 32 * (int64_t)blk + (wave * GPW + (q2 >> 1)) * GA;
    fu_issue<CPW>(((q2 & 1) ? a.wu : a.wg) + ((int64_t)e * I + r0) * rba, GA * rba, L.ring + stage_i * SB, lane);
    ++issued;
    stage_i = stage_i + 1 == FU_S ? 0 : stage_i + 1;
  };
  for (int j = 0; j < FU_S && j < ntiles_a; ++j) issue_a(j);

  const int gl = lane % LRA, rig = lane / LRA;
  const bool uv = gl < (int)(H / 64);
  const int un = uv ? gl : 0;
  ActUnit<FT_Q4_K> act[T];
#pragma unroll
  for (int i = 0; i < T; ++i) {
    if (uv && i < a.t) load_act_unit<FT_Q4_K, FT_Q8_1>(L.xreg + i * xrb, un / FT::UPB, un % FT::UPB, act[i]);
    else zero_act_unit<FT_Q4_K>(act[i]);
  }
  const uint32_t lane_off = (uint32_t)(rig * rba + (un / FT::UPB) * FT::BB);

  // the staged Q8_1 blocks of tasks j0 .. j1 -> hq, each to every slot naming it
  auto flush_hq = [&](int j0, int j1) {
    const int nent = (j1 - j0 + 1) * T * 9;   // 9 words per block
    for (int q = tid; q < nent; q += FU_THREADS) {
      const int ent = q / 9, wd = q - ent * 9;
      const int jj = j0 + ent / T, i = ent % T;
      const int task = (int)blockIdx.x + jj * P;
      const int u = task / nblk, blk = task - u * nblk;
      if (((L.s_um[u] >> i) & 1) == 0) continue;
      const uint64_t smask = L.s_us[u];
      const uint32_t v = ((const uint32_t*)(L.stg + ((jj % FU_STG) * T + i) * 36))[wd];
      for (int kk = 0; kk < a.topk; ++kk)
        if ((smask >> (8 * i + kk)) & 1) ((uint32_t*)(a.hq + (int64_t)(i * a.topk + kk) * hrb + 36 * blk))[wd] = v;
    }
  };

  int cur = 0, cs = 0, j0 = 0;
  for (int j = 0; j < my_tasks; ++j) {
    const int task = (int)blockIdx.x + j * P;
    const int u = task / nblk, blk = task - u * nblk;
    const uint32_t mask = __builtin_amdgcn_readfirstlane(L.s_um[u]);
    const uint64_t smask = L.s_us[u];
    float* s_h = L.s_h + (j & 1) * (T * 32);
#pragma unroll
    for (int q = 0; q < GPW; ++q) {
      float v[MA];
#pragma unroll
      for (int i = 0; i < MA; ++i) v[i] = 0.0f;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        wait_tiles<CPW, FU_S>(issued - 1 - cur);
        Unit<FT_Q4_K> uw;
        unpack_unit<FT_Q4_K, true>(rr, (uint32_t)(cs * SB) + lane_off, un % FT::UPB, uw);
#pragma unroll
        for (int i = 0; i < T; ++i)
          if ((mask >> i) & 1) v[m * T + i] = unit_combine<FT_Q4_K>(uw, act[i], v[m * T + i]);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0): the stage is read
        if (issued < ntiles_a) issue_a(issued);
        ++cur;
        cs = cs + 1 == FU_S ? 0 : cs + 1;
      }
      group_reduce_multi<MA, LRA>(v, gl);
      const int idx = gl / (LRA / MA);
      const bool leader = (gl % (LRA / MA)) == 0;
      const float other = __shfl_xor(v[0], LRA / 2, 64);   // the up value of the same token
      const int rb = (wave * GPW + q) * GA + rig;            // row in the 32-row block
      if (leader && idx < T && ((mask >> idx) & 1)) {
        const float gv = v[0], uvv = other, hv = gv / (1.0f + expf(-gv)) * uvv;
        s_h[idx * 32 + rb] = hv;
        if (a.h_tap || a.g_tap || a.u_tap) {   // taps (tests): stores in the loop are fine there
          const int64_t row = 32 * (int64_t)blk + rb;
          for (int kk = 0; kk < a.topk; ++kk) {
            if ((smask >> (8 * idx + kk)) & 1) {
              const int64_t o = (int64_t)(idx * a.topk + kk) * I + row;
              if (a.h_tap) a.h_tap[o] = hv;
              if (a.g_tap) a.g_tap[o] = gv;
              if (a.u_tap) a.u_tap[o] = uvv;
            }
          }
        }
      }
    }
    lds_barrier();
    // the block's h of each token -> one Q8_1 block in the staging area (s_h
    // alternates between tasks, so the next task's groups need no barrier first)
    if (!a.in_hq && tid < 4 * T) {
      const int i = tid >> 2, l4 = tid & 3;   // a token's four lanes stay together
      if ((mask >> i) & 1) {
        float hv8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) hv8[q] = s_h[i * 32 + 8 * l4 + q];
        q8_1_part(hv8, l4, L.stg + ((j % FU_STG) * T + i) * 36);
      }
    }
    if (!a.in_hq && j % FU_STG == FU_STG - 1 && j + 1 < my_tasks) {   // staging full
      lds_barrier();
      flush_hq(j0, j);
      j0 = j + 1;
      lds_barrier();
    }
  }

  if (!a.in_hq && my_tasks > 0) {
    lds_barrier();
    flush_hq(j0, my_tasks - 1);
  }
  if (a.in_hq && a.hq_tap) {
    const int nw = npairs * hrb / 4;
    for (int i = blockIdx.x * FU_THREADS + tid; i < nw; i += P * FU_THREADS)
      ((uint32_t*)a.hq_tap)[i] = ((const uint32_t*)a.in_hq)[i];
  }
  wait_vm<0>();
}

// K2: down projections of every selected expert for this workgroup's row blocks
// and the slot-order combine.
template <int T, int LRB>
__global__ void __launch_bounds__(FU_THREADS)
moe_q4k_down_kernel(FusedArgs a) {
  using FT = Fmt<FT_Q4_K>;
  constexpr int CPW = SegGeo<FT_Q4_K>::CPW;
  constexpr int SB = CPW * 1024;
  constexpr int GB = 64 / LRB;
  static_assert(T <= LRB && FU_STG * T * GB * 4 <= 1152, "");
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int P = (int)gridDim.x;
  const int64_t H = a.hidden, I = a.inter;
  const int hrb = (int)(I / 32 * 36);
  const int rbb = (int)(I / 256 * 144);
  const int npairs = a.t * a.topk;
  const FuLds L = fu_lds(8 * T * hrb, wave, SB);
  const Reader<const uint32_t*> rr{(const uint32_t*)L.ring};

  // the table K1 wrote
  if (tid < FU_MAXU) {
    L.s_ue[tid] = a.table->ue[tid];
    L.s_um[tid] = a.table->um[tid];
    L.s_us[tid] = a.table->us[tid];
    L.s_w[tid] = a.table->w[tid];
    if (tid == 0) L.s_misc[0] = a.table->nu;
  }
  lds_barrier();
  const int nu = __builtin_amdgcn_readfirstlane(L.s_misc[0]);

  // h-hat of every pair into LDS by DMA, issued before this wave's first stages
  // so that waiting for it does not wait for them
  const uint8_t* hsrc = a.in_hq ? a.in_hq : a.hq;
  const int nq = npairs * hrb / 16;
  for (int c = wave; c * 64 < nq; c += FU_WAVES)
    if (c * 64 + lane < nq) lds_dma16_cached(hsrc + 16 * (c * 64 + lane), L.xreg + 1024 * c);

  const int nrb = (int)((H + GB - 1) / GB);
  const int my_rb = (int)blockIdx.x < nrb ? (nrb - (int)blockIdx.x + P - 1) / P : 0;
  const int nuw = wave < nu ? (nu - wave + FU_WAVES - 1) / FU_WAVES : 0;
  const int ntiles_b = my_rb * nuw;
  int issued = 0, stage_i = 0;
  auto issue_b = [&](int j) {
    const int rb = (int)blockIdx.x + (j / nuw) * P;
    const int u = wave + FU_WAVES * (j % nuw);
    const int e = __builtin_amdgcn_readfirstlane(L.s_ue[u]);
    const int64_t r0 = (int64_t)rb * GB;
    const int nrows = (int)(H - r0 < GB ? H - r0 : GB);
    fu_issue<CPW>(a.wd + ((int64_t)e * H + r0) * rbb, nrows * rbb, L.ring + stage_i * SB, lane);
    ++issued;
    stage_i = stage_i + 1 == FU_S ? 0 : stage_i + 1;
  };
  for (int j = 0; j < FU_S && j < ntiles_b; ++j) issue_b(j);
  wait_stages<CPW>(issued);   // this wave's h chunks have landed
  lds_barrier();

  // the staged outputs of row blocks r0 .. r1 -> y
  float* s_y = (float*)L.stg;
  auto flush_y = [&](int r0, int r1) {
    const int n = (r1 - r0 + 1) * T * GB;
    for (int q = tid; q < n; q += FU_THREADS) {
      const int rbi = r0 + q / (T * GB), i = (q / GB) % T, rw = q % GB;
      const int64_t row = (int64_t)((int)blockIdx.x + rbi * P) * GB + rw;
      if (i < a.t && row < H) a.y[(int64_t)i * H + row] = s_y[((rbi % FU_STG) * T + i) * GB + rw];
    }
  };

  const int gl = lane % LRB, rig = lane / LRB;
  const bool uv = gl < (int)(I / 64);
  const int un = uv ? gl : 0;
  const uint32_t lane_off = (uint32_t)(rig * rbb + (un / FT::UPB) * FT::BB);
  int cur = 0, cs = 0, r0 = 0;
  for (int rbi = 0; rbi < my_rb; ++rbi) {
    const int rb = (int)blockIdx.x + rbi * P;
    float* s_d = L.s_d + (rbi & 1) * (T * 8 * GB);
    for (int ui = 0; ui < nuw; ++ui) {
      const int u = wave + FU_WAVES * ui;
      const uint32_t mask = __builtin_amdgcn_readfirstlane(L.s_um[u]);
      const uint64_t smask = L.s_us[u];
      // the h-hat units of the tokens that picked this expert (the other tokens'
      // slots are never read: their combines are skipped below)
      ActUnit<FT_Q4_K> act[T];
#pragma unroll
      for (int i = 0; i < T; ++i) {
        if (T == 1 || ((mask >> i) & 1)) {   // one token: it picked every expert of the table
          if (uv) {
            const int p0 = i * a.topk + (int)__builtin_ctzll((smask >> (8 * i)) & 0xFFull);
            load_act_unit<FT_Q4_K, FT_Q8_1>(L.xreg + p0 * hrb, un / FT::UPB, un % FT::UPB, act[i]);
          } else {
            zero_act_unit<FT_Q4_K>(act[i]);
          }
        }
      }
      wait_tiles<CPW, FU_S>(issued - 1 - cur);
      Unit<FT_Q4_K> uw;
      unpack_unit<FT_Q4_K, true>(rr, (uint32_t)(cs * SB) + lane_off, un % FT::UPB, uw);
      float v[T];
#pragma unroll
      for (int i = 0; i < T; ++i) v[i] = 0.0f;
#pragma unroll
      for (int i = 0; i < T; ++i)
        if ((mask >> i) & 1) v[i] = unit_combine<FT_Q4_K>(uw, act[i], v[i]);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0): the stage is read
      if (issued < ntiles_b) issue_b(issued);
      ++cur;
      cs = cs + 1 == FU_S ? 0 : cs + 1;
      group_reduce_multi<T, LRB>(v, gl);
      const int idx = gl / (LRB / T);
      if ((gl % (LRB / T)) == 0 && idx < T && ((mask >> idx) & 1)) {
        const int64_t row = (int64_t)rb * GB + rig;
        for (int kk = 0; kk < a.topk; ++kk) {
          if ((smask >> (8 * idx + kk)) & 1) {
            s_d[(idx * 8 + kk) * GB + rig] = v[0];
            if (a.d_tap && row < H) a.d_tap[(int64_t)(idx * a.topk + kk) * H + row] = v[0];
          }
        }
      }
    }
    lds_barrier();
    // the combine of this row block, slot order, into the staging area (s_d
    // alternates between row blocks, so the next block needs no barrier first)
    if (tid < T * GB) {
      const int i = tid / GB, rw = tid % GB;
      float sum = 0.0f;
      if (i < a.t)
        for (int kk = 0; kk < a.topk; ++kk) sum = fmaf(L.s_w[i * a.topk + kk], s_d[(i * 8 + kk) * GB + rw], sum);
      s_y[((rbi % FU_STG) * T + i) * GB + rw] = sum;
    }
    if (rbi % FU_STG == FU_STG - 1 && rbi + 1 < my_rb) {   // staging full
      lds_barrier();
      flush_y(r0, rbi);
      r0 = rbi + 1;
      lds_barrier();
    }
  }
  if (my_rb > 0) {
    lds_barrier();
    flush_y(r0, my_rb - 1);
  }
  wait_vm<0>();
}

template <int T>
static size_t k1_lds(int64_t hidden) {
  constexpr int SB = SegGeo<FT_Q4_K>::CPW * 1024;
  return (size_t)(((T * (hidden / 32 * 36) + 15) & ~15) + FU_TAB + FU_WAVES * (FU_S * SB + 16));
}
template <int T>
static size_t k2_lds(int64_t inter) {
  constexpr int SB = SegGeo<FT_Q4_K>::CPW * 1024;
  return (size_t)(((8 * T * (inter / 32 * 36) + 15) & ~15) + FU_TAB + FU_WAVES * (FU_S * SB + 16));
}

static int lanes_for(int64_t units) {
  int lr = 16;
  while (lr < units) lr *= 2;
  return lr;
}

template <int T, int LRA>
static hipError_t launch_k1(const FusedArgs& fa, hipStream_t st) {
  const size_t lds = k1_lds<T>(fa.hidden);
  static const bool attr = hipFuncSetAttribute((const void*)moe_q4k_gate_up_kernel<T, LRA>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
  if (lds > 65536 && !attr) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((moe_q4k_gate_up_kernel<T, LRA>), dim3((unsigned)ftk_num_cus()), dim3(FU_THREADS), lds, st,
                     fa);
  return hipGetLastError();
}
template <int T, int LRB>
static hipError_t launch_k2(const FusedArgs& fa, hipStream_t st) {
  const size_t lds = k2_lds<T>(fa.inter);
  static const bool attr = hipFuncSetAttribute((const void*)moe_q4k_down_kernel<T, LRB>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
  if (lds > 65536 && !attr) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((moe_q4k_down_kernel<T, LRB>), dim3((unsigned)ftk_num_cus()), dim3(FU_THREADS), lds, st, fa);
  return hipGetLastError();
}

template <int T>
static hipError_t fused_t(const FusedArgs& fa, int lra, int lrb, hipStream_t st) {
  hipError_t e = lra == 16 ? launch_k1<T, 16>(fa, st) : lra == 32 ? launch_k1<T, 32>(fa, st) : launch_k1<T, 64>(fa, st);
  if (e != hipSuccess) return e;
  if (lrb == 16) return launch_k2<T, 16>(fa, st);
  if (lrb == 32) return launch_k2<T, 32>(fa, st);
  return launch_k2<T, 64>(fa, st);
}

}  // namespace ftk

using namespace ftk;

size_t ftk_moe_fused_table_bytes() { return sizeof(FuTable); }

bool ftk_moe_fused_routes(int64_t n_expert) { return n_expert <= FU_MAXE; }

bool ftk_moe_fused_ok(int w, int act, int64_t hidden, int64_t inter, int topk) {
  if (w != FT_Q4_K || act != FT_Q8_1 || topk > 8) return false;
  if (hidden % 256 || inter % 256 || hidden > 4096 || inter > 4096 || hidden == 0 || inter == 0) return false;
  return k1_lds<4>(hidden) <= (size_t)(160 * 1024) && k2_lds<4>(inter) <= (size_t)(160 * 1024);
}

hipError_t ftk_launch_moe_fused(const MoeArgs& a, void* table, hipStream_t st) {
  if (!ftk_moe_fused_ok(a.w, a.act, a.hidden, a.inter, a.topk) || !table) return hipErrorInvalidValue;
  if (a.logits && !ftk_moe_fused_routes(a.n_expert)) return hipErrorInvalidValue;
  const int lra = lanes_for(a.hidden / 64), lrb = lanes_for(a.inter / 64);
  const int hrb = (int)(a.inter / 32 * 36);
  for (int64_t c0 = 0; c0 < a.t; c0 += 4) {
    const int tc = (int)(a.t - c0 < 4 ? a.t - c0 : 4);
    const size_t p0 = (size_t)c0 * a.topk;
    FusedArgs fa;
    fa.wg = (const uint8_t*)a.w_gate;
    fa.wu = (const uint8_t*)a.w_up;
    fa.wd = (const uint8_t*)a.w_down;
    fa.n_expert = a.n_expert;
    fa.hidden = a.hidden;
    fa.inter = a.inter;
    fa.x = a.x + (size_t)c0 * a.hidden;
    fa.ids = a.ids ? a.ids + p0 : nullptr;
    fa.ew = a.ew ? a.ew + p0 : nullptr;
    fa.logits = a.logits ? a.logits + (size_t)c0 * a.n_expert : nullptr;
    fa.ids_out = a.ids_out ? a.ids_out + p0 : nullptr;
    fa.w_out = a.w_out ? a.w_out + p0 : nullptr;
    fa.t = tc;
    fa.rc = 1;
    while (fa.rc < 8 && (int64_t)tc * a.n_expert * fa.rc * 2 <= FU_THREADS) fa.rc *= 2;
    fa.topk = a.topk;
    fa.h_tap = a.h_tap ? a.h_tap + p0 * a.inter : nullptr;
    fa.g_tap = a.g_tap ? a.g_tap + p0 * a.inter : nullptr;
    fa.u_tap = a.u_tap ? a.u_tap + p0 * a.inter : nullptr;
    fa.hq = (uint8_t*)a.hq + p0 * hrb;
    fa.in_hq = a.in_hq ? (const uint8_t*)a.in_hq + p0 * hrb : nullptr;
    fa.hq_tap = a.in_hq && a.hq_tap ? (uint8_t*)a.hq_tap + p0 * hrb : nullptr;
    fa.d_tap = a.d_tap ? a.d_tap + p0 * a.hidden : nullptr;
    fa.y = a.y + (size_t)c0 * a.hidden;
    fa.table = (FuTable*)table;
    hipError_t e;
    if (tc == 1) e = fused_t<1>(fa, lra, lrb, st);
    else if (tc == 2) e = fused_t<2>(fa, lra, lrb, st);
    else e = fused_t<4>(fa, lra, lrb, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

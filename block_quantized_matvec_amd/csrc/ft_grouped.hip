// ft_grouped.hip -- grouped keep-quant expert GEMM over expert-sorted pairs.
//
// vllm.cpp PR #523 "grouped + non-grouped keep-quant expert GEMM" (What changed:
// the keep-quant op grouped over expert_ids) and ds4 PR #656 (Summary: larger
// batches on expert-sorted tiles).  y[p] = W[ids[p]] . xhat_row(p) with
// p = token*topk + slot.  The token->expert sort (ft_moe.hip) gives each expert
// its contiguous list of pairs; a workgroup owns (expert, tile of output rows),
// streams that tile of the expert's weights into LDS once with 16-byte
// global_load_lds, and applies it to every pair of the expert, four pairs per
// pass with the activation codes in VGPRs.  Rows never mix across pairs, so the
// order inside the sort cannot change any result.
#include "ft_device.h"
#include "ft_internal.h"

namespace ftk {

constexpr int GRP_THREADS = 256;
constexpr int GRP_T = 4;  // pairs per pass

template <int F, int A, int LR, int P>
__global__ void __launch_bounds__(GRP_THREADS)
grouped_dot4_kernel(const uint8_t* __restrict__ W, int64_t n, int row_bytes, int units_per_row,
                    int rows_per_tile, const uint8_t* __restrict__ xq, int xrow_bytes, int x_per_pair,
                    int topk, const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs,
                    float* __restrict__ y) {
  using FT = Fmt<F>;
  constexpr int T = GRP_T;
  constexpr int G = GRP_THREADS / LR;
  constexpr int RA = 2;
  constexpr int M = RA * T;
  static_assert(M <= LR, "");
  extern __shared__ uint32_t smem[];
  const int tid = threadIdx.x, grp = tid / LR, gl = tid % LR;
  const int e = blockIdx.y;
  const int p0 = offsets[e], p1 = offsets[e + 1];
  if (p0 >= p1) return;

  const int64_t r0 = (int64_t)blockIdx.x * rows_per_tile;
  const int nrows = (int)min<int64_t>(rows_per_tile, n - r0);
  const uint8_t* src = W + ((int64_t)e * n + r0) * row_bytes;
  const uintptr_t sa = (uintptr_t)src;
  const uint8_t* a0 = (const uint8_t*)(sa & ~(uintptr_t)15);
  const uint32_t shift = (uint32_t)(sa & 15);
  const int nchunks = (int)((shift + (int64_t)nrows * row_bytes + 15) >> 4);
  for (int base = 0; base < nchunks; base += GRP_THREADS) {
    const int c = base + tid;
    if (c < nchunks)
      __builtin_amdgcn_global_load_lds((const void*)(a0 + 16 * (int64_t)c),
                                       (__attribute__((address_space(3))) void*)(smem + 4 * (base + (tid >> 6) * 64)),
                                       16, 0, 0);
  }

  int ub[P], uu[P];
  bool uv[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int u = gl + p * LR;
    uv[p] = u < units_per_row;
    ub[p] = u / FT::UPB;
    uu[p] = u % FT::UPB;
  }
  const Reader<const uint32_t*> rd{smem};

  for (int c0 = p0; c0 < p1; c0 += T) {
    const int tc = min(T, p1 - c0);
    int pr[T];
    ActUnit<F> act[P][T];
#pragma unroll
    for (int i = 0; i < T; ++i) {
      pr[i] = i < tc ? pairs[c0 + i] : 0;
      const int64_t xrow = x_per_pair ? pr[i] : pr[i] / topk;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if (uv[p] && i < tc) load_act_unit<F, A>(xq + xrow * xrow_bytes, ub[p], uu[p], act[p][i]);
        else zero_act_unit<F>(act[p][i]);
      }
    }
    if (c0 == p0) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    for (int rb = 0; rb < nrows; rb += G * RA) {
      float v[M];
#pragma unroll
      for (int i = 0; i < M; ++i) v[i] = 0.0f;
#pragma unroll
      for (int ra = 0; ra < RA; ++ra) {
        const int r = rb + ra * G + grp;
        if (r < nrows) {
#pragma unroll
          for (int p = 0; p < P; ++p) {
            if (uv[p]) {
              Unit<F> un;
              unpack_unit<F, (F == FT_Q4_K || F == FT_Q5_K)>(rd, shift + (uint32_t)r * row_bytes + (uint32_t)ub[p] * FT::BB, uu[p], un);
#pragma unroll
              for (int i = 0; i < T; ++i)
                if (i < tc) v[ra * T + i] = unit_combine<F>(un, act[p][i], v[ra * T + i]);
            }
          }
        }
      }
      group_reduce_multi<M, LR>(v, gl);
      const int idx = gl / (LR / M);
      if ((gl % (LR / M)) == 0) {
        const int ra = idx / T, i = idx % T;
        const int r = rb + ra * G + grp;
        if (r < nrows && i < tc) y[(int64_t)pr[i] * n + r0 + r] = v[0];
      }
    }
  }
}

template <int F, int A, int LR, int P>
static hipError_t launch_grouped_t(const GroupedArgs& a, int row_bytes, int units, int rpt, hipStream_t st) {
  const size_t lds = (((size_t)rpt * row_bytes + 32) & ~(size_t)15) + 64;
  const dim3 grid((unsigned)((a.n + rpt - 1) / rpt), (unsigned)a.n_expert);
  hipLaunchKernelGGL((grouped_dot4_kernel<F, A, LR, P>), grid, dim3(GRP_THREADS), lds, st, (const uint8_t*)a.W,
                     a.n, row_bytes, units, rpt, (const uint8_t*)a.xq, (int)(a.k / Act<A>::BLK * Act<A>::BB),
                     a.x_per_pair, a.topk, a.offsets, a.pairs, a.y);
  return hipGetLastError();
}

template <int F, int A>
static hipError_t grouped_fa(const GroupedArgs& a, hipStream_t st) {
  const int row_bytes = (int)(a.k / Fmt<F>::BLK * Fmt<F>::BB);
  const int units = (int)units_in_row<F>(a.k);
  int lr, p = 1;
  if (units <= 64) {
    lr = 16;
    while (lr < units) lr *= 2;
  } else {
    lr = 64;
    while (p * 64 < units) p *= 2;
  }
  const int G = GRP_THREADS / lr;
  int rpt = (32 * 1024) / row_bytes;
  if (rpt > G) rpt = rpt / G * G;
  if (rpt < 1) rpt = 1;
#define FT_G(LRV, PV) \
  if (lr == LRV && p == PV) return launch_grouped_t<F, A, LRV, PV>(a, row_bytes, units, rpt, st);
  FT_G(16, 1) FT_G(32, 1) FT_G(64, 1) FT_G(64, 2) FT_G(64, 4) FT_G(64, 8)
#undef FT_G
  return hipErrorInvalidValue;
}

}  // namespace ftk

using namespace ftk;

hipError_t ftk_launch_grouped(const GroupedArgs& a, hipStream_t st) {
  if (a.act != FT_Q8_K) return hipErrorInvalidValue;
  if (a.k / 32 > 512) return hipErrorInvalidValue;
  switch (a.w) {
    case FT_Q4_K: return grouped_fa<FT_Q4_K, FT_Q8_K>(a, st);
    case FT_Q5_K: return grouped_fa<FT_Q5_K, FT_Q8_K>(a, st);
    case FT_Q6_K: return grouped_fa<FT_Q6_K, FT_Q8_K>(a, st);
    case FT_MXFP4: return grouped_fa<FT_MXFP4, FT_Q8_K>(a, st);
  }
  return hipErrorInvalidValue;
}

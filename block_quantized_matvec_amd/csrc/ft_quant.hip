// ft_quant.hip -- activation quantizers (Q8_1, Q8_K), weight dequantization and
// the integer-partials debug tap.
//
// Quantizers: vllm.cpp PR #523 (What changed: Q8_0 / Q8_K activation quantizers)
// and ds4 PR #656 (Summary: Q8 prequant of activations).  The arithmetic is
// decided in fp32 so that the result is bit-identical on any IEEE device:
// amax, d = amax/127 (stored as fp16 for Q8_1, fp32 for Q8_K), q = clamp(round
// half away from zero of x/d against the stored d, +-127), with the IEEE
// correctly rounded division.
// Dequantization: FreeToken PR #136 (Summary: Q4_0 dequantization) and the packed
// K-quants of FreeToken PR #260; each weight is its exact value rounded once.
#include "ft_device.h"
#include "ft_internal.h"

namespace ftk {

// ---------------------------------------------------------------------------
// Q8_1: one 32-element block per half-wave, one element per lane
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
quant_q8_1_kernel(const float* __restrict__ x, int64_t total_blocks, int64_t nb, int64_t ldx,
                  uint8_t* __restrict__ xq) {
  const int64_t gb = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int l = threadIdx.x & 31;
  if (gb >= total_blocks) return;  // uniform over the half-wave
  const int64_t r = gb / nb, b = gb % nb;
  const float v = x[r * ldx + b * 32 + l];
  float a = fabsf(v);
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m, 32));
  uint32_t dh = f2h_bits(a / 127.0f);
  const float d = h2f(dh);
  int q = 0;
  if (d != 0.0f) {
    const float rq = roundf(v / d);
    q = rq > 127.0f ? 127 : (rq < -127.0f ? -127 : (int)rq);
  }
  int s = q;
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) s += __shfl_xor(s, m, 32);
  uint8_t* ob = xq + gb * 36;
  ob[4 + l] = (uint8_t)(int8_t)q;
  if (l == 0) {
    if (d == 0.0f) dh = 0;
    const uint32_t sh = f2h_bits(d * (float)s);
    *(uint32_t*)ob = dh | (sh << 16);
  }
}

// ---------------------------------------------------------------------------
// Q8_K: one 256-element block per wave, four consecutive elements per lane
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
quant_q8_k_kernel(const float* __restrict__ x, int64_t total_blocks, int64_t nb, int64_t ldx,
                  uint8_t* __restrict__ xq) {
  const int64_t gb = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (gb >= total_blocks) return;  // uniform over the wave
  const int64_t r = gb / nb, b = gb % nb;
  const float* xp = x + r * ldx + b * 256 + 4 * lane;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = xp[i];
  float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m, 64));
  const float d = a / 127.0f;
  uint32_t packed = 0;
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int q = 0;
    if (d != 0.0f) {
      const float rq = roundf(v[i] / d);
      q = rq > 127.0f ? 127 : (rq < -127.0f ? -127 : (int)rq);
    }
    s += q;
    packed |= ((uint32_t)(uint8_t)(int8_t)q) << (8 * i);
  }
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);  // 16-element group: lanes 4g .. 4g+3
  uint8_t* ob = xq + gb * 292;
  *(uint32_t*)(ob + 4 + 4 * lane) = packed;
  if ((lane & 3) == 0) *(int16_t*)(ob + 260 + 2 * (lane >> 2)) = (int16_t)s;
  if (lane == 0) *(float*)ob = d;
}

// ---------------------------------------------------------------------------
// dequantization: four consecutive elements per thread
// ---------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ float elem_value(const Reader<const uint32_t*>& rd, uint32_t bo, int e) {
  if constexpr (F == FT_Q4_0) {
    const uint32_t v = rd.u8(bo + 2 + (e & 15));
    const int n = e < 16 ? (int)(v & 15) : (int)(v >> 4);
    return h2f(rd.u16(bo)) * (float)(n - 8);
  } else if constexpr (F == FT_Q8_0) {
    return h2f(rd.u16(bo)) * (float)(int8_t)rd.u8(bo + 2 + e);
  } else if constexpr (F == FT_MXFP4) {
    const uint32_t v = rd.u8(bo + 1 + (e & 15));
    const uint32_t c = e < 16 ? (v & 15) : (v >> 4);
    const int v2 = (int)(int8_t)(e2m1x2_bytes(c) & 0xFF);
    return (float)v2 * e8m0_half(rd.u8(bo));
  } else if constexpr (F == FT_Q4_K || F == FT_Q5_K) {
    const int c = e >> 6, h = (e >> 5) & 1, l = e & 31;
    const uint32_t qoff = F == FT_Q4_K ? 16 : 48;
    const uint32_t v = rd.u8(bo + qoff + 32 * c + l);
    int n = h ? (int)(v >> 4) : (int)(v & 15);
    if (F == FT_Q5_K) n += 16 * (int)((rd.u8(bo + 16 + l) >> (2 * c + h)) & 1);
    uint32_t sc, m;
    kq_scale_min(rd.u32(bo + 4), rd.u32(bo + 8), rd.u32(bo + 12), e >> 5, sc, m);
    const uint32_t ddm = rd.u32(bo);
    const float d = h2f(ddm & 0xFFFF), dmin = h2f(ddm >> 16);
    const float a = (d * (float)sc) * (float)n;   // exact
    const float b = dmin * (float)m;              // exact
    return a - b;                                 // one rounding
  } else {  // Q6_K
    const int g = e >> 7, r = (e >> 5) & 3, l = e & 31;
    const uint32_t lq = rd.u8(bo + 64 * g + 32 * (r & 1) + l);
    const int lo = r < 2 ? (int)(lq & 15) : (int)(lq >> 4);
    const int hi = (int)((rd.u8(bo + 128 + 32 * g + l) >> (2 * r)) & 3);
    const float sc = (float)(int8_t)rd.u8(bo + 192 + (e >> 4));
    return (h2f(rd.u16(bo + 208)) * sc) * (float)((lo | (hi << 4)) - 32);
  }
}

template <int F>
__global__ void __launch_bounds__(256)
dequant_kernel(const uint8_t* __restrict__ blocks, int64_t rows, int64_t k, float* __restrict__ out) {
  using FT = Fmt<F>;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // group of 4 elements
  const int64_t groups_per_row = k / 4;
  if (q >= rows * groups_per_row) return;
  const int64_t r = q / groups_per_row, e0 = (q % groups_per_row) * 4;
  const int64_t b = e0 / FT::BLK;
  const int64_t boff = (r * (k / FT::BLK) + b) * FT::BB;
  const Reader<const uint32_t*> rd{(const uint32_t*)(blocks + (boff & ~(int64_t)3))};
  const uint32_t bo = (uint32_t)(boff & 3);
  const int e = (int)(e0 % FT::BLK);
  float4 o;
  o.x = elem_value<F>(rd, bo, e);
  o.y = elem_value<F>(rd, bo, e + 1);
  o.z = elem_value<F>(rd, bo, e + 2);
  o.w = elem_value<F>(rd, bo, e + 3);
  *(float4*)(out + r * k + e0) = o;
}

// ---------------------------------------------------------------------------
// integer partials: one thread per (token, row, weight block), through the same
// unit unpack and dot core as the matvec kernels
// ---------------------------------------------------------------------------
template <int F, int A>
__global__ void __launch_bounds__(256)
block_dots_kernel(const uint8_t* __restrict__ W, int64_t n, int64_t k, const uint8_t* __restrict__ xq,
                  int64_t t, int32_t* __restrict__ partials) {
  using FT = Fmt<F>;
  constexpr int NSUB = FT::BLK / FT::SUB;
  const int64_t nb = k / FT::BLK;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= t * n * nb) return;
  const int64_t tt = idx / (n * nb), r = (idx / nb) % n, b = idx % nb;
  const int64_t boff = (r * nb + b) * FT::BB;
  const Reader<const uint32_t*> rd{(const uint32_t*)(W + (boff & ~(int64_t)3))};
  const uint32_t bo = (uint32_t)(boff & 3);
  const uint8_t* xrow = xq + tt * (k / Act<A>::BLK) * Act<A>::BB;
  int acc[NSUB];
#pragma unroll
  for (int i = 0; i < NSUB; ++i) acc[i] = 0;
  for (int ui = 0; ui < FT::UPB; ++ui) {
    Unit<F> u;
    unpack_unit<F, false>(rd, bo, ui, u);
    ActUnit<F> au;
    load_act_unit<F, A>(xrow, (int)b, ui, au);
    int I[FT::S];
    unit_dots<F>(u, au, I);
#pragma unroll
    for (int s = 0; s < FT::S; ++s) {
      const int sub = FT::act_elem(ui, seg_first<F>(s)) / FT::SUB;
      const int val = seg_true_dot<F>(s, I[s], au.bsum[s]) - FT::CODE_OFF * au.bsum[s];
#pragma unroll
      for (int i = 0; i < NSUB; ++i)
        if (i == sub) acc[i] += val;
    }
  }
  int32_t* o = partials + ((tt * n + r) * nb + b) * NSUB;
#pragma unroll
  for (int i = 0; i < NSUB; ++i) o[i] = acc[i];
}

}  // namespace ftk

using namespace ftk;

hipError_t ftk_launch_quantize(int act, const float* x, int64_t rows, int64_t k, int64_t ldx, void* xq,
                               hipStream_t st) {
  if (act == FT_Q8_1) {
    const int64_t total = rows * (k / 32);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_q8_1_kernel, dim3((unsigned)((total + 7) / 8)), dim3(256), 0, st, x, total,
                       k / 32, ldx, (uint8_t*)xq);
  } else {
    const int64_t total = rows * (k / 256);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_q8_k_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, st, x, total,
                       k / 256, ldx, (uint8_t*)xq);
  }
  return hipGetLastError();
}

template <int F>
static hipError_t launch_dequant_t(const void* blocks, int64_t rows, int64_t k, float* out, hipStream_t st) {
  const int64_t groups = rows * (k / 4);
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_kernel<F>, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st,
                     (const uint8_t*)blocks, rows, k, out);
  return hipGetLastError();
}

hipError_t ftk_launch_dequant(int w, const void* blocks, int64_t rows, int64_t k, float* out, hipStream_t st) {
  switch (w) {
    case FT_Q4_0: return launch_dequant_t<FT_Q4_0>(blocks, rows, k, out, st);
    case FT_Q8_0: return launch_dequant_t<FT_Q8_0>(blocks, rows, k, out, st);
    case FT_Q4_K: return launch_dequant_t<FT_Q4_K>(blocks, rows, k, out, st);
    case FT_Q5_K: return launch_dequant_t<FT_Q5_K>(blocks, rows, k, out, st);
    case FT_Q6_K: return launch_dequant_t<FT_Q6_K>(blocks, rows, k, out, st);
    case FT_MXFP4: return launch_dequant_t<FT_MXFP4>(blocks, rows, k, out, st);
  }
  return hipErrorInvalidValue;
}

template <int F, int A>
static hipError_t launch_dots_t(const void* W, int64_t n, int64_t k, const void* xq, int64_t t, int32_t* p,
                                hipStream_t st) {
  const int64_t work = t * n * (k / Fmt<F>::BLK);
  if (work == 0) return hipSuccess;
  hipLaunchKernelGGL((block_dots_kernel<F, A>), dim3((unsigned)((work + 255) / 256)), dim3(256), 0, st,
                     (const uint8_t*)W, n, k, (const uint8_t*)xq, t, p);
  return hipGetLastError();
}

hipError_t ftk_launch_block_dots(int w, const void* W, int64_t n, int64_t k, int act, const void* xq,
                                 int64_t t, int32_t* partials, hipStream_t st) {
#define FT_D(F)                                                                              \
  case F:                                                                                    \
    return act == FT_Q8_1 ? launch_dots_t<F, FT_Q8_1>(W, n, k, xq, t, partials, st)          \
                          : launch_dots_t<F, FT_Q8_K>(W, n, k, xq, t, partials, st);
  switch (w) {
    FT_D(FT_Q4_0) FT_D(FT_Q8_0) FT_D(FT_Q4_K) FT_D(FT_Q5_K) FT_D(FT_Q6_K) FT_D(FT_MXFP4)
  }
#undef FT_D
  return hipErrorInvalidValue;
}

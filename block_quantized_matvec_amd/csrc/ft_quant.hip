// ft_quant.hip -- activation quantizers (Q8_1, Q8_0, Q8_K), weight dequantization
// and the integer-partials debug tap.
//
// Quantizers: vllm.cpp PR #523 (What changed: Q8_0 / Q8_K activation quantizers)
// and ds4 PR #656 (Summary: Q8 prequant of activations).  The arithmetic is
// decided in fp32 so that the result is bit-identical on any IEEE device:
// amax, d = amax/127 (stored as fp16 for Q8_1 and Q8_0, fp32 for Q8_K), q = clamp(round
// half away from zero of x/d against the stored d, +-127), with the IEEE
// correctly rounded division.
// Dequantization: FreeToken PR #136 (Summary: Q4_0 dequantization) and the packed
// K-quants of FreeToken PR #260; each weight is its exact value rounded once.
#include "ft_device.h"
#include "ft_internal.h"

namespace ftk {

// ---------------------------------------------------------------------------
// Q8_1: four lanes per 32-element block, eight consecutive elements per lane;
// the block's amax and code sum combine over its four lanes with DPP moves (no
// LDS round trips on the path).  VEC: x and ldx keep every block 16-byte
// aligned, so a lane reads its elements with two 16-byte loads.
// ---------------------------------------------------------------------------
template <bool VEC>
__global__ void __launch_bounds__(256)
quant_q8_1_kernel(const float* __restrict__ x, int64_t total_blocks, int64_t nb, int64_t ldx,
                  uint8_t* __restrict__ xq) {
  const int64_t gb = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int l4 = threadIdx.x & 3;
  if (gb >= total_blocks) return;  // uniform over the block's four lanes
  const int64_t r = gb / nb, b = gb % nb;
  const float* xp = x + r * ldx + b * 32 + 8 * l4;
  float v[8];
  if constexpr (VEC) {
    const float4 a = ((const float4*)xp)[0], c = ((const float4*)xp)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = xp[j];
  }
  q8_1_part(v, l4, xq + gb * 36);
}

// ---------------------------------------------------------------------------
// Q8_0: the Q8_1 arithmetic (fp16 d = amax/127, codes against the stored d) in
// the 34-byte block without the sum field: fp16 d at byte 0, the 32 codes from
// byte 2 (each lane's eight codes go out as four 16-bit stores).
// ---------------------------------------------------------------------------
template <bool VEC>
__global__ void __launch_bounds__(256)
quant_q8_0_kernel(const float* __restrict__ x, int64_t total_blocks, int64_t nb, int64_t ldx,
                  uint8_t* __restrict__ xq) {
  const int64_t gb = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int l4 = threadIdx.x & 3;
  if (gb >= total_blocks) return;  // uniform over the block's four lanes
  const int64_t r = gb / nb, b = gb % nb;
  const float* xp = x + r * ldx + b * 32 + 8 * l4;
  float v[8];
  if constexpr (VEC) {
    const float4 a = ((const float4*)xp)[0], c = ((const float4*)xp)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = xp[j];
  }
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[j]));
  a = fmaxf(a, xchg<1>(a));
  a = fmaxf(a, xchg<2>(a));
  uint32_t dh = f2h_bits(a / 127.0f);
  const float d = h2f(dh);
  uint8_t* ob = xq + gb * 34;
  uint16_t* o = (uint16_t*)(ob + 2 + 8 * l4);
  int qc[8];
  q8_codes<8>(v, d, qc);
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const uint32_t lo = (uint32_t)(uint8_t)(int8_t)qc[j];
    const uint32_t hi = (uint32_t)(uint8_t)(int8_t)qc[j + 1];
    o[j >> 1] = (uint16_t)(lo | (hi << 8));
  }
  if (l4 == 0) *(uint16_t*)ob = (uint16_t)(d == 0.0f ? 0u : dh);
}

// Q8_0 activation blocks (34 bytes) -> the Q8_1 layout (36 bytes: d, s = fp16(d *
// sum of codes), the same codes) that the matvec kernels read with aligned dword
// loads; the dots use d and the codes only, so the result is the Q8_0 one.  One
// thread per block.
__global__ void __launch_bounds__(256)
repack_q8_0_kernel(const uint8_t* __restrict__ src, int64_t nblocks, uint8_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblocks) return;
  const uint16_t* s = (const uint16_t*)(src + i * 34);   // 34 is even: 2-byte aligned
  uint32_t* o = (uint32_t*)(dst + i * 36);
  const uint32_t dh = s[0];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w = (uint32_t)s[1 + 2 * j] | ((uint32_t)s[2 + 2 * j] << 16);
    sum = dot4(w, 0x01010101u, sum);
    o[1 + j] = w;
  }
  o[0] = dh | (f2h_bits(h2f(dh) * (float)sum) << 16);
}

// ---------------------------------------------------------------------------
// Q8_K: sixteen lanes per 256-element block, sixteen consecutive elements per
// lane (one 16-element code sum each); amax over the sixteen lanes by DPP.
// ---------------------------------------------------------------------------
template <bool VEC>
__global__ void __launch_bounds__(256)
quant_q8_k_kernel(const float* __restrict__ x, int64_t total_blocks, int64_t nb, int64_t ldx,
                  uint8_t* __restrict__ xq) {
  const int64_t gb = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  if (gb >= total_blocks) return;  // uniform over the block's sixteen lanes
  const int64_t r = gb / nb, b = gb % nb;
  const float* xp = x + r * ldx + b * 256 + 16 * l16;
  float v[16];
  if constexpr (VEC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 a = ((const float4*)xp)[i];
      v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = xp[j];
  }
  q8_k_part(v, l16, xq + gb * 292);
}

// ---------------------------------------------------------------------------
// Q8_K codes -> exact FP8 halves for the block-scaled FP4 MFMA.
// Each code x in [-127, 127] is x = 16*hi + lo with hi = x >> 4 in [-8, 7] and
// lo = x & 15 in [0, 15]; both are exact OCP E4M3 values.  For every 256-element
// superblock the output holds 32 chunks of 16 bytes, chunk c = 16p + 2j + h
// (p = 0: lo, 1: hi; j = 32-element block; h = half): the FP8 codes of elements
// 8h..8h+7 and 16+8h..16+8h+7 of block j, interleaved (a0 b0 a1 b1 ...) so that
// byte i of the chunk multiplies nibble 16h + i of an MXFP4 block's qs bytes
// (nibble n is byte n/2, low nibble first: element n/2 + 16*(n&1)).
// ---------------------------------------------------------------------------
// FP8 codes of the 4-bit values in each byte of v (tables: entries 0-7 and 8-15)
__device__ __forceinline__ uint32_t fp8_lut(uint32_t v, uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3) {
  const uint32_t sel = v & 0x07070707u;
  const uint32_t a = __builtin_amdgcn_perm(t1, t0, sel);
  const uint32_t b = __builtin_amdgcn_perm(t3, t2, sel);
  const uint32_t m = ((v >> 3) & 0x01010101u) * 0xFFu;   // 0xFF in bytes whose value is >= 8
  return (a & ~m) | (b & m);
}

__global__ void __launch_bounds__(256)
fp8_split_kernel(const uint8_t* __restrict__ xq, int64_t total_chunks, uint8_t* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total_chunks) return;
  const int c = (int)(gid & 31);
  const int64_t rs = gid >> 5;   // (row, superblock)
  const int p = c >> 4, j = (c >> 1) & 7, h = c & 1;
  const uint32_t* blk = (const uint32_t*)(xq + rs * 292 + 4 + 32 * j);
  const uint32_t ra[2] = {blk[2 * h], blk[2 * h + 1]};           // elements 8h .. 8h+7
  const uint32_t rb[2] = {blk[4 + 2 * h], blk[5 + 2 * h]};       // elements 16+8h .. 16+8h+7
  // lo: x & 15 -> 0 1 2 3 4 5 6 7 | 8 .. 15;  hi: (x >> 4) as 4-bit two's complement
  const uint32_t t0 = 0x44403800u, t1 = 0x4E4C4A48u;             // 0, 1, 2, 3 | 4, 5, 6, 7
  const uint32_t t2 = p ? 0xCACCCED0u : 0x53525150u;             // hi: -8 -7 -6 -5 | lo: 8 9 10 11
  const uint32_t t3 = p ? 0xB8C0C4C8u : 0x57565554u;             // hi: -4 -3 -2 -1 | lo: 12 .. 15
  uint32_t ca[2], cb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t va = p ? (ra[i] >> 4) & 0x0F0F0F0Fu : ra[i] & 0x0F0F0F0Fu;
    const uint32_t vb = p ? (rb[i] >> 4) & 0x0F0F0F0Fu : rb[i] & 0x0F0F0F0Fu;
    ca[i] = fp8_lut(va, t0, t1, t2, t3);
    cb[i] = fp8_lut(vb, t0, t1, t2, t3);
  }
  u32x4 o;
  o.x = __builtin_amdgcn_perm(cb[0], ca[0], 0x05010400u);
  o.y = __builtin_amdgcn_perm(cb[0], ca[0], 0x07030602u);
  o.z = __builtin_amdgcn_perm(cb[1], ca[1], 0x05010400u);
  o.w = __builtin_amdgcn_perm(cb[1], ca[1], 0x07030602u);
  *(u32x4*)(out + gid * 16) = o;
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
  } else if constexpr (F == FT_Q4_1 || F == FT_Q5_0 || F == FT_Q5_1) {
    constexpr uint32_t QO = F == FT_Q4_1 ? 4 : F == FT_Q5_0 ? 6 : 8;
    const uint32_t v = rd.u8(bo + QO + (e & 15));
    int q = e < 16 ? (int)(v & 15) : (int)(v >> 4);
    if (F != FT_Q4_1) q += 16 * (int)((rd.u8(bo + QO - 4 + (e >> 3)) >> (e & 7)) & 1);
    const float d = h2f(rd.u16(bo));
    if (F == FT_Q5_0) return d * (float)(q - 16);       // exact
    return fmaf(d, (float)q, h2f(rd.u16(bo + 2)));      // d*q exact; one rounding
  } else if constexpr (F == FT_Q2_K) {
    const int g = e >> 7, r = (e >> 5) & 3, l = e & 31;
    const int q = (int)((rd.u8(bo + 16 + 32 * g + l) >> (2 * r)) & 3);
    const uint32_t sm = rd.u8(bo + (e >> 4));
    const uint32_t dd = rd.u32(bo + 80);
    const float a = (h2f(dd & 0xFFFF) * (float)(sm & 15)) * (float)q;   // exact
    const float b = h2f(dd >> 16) * (float)(sm >> 4);                     // exact
    return a - b;                                                         // one rounding
  } else if constexpr (F == FT_Q3_K) {
    const int g = e >> 7, r = (e >> 5) & 3, l = e & 31, j = e >> 4;
    const int lo2 = (int)((rd.u8(bo + 32 + 32 * g + l) >> (2 * r)) & 3);
    const int third = (int)((rd.u8(bo + l) >> (4 * g + r)) & 1);
    const uint32_t lo = (rd.u8(bo + 96 + (j & 7)) >> (j < 8 ? 0 : 4)) & 15;
    const uint32_t hi = (rd.u8(bo + 104 + (j & 3)) >> (2 * (j >> 2))) & 3;
    const float sc = (float)((int)(lo | (hi << 4)) - 32);
    return (h2f(rd.u16(bo + 108)) * sc) * (float)(lo2 + 4 * third - 4);
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
  const bool vec = ((uintptr_t)x & 15) == 0 && (ldx & 3) == 0;
  if (act == FT_Q8_0) {
    const int64_t total = rows * (k / 32);
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)((total + 63) / 64));
    if (vec) hipLaunchKernelGGL(quant_q8_0_kernel<true>, grid, dim3(256), 0, st, x, total, k / 32, ldx, (uint8_t*)xq);
    else hipLaunchKernelGGL(quant_q8_0_kernel<false>, grid, dim3(256), 0, st, x, total, k / 32, ldx, (uint8_t*)xq);
  } else if (act == FT_Q8_1) {
    const int64_t total = rows * (k / 32);
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)((total + 63) / 64));
    if (vec) hipLaunchKernelGGL(quant_q8_1_kernel<true>, grid, dim3(256), 0, st, x, total, k / 32, ldx, (uint8_t*)xq);
    else hipLaunchKernelGGL(quant_q8_1_kernel<false>, grid, dim3(256), 0, st, x, total, k / 32, ldx, (uint8_t*)xq);
  } else {
    const int64_t total = rows * (k / 256);
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)((total + 15) / 16));
    if (vec) hipLaunchKernelGGL(quant_q8_k_kernel<true>, grid, dim3(256), 0, st, x, total, k / 256, ldx, (uint8_t*)xq);
    else hipLaunchKernelGGL(quant_q8_k_kernel<false>, grid, dim3(256), 0, st, x, total, k / 256, ldx, (uint8_t*)xq);
  }
  return hipGetLastError();
}

hipError_t ftk_launch_repack_q8_0(const void* src, int64_t nblocks, void* dst, hipStream_t st) {
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(repack_q8_0_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, st,
                     (const uint8_t*)src, nblocks, (uint8_t*)dst);
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

hipError_t ftk_launch_fp8_split(const void* xq, int64_t rows, int64_t k, void* out, hipStream_t st) {
  const int64_t chunks = rows * (k / 256) * 32;
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(fp8_split_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st,
                     (const uint8_t*)xq, chunks, (uint8_t*)out);
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
    case FT_Q2_K: return launch_dequant_t<FT_Q2_K>(blocks, rows, k, out, st);
    case FT_Q3_K: return launch_dequant_t<FT_Q3_K>(blocks, rows, k, out, st);
    case FT_Q4_1: return launch_dequant_t<FT_Q4_1>(blocks, rows, k, out, st);
    case FT_Q5_0: return launch_dequant_t<FT_Q5_0>(blocks, rows, k, out, st);
    case FT_Q5_1: return launch_dequant_t<FT_Q5_1>(blocks, rows, k, out, st);
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
    FT_D(FT_Q2_K) FT_D(FT_Q3_K) FT_D(FT_Q4_1) FT_D(FT_Q5_0) FT_D(FT_Q5_1)
  }
#undef FT_D
  return hipErrorInvalidValue;
}

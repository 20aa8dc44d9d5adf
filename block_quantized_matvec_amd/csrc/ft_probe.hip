// ft_probe.hip -- measurement microkernels: the ceilings the hot path's kernels
// are held against, measured on the part itself next to the published peaks
// (a streaming HBM read, the int8 MFMA issue rate, the VALU dot4 rate).  They
// compute nothing of the method; every result goes to `out` only when it equals
// a value no input produces, so no load or instruction can be dropped.
#include "ft_device.h"
#include "ft_internal.h"

namespace ftk {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int PROBE_THREADS = 256;
constexpr uint32_t PROBE_MAGIC = 0x9E3779B9u;

// Streaming read: workgroup b reads its own contiguous span of per_wg 16-byte
// chunks (the last span may be shorter or empty), four loads in flight per thread.
__global__ void __launch_bounds__(PROBE_THREADS)
probe_stream_kernel(const u32x4* __restrict__ p, int64_t n16, int64_t per_wg, uint32_t* __restrict__ out) {
  const int64_t b0 = (int64_t)blockIdx.x * per_wg;
  const int64_t lim = b0 >= n16 ? 0 : (n16 - b0 < per_wg ? n16 - b0 : per_wg);
  uint32_t acc = 0;
  for (int64_t i = threadIdx.x; i < lim; i += 4 * PROBE_THREADS) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + (int64_t)u * PROBE_THREADS;
      v[u] = j < lim ? __builtin_nontemporal_load(p + b0 + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == PROBE_MAGIC) out[0] = acc;
}

// int8 MFMA issue rate: eight independent v_mfma_i32_16x16x32_i8 chains per wave,
// iters rounds (16384 ops each).
__global__ void __launch_bounds__(PROBE_THREADS) probe_mfma_kernel(int64_t iters, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const long a = (long)(0x0102030405060708ll * (lane + 1)), b = (long)(0x0807060504030201ll ^ lane);
  v4i acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = v4i{j, 0, 0, 0};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, acc[j], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if ((uint32_t)s == PROBE_MAGIC) out[0] = (uint32_t)s;
}

// the same with gfx950's v_mfma_i32_16x16x64_i8 (32768 ops each)
__global__ void __launch_bounds__(PROBE_THREADS) probe_mfma64_kernel(int64_t iters, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const v4i a = {0x01020304 * (lane + 1), 0x05060708, 0x090A0B0C, 0x0D0E0F10 ^ lane};
  const v4i b = {0x04030201 ^ lane, 0x08070605, 0x0C0B0A09, 0x100F0E0D};
  v4i acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = v4i{j, 0, 0, 0};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if ((uint32_t)s == PROBE_MAGIC) out[0] = (uint32_t)s;
}

// VALU dot4 rate: eight independent v_dot4_i32_i8 chains per lane, iters rounds
// (8 ops per lane and instruction).
__global__ void __launch_bounds__(PROBE_THREADS) probe_dot4_kernel(int64_t iters, uint32_t* __restrict__ out) {
  const uint32_t lane = threadIdx.x;
  const uint32_t a = 0x01020304u * (lane + 1), b = 0x04030201u ^ lane;
  int acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = j;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = dot4(a + (uint32_t)j, b, acc[j]);
  }
  int s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j];
  if ((uint32_t)s == PROBE_MAGIC) out[0] = (uint32_t)s;
}

}  // namespace ftk

using namespace ftk;

// which: 0 streaming read of `bytes` at buf (16-byte aligned, bytes % 16 == 0);
// 1 int8 MFMA (K = 32), 2 VALU dot4 and 3 int8 MFMA (K = 64) for `iters` rounds on
// 8 workgroups per CU.
hipError_t ftk_launch_probe(int which, const void* buf, int64_t bytes, int64_t iters, uint32_t* out, hipStream_t st) {
  const int cus = ftk_num_cus();
  if (which == 0) {
    const int64_t n16 = bytes / 16, wgs = (int64_t)cus * 8;
    const int64_t per = (n16 + wgs - 1) / wgs;
    hipLaunchKernelGGL(probe_stream_kernel, dim3((unsigned)wgs), dim3(PROBE_THREADS), 0, st, (const u32x4*)buf, n16,
                       per, out);
  } else if (which == 1) {
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)(cus * 8)), dim3(PROBE_THREADS), 0, st, iters, out);
  } else if (which == 2) {
    hipLaunchKernelGGL(probe_dot4_kernel, dim3((unsigned)(cus * 8)), dim3(PROBE_THREADS), 0, st, iters, out);
  } else if (which == 3) {
    hipLaunchKernelGGL(probe_mfma64_kernel, dim3((unsigned)(cus * 8)), dim3(PROBE_THREADS), 0, st, iters, out);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

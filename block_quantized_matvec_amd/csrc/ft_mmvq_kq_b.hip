// ft_mmvq_kq_b.hip -- dot4 quantized matvec instantiations for MXFP4 and Q2_K x Q8_1 (kernels in
// ft_mmvq_kernels.h; a translation unit of its own so that the formats compile in
// parallel; the dispatch is in ft_mmvq_kq.hip).
#include "ft_mmvq_kernels.h"

hipError_t ftk_launch_mmvq_dot4_mxfp4(const MmvqArgs& a, int64_t k, hipStream_t st) {
  return ftk::launch_fa<FT_MXFP4, FT_Q8_1>(a, k, st);
}
hipError_t ftk_launch_mmvq_dot4_q2_k(const MmvqArgs& a, int64_t k, hipStream_t st) {
  return ftk::launch_fa<FT_Q2_K, FT_Q8_1>(a, k, st);
}

// ft_mmvq_kq_c.hip -- dot4 quantized matvec instantiations for Q3_K and Q4_1 x Q8_1 (kernels in
// ft_mmvq_kernels.h; a translation unit of its own so that the formats compile in
// parallel; the dispatch is in ft_mmvq_kq.hip).
#include "ft_mmvq_kernels.h"

hipError_t ftk_launch_mmvq_dot4_q3_k(const MmvqArgs& a, int64_t k, hipStream_t st) {
  return ftk::launch_fa<FT_Q3_K, FT_Q8_1>(a, k, st);
}
hipError_t ftk_launch_mmvq_dot4_q4_1(const MmvqArgs& a, int64_t k, hipStream_t st) {
  return ftk::launch_fa<FT_Q4_1, FT_Q8_1>(a, k, st);
}

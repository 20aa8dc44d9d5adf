// ft_mmvq_kq_d.hip -- dot4 quantized matvec instantiations for Q5_0 and Q5_1 x Q8_1 (kernels in
// ft_mmvq_kernels.h; a translation unit of its own so that the formats compile in
// parallel; the dispatch is in ft_mmvq_kq.hip).
#include "ft_mmvq_kernels.h"

hipError_t ftk_launch_mmvq_dot4_q5_0(const MmvqArgs& a, int64_t k, hipStream_t st) {
  return ftk::launch_fa<FT_Q5_0, FT_Q8_1>(a, k, st);
}
hipError_t ftk_launch_mmvq_dot4_q5_1(const MmvqArgs& a, int64_t k, hipStream_t st) {
  return ftk::launch_fa<FT_Q5_1, FT_Q8_1>(a, k, st);
}

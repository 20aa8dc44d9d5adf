// ft_mmvq_kq.hip -- the dot4 quantized matvec for Q5_K, Q6_K, MXFP4, Q2_K, Q3_K, Q4_1,
// Q5_0 and Q5_1 weights
// against Q8_1 activations (kernels in ft_mmvq_kernels.h; translation units of
// their own -- this one for Q5_K and Q6_K, ft_mmvq_kq_{b,c,d}.hip for the rest --
// so that they compile in parallel with ft_mmvq.hip).  Same unit core as
// the expert kernels: Q5_K's fifth bits, Q6_K's 2-bit pairs and 16-element scale
// groups, MXFP4's E2M1 codes doubled to integers with the E8M0 exponent in the
// scale, Q2_K's and Q3_K's 2-bit fields with 16-element scale groups (Q3_K's third
// bit and -4 offset as for Q6_K's -32), and the 32-element Q4_1 / Q5_0 / Q5_1 blocks
// (fifth bits spread into the code bytes, the offset m or -16 through the min term).
#include "ft_mmvq_kernels.h"

hipError_t ftk_launch_mmvq_kq(const MmvqArgs& a, int64_t k, hipStream_t st) {
  using namespace ftk;
  if (a.act != FT_Q8_1) return hipErrorInvalidValue;
  switch (a.w) {
    case FT_Q5_K: return launch_fa<FT_Q5_K, FT_Q8_1>(a, k, st);
    case FT_Q6_K: return launch_fa<FT_Q6_K, FT_Q8_1>(a, k, st);
    case FT_MXFP4: return ftk_launch_mmvq_dot4_mxfp4(a, k, st);
    case FT_Q2_K: return ftk_launch_mmvq_dot4_q2_k(a, k, st);
    case FT_Q3_K: return ftk_launch_mmvq_dot4_q3_k(a, k, st);
    case FT_Q4_1: return ftk_launch_mmvq_dot4_q4_1(a, k, st);
    case FT_Q5_0: return ftk_launch_mmvq_dot4_q5_0(a, k, st);
    case FT_Q5_1: return ftk_launch_mmvq_dot4_q5_1(a, k, st);
    default: return hipErrorInvalidValue;
  }
}

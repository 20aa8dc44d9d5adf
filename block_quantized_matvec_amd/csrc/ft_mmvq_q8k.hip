// ft_mmvq_q8k.hip -- the non-grouped keep-quant matvec with Q8_K activations
// (vllm.cpp PR #523, What changed: Y = X.W^T with keep-quant W against Q8_K
// activations) for the formats of the grouped GEMM: Q4_K, Q5_K, Q6_K and MXFP4.
// The dot4 kernels of ft_mmvq_kernels.h with the 256-element Q8_K activation
// block in place of Q8_1's 32-element one (fp32 scale; the code sums of the min
// term are recomputed from the codes, as for Q8_1); every token count runs on
// dot4.
#include "ft_mmvq_kernels.h"

hipError_t ftk_launch_mmvq_q8k(const MmvqArgs& a, int64_t k, hipStream_t st) {
  using namespace ftk;
  if (a.act != FT_Q8_K) return hipErrorInvalidValue;
  switch (a.w) {
    case FT_Q4_K: return launch_fa<FT_Q4_K, FT_Q8_K>(a, k, st);
    case FT_Q5_K: return launch_fa<FT_Q5_K, FT_Q8_K>(a, k, st);
    case FT_Q6_K: return launch_fa<FT_Q6_K, FT_Q8_K>(a, k, st);
    case FT_MXFP4: return launch_fa<FT_MXFP4, FT_Q8_K>(a, k, st);
    default: return hipErrorInvalidValue;
  }
}

"""MI355X-native block-quantized matvec, routed-MoE vector path and grouped
keep-quant expert GEMM.  The kernels live in libft.so (HIP, gfx950) behind the C
ABI in include/ft.h; ``block_quantized_matvec_amd.ft`` is the Python binding and
``block_quantized_matvec_amd.synth`` the seeded synthetic inputs."""

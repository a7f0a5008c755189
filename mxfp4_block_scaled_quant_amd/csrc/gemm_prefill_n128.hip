// The large-M W4A4 GEMM kernel with 256 x 128 output tiles: the source of
// gemm_prefill.hip built again at that tile width (kernel
// gemm_prefill_n128_kernel, launcher launch_prefill_tiles_128), for M where
// 256-wide tiles leave most compute units idle.
#define MXFP4_PREFILL_BN 128
#include "gemm_prefill.hip"

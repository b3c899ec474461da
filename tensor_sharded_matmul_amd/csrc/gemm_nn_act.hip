// gemm_nn_act.hip — GEMM instantiations: forward column-parallel products with the GeLU / SwiGLU epilogue.
#include "gemm_launch.h"

TPS_INSTANTIATE_GEMM(false, true, tps::EPI_GELU)
TPS_INSTANTIATE_GEMM(false, true, tps::EPI_SWIGLU)

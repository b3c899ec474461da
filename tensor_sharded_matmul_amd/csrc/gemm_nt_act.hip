// gemm_nt_act.hip — GEMM instantiations: input-gradient products with the GeLU / SwiGLU backward epilogue.
#include "gemm_launch.h"

TPS_INSTANTIATE_GEMM(false, false, tps::EPI_GELU_BWD)
TPS_INSTANTIATE_GEMM(false, false, tps::EPI_SWIGLU_BWD)

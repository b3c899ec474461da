// gemm_tn.hip — GEMM instantiations: weight-gradient products X^T dY (fp32).
#include "gemm_launch.h"

TPS_INSTANTIATE_GEMM(true, true, tps::EPI_F32)

// gemm_nt_store.hip — GEMM instantiations: input-gradient products dY W^T with a plain store.
#include "gemm_launch.h"

TPS_INSTANTIATE_GEMM(false, false, tps::EPI_F32)
TPS_INSTANTIATE_GEMM(false, false, tps::EPI_BF16)

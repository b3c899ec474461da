// gemm_nn_store.hip — GEMM instantiations: forward products with a plain store: bf16 column-parallel output, fp32 row-parallel partial.
#include "gemm_launch.h"

TPS_INSTANTIATE_GEMM(false, true, tps::EPI_F32)
TPS_INSTANTIATE_GEMM(false, true, tps::EPI_BF16)

// gemm_nn_ce.hip — GEMM instantiations: the vocab-parallel cross-entropy epilogues of the LM head (per-row logit statistics; softmax-minus-one-hot gradient).
#include "gemm_launch.h"

TPS_INSTANTIATE_GEMM(false, true, tps::EPI_CE_STATS)
TPS_INSTANTIATE_GEMM(false, true, tps::EPI_CE_GRAD)

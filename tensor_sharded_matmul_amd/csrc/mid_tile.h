// mid_tile.h — which products run on mid tiles (shared by the split planner
// of the host entry points and the tile picker of the launches, so that the
// two take the same decision).
#pragma once

#include "gemm_kernel.h"

namespace tps {
// Compute units of the current device (cached per device; tpshard.hip).
int device_cus();

// Mid tiles: 128 x 256 tiles for the weight gradients (TN). A TN product
// with a plain epilogue (fp32 or bf16) whose 256 x 256 tiles would leave at
// least half of the CUs idle, but whose mid tiles fill more than half of
// them in one wave, runs mid tiles over its whole K instead of a K split: no
// fp32 partials, no reduction launch. On the attention shard of
// Llama-3-70B at t = 8 and 4096 tokens this is dW_O = O^T dY (1024 x 8192):
// 66 us in the backward sequence against 62 us for 2 splits plus 17 us for
// their reduction. The same rule on the NT and NN layouts (dO on 128 x 128
// tiles, the QKV forward on 128 x 160 tiles) ran faster alone but slower
// inside the sequences of products, where the chip sits at its power limit
// and a small tile's extra operand traffic costs clock: those keep the
// split.
template <bool A_T, bool B_KN>
struct MidTile {
    static constexpr bool kOn = false;
};
template <>
struct MidTile<true, true> {  // 8 waves of 64 x 64, rings of 6 x 8 KB (A) and 6 x 16 KB (B)
    static constexpr bool kOn = true;
    static constexpr int TM = 128, TN = 256, BKA = 32, SA = 6, BKB = 32, SB = 6, WAVES_M = 2, WAVES_N = 4;
};

template <bool A_T, bool B_KN, int EPI>
inline bool use_mid_tile(int M, int N, int K) {
    using MT = MidTile<A_T, B_KN>;
    if constexpr (!MT::kOn || !(EPI == EPI_F32 || EPI == EPI_BF16)) {
        return false;
    } else {
        const long long cus = device_cus();
        const long long big = (long long)((M + 255) / 256) * ((N + 255) / 256);
        const long long mid = (long long)((M + MT::TM - 1) / MT::TM) * ((N + MT::TN - 1) / MT::TN);
        return M >= 256 && K >= 2048 && 2 * big <= cus && 2 * mid > cus && mid <= cus;
    }
}

}  // namespace tps

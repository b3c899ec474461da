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

// Forward fp32 products of few token rows, such as the row-parallel partial
// in token-row chunks (the collective-matmul schedule: the GEMM2 shard of
// Llama-3-70B in 4 or 8 chunks of 1024 or 512 tokens has 128 or 64 large
// tiles per chunk, half or a quarter of the CUs): NN mid tiles of 128 x 256
// or 128 x 128 give each chunk one full wave over its whole K instead of a
// K split. They are taken only when they fill at least 7/8 of the CUs (the
// QKV forward, 160 tiles of 128 x 256, keeps its split).
#ifndef TPS_MID_NN
#define TPS_MID_NN 1
#endif
template <int TM_, int TN_, int SB_>
struct MidNN {  // 4 waves; A in 64-row stages of 16 KB, B in 32-row stages
    static constexpr int TM = TM_, TN = TN_, BKA = 64, SA = 4, BKB = 32, SB = SB_, WAVES_M = 2, WAVES_N = 2;
};
using MidNNWide = MidNN<128, 256, 6>;    // 4 x 16 KB + 6 x 16 KB
using MidNNNarrow = MidNN<128, 128, 8>;  // 4 x 16 KB + 8 x 8 KB

// The same for the NT fp32 products of few token rows, on the wide tile
// only: dX_part of the column-parallel backward in token-row chunks. The MLP
// shard's dX of Llama-3-70B in 4 chunks of 1024 tokens: 423-425 us against
// 472-475 us for the K split alone, 794-798 against 813-815 us followed by
// dW (three interleaved runs). 128 x 128 tiles for 8 chunks of 512 tokens
// were faster alone (534 against 548 us) but slower followed by dW (928
// against 918 us): those keep the split.
#ifndef TPS_MID_NT
#define TPS_MID_NT 1
#endif
struct MidNTWide {  // 4 waves; both operands in 64-row stages, 4 x 16 KB + 3 x 32 KB
    static constexpr int TM = 128, TN = 256, BKA = 64, SA = 4, BKB = 64, SB = 3, WAVES_M = 2, WAVES_N = 2;
};

// 0: no mid tile; 1: MidTile (TN), MidNNWide (NN) or MidNTWide (NT);
// 2: MidNNNarrow (NN).
template <bool A_T, bool B_KN, int EPI>
inline int mid_tile_choice(int M, int N, int K) {
    const long long cus = device_cus();
    const long long big = (long long)((M + 255) / 256) * ((N + 255) / 256);
    auto tiles = [&](int tm, int tn) { return (long long)((M + tm - 1) / tm) * ((N + tn - 1) / tn); };
    if (M < 256 || K < 2048 || 2 * big > cus) return 0;
    if constexpr (A_T && B_KN && (EPI == EPI_F32 || EPI == EPI_BF16)) {
        using MT = MidTile<A_T, B_KN>;
        const long long mid = tiles(MT::TM, MT::TN);
        return 2 * mid > cus && mid <= cus ? 1 : 0;
    } else if constexpr (!A_T && EPI == EPI_F32 && (B_KN ? TPS_MID_NN != 0 : TPS_MID_NT != 0)) {
        // (the wide tiles have the same shape on both layouts)
        auto full = [&](long long t) { return 8 * t >= 7 * cus && t <= cus; };
        if (full(tiles(MidNNWide::TM, MidNNWide::TN))) return 1;
        if (B_KN && full(tiles(MidNNNarrow::TM, MidNNNarrow::TN))) return 2;
        return 0;
    } else {
        return 0;
    }
}

static_assert(MidNTWide::TM == MidNNWide::TM && MidNTWide::TN == MidNNWide::TN,
              "mid_tile_choice counts the NN wide tile shape for both layouts");

template <bool A_T, bool B_KN, int EPI>
inline bool use_mid_tile(int M, int N, int K) {
    return mid_tile_choice<A_T, B_KN, EPI>(M, N, K) != 0;
}

}  // namespace tps

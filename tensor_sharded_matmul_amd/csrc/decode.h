// decode.h — plan and arguments of the decode-sized forward products
// (C[M, N] = A[M, K] B[K, N] with at most 32 token rows), shared by the host
// dispatch (tpshard.hip) and the kernel (gemm_decode.hip).
//
// At decode the token rows are few and the product is bound by streaming the
// weight B from HBM once (r00kie-liu, "Scaling Book 入门第 5 章：Sharded
// Matrices 上篇 — 集合通信原语", §5.7, its Mini-SGLang practice note: at
// decode, what tensor parallelism buys a card is fewer weight bytes to load).
// The weight is cut into slabs of product columns (64: one 128-byte line of
// every k-row) and, when the slabs alone do not fill the CUs, K into a few
// splits; each workgroup issues every load of its share (up to about 100 KB
// of B) before its first MFMA, so that one CU keeps its whole share in
// flight. A product with more than one split writes fp32 partials that the
// split reduction (a second kernel) sums.
#pragma once

#include <stdint.h>

#include <algorithm>

namespace tps {

// Product columns per slab (SwiGLU: half gate, half up): 64 columns are one
// 128-byte line of every weight row; 32-column slabs run in pairs that share
// their lines (see gemm_decode.hip).
constexpr int kDecWaves = 8;   // waves per workgroup; wave w takes k-blocks w, w + 8, ...
constexpr int kDecMaxRows = 32;
constexpr int kDecLdsBudget = 144 * 1024;

// k-blocks of 32 rows one wave keeps in flight (LDS: MT rows of A and 32
// k-rows of the SC-column slab per block)
constexpr int dec_blocks_per_wave(int MT, int SC) { return kDecLdsBudget / (kDecWaves * (MT * 64 + SC * 64)); }
// A token tile fits when a wave keeps a block in flight and its slots can
// hold its MT x SC f32 sums at the end.
constexpr bool dec_tile_fits(int MT, int SC) {
    return dec_blocks_per_wave(MT, SC) >= 1 && dec_blocks_per_wave(MT, SC) * (MT * 64 + SC * 64) >= MT * SC * 4;
}

struct DecodeArgs {
    const uint16_t* A;  // [M][lda] bf16, K-contiguous
    const uint16_t* B;  // [K][ldb] bf16, N-contiguous
    void* C;            // split products: the fp32 partials [nsplit][M][ldc] (workspace)
    uint16_t* out;      // bf16 output [M][ldo] (BF16, GELU, SWIGLU)
    float* out_f32;     // fp32 output [M][ldo] (F32)
    uint16_t* C2;       // saved pre-activation (GeLU, SwiGLU), or NULL
    int M, K, lda, ldb;
    int ldc;            // pitch of the partials: the product's columns Nw
    int ldo, ldc2;
    int f;              // SwiGLU: output columns (B holds gate f | up f)
    int nslab, nsplit, nkb;
    int accumulate;     // fp32 output: C += product
};

struct DecodePlan {
    int nslab = 0;   // 0: not run by the decode kernel
    int sc = 0;      // slab width (product columns)
    int nsplit = 0;
    int nkb = 0;
    size_t bytes = 0;  // workspace: the split partials
};

// The plan with SC-column slabs, or nslab = 0 when its slab x split
// workgroups do not fit in one wave over the CUs.
inline DecodePlan decode_plan_sc(int M, int K, int Nw, int ldb, int cus, int SC) {
    DecodePlan p;
    if (M < 1 || M > kDecMaxRows || K < 32 || K % 32 != 0 || Nw % SC != 0) return p;
    const int mt = M <= 16 ? 16 : 32;
    if (!dec_tile_fits(mt, SC)) return p;
    const int max_blocks = kDecWaves * dec_blocks_per_wave(mt, SC);
    // 32-bit byte offsets of the B rows one workgroup reads
    if ((int64_t)max_blocks * 32 * ldb * 2 >= ((int64_t)1 << 31)) return p;
    const int nslab = Nw / SC, nkb = K / 32;
    int nsplit = (nkb + max_blocks - 1) / max_blocks;
    if ((int64_t)nslab * nsplit > cus) return p;
    // more splits while they fill CUs, each keeping a block per wave
    nsplit = std::max(nsplit, std::min(cus / nslab, nkb / kDecWaves));
    p.nslab = nslab;
    p.sc = SC;
    p.nsplit = nsplit;
    p.nkb = nkb;
    if (nsplit > 1) p.bytes = (size_t)nsplit * M * Nw * sizeof(float);
    return p;
}

// Whether (and how) the decode kernel runs a forward product of M token rows,
// contraction K and Nw product columns whose weight pitch is ldb elements:
// 32-column slabs when they need no K split (no partials to sum), else
// 64-column slabs (whole lines; a 32-column plan would need as many
// workgroups or more).
inline DecodePlan decode_plan(int M, int K, int Nw, int ldb, int cus) {
    const DecodePlan p32 = decode_plan_sc(M, K, Nw, ldb, cus, 32);
    if (p32.nslab > 0 && p32.nsplit == 1) return p32;
    return decode_plan_sc(M, K, Nw, ldb, cus, 64);
}

}  // namespace tps

// gemm_launch.h — tile-shape selection and launch of the GEMM kernel for the
// host entry points of libtpshard.so. Each gemm_*.hip source instantiates
// launch_gemm for one operand layout and family of epilogues, so that the
// kernel variants compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/tpshard.h"
#include "gemm_kernel.h"
#include "mid_tile.h"

namespace tps {
// Products of one K split whose operand windows are below 2^31 bytes run the
// ping-pong schedule (8 waves, the two of a SIMD alternating between MFMAs
// and memory work) on the large tiles.
#ifndef TPS_PP
#define TPS_PP 1
#endif

// Records a formatted message for tp_last_error and returns st.
tp_status fail(tp_status st, const char* fmt, ...);

// Does an MN-contiguous operand's window (its K rows plus the stages loaded
// past the end, times its pitch) reach 2^31 bytes? Then the kernel moves its
// descriptor along K (the WIDE variant).
inline bool mn_window_wide(bool mn, int64_t K, int64_t ld) {
    return mn && (K + 512) * ld * 2 >= ((int64_t)1 << 31);
}

template <class CF, bool A_T, bool B_KN, int EPI>
inline tp_status launch_cfg(const char* fn, const GemmArgs& a, hipStream_t s);

// The ping-pong configuration PPC when the product allows it (no WIDE
// window, no fp32 accumulation into C; a K split's fp32 partials are plain
// stores), else the interleaved one CF. The QKV forward's 3-split partials
// of Llama-3-70B at t = 8 measured 90.3-90.9 us on it against 93.1-95.1 us
// on the interleaved kernel.
template <class CF, class PPC, bool A_T, bool B_KN, int EPI>
inline tp_status launch_pp_or(const char* fn, const GemmArgs& a, hipStream_t s) {
    // forward (NN) products only: on the backward layouts the ping-pong
    // kernels measured 2-5 % slower (NT: the 160 KB ring leaves group 1's
    // share of a stage one sub-step to land; TN: lower MFMA busy at the
    // same clock)
    if constexpr (TPS_PP != 0 && !A_T && B_KN) {
        bool wide = false;
        if constexpr (A_T || B_KN)
            wide = mn_window_wide(A_T, a.K, a.lda) || mn_window_wide(B_KN, a.K, a.ldb);
        // (an fp32 product that adds into C runs the interleaved kernel: the
        // ping-pong one stores its accumulators as they are)
        const bool adds = EPI == EPI_F32 && a.accumulate;
        if ((a.ksplit == 1 || TPS_PP_SPLIT != 0) && !wide && !adds) return launch_cfg<PPC, A_T, B_KN, EPI>(fn, a, s);
    }
    return launch_cfg<CF, A_T, B_KN, EPI>(fn, a, s);
}

template <class CF, bool A_T, bool B_KN, int EPI>
inline tp_status launch_cfg(const char* fn, const GemmArgs& a, hipStream_t s) {
    constexpr int TNZ = EPI == EPI_SWIGLU ? CF::TN / 2 : CF::TN;
    const long long tiles = (long long)((a.M + CF::TM - 1) / CF::TM) * ((a.N + TNZ - 1) / TNZ) * a.ksplit;
    if (tiles == 0) return TP_OK;
    if (tiles > 0x7fffffffLL) return fail(TP_ERR_UNSUPPORTED, "%s: too many tiles", fn);
    const dim3 grid((unsigned)tiles), block(64 * CF::WAVES_M * CF::WAVES_N);
    bool wide = false;
    if constexpr (A_T || B_KN)
        wide = mn_window_wide(A_T, a.K, a.lda) || mn_window_wide(B_KN, a.K, a.ldb);
    if (wide) {
        if constexpr ((A_T || B_KN) && !CF::PP)
            hipLaunchKernelGGL((gemm_kernel<CF, A_T, B_KN, EPI, true>), grid, block, 0, s, a);
    } else {
        hipLaunchKernelGGL((gemm_kernel<CF, A_T, B_KN, EPI, false>), grid, block, 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return TP_OK;
}

#ifndef TPS_DEC_SB
#define TPS_DEC_SB 8  // stages of the weight ring of the decode tiles
#endif

// Operands of any size are addressed from 64-bit descriptor bases (a tile's
// first row; a workgroup's first k-row). The 32-bit per-lane offsets then
// span one tile of a K-contiguous operand (256 rows of its pitch) or one
// stage of an MN-contiguous one (the WIDE variant) or its whole window, which
// bounds the pitches (elements) so that every offset stays below 2^31.
static constexpr int64_t kMaxKPitch = (int64_t)1 << 21;
static constexpr int64_t kMaxMNPitch = (int64_t)1 << 23;

// LDS rings per operand layout: K-contiguous operands in stages of 64 k-rows
// (a tile row is one whole 128-byte line), MN-contiguous ones in 32-row
// stages. Depths are the fastest measured on MI355X for the Llama-3-70B
// shard products. NT fills the 160 KB of LDS with a third B stage (dX and
// dZ products 2-3 % faster than with two); for NN and TN a deeper ring or
// the full LDS did not help.
template <bool A_T, bool B_KN>
struct Rings;
#ifndef TPS_NN_RING
#define TPS_NN_RING 64, 2, 32, 4
#endif
#ifndef TPS_NT_RING
#define TPS_NT_RING 64, 2, 64, 3
#endif
#ifndef TPS_TN_RING
#define TPS_TN_RING 32, 4, 32, 3
#endif
template <int BKA_, int SA_, int BKB_, int SB_>
struct RingOf {
    static constexpr int BKA = BKA_, SA = SA_, BKB = BKB_, SB = SB_;
};
template <>
struct Rings<false, true> : RingOf<TPS_NN_RING> {};   // NN: A K-contiguous, B MN-contiguous (128 KB)
template <>
struct Rings<false, false> : RingOf<TPS_NT_RING> {};  // NT: both K-contiguous (160 KB)
template <>
struct Rings<true, true> : RingOf<TPS_TN_RING> {};    // TN: both MN-contiguous (106 KB)

template <bool A_T, bool B_KN, int BM, int BN, int TM, int TN, int WVM, int WVN>
using CfgOf = Cfg<BM, BN, TM, TN, Rings<A_T, B_KN>::BKA, Rings<A_T, B_KN>::SA, Rings<A_T, B_KN>::BKB,
                  Rings<A_T, B_KN>::SB, WVM, WVN>;

// Rings of the ping-pong schedule. The share of a stage that group 1 loads
// is issued one phase after group 0's, so a ring of two 64-row stages leaves
// it one sub-step to land; NN and TN take a deeper ring (NN fills the LDS),
// NT is already full at 160 KB.
template <bool A_T, bool B_KN>
struct RingsPP;
#ifndef TPS_PP_NN_RING
#define TPS_PP_NN_RING 64, 3, 32, 4
#endif
#ifndef TPS_PP_NT_RING
#define TPS_PP_NT_RING 64, 2, 64, 3
#endif
#ifndef TPS_PP_TN_RING
#define TPS_PP_TN_RING 32, 4, 32, 4
#endif
template <>
struct RingsPP<false, true> : RingOf<TPS_PP_NN_RING> {};   // 160 KB
template <>
struct RingsPP<false, false> : RingOf<TPS_PP_NT_RING> {};  // 160 KB
template <>
struct RingsPP<true, true> : RingOf<TPS_PP_TN_RING> {};    // 128 KB

template <bool A_T, bool B_KN, int BM, int BN, int TM, int TN, int WVM, int WVN>
using CfgPP = Cfg<BM, BN, TM, TN, RingsPP<A_T, B_KN>::BKA, RingsPP<A_T, B_KN>::SA, RingsPP<A_T, B_KN>::BKB,
                  RingsPP<A_T, B_KN>::SB, WVM, WVN, true>;


enum Shape { SHAPE_SQ, SHAPE_N224, SHAPE_M224, SHAPE_N160 };

// Tile shape with the fewest waves of workgroups (ksplit per tile) times
// tile area, i.e. the least padded work per CU. 256 x 160 tiles (weight
// gradients only) fill the 256 CUs with the 1280-wide QKV shard of
// Llama-3-70B at t = 8 (32 x 8 tiles against 32 x 6 of 256 x 224). The
// SwiGLU forward always takes 256 x 256 tiles (128 gate + 128 up columns,
// both halves in every wave; a 256 x 224 tile has 112 + 112 and never needs
// fewer waves): on the Llama-3-70B GEMM1, 448 tiles against 512 in two
// waves, measured 4.6 % faster than 256 x 224 tiles with gate and up in
// separate waves (0.344 against 0.361 ms, interleaved runs). The other
// products keep the area rule (256 x 256 on the same wave count measured
// 1-10 % slower for dZ and the weight gradients).
inline Shape pick_shape(int M, int Nout, bool swiglu, bool allow_m224, int ksplit, bool allow_n160 = false) {
    if (swiglu) return SHAPE_SQ;
    const long long cus = device_cus();
    auto cost = [&](int tm, int tnz, int area) {
        const long long t = (long long)((M + tm - 1) / tm) * ((Nout + tnz - 1) / tnz) * ksplit;
        return ((t + cus - 1) / cus) * area;
    };
    Shape best = SHAPE_SQ;
    long long c_best = cost(256, 256, 256 * 256);
    const long long c_n = cost(256, 224, 256 * 224);
    if (c_n < c_best) { best = SHAPE_N224; c_best = c_n; }
    if (allow_m224) {
        const long long c_m = cost(224, 256, 224 * 256);
        if (c_m < c_best) { best = SHAPE_M224; c_best = c_m; }
    }
    if (allow_n160) {
        const long long c_n160 = cost(256, 160, 256 * 160);
        if (c_n160 < c_best) { best = SHAPE_N160; c_best = c_n160; }
    }
    return best;
}

// Every other product: the tile shape and ring for its layout and size.
template <bool A_T, bool B_KN, int EPI>
tp_status launch_by_shape(const char* fn, const GemmArgs& a, hipStream_t s) {
    constexpr bool SW = (EPI == EPI_SWIGLU);
    // Weight-gradient (TN) products run 8 waves, two per SIMD (128 x 64 or
    // 64 x 112 accumulator blocks): their two transposing LDS reads per
    // fragment leave gaps the second wave fills (+2 % measured). So does the
    // NT 256 x 224 tile (the SwiGLU' dZ product: +4 %); the other NN and NT
    // tiles are as fast or faster with 4 waves.
    constexpr int WM_SQ = 2, WN_SQ = A_T ? 4 : 2;
    using Sq = CfgOf<A_T, B_KN, 256, 256, 256, 256, WM_SQ, WN_SQ>;
    using N224 = CfgOf<A_T, B_KN, 256, 256, 256, 224, (A_T || !B_KN) ? 4 : 2, 2>;
    using M224 = CfgOf<A_T, B_KN, 256, 256, 224, 256, 2, A_T ? 4 : 2>;
    if constexpr (!A_T && B_KN && EPI == EPI_F32) {
        // split-K partials of a product with few token rows (decode): the
        // weight streams from HBM through a deep ring of 32-row stages, and
        // the token tile is no taller than the rows there are
        using Dec16 = Cfg<16, 128, 16, 128, 64, 4, 32, TPS_DEC_SB, 1, 2>;
        using Dec32 = Cfg<32, 128, 32, 128, 64, 4, 32, TPS_DEC_SB, 1, 2>;
        if (a.ksplit > 1 && a.M <= 16) return launch_cfg<Dec16, A_T, B_KN, EPI>(fn, a, s);
        if (a.ksplit > 1 && a.M <= 32) return launch_cfg<Dec32, A_T, B_KN, EPI>(fn, a, s);
    }
    if constexpr (!A_T) {
        // few token rows: 64 x 128 tiles, a smaller ring of the same shape
        using Small = Cfg<64, 128, 64, 128, 64, 3, Rings<A_T, B_KN>::BKB, B_KN ? 4 : 3, 2, 2>;
        if (a.M < 256) return launch_cfg<Small, A_T, B_KN, EPI>(fn, a, s);
    }
    if constexpr (MidTile<A_T, B_KN>::kOn && (EPI == EPI_F32 || EPI == EPI_BF16)) {
        if (a.ksplit == 1 && use_mid_tile<A_T, B_KN, EPI>(a.M, a.N, a.K)) {
            using MT = MidTile<A_T, B_KN>;
            using Mid = Cfg<MT::TM, MT::TN, MT::TM, MT::TN, MT::BKA, MT::SA, MT::BKB, MT::SB, MT::WAVES_M, MT::WAVES_N>;
            return launch_cfg<Mid, A_T, B_KN, EPI>(fn, a, s);
        }
    }
    if constexpr (!A_T && EPI == EPI_F32) {
        if (a.ksplit == 1) {
            auto run = [&](auto mc) {
                using MT = decltype(mc);
                using Mid = Cfg<MT::TM, MT::TN, MT::TM, MT::TN, MT::BKA, MT::SA, MT::BKB, MT::SB, MT::WAVES_M,
                                MT::WAVES_N>;
                return launch_cfg<Mid, A_T, B_KN, EPI>(fn, a, s);
            };
            using Wide = typename std::conditional<B_KN, MidNNWide, MidNTWide>::type;
            switch (mid_tile_choice<A_T, B_KN, EPI>(a.M, a.N, a.K)) {
                case 1: return run(Wide{});
                case 2:
                    if constexpr (B_KN) return run(MidNNNarrow{});
                    break;
                default: break;
            }
        }
    }
    // ping-pong forms: 8 waves, 128 x 64 (2 x 4) or 64 x 112 / 112 x 64
    using PSq = CfgPP<A_T, B_KN, 256, 256, 256, 256, 2, 4>;
    using PN224 = CfgPP<A_T, B_KN, 256, 256, 256, 224, 4, 2>;
    using PM224 = CfgPP<A_T, B_KN, 256, 256, 224, 256, 2, 4>;
    constexpr bool TN_F32 = A_T && B_KN && EPI == EPI_F32;
    switch (pick_shape(a.M, a.N, SW, true, a.ksplit, TN_F32)) {
        case SHAPE_N160:
            if constexpr (TN_F32) {
                // 8 waves of 64 x 80; loads stay 256 columns wide
                using N160 = CfgOf<A_T, B_KN, 256, 256, 256, 160, 4, 2>;
                return launch_cfg<N160, A_T, B_KN, EPI>(fn, a, s);
            }
            return launch_pp_or<Sq, PSq, A_T, B_KN, EPI>(fn, a, s);
        case SHAPE_N224:
            if constexpr (!SW) return launch_pp_or<N224, PN224, A_T, B_KN, EPI>(fn, a, s);
            else return launch_pp_or<Sq, PSq, A_T, B_KN, EPI>(fn, a, s);
        case SHAPE_M224:
            if constexpr (!SW) return launch_pp_or<M224, PM224, A_T, B_KN, EPI>(fn, a, s);
            else return launch_pp_or<Sq, PSq, A_T, B_KN, EPI>(fn, a, s);
        default:
            return launch_pp_or<Sq, PSq, A_T, B_KN, EPI>(fn, a, s);
    }
}


template <bool A_T, bool B_KN, int EPI>
tp_status launch_gemm(const char* fn, GemmArgs a, hipStream_t s) {
    if (a.M == 0 || a.N == 0) return TP_OK;
    if (a.lda > (A_T ? kMaxMNPitch : kMaxKPitch) || a.ldb > (B_KN ? kMaxMNPitch : kMaxKPitch))
        return fail(TP_ERR_UNSUPPORTED, "%s: an operand's row pitch is too large", fn);
    a.a_bytes = (uint64_t)(A_T ? a.K : a.M) * (uint64_t)a.lda * 2u;
    a.b_bytes = (uint64_t)(B_KN ? a.K : a.N) * (uint64_t)a.ldb * 2u;
    if constexpr (EPI == EPI_CE_STATS) {
        // one record per row for each wave column block: the host sizes its
        // record buffer for the shape ce_parts names (the interleaved
        // 256 x 256 tile of 4 waves would spill a register)
        static_assert(!A_T && B_KN, "the statistics GEMM is a forward (NN) product");
        if (ce_stats_pingpong(a.K, a.ldb)) {
            using PSq = CfgPP<A_T, B_KN, 256, 256, 256, 256, 2, 4>;
            return launch_cfg<PSq, A_T, B_KN, EPI>(fn, a, s);
        }
        using N224 = CfgOf<A_T, B_KN, 256, 256, 256, 224, 2, 2>;
        return launch_cfg<N224, A_T, B_KN, EPI>(fn, a, s);
    } else {
        return launch_by_shape<A_T, B_KN, EPI>(fn, a, s);
    }
}

}  // namespace tps

#define TPS_INSTANTIATE_GEMM(A_T, B_KN, EPI) \
    template tp_status tps::launch_gemm<A_T, B_KN, EPI>(const char*, tps::GemmArgs, hipStream_t);

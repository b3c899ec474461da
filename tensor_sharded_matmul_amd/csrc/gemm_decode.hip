// gemm_decode.hip — the decode-sized forward products (at most 32 token
// rows): C = A B streamed slab by slab, with the column-parallel epilogues
// ([TPSP] "矩阵乘法的两种切法" for the product, "MLP：先列后行，只通信一次"
// for GeLU and SiLU(gate) * up) or fp32 partials for the split reduction.
//
// Workgroup (slab, split): 8 waves; the split's k-blocks of 32 rows are dealt
// round-robin to the waves. Each wave first issues the LDS-DMA loads of all
// of its blocks (MT token rows of A, 32 k-rows x the slab's columns of B,
// whole 128-byte lines of every weight row), then computes each block as it
// lands (vmcnt counts down in issue order), accumulating MT x slab in f32 with
// v_mfma_f32_16x16x32_bf16. No barrier until the end, where the 8 waves'
// accumulators are summed through LDS in wave order and the epilogue stores
// the slab. B fragments are read with ds_read_b64_tr_b16 (4 consecutive k of
// one column per read), A fragments with 16-byte reads; the operands are
// swapped in the MFMA so that each lane holds 4 consecutive columns of a row.
#include "decode.h"
#include "gemm_launch.h"

namespace tps {

template <int MT, int SC_>
struct DecGeom {
    static constexpr int SC = SC_;
    static constexpr int R = dec_blocks_per_wave(MT, SC);  // k-blocks per wave at most
    static constexpr int AB = MT * 64;                 // A bytes of a k-block: [MT][32] bf16
    static constexpr int BB = SC * 64;                 // B bytes of a k-block: [32][SC] bf16
    static constexpr int SLOT = AB + BB;
    static constexpr int WAVE_LDS = R * SLOT;
    static constexpr int LDS = kDecWaves * WAVE_LDS;
    static constexpr int CPR = SC / 8;     // 16-byte chunks of a B row
    static constexpr int RPI = 64 / CPR;   // B rows per load (1 KB)
    static constexpr int BI = BB / 1024;   // B loads per k-block
    static constexpr int NJ = SC / 16;     // 16-column MFMA blocks
    static constexpr int L = MT / 16 + BI; // LDS-DMA loads per k-block
    static_assert(R >= 1 && L * R <= 63, "a wave's loads must fit the vmcnt counter");
    static_assert(LDS <= 160 * 1024, "LDS");
    static_assert(WAVE_LDS >= MT * SC * 4, "a wave's slots hold its accumulators at the end");
};

// Workgroup -> (slab, split). 32-column slabs run unsplit, and two
// neighbouring slabs share every 128-byte line of the weight: slabs 16q + 2x
// and 16q + 2x + 1 go to workgroups b = 16q + x and b + 8, which the hardware
// (dealing workgroups round-robin over the 8 XCDs) places on the same XCD, so
// that the line is fetched into that XCD's L2 once (measured: the 16-token
// W_O product of Llama-3-70B at t = 8, 256 slabs, 7.6 us unpaired, 5.7 us
// paired). A tail of fewer than 16 slabs keeps the plain order.
template <int SC>
__device__ __forceinline__ void dec_unit(int b, int nslab, int nsplit, int& slab, int& split) {
    if (SC == 32 && nsplit == 1 && b < nslab / 16 * 16) {
        const int i = b >> 3;
        slab = 16 * (i >> 1) + 2 * (b & 7) + (i & 1);
        split = 0;
    } else {
        slab = b / nsplit;
        split = b % nsplit;
    }
}

// MODE 0: one split, the epilogue EPI stores the output; MODE 1: fp32
// partials to the workspace, for the split reduction. SWCOLS: the slab's SC
// B columns are SC/2 gate columns j0.. and the SC/2 up columns f + j0..
// (SwiGLU), and an fp32 output (the split partials) goes to those same
// columns; otherwise slab s is columns SC s .. SC s + SC - 1.
template <int MT, int SC, int EPI, bool SWCOLS, int MODE>
__global__ void __launch_bounds__(64 * kDecWaves) decode_nn_kernel(DecodeArgs d) {
    using G = DecGeom<MT, SC>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[G::LDS];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int slab, split;
    dec_unit<SC>(blockIdx.x, d.nslab, d.nsplit, slab, split);
    // (split x nkb < 2^31: nkb <= 2^15 k-blocks, nsplit <= the CUs)
    const int kb0 = (int)((uint32_t)(split * d.nkb) / (uint32_t)d.nsplit);
    const int kb1 = (int)((uint32_t)((split + 1) * d.nkb) / (uint32_t)d.nsplit);
    const int nb = kb1 - kb0;
    const int nw = nb > wave ? (nb - wave + kDecWaves - 1) / kDecWaves : 0;  // this wave's blocks (<= R)
    const int j0 = slab * (SWCOLS ? SC / 2 : SC);

    // B: this lane's 16-byte chunk of each load is row lane / CPR (+ RPI per
    // load) at chunk lane % CPR; A: row lane / 4 (+ 16 per load), 8 k at
    // chunk lane % 4
    const int rb = lane / G::CPR, cb = lane % G::CPR;
    const int colB = SWCOLS ? (cb < G::CPR / 2 ? j0 + 8 * cb : d.f + j0 + 8 * (cb - G::CPR / 2)) : j0 + 8 * cb;
    const i32x4_t rsB = window_rsrc(d.B, (uint64_t)d.K * d.ldb * 2, (uint64_t)kb0 * 32 * d.ldb * 2);
    const i32x4_t rsA = window_rsrc(d.A, (uint64_t)d.M * d.lda * 2, (uint64_t)kb0 * 64);
    const uint32_t blk_B = 32u * (uint32_t)d.ldb * 2u * kDecWaves;  // B bytes between a wave's blocks
    const uint32_t inst_B = (uint32_t)G::RPI * (uint32_t)d.ldb * 2u;  // B bytes between a block's loads
    uint32_t offB = ((uint32_t)(wave * 32 + rb) * (uint32_t)d.ldb + (uint32_t)colB) * 2u;
    uint32_t offA[MT / 16];
    const int ra = lane >> 2, ca = lane & 3;
#pragma unroll
    for (int h = 0; h < MT / 16; ++h) {
        const int m = min(ra + 16 * h, d.M - 1);  // rows past M: any valid row (not stored)
        offA[h] = ((uint32_t)m * (uint32_t)d.lda + (uint32_t)(wave * 32 + 8 * ca)) * 2u;
    }
    const uint32_t lds_wave = lds_addr(lds) + (uint32_t)(wave * G::WAVE_LDS);

    // every load of this wave's blocks, in block order
    for (int t = 0; t < nw; ++t) {
        const uint32_t slot = lds_wave + (uint32_t)(t * G::SLOT);
#pragma unroll
        for (int h = 0; h < MT / 16; ++h) dma16(rsA, offA[h] + (uint32_t)t * (64u * kDecWaves), slot + 1024u * h);
#pragma unroll
        for (int i = 0; i < G::BI; ++i) dma16(rsB, offB + (uint32_t)i * inst_B, slot + G::AB + 1024u * i);
        offB += blk_B;
    }

    const int x = lane & 15, g = lane >> 4;
    f32x4_t acc[MT / 16][G::NJ];
    static_for<0, MT / 16>([&](auto ii) {
        static_for<0, G::NJ>([&](auto jj) {
            acc[decltype(ii)::value][decltype(jj)::value] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        });
    });
    // block t = nw - 1 - rem once at most rem blocks' loads are outstanding
    static_for<0, G::R>([&](auto ic) {
        constexpr int rem = G::R - 1 - decltype(ic)::value;
        if (rem < nw) {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(G::L * rem) : "memory");
            const uint32_t slot = lds_wave + (uint32_t)((nw - 1 - rem) * G::SLOT);
            bf16x8_t a[MT / 16];
            static_for<0, MT / 16>([&](auto ii) {
                constexpr int i = decltype(ii)::value;
                a[i] = lds_read16(slot + (uint32_t)((16 * i + x) * 64 + 16 * g));
            });
            static_for<0, G::NJ>([&](auto jj) {
                constexpr int j = decltype(jj)::value;
                const int k0 = 8 * g + (x >> 2), col = 16 * j + 4 * (x & 3);
                const bf16x8_t b = lds_read_tr2<SC>(slot + G::AB + (uint32_t)(k0 * SC * 2 + col * 2));
                static_for<0, MT / 16>([&](auto ii) {
                    constexpr int i = decltype(ii)::value;
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a[i], acc[i][j], 0, 0, 0);
                });
            });
        }
    });

    // lane (x, g) holds C[16 i + x][16 j + 4 g .. + 3]; each wave parks its
    // sums in its own (now idle) slots, then the waves' sums are added in
    // wave order
    typedef __attribute__((address_space(3))) f32x4_t lds_f32x4;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS reads are done
    static_for<0, MT / 16>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        static_for<0, G::NJ>([&](auto jj) {
            constexpr int j = decltype(jj)::value;
            const uint32_t o = lds_wave + (uint32_t)(((16 * i + x) * SC + 16 * j + 4 * g) * 4);
            *(lds_f32x4*)(uintptr_t)o = acc[i][j];
        });
    });
    __syncthreads();
    const uint32_t base = lds_addr(lds);
    auto sum_at = [&](int m, int col) {
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < kDecWaves; ++w)
            v += *(const lds_f32x4*)(uintptr_t)(base + (uint32_t)(w * G::WAVE_LDS + (m * SC + col) * 4));
        return v;
    };
    // partial column n (of the Nw product columns) of slab column c
    auto pcol = [&](int c) { return SWCOLS ? (c < SC / 2 ? j0 + c : d.f + j0 + c - SC / 2) : j0 + c; };
    if constexpr (MODE == 1) {
        // this split's partial: [split][M][Nw]
        float* part = static_cast<float*>(d.C);
        for (int t = threadIdx.x; t < MT * (SC / 4); t += 64 * kDecWaves) {
            const int m = t / (SC / 4), q = t % (SC / 4);
            if (m >= d.M) break;
            *reinterpret_cast<f32x4_t*>(part + ((size_t)split * d.M + m) * d.ldc + pcol(4 * q)) = sum_at(m, 4 * q);
        }
        return;
    }
    if constexpr (EPI == EPI_SWIGLU) {
        // row m, outputs j0 + 4 q .. + 3: gate at slab columns 4 q, up at SC/2 + 4 q
        for (int t = threadIdx.x; t < MT * (SC / 8); t += 64 * kDecWaves) {
            const int m = t / (SC / 8), q = t % (SC / 8);
            if (m >= d.M) break;
            const f32x4_t gt = sum_at(m, 4 * q), up = sum_at(m, SC / 2 + 4 * q);
            float z[4];
            for (int e = 0; e < 4; ++e) z[e] = gt[e] * sigmoid_f(gt[e]) * up[e];
            const int n = j0 + 4 * q;
            *reinterpret_cast<u32x2_t*>(d.out + (size_t)m * d.ldo + n) = pack4(z[0], z[1], z[2], z[3]);
            if (d.C2) {
                *reinterpret_cast<u32x2_t*>(d.C2 + (size_t)m * d.ldc2 + n) = pack4(gt[0], gt[1], gt[2], gt[3]);
                *reinterpret_cast<u32x2_t*>(d.C2 + (size_t)m * d.ldc2 + d.f + n) = pack4(up[0], up[1], up[2], up[3]);
            }
        }
    } else {
        // row m, output columns j0 + 4 q .. + 3
        for (int t = threadIdx.x; t < MT * (SC / 4); t += 64 * kDecWaves) {
            const int m = t / (SC / 4), q = t % (SC / 4);
            if (m >= d.M) break;
            const f32x4_t v = sum_at(m, 4 * q);
            const int n = j0 + 4 * q;
            if constexpr (EPI == EPI_F32) {
                f32x4_t* p = reinterpret_cast<f32x4_t*>(d.out_f32 + (size_t)m * d.ldo + n);
                *p = d.accumulate ? *p + v : v;
            } else if constexpr (EPI == EPI_BF16) {
                *reinterpret_cast<u32x2_t*>(d.out + (size_t)m * d.ldo + n) = pack4(v[0], v[1], v[2], v[3]);
            } else if constexpr (EPI == EPI_GELU) {
                *reinterpret_cast<u32x2_t*>(d.out + (size_t)m * d.ldo + n) =
                    pack4(gelu_f(v[0]), gelu_f(v[1]), gelu_f(v[2]), gelu_f(v[3]));
                if (d.C2) *reinterpret_cast<u32x2_t*>(d.C2 + (size_t)m * d.ldc2 + n) = pack4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

template <int MT, int SC, int EPI, bool SWCOLS, int MODE>
static tp_status launch_decode_mt(const char* fn, const DecodeArgs& d, hipStream_t s) {
    if constexpr (!dec_tile_fits(MT, SC)) {
        return fail(TP_ERR_UNSUPPORTED, "%s: no decode tile of %d rows and %d columns", fn, MT, SC);
    } else {
        const unsigned blocks = (unsigned)d.nslab * (unsigned)d.nsplit;
        hipLaunchKernelGGL((decode_nn_kernel<MT, SC, EPI, SWCOLS, MODE>), dim3(blocks), dim3(64 * kDecWaves), 0, s,
                           d);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
        return TP_OK;
    }
}

// 32-column slabs run unsplit only (decode_plan)
template <int EPI, bool SW, int MODE>
static tp_status launch_decode_mode(const char* fn, const DecodeArgs& d, int sc, hipStream_t s) {
    if constexpr (MODE == 0) {
        if (sc == 32)
            return d.M <= 16 ? launch_decode_mt<16, 32, EPI, SW, MODE>(fn, d, s)
                             : launch_decode_mt<32, 32, EPI, SW, MODE>(fn, d, s);
    }
    return d.M <= 16 ? launch_decode_mt<16, 64, EPI, SW, MODE>(fn, d, s)
                     : launch_decode_mt<32, 64, EPI, SW, MODE>(fn, d, s);
}

// The product a (NN, M <= 32 rows) as planned by decode_plan: with one split
// the epilogue EPI is applied here; with several, the splits' fp32 partials
// [nsplit][M][Nw] go to ws (Nw = product columns; SwiGLU: gate f | up f) for
// the split reduction the caller launches next.
template <int EPI>
tp_status launch_decode(const char* fn, const GemmArgs& a, const DecodePlan& p, void* ws, hipStream_t s) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    // what the kernel assumes of the plan: whole slabs, whole 32-row k-blocks,
    // at most dec_blocks_per_wave blocks per wave in every split
    const int Nw = SW ? 2 * a.N : a.N;
    const int mt = a.M <= 16 ? 16 : 32;
    if (a.M < 1 || a.M > kDecMaxRows || !(p.sc == 64 || (p.sc == 32 && p.nsplit == 1)) || p.nslab * p.sc != Nw ||
        p.nkb * 32 != a.K || p.nsplit < 1 || (p.nkb + p.nsplit - 1) / p.nsplit > kDecWaves * dec_blocks_per_wave(mt, p.sc))
        return fail(TP_ERR_UNSUPPORTED, "%s: decode plan does not fit the kernel", fn);
    DecodeArgs d;
    d.A = a.A;
    d.B = a.B;
    d.C = ws;
    d.out = static_cast<uint16_t*>(a.C);
    d.out_f32 = static_cast<float*>(a.C);
    d.C2 = a.C2;
    d.M = a.M;
    d.K = a.K;
    d.lda = a.lda;
    d.ldb = a.ldb;
    d.ldc = Nw;
    d.ldo = a.ldc;
    d.ldc2 = a.ldc2;
    d.f = a.f;
    d.nslab = p.nslab;
    d.nsplit = p.nsplit;
    d.nkb = p.nkb;
    d.accumulate = a.accumulate;
    if (p.nsplit == 1) return launch_decode_mode<EPI, SW, 0>(fn, d, p.sc, s);
    return launch_decode_mode<EPI_F32, SW, 1>(fn, d, p.sc, s);
}

template tp_status launch_decode<EPI_F32>(const char*, const GemmArgs&, const DecodePlan&, void*, hipStream_t);
template tp_status launch_decode<EPI_BF16>(const char*, const GemmArgs&, const DecodePlan&, void*, hipStream_t);
template tp_status launch_decode<EPI_GELU>(const char*, const GemmArgs&, const DecodePlan&, void*, hipStream_t);
template tp_status launch_decode<EPI_SWIGLU>(const char*, const GemmArgs&, const DecodePlan&, void*, hipStream_t);

}  // namespace tps

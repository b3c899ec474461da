// gemm_kernel.h — bf16 MFMA GEMM for gfx950 with the epilogues of a TP shard.
//
// One template computes C[M,N] = op(A) op(B) for the three operand layouts a
// tensor-parallel shard needs ([TPSP] "矩阵乘法的两种切法": forward Y = X W,
// backward dX = dY W^T and dW = X^T dY):
//   NN  A[M][K], B[K][N]   forward products
//   NT  A[M][K], B[N][K]   input gradients  (dY W^T)
//   TN  A[K][M], B[K][N]   weight gradients (X^T dY)
// and fuses the shard's elementwise work into the epilogue
// ([TPSP] "MLP：先列后行": GeLU and SiLU(gate)*up are local, per element).
//
// Design (gfx950 / CDNA4):
//  * WAVES_M x WAVES_N waves of 64 lanes (4, or 8 = two per SIMD), one
//    workgroup per CU. Each wave owns a (TM/WAVES_M) x (TN/WAVES_N) sub-tile
//    of C in f32 accumulators (AGPRs).
//  * v_mfma_f32_16x16x32_bf16. For the bf16 and fused epilogues the operands
//    are swapped (the MFMA "A" operand is the B tile), so each lane ends with
//    4 consecutive columns of one C row (8-byte bf16 stores, per-row
//    reductions within a lane). fp32 outputs keep the MFMA's own layout (a
//    lane holds one column of 4 rows): 16 consecutive lanes then store 64
//    contiguous bytes, which the CU's store path takes at 64 B per clock.
//  * Operand tiles go HBM -> LDS directly (buffer_load_dwordx4 ... lds: no
//    staging registers) into a ring of STAGES buffers of BK k-rows. A stage
//    is refilled as soon as its MFMA fragments are in registers, so STAGES-1
//    stages of loads are in flight while one is read. The loads are issued
//    from inline asm with explicit vmcnt waits (the compiler would otherwise
//    drain every LDS-DMA load before each barrier). Rows past K (and past
//    M / N) read as zero through the buffer descriptor's range check.
//  * Fragments are double-buffered in registers: the LDS reads of k-step
//    kt+1 are interleaved with the MFMAs of k-step kt (at issue slots fixed
//    at compile time and pinned with sched_barrier fences), so the matrix
//    core does not wait on LDS latency; one barrier per k-step.
//  * The loaded tile (BM x BN) may be wider than the computed one (TM x TN):
//    224-wide computed tiles divide the 3584 / 7168 widths of the Llama-3-70B
//    shard into a whole number of waves of 256 workgroups, while loads stay in
//    64-lane-aligned 256-wide rows.
//  * LDS layouts keep the operand as stored in HBM:
//      K-contiguous tile [rows][BK]: 16-byte chunk c of row r is stored at
//        c ^ swz(r), swz(r) = (r>>1)&7 (BK=64) or (r>>2)&3 (BK=32), so the 16
//        rows one MFMA fragment read touches fall in 16 distinct bank groups
//        (gfx950 LDS: 64 banks x 4 B).
//      MN-contiguous tile [BK][cols]: chunk c of k-row k at c ^ (2(k&3) +
//        8((k>>3)&1)); fragments are read with ds_read_b64_tr_b16, which
//        transposes 4x4 blocks of 16-bit values across each 16-lane group,
//        giving every lane 4 consecutive k of one column.
//    so the MFMA inner loop is the same for every layout.
//  * SwiGLU loads the B tile as [gate | up] halves over the same F indices;
//    every wave holds both halves of its output columns (EPI_SWIGLU).
//  * Workgroup -> tile mapping is XCD-aware: the hardware deals workgroups
//    round-robin over the 8 XCDs, so consecutive blocks of tiles are mapped
//    to one XCD (sharing its L2), grouped GROUP_M tile rows at a time.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace tps {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Compile-time loops. Register arrays (accumulators, fragments) are indexed
// only through these: an index that depends on whether the compiler chose to
// unroll a loop can demote a whole array to scratch memory, whose accesses
// would also upset the explicit vmcnt accounting of the LDS-DMA pipeline.
// ---------------------------------------------------------------------------
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

constexpr int kGroupM = 4;     // tile rows per L2 group
#ifndef TPS_PP_SPLIT
#define TPS_PP_SPLIT 1         // split-K partials of forward (NN) products on the ping-pong kernel
#endif
#ifndef TPS_F32_COLS
#define TPS_F32_COLS 1         // fp32 outputs stored from the MFMA's own layout
#endif

enum Epi : int {
    EPI_F32 = 0,        // C f32 = acc (or += acc)
    EPI_BF16 = 1,       // C bf16 = acc
    EPI_GELU = 2,       // C bf16 = GeLU(acc); C2 bf16 = acc (optional)
    EPI_SWIGLU = 3,     // C bf16 = SiLU(g)*u; C2 bf16 = [g | u] (optional)
    EPI_GELU_BWD = 4,   // C bf16 = acc * GeLU'(aux)
    EPI_SWIGLU_BWD = 5, // C bf16 = [acc*u*SiLU'(g) | acc*SiLU(g)], aux = [g|u]
    EPI_CE_STATS = 6,   // logits -> per (row, wave column block) {max, sum exp(z - max), z_target}
    EPI_CE_GRAD = 7,    // C bf16 = (exp(acc - m) / S - [col = target]) * dloss, per row
};

struct GemmArgs {
    const uint16_t* A;
    const uint16_t* B;
    void* C;
    uint16_t* C2;
    const uint16_t* aux;
    int M, N, K;     // C is M x N (SWIGLU: N = f, B has 2f columns)
    int lda, ldb;    // leading dims of A and B as stored (elements)
    int ldc, ldc2;   // leading dims of C and C2 / aux (elements)
    int f;           // SWIGLU / SWIGLU_BWD: column offset of the "up" half
    int accumulate;  // EPI_F32: add into C
    uint64_t a_bytes, b_bytes;  // extent of A and B in bytes (buffer range check)
    // Split-K: ksplit workgroups per output tile, each contracting kper rows
    // of K (a multiple of 64; the last split ends at K); split s writes its
    // fp32 partial to C + s * M * ldc. ksplit = 1: the whole K, C as given.
    int ksplit, kper;
    // Cross-entropy epilogues: per-row target vocab id (tgt), the vocab id of
    // column 0 (col0); EPI_CE_GRAD also the per-row max m (rm), sum S (rs)
    // and upstream gradient (rd). EPI_CE_STATS writes 3-float records to C,
    // ldc records per row.
    const int* tgt;
    const float *rm, *rs, *rd;
    int col0;
};

// The cross-entropy statistics GEMM writes one record per row for each
// wave column block of its tiles. It runs the ping-pong 256 x 256 tile (4
// wave column blocks of 64 columns) unless the weight's window reaches 2^31
// bytes (the WIDE variant, which the ping-pong kernel does not have): then
// 256 x 224 tiles of 2 x 2 waves (2 blocks of 112 columns). K = h, the
// weight's pitch ldb = v_loc.
#ifndef TPS_CE_PP
#define TPS_CE_PP 1
#endif
inline bool ce_stats_pingpong(int64_t K, int64_t ldb) {
    return TPS_CE_PP != 0 && (K + 512) * ldb * 2 < ((int64_t)1 << 31);
}
inline int ce_parts(int64_t K, int64_t v_loc) {
    return ce_stats_pingpong(K, v_loc) ? (int)(4 * ((v_loc + 255) / 256)) : (int)(2 * ((v_loc + 223) / 224));
}

// Token rows of the tile a split-K product of M rows runs with.
inline int splitk_tile_m(int M) { return M <= 16 ? 16 : M <= 32 ? 32 : 64; }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// erf from Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: for x >= 0, erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5))))
// exp(-x^2) with t = 1 / (1 + p x), absolute error at most 1.5e-7 (far below
// the 2^-9 relative rounding of the bf16 outputs); odd in x. Straight-line
// code: one reciprocal, one exponential, five multiply-adds.
__device__ __forceinline__ float erf_as(float x) {
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
    const float poly =
        t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    return copysignf(1.0f - poly * __expf(-ax * ax), x);
}

__device__ __forceinline__ float gelu_f(float x) {
    return 0.5f * x * (1.0f + erf_as(x * 0.70710678118654752f));
}

__device__ __forceinline__ float gelu_grad_f(float x) {
    const float cdf = 0.5f * (1.0f + erf_as(x * 0.70710678118654752f));
    const float pdf = 0.39894228040143268f * __expf(-0.5f * x * x);
    return cdf + x * pdf;
}

// 1 / (1 + e^-x) with the hardware reciprocal (1 ulp) instead of a division
__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// ---------------------------------------------------------------------------
// Buffer descriptor and the LDS-DMA load (16 bytes per lane; lane l writes
// LDS bytes [m0 + 16 l, m0 + 16 l + 16)).
// ---------------------------------------------------------------------------
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    i32x4_t r;
    r[0] = (int32_t)(uint32_t)p;
    r[1] = (int32_t)((uint32_t)(p >> 32) & 0xffffu);  // stride 0, no swizzle
    r[2] = (int32_t)bytes;                            // range-checked extent
    r[3] = 0x00020000;                                // gfx9 data format word
    return r;
}

// Descriptor of the part of an operand that starts `off` bytes into its
// `total`-byte extent: 64-bit base, so that the 32-bit per-lane offsets only
// span one tile (K-contiguous operands) or one stage (MN-contiguous ones)
// whatever the operand's size; the range checked is what remains of the
// extent, clamped to 32 bits (no offset reaches the clamp).
__device__ __forceinline__ i32x4_t window_rsrc(const uint16_t* base, uint64_t total, uint64_t off) {
    const uint64_t rest = off < total ? total - off : 0;
    return make_rsrc(reinterpret_cast<const uint8_t*>(base) + off,
                     rest > 0xffffffffull ? 0xffffffffu : (uint32_t)rest);
}

// The stage of an operand that is loaded next, and how to move to the one
// after it. Normally the descriptor stays and the per-lane k offset moves by
// a stage (k-rows x 2 bytes, K-contiguous; k-rows x pitch x 2 bytes,
// MN-contiguous). An MN-contiguous operand whose window spans 2^31 bytes or
// more (MOVE_BASE: K x pitch that large) instead moves the descriptor's base
// by a stage and shrinks the remaining extent, saturating at 0: scalar
// instructions only, issued right after the stage's last load, in the
// shadow of the MFMAs (about 1.5 % of the product's time, which is why it is
// not the default).
template <bool MOVE_BASE>
struct StageCursor {
    i32x4_t rs;          // descriptor of the next stage
    uint32_t ko;         // its per-lane k offset (K-contiguous operand)
    uint32_t step_lo, step_hi;
    uint64_t base;       // MN: first byte of the next stage
    uint32_t rest_lo, rest_hi;  // MN: bytes of the extent from base on

    __device__ __forceinline__ void init(const uint16_t* p, uint64_t total, uint64_t org, uint64_t step) {
        rs = window_rsrc(p, total, org);
        ko = 0;
        step_lo = (uint32_t)step;
        step_hi = (uint32_t)(step >> 32);
        base = reinterpret_cast<uint64_t>(p) + org;
        const uint64_t rest = org < total ? total - org : 0;
        rest_lo = (uint32_t)rest;
        rest_hi = (uint32_t)(rest >> 32);
    }
    __device__ __forceinline__ void next() {
        if constexpr (MOVE_BASE) {
            base += ((uint64_t)step_hi << 32) | step_lo;
            asm volatile(
                "s_sub_u32 %0, %0, %2\n\t"
                "s_subb_u32 %1, %1, %3\n\t"
                "s_cselect_b32 %0, 0, %0\n\t"
                "s_cselect_b32 %1, 0, %1"
                : "+s"(rest_lo), "+s"(rest_hi)
                : "s"(step_lo), "s"(step_hi)
                : "scc");
            rs[0] = (int32_t)(uint32_t)base;
            rs[1] = (int32_t)((uint32_t)(base >> 32) & 0xffffu);
            rs[2] = (int32_t)(rest_hi != 0 ? 0xffffffffu : rest_lo);
        } else {
            ko += step_lo;
        }
    }
};

__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t voff, uint32_t lds_base) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base)
                 : "memory");
}

// Wait until at most N of this wave's LDS-DMA loads are outstanding and its LDS
// reads are done, then barrier: afterwards every wave's loads of the stage the
// wait covers are in LDS, and no wave still reads a stage about to be refilled.
// The LDS-read drain is issued as a builtin so that the compiler's own wait
// tracking knows every LDS read is complete after it (an asm wait is opaque to
// it and it would then stall on reads issued after the barrier).
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ bf16x8_t lds_read16(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>((uintptr_t)addr);
}

// One 16x32 MFMA operand block from an MN-contiguous tile of C columns: two
// ds_read_b64_tr_b16, the second 4 k-rows further on (the swizzle of k-row
// k + 4 equals that of k for the rows a fragment touches, see mntile_frag_addr).
template <int C>
__device__ __forceinline__ bf16x8_t lds_read_tr2(uint32_t addr) {
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)addr);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)(addr + 4 * C * 2));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// swizzles (see the header comment)
template <int BK>
__device__ __forceinline__ int swz_k(int row) {
    return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
__device__ __forceinline__ int swz_mn(int k) {
    return 2 * (k & 3) + 8 * ((k >> 3) & 1);
}

struct IdentityCols {
    int col0, cols_total;
    __device__ __forceinline__ int operator()(int c) const {
        const int g = col0 + c;
        return g < cols_total ? g : 0;  // columns past the edge: any valid column
    }
};

// SwiGLU B tile of HALF + HALF loaded columns: the first half holds gate
// columns z0 .. z0+HALF-1, the second the up columns of the same F indices.
template <int HALF>
struct SwigluCols {
    int z0, f;
    __device__ __forceinline__ int operator()(int c) const {
        const int p = c % HALF;
        const int j = z0 + p;
        if (j >= f) return 0;  // outputs past f are never stored
        return c < HALF ? j : f + j;
    }
};

// ---------------------------------------------------------------------------
// Per-lane DMA offsets of one operand tile (bytes, relative to the matrix).
// ---------------------------------------------------------------------------

// Keep a loop-invariant 32-bit value in one VGPR. Without this the compiler
// forms such offsets with a 64-bit multiply-add, keeps both halves live across
// the k-loop and spills them; a spill reload inside the loop waits for every
// outstanding LDS-DMA load.
__device__ __forceinline__ void pin32(uint32_t& v) { asm volatile("" : "+v"(v)); }


// K-contiguous operand [rows][K]: tile [R][BK].
template <int R, int BK, int NWAVES>
struct KTileDma {
    static constexpr int kCpr = BK / 8;              // 16-byte chunks per row
    static constexpr int kRpi = 64 / kCpr;           // rows per 1 KB instruction
    static constexpr int kInst = R * kCpr / 64;      // instructions per tile
    static constexpr int kPerWave = kInst / NWAVES;
    static_assert(kInst % NWAVES == 0, "tile rows must split evenly over the waves");
    uint32_t off[kPerWave];

    __device__ __forceinline__ void init(int wave, int lane, int row0, int ld) {
        static_for<0, kPerWave>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const int I = wave * kPerWave + i;
            const int row = I * kRpi + lane / kCpr;
            const int c = (lane % kCpr) ^ swz_k<BK>(row);
            off[i] = (uint32_t)(row0 + row) * (uint32_t)ld * 2u + (uint32_t)c * 16u;
            pin32(off[i]);
        });
    }
    // load i of this wave's share of the tile (1 KB of LDS per load)
    __device__ __forceinline__ void issue_one(int i, i32x4_t rsrc, uint32_t lds_tile, int wave,
                                              uint32_t kbytes) const {
        dma16(rsrc, off[i] + kbytes, lds_tile + (uint32_t)(wave * kPerWave + i) * 1024u);
    }
};

// MN-contiguous operand [K][cols]: tile [BK][C].
template <int C, int BK, int NWAVES>
struct MNTileDma {
    static constexpr int kCpr = C / 8;
    static constexpr int kRpi = 64 / kCpr;
    static constexpr int kInst = BK * kCpr / 64;
    static constexpr int kPerWave = kInst / NWAVES;
    static_assert(kCpr >= 16 && 64 % kCpr == 0, "MN tile needs 128..512 columns");
    static_assert(kInst % NWAVES == 0, "tile must split evenly over the waves");
    uint32_t off[kPerWave];

    template <class ColMap>
    __device__ __forceinline__ void init(int wave, int lane, int ld, const ColMap& colmap) {
        static_for<0, kPerWave>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const int I = wave * kPerWave + i;
            const int k = I * kRpi + lane / kCpr;
            const int c = (lane % kCpr) ^ swz_mn(k);
            off[i] = (uint32_t)k * (uint32_t)ld * 2u + (uint32_t)colmap(c * 8) * 2u;
            pin32(off[i]);
        });
    }
    // load i of this wave's share of the tile (1 KB of LDS per load)
    __device__ __forceinline__ void issue_one(int i, i32x4_t rsrc, uint32_t lds_tile, int wave,
                                              uint32_t kbytes) const {
        dma16(rsrc, off[i] + kbytes, lds_tile + (uint32_t)(wave * kPerWave + i) * 1024u);
    }
};

// Fragment address of one 16x32 MFMA operand block (rows rb..rb+15, k32 step s).
template <int BK>
__device__ __forceinline__ uint32_t ktile_frag_addr(uint32_t tile, int rb, int s, int lane) {
    const int x = lane & 15, g = lane >> 4;
    const int row = rb + x;
    const int c = (4 * s + g) ^ swz_k<BK>(row);
    return tile + (uint32_t)(row * BK * 2 + c * 16);
}

// Address of the first of the two ds_read_b64_tr_b16 of a 16x32 operand block
// whose index (column of the [BK][C] tile) runs over cb..cb+15, k32 step s.
// Lane (x, g) reads k-rows k0 = 32 s + 8 g + (x >> 2) and k0 + 4; both have
// the same swizzle (k0 & 3 and bit 3 of k0 agree), so the second read is the
// first plus 4 rows.
template <int C>
__device__ __forceinline__ uint32_t mntile_frag_addr(uint32_t tile, int cb, int s, int lane) {
    const int x = lane & 15, g = lane >> 4;
    const int col = cb + 4 * (x & 3);
    const int k0 = 32 * s + 8 * g + (x >> 2);
    const int c0 = (col >> 3) ^ swz_mn(k0);
    const int h = (col & 7) * 2;  // 0 or 8 bytes inside the chunk
    return tile + (uint32_t)(k0 * C * 2 + c0 * 16 + h);
}

// ---------------------------------------------------------------------------
// Epilogue: lane holds C[m][n .. n+3] of each 16x16 block (i, j). mb: row of
// block i = 0 for this lane; nb: first column of block j = 0 (SWIGLU: of the
// gate block j = 0; the up block j + NI/2 covers the same output columns).
// Rows are handled one at a time (sched_barrier) to bound live registers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x2_t pack4(float a, float b, float c, float d) {
    u32x2_t o;
    o[0] = pack_bf16x2(a, b);
    o[1] = pack_bf16x2(c, d);
    return o;
}

__device__ __forceinline__ void unpack4(u32x2_t v, float (&x)[4]) {
    x[0] = bf16_bits_to_f32(v[0] & 0xffffu);
    x[1] = bf16_bits_to_f32(v[0] >> 16);
    x[2] = bf16_bits_to_f32(v[1] & 0xffffu);
    x[3] = bf16_bits_to_f32(v[1] >> 16);
}

// Activation-backward epilogues (GeLU', SwiGLU'): dZ in the accumulators,
// the saved pre-activation H read from memory. H of row block i + 1 is
// loaded before row block i is computed and stored, so that its latency
// overlaps the math (two row blocks of H in registers).
template <int MI, int NI, int EPI>
__device__ __forceinline__ void epilogue_act_bwd(const f32x4_t (&acc)[MI][NI], const GemmArgs& args, int mb,
                                                 int nb) {
    constexpr int NH = EPI == EPI_SWIGLU_BWD ? 2 : 1;  // H columns read per output column: g (and u)
    u32x2_t hb[2][NI][NH];
    auto load_rows = [&](auto ic) {
        constexpr int i = decltype(ic)::value, buf = i % 2;
        const int m = mb + i * 16;
        const uint16_t* hrow = args.aux + (size_t)m * args.ldc2;
        static_for<0, NI>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int n = nb + j * 16;
            if (m < args.M && n < args.N) {
                hb[buf][j][0] = *reinterpret_cast<const u32x2_t*>(hrow + n);
                if constexpr (NH == 2) hb[buf][j][1] = *reinterpret_cast<const u32x2_t*>(hrow + args.f + n);
            }
        });
    };
    load_rows(std::integral_constant<int, 0>{});
    static_for<0, MI>([&](auto ic) {
        constexpr int i = decltype(ic)::value, buf = i % 2;
        if constexpr (i + 1 < MI) load_rows(std::integral_constant<int, i + 1>{});
        __builtin_amdgcn_sched_barrier(0);
        const int m = mb + i * 16;
        if (m < args.M) {
            uint16_t* crow = reinterpret_cast<uint16_t*>(args.C) + (size_t)m * args.ldc;
            static_for<0, NI>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                const int n = nb + j * 16;
                if (n < args.N) {
                    const f32x4_t dz = acc[i][j];
                    if constexpr (EPI == EPI_GELU_BWD) {
                        float x[4];
                        unpack4(hb[buf][j][0], x);
                        *reinterpret_cast<u32x2_t*>(crow + n) =
                            pack4(dz[0] * gelu_grad_f(x[0]), dz[1] * gelu_grad_f(x[1]),
                                  dz[2] * gelu_grad_f(x[2]), dz[3] * gelu_grad_f(x[3]));
                    } else {
                        float g[4], u[4], dg[4], du[4];
                        unpack4(hb[buf][j][0], g);
                        unpack4(hb[buf][j][1], u);
                        static_for<0, 4>([&](auto rc) {
                            constexpr int r = decltype(rc)::value;
                            const float sg = sigmoid_f(g[r]);
                            du[r] = dz[r] * g[r] * sg;
                            dg[r] = dz[r] * u[r] * (sg + g[r] * sg * (1.0f - sg));
                        });
                        *reinterpret_cast<u32x2_t*>(crow + n) = pack4(dg[0], dg[1], dg[2], dg[3]);
                        *reinterpret_cast<u32x2_t*>(crow + args.f + n) = pack4(du[0], du[1], du[2], du[3]);
                    }
                }
            });
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

// One accumulator read from its AGPR into a VGPR (inline asm: as plain C++
// the compiler may copy a whole accumulator array to VGPRs first).
__device__ __forceinline__ float read_acc(float v) {
    float x;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(v));
    return x;
}

// Vocab-parallel cross-entropy, forward: the logits never leave registers.
// For each row, the 4 lanes that hold it (lane, lane ^ 16, lane ^ 32,
// lane ^ 48) reduce this wave's 16 NI columns to the record
// {max z, sum exp(z - max), z of the target column (0 if not here)}, written
// to record `part` of the row, part = the wave's column block index across
// the grid (tile column x waves per tile row + wave column). One pass over
// the accumulators: a running maximum with the running sum rescaled when it
// grows (4 logits live at a time, so the 256 accumulators need no copies).
__device__ __forceinline__ void ce_merge(float& m, float& s, float m2, float s2) {
    const float mx = fmaxf(m, m2);
    if (mx == -__builtin_inff()) return;  // both empty
    s = s * __expf(m - mx) + s2 * __expf(m2 - mx);
    m = mx;
}

template <int MI, int NI>
__device__ __forceinline__ void epilogue_ce_stats(const f32x4_t (&acc)[MI][NI], const GemmArgs& args, int mb,
                                                  int nb) {
    const int lane = threadIdx.x & 63;
    const int part = (nb - 4 * (lane >> 4)) / (16 * NI);
    float* rec = static_cast<float*>(args.C);
    static_for<0, MI>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int m = mb + i * 16;
        const int yt = args.tgt[m < args.M ? m : 0] - args.col0 - nb;  // target column - this lane's first
        float run_m = -__builtin_inff(), run_s = 0.f, zy = 0.f;
        static_for<0, NI>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            float v[4];
            static_for<0, 4>([&](auto rc) { v[decltype(rc)::value] = read_acc(acc[i][j][decltype(rc)::value]); });
            float gm = -__builtin_inff();
            static_for<0, 4>([&](auto rc) {
                constexpr int r = decltype(rc)::value;
                if (nb + 16 * j + r < args.N) {
                    gm = fmaxf(gm, v[r]);
                    if (yt == 16 * j + r) zy = v[r];
                }
            });
            if (gm != -__builtin_inff()) {
                const float mx = fmaxf(run_m, gm);
                float gs = 0.f;
                static_for<0, 4>([&](auto rc) {
                    constexpr int r = decltype(rc)::value;
                    if (nb + 16 * j + r < args.N) gs += __expf(v[r] - mx);
                });
                run_s = run_s * __expf(run_m - mx) + gs;
                run_m = mx;
            }
        });
        ce_merge(run_m, run_s, __shfl_xor(run_m, 16, 64), __shfl_xor(run_s, 16, 64));
        ce_merge(run_m, run_s, __shfl_xor(run_m, 32, 64), __shfl_xor(run_s, 32, 64));
        zy += __shfl_xor(zy, 16, 64);
        zy += __shfl_xor(zy, 32, 64);
        if ((lane >> 4) == 0 && m < args.M) {
            float* p = rec + ((size_t)m * args.ldc + part) * 3;
            p[0] = run_m;
            p[1] = run_s;
            p[2] = zy;
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Vocab-parallel cross-entropy, backward: dZ = (softmax(z) - one-hot) * dloss
// with the global per-row max and sum (bf16 store).
template <int MI, int NI>
__device__ __forceinline__ void epilogue_ce_grad(const f32x4_t (&acc)[MI][NI], const GemmArgs& args, int mb,
                                                 int nb) {
    static_for<0, MI>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int m = mb + i * 16;
        if (m < args.M) {
            const float mm = args.rm[m], inv = 1.0f / args.rs[m], dl = args.rd[m];
            const int yt = args.tgt[m] - args.col0;
            uint16_t* crow = static_cast<uint16_t*>(args.C) + (size_t)m * args.ldc;
            static_for<0, NI>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                const int n = nb + 16 * j;
                if (n < args.N) {
                    float g[4];
                    static_for<0, 4>([&](auto rc) {
                        constexpr int r = decltype(rc)::value;
                        g[r] = (__expf(acc[i][j][r] - mm) * inv - (n + r == yt ? 1.0f : 0.0f)) * dl;
                    });
                    *reinterpret_cast<u32x2_t*>(crow + n) = pack4(g[0], g[1], g[2], g[3]);
                }
            });
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

template <int MI, int NI, int EPI>
__device__ __forceinline__ void epilogue(const f32x4_t (&acc)[MI][NI], const GemmArgs& args, int mb, int nb) {
    if constexpr (EPI == EPI_GELU_BWD || EPI == EPI_SWIGLU_BWD) {
        epilogue_act_bwd<MI, NI, EPI>(acc, args, mb, nb);
        return;
    }
    if constexpr (EPI == EPI_CE_STATS) {
        epilogue_ce_stats<MI, NI>(acc, args, mb, nb);
        return;
    }
    if constexpr (EPI == EPI_CE_GRAD) {
        epilogue_ce_grad<MI, NI>(acc, args, mb, nb);
        return;
    }
    if constexpr (EPI == EPI_F32) {
        // one pass per mode, rows one at a time: the accumulators move to
        // VGPRs a row at a time (a test inside the row loop made the
        // compiler copy them all first)
        auto rows = [&](auto accc) {
            constexpr bool ACC = decltype(accc)::value;
            static_for<0, MI>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                const int m = mb + i * 16;
                if (m < args.M) {
                    f32x4_t* row =
                        reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(args.C) + (size_t)m * args.ldc + nb);
                    static_for<0, NI>([&](auto jc) {
                        constexpr int j = decltype(jc)::value;
                        if (nb + j * 16 < args.N) {
                            if constexpr (ACC) row[j * 4] = acc[i][j] + row[j * 4];
                            else row[j * 4] = acc[i][j];
                        }
                    });
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        if (args.accumulate) rows(std::true_type{});
        else rows(std::false_type{});
        return;
    }
    static_for<0, MI>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int m = mb + i * 16;
        if (m < args.M) {
            if constexpr (EPI == EPI_BF16 || EPI == EPI_GELU) {
                uint16_t* crow = reinterpret_cast<uint16_t*>(args.C) + (size_t)m * args.ldc;
                static_for<0, NI>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    const int n = nb + j * 16;
                    if (n < args.N) {
                        const f32x4_t v = acc[i][j];
                        if constexpr (EPI == EPI_GELU) {
                            *reinterpret_cast<u32x2_t*>(crow + n) =
                                pack4(gelu_f(v[0]), gelu_f(v[1]), gelu_f(v[2]), gelu_f(v[3]));
                            if (args.C2)
                                *reinterpret_cast<u32x2_t*>(args.C2 + (size_t)m * args.ldc2 + n) =
                                    pack4(v[0], v[1], v[2], v[3]);
                        } else {
                            *reinterpret_cast<u32x2_t*>(crow + n) = pack4(v[0], v[1], v[2], v[3]);
                        }
                    }
                });
            } else if constexpr (EPI == EPI_SWIGLU) {
                uint16_t* crow = reinterpret_cast<uint16_t*>(args.C) + (size_t)m * args.ldc;
                static_for<0, NI / 2>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    const int n = nb + j * 16;
                    if (n < args.N) {
                        const f32x4_t g = acc[i][j];
                        const f32x4_t u = acc[i][j + NI / 2];
                        float z[4];
                        static_for<0, 4>([&](auto rc) {
                            constexpr int r = decltype(rc)::value;
                            z[r] = g[r] * sigmoid_f(g[r]) * u[r];
                        });
                        *reinterpret_cast<u32x2_t*>(crow + n) = pack4(z[0], z[1], z[2], z[3]);
                        if (args.C2) {
                            uint16_t* hrow = args.C2 + (size_t)m * args.ldc2;
                            *reinterpret_cast<u32x2_t*>(hrow + n) = pack4(g[0], g[1], g[2], g[3]);
                            *reinterpret_cast<u32x2_t*>(hrow + args.f + n) = pack4(u[0], u[1], u[2], u[3]);
                        }
                    }
                });
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

// fp32 store of the accumulators straight from their registers (ping-pong
// kernels, which keep only half of the VGPRs: a plain C++ store makes the
// compiler copy every accumulator to VGPRs first). Overwrites C; the
// launcher runs products that add into C on the other kernels.
__device__ __forceinline__ void store_f32x4_acc(float* p, const f32x4_t& v) {
    asm volatile("global_store_dwordx4 %0, %1, off" ::"v"(p), "a"(v) : "memory");
}

template <int MI, int NI>
__device__ __forceinline__ void epilogue_f32_store_acc(const f32x4_t (&acc)[MI][NI], const GemmArgs& args, int mb,
                                                       int nb) {
    static_for<0, MI>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int m = mb + i * 16;
        if (m < args.M) {
            float* row = reinterpret_cast<float*>(args.C) + (size_t)m * args.ldc + nb;
            static_for<0, NI>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                if (nb + j * 16 < args.N) store_f32x4_acc(row + j * 16, acc[i][j]);
            });
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

// fp32 stores from the MFMA's own accumulator layout: lane l holds column
// l % 16 of rows 4 (l / 16) + r, r = 0..3, of each 16 x 16 block. A store of
// register r then writes 64 contiguous bytes from each 16 lanes (4 rows of
// the block): the CU's store path takes 64 bytes of consecutive lanes per
// clock, against one lane (16 bytes) per clock when consecutive lanes write
// different rows, as the 16-byte stores of the swapped layout do (measured
// with the store-rate probe: 95 against 38 GB/s per CU, 54 against 37 GB/s
// with all 256 CUs storing).
// Each value leaves its AGPR through inline asm (a store, or read_acc into a
// VGPR to add it to C): written as plain C++, the compiler copies the whole
// accumulator array to VGPRs first and spills.
// (the 16-column blocks of a row differ by a constant, folded into the
// instruction's offset: one address per row)
template <int OFF>
__device__ __forceinline__ void store_f32_acc(float* p, float v) {
    asm volatile("global_store_dword %0, %1, off offset:%2" ::"v"(p), "a"(v), "i"(OFF) : "memory");
}


template <int MI, int NI>
__device__ __forceinline__ void epilogue_f32_cols(const f32x4_t (&acc)[MI][NI], const GemmArgs& args, int mb,
                                                  int nb) {
    auto rows = [&](auto accc) {
        constexpr bool ACC = decltype(accc)::value;
        static_for<0, MI>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            static_for<0, 4>([&](auto rc) {
                constexpr int r = decltype(rc)::value;
                const int m = mb + i * 16 + r;
                if (m < args.M) {
                    float* row = reinterpret_cast<float*>(args.C) + (size_t)m * args.ldc + nb;
                    static_for<0, NI>([&](auto jc) {
                        constexpr int j = decltype(jc)::value;
                        if (nb + j * 16 < args.N) {
                            if constexpr (ACC) row[j * 16] += read_acc(acc[i][j][r]);
                            else store_f32_acc<j * 64>(row, acc[i][j][r]);
                        }
                    });
                }
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    if (args.accumulate) rows(std::true_type{});
    else rows(std::false_type{});
}

template <int MI, int NI>
__device__ __forceinline__ void epilogue_f32_cols_store_acc(const f32x4_t (&acc)[MI][NI], const GemmArgs& args,
                                                            int mb, int nb) {
    static_for<0, MI>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        static_for<0, 4>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const int m = mb + i * 16 + r;
            if (m < args.M) {
                float* row = reinterpret_cast<float*>(args.C) + (size_t)m * args.ldc + nb;
                static_for<0, NI>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    if (nb + j * 16 < args.N) store_f32_acc<j * 64>(row, acc[i][j][r]);
                });
            }
        });
        __builtin_amdgcn_sched_barrier(0);
    });
}

// ---------------------------------------------------------------------------
// Tile configuration.
//   BM x BN   loaded operand tiles (LDS); TM x TN computed tile (TM <= BM,
//             TN <= BN); for SWIGLU, TN counts gate and up columns (TN/2 of
//             each, output tile TN/2 wide) and BN/2 columns of each half are
//             loaded
//   BKA, SA   k-rows per stage and stages of the A operand's LDS ring
//   BKB, SB   the same for B
// A K-contiguous operand is staged 64 k-rows at a time: each tile row is then
// one whole 128-byte line (rows of half a line halve the rate at which the
// load unit returns data). An MN-contiguous operand has whole lines at any
// depth and uses 32-row stages, so that more of them fit in flight.
// ---------------------------------------------------------------------------
//   PP        ping-pong schedule (8 waves; see the kernel's k-loop)
template <int BM_, int BN_, int TM_, int TN_, int BKA_, int SA_, int BKB_, int SB_, int WAVES_M_, int WAVES_N_,
          bool PP_ = false>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, TM = TM_, TN = TN_;
    static constexpr int BKA = BKA_, SA = SA_, BKB = BKB_, SB = SB_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr bool PP = PP_;
};

// ---------------------------------------------------------------------------
// The LDS-DMA issue order, as a compile-time model. The k-loop runs in k32
// sub-steps u; operand o (0 = A, 1 = B) has stages of p_o sub-steps in a ring
// of S_o buffers. The buffer of stage s is free once the reads of its last
// sub-step are done, i.e. at the barrier of sub-step (s + 1) p_o - 1, where
// stage s + S_o is issued into it: stage s is issued at sub-step
// t_o(s) = (s - S_o + 1) p_o - 1 (A before B within a sub-step), and the
// prologue issues every stage with t_o(s) < 0 in that same order, so the
// sequence is periodic from the start. At the barrier of sub-step u the
// fragments of sub-step u + 1 are needed: stages (u + 1) / p_o. vmcnt counts
// this wave's loads in issue order, so the wait allows the loads issued after
// the last needed one to stay outstanding.
// ---------------------------------------------------------------------------
// Issue slots inside a sub-step: NOPS memory operations (NDMA LDS-DMA loads,
// NRD fragment reads) spread evenly over the first W of its NMFMA MFMAs, the
// loads evenly among the reads. Bursts of loads (all waves leave a barrier
// together) would queue at the CU's address unit and stall every wave's
// in-order MFMA stream behind them.
template <int NMFMA, int NDMA, int NRD>
struct Slots {
    static constexpr int NOPS = NDMA + NRD;
    static constexpr int W = NMFMA * 7 / 8 > 0 ? NMFMA * 7 / 8 : 1;
    // operations k in [begin(m), begin(m + 1)) follow MFMA m
    static constexpr int begin(int m) { return (m * NOPS + W - 1) / W; }
    static constexpr int MAXPER = (NOPS + W - 1) / W + 1;
    // loads before operation k, and whether operation k is a load
    static constexpr int loads_before(int k) { return NDMA == 0 ? 0 : (k * NDMA + NOPS - 1) / NOPS; }
    static constexpr bool is_load(int k) {
        return NDMA > 0 && loads_before(k) < NDMA && loads_before(k) * NOPS / NDMA == k;
    }
};

struct RingModel {
    int pA, SA, LA, pB, SB, LB;
    constexpr int t_of(int o, int st) const { return o == 0 ? (st - SA + 1) * pA - 1 : (st - SB + 1) * pB - 1; }
    constexpr int key(int o, int st) const { return 2 * t_of(o, st) + o; }
    // loads this wave may leave outstanding at the barrier of sub-step u
    constexpr int wait_count(int u) const {
        const int ka = key(0, (u + 1) / pA), kb = key(1, (u + 1) / pB);
        const int kmax = ka > kb ? ka : kb;
        int x = 0;
        for (int st = 0; t_of(0, st) < u; ++st)
            if (key(0, st) > kmax) x += LA;
        for (int st = 0; t_of(1, st) < u; ++st)
            if (key(1, st) > kmax) x += LB;
        return x;
    }
    // does operand o issue a stage at sub-step u (u >= 0)?
    constexpr bool issues(int o, int u) const { return (u + 1) % (o == 0 ? pA : pB) == 0; }
};

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <class CF, bool A_T, bool B_KN, int EPI, bool WIDE>
__global__ void __launch_bounds__(64 * CF::WAVES_M * CF::WAVES_N)
gemm_kernel(const GemmArgs args) {
    constexpr int BM = CF::BM, BN = CF::BN, TM = CF::TM, TN = CF::TN;
    constexpr int BKA = CF::BKA, SA = CF::SA, BKB = CF::BKB, SB = CF::SB;
    constexpr int WAVES_M = CF::WAVES_M, WAVES_N = CF::WAVES_N;
    constexpr int NWAVES = WAVES_M * WAVES_N;
    constexpr bool SWIGLU = (EPI == EPI_SWIGLU);
    constexpr bool GATEUP = SWIGLU;                  // B tile = [gate | up] halves
    // fp32 outputs: accumulators in the MFMA's own layout (a lane holds one
    // column of 4 rows), stored a row of 16 consecutive floats per 16 lanes
    constexpr bool COLS = (EPI == EPI_F32) && TPS_F32_COLS != 0;
    constexpr int WM = TM / WAVES_M, WN = TN / WAVES_N;
    constexpr int MI = WM / 16, NI = WN / 16;
    constexpr int PA = BKA / 32, PB = BKB / 32;     // k32 sub-steps per stage
    constexpr int TNZ = GATEUP ? TN / 2 : TN;       // output columns per tile
    constexpr int A_STAGE = BM * BKA * 2, B_STAGE = BN * BKB * 2;
    static_assert(TM <= BM && TN <= BN, "computed tile must fit the loaded tile");
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert((BKA == 32 || BKA == 64) && (BKB == 32 || BKB == 64), "stages of 32 or 64 k-rows");
    static_assert(!SWIGLU || (NI % 2 == 0 && B_KN && WN % 32 == 0), "SwiGLU needs an even gate/up split");
    static_assert(SA >= 2 && SB >= 2, "at least two stages per ring");
    static_assert(SA * A_STAGE + SB * B_STAGE <= 160 * 1024, "gfx950 LDS is 160 KB");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[SA * A_STAGE + SB * B_STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // --- tile index (XCD-aware, grouped) ---
    const int tiles_m = (args.M + TM - 1) / TM;
    const int tiles_n = (args.N + TNZ - 1) / TNZ;
    const int T = tiles_m * tiles_n;
    const int split = (int)(blockIdx.x % (unsigned)args.ksplit);
    const int bid = (int)(blockIdx.x / (unsigned)args.ksplit);
    const int per = T >> 3;
    const int lid = (bid < per * 8) ? (bid & 7) * per + (bid >> 3) : bid;
    const int group = lid / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gsz = min(tiles_m - first_m, kGroupM);
    const int in_group = lid % (kGroupM * tiles_n);
    const int tm = first_m + in_group % gsz;
    const int tn = in_group / gsz;
    const int m0 = tm * TM;
    const int n0 = tn * TNZ;

    // --- this workgroup's K range (split-K) ---
    const int k0 = split * args.kper;
    const int Kloc = args.ksplit > 1 ? min(args.K, k0 + args.kper) - k0 : args.K;
    // --- DMA descriptors and per-lane offsets ---
    // The window of an operand starts at this workgroup's first k-row (and,
    // K-contiguous, at its tile's first row): byte offset org.
    const uint64_t a_org = (uint64_t)k0 * (A_T ? (uint64_t)args.lda : 1u) * 2u +
                           (A_T ? 0u : (uint64_t)m0 * (uint64_t)args.lda * 2u);
    const uint64_t b_org = (uint64_t)k0 * (B_KN ? (uint64_t)args.ldb : 1u) * 2u +
                           (B_KN ? 0u : (uint64_t)n0 * (uint64_t)args.ldb * 2u);
    // every wave issues its share of each stage's LDS-DMA loads
    constexpr bool PP = CF::PP;
    constexpr int NWD = NWAVES;
    const int dw = wave;
    using ADma = typename std::conditional<A_T, MNTileDma<BM, BKA, NWD>, KTileDma<BM, BKA, NWD>>::type;
    using BDma = typename std::conditional<B_KN, MNTileDma<BN, BKB, NWD>, KTileDma<BN, BKB, NWD>>::type;
    ADma da;
    BDma db;
    if constexpr (A_T) {
        da.init(dw, lane, args.lda, IdentityCols{m0, args.M});
    } else {
        da.init(dw, lane, 0, args.lda);
    }
    if constexpr (B_KN) {
        if constexpr (GATEUP) {
            db.init(dw, lane, args.ldb, SwigluCols<BN / 2>{n0, args.f});
        } else {
            db.init(dw, lane, args.ldb, IdentityCols{n0, args.N});
        }
    } else {
        db.init(dw, lane, 0, args.ldb);
    }
    // An MN-contiguous operand of a split-K product is range-checked up to
    // the end of this split's K rows: the ring's loads past the chunk (issued
    // to keep the waits constant) then read zeros instead of fetching the
    // next split's rows from memory.
    const uint64_t k_end = (uint64_t)(k0 + Kloc);
    const uint64_t a_ext = (A_T && args.ksplit > 1) ? min(args.a_bytes, k_end * (uint64_t)args.lda * 2u) : args.a_bytes;
    const uint64_t b_ext = (B_KN && args.ksplit > 1) ? min(args.b_bytes, k_end * (uint64_t)args.ldb * 2u) : args.b_bytes;
    StageCursor<A_T && WIDE> ca;
    StageCursor<B_KN && WIDE> cb;
    ca.init(args.A, a_ext, a_org, A_T ? (uint64_t)BKA * (uint64_t)args.lda * 2u : (uint64_t)BKA * 2u);
    cb.init(args.B, b_ext, b_org, B_KN ? (uint64_t)BKB * (uint64_t)args.ldb * 2u : (uint64_t)BKB * 2u);
    const uint32_t ldsA = lds_addr(smem), ldsB = ldsA + SA * A_STAGE;
    constexpr int LA = ADma::kPerWave, LB = BDma::kPerWave;  // loads per stage per wave
    constexpr RingModel ring{PA, SA, LA, PB, SB, LB};

    // load d of this wave's share of a stage of operand A / B: LDS buffer at
    // byte offset `buf` of the ring, the stage's descriptor and k offset
    auto issue_a = [&](auto dc, uint32_t buf, i32x4_t rs, uint32_t ko) {
        da.issue_one(decltype(dc)::value, rs, ldsA + buf, dw, ko);
    };
    auto issue_b = [&](auto dc, uint32_t buf, i32x4_t rs, uint32_t ko) {
        db.issue_one(decltype(dc)::value, rs, ldsB + buf, dw, ko);
    };

    // --- fragment addresses in buffer 0 of each ring ---
    // B column of fragment j inside the loaded tile
    auto bcol = [&](int j) -> int {
        if constexpr (SWIGLU) {
            return j < NI / 2 ? wn * (WN / 2) + 16 * j : BN / 2 + wn * (WN / 2) + 16 * (j - NI / 2);
        } else {
            return wn * WN + 16 * j;
        }
    };
    // K-contiguous fragments of one wave differ by whole 16-row blocks, whose
    // swizzle is the same, so they are a base address plus a constant (folded
    // into the LDS instruction's offset); MN-contiguous ones need one address
    // per fragment. Index h: k32 half of a 64-row stage.
    uint32_t fa[MI][PA];
    uint32_t fb[NI][PB];
    static_for<0, PA>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const uint32_t a_base = ktile_frag_addr<BKA>(ldsA, wm * WM, h, lane);
        static_for<0, MI>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (A_T) fa[i][h] = mntile_frag_addr<BM>(ldsA, wm * WM + 16 * i, h, lane);
            else fa[i][h] = a_base + (uint32_t)(i * 16 * BKA * 2);
        });
    });
    static_for<0, PB>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const uint32_t b_base = ktile_frag_addr<BKB>(ldsB, wn * WN, h, lane);
        static_for<0, NI>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr (B_KN) fb[j][h] = mntile_frag_addr<BN>(ldsB, bcol(j), h, lane);
            else fb[j][h] = b_base + (uint32_t)(j * 16 * BKB * 2);
        });
    });

    f32x4_t acc[MI][NI];
    static_for<0, MI>([&](auto ic) {
        static_for<0, NI>([&](auto jc) {
            acc[decltype(ic)::value][decltype(jc)::value] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        });
    });

    // Fragments of one k32 sub-step: the wave's MI A blocks and NI B blocks.
    struct Frags {
        bf16x8_t a[MI];
        bf16x8_t b[NI];
    };
    // Fragment read r (0 <= r < NFR) of a sub-step whose A data sits at LDS
    // offset soa (half ha of the A stage) and B data at sob (half hb): the
    // wave's A blocks, then its B blocks.
    constexpr int NFR = MI + NI;
    auto read_one = [&](Frags& fr, auto rc, uint32_t soa, uint32_t sob, auto hac, auto hbc) {
        constexpr int r = decltype(rc)::value;
        constexpr int ha = decltype(hac)::value, hb = decltype(hbc)::value;
        if constexpr (r < MI) {
            if constexpr (A_T) fr.a[r] = lds_read_tr2<BM>(fa[r][ha] + soa);
            else fr.a[r] = lds_read16(fa[r][ha] + soa);
        } else {
            if constexpr (B_KN) fr.b[r - MI] = lds_read_tr2<BN>(fb[r - MI][hb] + sob);
            else fr.b[r - MI] = lds_read16(fb[r - MI][hb] + sob);
        }
    };
    // MFMA m (0 <= m < NMFMA) of a sub-step, A block major. The accumulator is
    // tied to its AGPRs (inline asm): the builtin leaves the register
    // allocator free to pick an untied destination, and it then copies
    // accumulators between AGPRs and VGPRs on every k-step.
    constexpr int NMFMA = MI * NI;
    auto mfma_one = [&acc](const Frags& fr, auto mc) {
        constexpr int m = decltype(mc)::value;
        constexpr int i = m / NI, j = m % NI;
        if constexpr (COLS)
            asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(fr.a[i]), "v"(fr.b[j]));
        else
            asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(fr.b[j]), "v"(fr.a[i]));
    };
    // (decode tiles, at most 32 token rows, stream the weight and are bound
    // by HBM, not by the MFMA issue; they may load more often than they MFMA)
    static_assert(PP || NMFMA >= LA + LB || TM <= 32, "fewer MFMAs than loads per sub-step");

    // the waits the model derives are the same for every sub-step of a parity
    static_assert(ring.wait_count(0) == ring.wait_count(2) && ring.wait_count(2) == ring.wait_count(4) &&
                      ring.wait_count(1) == ring.wait_count(3) && ring.wait_count(3) == ring.wait_count(5),
                  "LDS-DMA waits are not periodic");
    static_assert(ring.wait_count(0) <= 63 && ring.wait_count(1) <= 63, "vmcnt range");

    // k32 sub-steps, an even count (the register double buffer alternates per
    // sub-step and the loop runs pairs). NN / NT contract over a model width,
    // a multiple of 64: nothing is added. TN contracts over tokens: k-rows
    // past K read as zeros (buffer range check).
    const int U = ((Kloc + 63) / 64) * 2;

    // Ring positions (uniform, kept in scalar registers and advanced with a
    // compare-and-wrap, no division): the buffer the next fragment reads
    // come from, the buffer the next load goes to, and that load's k offset.
    uint32_t a_rd = 0, b_rd = 0, a_wr = 0, b_wr = 0;
    auto wrap_a = [](uint32_t x) { x += A_STAGE; return x == (uint32_t)(SA * A_STAGE) ? 0u : x; };
    auto wrap_b = [](uint32_t x) { x += B_STAGE; return x == (uint32_t)(SB * B_STAGE) ? 0u : x; };

    // Sub-step of parity PAR: MFMAs on `cur` while the fragments of the next
    // sub-step are read into `nxt`. If a ring starts a new stage with the next
    // sub-step, this sub-step first waits for it (and for every wave to have
    // read the buffer that stage's predecessor left, which it then refills).
    // Loads are issued for every stage, also past the last one: those read
    // past K (range-checked) into buffers no later read uses, which keeps the
    // waits constant; the last sub-step's fragment reads likewise fetch data
    // nothing uses. Loads and reads are spread over the MFMAs (Slots); the
    // sched_barrier fences keep that order.
    auto substep = [&](auto parc, Frags& cur, Frags& nxt) {
        constexpr int PAR = decltype(parc)::value;
        constexpr bool IA = ring.issues(0, PAR), IB = ring.issues(1, PAR);
        constexpr int NDA = IA ? LA : 0, NDMA = NDA + (IB ? LB : 0);
        using SL = Slots<NMFMA, NDMA, NFR>;
        constexpr int HA = (PAR + 1) % PA, HB = (PAR + 1) % PB;  // halves the reads fetch
        if constexpr (IA || IB) {
            wait_vmcnt_barrier<ring.wait_count(PAR)>();
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (IA) a_rd = wrap_a(a_rd);
        if constexpr (IB) b_rd = wrap_b(b_rd);
        const uint32_t soa = a_rd, sob = b_rd, wa = a_wr, wb = b_wr;
        const i32x4_t ra = ca.rs, rb = cb.rs;
        const uint32_t ka = ca.ko, kb = cb.ko;
        static_for<0, NMFMA>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            mfma_one(cur, mc);
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, SL::MAXPER>([&](auto cc) {
                constexpr int k = SL::begin(m) + decltype(cc)::value;
                if constexpr (k < SL::begin(m + 1) && k < SL::NOPS) {
                    if constexpr (SL::is_load(k)) {
                        constexpr int d = SL::loads_before(k);
                        // after a stage's last load, its cursor moves on
                        // (scalar work in the shadow of the MFMAs)
                        if constexpr (d < NDA) {
                            issue_a(std::integral_constant<int, d>{}, wa, ra, ka);
                            if constexpr (d == NDA - 1) ca.next();
                        } else {
                            issue_b(std::integral_constant<int, d - NDA>{}, wb, rb, kb);
                            if constexpr (d == NDMA - 1) cb.next();
                        }
                    } else {
                        read_one(nxt, std::integral_constant<int, k - SL::loads_before(k)>{}, soa, sob,
                                 std::integral_constant<int, HA>{}, std::integral_constant<int, HB>{});
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
        });
        if constexpr (IA) a_wr = wrap_a(a_wr);
        if constexpr (IB) b_wr = wrap_b(b_wr);
    };

    if constexpr (PP) {
        // Ping-pong: the two waves of each SIMD (wave w and w + 4: groups 0
        // and 1) take turns, phase by phase, between a run of MFMAs and the
        // memory work of their next sub-step (fragment reads and their share
        // of the LDS-DMA loads), so the matrix pipe of a SIMD is fed by one
        // wave while the other's loads and reads are in flight. Per sub-step
        // u, with a barrier after each phase:
        //   phase 2u:     group 0 MFMAs of u  | group 1 reads u, issues the
        //                                       stages due at u - 1
        //   phase 2u + 1: group 1 MFMAs of u  | group 0 reads u + 1, issues
        //                                       the stages due at u
        // (a stage is due when the buffer it refills has been read by both
        // groups). Each wave issues its share of every stage (the ring model
        // of the interleaved schedule, with 8 waves' shares), so the loads
        // of a sub-step are spread over both phases; a group waits for a
        // stage at the end of the phase before the first reads of it, and
        // drains its LDS reads before the barrier that ends its memory
        // phase. Fragments are single-buffered: a wave's reads follow its
        // own MFMAs.
        static_assert(NWAVES == 8, "ping-pong: two groups of four waves, one of each per SIMD");
        const bool g0 = wave < NWAVES / 2;
        if (U > 0) {
            constexpr int kmin = ring.key(0, 0) < ring.key(1, 0) ? ring.key(0, 0) : ring.key(1, 0);
            {
                static_for<0, -kmin>([&](auto kc) {
                    constexpr int key = decltype(kc)::value + kmin;
                    constexpr int o = ((key % 2) + 2) % 2;
                    constexpr int t = (key - o) / 2;
                    constexpr int pp = o == 0 ? PA : PB, SS = o == 0 ? SA : SB;
                    if constexpr ((t + 1) % pp == 0 && (t + 1) / pp + SS - 1 >= 0) {
                        constexpr int st = (t + 1) / pp + SS - 1;
                        if constexpr (o == 0) {
                            static_for<0, LA>([&](auto dc) { issue_a(dc, (uint32_t)(st * A_STAGE), ca.rs, ca.ko); });
                            ca.next();
                        } else {
                            static_for<0, LB>([&](auto dc) { issue_b(dc, (uint32_t)(st * B_STAGE), cb.rs, cb.ko); });
                            cb.next();
                        }
                    }
                });
            }
            constexpr int W0 = [] {
                constexpr RingModel rm{PA, SA, LA, PB, SB, LB};
                const int kmax = rm.key(0, 0) > rm.key(1, 0) ? rm.key(0, 0) : rm.key(1, 0);
                int x = 0;
                for (int st = 0; rm.t_of(0, st) < 0; ++st)
                    if (rm.key(0, st) > kmax) x += LA;
                for (int st = 0; rm.t_of(1, st) < 0; ++st)
                    if (rm.key(1, st) > kmax) x += LB;
                return x;
            }();
            wait_vmcnt_barrier<W0>();
            Frags fr;
            auto read_all = [&](auto hac, auto hbc) {
                static_for<0, NFR>([&](auto rc) { read_one(fr, rc, a_rd, b_rd, hac, hbc); });
            };
            auto mfma_run = [&]() {
                __builtin_amdgcn_s_setprio(1);
                __builtin_amdgcn_sched_barrier(0);
                static_for<0, NMFMA>([&](auto mc) {
                    mfma_one(fr, mc);
                    __builtin_amdgcn_sched_barrier(0);
                });
                __builtin_amdgcn_s_setprio(0);
                __builtin_amdgcn_sched_barrier(0);
            };
            // end of a memory phase: this wave's reads are in registers (and
            // its last reads of a buffer are done) before the barrier
            auto reads_done_barrier = [&]() {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                asm volatile("s_barrier" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            };
            // after a barrier, before reads overwrite fragments that MFMAs of
            // the previous phase took as operands
            auto operand_gap = [&]() {
                asm volatile("s_nop 7" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            };
            if (g0) read_all(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(0xC07F);
            asm volatile("s_nop 4" ::: "memory");  // VALU-zeroed accumulators before the first MFMA
            __builtin_amdgcn_sched_barrier(0);
            auto g0_step = [&](auto parc) {
                constexpr int PAR = decltype(parc)::value;
                constexpr bool IA = ring.issues(0, PAR), IB = ring.issues(1, PAR);
                mfma_run();
                if constexpr (IA || IB) {
                    wait_vmcnt_barrier<ring.wait_count(PAR)>();
                } else {
                    asm volatile("s_barrier" ::: "memory");
                }
                __builtin_amdgcn_sched_barrier(0);
                operand_gap();
                if constexpr (IA) a_rd = wrap_a(a_rd);
                if constexpr (IB) b_rd = wrap_b(b_rd);
                read_all(std::integral_constant<int, (PAR + 1) % PA>{}, std::integral_constant<int, (PAR + 1) % PB>{});
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (IA) {
                    static_for<0, LA>([&](auto dc) {
                        issue_a(dc, a_wr, ca.rs, ca.ko);
                        __builtin_amdgcn_sched_barrier(0);
                    });
                    ca.next();
                    a_wr = wrap_a(a_wr);
                }
                if constexpr (IB) {
                    static_for<0, LB>([&](auto dc) {
                        issue_b(dc, b_wr, cb.rs, cb.ko);
                        __builtin_amdgcn_sched_barrier(0);
                    });
                    cb.next();
                    b_wr = wrap_b(b_wr);
                }
                reads_done_barrier();
            };
            auto g1_step = [&](auto parc, bool first) {
                constexpr int PAR = decltype(parc)::value;
                // stages due at u - 1 (none before sub-step 1: the
                // prologue issued those)
                constexpr bool JA = PAR % PA == 0, JB = PAR % PB == 0;
                constexpr bool IA = ring.issues(0, PAR), IB = ring.issues(1, PAR);
                operand_gap();
                read_all(std::integral_constant<int, PAR % PA>{}, std::integral_constant<int, PAR % PB>{});
                if constexpr (IA) a_rd = wrap_a(a_rd);
                if constexpr (IB) b_rd = wrap_b(b_rd);
                __builtin_amdgcn_sched_barrier(0);
                if (!first) {
                    if constexpr (JA) {
                        static_for<0, LA>([&](auto dc) {
                            issue_a(dc, a_wr, ca.rs, ca.ko);
                            __builtin_amdgcn_sched_barrier(0);
                        });
                        ca.next();
                        a_wr = wrap_a(a_wr);
                    }
                    if constexpr (JB) {
                        static_for<0, LB>([&](auto dc) {
                            issue_b(dc, b_wr, cb.rs, cb.ko);
                            __builtin_amdgcn_sched_barrier(0);
                        });
                        cb.next();
                        b_wr = wrap_b(b_wr);
                    }
                }
                // group 0 reads stage (u + 1) / p next: this wave's share of
                // it has landed (and its reads are in registers)
                if constexpr (IA || IB) {
                    wait_vmcnt_barrier<ring.wait_count(PAR)>();
                } else {
                    reads_done_barrier();
                }
                __builtin_amdgcn_sched_barrier(0);
                mfma_run();
                asm volatile("s_barrier" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            };
            if (g0) {
                for (int u = 0; u < U; u += 2) {
                    g0_step(std::integral_constant<int, 0>{});
                    g0_step(std::integral_constant<int, 1>{});
                }
            } else {
                for (int u = 0; u < U; u += 2) {
                    g1_step(std::integral_constant<int, 0>{}, u == 0);
                    g1_step(std::integral_constant<int, 1>{}, false);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 15\n\ts_nop 7" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        if (U > 0) {  // K = 0 (no tokens in a weight gradient): C = 0
            // prologue: the stages issued "before sub-step 0", in the model's
            // order, then sub-step 0's fragments go to registers
            // (keys run from the earlier of the two stage 0s up to -1)
            constexpr int kmin = ring.key(0, 0) < ring.key(1, 0) ? ring.key(0, 0) : ring.key(1, 0);
            static_for<0, -kmin>([&](auto kc) {
                constexpr int key = decltype(kc)::value + kmin;
                {
                    constexpr int o = ((key % 2) + 2) % 2;      // operand of this key
                    constexpr int t = (key - o) / 2;            // its sub-step
                    // stage st with t_o(st) == t, if any and if st >= 0
                    constexpr int pp = o == 0 ? PA : PB, SS = o == 0 ? SA : SB;
                    if constexpr ((t + 1) % pp == 0 && (t + 1) / pp + SS - 1 >= 0) {
                        constexpr int st = (t + 1) / pp + SS - 1;
                        if constexpr (o == 0) {
                            static_for<0, LA>([&](auto dc) { issue_a(dc, (uint32_t)(st * A_STAGE), ca.rs, ca.ko); });
                            ca.next();
                        } else {
                            static_for<0, LB>([&](auto dc) { issue_b(dc, (uint32_t)(st * B_STAGE), cb.rs, cb.ko); });
                            cb.next();
                        }
                    }
                }
            });
            // stage 0 of both rings landed: every load issued after the later of
            // the two may stay outstanding
            constexpr int W0 = [] {
                constexpr RingModel rm{PA, SA, LA, PB, SB, LB};
                const int kmax = rm.key(0, 0) > rm.key(1, 0) ? rm.key(0, 0) : rm.key(1, 0);
                int x = 0;
                for (int st = 0; rm.t_of(0, st) < 0; ++st)
                    if (rm.key(0, st) > kmax) x += LA;
                for (int st = 0; rm.t_of(1, st) < 0; ++st)
                    if (rm.key(1, st) > kmax) x += LB;
                return x;
            }();
            wait_vmcnt_barrier<W0>();
            Frags f0, f1;
            static_for<0, NFR>([&](auto rc) {
                read_one(f0, rc, 0, 0, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
            });
            // the accumulators were zeroed by VALU writes, which the first MFMA
            // (inline asm, invisible to the hazard checks) must not overtake
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_nop 4" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            for (int u = 0; u < U; u += 2) {
                substep(std::integral_constant<int, 0>{}, f0, f1);
                substep(std::integral_constant<int, 1>{}, f1, f0);
            }
            // MFMA results are read by the epilogue only after the longest
            // MFMA-write -> read wait (the checks do not see the asm MFMAs), and
            // after every LDS-DMA load has retired
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 15\n\ts_nop 7" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    const int lr = lane & 15, lq = lane >> 4;
    // the lane's first output row and column: row l % 16 and 4 columns from
    // 4 (l / 16) (operands swapped), or column l % 16 and 4 rows (COLS)
    const int mb = m0 + wm * WM + (COLS ? 4 * lq : lr);
    const int nb = n0 + wn * (SWIGLU ? WN / 2 : WN) + (COLS ? lr : 4 * lq);
    if constexpr (EPI == EPI_F32 && !PP) {  // split-K partials are plain fp32 stores
        GemmArgs part = args;
        if (args.ksplit > 1) {
            part.C = reinterpret_cast<float*>(args.C) + (size_t)split * args.M * args.ldc;
            part.accumulate = 0;
        }
        if constexpr (COLS) epilogue_f32_cols<MI, NI>(acc, part, mb, nb);
        else epilogue<MI, NI, EPI_F32>(acc, part, mb, nb);
    } else if constexpr (EPI == EPI_F32) {  // ping-pong: C (or split s's partial) overwritten
        GemmArgs part = args;
        if (TPS_PP_SPLIT != 0 && args.ksplit > 1)
            part.C = reinterpret_cast<float*>(args.C) + (size_t)split * args.M * args.ldc;
        if constexpr (COLS) epilogue_f32_cols_store_acc<MI, NI>(acc, part, mb, nb);
        else epilogue_f32_store_acc<MI, NI>(acc, part, mb, nb);
    } else {
        epilogue<MI, NI, EPI>(acc, args, mb, nb);
    }
}

}  // namespace tps

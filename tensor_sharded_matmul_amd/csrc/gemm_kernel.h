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
//  * WAVES_M x WAVES_N waves of 64 lanes; each wave owns a (BM/WAVES_M) x
//    (BN/WAVES_N) sub-tile of C in f32 accumulators.
//  * v_mfma_f32_16x16x32_bf16 with the operands swapped (the MFMA "A" operand
//    is the B tile), so each lane ends with 4 consecutive columns of one C row
//    and epilogue stores are 16-byte (f32) or 8-byte (bf16) vectors.
//  * Operand tiles go HBM -> LDS directly (buffer_load_dwordx4 ... lds: no
//    staging registers), STAGES deep, so STAGES-1 K-steps of loads are in
//    flight while the MFMAs consume the oldest one; one barrier per K-step.
//    The loads are issued from inline asm with explicit vmcnt waits, because
//    the compiler would otherwise drain every LDS-DMA load before each
//    barrier. Rows past K (and past M / N) read as zero through the buffer
//    descriptor's range check.
//  * LDS layouts keep the operand as stored in HBM:
//      K-contiguous tile [rows][BK]: 16-byte chunk c of row r is stored at
//        c ^ swz(r), swz(r) = (r>>1)&7 (BK=64) or (r>>2)&3 (BK=32), so the 16
//        rows one MFMA fragment read touches fall in 16 distinct bank groups
//        (gfx950 LDS: 64 banks x 4 B, 16 lanes of a ds_read_b128 per clock).
//      MN-contiguous tile [BK][cols]: chunk c of k-row k at c ^ (2(k&3) +
//        8((k>>3)&1)); fragments are read with ds_read_b64_tr_b16, which
//        transposes 4x4 blocks of 16-bit values across each 16-lane group,
//        giving every lane 4 consecutive k of one column.
//    so the MFMA inner loop is the same for every layout.
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

constexpr int kGroupM = 4;     // tile rows per L2 group

enum Epi : int {
    EPI_F32 = 0,        // C f32 = acc (or += acc)
    EPI_BF16 = 1,       // C bf16 = acc
    EPI_GELU = 2,       // C bf16 = GeLU(acc); C2 bf16 = acc (optional)
    EPI_SWIGLU = 3,     // C bf16 = SiLU(g)*u; C2 bf16 = [g | u] (optional)
    EPI_GELU_BWD = 4,   // C bf16 = acc * GeLU'(aux)
    EPI_SWIGLU_BWD = 5, // C bf16 = [acc*u*SiLU'(g) | acc*SiLU(g)], aux = [g|u]
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
    uint32_t a_bytes, b_bytes;  // extent of A and B in bytes (buffer range check)
};

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

__device__ __forceinline__ float gelu_f(float x) {
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

__device__ __forceinline__ float gelu_grad_f(float x) {
    const float cdf = 0.5f * (1.0f + erff(x * 0.70710678118654752f));
    const float pdf = 0.39894228040143268f * __expf(-0.5f * x * x);
    return cdf + x * pdf;
}

__device__ __forceinline__ float sigmoid_f(float x) {
    return 1.0f / (1.0f + __expf(-x));
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

__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t voff, uint32_t lds_base) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base)
                 : "memory");
}

// Wait until at most N of this wave's LDS-DMA loads are outstanding and its LDS
// reads are done, then barrier: afterwards every wave's loads of the stage the
// wait covers are in LDS, and no wave still reads the stage about to be refilled.
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ bf16x8_t lds_read16(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>((uintptr_t)addr);
}

__device__ __forceinline__ bf16x8_t lds_read_tr2(uint32_t addr0, uint32_t addr1) {
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)addr0);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)addr1);
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

// SwiGLU B tile: each wave column of WN tile columns holds WN/2 gate columns
// followed by the WN/2 up columns of the same F indices.
template <int WN>
struct SwigluCols {
    int z0, f;
    __device__ __forceinline__ int operator()(int c) const {
        const int wc = c / WN;
        const int p = c % WN;
        const int j = z0 + wc * (WN / 2) + (p % (WN / 2));
        if (j >= f) return 0;  // outputs past f are never stored
        return p < WN / 2 ? j : f + j;
    }
};

// ---------------------------------------------------------------------------
// Per-lane DMA offsets of one operand tile (bytes, relative to the matrix).
// ---------------------------------------------------------------------------

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
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const int I = wave * kPerWave + i;
            const int row = I * kRpi + lane / kCpr;
            const int c = (lane % kCpr) ^ swz_k<BK>(row);
            off[i] = (uint32_t)(row0 + row) * (uint32_t)ld * 2u + (uint32_t)c * 16u;
        }
    }
    __device__ __forceinline__ void issue(i32x4_t rsrc, uint32_t lds_tile, int wave, uint32_t kbytes) const {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i)
            dma16(rsrc, off[i] + kbytes, lds_tile + (uint32_t)(wave * kPerWave + i) * 1024u);
    }
    static constexpr uint32_t step_bytes(int /*ld*/) { return BK * 2; }
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
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const int I = wave * kPerWave + i;
            const int k = I * kRpi + lane / kCpr;
            const int c = (lane % kCpr) ^ swz_mn(k);
            off[i] = (uint32_t)k * (uint32_t)ld * 2u + (uint32_t)colmap(c * 8) * 2u;
        }
    }
    __device__ __forceinline__ void issue(i32x4_t rsrc, uint32_t lds_tile, int wave, uint32_t kbytes) const {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i)
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

// The two ds_read_b64_tr_b16 addresses of a 16x32 operand block whose index
// (column of the [BK][C] tile) runs over cb..cb+15, k32 step s.
template <int C>
__device__ __forceinline__ void mntile_frag_addr(uint32_t tile, int cb, int s, int lane, uint32_t& a0,
                                                 uint32_t& a1) {
    const int x = lane & 15, g = lane >> 4;
    const int col = cb + 4 * (x & 3);
    const int k0 = 32 * s + 8 * g + (x >> 2);
    const int k1 = k0 + 4;
    const int c0 = (col >> 3) ^ swz_mn(k0);
    const int c1 = (col >> 3) ^ swz_mn(k1);
    const int h = (col & 7) * 2;  // 0 or 8 bytes inside the chunk
    a0 = tile + (uint32_t)(k0 * C * 2 + c0 * 16 + h);
    a1 = tile + (uint32_t)(k1 * C * 2 + c1 * 16 + h);
}

// ---------------------------------------------------------------------------
// Epilogue: lane holds C[m][n .. n+3] of each 16x16 block (i, j).
// ---------------------------------------------------------------------------
template <int MI, int NI, int WM, int WN, int EPI>
__device__ __forceinline__ void epilogue(const f32x4_t (&acc)[MI][NI], const GemmArgs& args, int m0,
                                         int n0, int wm, int wn, int lr, int lq) {
    const int mb = m0 + wm * WM + lr;
    if constexpr (EPI == EPI_F32) {
        float* C = reinterpret_cast<float*>(args.C);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int m = mb + i * 16;
            if (m >= args.M) continue;
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int n = n0 + wn * WN + j * 16 + lq * 4;
                if (n >= args.N) continue;
                f32x4_t* p = reinterpret_cast<f32x4_t*>(C + (size_t)m * args.ldc + n);
                f32x4_t v = acc[i][j];
                if (args.accumulate) v += *p;
                *p = v;
            }
        }
    } else if constexpr (EPI == EPI_BF16 || EPI == EPI_GELU) {
        uint16_t* C = reinterpret_cast<uint16_t*>(args.C);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int m = mb + i * 16;
            if (m >= args.M) continue;
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int n = n0 + wn * WN + j * 16 + lq * 4;
                if (n >= args.N) continue;
                const f32x4_t v = acc[i][j];
                u32x2_t o;
                if constexpr (EPI == EPI_GELU) {
                    o[0] = pack_bf16x2(gelu_f(v[0]), gelu_f(v[1]));
                    o[1] = pack_bf16x2(gelu_f(v[2]), gelu_f(v[3]));
                    if (args.C2) {
                        u32x2_t h;
                        h[0] = pack_bf16x2(v[0], v[1]);
                        h[1] = pack_bf16x2(v[2], v[3]);
                        *reinterpret_cast<u32x2_t*>(args.C2 + (size_t)m * args.ldc2 + n) = h;
                    }
                } else {
                    o[0] = pack_bf16x2(v[0], v[1]);
                    o[1] = pack_bf16x2(v[2], v[3]);
                }
                *reinterpret_cast<u32x2_t*>(C + (size_t)m * args.ldc + n) = o;
            }
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
        uint16_t* C = reinterpret_cast<uint16_t*>(args.C);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int m = mb + i * 16;
            if (m >= args.M) continue;
#pragma unroll
            for (int j = 0; j < NI / 2; ++j) {
                const int n = n0 + wn * (WN / 2) + j * 16 + lq * 4;
                if (n >= args.N) continue;
                const f32x4_t g = acc[i][j];
                const f32x4_t u = acc[i][j + NI / 2];
                float z[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) z[r] = g[r] * sigmoid_f(g[r]) * u[r];
                u32x2_t o;
                o[0] = pack_bf16x2(z[0], z[1]);
                o[1] = pack_bf16x2(z[2], z[3]);
                *reinterpret_cast<u32x2_t*>(C + (size_t)m * args.ldc + n) = o;
                if (args.C2) {
                    u32x2_t hg, hu;
                    hg[0] = pack_bf16x2(g[0], g[1]);
                    hg[1] = pack_bf16x2(g[2], g[3]);
                    hu[0] = pack_bf16x2(u[0], u[1]);
                    hu[1] = pack_bf16x2(u[2], u[3]);
                    uint16_t* hrow = args.C2 + (size_t)m * args.ldc2;
                    *reinterpret_cast<u32x2_t*>(hrow + n) = hg;
                    *reinterpret_cast<u32x2_t*>(hrow + args.f + n) = hu;
                }
            }
        }
    } else if constexpr (EPI == EPI_GELU_BWD || EPI == EPI_SWIGLU_BWD) {
        uint16_t* C = reinterpret_cast<uint16_t*>(args.C);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int m = mb + i * 16;
            if (m >= args.M) continue;
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int n = n0 + wn * WN + j * 16 + lq * 4;
                if (n >= args.N) continue;
                const f32x4_t dz = acc[i][j];
                const uint16_t* hrow = args.aux + (size_t)m * args.ldc2;
                uint16_t* crow = C + (size_t)m * args.ldc;
                if constexpr (EPI == EPI_GELU_BWD) {
                    const u32x2_t a = *reinterpret_cast<const u32x2_t*>(hrow + n);
                    float x[4] = {bf16_bits_to_f32(a[0] & 0xffffu), bf16_bits_to_f32(a[0] >> 16),
                                  bf16_bits_to_f32(a[1] & 0xffffu), bf16_bits_to_f32(a[1] >> 16)};
                    u32x2_t o;
                    o[0] = pack_bf16x2(dz[0] * gelu_grad_f(x[0]), dz[1] * gelu_grad_f(x[1]));
                    o[1] = pack_bf16x2(dz[2] * gelu_grad_f(x[2]), dz[3] * gelu_grad_f(x[3]));
                    *reinterpret_cast<u32x2_t*>(crow + n) = o;
                } else {
                    const u32x2_t gb = *reinterpret_cast<const u32x2_t*>(hrow + n);
                    const u32x2_t ub = *reinterpret_cast<const u32x2_t*>(hrow + args.f + n);
                    float g[4] = {bf16_bits_to_f32(gb[0] & 0xffffu), bf16_bits_to_f32(gb[0] >> 16),
                                  bf16_bits_to_f32(gb[1] & 0xffffu), bf16_bits_to_f32(gb[1] >> 16)};
                    float u[4] = {bf16_bits_to_f32(ub[0] & 0xffffu), bf16_bits_to_f32(ub[0] >> 16),
                                  bf16_bits_to_f32(ub[1] & 0xffffu), bf16_bits_to_f32(ub[1] >> 16)};
                    float dg[4], du[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float s = sigmoid_f(g[r]);
                        du[r] = dz[r] * g[r] * s;
                        dg[r] = dz[r] * u[r] * (s + g[r] * s * (1.0f - s));
                    }
                    u32x2_t og, ou;
                    og[0] = pack_bf16x2(dg[0], dg[1]);
                    og[1] = pack_bf16x2(dg[2], dg[3]);
                    ou[0] = pack_bf16x2(du[0], du[1]);
                    ou[1] = pack_bf16x2(du[2], du[3]);
                    *reinterpret_cast<u32x2_t*>(crow + n) = og;
                    *reinterpret_cast<u32x2_t*>(crow + args.f + n) = ou;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int STAGES, int WAVES_M, int WAVES_N, bool A_T, bool B_KN, int EPI>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
gemm_kernel(const GemmArgs args) {
    constexpr int NWAVES = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int MI = WM / 16, NI = WN / 16;
    constexpr bool SWIGLU = (EPI == EPI_SWIGLU);
    constexpr int BNZ = SWIGLU ? BN / 2 : BN;  // output columns per tile
    constexpr int STAGE_BYTES = (BM + BN) * BK * 2;
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BK == 32 || BK == 64, "BK is 32 or 64");
    static_assert(!SWIGLU || (NI % 2 == 0 && B_KN), "SwiGLU needs an even gate/up split");
    static_assert(STAGES >= 2, "at least two stages");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int lr = lane & 15, lq = lane >> 4;

    // --- tile index (XCD-aware, grouped) ---
    const int tiles_m = (args.M + BM - 1) / BM;
    const int tiles_n = (args.N + BNZ - 1) / BNZ;
    const int T = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int per = T >> 3;
    const int lid = (bid < per * 8) ? (bid & 7) * per + (bid >> 3) : bid;
    const int group = lid / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gsz = min(tiles_m - first_m, kGroupM);
    const int in_group = lid % (kGroupM * tiles_n);
    const int tm = first_m + in_group % gsz;
    const int tn = in_group / gsz;
    const int m0 = tm * BM;
    const int n0 = tn * BNZ;

    // --- DMA descriptors and per-lane offsets ---
    const i32x4_t rsA = make_rsrc(args.A, args.a_bytes);
    const i32x4_t rsB = make_rsrc(args.B, args.b_bytes);
    using ADma = typename std::conditional<A_T, MNTileDma<BM, BK, NWAVES>, KTileDma<BM, BK, NWAVES>>::type;
    using BDma = typename std::conditional<B_KN, MNTileDma<BN, BK, NWAVES>, KTileDma<BN, BK, NWAVES>>::type;
    ADma da;
    BDma db;
    if constexpr (A_T) {
        da.init(wave, lane, args.lda, IdentityCols{m0, args.M});
    } else {
        da.init(wave, lane, m0, args.lda);
    }
    if constexpr (B_KN) {
        if constexpr (SWIGLU) {
            db.init(wave, lane, args.ldb, SwigluCols<WN>{n0, args.f});
        } else {
            db.init(wave, lane, args.ldb, IdentityCols{n0, args.N});
        }
    } else {
        db.init(wave, lane, n0, args.ldb);
    }
    const uint32_t a_step = A_T ? (uint32_t)BK * (uint32_t)args.lda * 2u : (uint32_t)BK * 2u;
    const uint32_t b_step = B_KN ? (uint32_t)BK * (uint32_t)args.ldb * 2u : (uint32_t)BK * 2u;
    const uint32_t lds0 = lds_addr(smem);
    constexpr int LOADS_PER_STAGE = ADma::kPerWave + BDma::kPerWave;

    auto issue = [&](int kt) {
        const uint32_t st = lds0 + (uint32_t)((kt % STAGES) * STAGE_BYTES);
        da.issue(rsA, st, wave, (uint32_t)kt * a_step);
        db.issue(rsB, st + BM * BK * 2, wave, (uint32_t)kt * b_step);
    };

    // --- fragment base addresses (stage 0) ---
    uint32_t fa[MI][BK / 32][2];
    uint32_t fb[NI][BK / 32][2];
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            if constexpr (A_T) {
                mntile_frag_addr<BM>(lds0, wm * WM + 16 * i, s, lane, fa[i][s][0], fa[i][s][1]);
            } else {
                fa[i][s][0] = ktile_frag_addr<BK>(lds0, wm * WM + 16 * i, s, lane);
                fa[i][s][1] = 0;
            }
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            if constexpr (B_KN) {
                mntile_frag_addr<BN>(lds0 + BM * BK * 2, wn * WN + 16 * j, s, lane, fb[j][s][0], fb[j][s][1]);
            } else {
                fb[j][s][0] = ktile_frag_addr<BK>(lds0 + BM * BK * 2, wn * WN + 16 * j, s, lane);
                fb[j][s][1] = 0;
            }
        }
    }

    f32x4_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int KT = (args.K + BK - 1) / BK;
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < KT) issue(st);

    for (int kt = 0; kt < KT; ++kt) {
        if (kt + STAGES - 2 < KT) {
            wait_vmcnt_barrier<(STAGES - 2) * LOADS_PER_STAGE>();
        } else {
            wait_vmcnt_barrier<0>();
        }
        if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1);

        const uint32_t so = (uint32_t)((kt % STAGES) * STAGE_BYTES);
#pragma unroll
        for (int s = 0; s < BK / 32; ++s) {
            bf16x8_t af[MI], bfr[NI];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                if constexpr (A_T) af[i] = lds_read_tr2(fa[i][s][0] + so, fa[i][s][1] + so);
                else af[i] = lds_read16(fa[i][s][0] + so);
            }
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                if constexpr (B_KN) bfr[j] = lds_read_tr2(fb[j][s][0] + so, fb[j][s][1] + so);
                else bfr[j] = lds_read16(fb[j][s][0] + so);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    epilogue<MI, NI, WM, WN, EPI>(acc, args, m0, n0, wm, wn, lr, lq);
}

}  // namespace tps

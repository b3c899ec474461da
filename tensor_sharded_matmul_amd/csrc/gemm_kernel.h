// gemm_kernel.h — bf16 MFMA GEMM for gfx950 with the epilogues of a TP shard.
//
// One template computes C[M,N] = op(A) op(B) for the three operand layouts a
// tensor-parallel shard needs ([TPSP] "矩阵乘法的两种切法": forward Y = X W,
// backward dX = dY W^T and dW = X^T dY):
//   NN  A[M][K], B[K][N]   forward products
//   NT  A[M][K], B[N][K]   input gradients  (dY W^T)
//   TN  A[K][M], B[K][N]   weight gradients (X^T dY)
// and fuses the shard's elementwise work into the epilogue
// ([TPSP] "MLP：先列后行": GeLU / SiLU(gate)*up are local, per element).
//
// Design (gfx950 / CDNA4):
//  * 256 threads = 4 waves of 64 in a 2x2 grid; each wave owns a
//    (BM/2) x (BN/2) sub-tile of C held in f32 accumulators
//    (128 x 128 -> 256 accumulator registers per lane).
//  * v_mfma_f32_16x16x32_bf16, with operands swapped (the MFMA "A" operand is
//    the B tile) so that each lane ends with 4 *consecutive columns* of one C
//    row: epilogue stores are 16-byte (f32) or 8-byte (bf16) vectors.
//  * LDS holds both tiles K-contiguous ([row][k], 64 k per stage, rows padded
//    to 72 elements = 144 B so that the 16 rows read by one MFMA fragment load
//    fall in distinct banks). Two stages (double buffer), one barrier per
//    K step; the next stage's global loads are in flight during the MFMAs.
//  * Operands stored MN-contiguous in HBM (B in NN, both in TN) are loaded as
//    8x8 bf16 blocks and transposed in registers with byte permutes before
//    the 16-byte LDS writes, so the MFMA loop is the same for every layout.
//  * Workgroup -> tile mapping is XCD-aware: the hardware deals workgroups
//    round-robin over the 8 XCDs, so consecutive blocks of tiles are mapped
//    to one XCD (sharing its L2), grouped GROUP_M tile rows at a time.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kBK = 64;        // K per pipeline stage
constexpr int kLdsStride = 72; // bf16 elements per LDS row (64 + 8 pad)
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
// Global -> register loaders. Each returns the 16-byte chunks a thread owns;
// the matching LDS writer puts them in the [row][k] tile.
// ---------------------------------------------------------------------------

// K-contiguous operand: rows x 64 k. Chunk q = tid + 256 i: row q/8, k-chunk q%8.
template <int ROWS>
struct KContigLoader {
    static constexpr int kLoads = ROWS * 8 / kThreads;
    static_assert(ROWS * 8 % kThreads == 0, "tile rows must be a multiple of 32");
    u32x4_t r[kLoads];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int ld,
                                         int row0, int rows_total, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int q = tid + kThreads * i;
            const int row = row0 + (q >> 3);
            const int kc = k0 + (q & 7) * 8;
            if (row < rows_total) {
                r[i] = *reinterpret_cast<const u32x4_t*>(base + (size_t)row * ld + kc);
            } else {
                r[i] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    }

    __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int q = tid + kThreads * i;
            *reinterpret_cast<u32x4_t*>(lds + (q >> 3) * kLdsStride + (q & 7) * 8) = r[i];
        }
    }
};

// MN-contiguous operand stored [K][cols]: 64 k x ROWS columns, loaded as 8x8
// blocks (block b: k-chunk b%8, column group b/8) and transposed in registers.
// COLMAP maps a tile column group to a global column (or -1 = zero fill).
template <int ROWS>
struct MNContigLoader {
    static constexpr int kBlocks = ROWS;  // 8 k-chunks x ROWS/8 column groups
    static constexpr int kPerThread = (kBlocks + kThreads - 1) / kThreads;
    u32x4_t r[kPerThread][8];

    template <class ColMap>
    __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int ld,
                                         int k0, int k_total, int tid, const ColMap& colmap) {
#pragma unroll
        for (int p = 0; p < kPerThread; ++p) {
            const int b = tid + kThreads * p;
            const int kb = b & 7;
            const int cg = b >> 3;
            const int gcol = (b < kBlocks) ? colmap(cg * 8) : -1;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int gk = k0 + kb * 8 + kk;
                if (gcol >= 0 && gk < k_total) {
                    r[p][kk] = *reinterpret_cast<const u32x4_t*>(base + (size_t)gk * ld + gcol);
                } else {
                    r[p][kk] = u32x4_t{0u, 0u, 0u, 0u};
                }
            }
        }
    }

    __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
        for (int p = 0; p < kPerThread; ++p) {
            const int b = tid + kThreads * p;
            if (b >= kBlocks) continue;
            const int kb = b & 7;
            const int cg = b >> 3;
            // r[p][kk] word w holds columns (2w, 2w+1) of row k = kb*8 + kk.
            // out[e] word w must hold rows (2w, 2w+1) of column e.
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                u32x4_t o;
                o[0] = __builtin_amdgcn_perm(r[p][1][e >> 1], r[p][0][e >> 1], sel);
                o[1] = __builtin_amdgcn_perm(r[p][3][e >> 1], r[p][2][e >> 1], sel);
                o[2] = __builtin_amdgcn_perm(r[p][5][e >> 1], r[p][4][e >> 1], sel);
                o[3] = __builtin_amdgcn_perm(r[p][7][e >> 1], r[p][6][e >> 1], sel);
                *reinterpret_cast<u32x4_t*>(lds + (cg * 8 + e) * kLdsStride + kb * 8) = o;
            }
        }
    }
};

struct IdentityCols {
    int col0, cols_total;
    __device__ __forceinline__ int operator()(int c) const {
        const int g = col0 + c;
        return g < cols_total ? g : -1;
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
        if (j >= f) return -1;
        return p < WN / 2 ? j : f + j;
    }
};

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int BM, int BN, bool A_T, bool B_KN, int EPI>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_kernel(const GemmArgs args) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MI = WM / 16, NI = WN / 16;
    constexpr bool SWIGLU = (EPI == EPI_SWIGLU);
    constexpr int BNZ = SWIGLU ? BN / 2 : BN;  // output columns per tile
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(!SWIGLU || (NI % 2 == 0 && B_KN), "SwiGLU needs an even gate/up split");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * kLdsStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
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

    using ALoader = typename std::conditional<A_T, MNContigLoader<BM>, KContigLoader<BM>>::type;
    using BLoader = typename std::conditional<B_KN, MNContigLoader<BN>, KContigLoader<BN>>::type;
    ALoader la;
    BLoader lb;

    const int KT = (args.K + kBK - 1) / kBK;

    auto load_stage = [&](int kt) {
        const int k0 = kt * kBK;
        if constexpr (A_T) {
            la.load(args.A, args.lda, k0, args.K, tid, IdentityCols{m0, args.M});
        } else {
            la.load(args.A, args.lda, m0, args.M, k0, tid);
        }
        if constexpr (B_KN) {
            if constexpr (SWIGLU) {
                lb.load(args.B, args.ldb, k0, args.K, tid, SwigluCols<WN>{n0, args.f});
            } else {
                lb.load(args.B, args.ldb, k0, args.K, tid, IdentityCols{n0, args.N});
            }
        } else {
            lb.load(args.B, args.ldb, n0, args.N, k0, tid);
        }
    };
    auto store_stage = [&](int buf) {
        uint16_t* As = smem + buf * (BM + BN) * kLdsStride;
        uint16_t* Bs = As + BM * kLdsStride;
        la.store(As, tid);
        lb.store(Bs, tid);
    };

    f32x4_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if (KT > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load_stage(kt + 1);

        const uint16_t* As = smem + cur * (BM + BN) * kLdsStride + (wm * WM + lr) * kLdsStride;
        const uint16_t* Bs = smem + cur * (BM + BN) * kLdsStride + (BM + wn * WN + lr) * kLdsStride;
#pragma unroll
        for (int s = 0; s < kBK / 32; ++s) {
            bf16x8_t af[MI], bfr[NI];
            const int koff = s * 32 + lq * 8;
#pragma unroll
            for (int i = 0; i < MI; ++i)
                af[i] = *reinterpret_cast<const bf16x8_t*>(As + i * 16 * kLdsStride + koff);
#pragma unroll
            for (int j = 0; j < NI; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + j * 16 * kLdsStride + koff);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j],
                                                                         0, 0, 0);
        }

        if (kt + 1 < KT) store_stage(cur ^ 1);
        __syncthreads();
    }

    // --- epilogue: lane holds C[m][n .. n+3] for each (i, j) block ---
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

}  // namespace tps

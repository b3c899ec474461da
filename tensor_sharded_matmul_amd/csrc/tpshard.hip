// tpshard.hip — host side of libtpshard.so: argument validation, kernel
// selection and launch for every entry point declared in include/tpshard.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/tpshard.h"
#include "decode.h"
#include "gemm_kernel.h"
#include "mid_tile.h"

namespace tps {

// ---------------------------------------------------------------------------
// Errors
// ---------------------------------------------------------------------------
static thread_local std::string g_last_error;

tp_status fail(tp_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

static tp_status ok() {
    g_last_error.clear();
    return TP_OK;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define TP_CHECK_PTR(p, name)                                                             \
    do {                                                                                  \
        if ((p) == nullptr) return fail(TP_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);  \
        if (!aligned16(p))                                                                \
            return fail(TP_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, name);   \
    } while (0)

// Token-sized buffers ([N, *]) may be NULL when N == 0 (an empty torch tensor).
#define TP_CHECK_TOK_PTR(p, name)                                                         \
    do {                                                                                  \
        if (N != 0) TP_CHECK_PTR(p, name);                                                \
        else TP_CHECK_OPT_PTR(p, name);                                                   \
    } while (0)

#define TP_CHECK_OPT_PTR(p, name)                                                         \
    do {                                                                                  \
        if ((p) != nullptr && !aligned16(p))                                              \
            return fail(TP_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, name);   \
    } while (0)

static tp_status check_tokens(const char* fn, int64_t N) {
    if (N < 0) return fail(TP_ERR_INVALID_ARG, "%s: N = %lld < 0", fn, (long long)N);
    if (N > (int64_t)1 << 30) return fail(TP_ERR_UNSUPPORTED, "%s: N = %lld too large", fn, (long long)N);
    return TP_OK;
}

// Widths become the row pitches of the GEMM operands (a SwiGLU weight's is
// twice its width); 2^20 keeps every pitch inside the kernel's limits.
static constexpr int64_t kMaxWidth = (int64_t)1 << 20;

static tp_status check_width(const char* fn, const char* name, int64_t v) {
    if (v <= 0) return fail(TP_ERR_INVALID_ARG, "%s: %s = %lld must be positive", fn, name, (long long)v);
    if (v % 64 != 0)
        return fail(TP_ERR_UNSUPPORTED, "%s: %s = %lld is not a multiple of 64", fn, name, (long long)v);
    if (v > kMaxWidth) return fail(TP_ERR_UNSUPPORTED, "%s: %s = %lld too large", fn, name, (long long)v);
    return TP_OK;
}

// Element offsets of every operand must fit the kernels' 32-bit row indices
// times a 64-bit stride; the product itself is formed in size_t.
static tp_status check_elems(const char* fn, int64_t rows, int64_t cols) {
    if (rows * cols > ((int64_t)1 << 40)) return fail(TP_ERR_UNSUPPORTED, "%s: operand too large", fn);
    return TP_OK;
}

#define TP_TRY(expr)                      \
    do {                                  \
        tp_status _st = (expr);           \
        if (_st != TP_OK) return _st;     \
    } while (0)

// ---------------------------------------------------------------------------
// GEMM dispatch
// ---------------------------------------------------------------------------
// GEMM launches: defined in gemm_launch.h and instantiated, one layout and
// epilogue family per file, in the gemm_*.hip sources (compiled in parallel).
template <bool A_T, bool B_KN, int EPI>
tp_status launch_gemm(const char* fn, GemmArgs a, hipStream_t s);
// Decode-sized forward products (gemm_decode.hip).
template <int EPI>
tp_status launch_decode(const char* fn, const GemmArgs& a, const DecodePlan& p, void* ws, hipStream_t s);

static GemmArgs make_args(const void* A, const void* B, void* C, int M, int N, int K, int lda, int ldb,
                          int ldc) {
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.A = static_cast<const uint16_t*>(A);
    a.B = static_cast<const uint16_t*>(B);
    a.C = C;
    a.M = M;
    a.N = N;
    a.K = K;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.ksplit = 1;
    a.kper = K;
    return a;
}

// ---------------------------------------------------------------------------
// Split-K. A product with too few output tiles for the CUs (decode-sized
// token counts, or the narrow attention shards) has K split over workgroups:
// each writes an fp32 partial of the whole product to scratch memory, and
// splitk_reduce sums the partials in split order and applies the epilogue
// (store, accumulate, GeLU, SwiGLU). (Summing in the GEMM kernel by the last
// workgroup of a tile needs device-scope fences, which write back and
// invalidate each XCD's L2 for every workgroup: measured 1.5-3x slower.)
// The scratch belongs to the caller: every entry point that may need some
// takes a device buffer and its size, and a host-only query gives the bytes
// a call needs. The library allocates nothing, keeps no pointer and never
// synchronises.
// ---------------------------------------------------------------------------
struct Workspace {
    void* p;
    size_t bytes;
};

// The caller's workspace holds `need` bytes (checked before any launch).
static tp_status check_workspace(const char* fn, const Workspace& ws, size_t need) {
    if (ws.p != nullptr && !aligned16(ws.p))
        return fail(TP_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
    if (need == 0) return TP_OK;
    if (ws.p == nullptr || ws.bytes < need)
        return fail(TP_ERR_INVALID_ARG, "%s: the call needs %zu bytes of workspace, got %zu%s", fn, need,
                    ws.p ? ws.bytes : (size_t)0, ws.p ? "" : " (NULL)");
    return TP_OK;
}

// out[m][n..n+3] from the sum over splits of ws[s][m][*]. A wave covers
// 64 / S output quads (4 columns each) with S lanes per quad (S a power of
// two, chosen so that a lane has at most kReduceLoads splits to add): lane si
// of a group loads splits si, si + S, ... (all of its loads issued before
// the first add, so that each lane keeps several in flight), adds them in
// that order, the S partial sums are combined with butterfly shuffles, and
// lane 0 of the group applies the epilogue. EPI_SWIGLU: ws holds [gate | up]
// (2 f columns).
constexpr int kReduceLoads = 4;

template <int EPI>
__global__ void __launch_bounds__(256) splitk_reduce(const float* __restrict__ ws, int ksplit, int S, int M,
                                                     int Nw, int Nout, void* C, int ldc, uint16_t* C2,
                                                     int ldc2, int f, int accumulate) {
    const int lane = threadIdx.x & 63;
    const int si = lane % S;
    const int q = Nout / 4;
    const int64_t total = (int64_t)M * q;
    const int64_t quads_per_block = (int64_t)(blockDim.x / 64) * (64 / S);
    const int64_t first = (int64_t)blockIdx.x * quads_per_block + (threadIdx.x / 64) * (64 / S) + lane / S;
    const size_t split_stride = (size_t)M * Nw;
    for (int64_t idx = first; idx - lane / S < total; idx += (int64_t)gridDim.x * quads_per_block) {
        const bool live = idx < total;  // every lane runs the shuffles
        const int m = live ? (int)(idx / q) : 0, n = live ? (int)(idx % q) * 4 : 0;
        const float* row0 = ws + (size_t)m * Nw + n;
        f32x4_t v = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
        for (int base = 0; base < ksplit; base += kReduceLoads * S) {
            f32x4_t tv[kReduceLoads], tu[kReduceLoads];
#pragma unroll
            for (int r = 0; r < kReduceLoads; ++r) {
                const int sp = base + si + r * S;
                const bool ok = live && sp < ksplit;
                const float* p = row0 + (ok ? sp : 0) * split_stride;
                tv[r] = ok ? *reinterpret_cast<const f32x4_t*>(p) : f32x4_t{0.f, 0.f, 0.f, 0.f};
                if constexpr (EPI == EPI_SWIGLU)
                    tu[r] = ok ? *reinterpret_cast<const f32x4_t*>(p + f) : f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int r = 0; r < kReduceLoads; ++r) {
                v += tv[r];
                if constexpr (EPI == EPI_SWIGLU) u += tu[r];
            }
        }
        for (int off = S / 2; off > 0; off /= 2) {
            for (int r = 0; r < 4; ++r) {
                v[r] += __shfl_xor(v[r], off, 64);
                if constexpr (EPI == EPI_SWIGLU) u[r] += __shfl_xor(u[r], off, 64);
            }
        }
        if (!live || si != 0) continue;
        if constexpr (EPI == EPI_F32) {
            f32x4_t* p = reinterpret_cast<f32x4_t*>(static_cast<float*>(C) + (size_t)m * ldc + n);
            *p = accumulate ? *p + v : v;
        } else if constexpr (EPI == EPI_BF16) {
            *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(C) + (size_t)m * ldc + n) = pack4(v[0], v[1], v[2], v[3]);
        } else if constexpr (EPI == EPI_GELU) {
            *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(C) + (size_t)m * ldc + n) =
                pack4(gelu_f(v[0]), gelu_f(v[1]), gelu_f(v[2]), gelu_f(v[3]));
            if (C2) *reinterpret_cast<u32x2_t*>(C2 + (size_t)m * ldc2 + n) = pack4(v[0], v[1], v[2], v[3]);
        } else if constexpr (EPI == EPI_SWIGLU) {
            float z[4];
            for (int r = 0; r < 4; ++r) z[r] = v[r] * sigmoid_f(v[r]) * u[r];
            *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(C) + (size_t)m * ldc + n) = pack4(z[0], z[1], z[2], z[3]);
            if (C2) {
                *reinterpret_cast<u32x2_t*>(C2 + (size_t)m * ldc2 + n) = pack4(v[0], v[1], v[2], v[3]);
                *reinterpret_cast<u32x2_t*>(C2 + (size_t)m * ldc2 + f + n) = pack4(u[0], u[1], u[2], u[3]);
            }
        }
    }
}

// Compute units of the current device, queried once per device (callers on
// several threads may race to fill an entry; they store the same value).
int device_cus() {
    static std::atomic<int> cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cus[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cus[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// How a product is run: dec.nslab > 0 means the decode kernel (with
// dec.nsplit > 1, its f32 partials take `bytes` of workspace and
// splitk_reduce applies the epilogue); else ksplit == 0 means one launch of
// the tiled kernel; otherwise K is cut into ksplit chunks of kper (a
// multiple of 64) whose f32 partials take `bytes` of workspace and
// splitk_reduce applies the epilogue.
//  - At most 32 token rows (NN): the decode kernel when its slabs x splits
//    fit one wave of workgroups (decode.h).
//  - Other few-row products (M <= 64, NN): the weight is streamed from HBM
//    by one split workgroup per CU, in chunks of at least
//    TPS_SPLIT_MIN_KPER rows.
//  - Large products whose 256 x 256 tiles do not fill the CUs once (the
//    attention projections' N = 1024 or 1280 shard widths): the split count
//    that minimises an estimate of tile waves x chunk length plus the
//    partials' write and read is used.
// `a` describes the product as for launch_gemm<A_T, B_KN, EPI> (for SWIGLU:
// N = f output columns, B has 2 f columns). The activation-backward
// epilogues are never split (their reduce would need H as well).
#ifndef TPS_SPLIT_BLOCKS_PER_CU
#define TPS_SPLIT_BLOCKS_PER_CU 1  // split workgroups aimed at, per CU
#endif
#ifndef TPS_SPLIT_MIN_KPER
#define TPS_SPLIT_MIN_KPER 512  // smallest K chunk of one workgroup
#endif

struct SplitPlan {
    int ksplit = 0, kper = 0, Nw = 0;
    size_t bytes = 0;
    DecodePlan dec;
};

static SplitPlan make_plan(const GemmArgs& a, int Nw, int ksplit_wanted) {
    SplitPlan p;
    p.Nw = Nw;
    const int kper = ((a.K + ksplit_wanted - 1) / ksplit_wanted + 63) / 64 * 64;
    const int ksplit = (a.K + kper - 1) / kper;
    if (ksplit < 2 || (long long)ksplit * a.M * Nw >= (1LL << 31)) return p;
    p.ksplit = ksplit;
    p.kper = kper;
    p.bytes = (size_t)ksplit * a.M * Nw * sizeof(float);
    return p;
}

static SplitPlan plan_split(const GemmArgs& a, bool swiglu, bool nn, bool splittable) {
    SplitPlan none;
    none.Nw = swiglu ? 2 * a.N : a.N;  // columns of the product
    if (a.M == 0 || a.N == 0 || !splittable) return none;
    const int Nw = none.Nw;
    const long long cus = device_cus();
    if (a.M <= 64) {
        if (!nn) return none;
        const DecodePlan dec = decode_plan(a.M, a.K, Nw, a.ldb, (int)cus);
        if (dec.nslab > 0) {
            SplitPlan p = none;
            p.dec = dec;
            p.ksplit = dec.nsplit;
            p.bytes = dec.bytes;
            return p;
        }
        const int tm = splitk_tile_m(a.M);
        const long long tiles = (long long)((a.M + tm - 1) / tm) * ((Nw + 127) / 128);
        if (tiles >= 2 * cus || a.K < 2 * TPS_SPLIT_MIN_KPER) return none;
        const long long want = std::min<long long>((TPS_SPLIT_BLOCKS_PER_CU * cus + tiles - 1) / tiles,
                                                   a.K / TPS_SPLIT_MIN_KPER);
        return make_plan(a, Nw, (int)want);
    }
    const long long tiles = (long long)((a.M + 255) / 256) * ((Nw + 255) / 256);
    if (tiles >= cus || a.K < 2048) return none;
    // seconds: a CU finishes a 256 x 256 x k tile at ~4.6 TFLOP/s; partials
    // move at ~5 TB/s; the reduce launch costs ~4 us
    auto estimate = [&](int ksplit, int kper) {
        const double waves = (double)((tiles * ksplit + cus - 1) / cus);
        double t = waves * kper * (2.0 * 256 * 256 / 4.6e12);
        if (ksplit > 1) t += (double)ksplit * a.M * Nw * 8 / 5.0e12 + 4e-6;
        return t;
    };
    int best = 1;
    double t_best = estimate(1, a.K);
    for (int want = 2; want <= 16; ++want) {
        const int kper = ((a.K + want - 1) / want + 63) / 64 * 64;
        if (kper < 512) break;
        const int ksplit = (a.K + kper - 1) / kper;
        const double t = estimate(ksplit, kper);
        if (t < 0.95 * t_best) {
            best = ksplit;
            t_best = t;
        }
    }
    return best > 1 ? make_plan(a, Nw, best) : none;
}

template <int EPI>
constexpr bool reducible() {
    return EPI == EPI_F32 || EPI == EPI_BF16 || EPI == EPI_GELU || EPI == EPI_SWIGLU;
}

template <bool A_T, bool B_KN, int EPI>
static SplitPlan plan_of(const GemmArgs& a) {
    // (a product that runs on mid tiles over its whole K is not split)
    if (use_mid_tile<A_T, B_KN, EPI>(a.M, a.N, a.K)) return plan_split(a, false, false, false);
    return plan_split(a, EPI == EPI_SWIGLU, !A_T && B_KN, reducible<EPI>());
}

// Workspace bytes of a call that runs several products one after another on
// its stream (they reuse one buffer): the largest of their plans.
static size_t need_of(std::initializer_list<SplitPlan> plans) {
    size_t bytes = 0;
    for (const SplitPlan& p : plans) bytes = std::max(bytes, p.bytes);
    return bytes;
}

// A product with its epilogue, run as plan_of decides; a split product puts
// its partials in ws (sized by the caller from the same plan).
// The sum of ksplit f32 partials [ksplit][M][Nw] in ws, with a's epilogue.
template <int EPI>
static tp_status launch_reduce(const char* fn, const GemmArgs& a, int ksplit, int Nw, const void* ws,
                               hipStream_t s) {
    int S = 1;
    while (S * kReduceLoads < ksplit && S < 64) S *= 2;
    const long long quads = (long long)a.M * (a.N / 4);
    const long long per_block = 4 * (64 / S);
    const unsigned blocks = (unsigned)std::min<long long>((quads + per_block - 1) / per_block, 8192);
    hipLaunchKernelGGL(splitk_reduce<EPI>, dim3(blocks), dim3(256), 0, s, static_cast<const float*>(ws), ksplit, S,
                       a.M, Nw, a.N, a.C, a.ldc, a.C2, a.ldc2, a.f, a.accumulate);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return TP_OK;
}

template <bool A_T, bool B_KN, int EPI>
static tp_status run_gemm(const char* fn, const GemmArgs& a, void* ws, hipStream_t s) {
    if (a.M == 0 || a.N == 0) return TP_OK;
    const SplitPlan plan = plan_of<A_T, B_KN, EPI>(a);
    if constexpr (reducible<EPI>() && !A_T && B_KN) {
        if (plan.dec.nslab > 0) {
            if (plan.dec.nsplit > 1 && ws == nullptr)
                return fail(TP_ERR_INVALID_ARG, "%s: a split product without workspace", fn);
            TP_TRY(launch_decode<EPI>(fn, a, plan.dec, ws, s));
            if (plan.dec.nsplit == 1) return TP_OK;
            return launch_reduce<EPI>(fn, a, plan.dec.nsplit, plan.Nw, ws, s);
        }
    }
    if (plan.ksplit == 0) return launch_gemm<A_T, B_KN, EPI>(fn, a, s);
    if constexpr (reducible<EPI>()) {
        if (ws == nullptr) return fail(TP_ERR_INVALID_ARG, "%s: a split product without workspace", fn);
        GemmArgs p = a;
        p.C = ws;
        p.ldc = plan.Nw;
        p.N = plan.Nw;
        p.C2 = nullptr;
        p.accumulate = 0;
        p.ksplit = plan.ksplit;
        p.kper = plan.kper;
        TP_TRY((launch_gemm<A_T, B_KN, EPI_F32>(fn, p, s)));
        return launch_reduce<EPI>(fn, a, plan.ksplit, plan.Nw, p.C, s);
    } else {
        return fail(TP_ERR_UNSUPPORTED, "%s: split of an unsplittable epilogue", fn);
    }
}

// KV-head rules of the QKV split: t | n_kv (each rank takes n_kv / t heads),
// or n_kv < t with n_kv | t (each head replicated on t / n_kv ranks).
static tp_status check_kv_heads(const char* fn, int n_kv, int t) {
    if (t <= n_kv && n_kv % t != 0)
        return fail(TP_ERR_NOT_DIVISIBLE,
                    "%s: num_kv_heads (%d) must be a multiple of tensor_model_parallel_size (%d).", fn, n_kv,
                    t);
    if (t > n_kv && t % n_kv != 0)
        return fail(TP_ERR_NOT_DIVISIBLE,
                    "%s: tensor_model_parallel_size (%d) must be a multiple of num_kv_heads (%d) to "
                    "replicate KV heads.",
                    fn, t, n_kv);
    return TP_OK;
}

// dst[row][c0 + c] += src[row][c0 + c] for c in [0, w): one thread per 4
// columns, rows of width ld (f32).
__global__ void __launch_bounds__(256) kv_grad_accumulate_kernel(float* __restrict__ dst,
                                                                 const float* __restrict__ src, int64_t h,
                                                                 int ld, int c0, int w) {
    const int q = w >> 2;
    const int64_t total = h * q;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / q;
        const int c = c0 + (int)(i - row * q) * 4;
        f32x4_t* d = reinterpret_cast<f32x4_t*>(dst + row * ld + c);
        *d = *d + *reinterpret_cast<const f32x4_t*>(src + row * ld + c);
    }
}

// Vocab-parallel cross-entropy: the rank's local statistics from the GEMM's
// per-(row, wave column block) records {max, sum exp(z - max), z_target}.
// One wave per row: m = max over records, s = sum_p s_p exp(m_p - m),
// z_y = sum_p z_p (one record at most holds the target).
__global__ void __launch_bounds__(256) ce_stats_merge_kernel(const float* __restrict__ rec, int nparts, int M,
                                                             float* __restrict__ m_out, float* __restrict__ s_out,
                                                             float* __restrict__ zy_out) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;  // whole waves leave together
    const float* r = rec + (size_t)row * nparts * 3;
    float m = -__builtin_inff();
    for (int p = lane; p < nparts; p += 64) m = fmaxf(m, r[3 * p]);
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float s = 0.f, zy = 0.f;
    for (int p = lane; p < nparts; p += 64) {
        const float mp = r[3 * p];
        if (mp != -__builtin_inff()) s += r[3 * p + 1] * __expf(mp - m);
        zy += r[3 * p + 2];
    }
    for (int off = 32; off > 0; off >>= 1) {
        s += __shfl_xor(s, off, 64);
        zy += __shfl_xor(zy, off, 64);
    }
    if (lane == 0) {
        m_out[row] = m;
        s_out[row] = s;
        zy_out[row] = zy;
    }
}

// The exchange of the fused cross-entropy on one device: for each token the
// t ranks' local statistics (stacked [t][N]) give m = max_i m_i,
// S = sum_i s_i exp(m_i - m), z_y = sum_i z_y,i and loss = log S + m - z_y.
__global__ void __launch_bounds__(256) ce_combine_kernel(const float* __restrict__ mp, const float* __restrict__ sp,
                                                         const float* __restrict__ zp, int t, int64_t N,
                                                         float* __restrict__ loss, float* __restrict__ m_out,
                                                         float* __restrict__ S_out) {
    for (int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; n < N; n += (int64_t)gridDim.x * blockDim.x) {
        float m = -__builtin_inff();
        for (int i = 0; i < t; ++i) m = fmaxf(m, mp[i * N + n]);
        float S = 0.f, zy = 0.f;
        for (int i = 0; i < t; ++i) {
            S += sp[i * N + n] * __expf(mp[i * N + n] - m);
            zy += zp[i * N + n];
        }
        loss[n] = __logf(S) + m - zy;
        if (m_out) m_out[n] = m;
        if (S_out) S_out[n] = S;
    }
}

// Vocab-parallel embedding, forward: one workgroup per token. A token whose
// id is in this rank's rows gets its row (16-byte chunks; with accumulate
// the row is added to the output in f32 and rounded to bf16, exact when the
// output holds the zero row of another rank); any other token gets a zero
// row (left as it is with accumulate).
__global__ void __launch_bounds__(256) embed_fwd_kernel(const int32_t* __restrict__ ids,
                                                        const uint16_t* __restrict__ E, int64_t vocab_start,
                                                        int v_loc, int h, uint16_t* __restrict__ out,
                                                        int accumulate) {
    const int64_t n = blockIdx.x;
    const int64_t v = (int64_t)ids[n] - vocab_start;
    const bool inside = v >= 0 && v < v_loc;
    if (!inside && accumulate) return;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(E + (inside ? v : 0) * h);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + n * h);
    for (int c = threadIdx.x; c < h / 8; c += 256) {
        if (!inside) {
            dst[c] = u32x4_t{0u, 0u, 0u, 0u};
        } else if (!accumulate) {
            dst[c] = src[c];
        } else {
            const u32x4_t a = src[c], b = dst[c];
            u32x4_t r;
            for (int k = 0; k < 4; ++k) {
                const float lo = bf16_bits_to_f32(a[k] & 0xffffu) + bf16_bits_to_f32(b[k] & 0xffffu);
                const float hi = bf16_bits_to_f32(a[k] >> 16) + bf16_bits_to_f32(b[k] >> 16);
                r[k] = pack_bf16x2(lo, hi);
            }
            dst[c] = r;
        }
    }
}

// Vocab-parallel embedding, backward, in three kernels. Most rows of a shard
// receive no token (4096 tokens over Llama-3's 128256 ids put about 512 into
// a shard's 16128 rows), so the table gradient is mostly its zeros:
//  1. embed_clear_kernel clears the call's bookkeeping in the workspace: a
//     row count, one flag per table row and a list of rows.
//  2. embed_fill_mark_kernel stores the zeros of the whole table, one 16-byte
//     unit per thread in address order (the rate of a plain fill, every
//     store independent of any load), and its first threads mark the rows
//     the tokens use: the first token to flag a row (an atomic exchange)
//     appends it to the list (an atomic counter).
//  3. embed_rows_kernel gives each listed row a workgroup that sums the
//     gradient rows of the tokens whose id is vocab_start + v, in token
//     order, and overwrites the row's zeros.
// A row's h columns are spread over the 256 threads of its workgroup (4
// columns per thread per 1024, held in registers). The ids are scanned in
// chunks of 256, 16 chunks of ids loaded into registers at a time; a chunk's
// matching tokens are listed in ascending order (a wave ballot per 64 ids,
// the four waves' matches placed by prefix counts in LDS) and their rows
// added in that order. Masks and lists alternate between two LDS buffers, so
// a chunk without a match costs one barrier. Every row's sum is taken in
// token order: the result does not depend on scheduling or on the order of
// the list. The bookkeeping is cleared by every call, so the workspace's
// earlier contents never matter. (One workgroup per table row, storing its
// zeros or its sum, took 113-116 us on the Llama-3-70B shard: its register
// use, set by the summing path, limits the stores in flight.)
constexpr int kEmbedMaxH = 16384;

__global__ void __launch_bounds__(256) embed_clear_kernel(uint32_t* __restrict__ ws, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
        ws[i] = 0u;
}

__global__ void __launch_bounds__(256) embed_fill_mark_kernel(float* __restrict__ dE, int64_t units,
                                                              const int32_t* __restrict__ ids, int64_t vocab_start,
                                                              int64_t N, int v_loc, uint32_t* __restrict__ count,
                                                              uint32_t* __restrict__ used,
                                                              uint32_t* __restrict__ list) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < units) reinterpret_cast<f32x4_t*>(dE)[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (i < N) {
        const int64_t v = (int64_t)ids[i] - vocab_start;
        if (v >= 0 && v < v_loc && atomicExch(&used[v], 1u) == 0u) list[atomicAdd(count, 1u)] = (uint32_t)v;
    }
}

// Row `target - vocab_start` of dE: the sum, in token order, of the dY rows
// of the tokens whose id is `target` (the whole workgroup; chunk numbers
// continue from one row to the next so that the LDS buffers keep
// alternating).
__device__ __forceinline__ void embed_row_sum(const int32_t* __restrict__ ids, const float* __restrict__ dY,
                                              int64_t target, int N, int h, float* __restrict__ row,
                                              int (&list)[2][256], uint64_t (&masks)[2][4], int& chunk, int tid,
                                              int lane, int wave) {
    constexpr int Q = kEmbedMaxH / 1024;  // column quads per thread
    constexpr int U = 16;                 // id chunks loaded at a time
    f32x4_t acc[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < N; g += 256 * U) {
        int my[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int n = g + u * 256 + tid;
            my[u] = n < N ? ids[n] : -1;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (g + u * 256 >= N) break;  // uniform
            const int buf = chunk & 1;
            ++chunk;
            const bool match = my[u] >= 0 && (int64_t)my[u] == target;
            const uint64_t mask = __ballot(match);
            if (lane == 0) masks[buf][wave] = mask;
            __syncthreads();
            const int cnt = __popcll(masks[buf][0]) + __popcll(masks[buf][1]) + __popcll(masks[buf][2]) +
                            __popcll(masks[buf][3]);
            if (cnt == 0) continue;  // uniform
            int before = 0;
            for (int w = 0; w < wave; ++w) before += __popcll(masks[buf][w]);
            if (match) list[buf][before + __popcll(mask & ((1ull << lane) - 1ull))] = g + u * 256 + tid;
            __syncthreads();
            for (int k = 0; k < cnt; ++k) {
                const float* src = dY + (int64_t)list[buf][k] * h;
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const int c = q * 1024 + tid * 4;
                    if (c < h) acc[q] += *reinterpret_cast<const f32x4_t*>(src + c);
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int c = q * 1024 + tid * 4;
        if (c < h) *reinterpret_cast<f32x4_t*>(row + c) = acc[q];
    }
}

__global__ void __launch_bounds__(256) embed_rows_kernel(const int32_t* __restrict__ ids,
                                                         const float* __restrict__ dY, int64_t vocab_start, int N,
                                                         int h, float* __restrict__ dE,
                                                         const uint32_t* __restrict__ count,
                                                         const uint32_t* __restrict__ list) {
    __shared__ int lst[2][256];
    __shared__ uint64_t masks[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rows = (int)*count;  // the same in every thread: the loop below is uniform
    int chunk = 0;
    for (int b = blockIdx.x; b < rows; b += gridDim.x) {
        const int v = (int)list[b];
        embed_row_sum(ids, dY, vocab_start + v, N, h, dE + (int64_t)v * h, lst, masks, chunk, tid, lane, wave);
    }
}

// ---------------------------------------------------------------------------
// Fused-QKV regroup: a bit-exact gather of three contiguous column runs per
// row. A workgroup moves kRegroupRows whole output rows as 16-byte chunks in
// output order (coalesced writes, and reads coalesced within each run); a
// thread issues the loads of up to kRegroupLoads chunks before their stores.
// All index arithmetic is 32-bit within the workgroup's rows; the row base
// is 64-bit. (2 rows x 2 loads was the fastest of 1-32 rows x 2-8 loads on
// the Llama-3-70B t = 8 shapes: 9.3 us, against 7.0 us for a contiguous copy
// of the same bytes; the 256-byte K and V runs of each source row cost the
// difference.)
// ---------------------------------------------------------------------------
constexpr int kRegroupRows = 2, kRegroupLoads = 2;

__global__ void __launch_bounds__(256) qkv_regroup_kernel(const uint16_t* __restrict__ src,
                                                          uint16_t* __restrict__ dst, int64_t h,
                                                          int src_w, int q_w, int kv_w, int q_src0,
                                                          int k_src0, int v_src0) {
    const int out_w = q_w + 2 * kv_w;
    const int cpr = out_w >> 3;  // 16-byte chunks per output row
    const int64_t row0 = (int64_t)blockIdx.x * kRegroupRows;
    const int rows = (int)min<int64_t>(kRegroupRows, h - row0);
    const int total = rows * cpr;
    const uint16_t* s0 = src + row0 * src_w;
    uint16_t* d0 = dst + row0 * out_w;
    for (int base = threadIdx.x; base < total; base += kRegroupLoads * 256) {
        u32x4_t v[kRegroupLoads];
        int doff[kRegroupLoads];
#pragma unroll
        for (int u = 0; u < kRegroupLoads; ++u) {
            const int c = base + u * 256;
            if (c < total) {
                const int r = c / cpr;
                const int col = (c - r * cpr) << 3;
                const int scol = col < q_w ? q_src0 + col
                                 : col < q_w + kv_w ? k_src0 + (col - q_w)
                                                    : v_src0 + (col - q_w - kv_w);
                v[u] = *reinterpret_cast<const u32x4_t*>(s0 + r * src_w + scol);
                doff[u] = r * out_w + col;
            }
        }
#pragma unroll
        for (int u = 0; u < kRegroupLoads; ++u)
            if (base + u * 256 < total) *reinterpret_cast<u32x4_t*>(d0 + doff[u]) = v[u];
    }
}

}  // namespace tps

// ---------------------------------------------------------------------------
// Scratch of tp_col_linear_noalloc: device memory that is part of the code
// object, so that callers that cannot allocate (graph capture of a serving
// loop, harnesses that forbid allocation) can run split products. Each device
// holds its own copy at its own address, looked up once per device; in host
// code the array's name is not a device address.
// ---------------------------------------------------------------------------
namespace tps {

constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static tp_status scratch_address(const char* fn, void** out) {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(TP_ERR_UNSUPPORTED, "%s: device %d", fn, dev);
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(TP_ERR_HIP, "%s: address of the device scratch: %s", fn, hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = addr[dev];
    return TP_OK;
}

}  // namespace tps

// ---------------------------------------------------------------------------
// Each entry point that runs GEMMs first validates its sizes and describes
// its products (pointers may be NULL here: the host-only workspace queries
// run the same code), giving the workspace bytes its split products need.
// ---------------------------------------------------------------------------
namespace tps {

static tp_status check_act(const char* fn, int act, bool allow_none) {
    if ((allow_none && act == TP_ACT_NONE) || act == TP_ACT_GELU || act == TP_ACT_SWIGLU) return TP_OK;
    if (!allow_none && act == TP_ACT_NONE)
        return fail(TP_ERR_INVALID_ARG, "%s: act must be GELU or SWIGLU (got %d)", fn, act);
    return fail(TP_ERR_INVALID_ARG, "%s: unknown act %d", fn, act);
}

static tp_status col_linear_plan(const char* fn, const void* X, const void* W, void* Y, int64_t N, int64_t k,
                                 int64_t n_out, int act, void* H_save, GemmArgs& a, size_t& need) {
    TP_TRY(check_tokens(fn, N));
    TP_TRY(check_width(fn, "k", k));
    TP_TRY(check_width(fn, "n_out", n_out));
    TP_TRY(check_act(fn, act, true));
    if (act == TP_ACT_NONE && H_save != nullptr)
        return fail(TP_ERR_INVALID_ARG, "%s: H_save must be NULL for act NONE", fn);
    const int64_t n_w = act == TP_ACT_SWIGLU ? 2 * n_out : n_out;
    TP_TRY(check_elems(fn, N, k));
    TP_TRY(check_elems(fn, k, n_w));
    TP_TRY(check_elems(fn, N, n_w));
    a = make_args(X, W, Y, (int)N, (int)n_out, (int)k, (int)k, (int)n_w, (int)n_out);
    a.C2 = static_cast<uint16_t*>(H_save);
    a.ldc2 = (int)n_w;
    a.f = (int)n_out;
    need = act == TP_ACT_NONE   ? plan_of<false, true, EPI_BF16>(a).bytes
           : act == TP_ACT_GELU ? plan_of<false, true, EPI_GELU>(a).bytes
                                : plan_of<false, true, EPI_SWIGLU>(a).bytes;
    return TP_OK;
}

static tp_status col_linear_run(const char* fn, const GemmArgs& a, int act, void* ws, hipStream_t s) {
    if (act == TP_ACT_NONE) return run_gemm<false, true, EPI_BF16>(fn, a, ws, s);
    if (act == TP_ACT_GELU) return run_gemm<false, true, EPI_GELU>(fn, a, ws, s);
    return run_gemm<false, true, EPI_SWIGLU>(fn, a, ws, s);
}

static tp_status row_partial_plan(const char* fn, const void* Z, const void* W, float* P, int64_t N,
                                  int64_t k_loc, int64_t n, int accumulate, GemmArgs& a, size_t& need) {
    TP_TRY(check_tokens(fn, N));
    TP_TRY(check_width(fn, "k_loc", k_loc));
    TP_TRY(check_width(fn, "n", n));
    TP_TRY(check_elems(fn, N, k_loc));
    TP_TRY(check_elems(fn, k_loc, n));
    TP_TRY(check_elems(fn, N, n));
    a = make_args(Z, W, P, (int)N, (int)n, (int)k_loc, (int)k_loc, (int)n, (int)n);
    a.accumulate = accumulate ? 1 : 0;
    need = plan_of<false, true, EPI_F32>(a).bytes;
    return TP_OK;
}

// chunk c of the chunked row partial: token rows [c rows, (c + 1) rows),
// rows = ceil(N / nchunks) rounded up to 16
// Token rows [r0, r1) of chunk c when N rows are cut into nchunks chunks of
// ceil(N / nchunks) rows rounded up to 16 (the last may be shorter or empty).
static void chunk_rows(int64_t N, int nchunks, int c, int64_t& r0, int64_t& r1) {
    const int64_t rows = ((N + nchunks - 1) / nchunks + 15) / 16 * 16;
    r0 = std::min<int64_t>(N, c * rows);
    r1 = std::min<int64_t>(N, r0 + rows);
}

static tp_status check_nchunks(const char* fn, int32_t nchunks) {
    if (nchunks < 1 || nchunks > 64) return fail(TP_ERR_INVALID_ARG, "%s: nchunks = %d outside [1, 64]", fn, nchunks);
    return TP_OK;
}

static GemmArgs row_chunk(const void* Z, const void* W, float* P, int64_t N, int64_t k_loc, int64_t n,
                          int accumulate, int nchunks, int c) {
    int64_t r0, r1;
    chunk_rows(N, nchunks, c, r0, r1);
    GemmArgs a = make_args(Z ? static_cast<const uint16_t*>(Z) + r0 * k_loc : nullptr, W, P ? P + r0 * n : nullptr,
                           (int)(r1 - r0), (int)n, (int)k_loc, (int)k_loc, (int)n, (int)n);
    a.accumulate = accumulate ? 1 : 0;
    return a;
}

static tp_status row_chunked_plan(const char* fn, int64_t N, int64_t k_loc, int64_t n, int32_t nchunks,
                                  size_t& need) {
    TP_TRY(check_tokens(fn, N));
    TP_TRY(check_width(fn, "k_loc", k_loc));
    TP_TRY(check_width(fn, "n", n));
    TP_TRY(check_nchunks(fn, nchunks));
    TP_TRY(check_elems(fn, N, k_loc));
    TP_TRY(check_elems(fn, k_loc, n));
    TP_TRY(check_elems(fn, N, n));
    need = 0;  // the chunks run one after another and reuse one workspace
    for (int c = 0; c < nchunks; ++c)
        need = std::max(need, plan_of<false, true, EPI_F32>(row_chunk(nullptr, nullptr, nullptr, N, k_loc, n, 0,
                                                                       nchunks, c)).bytes);
    return TP_OK;
}

static tp_status mlp_fwd_plan(const char* fn, const void* X, const void* W_in, const void* W_out, int64_t N,
                              int64_t h, int64_t f, int act, void* Z, void* H_save, float* P, int accumulate,
                              GemmArgs& a, GemmArgs& b, size_t& need) {
    TP_TRY(check_act(fn, act, false));
    TP_TRY(check_tokens(fn, N));
    TP_TRY(check_width(fn, "h", h));
    TP_TRY(check_width(fn, "f", f));
    const int64_t n_w = act == TP_ACT_SWIGLU ? 2 * f : f;
    TP_TRY(check_elems(fn, N, h));
    TP_TRY(check_elems(fn, h, n_w));
    TP_TRY(check_elems(fn, N, n_w));
    a = make_args(X, W_in, Z, (int)N, (int)f, (int)h, (int)h, (int)n_w, (int)f);
    a.C2 = static_cast<uint16_t*>(H_save);
    a.ldc2 = (int)n_w;
    a.f = (int)f;
    b = make_args(Z, W_out, P, (int)N, (int)h, (int)f, (int)f, (int)h, (int)h);
    b.accumulate = accumulate ? 1 : 0;
    need = need_of({act == TP_ACT_GELU ? plan_of<false, true, EPI_GELU>(a) : plan_of<false, true, EPI_SWIGLU>(a),
                    plan_of<false, true, EPI_F32>(b)});
    return TP_OK;
}

// The backward's products: a = dZ with the activation backward -> dH (NT),
// b = dX_part (NT), c = dW_in (TN), d = dW_out (TN); a product whose output
// is NULL is not run (its workspace is not counted).
static tp_status mlp_bwd_plan(const char* fn, const void* X, const void* W_in, const void* W_out,
                              const void* H_save, const void* Z, const void* dY, int64_t N, int64_t h, int64_t f,
                              int act, void* dH, float* dX_part, float* dW_in, float* dW_out, int accumulate,
                              bool query, GemmArgs& a, GemmArgs& b, GemmArgs& c, GemmArgs& d, size_t& need) {
    TP_TRY(check_act(fn, act, false));
    TP_TRY(check_tokens(fn, N));
    TP_TRY(check_width(fn, "h", h));
    TP_TRY(check_width(fn, "f", f));
    const int64_t n_w = act == TP_ACT_SWIGLU ? 2 * f : f;
    TP_TRY(check_elems(fn, N, h));
    TP_TRY(check_elems(fn, h, n_w));
    TP_TRY(check_elems(fn, N, n_w));
    // dZ = dY W_out^T (NT) with the activation backward in the epilogue -> dH
    a = make_args(dY, W_out, dH, (int)N, (int)f, (int)h, (int)h, (int)h, (int)n_w);
    a.aux = static_cast<const uint16_t*>(H_save);
    a.ldc2 = (int)n_w;
    a.f = (int)f;
    // dX_part = dH W_in^T (NT)
    b = make_args(dH, W_in, dX_part, (int)N, (int)h, (int)n_w, (int)n_w, (int)n_w, (int)h);
    b.accumulate = accumulate ? 1 : 0;
    // dW_in = X^T dH (TN): A = X stored [K=N][M=h], B = dH stored [K=N][n_w]
    c = make_args(X, dH, dW_in, (int)h, (int)n_w, (int)N, (int)h, (int)n_w, (int)n_w);
    // dW_out = Z^T dY (TN): A = Z stored [N][f], B = dY stored [N][h]
    d = make_args(Z, dY, dW_out, (int)f, (int)h, (int)N, (int)f, (int)h, (int)h);
    need = need_of({(query || dX_part) ? plan_of<false, false, EPI_F32>(b) : SplitPlan{},
                    (query || dW_in) ? plan_of<true, true, EPI_F32>(c) : SplitPlan{},
                    (query || dW_out) ? plan_of<true, true, EPI_F32>(d) : SplitPlan{}});
    return TP_OK;
}

static tp_status col_bwd_plan(const char* fn, const void* X, const void* W, const void* dY, float* dX_part,
                              float* dW, int64_t N, int64_t k, int64_t n, int accumulate, bool query, GemmArgs& a,
                              GemmArgs& b, size_t& need) {
    TP_TRY(check_tokens(fn, N));
    TP_TRY(check_width(fn, "k", k));
    TP_TRY(check_width(fn, "n", n));
    TP_TRY(check_elems(fn, N, k));
    TP_TRY(check_elems(fn, k, n));
    TP_TRY(check_elems(fn, N, n));
    a = make_args(dY, W, dX_part, (int)N, (int)k, (int)n, (int)n, (int)n, (int)k);
    a.accumulate = accumulate ? 1 : 0;
    b = make_args(X, dY, dW, (int)k, (int)n, (int)N, (int)k, (int)n, (int)n);
    need = need_of({(query || dX_part) ? plan_of<false, false, EPI_F32>(a) : SplitPlan{},
                    (query || dW) ? plan_of<true, true, EPI_F32>(b) : SplitPlan{}});
    return TP_OK;
}

// Chunk c of the chunked column-parallel backward: dY's token rows [r0, r1)
// times W^T into the same rows of dX_part.
static GemmArgs col_dx_chunk(const void* dY, const void* W, float* dX_part, int64_t N, int64_t k, int64_t n,
                             int accumulate, int nchunks, int c) {
    int64_t r0, r1;
    chunk_rows(N, nchunks, c, r0, r1);
    GemmArgs a = make_args(dY ? static_cast<const uint16_t*>(dY) + r0 * n : nullptr, W,
                           dX_part ? dX_part + r0 * k : nullptr, (int)(r1 - r0), (int)k, (int)n, (int)n, (int)n,
                           (int)k);
    a.accumulate = accumulate ? 1 : 0;
    return a;
}

// dW (b, over all N tokens) and the validation of the chunked call; the
// chunks and dW run one after another and reuse one workspace.
static tp_status col_bwd_chunked_plan(const char* fn, const void* X, const void* dY, float* dW, int64_t N, int64_t k,
                                      int64_t n, int32_t nchunks, bool query, GemmArgs& b, size_t& need) {
    GemmArgs a;
    TP_TRY(col_bwd_plan(fn, X, nullptr, dY, nullptr, dW, N, k, n, 0, query, a, b, need));
    TP_TRY(check_nchunks(fn, nchunks));
    need = (query || dW) ? plan_of<true, true, EPI_F32>(b).bytes : 0;
    for (int c = 0; c < nchunks; ++c)
        need = std::max(need, plan_of<false, false, EPI_F32>(col_dx_chunk(nullptr, nullptr, nullptr, N, k, n, 0,
                                                                          nchunks, c)).bytes);
    return TP_OK;
}

static tp_status row_bwd_plan(const char* fn, const void* Z, const void* W, const void* dY, void* dZ, float* dW,
                              int64_t N, int64_t k_loc, int64_t n, bool query, GemmArgs& a, GemmArgs& b,
                              size_t& need) {
    TP_TRY(check_tokens(fn, N));
    TP_TRY(check_width(fn, "k_loc", k_loc));
    TP_TRY(check_width(fn, "n", n));
    TP_TRY(check_elems(fn, N, k_loc));
    TP_TRY(check_elems(fn, k_loc, n));
    TP_TRY(check_elems(fn, N, n));
    a = make_args(dY, W, dZ, (int)N, (int)k_loc, (int)n, (int)n, (int)n, (int)k_loc);
    b = make_args(Z, dY, dW, (int)k_loc, (int)n, (int)N, (int)k_loc, (int)n, (int)n);
    need = need_of({(query || dZ) ? plan_of<false, false, EPI_BF16>(a) : SplitPlan{},
                    (query || dW) ? plan_of<true, true, EPI_F32>(b) : SplitPlan{}});
    return TP_OK;
}

// Common checks of the vocab-parallel cross-entropy calls.
static tp_status check_ce(const char* fn, int64_t N, int64_t h, int64_t v_loc, int64_t vocab_start) {
    TP_TRY(check_tokens(fn, N));
    TP_TRY(check_width(fn, "h", h));
    TP_TRY(check_width(fn, "v_loc", v_loc));
    if (vocab_start < 0 || vocab_start + v_loc > 0x7fffffffLL)
        return fail(TP_ERR_INVALID_ARG, "%s: vocab range [%lld, %lld) outside int32", fn, (long long)vocab_start,
                    (long long)(vocab_start + v_loc));
    TP_TRY(check_elems(fn, N, h));
    TP_TRY(check_elems(fn, h, v_loc));
    TP_TRY(check_elems(fn, N, v_loc));
    return TP_OK;
}

static tp_status check_targets(const char* fn, int64_t N, const int32_t* targets) {
    if (N > 0 && (targets == nullptr || (reinterpret_cast<uintptr_t>(targets) & 3u)))
        return fail(TP_ERR_INVALID_ARG, "%s: targets is NULL or not 4-byte aligned", fn);
    return TP_OK;
}

// records: one per row and wave column block of the statistics GEMM's tiles
// (ce_parts), 3 floats each
static size_t ce_fwd_need(int64_t N, int64_t h, int64_t v_loc) {
    return (size_t)N * ce_parts(h, v_loc) * 3 * sizeof(float);
}

static void ce_bwd_args(const void* X, const void* W_i, void* dZ, float* dX_part, float* dW_i, int64_t N, int64_t h,
                        int64_t v_loc, int accumulate, GemmArgs& b, GemmArgs& c) {
    // dX_part = dZ W_i^T (NT, {U}); dW_i = X^T dZ (TN)
    b = make_args(dZ, W_i, dX_part, (int)N, (int)h, (int)v_loc, (int)v_loc, (int)v_loc, (int)h);
    b.accumulate = accumulate ? 1 : 0;
    c = make_args(X, dZ, dW_i, (int)h, (int)v_loc, (int)N, (int)h, (int)v_loc, (int)v_loc);
}

static size_t ce_bwd_need(const GemmArgs& b, const GemmArgs& c) {
    return need_of({plan_of<false, false, EPI_F32>(b), plan_of<true, true, EPI_F32>(c)});
}

static tp_status check_embed(const char* fn, int64_t N, int64_t v_loc, int64_t h, int64_t vocab_start) {
    TP_TRY(check_tokens(fn, N));
    TP_TRY(check_width(fn, "h", h));
    if (v_loc <= 0 || v_loc > 0x7fffffffLL) return fail(TP_ERR_INVALID_ARG, "%s: v_loc = %lld", fn, (long long)v_loc);
    if (vocab_start < 0) return fail(TP_ERR_INVALID_ARG, "%s: vocab_start < 0", fn);
    TP_TRY(check_elems(fn, v_loc, h));
    TP_TRY(check_elems(fn, N, h));
    return TP_OK;
}

static tp_status check_ids(const char* fn, int64_t N, const int32_t* ids) {
    if (N > 0 && (ids == nullptr || (reinterpret_cast<uintptr_t>(ids) & 3u)))
        return fail(TP_ERR_INVALID_ARG, "%s: ids is NULL or not 4-byte aligned", fn);
    return TP_OK;
}

static tp_status embed_bwd_plan(const char* fn, int64_t N, int64_t v_loc, int64_t h, int64_t vocab_start,
                                size_t& need) {
    TP_TRY(check_embed(fn, N, v_loc, h, vocab_start));
    if (h > kEmbedMaxH) return fail(TP_ERR_UNSUPPORTED, "%s: h = %lld above %d", fn, (long long)h, kEmbedMaxH);
    if (N > 0x7fffffffLL) return fail(TP_ERR_UNSUPPORTED, "%s: too many tokens", fn);
    // a row count, a flag per table row, a list of at most min(N, v_loc) rows
    need = ((size_t)(1 + v_loc + std::min(N, v_loc)) * sizeof(uint32_t) + 15) / 16 * 16;
    return TP_OK;
}

}  // namespace tps

using namespace tps;

#define TP_QUERY_OUT(p)                                                                 \
    do {                                                                                \
        if ((p) == nullptr) return fail(TP_ERR_INVALID_ARG, "%s: bytes is NULL", fn);   \
    } while (0)

extern "C" {

int tp_version(void) { return (0 << 16) | 2; }

const char* tp_last_error(void) { return g_last_error.c_str(); }

tp_status tp_col_linear_workspace_size(int64_t N, int64_t k, int64_t n_out, int act, size_t* bytes) {
    const char* fn = "tp_col_linear_workspace_size";
    TP_QUERY_OUT(bytes);
    GemmArgs a;
    size_t need = 0;
    TP_TRY(col_linear_plan(fn, nullptr, nullptr, nullptr, N, k, n_out, act, nullptr, a, need));
    *bytes = need;
    return ok();
}

tp_status tp_col_linear(const void* X, const void* W, void* Y, int64_t N, int64_t k, int64_t n_out, int act,
                        void* H_save, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "tp_col_linear";
    GemmArgs a;
    size_t need = 0;
    TP_TRY(col_linear_plan(fn, X, W, Y, N, k, n_out, act, H_save, a, need));
    TP_CHECK_TOK_PTR(X, "X");
    TP_CHECK_PTR(W, "W");
    TP_CHECK_TOK_PTR(Y, "Y");
    TP_CHECK_OPT_PTR(H_save, "H_save");
    TP_TRY(check_workspace(fn, {workspace, workspace_bytes}, need));
    TP_TRY(col_linear_run(fn, a, act, workspace, static_cast<hipStream_t>(stream)));
    return ok();
}

tp_status tp_col_linear_noalloc(const void* X, const void* W, void* Y, int64_t N, int64_t k, int64_t n_out,
                                int act, void* H_save, void* stream) {
    const char* fn = "tp_col_linear_noalloc";
    GemmArgs a;
    size_t need = 0;
    TP_TRY(col_linear_plan(fn, X, W, Y, N, k, n_out, act, H_save, a, need));
    TP_CHECK_TOK_PTR(X, "X");
    TP_CHECK_PTR(W, "W");
    TP_CHECK_TOK_PTR(Y, "Y");
    TP_CHECK_OPT_PTR(H_save, "H_save");
    if (need > kScratchBytes)
        return fail(TP_ERR_UNSUPPORTED, "%s: the product needs %zu bytes of scratch, above the library's %zu",
                    fn, need, kScratchBytes);
    void* ws = nullptr;
    if (need > 0) TP_TRY(scratch_address(fn, &ws));
    TP_TRY(col_linear_run(fn, a, act, ws, static_cast<hipStream_t>(stream)));
    return ok();
}

tp_status tp_row_linear_partial_workspace_size(int64_t N, int64_t k_loc, int64_t n, size_t* bytes) {
    const char* fn = "tp_row_linear_partial_workspace_size";
    TP_QUERY_OUT(bytes);
    GemmArgs a;
    size_t need = 0;
    TP_TRY(row_partial_plan(fn, nullptr, nullptr, nullptr, N, k_loc, n, 0, a, need));
    *bytes = need;
    return ok();
}

tp_status tp_row_linear_partial(const void* Z, const void* W, float* P, int64_t N, int64_t k_loc, int64_t n,
                                int accumulate, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "tp_row_linear_partial";
    GemmArgs a;
    size_t need = 0;
    TP_TRY(row_partial_plan(fn, Z, W, P, N, k_loc, n, accumulate, a, need));
    TP_CHECK_TOK_PTR(Z, "Z");
    TP_CHECK_PTR(W, "W");
    TP_CHECK_TOK_PTR(P, "P");
    TP_TRY(check_workspace(fn, {workspace, workspace_bytes}, need));
    TP_TRY((run_gemm<false, true, EPI_F32>(fn, a, workspace, static_cast<hipStream_t>(stream))));
    return ok();
}

tp_status tp_row_linear_partial_chunked_workspace_size(int64_t N, int64_t k_loc, int64_t n, int32_t nchunks,
                                                       size_t* bytes) {
    const char* fn = "tp_row_linear_partial_chunked_workspace_size";
    TP_QUERY_OUT(bytes);
    size_t need = 0;
    TP_TRY(row_chunked_plan(fn, N, k_loc, n, nchunks, need));
    *bytes = need;
    return ok();
}

tp_status tp_row_linear_partial_chunked(const void* Z, const void* W, float* P, int64_t N, int64_t k_loc,
                                        int64_t n, int accumulate, int32_t nchunks, void* const* events,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "tp_row_linear_partial_chunked";
    size_t need = 0;
    TP_TRY(row_chunked_plan(fn, N, k_loc, n, nchunks, need));
    TP_CHECK_TOK_PTR(Z, "Z");
    TP_CHECK_PTR(W, "W");
    TP_CHECK_TOK_PTR(P, "P");
    if (events)
        for (int c = 0; c < nchunks; ++c)
            if (!events[c]) return fail(TP_ERR_INVALID_ARG, "%s: events[%d] is NULL", fn, c);
    TP_TRY(check_workspace(fn, {workspace, workspace_bytes}, need));
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int c = 0; c < nchunks; ++c) {
        TP_TRY((run_gemm<false, true, EPI_F32>(fn, row_chunk(Z, W, P, N, k_loc, n, accumulate, nchunks, c),
                                               workspace, s)));
        if (events) {
            hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[c]), s);
            if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: event %d: %s", fn, c, hipGetErrorString(e));
        }
    }
    return ok();
}

tp_status tp_mlp_shard_fwd_workspace_size(int64_t N, int64_t h, int64_t f, int act, size_t* bytes) {
    const char* fn = "tp_mlp_shard_fwd_workspace_size";
    TP_QUERY_OUT(bytes);
    GemmArgs a, b;
    size_t need = 0;
    TP_TRY(mlp_fwd_plan(fn, nullptr, nullptr, nullptr, N, h, f, act, nullptr, nullptr, nullptr, 0, a, b, need));
    *bytes = need;
    return ok();
}

tp_status tp_mlp_shard_fwd(const void* X, const void* W_in, const void* W_out, int64_t N, int64_t h, int64_t f,
                           int act, void* Z, void* H_save, float* P, int accumulate, void* workspace,
                           size_t workspace_bytes, void* stream) {
    const char* fn = "tp_mlp_shard_fwd";
    GemmArgs a, b;
    size_t need = 0;
    TP_TRY(mlp_fwd_plan(fn, X, W_in, W_out, N, h, f, act, Z, H_save, P, accumulate, a, b, need));
    TP_CHECK_TOK_PTR(X, "X");
    TP_CHECK_PTR(W_in, "W_in");
    TP_CHECK_PTR(W_out, "W_out");
    TP_CHECK_TOK_PTR(Z, "Z");
    TP_CHECK_TOK_PTR(P, "P");
    TP_CHECK_OPT_PTR(H_save, "H_save");
    TP_TRY(check_workspace(fn, {workspace, workspace_bytes}, need));
    hipStream_t s = static_cast<hipStream_t>(stream);
    TP_TRY((act == TP_ACT_GELU ? run_gemm<false, true, EPI_GELU>(fn, a, workspace, s)
                               : run_gemm<false, true, EPI_SWIGLU>(fn, a, workspace, s)));
    TP_TRY((run_gemm<false, true, EPI_F32>(fn, b, workspace, s)));
    return ok();
}

tp_status tp_mlp_shard_bwd_workspace_size(int64_t N, int64_t h, int64_t f, int act, size_t* bytes) {
    const char* fn = "tp_mlp_shard_bwd_workspace_size";
    TP_QUERY_OUT(bytes);
    GemmArgs a, b, c, d;
    size_t need = 0;
    TP_TRY(mlp_bwd_plan(fn, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, N, h, f, act, nullptr, nullptr,
                        nullptr, nullptr, 0, true, a, b, c, d, need));
    *bytes = need;
    return ok();
}

tp_status tp_mlp_shard_bwd(const void* X, const void* W_in, const void* W_out, const void* H_save, const void* Z,
                           const void* dY, int64_t N, int64_t h, int64_t f, int act, void* dH, float* dX_part,
                           float* dW_in, float* dW_out, int accumulate, void* workspace, size_t workspace_bytes,
                           void* stream) {
    const char* fn = "tp_mlp_shard_bwd";
    GemmArgs a, b, c, d;
    size_t need = 0;
    TP_TRY(mlp_bwd_plan(fn, X, W_in, W_out, H_save, Z, dY, N, h, f, act, dH, dX_part, dW_in, dW_out, accumulate,
                        false, a, b, c, d, need));
    TP_CHECK_PTR(W_out, "W_out");
    TP_CHECK_TOK_PTR(H_save, "H_save");
    TP_CHECK_TOK_PTR(dY, "dY");
    TP_CHECK_TOK_PTR(dH, "dH");
    TP_CHECK_OPT_PTR(dX_part, "dX_part");
    TP_CHECK_OPT_PTR(dW_in, "dW_in");
    TP_CHECK_OPT_PTR(dW_out, "dW_out");
    if (dX_part) TP_CHECK_PTR(W_in, "W_in");
    if (dW_in) TP_CHECK_TOK_PTR(X, "X");
    if (dW_out) TP_CHECK_TOK_PTR(Z, "Z");
    TP_TRY(check_workspace(fn, {workspace, workspace_bytes}, need));
    hipStream_t s = static_cast<hipStream_t>(stream);
    TP_TRY((act == TP_ACT_GELU ? launch_gemm<false, false, EPI_GELU_BWD>(fn, a, s)
                               : launch_gemm<false, false, EPI_SWIGLU_BWD>(fn, a, s)));
    if (dX_part) TP_TRY((run_gemm<false, false, EPI_F32>(fn, b, workspace, s)));
    if (dW_in) TP_TRY((run_gemm<true, true, EPI_F32>(fn, c, workspace, s)));
    if (dW_out) TP_TRY((run_gemm<true, true, EPI_F32>(fn, d, workspace, s)));
    return ok();
}

tp_status tp_col_linear_bwd_workspace_size(int64_t N, int64_t k, int64_t n, size_t* bytes) {
    const char* fn = "tp_col_linear_bwd_workspace_size";
    TP_QUERY_OUT(bytes);
    GemmArgs a, b;
    size_t need = 0;
    TP_TRY(col_bwd_plan(fn, nullptr, nullptr, nullptr, nullptr, nullptr, N, k, n, 0, true, a, b, need));
    *bytes = need;
    return ok();
}

tp_status tp_col_linear_bwd(const void* X, const void* W, const void* dY, float* dX_part, float* dW, int64_t N,
                            int64_t k, int64_t n, int accumulate, void* workspace, size_t workspace_bytes,
                            void* stream) {
    const char* fn = "tp_col_linear_bwd";
    GemmArgs a, b;
    size_t need = 0;
    TP_TRY(col_bwd_plan(fn, X, W, dY, dX_part, dW, N, k, n, accumulate, false, a, b, need));
    TP_CHECK_TOK_PTR(dY, "dY");
    TP_CHECK_OPT_PTR(dX_part, "dX_part");
    TP_CHECK_OPT_PTR(dW, "dW");
    if (dX_part) TP_CHECK_PTR(W, "W");
    if (dW) TP_CHECK_TOK_PTR(X, "X");
    TP_TRY(check_workspace(fn, {workspace, workspace_bytes}, need));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dX_part) TP_TRY((run_gemm<false, false, EPI_F32>(fn, a, workspace, s)));
    if (dW) TP_TRY((run_gemm<true, true, EPI_F32>(fn, b, workspace, s)));
    return ok();
}

tp_status tp_col_linear_bwd_chunked_workspace_size(int64_t N, int64_t k, int64_t n, int32_t nchunks,
                                                   size_t* bytes) {
    const char* fn = "tp_col_linear_bwd_chunked_workspace_size";
    TP_QUERY_OUT(bytes);
    GemmArgs b;
    size_t need = 0;
    TP_TRY(col_bwd_chunked_plan(fn, nullptr, nullptr, nullptr, N, k, n, nchunks, true, b, need));
    *bytes = need;
    return ok();
}

tp_status tp_col_linear_bwd_chunked(const void* X, const void* W, const void* dY, float* dX_part, float* dW,
                                    int64_t N, int64_t k, int64_t n, int accumulate, int32_t nchunks,
                                    void* const* events, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "tp_col_linear_bwd_chunked";
    GemmArgs b;
    size_t need = 0;
    TP_TRY(col_bwd_chunked_plan(fn, X, dY, dW, N, k, n, nchunks, false, b, need));
    TP_CHECK_TOK_PTR(dY, "dY");
    TP_CHECK_TOK_PTR(dX_part, "dX_part");
    TP_CHECK_PTR(W, "W");
    TP_CHECK_OPT_PTR(dW, "dW");
    if (dW) TP_CHECK_TOK_PTR(X, "X");
    if (events)
        for (int c = 0; c < nchunks; ++c)
            if (!events[c]) return fail(TP_ERR_INVALID_ARG, "%s: events[%d] is NULL", fn, c);
    TP_TRY(check_workspace(fn, {workspace, workspace_bytes}, need));
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int c = 0; c < nchunks; ++c) {
        TP_TRY((run_gemm<false, false, EPI_F32>(fn, col_dx_chunk(dY, W, dX_part, N, k, n, accumulate, nchunks, c),
                                                workspace, s)));
        if (events) {
            hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[c]), s);
            if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: event %d: %s", fn, c, hipGetErrorString(e));
        }
    }
    if (dW) TP_TRY((run_gemm<true, true, EPI_F32>(fn, b, workspace, s)));
    return ok();
}

tp_status tp_row_linear_bwd_workspace_size(int64_t N, int64_t k_loc, int64_t n, size_t* bytes) {
    const char* fn = "tp_row_linear_bwd_workspace_size";
    TP_QUERY_OUT(bytes);
    GemmArgs a, b;
    size_t need = 0;
    TP_TRY(row_bwd_plan(fn, nullptr, nullptr, nullptr, nullptr, nullptr, N, k_loc, n, true, a, b, need));
    *bytes = need;
    return ok();
}

tp_status tp_row_linear_bwd(const void* Z, const void* W, const void* dY, void* dZ, float* dW, int64_t N,
                            int64_t k_loc, int64_t n, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "tp_row_linear_bwd";
    GemmArgs a, b;
    size_t need = 0;
    TP_TRY(row_bwd_plan(fn, Z, W, dY, dZ, dW, N, k_loc, n, false, a, b, need));
    TP_CHECK_TOK_PTR(dY, "dY");
    TP_CHECK_OPT_PTR(dZ, "dZ");
    TP_CHECK_OPT_PTR(dW, "dW");
    if (dZ) TP_CHECK_PTR(W, "W");
    if (dW) TP_CHECK_TOK_PTR(Z, "Z");
    TP_TRY(check_workspace(fn, {workspace, workspace_bytes}, need));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dZ) TP_TRY((run_gemm<false, false, EPI_BF16>(fn, a, workspace, s)));
    if (dW) TP_TRY((run_gemm<true, true, EPI_F32>(fn, b, workspace, s)));
    return ok();
}

tp_status tp_qkv_regroup(const void* W_qkv, void* W_r, int64_t h, int32_t n_h, int32_t n_kv, int32_t d_h,
                         int32_t t, int32_t rank, void* stream) {
    const char* fn = "tp_qkv_regroup";
    if (t <= 0) return fail(TP_ERR_INVALID_ARG, "%s: TP degree t = %d must be positive", fn, t);
    if (n_h <= 0 || n_kv <= 0 || d_h <= 0)
        return fail(TP_ERR_INVALID_ARG, "%s: head counts and head width must be positive", fn);
    if (n_h % t != 0)
        return fail(TP_ERR_NOT_DIVISIBLE,
                    "%s: num_attention_heads (%d) must be a multiple of tensor_model_parallel_size (%d).",
                    fn, n_h, t);
    TP_TRY(check_kv_heads(fn, n_kv, t));
    if (rank < 0 || rank >= t) return fail(TP_ERR_INVALID_ARG, "%s: rank %d outside [0, %d)", fn, rank, t);
    if (d_h % 8 != 0) return fail(TP_ERR_INVALID_ARG, "%s: d_h = %d must be a multiple of 8", fn, d_h);
    if (h < 0) return fail(TP_ERR_INVALID_ARG, "%s: h = %lld < 0", fn, (long long)h);
    const int64_t src_w64 = (int64_t)(n_h + 2 * n_kv) * d_h;
    if (src_w64 > 0x7fffffff) return fail(TP_ERR_UNSUPPORTED, "%s: fused width too large", fn);
    if (h == 0) return ok();
    TP_CHECK_PTR(W_qkv, "W_qkv");
    TP_CHECK_PTR(W_r, "W_r");
    // t <= n_kv: KV heads [r n_kv/t, (r+1) n_kv/t); n_kv < t: the one head
    // r / (t / n_kv), replicated on t / n_kv ranks
    const int q_w = n_h / t * d_h;
    const int kv_heads = t <= n_kv ? n_kv / t : 1;
    const int kv_first = t <= n_kv ? rank * (n_kv / t) : rank / (t / n_kv);
    const int kv_w = kv_heads * d_h;
    const int src_w = (int)src_w64;
    const int q_src0 = rank * q_w;
    const int k_src0 = n_h * d_h + kv_first * d_h;
    const int v_src0 = (n_h + n_kv) * d_h + kv_first * d_h;
    const int64_t blocks = (h + kRegroupRows - 1) / kRegroupRows;
    if (blocks > 0x7fffffffLL || (int64_t)kRegroupRows * src_w > 0x7fffffffLL)
        return fail(TP_ERR_UNSUPPORTED, "%s: h or the fused width is too large", fn);
    hipLaunchKernelGGL(qkv_regroup_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(W_qkv),
                       static_cast<uint16_t*>(W_r), h, src_w, q_w, kv_w, q_src0, k_src0, v_src0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

tp_status tp_kv_grad_accumulate(float* dW_dst, const float* dW_src, int64_t h, int32_t n_h, int32_t n_kv,
                                int32_t d_h, int32_t t, void* stream) {
    const char* fn = "tp_kv_grad_accumulate";
    if (t <= 0) return fail(TP_ERR_INVALID_ARG, "%s: TP degree t = %d must be positive", fn, t);
    if (n_h <= 0 || n_kv <= 0 || d_h <= 0)
        return fail(TP_ERR_INVALID_ARG, "%s: head counts and head width must be positive", fn);
    if (n_h % t != 0)
        return fail(TP_ERR_NOT_DIVISIBLE,
                    "%s: num_attention_heads (%d) must be a multiple of tensor_model_parallel_size (%d).",
                    fn, n_h, t);
    TP_TRY(check_kv_heads(fn, n_kv, t));
    if (t <= n_kv)
        return fail(TP_ERR_INVALID_ARG, "%s: KV heads are replicated only when n_kv (%d) < t (%d)", fn, n_kv,
                    t);
    if (d_h % 4 != 0) return fail(TP_ERR_INVALID_ARG, "%s: d_h = %d must be a multiple of 4", fn, d_h);
    if (h < 0) return fail(TP_ERR_INVALID_ARG, "%s: h = %lld < 0", fn, (long long)h);
    const int64_t ld = (int64_t)(n_h / t + 2) * d_h;
    if (ld > 0x7fffffff) return fail(TP_ERR_UNSUPPORTED, "%s: shard width too large", fn);
    TP_TRY(check_elems(fn, h, ld));
    if (h == 0) return ok();
    TP_CHECK_PTR(dW_dst, "dW_dst");
    TP_CHECK_PTR(dW_src, "dW_src");
    const int c0 = n_h / t * d_h, w = 2 * d_h;
    const int64_t work = h * (w / 4);
    const unsigned blocks = (unsigned)std::min<int64_t>((work + 255) / 256, 8192);
    hipLaunchKernelGGL(kv_grad_accumulate_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       dW_dst, dW_src, h, (int)ld, c0, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

tp_status tp_vocab_ce_fwd_workspace_size(int64_t N, int64_t h, int64_t v_loc, size_t* bytes) {
    const char* fn = "tp_vocab_ce_fwd_workspace_size";
    TP_QUERY_OUT(bytes);
    TP_TRY(check_ce(fn, N, h, v_loc, 0));
    *bytes = ce_fwd_need(N, h, v_loc);
    return ok();
}

tp_status tp_vocab_ce_fwd(const void* X, const void* W_i, const int32_t* targets, int64_t vocab_start, int64_t N,
                          int64_t h, int64_t v_loc, float* m_i, float* s_i, float* zy_i, void* workspace,
                          size_t workspace_bytes, void* stream) {
    const char* fn = "tp_vocab_ce_fwd";
    TP_TRY(check_ce(fn, N, h, v_loc, vocab_start));
    TP_TRY(check_targets(fn, N, targets));
    TP_CHECK_TOK_PTR(X, "X");
    TP_CHECK_PTR(W_i, "W_i");
    TP_CHECK_TOK_PTR(m_i, "m_i");
    TP_CHECK_TOK_PTR(s_i, "s_i");
    TP_CHECK_TOK_PTR(zy_i, "zy_i");
    TP_TRY(check_workspace(fn, {workspace, workspace_bytes}, ce_fwd_need(N, h, v_loc)));
    if (N == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int nparts = ce_parts(h, v_loc);
    float* rec = static_cast<float*>(workspace);
    GemmArgs a = make_args(X, W_i, rec, (int)N, (int)v_loc, (int)h, (int)h, (int)v_loc, nparts);
    a.tgt = targets;
    a.col0 = (int)vocab_start;
    TP_TRY((launch_gemm<false, true, EPI_CE_STATS>(fn, a, s)));
    hipLaunchKernelGGL(ce_stats_merge_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, rec, nparts, (int)N,
                       m_i, s_i, zy_i);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

tp_status tp_vocab_ce_combine(const float* m_parts, const float* s_parts, const float* zy_parts, int32_t t,
                              int64_t N, float* loss, float* m, float* S, void* stream) {
    const char* fn = "tp_vocab_ce_combine";
    if (t <= 0) return fail(TP_ERR_INVALID_ARG, "%s: t = %d must be positive", fn, t);
    TP_TRY(check_tokens(fn, N));
    if (N == 0) return ok();
    if (!m_parts || !s_parts || !zy_parts || !loss)
        return fail(TP_ERR_INVALID_ARG, "%s: m_parts, s_parts, zy_parts and loss must not be NULL", fn);
    TP_TRY(check_elems(fn, t, N));
    const unsigned blocks = (unsigned)std::min<int64_t>((N + 255) / 256, 8192);
    hipLaunchKernelGGL(ce_combine_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), m_parts,
                       s_parts, zy_parts, (int)t, N, loss, m, S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

tp_status tp_vocab_ce_bwd_workspace_size(int64_t N, int64_t h, int64_t v_loc, size_t* bytes) {
    const char* fn = "tp_vocab_ce_bwd_workspace_size";
    TP_QUERY_OUT(bytes);
    TP_TRY(check_ce(fn, N, h, v_loc, 0));
    GemmArgs b, c;
    ce_bwd_args(nullptr, nullptr, nullptr, nullptr, nullptr, N, h, v_loc, 0, b, c);
    *bytes = ce_bwd_need(b, c);
    return ok();
}

tp_status tp_vocab_ce_bwd(const void* X, const void* W_i, const int32_t* targets, int64_t vocab_start,
                          const float* m, const float* S, const float* dloss, int64_t N, int64_t h, int64_t v_loc,
                          void* dZ, float* dX_part, float* dW_i, int accumulate, void* workspace,
                          size_t workspace_bytes, void* stream) {
    const char* fn = "tp_vocab_ce_bwd";
    TP_TRY(check_ce(fn, N, h, v_loc, vocab_start));
    TP_TRY(check_targets(fn, N, targets));
    TP_CHECK_TOK_PTR(X, "X");
    TP_CHECK_PTR(W_i, "W_i");
    TP_CHECK_TOK_PTR(dZ, "dZ");
    TP_CHECK_TOK_PTR(dX_part, "dX_part");
    TP_CHECK_PTR(dW_i, "dW_i");
    if (N > 0 && (!m || !S || !dloss))
        return fail(TP_ERR_INVALID_ARG, "%s: m, S and dloss must not be NULL", fn);
    // dZ = (softmax(X W_i) - one-hot) * dloss, the logits recomputed
    GemmArgs a = make_args(X, W_i, dZ, (int)N, (int)v_loc, (int)h, (int)h, (int)v_loc, (int)v_loc);
    a.tgt = targets;
    a.col0 = (int)vocab_start;
    a.rm = m;
    a.rs = S;
    a.rd = dloss;
    GemmArgs b, c;
    ce_bwd_args(X, W_i, dZ, dX_part, dW_i, N, h, v_loc, accumulate, b, c);
    TP_TRY(check_workspace(fn, {workspace, workspace_bytes}, ce_bwd_need(b, c)));
    hipStream_t s = static_cast<hipStream_t>(stream);
    TP_TRY((launch_gemm<false, true, EPI_CE_GRAD>(fn, a, s)));
    TP_TRY((run_gemm<false, false, EPI_F32>(fn, b, workspace, s)));
    TP_TRY((run_gemm<true, true, EPI_F32>(fn, c, workspace, s)));
    return ok();
}

tp_status tp_vocab_embed_fwd(const int32_t* ids, const void* E_i, int64_t vocab_start, int64_t N, int64_t v_loc,
                             int64_t h, void* out, int accumulate, void* stream) {
    const char* fn = "tp_vocab_embed_fwd";
    TP_TRY(check_embed(fn, N, v_loc, h, vocab_start));
    TP_TRY(check_ids(fn, N, ids));
    TP_CHECK_PTR(E_i, "E_i");
    TP_CHECK_TOK_PTR(out, "out");
    if (N == 0) return ok();
    if (N > 0x7fffffffLL) return fail(TP_ERR_UNSUPPORTED, "%s: too many tokens", fn);
    hipLaunchKernelGGL(embed_fwd_kernel, dim3((unsigned)N), dim3(256), 0, static_cast<hipStream_t>(stream), ids,
                       static_cast<const uint16_t*>(E_i), vocab_start, (int)v_loc, (int)h,
                       static_cast<uint16_t*>(out), accumulate ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

tp_status tp_vocab_embed_bwd_workspace_size(int64_t N, int64_t v_loc, int64_t h, size_t* bytes) {
    const char* fn = "tp_vocab_embed_bwd_workspace_size";
    TP_QUERY_OUT(bytes);
    size_t need = 0;
    TP_TRY(embed_bwd_plan(fn, N, v_loc, h, 0, need));
    *bytes = need;
    return ok();
}

tp_status tp_vocab_embed_bwd(const int32_t* ids, const float* dY, int64_t vocab_start, int64_t N, int64_t v_loc,
                             int64_t h, float* dE_i, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "tp_vocab_embed_bwd";
    size_t need = 0;
    TP_TRY(embed_bwd_plan(fn, N, v_loc, h, vocab_start, need));
    TP_TRY(check_ids(fn, N, ids));
    TP_CHECK_TOK_PTR(dY, "dY");
    TP_CHECK_PTR(dE_i, "dE_i");
    TP_TRY(check_workspace(fn, {workspace, workspace_bytes}, need));
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t* count = static_cast<uint32_t*>(workspace);
    uint32_t* used = count + 1;
    uint32_t* list = used + v_loc;
    const int64_t words = 1 + v_loc;  // the list needs no clearing: only its first *count entries are read
    hipLaunchKernelGGL(embed_clear_kernel, dim3((unsigned)std::min<int64_t>((words + 255) / 256, 1024)), dim3(256),
                       0, s, count, words);
    const int64_t units = v_loc * h / 4;  // 16-byte units of the table (h is a multiple of 64)
    hipLaunchKernelGGL(embed_fill_mark_kernel, dim3((unsigned)((std::max(units, N) + 255) / 256)), dim3(256), 0, s,
                       dE_i, units, ids, vocab_start, N, (int)v_loc, count, used, list);
    if (N > 0)
        hipLaunchKernelGGL(embed_rows_kernel, dim3((unsigned)std::min<int64_t>(std::min(N, v_loc), 1024)),
                           dim3(256), 0, s, ids, dY, vocab_start, (int)N, (int)h, dE_i, count, list);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

tp_status tp_shard_shape(int32_t ndim, const int64_t* shape, int32_t elem_bytes, int32_t n_axes,
                         const int64_t* axis_sizes, const uint32_t* dim_axis_mask, int64_t* local_shape_out,
                         int64_t* local_bytes_out, int64_t* total_bytes_out) {
    const char* fn = "tp_shard_shape";
    if (ndim < 0 || ndim > 64) return fail(TP_ERR_INVALID_ARG, "%s: ndim = %d", fn, ndim);
    if (n_axes < 0 || n_axes > 32) return fail(TP_ERR_INVALID_ARG, "%s: n_axes = %d", fn, n_axes);
    if (elem_bytes <= 0) return fail(TP_ERR_INVALID_ARG, "%s: elem_bytes = %d", fn, elem_bytes);
    if ((ndim > 0 && (!shape || !dim_axis_mask || !local_shape_out)) || (n_axes > 0 && !axis_sizes) ||
        !local_bytes_out || !total_bytes_out)
        return fail(TP_ERR_INVALID_ARG, "%s: NULL argument", fn);
    int64_t devices = 1;
    for (int a = 0; a < n_axes; ++a) {
        if (axis_sizes[a] <= 0) return fail(TP_ERR_INVALID_ARG, "%s: mesh axis %d has size %lld", fn, a,
                                            (long long)axis_sizes[a]);
        devices *= axis_sizes[a];
    }
    uint32_t used = 0;
    int64_t elems = 1;
    for (int d = 0; d < ndim; ++d) {
        const uint32_t m = dim_axis_mask[d];
        if (n_axes < 32 && (m >> n_axes) != 0)
            return fail(TP_ERR_INVALID_ARG, "%s: dim %d names a mesh axis >= %d", fn, d, n_axes);
        if (m & used)
            return fail(TP_ERR_INVALID_ARG, "%s: a mesh axis shards two dims (dim %d)", fn, d);
        used |= m;
        if (shape[d] < 0) return fail(TP_ERR_INVALID_ARG, "%s: dim %d is negative", fn, d);
        int64_t div = 1;
        for (int a = 0; a < n_axes; ++a)
            if (m & (1u << a)) div *= axis_sizes[a];
        if (shape[d] % div != 0)
            return fail(TP_ERR_NOT_DIVISIBLE, "%s: dim %d (%lld) is not divisible by %lld", fn, d,
                        (long long)shape[d], (long long)div);
        local_shape_out[d] = shape[d] / div;
        elems *= local_shape_out[d];
    }
    *local_bytes_out = elems * elem_bytes;
    *total_bytes_out = elems * elem_bytes * devices;
    return ok();
}

}  // extern "C"

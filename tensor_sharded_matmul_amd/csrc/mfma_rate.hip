// mfma_rate.hip — the sustained rate of v_mfma_f32_16x16x32_bf16 on this GPU
// with no memory traffic: the ceiling the GEMM kernels are measured against
// besides the nominal peak. Each lane holds 8 A and 8 B operand fragments
// drawn once from a buffer (seeded random bf16 values, or all zeros); every
// wave then runs 16 independent accumulators through `iters` rounds of 32
// MFMAs whose operands rotate over the fragments, so that the matrix core
// sees changing data as in a GEMM's k-loop. One workgroup of 4 waves per
// CU-slot, 1024 workgroups. Prints the device's CU count and peak clock,
// then one JSON line per timed launch.
//
// Usage: mfma_rate [iters] [reps]
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                       \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "mfma_rate: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                   \
        }                                                                              \
    } while (0)

constexpr int kThreads = 256;
constexpr int kBlocks = 1024;
constexpr int kMfmaPerRound = 32;

__global__ void __launch_bounds__(kThreads) mfma_loop(const bf16x8_t* __restrict__ src, float* __restrict__ out,
                                                     int iters) {
    const int gid = blockIdx.x * kThreads + threadIdx.x;
    bf16x8_t a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = src[gid * 16 + i];
        b[i] = src[gid * 16 + 8 + i];
    }
    f32x4_t acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i * 4 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(i + 4 * r) & 7], b[(j + 4 * r + 1) & 7],
                                                                              acc[i * 4 + j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    out[gid] = s;  // keeps the loop live
}

int main(int argc, char** argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 20000;
    const int reps = argc > 2 ? atoi(argv[2]) : 3;
    if (iters < 4 || reps < 1) {
        fprintf(stderr, "usage: mfma_rate [iters >= 4] [reps >= 1]\n");
        return 2;
    }
    // the device's compute units and peak engine clock, as the runtime reports them
    int dev = 0, cus = 0, clk_khz = 0;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    CHECK(hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeClockRate, dev));
    printf("{\"cus\": %d, \"max_sclk_mhz\": %d, \"bf16_dense_peak_tflops\": %.1f}\n", cus, clk_khz / 1000,
           (double)cus * clk_khz * 1e3 * 4096 / 1e12);
    fflush(stdout);
    const size_t frags = (size_t)kBlocks * kThreads * 16;  // 16 fragments of 16 bytes per lane
    std::vector<uint16_t> host(frags * 8);
    bf16x8_t* src = nullptr;
    float* out = nullptr;
    CHECK(hipMalloc(&src, frags * 16));
    CHECK(hipMalloc(&out, (size_t)kBlocks * kThreads * sizeof(float)));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const double flop = (double)kBlocks * (kThreads / 64) * iters * kMfmaPerRound * (2.0 * 16 * 16 * 32);
    for (int zeros = 0; zeros < 2; ++zeros) {
        // random: bf16 with exponent 127 and random sign and mantissa bits
        // (magnitudes in [1, 2)); zeros: +0
        uint32_t x = 12345u;
        for (auto& v : host) {
            x = x * 1664525u + 1013904223u;
            v = zeros ? (uint16_t)0 : (uint16_t)(0x3f80u | ((x >> 9) & 0x807fu));
        }
        CHECK(hipMemcpy(src, host.data(), frags * 16, hipMemcpyHostToDevice));
        hipLaunchKernelGGL(mfma_loop, dim3(kBlocks), dim3(kThreads), 0, 0, src, out, iters / 4);  // warm-up
        CHECK(hipGetLastError());
        for (int r = 0; r < reps; ++r) {
            CHECK(hipEventRecord(e0, 0));
            hipLaunchKernelGGL(mfma_loop, dim3(kBlocks), dim3(kThreads), 0, 0, src, out, iters);
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(e1, 0));
            CHECK(hipEventSynchronize(e1));
            float ms = 0.f;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            printf("{\"data\": \"%s\", \"rep\": %d, \"ms\": %.4f, \"tflops\": %.1f}\n", zeros ? "zeros" : "random", r, ms,
                   flop / (ms * 1e-3) / 1e12);
            fflush(stdout);
        }
    }
    CHECK(hipFree(src));
    CHECK(hipFree(out));
    return 0;
}

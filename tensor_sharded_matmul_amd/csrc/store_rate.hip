// store_rate.hip — how fast one compute unit writes to memory: the cost a
// GEMM pays after its k-loop to store its output tile. Each workgroup writes
// 8 tiles of 256 x 256 elements (fp32: 256 KB each; tile w * 8 + i mod 512 of
// a [4096][8192] matrix, every address in bounds) with W waves, in 16 x 16
// blocks as a GEMM epilogue holds them: with the MFMA operands swapped (a
// lane holds 4 consecutive values of one row, so one store instruction
// covers 16 rows, 64 bytes of each in fp32 or 32 in bf16), or in the MFMA's
// own layout (a lane holds one column of 4 rows: 4 stores of 4 bytes, each
// covering 4 rows with 16 lanes along each), or row-contiguously (1 KB per
// fp32 instruction).
// 32 or 256 workgroups (one per CU). The time of each workgroup comes from
// the constant 100 MHz clock (s_memrealtime), from the first store to the
// last one's completion; the launch is timed with events as well. Prints the
// device's CU count, then one JSON line per case.
//
// Usage: store_rate
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define CHECK(x)                                                                         \
    do {                                                                                 \
        hipError_t e_ = (x);                                                             \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "store_rate: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                     \
        }                                                                                \
    } while (0)

constexpr int kRows = 4096, kCols = 8192, kTiles = 8;

enum Pattern { EPI_F32 = 0, EPI_BF16 = 1, ROWS_F32 = 2, COLS_F32 = 3 };

template <int W, int PAT>
__global__ void __launch_bounds__(64 * W) store_tiles(void* out, unsigned long long* ticks) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < kTiles; ++i) {
        const int tile = (int)((blockIdx.x * kTiles + i) % 512);
        const int r0 = (tile / 32) * 256, c0 = (tile % 32) * 256;
        if constexpr (PAT == COLS_F32) {
            // the MFMA's own layout: column l % 16 of rows 4 (l / 16) + v
            const int c = lane & 15, q = lane >> 4;
            for (int b = wave; b < 256; b += W) {
                const int row = r0 + (b / 16) * 16 + 4 * q, col = c0 + (b % 16) * 16 + c;
                float* p = static_cast<float*>(out) + (size_t)row * kCols + col;
                for (int v = 0; v < 4; ++v) p[(size_t)v * kCols] = (float)v;
            }
        } else if constexpr (PAT == ROWS_F32) {
            // row-contiguous: one instruction writes 256 consecutive floats
            for (int b = wave; b < 256; b += W) {
                float* p = static_cast<float*>(out) + (size_t)(r0 + b) * kCols + c0 + 4 * lane;
                *reinterpret_cast<f32x4_t*>(p) = f32x4_t{1.f, 2.f, 3.f, (float)lane};
            }
        } else {
            const int r = lane & 15, q = lane >> 4;
            for (int b = wave; b < 256; b += W) {
                const int row = r0 + (b / 16) * 16 + r, col = c0 + (b % 16) * 16 + 4 * q;
                if constexpr (PAT == EPI_F32) {
                    float* p = static_cast<float*>(out) + (size_t)row * kCols + col;
                    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{1.f, 2.f, 3.f, (float)lane};
                } else {
                    uint16_t* p = static_cast<uint16_t*>(out) + (size_t)row * kCols + col;
                    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{0x3f803f80u, (uint32_t)lane};
                }
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) ticks[blockIdx.x] = t1 - t0;
}

template <int W, int PAT>
static void run(void* out, unsigned long long* d_ticks, int wgs, hipEvent_t e0, hipEvent_t e1) {
    hipLaunchKernelGGL((store_tiles<W, PAT>), dim3(wgs), dim3(64 * W), 0, 0, out, d_ticks);  // warm-up
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL((store_tiles<W, PAT>), dim3(wgs), dim3(64 * W), 0, 0, out, d_ticks);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    std::vector<unsigned long long> h(wgs);
    CHECK(hipMemcpy(h.data(), d_ticks, sizeof(unsigned long long) * wgs, hipMemcpyDeviceToHost));
    double mean = 0.0;
    for (unsigned long long v : h) mean += (double)v;
    const double wg_us = mean / wgs / 100.0;  // 100 MHz ticks
    const double bytes = (double)kTiles * 256 * 256 * (PAT == EPI_BF16 ? 2 : 4);
    const char* name = PAT == EPI_F32    ? "epilogue_fp32"
                       : PAT == EPI_BF16 ? "epilogue_bf16"
                       : PAT == COLS_F32 ? "mfma_layout_fp32"
                                         : "rows_fp32";
    printf("{\"pattern\": \"%s\", \"waves\": %d, \"workgroups\": %d, \"bytes_per_workgroup\": %.0f, "
           "\"workgroup_us\": %.2f, \"gbs_per_workgroup\": %.1f, \"launch_us\": %.2f, \"total_tbs\": %.2f}\n",
           name, W, wgs, bytes, wg_us, bytes / (wg_us * 1e3), ms * 1e3, bytes * wgs / (ms * 1e-3) / 1e12);
    fflush(stdout);
}

int main() {
    int dev = 0, cus = 0;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    printf("{\"cus\": %d}\n", cus);
    fflush(stdout);
    void* out = nullptr;
    unsigned long long* d_ticks = nullptr;
    CHECK(hipMalloc(&out, (size_t)kRows * kCols * sizeof(float)));
    CHECK(hipMalloc(&d_ticks, 256 * sizeof(unsigned long long)));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int wgs : {32, 256}) {
        run<4, EPI_F32>(out, d_ticks, wgs, e0, e1);
        run<8, EPI_F32>(out, d_ticks, wgs, e0, e1);
        run<16, EPI_F32>(out, d_ticks, wgs, e0, e1);
        run<8, COLS_F32>(out, d_ticks, wgs, e0, e1);
        run<8, ROWS_F32>(out, d_ticks, wgs, e0, e1);
        run<8, EPI_BF16>(out, d_ticks, wgs, e0, e1);
    }
    CHECK(hipFree(out));
    CHECK(hipFree(d_ticks));
    return 0;
}

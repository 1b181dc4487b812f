// hbm_ceiling.hip -- attainable HBM bandwidth of plain streaming kernels on this GPU:
// read-only, write-only, copy and in-place read-modify-write over one large buffer.
// These are the ceilings the perturb pass (an in-place read-modify-write of every
// parameter) is compared with, besides the datasheet peak.
//
//   hbm_ceiling [GB]      (default 59.92 GB, the OPT-30B-shaped bf16 parameter set)
//
// Each kernel is a grid-stride loop over 16 KiB chunks per wave (16 dwordx4 per lane, one
// contiguous KiB per instruction), launched with a few workgroups per CU; loads and stores
// carry the non-temporal hint (the fastest setting measured for streaming here).  Every
// figure is bytes moved / kernel time (HIP events), best over the launch shapes tried.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                       \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                   \
        }                                                                              \
    } while (0)

constexpr int kLoads = 16;                      // dwordx4 per lane per chunk
constexpr uint64_t kChunk16 = kLoads * 64;      // 16-byte units per wave chunk (16 KiB)

__global__ __launch_bounds__(256) void k_read(const u32x4_t *__restrict__ p, uint64_t nchunks,
                                              uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (uint64_t ch = (uint64_t)blockIdx.x * 4 + wv; ch < nchunks; ch += (uint64_t)gridDim.x * 4) {
        const u32x4_t *b = p + ch * kChunk16 + lane;
#pragma unroll
        for (int k = 0; k < kLoads; ++k) acc ^= __builtin_nontemporal_load(b + k * 64);
    }
    sink[blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ __launch_bounds__(256) void k_write(u32x4_t *__restrict__ p, uint64_t nchunks)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const u32x4_t v = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
    for (uint64_t ch = (uint64_t)blockIdx.x * 4 + wv; ch < nchunks; ch += (uint64_t)gridDim.x * 4) {
        u32x4_t *b = p + ch * kChunk16 + lane;
#pragma unroll
        for (int k = 0; k < kLoads; ++k) b[k * 64] = v;
    }
}

__global__ __launch_bounds__(256) void k_copy(const u32x4_t *__restrict__ src,
                                              u32x4_t *__restrict__ dst, uint64_t nchunks)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (uint64_t ch = (uint64_t)blockIdx.x * 4 + wv; ch < nchunks; ch += (uint64_t)gridDim.x * 4) {
        const u32x4_t *s = src + ch * kChunk16 + lane;
        u32x4_t *d = dst + ch * kChunk16 + lane;
        u32x4_t v[kLoads];
#pragma unroll
        for (int k = 0; k < kLoads; ++k) v[k] = __builtin_nontemporal_load(s + k * 64);
#pragma unroll
        for (int k = 0; k < kLoads; ++k) __builtin_nontemporal_store(v[k], d + k * 64);
    }
}

__global__ __launch_bounds__(256) void k_rmw(u32x4_t *__restrict__ p, uint64_t nchunks)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (uint64_t ch = (uint64_t)blockIdx.x * 4 + wv; ch < nchunks; ch += (uint64_t)gridDim.x * 4) {
        u32x4_t *b = p + ch * kChunk16 + lane;
        u32x4_t v[kLoads];
#pragma unroll
        for (int k = 0; k < kLoads; ++k) v[k] = __builtin_nontemporal_load(b + k * 64);
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            v[k] += 0x00010001u;
            __builtin_nontemporal_store(v[k], b + k * 64);
        }
    }
}

template <typename F>
static float time_ms(F launch, int iters)
{
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    launch();
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(a));
    for (int i = 0; i < iters; ++i) launch();
    CHECK(hipEventRecord(b));
    CHECK(hipEventSynchronize(b));
    CHECK(hipGetLastError());
    float ms;
    CHECK(hipEventElapsedTime(&ms, a, b));
    CHECK(hipEventDestroy(a));
    CHECK(hipEventDestroy(b));
    return ms / iters;
}

int main(int argc, char **argv)
{
    const double gb = argc > 1 ? atof(argv[1]) : 59.919663104;
    int cus = 0;
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    const uint64_t chunk_bytes = kChunk16 * 16;
    const uint64_t nchunks = (uint64_t)(gb * 1e9) / chunk_bytes / 2 * 2;  // even
    const uint64_t bytes = nchunks * chunk_bytes;
    char *buf;
    CHECK(hipMalloc(&buf, bytes));
    CHECK(hipMemset(buf, 0x3C, bytes));
    const int max_grid = cus * 32;
    uint32_t *sink;
    CHECK(hipMalloc(&sink, (size_t)max_grid * 256 * sizeof(uint32_t)));
    CHECK(hipDeviceSynchronize());
    printf("device CUs %d, buffer %.3f GB (%llu chunks of %llu bytes)\n", cus, bytes / 1e9,
           (unsigned long long)nchunks, (unsigned long long)chunk_bytes);
    const int shapes[] = {2, 4, 8, 16, 32};
    double best[4] = {0, 0, 0, 0};
    const char *names[4] = {"read-only", "write-only", "copy (half -> half)", "in-place RMW"};
    for (int wpc : shapes) {
        const int grid = cus * wpc;
        u32x4_t *p = reinterpret_cast<u32x4_t *>(buf);
        double gbs[4];
        gbs[0] = bytes / (time_ms([&] { hipLaunchKernelGGL(k_read, dim3(grid), dim3(256), 0, 0, p, nchunks, sink); }, 5) * 1e6);
        gbs[1] = bytes / (time_ms([&] { hipLaunchKernelGGL(k_write, dim3(grid), dim3(256), 0, 0, p, nchunks); }, 5) * 1e6);
        const uint64_t half = nchunks / 2;
        gbs[2] = 2.0 * half * chunk_bytes /
                 (time_ms([&] { hipLaunchKernelGGL(k_copy, dim3(grid), dim3(256), 0, 0, p, p + half * kChunk16, half); }, 5) * 1e6);
        gbs[3] = 2.0 * bytes / (time_ms([&] { hipLaunchKernelGGL(k_rmw, dim3(grid), dim3(256), 0, 0, p, nchunks); }, 5) * 1e6);
        printf("workgroups/CU %2d: read %.1f  write %.1f  copy %.1f  rmw %.1f GB/s\n", wpc, gbs[0],
               gbs[1], gbs[2], gbs[3]);
        fflush(stdout);
        for (int i = 0; i < 4; ++i)
            if (gbs[i] > best[i]) best[i] = gbs[i];
    }
    for (int i = 0; i < 4; ++i)
        printf("best %-20s %8.1f GB/s  (%.1f%% of 8000 GB/s)\n", names[i], best[i], best[i] / 80.0);
    CHECK(hipFree(sink));
    CHECK(hipFree(buf));
    return 0;
}

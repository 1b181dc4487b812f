// philox_ceiling.hip -- attainable Philox4x32-10 rate of this GPU with the library's own
// generator (zo_device.hpp), and nothing else in the loop: the compute ceiling that the
// kernels regenerating probe bits (perturb, update) are compared with.
//
//   philox_ceiling
//
// Every lane evaluates `iters` blocks with distinct counters (block index varying, probe and
// step fixed, key uniform across the grid as in the library's kernels) and folds the 128
// output bits into one word, which it stores once so that no call is dead code.  Reported:
// calls per second = lanes x iters / kernel time (HIP events), best over the launch shapes
// tried; each call yields the sign bits of 128 parameters of one probe.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../csrc/zo_device.hpp"

#define CHECK(x)                                                                       \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                   \
        }                                                                              \
    } while (0)

__global__ __launch_bounds__(256) void k_philox(uint32_t iters, uint32_t probe, uint32_t step,
                                                uint32_t k0, uint32_t k1,
                                                uint32_t *__restrict__ sink)
{
    const uint64_t lane = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t lanes = (uint64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    for (uint32_t i = 0; i < iters; ++i) {
        const zo::U32x4 r = zo::probe_block_bits(lane + (uint64_t)i * lanes, probe, step, k0, k1);
        acc ^= ZO_BITOP3(r.x, r.y, r.z, zo::kXor3) ^ r.w;
    }
    sink[lane] = acc;
}

int main()
{
    int cus = 0;
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    const int shapes[] = {4, 8, 16, 32};
    const uint32_t iters = 4096;
    uint32_t *sink;
    CHECK(hipMalloc(&sink, (size_t)cus * 32 * 256 * sizeof(uint32_t)));
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    double best = 0.0;
    printf("device CUs %d, %u Philox4x32-10 calls per lane\n", cus, iters);
    for (int wpc : shapes) {
        const int grid = cus * wpc;
        hipLaunchKernelGGL(k_philox, dim3(grid), dim3(256), 0, 0, iters, 7u, 3u, 0x12345678u,
                           0x9abcdef0u, sink);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
        const int reps = 5;
        CHECK(hipEventRecord(a));
        for (int r = 0; r < reps; ++r)
            hipLaunchKernelGGL(k_philox, dim3(grid), dim3(256), 0, 0, iters, 7u, 3u + r,
                               0x12345678u, 0x9abcdef0u, sink);
        CHECK(hipEventRecord(b));
        CHECK(hipEventSynchronize(b));
        CHECK(hipGetLastError());
        float ms;
        CHECK(hipEventElapsedTime(&ms, a, b));
        const double calls = (double)grid * 256 * iters;
        const double rate = calls / (ms / reps * 1e-3);
        printf("workgroups/CU %2d: %.3f ms per launch, %.4e calls/s\n", wpc, ms / reps, rate);
        fflush(stdout);
        if (rate > best) best = rate;
    }
    printf("best %.4e Philox4x32-10 calls/s (%.4e probe*params/s of sign bits)\n", best,
           best * 128.0);
    CHECK(hipFree(sink));
    return 0;
}

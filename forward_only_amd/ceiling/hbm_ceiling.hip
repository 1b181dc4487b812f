// hbm_ceiling.hip -- attainable HBM bandwidth of plain streaming kernels on this GPU:
// read-only, write-only, copy and in-place read-modify-write over one large buffer.
// These are the ceilings the perturb pass (an in-place read-modify-write of every
// parameter) is compared with, besides the datasheet peak.
//
//   hbm_ceiling [GB] [rounds]   (default 59.92 GB, the OPT-30B-shaped bf16 parameter set;
//                                3 rounds)
//   hbm_ceiling --allocations [GB] [count]   in-place RMW speed of successive allocations:
//                                count rounds of allocate / measure / free, then up to count
//                                allocations held at once (default 59.92 GB, 6)
//
// The buffer is split into eight contiguous ranges, one per XCD (workgroup b runs on XCD
// b % 8), every load and store instruction moving one contiguous KiB per wave.  Two forms:
// persistent (16 KiB chunks, each XCD's range walked grid-stride by a few resident
// four-wave workgroups per CU, launch shapes 2-16 workgroups per CU) and non-persistent
// (single-wave workgroups, one chunk each, each XCD's chunks taken in dispatch order -- the
// form of the library's passes: 8 KiB chunks, and 4 KiB for the write-only kernel as in the
// plane generator).  Loads and stores carry the non-temporal hint (the fastest
// setting measured for streaming here).  Every figure is bytes moved / kernel time (HIP
// events), best over the launch shapes tried.  A large buffer's bandwidth depends on the
// physical memory the allocation lands on (the same physical memory mapped at other
// virtual addresses runs at the same speed), so each round allocates the buffer afresh
// and the rounds are reported separately.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

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

// Chunk range of this workgroup's XCD and its first chunk / stride (gridDim.x % 8 == 0).
struct XcdWalk {
    uint64_t first, end, stride;
};
__device__ __forceinline__ XcdWalk xcd_walk(uint64_t nchunks)
{
    const uint32_t x = blockIdx.x & 7u;
    const uint64_t lo = nchunks * x / 8;
    return {lo + (uint64_t)(blockIdx.x >> 3) * 4 + (threadIdx.x >> 6), nchunks * (x + 1) / 8,
            (uint64_t)(gridDim.x >> 3) * 4};
}

__global__ __launch_bounds__(256) void k_read(const u32x4_t *__restrict__ p, uint64_t nchunks,
                                              uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const XcdWalk w = xcd_walk(nchunks);
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (uint64_t ch = w.first; ch < w.end; ch += w.stride) {
        const u32x4_t *b = p + ch * kChunk16 + lane;
#pragma unroll
        for (int k = 0; k < kLoads; ++k) acc ^= __builtin_nontemporal_load(b + k * 64);
    }
    sink[blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ __launch_bounds__(256) void k_write(u32x4_t *__restrict__ p, uint64_t nchunks)
{
    const int lane = threadIdx.x & 63;
    const XcdWalk w = xcd_walk(nchunks);
    const u32x4_t v = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
    for (uint64_t ch = w.first; ch < w.end; ch += w.stride) {
        u32x4_t *b = p + ch * kChunk16 + lane;
#pragma unroll
        for (int k = 0; k < kLoads; ++k) b[k * 64] = v;
    }
}

__global__ __launch_bounds__(256) void k_copy(const u32x4_t *__restrict__ src,
                                              u32x4_t *__restrict__ dst, uint64_t nchunks)
{
    const int lane = threadIdx.x & 63;
    const XcdWalk w = xcd_walk(nchunks);
    for (uint64_t ch = w.first; ch < w.end; ch += w.stride) {
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
    const int lane = threadIdx.x & 63;
    const XcdWalk w = xcd_walk(nchunks);
    for (uint64_t ch = w.first; ch < w.end; ch += w.stride) {
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

// Non-persistent walk (the library's passes): single-wave workgroups, one chunk of kL KiB
// (kL dwordx4 per lane) each, XCD ranges in dispatch order.  Returns the chunk, or n.
__device__ __forceinline__ uint64_t np_chunk(uint64_t n)
{
    const uint64_t x = blockIdx.x & 7u;
    const uint64_t ch = n * x / 8 + (blockIdx.x >> 3);
    return ch < n * (x + 1) / 8 ? ch : n;
}
static uint32_t np_grid(uint64_t n) { return (uint32_t)(8 * ((n + 7) / 8)); }
constexpr int kNpLoads = 8;        // read, copy, in-place RMW: 8 KiB per wave (the passes)
constexpr int kNpWriteLoads = 4;   // write: 4 KiB per wave (the plane generator)

template <int kL>
__global__ __launch_bounds__(64) void k_read_np(const u32x4_t *__restrict__ p, uint64_t n,
                                                uint32_t *__restrict__ sink)
{
    const uint64_t ch = np_chunk(n);
    if (ch >= n) return;
    const u32x4_t *b = p + ch * (kL * 64) + threadIdx.x;
    u32x4_t acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < kL; ++k) acc ^= __builtin_nontemporal_load(b + k * 64);
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[0] = acc.x;   // keeps the loads
}

template <int kL>
__global__ __launch_bounds__(64) void k_write_np(u32x4_t *__restrict__ p, uint64_t n)
{
    const uint64_t ch = np_chunk(n);
    if (ch >= n) return;
    u32x4_t *b = p + ch * (kL * 64) + threadIdx.x;
    const u32x4_t v = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
#pragma unroll
    for (int k = 0; k < kL; ++k) __builtin_nontemporal_store(v, b + k * 64);
}

template <int kL>
__global__ __launch_bounds__(64) void k_copy_np(const u32x4_t *__restrict__ src,
                                                u32x4_t *__restrict__ dst, uint64_t n)
{
    const uint64_t ch = np_chunk(n);
    if (ch >= n) return;
    const u32x4_t *s = src + ch * (kL * 64) + threadIdx.x;
    u32x4_t *d = dst + ch * (kL * 64) + threadIdx.x;
    u32x4_t v[kL];
#pragma unroll
    for (int k = 0; k < kL; ++k) v[k] = __builtin_nontemporal_load(s + k * 64);
#pragma unroll
    for (int k = 0; k < kL; ++k) __builtin_nontemporal_store(v[k], d + k * 64);
}

template <int kL>
__global__ __launch_bounds__(64) void k_rmw_np(u32x4_t *__restrict__ p, uint64_t n)
{
    const uint64_t ch = np_chunk(n);
    if (ch >= n) return;
    u32x4_t *b = p + ch * (kL * 64) + threadIdx.x;
    u32x4_t v[kL];
#pragma unroll
    for (int k = 0; k < kL; ++k) v[k] = __builtin_nontemporal_load(b + k * 64);
#pragma unroll
    for (int k = 0; k < kL; ++k) {
        v[k] += 0x00010001u;
        __builtin_nontemporal_store(v[k], b + k * 64);
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

// In-place RMW bandwidth of one buffer: persistent (one launch of 8 workgroups per CU),
// non-persistent (8 KiB single-wave chunks) as one launch, and the same per 1 GiB slice.
struct RmwRates {
    double persistent, np, np_sliced;
};
static RmwRates rmw_gbps(char *buf, uint64_t nchunks, int cus)
{
    u32x4_t *p = reinterpret_cast<u32x4_t *>(buf);
    const int grid = cus * 8;
    const double bytes = 2.0 * nchunks * kChunk16 * 16;
    const uint64_t nnp = nchunks * kChunk16 / (kNpLoads * 64);   // 8 KiB chunks
    const uint64_t sl = (1ull << 30) / (kNpLoads * 1024);         // 8 KiB chunks per 1 GiB
    RmwRates r;
    r.persistent = bytes / (time_ms([&] { hipLaunchKernelGGL(k_rmw, dim3(grid), dim3(256), 0, 0, p, nchunks); }, 3) * 1e6);
    r.np = bytes / (time_ms([&] { hipLaunchKernelGGL(k_rmw_np<kNpLoads>, dim3(np_grid(nnp)), dim3(64), 0, 0, p, nnp); }, 3) * 1e6);
    r.np_sliced = bytes / (time_ms([&] {
        for (uint64_t s0 = 0; s0 < nnp; s0 += sl) {
            const uint64_t m = nnp - s0 < sl ? nnp - s0 : sl;
            hipLaunchKernelGGL(k_rmw_np<kNpLoads>, dim3(np_grid(m)), dim3(64), 0, 0, p + s0 * (kNpLoads * 64), m);
        } }, 3) * 1e6);
    return r;
}

// --allocations mode: the placement of successive allocations of one size.  First `count`
// rounds of allocate / measure / free, then up to `count` allocations held at once (while
// free memory stays above the size plus 4 GiB), each measured as it is made.
static int allocations(double gb, int count)
{
    int cus = 0;
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    const uint64_t chunk_bytes = kChunk16 * 16;
    const uint64_t nchunks = (uint64_t)(gb * 1e9) / chunk_bytes;
    const uint64_t bytes = nchunks * chunk_bytes;
    size_t fr, tot;
    CHECK(hipMemGetInfo(&fr, &tot));
    printf("allocations of %.3f GB; device memory free %.1f of %.1f GB; in-place RMW GB/s: "
           "persistent (8 workgroups per CU) / non-persistent / non-persistent per 1 GiB slice\n",
           bytes / 1e9, fr / 1e9, tot / 1e9);
    for (int r = 0; r < count; ++r) {
        char *buf;
        CHECK(hipMalloc(&buf, bytes));
        CHECK(hipMemset(buf, 0, bytes));
        const RmwRates g = rmw_gbps(buf, nchunks, cus);
        printf("allocate-measure-free %d: %.0f / %.0f / %.0f\n", r, g.persistent, g.np, g.np_sliced);
        fflush(stdout);
        CHECK(hipFree(buf));
    }
    char *held[16];
    int nh = 0;
    while (nh < count && nh < 16) {
        CHECK(hipMemGetInfo(&fr, &tot));
        if (fr < bytes + (4ull << 30)) break;
        CHECK(hipMalloc(&held[nh], bytes));
        CHECK(hipMemset(held[nh], 0, bytes));
        const RmwRates g = rmw_gbps(held[nh], nchunks, cus);
        printf("held %d: %.0f / %.0f / %.0f\n", nh, g.persistent, g.np, g.np_sliced);
        fflush(stdout);
        ++nh;
    }
    for (int i = 0; i < nh; ++i) CHECK(hipFree(held[i]));
    return 0;
}

int main(int argc, char **argv)
{
    if (argc > 1 && strcmp(argv[1], "--allocations") == 0)
        return allocations(argc > 2 ? atof(argv[2]) : 59.919663104, argc > 3 ? atoi(argv[3]) : 6);
    const double gb = argc > 1 ? atof(argv[1]) : 59.919663104;
    const int rounds = argc > 2 ? atoi(argv[2]) : 3;
    int cus = 0;
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    const uint64_t chunk_bytes = kChunk16 * 16;
    const uint64_t nchunks = (uint64_t)(gb * 1e9) / chunk_bytes / 2 * 2;  // even
    const uint64_t bytes = nchunks * chunk_bytes;
    const int shapes[] = {2, 4, 6, 8, 16};
    const int max_grid = cus * 16;
    uint32_t *sink;
    CHECK(hipMalloc(&sink, (size_t)max_grid * 256 * sizeof(uint32_t)));
    printf("device CUs %d, buffer %.3f GB (%llu chunks of %llu bytes), %d allocation rounds\n",
           cus, bytes / 1e9, (unsigned long long)nchunks, (unsigned long long)chunk_bytes, rounds);
    const char *names[4] = {"read-only", "write-only", "copy (half -> half)", "in-place RMW"};
    double overall[4] = {0, 0, 0, 0};
    for (int r = 0; r < rounds; ++r) {
        char *buf;
        CHECK(hipMalloc(&buf, bytes));
        CHECK(hipMemset(buf, 0x3C, bytes));
        CHECK(hipDeviceSynchronize());
        double best[4] = {0, 0, 0, 0};
        for (int wpc : shapes) {
            const int grid = cus * wpc / 8 * 8;
            u32x4_t *p = reinterpret_cast<u32x4_t *>(buf);
            double gbs[4];
            gbs[0] = bytes / (time_ms([&] { hipLaunchKernelGGL(k_read, dim3(grid), dim3(256), 0, 0, p, nchunks, sink); }, 5) * 1e6);
            gbs[1] = bytes / (time_ms([&] { hipLaunchKernelGGL(k_write, dim3(grid), dim3(256), 0, 0, p, nchunks); }, 5) * 1e6);
            const uint64_t half = nchunks / 2;
            gbs[2] = 2.0 * half * chunk_bytes /
                     (time_ms([&] { hipLaunchKernelGGL(k_copy, dim3(grid), dim3(256), 0, 0, p, p + half * kChunk16, half); }, 5) * 1e6);
            gbs[3] = 2.0 * bytes / (time_ms([&] { hipLaunchKernelGGL(k_rmw, dim3(grid), dim3(256), 0, 0, p, nchunks); }, 5) * 1e6);
            printf("round %d workgroups/CU %2d: read %.1f  write %.1f  copy %.1f  rmw %.1f GB/s\n", r,
                   wpc, gbs[0], gbs[1], gbs[2], gbs[3]);
            fflush(stdout);
            for (int i = 0; i < 4; ++i)
                if (gbs[i] > best[i]) best[i] = gbs[i];
        }
        {   // non-persistent form: single-wave workgroups, one chunk each
            u32x4_t *p = reinterpret_cast<u32x4_t *>(buf);
            const uint64_t n8 = bytes / (kNpLoads * 1024), n4 = bytes / (kNpWriteLoads * 1024);
            const uint64_t half = n8 / 2;
            double gbs[4];
            gbs[0] = 1024.0 * kNpLoads * n8 / (time_ms([&] { hipLaunchKernelGGL(k_read_np<kNpLoads>, dim3(np_grid(n8)), dim3(64), 0, 0, p, n8, sink); }, 5) * 1e6);
            gbs[1] = 1024.0 * kNpWriteLoads * n4 / (time_ms([&] { hipLaunchKernelGGL(k_write_np<kNpWriteLoads>, dim3(np_grid(n4)), dim3(64), 0, 0, p, n4); }, 5) * 1e6);
            gbs[2] = 2.0 * 1024.0 * kNpLoads * half /
                     (time_ms([&] { hipLaunchKernelGGL(k_copy_np<kNpLoads>, dim3(np_grid(half)), dim3(64), 0, 0, p, p + half * (kNpLoads * 64), half); }, 5) * 1e6);
            gbs[3] = 2.0 * 1024.0 * kNpLoads * n8 / (time_ms([&] { hipLaunchKernelGGL(k_rmw_np<kNpLoads>, dim3(np_grid(n8)), dim3(64), 0, 0, p, n8); }, 5) * 1e6);
            printf("round %d non-persistent  : read %.1f  write %.1f  copy %.1f  rmw %.1f GB/s\n", r,
                   gbs[0], gbs[1], gbs[2], gbs[3]);
            fflush(stdout);
            for (int i = 0; i < 4; ++i)
                if (gbs[i] > best[i]) best[i] = gbs[i];
        }
        for (int i = 0; i < 4; ++i) {
            printf("round %d best %-20s %8.1f GB/s  (%.1f%% of 8000 GB/s)\n", r, names[i], best[i],
                   best[i] / 80.0);
            if (best[i] > overall[i]) overall[i] = best[i];
        }
        fflush(stdout);
        CHECK(hipFree(buf));
    }
    for (int i = 0; i < 4; ++i)
        printf("best of all rounds %-20s %8.1f GB/s  (%.1f%% of 8000 GB/s)\n", names[i], overall[i],
               overall[i] / 80.0);
    CHECK(hipFree(sink));
    return 0;
}

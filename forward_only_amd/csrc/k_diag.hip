// k_diag.hip -- diagnostic streaming kernel: every 16-byte word of a buffer is read, xored
// with a mask and written back, in the perturb kernel's order and form (eight contiguous
// chunk ranges, one per XCD, one 8 KiB chunk per single-wave workgroup, non-persistent,
// non-temporal loads and stores).  With
// mask 0 the buffer is unchanged, and timing the call on a parameter buffer gives the
// in-place read-modify-write ceiling of the physical memory that buffer occupies.  The mask
// is a run-time argument on purpose: a store of the value just loaded from the same address
// is dead code to the compiler, which would otherwise delete the whole pass.
#include "zo_device.hpp"
#include "zo_launch.hpp"

namespace zo {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDiagLoads = 8;                          // dwordx4 per lane per chunk
constexpr uint64_t kDiagChunk16 = kDiagLoads * kWave;  // 16-byte words per chunk (8 KiB)

__global__ __launch_bounds__(kWave) void k_stream_rmw(u32x4_t *__restrict__ p, uint64_t nchunks,
                                                      uint32_t mask)
{
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t ch = xcd_range_chunk<1>(nchunks);
    if (ch < nchunks) {
        u32x4_t *b = p + ch * kDiagChunk16 + lane;
        u32x4_t v[kDiagLoads];
#pragma unroll
        for (int k = 0; k < kDiagLoads; ++k) v[k] = __builtin_nontemporal_load(b + k * kWave);
#pragma unroll
        for (int k = 0; k < kDiagLoads; ++k) __builtin_nontemporal_store(v[k] ^ mask, b + k * kWave);
    }
}

// Words past the last whole chunk: one thread per 16-byte word.
__global__ __launch_bounds__(256) void k_stream_rmw_tail(u32x4_t *__restrict__ p, uint64_t start,
                                                         uint64_t nwords, uint32_t mask)
{
    const uint64_t i = start + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nwords) p[i] = p[i] ^ mask;
}

static hipError_t stream_rmw_range(void *buf, uint64_t bytes, uint32_t mask, int num_cus,
                                   hipStream_t stream)
{
    const uint64_t nwords = bytes / 16;
    const uint64_t nchunks = nwords / kDiagChunk16;
    u32x4_t *p = static_cast<u32x4_t *>(buf);
    (void)num_cus;
    if (nchunks)
        hipLaunchKernelGGL(k_stream_rmw, dim3(xcd_range_grid(nchunks, 1)), dim3(kWave), 0,
                           stream, p, nchunks, mask);
    const uint64_t start = nchunks * kDiagChunk16;
    if (start < nwords) {
        const uint32_t grid = (uint32_t)((nwords - start + 255) / 256);
        hipLaunchKernelGGL(k_stream_rmw_tail, dim3(grid), dim3(256), 0, stream, p, start, nwords,
                           mask);
    }
    return hipGetLastError();
}

hipError_t launch_stream_rmw(void *buf, uint64_t bytes, uint32_t mask, int num_cus,
                             hipStream_t stream, uint64_t slice_bytes)
{
    constexpr uint64_t kMaxLaunchBytes = kMaxChunksPerLaunch * kDiagChunk16 * 16;
    if (slice_bytes == 0 || slice_bytes > kMaxLaunchBytes) slice_bytes = kMaxLaunchBytes;
    if (slice_bytes >= bytes)
        return stream_rmw_range(buf, bytes, mask, num_cus, stream);
    for (uint64_t b0 = 0; b0 < bytes; b0 += slice_bytes) {
        const uint64_t m = (bytes - b0) < slice_bytes ? (bytes - b0) : slice_bytes;
        const hipError_t e = stream_rmw_range(static_cast<char *>(buf) + b0, m, mask, num_cus,
                                              stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace zo

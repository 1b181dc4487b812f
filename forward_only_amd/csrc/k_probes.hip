// k_probes.hip -- packed probe generator: one Philox4x32-10 call per (probe, 128-param
// block) writes that block's 16 bytes of sign bits.
//
// A single-wave workgroup writes one chunk of kGenPerLane * 64 consecutive blocks (4 KiB)
// of one probe row and exits: kGenPerLane store instructions per lane, each covering 64
// consecutive blocks, i.e. one contiguous KiB per instruction, with the non-temporal hint
// (the plane is streamed out, not re-read here).  Each row's chunks are split into eight
// contiguous ranges, one per XCD (workgroup b runs on XCD b % 8, round-robin dispatch), and
// the grid is non-persistent: workgroups take the chunks of their XCD's range in dispatch
// order, so the waves in flight stay in one compact window per XCD.  On 3.7 GB planes:
// persistent grid-stride walk of the same ranges 5.4-5.6 TB/s; non-persistent 16 KiB per
// wave in four-wave workgroups 6.06-6.19; this form 6.30-6.45 (8, 16 and 32 KiB
// single-wave chunks 5.7-6.3).  The split is a plain partition of the chunks; the output
// does not depend on where workgroups run.
#include "zo_device.hpp"
#include "zo_launch.hpp"

namespace zo {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGenPerLane = 4;                                  // blocks per lane per chunk
constexpr uint64_t kGenChunk = (uint64_t)kWave * kGenPerLane;   // blocks per chunk
constexpr int kGenWavesPerWG = 1;

// Rows p = probe0 + blockIdx.y (+ gridDim.y ...) over blocks [0, nblk) of the launch;
// block b of row p is written at rows + p * row_stride + b (16-byte units).
__global__ __launch_bounds__(kWave * kGenWavesPerWG) void k_gen_probes(u32x4_t *__restrict__ rows,
                                                    uint64_t row_stride, uint64_t nblk,
                                                    uint64_t blk0, uint32_t step,
                                                    uint32_t probe0, uint32_t nprobes,
                                                    uint32_t k0, uint32_t k1)
{
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint64_t nch = (nblk + kGenChunk - 1) / kGenChunk;
    const uint64_t ch = xcd_range_chunk<kGenWavesPerWG>(nch);
    if (ch >= nch) return;
    for (uint32_t p = blockIdx.y; p < nprobes; p += gridDim.y) {
        u32x4_t *row = rows + (uint64_t)p * row_stride;
#pragma unroll
        for (int k = 0; k < kGenPerLane; ++k) {
            const uint64_t b = ch * kGenChunk + (uint64_t)k * kWave + lane;
            if (b < nblk) {
                const U32x4 w = probe_block_bits(blk0 + b, probe0 + p, step, k0, k1);
                __builtin_nontemporal_store(u32x4_t{w.x, w.y, w.z, w.w}, row + b);
            }
        }
    }
}

hipError_t launch_gen_probes(Key key, uint32_t step, uint32_t probe0, uint32_t nprobes,
                             uint64_t offset, uint64_t n, uint8_t *bits, int num_cus,
                             hipStream_t stream)
{
    (void)num_cus;
    const uint64_t nblk = (n + kBlockParams - 1) / kBlockParams;
    const uint32_t gy = nprobes < 65535u ? nprobes : 65535u;
    u32x4_t *rows = reinterpret_cast<u32x4_t *>(bits);
    // one launch per kMaxChunksPerLaunch chunks of the row (a single launch at any real size)
    const uint64_t span = kMaxChunksPerLaunch * kGenChunk;
    for (uint64_t b0 = 0; b0 < nblk; b0 += span) {
        const uint64_t m = (nblk - b0) < span ? (nblk - b0) : span;
        const uint64_t nch = (m + kGenChunk - 1) / kGenChunk;
        hipLaunchKernelGGL(k_gen_probes, dim3(xcd_range_grid(nch, kGenWavesPerWG), gy),
                           dim3(kWave * kGenWavesPerWG), 0, stream, rows + b0, nblk, m, offset / kBlockParams + b0,
                           step, probe0, nprobes, key.k0, key.k1);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace zo

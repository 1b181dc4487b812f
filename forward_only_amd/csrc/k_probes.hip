// k_probes.hip -- packed probe generator: one Philox4x32-10 call per (probe, 128-param
// block) writes that block's 16 bytes of sign bits.
//
// A wave writes chunks of 256 consecutive blocks of one probe row: four store
// instructions per lane, each covering 64 consecutive blocks, i.e. one contiguous KiB per
// instruction, with the non-temporal hint (the plane is streamed out, not re-read here).
// Each row's chunks are split into eight contiguous ranges, one per XCD: workgroup b runs
// on XCD b % 8 (round-robin dispatch) and walks range b % 8 grid-stride, so every XCD
// streams through its own eighth of the row.  The split is a plain partition of the
// chunks; the output does not depend on where workgroups run.
#include "zo_device.hpp"
#include "zo_launch.hpp"

namespace zo {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGenPerLane = 4;                          // blocks per lane per chunk
constexpr uint64_t kGenChunk = (uint64_t)kWave * kGenPerLane;   // blocks per chunk

__global__ __launch_bounds__(256) void k_gen_probes(u32x4_t *__restrict__ out, uint64_t nblk,
                                                    uint64_t blk0, uint32_t step,
                                                    uint32_t probe0, uint32_t nprobes,
                                                    uint32_t k0, uint32_t k1)
{
    const uint32_t lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const uint64_t nch = (nblk + kGenChunk - 1) / kGenChunk;
    const uint32_t xcd = blockIdx.x & 7u;
    const uint64_t stride = (uint64_t)(gridDim.x >> 3) * 4;      // waves per XCD range
    const uint64_t end = nch * (xcd + 1) / 8;
    for (uint32_t p = blockIdx.y; p < nprobes; p += gridDim.y) {
        u32x4_t *row = out + (uint64_t)p * nblk;
        for (uint64_t ch = nch * xcd / 8 + (uint64_t)(blockIdx.x >> 3) * 4 + wv; ch < end;
             ch += stride) {
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
}

hipError_t launch_gen_probes(Key key, uint32_t step, uint32_t probe0, uint32_t nprobes,
                             uint64_t offset, uint64_t n, uint8_t *bits, int num_cus,
                             hipStream_t stream)
{
    const uint64_t nblk = (n + kBlockParams - 1) / kBlockParams;
    const uint64_t nch = (nblk + kGenChunk - 1) / kGenChunk;
    // four waves per workgroup, a multiple of 8 workgroups (one share per XCD range)
    const uint64_t want_x = (nch + 3) / 4;
    const uint64_t cap_x = (uint64_t)num_cus * 8;
    const uint32_t gx = (uint32_t)(((want_x < cap_x ? want_x : cap_x) + 7) / 8 * 8);
    const uint32_t gy = nprobes < 65535u ? nprobes : 65535u;
    hipLaunchKernelGGL(k_gen_probes, dim3(gx, gy), dim3(256), 0, stream,
                       reinterpret_cast<u32x4_t *>(bits), nblk, offset / kBlockParams, step,
                       probe0, nprobes, key.k0, key.k1);
    return hipGetLastError();
}

}  // namespace zo

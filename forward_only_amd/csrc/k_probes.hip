// k_probes.hip -- packed probe generator: one Philox4x32-10 call per (probe, 128-param
// block) writes that block's 16 bytes of sign bits.  Consecutive lanes own consecutive
// blocks, so each wave stores one contiguous 1 KiB run per row (fully coalesced
// global_store_dwordx4).
#include "zo_device.hpp"
#include "zo_launch.hpp"

namespace zo {

__global__ __launch_bounds__(256) void k_gen_probes(uint4 *__restrict__ out, uint64_t nblk,
                                                    uint64_t blk0, uint32_t step,
                                                    uint32_t probe0, uint32_t nprobes,
                                                    uint32_t k0, uint32_t k1)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint32_t p = blockIdx.y; p < nprobes; p += gridDim.y) {
        uint4 *row = out + (uint64_t)p * nblk;
        for (uint64_t b = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
            const U32x4 w = probe_block_bits(blk0 + b, probe0 + p, step, k0, k1);
            row[b] = make_uint4(w.x, w.y, w.z, w.w);
        }
    }
}

hipError_t launch_gen_probes(Key key, uint32_t step, uint32_t probe0, uint32_t nprobes,
                             uint64_t offset, uint64_t n, uint8_t *bits, int num_cus,
                             hipStream_t stream)
{
    const uint64_t nblk = (n + kBlockParams - 1) / kBlockParams;
    const uint64_t want_x = (nblk + 255) / 256;
    const uint64_t cap_x = (uint64_t)num_cus * 16;
    const uint32_t gx = (uint32_t)(want_x < cap_x ? want_x : cap_x);
    const uint32_t gy = nprobes < 65535u ? nprobes : 65535u;
    hipLaunchKernelGGL(k_gen_probes, dim3(gx, gy), dim3(256), 0, stream,
                       reinterpret_cast<uint4 *>(bits), nblk, offset / kBlockParams, step,
                       probe0, nprobes, key.k0, key.k1);
    return hipGetLastError();
}

}  // namespace zo

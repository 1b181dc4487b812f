// zo_device.hpp -- device helpers of the gfx950 kernels: Philox4x32-10, bf16 packing,
// sign application, and wave-scope LDS ordering.  Device code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zo {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kBlockParams = 128;   // params covered by one Philox4x32-10 call

// Three-input bitwise function (gfx950 v_bitop3_b32); `tt` is the truth table over the
// canonical inputs a = 0xF0, b = 0xCC, c = 0xAA.
constexpr uint32_t kXor3 = 0x96;          // a ^ b ^ c
constexpr uint32_t kXorAnd = 0x28;        // (a ^ b) & c
#define ZO_BITOP3(a, b, c, tt) __builtin_amdgcn_bitop3_b32((a), (b), (c), (tt))

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2,
// 3", SC'11, section 4).  Per round two 32x32->64 products (one v_mad_u64_u32 each on
// gfx950) and two three-way xors (one v_bitop3_b32 each); the key schedule is uniform
// across the wave, so the compiler keeps it in scalar registers.
struct U32x4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ U32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        const uint32_t n0 = ZO_BITOP3((uint32_t)(p1 >> 32), c1, k0, kXor3);
        const uint32_t n2 = ZO_BITOP3((uint32_t)(p0 >> 32), c3, k1, kXor3);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return {c0, c1, c2, c3};
}

// The 128 sign bits of global block `blk` for (probe, step) under key (k0, k1).
__device__ __forceinline__ U32x4 probe_block_bits(uint64_t blk, uint32_t probe, uint32_t step,
                                                  uint32_t k0, uint32_t k1)
{
    return philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), probe, step, k0, k1);
}

// ---- bf16 <-> fp32 ------------------------------------------------------------------
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w)
{
    return __uint_as_float(w & 0xFFFF0000u);
}

// Two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2_t v = {lo, hi};
    bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

// +a if bit `b` of `m` is set, else -a: flip the sign bit of a when the bit is clear.
// nm = ~m, abits = bit pattern of a; b is a compile-time constant after unrolling.
__device__ __forceinline__ float signed_alpha(uint32_t nm, int b, uint32_t abits)
{
    const uint32_t s = (b <= 31 ? (nm << (31 - b)) : 0u) & 0x80000000u;
    return __uint_as_float(abits ^ s);
}

// Chunk of this wave in a non-persistent XCD-range launch over chunks [0, n): the chunks
// are split into eight contiguous ranges, one per XCD (workgroups are dispatched to the XCDs
// round-robin, so workgroup b runs on XCD b % 8), and workgroup b gives each of its
// kWavesPerWG waves the next chunk of range b % 8 in dispatch order.  Every wave handles one
// chunk and exits, so the waves in flight on an XCD always cover one compact window of its
// range: a persistent loop lets waves drift apart over a wide window, which some physical
// placements of a large buffer serve much more slowly.  Returns n for a wave past its range.
template <int kWavesPerWG>
__device__ __forceinline__ uint64_t xcd_range_chunk(uint64_t n)
{
    const uint64_t x = blockIdx.x & 7u;
    const uint64_t ch = n * x / 8 + (uint64_t)(blockIdx.x >> 3) * kWavesPerWG + threadIdx.x / kWave;
    return ch < n * (x + 1) / 8 ? ch : n;
}

// Order LDS traffic among the lanes of one wavefront: no compiler reordering across it,
// and the wave's LDS operations complete in issue order in hardware.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace zo

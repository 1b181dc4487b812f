// k_perturb.hip -- in-place perturbation theta <- round(theta + alpha * z) of one probe,
// the fused unpack/apply step of 1.5-SPSA (abstract of "Probe-Space Preconditioning for
// Fast and Stable Zero-Order Training"; the moves to theta +/- eps*z_i of "How 1.5-SPSA
// Works" on "Stanford's 1.5-SPSA Trains OPT-30B Without Backpropagation").
//
// Layout and mapping (gfx950, wave64):
//  * A workgroup is one wave; it owns one 8 KiB chunk (4096 bf16 or 2048 fp32 consecutive
//    params: 32 or 16 Philox blocks) and exits.  The chunks are split into eight contiguous
//    ranges, one per XCD: workgroups are dispatched to the XCDs round-robin, so workgroup b
//    (on XCD b % 8) takes the next chunk of range b % 8 in dispatch order.  Each XCD then
//    streams through its own eighth of the buffer (its L2 and address translation see one
//    compact window instead of every XCD touching every window), and since no wave loops,
//    the waves in flight never drift apart.  Measured on 60 GB buffers (in-place streaming
//    of the same shape): a persistent grid-stride walk of the same ranges ran at 6.16-6.24
//    TB/s on fast physical placements and 5.2 on slow ones; non-persistent 16 KiB chunks in
//    four-wave workgroups 6.34-6.39 and 5.86-5.92; 8 KiB single-wave workgroups, this form,
//    6.42-6.47 and 6.00-6.07.  The split is a plain partition of the chunks, so results do
//    not depend on where workgroups actually run.
//  * Each lane issues its 8 global_load_dwordx4 first; load k of lane L covers 16 bytes at
//    chunk + 1 KiB*k + 16*L, so every load instruction moves one contiguous KiB per wave.
//  * While those loads are in flight, lane L < 32 (bf16; < 16 for fp32) computes Philox for
//    block L of the chunk (or reads its 16 bytes of a stored plane) and writes the 16 bytes
//    to an LDS slice private to the wave.  The chunk's sign bits are then a linear array:
//    bf16 load k of lane L needs byte 64k + L, fp32 load k needs the nibble (L & 1) of byte
//    32k + L/2 -- one ds_read_u8 each, with the load index folded into the instruction's
//    offset.
//  * Apply: flip alpha's sign bit when the param's bit is clear, one fp32 add, and for
//    bf16 one v_cvt_pk_bf16_f32 (round to nearest even) per pair; store dwordx4.
//  * The ragged end (fewer than 8192 params) goes to a small per-element kernel.
//  * A pass may be issued as consecutive launches over slices of the buffer (the context's
//    slice setting, chosen per buffer by zo_tune_placement); the result is the same.
//  * Two-probe variant (zo_perturb2): the restore of probe a and the move of probe b in
//    one pass.  Each lane computes both Philox blocks, both land in LDS, and the step is
//    d = (+/-alpha_a) + (+/-alpha_b) in fp32 followed by the same add and narrow; this
//    halves the passes of a step (two per probe instead of four).
// Every element is read once and written once; no element is touched by two lanes.
#include "zo_device.hpp"
#include "zo_launch.hpp"

namespace zo {

// Params per chunk (one wave's 8 KiB): 4096 bf16 or 2048 fp32.
template <bool kBF16>
constexpr int chunk_params() { return kBF16 ? 4096 : 2048; }
constexpr int kWavesPerWG = 1;
static_assert(kPerturbChunkParams % chunk_params<true>() == 0 &&
                  kPerturbChunkParams % chunk_params<false>() == 0,
              "slices are whole chunks of either type");

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool kBF16, bool kBits, bool kTwo>
__global__ __launch_bounds__(kWave * kWavesPerWG) void k_perturb_chunks(u32x4_t *__restrict__ theta,
                                                        uint64_t nchunks, uint64_t blk0,
                                                        uint32_t step, uint32_t probe_a,
                                                        uint32_t probe_b, uint32_t k0,
                                                        uint32_t k1, uint32_t abits,
                                                        uint32_t bbits,
                                                        const u32x4_t *__restrict__ bits_a,
                                                        const u32x4_t *__restrict__ bits_b)
{
    constexpr int kChunkParams = chunk_params<kBF16>();
    constexpr int kPerLoad = kBF16 ? 8 : 4;                      // params per 16 bytes
    constexpr int kLoads = kChunkParams / (kPerLoad * kWave);   // 8
    constexpr int kBlocks = kChunkParams / kBlockParams;         // 32 or 16
    constexpr int kProbes = kTwo ? 2 : 1;
    __shared__ u32x4_t xch_all[kWavesPerWG][kProbes][kBlocks];

    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    u32x4_t *xa = xch_all[wv][0];
    u32x4_t *xb = xch_all[wv][kProbes - 1];
    const uint8_t *ba = reinterpret_cast<const uint8_t *>(xa);
    const uint8_t *bb = reinterpret_cast<const uint8_t *>(xb);
    const uint64_t ch = xcd_range_chunk<kWavesPerWG>(nchunks);   // wave-uniform
    if (ch < nchunks) {
        u32x4_t *base = theta + ch * (uint64_t)(kChunkParams / kPerLoad) + lane;
        u32x4_t v[kLoads];
#pragma unroll
        for (int k = 0; k < kLoads; ++k) v[k] = __builtin_nontemporal_load(base + k * kWave);

        if (lane < kBlocks) {
            const uint64_t lb = ch * kBlocks + lane;  // block index local to the buffer
            u32x4_t wa, wb;
            if constexpr (kBits) {
                wa = bits_a[lb];
                if constexpr (kTwo) wb = bits_b[lb];
            } else {
                const U32x4 r = probe_block_bits(blk0 + lb, probe_a, step, k0, k1);
                wa = u32x4_t{r.x, r.y, r.z, r.w};
                if constexpr (kTwo) {
                    const U32x4 q = probe_block_bits(blk0 + lb, probe_b, step, k0, k1);
                    wb = u32x4_t{q.x, q.y, q.z, q.w};
                }
            }
            xa[lane] = wa;
            if constexpr (kTwo) xb[lane] = wb;
        }
        wave_lds_sync();

#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            uint32_t ma, mb = 0;
            if constexpr (kBF16) {
                ma = ba[64 * k + lane];
                if constexpr (kTwo) mb = bb[64 * k + lane];
            } else {
                ma = (uint32_t)ba[32 * k + (lane >> 1)] >> (4 * (lane & 1));
                if constexpr (kTwo) mb = (uint32_t)bb[32 * k + (lane >> 1)] >> (4 * (lane & 1));
            }
            const uint32_t nma = ~ma, nmb = ~mb;
            u32x4_t q = v[k];
            if constexpr (kBF16) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float dlo = signed_alpha(nma, 2 * j, abits);
                    float dhi = signed_alpha(nma, 2 * j + 1, abits);
                    if constexpr (kTwo) {
                        dlo = dlo + signed_alpha(nmb, 2 * j, bbits);
                        dhi = dhi + signed_alpha(nmb, 2 * j + 1, bbits);
                    }
                    q[j] = pack_bf16x2(bf16lo_to_f32(q[j]) + dlo, bf16hi_to_f32(q[j]) + dhi);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float d = signed_alpha(nma, j, abits);
                    if constexpr (kTwo) d = d + signed_alpha(nmb, j, bbits);
                    q[j] = __float_as_uint(__uint_as_float(q[j]) + d);
                }
            }
            __builtin_nontemporal_store(q, base + k * kWave);
        }
    }
}

// Ragged end: one thread per element of [start, n).
__device__ __forceinline__ uint32_t element_bit(uint64_t e, uint64_t blk0, uint32_t probe,
                                                uint32_t step, uint32_t k0, uint32_t k1,
                                                const uint8_t *bits)
{
    if (bits) return (bits[e >> 3] >> (e & 7)) & 1u;
    const U32x4 r = probe_block_bits(blk0 + (e >> 7), probe, step, k0, k1);
    const uint32_t sel = (uint32_t)(e >> 5) & 3u;
    const uint32_t word = sel == 0 ? r.x : sel == 1 ? r.y : sel == 2 ? r.z : r.w;
    return (word >> (e & 31)) & 1u;
}

template <bool kBF16, bool kTwo>
__global__ __launch_bounds__(256) void k_perturb_tail(void *__restrict__ theta, uint64_t start,
                                                      uint64_t n, uint64_t blk0, uint32_t step,
                                                      uint32_t probe_a, uint32_t probe_b,
                                                      uint32_t k0, uint32_t k1, uint32_t abits,
                                                      uint32_t bbits,
                                                      const uint8_t *__restrict__ bits_a,
                                                      const uint8_t *__restrict__ bits_b)
{
    const uint64_t e = start + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n) return;
    const uint32_t bit_a = element_bit(e, blk0, probe_a, step, k0, k1, bits_a);
    float d = __uint_as_float(abits ^ (bit_a ? 0u : 0x80000000u));
    if constexpr (kTwo) {
        const uint32_t bit_b = element_bit(e, blk0, probe_b, step, k0, k1, bits_b);
        d = d + __uint_as_float(bbits ^ (bit_b ? 0u : 0x80000000u));
    }
    if constexpr (kBF16) {
        uint16_t *t = static_cast<uint16_t *>(theta);
        const float f = __uint_as_float((uint32_t)t[e] << 16) + d;
        t[e] = (uint16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu);
    } else {
        float *t = static_cast<float *>(theta);
        t[e] = t[e] + d;
    }
}

template <bool kBF16, bool kBits, bool kTwo>
static hipError_t perturb_range(void *theta, uint64_t n, uint64_t blk0, uint32_t step,
                                uint32_t probe_a, uint32_t probe_b, Key key, uint32_t abits,
                                uint32_t bbits, const uint8_t *bits_a, const uint8_t *bits_b,
                                int num_cus, hipStream_t stream)
{
    constexpr uint64_t kChunkParams = chunk_params<kBF16>();
    const uint64_t nchunks = n / kChunkParams;
    (void)num_cus;
    if (nchunks) {
        // Non-persistent: one chunk per single-wave workgroup, eight XCD ranges (a caller
        // splits passes longer than kMaxChunksPerLaunch chunks into several launches).
        const uint32_t grid = xcd_range_grid(nchunks, kWavesPerWG);
        hipLaunchKernelGGL((k_perturb_chunks<kBF16, kBits, kTwo>), dim3(grid),
                           dim3(kWave * kWavesPerWG), 0,
                           stream, static_cast<u32x4_t *>(theta), nchunks, blk0, step, probe_a,
                           probe_b, key.k0, key.k1, abits, bbits,
                           reinterpret_cast<const u32x4_t *>(bits_a),
                           reinterpret_cast<const u32x4_t *>(bits_b));
    }
    const uint64_t start = nchunks * kChunkParams;
    if (start < n) {
        const uint32_t grid = (uint32_t)((n - start + 255) / 256);
        hipLaunchKernelGGL((k_perturb_tail<kBF16, kTwo>), dim3(grid), dim3(256), 0, stream,
                           theta, start, n, blk0, step, probe_a, probe_b, key.k0, key.k1,
                           abits, bbits, bits_a, bits_b);
    }
    return hipGetLastError();
}

// The pass over [0, n) as one launch, or (slice > 0, a multiple of kPerturbChunkParams) as one
// launch per slice of `slice` params in order: each slice is the same pass over its own
// range (its block index and plane bytes advanced with it), so the result is identical.
// Separate launches keep all waves within one slice at a time; on a large buffer whose
// physical placement slows the single launch's eight far-apart XCD streams, this is
// faster (the choice is made per buffer by zo_tune_placement).
template <bool kBF16, bool kBits, bool kTwo>
static hipError_t perturb_impl(void *theta, uint64_t n, uint64_t blk0, uint32_t step,
                               uint32_t probe_a, uint32_t probe_b, Key key, uint32_t abits,
                               uint32_t bbits, const uint8_t *bits_a, const uint8_t *bits_b,
                               uint64_t slice, int num_cus, hipStream_t stream)
{
    constexpr uint64_t kMaxLaunchParams = kMaxChunksPerLaunch * chunk_params<kBF16>();
    if (slice == 0 || slice > kMaxLaunchParams) slice = kMaxLaunchParams;
    if (slice >= n)
        return perturb_range<kBF16, kBits, kTwo>(theta, n, blk0, step, probe_a, probe_b, key,
                                                 abits, bbits, bits_a, bits_b, num_cus, stream);
    constexpr uint64_t kElem = kBF16 ? 2 : 4;
    for (uint64_t s0 = 0; s0 < n; s0 += slice) {
        const uint64_t m = (n - s0) < slice ? (n - s0) : slice;
        const hipError_t e = perturb_range<kBF16, kBits, kTwo>(
            static_cast<char *>(theta) + s0 * kElem, m, blk0 + s0 / kBlockParams, step, probe_a,
            probe_b, key, abits, bbits, bits_a ? bits_a + s0 / 8 : nullptr,
            bits_b ? bits_b + s0 / 8 : nullptr, num_cus, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_perturb(void *theta, bool bf16, uint64_t offset, uint64_t n, Key key,
                          uint32_t step, uint32_t probe, float alpha, const uint8_t *bits,
                          int num_cus, hipStream_t stream, uint64_t slice)
{
    const uint32_t ab = __builtin_bit_cast(uint32_t, alpha);
    const uint64_t b0 = offset / kBlockParams;
    if (bf16)
        return bits ? perturb_impl<true, true, false>(theta, n, b0, step, probe, probe, key, ab,
                                                      0u, bits, nullptr, slice, num_cus, stream)
                    : perturb_impl<true, false, false>(theta, n, b0, step, probe, probe, key, ab,
                                                       0u, nullptr, nullptr, slice, num_cus,
                                                       stream);
    return bits ? perturb_impl<false, true, false>(theta, n, b0, step, probe, probe, key, ab, 0u,
                                                   bits, nullptr, slice, num_cus, stream)
                : perturb_impl<false, false, false>(theta, n, b0, step, probe, probe, key, ab, 0u,
                                                    nullptr, nullptr, slice, num_cus, stream);
}

hipError_t launch_perturb2(void *theta, bool bf16, uint64_t offset, uint64_t n, Key key,
                           uint32_t step, uint32_t probe_a, float alpha_a, uint32_t probe_b,
                           float alpha_b, const uint8_t *bits_a, const uint8_t *bits_b,
                           int num_cus, hipStream_t stream, uint64_t slice)
{
    const uint32_t ab = __builtin_bit_cast(uint32_t, alpha_a);
    const uint32_t bb = __builtin_bit_cast(uint32_t, alpha_b);
    const uint64_t b0 = offset / kBlockParams;
    const uint32_t pa = probe_a, pb = probe_b;
    if (bf16)
        return bits_a ? perturb_impl<true, true, true>(theta, n, b0, step, pa, pb, key, ab, bb,
                                                       bits_a, bits_b, slice, num_cus, stream)
                      : perturb_impl<true, false, true>(theta, n, b0, step, pa, pb, key, ab, bb,
                                                        nullptr, nullptr, slice, num_cus, stream);
    return bits_a ? perturb_impl<false, true, true>(theta, n, b0, step, pa, pb, key, ab, bb,
                                                    bits_a, bits_b, slice, num_cus, stream)
                  : perturb_impl<false, false, true>(theta, n, b0, step, pa, pb, key, ab, bb,
                                                     nullptr, nullptr, slice, num_cus, stream);
}

}  // namespace zo

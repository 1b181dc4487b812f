// k_update.hip -- fused multi-probe update theta <- round(theta - eta * sum_i c_i z_i)
// (the update box of the ZOO loop flowchart in "Pretraining Transformers Without Backprop:
// What Two Zero-Order Papers Actually Measure"; the probe sum of "How 1.5-SPSA Works" on
// "Stanford's 1.5-SPSA Trains OPT-30B Without Backpropagation").
//
// Design (gfx950, wave64, 256-thread workgroups):
//  * Tables.  Probes are taken eight at a time (group g = probes 8g .. 8g+7).  For each
//    group the workgroup builds T_g[b] = sum_{k<8} (bit k of b ? +c : -c)_{8g+k} for all
//    256 byte values b (k ascending, fp64) in LDS; n_pert = 160 needs 40 KiB.  Probes past
//    n_pert are padded with c = 0.  Then s_j = sum_g T_g[b_gj] with b_gj the byte whose bit
//    k is the sign bit of probe 8g+k at param j -- one LDS lookup per 8 probes.
//  * Precision.  Tables and sums are fp64 (full-rate VALU adds on CDNA4), so s_j carries
//    ~1e-16 relative error; the new value is (double)theta - (double)eta * s_j, rounded
//    once: to fp32 directly, or to bf16 through round-to-odd fp32 and the hardware
//    nearest-even fp32->bf16 convert, which together round the double correctly.  With
//    fp32 sums the update could miss the bf16 result by several ulps wherever theta and
//    eta*s nearly cancel.
//  * Work split.  A wave takes 8 consecutive 128-param blocks; the 8 lanes of an "octet"
//    share one block.  Per group, lane r of an octet produces probe 8g+r's 128 bits for
//    that block (Philox, or 16 bytes of a stored row), so no Philox call is repeated.
//    Lane r of the octet owns two runs of 8 params, 8r .. 8r+7 and 64+8r .. 64+8r+7 (sign
//    bytes r and r+8 of the block), so that the octet's 16-byte accesses to a run of theta
//    cover whole 128-byte lines in one instruction (a lane owning 16 consecutive params
//    instead would leave each instruction 16-byte pieces 32 or 64 bytes apart: measured
//    on a 500 MB buffer, 2.7 against 5.4 TB/s in fp32, 4.9 against 5.9 in bf16).  The
//    octet swaps the 16-bit byte pairs (byte j, byte j+8) of its eight probes through a
//    1 KiB per-wave LDS slice (four v_perm_b32 and eight 16-bit stores per lane, one
//    16-byte read); four v_perm_b32 and two 8x8 bit transposes then turn the eight
//    probes' bytes r and r+8 into the lane's 16 table indices.
//  * Each lane keeps 16 fp64 sums (tables in ascending group order), then reads its 16
//    params once, forms and rounds the new values, and writes them once.
//  * Deterministic: every sum is taken in a fixed order independent of the grid.
//  * Restore variant (kRestore): before the update, each parameter first gets the in-place
//    move theta + (bit ? alpha_r : -alpha_r) of one of the step's probes, rounded exactly
//    as zo_perturb rounds it -- the last restore of the two-pass schedule, which nothing
//    reads before the update, folded into the update's single pass over theta.  That
//    probe's bits are produced by the update anyway: after the octet exchange of its group,
//    lane r holds bytes r and r+8 of every probe of the group, the 16 sign bits of its own
//    params, so the fold costs no extra Philox call.  (The unrolled
//    form below takes them from one Philox call of their own per lane and block instead.)
//  * Unrolled form.  At the group counts of the usual probe counts (2, 4, 8, 20 groups) the
//    group loop is unrolled and the tables sit at fixed LDS addresses, so each lookup's
//    table offset is an immediate of the LDS read and its index one byte-select shift.
#include <stdlib.h>

#include "zo_device.hpp"
#include "zo_launch.hpp"

namespace zo {

constexpr int kUpdWavesPerWG = 8;
constexpr int kUpdThreads = kUpdWavesPerWG * kWave;
constexpr int kUpdBlocksPerWave = 8;
// 8 octets x (8 readers x 8 probes x 16 bits), octet slices 40 words apart so that the
// eight octets' stores of one slot fall in distinct LDS banks (a 32-word stride would put
// the even and the odd octets on the same banks).
constexpr uint32_t kOctetStride = 40;
constexpr uint32_t kXchWordsPerWave = 8 * kOctetStride;
static_assert(kUpdWavesPerWG * kXchWordsPerWave >= 8 * ((kMaxNpert + 7) / 8),
              "the exchange slices stage the weights of every group");

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// In-register transpose of an 8x8 bit matrix held as two dwords (rows 0-3 in L, rows
// 4-7 in H, row k = byte k, column b = bit b): afterwards byte b holds column b.
// Three masked delta swaps, one per bit of the row and column index (distances 7, 14, 28
// in the 64-bit view; they commute).  A swap is t = (x ^ (x >> d)) & mask;
// x ^= t ^ (t << d).  For d = 7 and 14 the shifts act on the register pair as one 64-bit
// value (no masked bit crosses the dword boundary), one v_lshrrev_b64 / v_lshlrev_b64
// each instead of two 32-bit shifts; the compiler turns 64-bit shifts written in C into
// 32-bit pairs or multiplies, so they are spelled out (plain ALU instructions, no memory
// access).  The d = 28 swap exchanges L's high nibbles with H's
// low nibbles: two shifts and two bit selects.
template <int D>
__device__ __forceinline__ uint64_t shr64(uint64_t x)
{
    uint64_t r;
    asm("v_lshrrev_b64 %0, %1, %2" : "=v"(r) : "n"(D), "v"(x));
    return r;
}
template <int D>
__device__ __forceinline__ uint64_t shl64(uint64_t x)
{
    uint64_t r;
    asm("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "n"(D), "v"(x));
    return r;
}

template <int D>
__device__ __forceinline__ void delta_swap2(uint32_t &L, uint32_t &H, uint32_t mask)
{
    const uint64_t x = ((uint64_t)H << 32) | L;
    const uint64_t s = shr64<D>(x);
    const uint32_t tl = ZO_BITOP3(L, (uint32_t)s, mask, kXorAnd);
    const uint32_t th = ZO_BITOP3(H, (uint32_t)(s >> 32), mask, kXorAnd);
    const uint64_t u = shl64<D>(((uint64_t)th << 32) | tl);
    L = ZO_BITOP3(L, tl, (uint32_t)u, kXor3);
    H = ZO_BITOP3(H, th, (uint32_t)(u >> 32), kXor3);
}

__device__ __forceinline__ void transpose8x8(uint32_t &L, uint32_t &H)
{
    delta_swap2<7>(L, H, 0x00AA00AAu);
    delta_swap2<14>(L, H, 0x0000CCCCu);
    const uint32_t l = L, h = H;
    L = ZO_BITOP3(l, h << 4, 0xF0F0F0F0u, 0xD8);   // mask ? h << 4 : l
    H = ZO_BITOP3(l >> 4, h, 0xF0F0F0F0u, 0xD8);   // mask ? h : l >> 4
}

// double -> fp32 rounded to odd: truncate toward zero, then set the last bit if anything
// was lost.  A later round-to-nearest-even to a format with at least two fewer
// significand bits (bf16 has 8 against fp32's 24) then rounds the double correctly.
__device__ __forceinline__ float f64_to_f32_round_odd(double d)
{
    const float f = (float)d;
    const double back = (double)f;
    uint32_t u = __float_as_uint(f);
    if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1u;   // RNE rounded away from zero
    if (back != d) u |= 1u;                                  // inexact (NaN stays NaN)
    return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t bf16pair_from_f64(double lo, double hi)
{
    return pack_bf16x2(f64_to_f32_round_odd(lo), f64_to_f32_round_odd(hi));
}

// The restore move of parameter e0 + q: +alpha_r if bit q of rmask is set, else -alpha_r
// (the sign bit of alpha_r flipped where the bit is clear; q is a constant after unrolling).
__device__ __forceinline__ float restore_step(uint32_t rmask, int q, uint32_t rabits)
{
    return __uint_as_float(rabits ^ ((~rmask << (31 - q)) & 0x80000000u));
}

// theta_j + d rounded as zo_perturb rounds it, for a packed bf16 pair (lo = param 2j).
__device__ __forceinline__ uint32_t restore_bf16_pair(uint32_t w, float dlo, float dhi)
{
    return pack_bf16x2(bf16lo_to_f32(w) + dlo, bf16hi_to_f32(w) + dhi);
}

// Table entry of byte q of x, the byte times 8 being its LDS byte offset: one shift with an
// SDWA byte select.  The compiler emits that form for bytes 1-3 by itself but masks and
// shifts byte 0 in two instructions, so byte 0's is spelled out (a plain ALU instruction).
__device__ __forceinline__ double lookup(const double *tg, uint32_t x, int q)
{
    uint32_t off;
    if (q == 0)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
            : "=v"(off) : "v"(x));
    else
        off = ((x >> (8 * q)) & 255u) << 3;
    return *reinterpret_cast<const double *>(reinterpret_cast<const char *>(tg) + off);
}

// The lane's 16 params are the runs e0 .. e0+7 and e0+64 .. e0+71: s[q] and bit q of rmask
// belong to param e0 + q for q < 8 and to param e0 + 56 + q for q >= 8.
template <bool kBF16, bool kRestore>
__device__ __forceinline__ void apply_update(void *theta, uint64_t e0, uint64_t n,
                                             const double (&s)[16], double eta, uint32_t rmask,
                                             uint32_t rabits)
{
    if (e0 + 72 <= n) {
        if constexpr (kBF16) {
            uint16_t *base = static_cast<uint16_t *>(theta) + e0;
            u32x4_t *p0 = reinterpret_cast<u32x4_t *>(base);
            u32x4_t *p1 = reinterpret_cast<u32x4_t *>(base + 64);
            u32x4_t t0 = __builtin_nontemporal_load(p0);
            u32x4_t t1 = __builtin_nontemporal_load(p1);
            if constexpr (kRestore) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    t0[j] = restore_bf16_pair(t0[j], restore_step(rmask, 2 * j, rabits),
                                              restore_step(rmask, 2 * j + 1, rabits));
                    t1[j] = restore_bf16_pair(t1[j], restore_step(rmask, 8 + 2 * j, rabits),
                                              restore_step(rmask, 9 + 2 * j, rabits));
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                t0[j] = bf16pair_from_f64((double)bf16lo_to_f32(t0[j]) - eta * s[2 * j],
                                          (double)bf16hi_to_f32(t0[j]) - eta * s[2 * j + 1]);
                t1[j] = bf16pair_from_f64((double)bf16lo_to_f32(t1[j]) - eta * s[8 + 2 * j],
                                          (double)bf16hi_to_f32(t1[j]) - eta * s[9 + 2 * j]);
            }
            __builtin_nontemporal_store(t0, p0);
            __builtin_nontemporal_store(t1, p1);
        } else {
            float *base = static_cast<float *>(theta) + e0;
            u32x4_t *p[4] = {reinterpret_cast<u32x4_t *>(base), reinterpret_cast<u32x4_t *>(base + 4),
                             reinterpret_cast<u32x4_t *>(base + 64),
                             reinterpret_cast<u32x4_t *>(base + 68)};
            u32x4_t t[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) t[v] = __builtin_nontemporal_load(p[v]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                if constexpr (kRestore) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        t[v][j] = __float_as_uint(__uint_as_float(t[v][j]) +
                                                  restore_step(rmask, 4 * v + j, rabits));
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    t[v][j] = __float_as_uint(
                        (float)((double)__uint_as_float(t[v][j]) - eta * s[4 * v + j]));
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) __builtin_nontemporal_store(t[v], p[v]);
        }
    } else if (e0 < n) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const uint64_t e = e0 + (q < 8 ? (uint64_t)q : (uint64_t)(56 + q));
            if (e < n) {
                if constexpr (kBF16) {
                    uint16_t *t = static_cast<uint16_t *>(theta);
                    uint32_t w = t[e];
                    if constexpr (kRestore)
                        w = restore_bf16_pair(w, restore_step(rmask, q, rabits), 0.0f) & 0xFFFFu;
                    const double v = (double)__uint_as_float(w << 16) - eta * s[q];
                    t[e] = (uint16_t)(bf16pair_from_f64(v, 0.0) & 0xFFFFu);
                } else {
                    float *t = static_cast<float *>(theta);
                    float x = t[e];
                    if constexpr (kRestore) x = x + restore_step(rmask, q, rabits);
                    t[e] = (float)((double)x - eta * s[q]);
                }
            }
        }
    }
}

// Occupancy is bounded by the LDS (sign tables + exchange, ~50 KiB per 512-thread
// workgroup at n_pert = 160: three workgroups, six waves per SIMD), which the compiler
// cannot see for the dynamic-LDS form; telling it so lets it keep several table lookups in
// flight instead of squeezing registers for an occupancy the LDS never allows.
//
// kNG > 0: the group count is a compile-time constant; the tables and the exchange slices
// are static LDS at known addresses and the group loop is unrolled, so every table read
// carries its group's table offset as the instruction's immediate offset and the lookup
// index costs a single byte-select shift.  kNG == 0: any group count, tables in dynamic LDS.
// Two unrolled groups leave the compiler more to interleave: at six waves (80 registers)
// the restore form would spill two loop-invariant registers; five waves (96) do not.
template <int kNG>
constexpr int kUpdWaves = kNG == 2 ? 5 : 6;

template <bool kBF16, bool kBits, bool kRestore, int kNG>
__global__ __launch_bounds__(kUpdThreads) __attribute__((amdgpu_waves_per_eu(kUpdWaves<kNG>, kUpdWaves<kNG>))) void k_update(void *__restrict__ theta, uint64_t n,
                                                        uint64_t blk0, uint32_t step,
                                                        uint32_t k0, uint32_t k1,
                                                        const float *__restrict__ c,
                                                        uint32_t npert, uint32_t ngroups,
                                                        double eta,
                                                        const uint8_t *__restrict__ bits,
                                                        uint64_t stride, uint32_t rprobe,
                                                        uint32_t rabits)
{
    __shared__ double stbl[kNG > 0 ? kNG * 256 : 1];
    __shared__ uint32_t sxch[kNG > 0 ? kUpdWavesPerWG * kXchWordsPerWave : 1];
    extern __shared__ double lds_d[];
    const uint32_t ng = kNG > 0 ? (uint32_t)kNG : ngroups;
    double *tbl = kNG > 0 ? stbl : lds_d;
    const int wv = threadIdx.x / kWave;
    uint32_t *xbase = kNG > 0 ? sxch : reinterpret_cast<uint32_t *>(lds_d + ngroups * 256u);
    uint32_t *xch = xbase + wv * kXchWordsPerWave;

    // The weights, padded with zeros to whole groups, staged once in the (not yet used)
    // exchange slices: one global read per probe instead of eight per table entry.
    float *cw = reinterpret_cast<float *>(xbase);
    for (uint32_t i = threadIdx.x; i < ng * 8u; i += blockDim.x) cw[i] = i < npert ? c[i] : 0.0f;
    __syncthreads();
    // Signed partial-sum tables, probes ascending within each group.
    for (uint32_t e = threadIdx.x; e < ng * 256u; e += blockDim.x) {
        const uint32_t g = e >> 8, b = e & 255u;
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const double ci = (double)cw[g * 8u + (uint32_t)k];
            acc = acc + (((b >> k) & 1u) ? ci : -ci);
        }
        tbl[e] = acc;
    }
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const int oct = lane >> 3;
    const int r = lane & 7;
    uint32_t *oxch = xch + oct * kOctetStride;
    // 16-bit slot (reader j, probe k) of the octet's slice: reader j's eight slots are one
    // aligned 16-byte read.
    uint16_t *oslot = reinterpret_cast<uint16_t *>(oxch);

    const uint64_t nblk = (n + kBlockParams - 1) / kBlockParams;
    const uint64_t nwc = (nblk + kUpdBlocksPerWave - 1) / kUpdBlocksPerWave;
    const uint64_t nwaves = (uint64_t)gridDim.x * kUpdWavesPerWG;

    for (uint64_t wc = (uint64_t)blockIdx.x * kUpdWavesPerWG + wv; wc < nwc; wc += nwaves) {
        const uint64_t lb = wc * kUpdBlocksPerWave + oct;  // local block of this octet
        const uint64_t e0 = lb * kBlockParams + 8u * (uint32_t)r;   // the lane's first run
        double s[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) s[q] = 0.0;
        uint32_t rmask = 0;   // kRestore: bit q = sign bit of probe rprobe at the lane's param q
        // The lane's probe slot, opaque to the optimiser inside this loop: with the group
        // loop unrolled, everything derived from it per group (the probe's first Philox
        // product, its bit-row address) would otherwise be hoisted out of the block loop and
        // held in registers for all groups at once.
        uint32_t rr = (uint32_t)r;
        if constexpr (kNG > 0) asm volatile("" : "+v"(rr));

        auto group = [&](uint32_t g) {
            const uint32_t i = g * 8u + rr;
            u32x4_t w = {0u, 0u, 0u, 0u};
            if constexpr (kBits) {
                if (i < npert && lb < nblk)
                    w = *reinterpret_cast<const u32x4_t *>(bits + (uint64_t)i * stride + lb * 16u);
            } else if (kNG > 0) {
                // Probes past n_pert carry c = 0: their table entries do not depend on the
                // bits, so they are generated unconditionally (no divergent branch).
                const U32x4 q = probe_block_bits(blk0 + lb, i, step, k0, k1);
                w = u32x4_t{q.x, q.y, q.z, q.w};
            } else if (i < npert) {
                const U32x4 q = probe_block_bits(blk0 + lb, i, step, k0, k1);
                w = u32x4_t{q.x, q.y, q.z, q.w};
            }
            // pair j = byte j | byte j+8 << 8 of this lane's probe, for j = 0 .. 7
            const uint32_t p01 = __builtin_amdgcn_perm(w.z, w.x, 0x05010400u);
            const uint32_t p23 = __builtin_amdgcn_perm(w.z, w.x, 0x07030602u);
            const uint32_t p45 = __builtin_amdgcn_perm(w.w, w.y, 0x05010400u);
            const uint32_t p67 = __builtin_amdgcn_perm(w.w, w.y, 0x07030602u);
            wave_lds_sync();  // previous group's reads precede these writes
            oslot[0 * 8 + r] = (uint16_t)p01;
            oslot[1 * 8 + r] = (uint16_t)(p01 >> 16);
            oslot[2 * 8 + r] = (uint16_t)p23;
            oslot[3 * 8 + r] = (uint16_t)(p23 >> 16);
            oslot[4 * 8 + r] = (uint16_t)p45;
            oslot[5 * 8 + r] = (uint16_t)(p45 >> 16);
            oslot[6 * 8 + r] = (uint16_t)p67;
            oslot[7 * 8 + r] = (uint16_t)(p67 >> 16);
            wave_lds_sync();
            // x.k/2 = (byte r, byte r+8) of probes k and k+1 of the group, k even
            const u32x4_t x = *reinterpret_cast<const u32x4_t *>(oxch + 4 * r);
            uint32_t Llo = __builtin_amdgcn_perm(x.y, x.x, 0x06040200u);   // byte r, probes 0-3
            uint32_t Lhi = __builtin_amdgcn_perm(x.y, x.x, 0x07050301u);   // byte r+8
            uint32_t Hlo = __builtin_amdgcn_perm(x.w, x.z, 0x06040200u);   // probes 4-7
            uint32_t Hhi = __builtin_amdgcn_perm(x.w, x.z, 0x07050301u);
            transpose8x8(Llo, Hlo);
            transpose8x8(Lhi, Hhi);
            if constexpr (kRestore && kNG == 0) {
                if (g == (rprobe >> 3)) {   // uniform: the restore probe's group
                    const uint32_t k = rprobe & 7u;
                    const uint32_t word = k < 2 ? x.x : k < 4 ? x.y : k < 6 ? x.z : x.w;
                    rmask = (word >> (16u * (k & 1u))) & 0xFFFFu;
                }
            }
            const double *tg = tbl + g * 256u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s[q] += lookup(tg, Llo, q);
                s[4 + q] += lookup(tg, Hlo, q);
                s[8 + q] += lookup(tg, Lhi, q);
                s[12 + q] += lookup(tg, Hhi, q);
            }
        };
        if constexpr (kNG > 0) {
#pragma unroll
            for (int g = 0; g < kNG; ++g) {
                group((uint32_t)g);
                // Keep each group's work together: interleaving groups only raises the
                // register demand past the occupancy budget (and spills).
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            for (uint32_t g = 0; g < ngroups; ++g) group(g);
        }
        if constexpr (kNG > 0 && kRestore) {
            // The restore probe's bits for the lane's 16 params from their own Philox call
            // (bytes r and r+8), instead of picking them out of whichever unrolled group
            // holds that probe.
            const U32x4 q = probe_block_bits(blk0 + lb, rprobe, step, k0, k1);
            const uint32_t lo = (rr >> 2) ? q.y : q.x, hi = (rr >> 2) ? q.w : q.z;
            const uint32_t b = rr & 3u;   // byte b of lo, byte b of hi, then zeros
            rmask = __builtin_amdgcn_perm(hi, lo, b | ((4u + b) << 8) | 0x0C0C0000u);
        }
        apply_update<kBF16, kRestore>(theta, e0, n, s, eta, rmask, rabits);
    }
}

// Dynamic LDS of the general kernel: the sign tables of `ngroups` groups and the
// per-wave exchange slices.
static size_t general_lds_bytes(uint32_t ngroups)
{
    return (size_t)ngroups * 256u * 8u + (size_t)kUpdWavesPerWG * kXchWordsPerWave * 4u;
}

// Launch-shape override from the environment (read once per process): workgroups per CU,
// accepted in [1, 64], anything else keeps the default.
static int env_int(const char *name, int dflt)
{
    const char *s = getenv(name);
    if (!s || !*s) return dflt;
    const int v = atoi(s);
    return (v >= 1 && v <= 64) ? v : dflt;
}

template <bool kBF16, bool kBits, bool kRestore, int kNG>
static hipError_t update_launch(void *theta, uint64_t n, uint64_t blk0, uint32_t step, Key key,
                                const float *c, uint32_t npert, float eta, const uint8_t *bits,
                                uint32_t rprobe, float ralpha, int num_cus, hipStream_t stream)
{
    const uint32_t ngroups = (npert + 7u) / 8u;
    // above 64 KiB the general kernel relies on the limit raised once per device by
    // prepare_update (from zo_init), so that a launch makes no runtime call but the launch
    const size_t lds = kNG > 0 ? 0 : general_lds_bytes(ngroups);
    const uint64_t nblk = (n + kBlockParams - 1) / kBlockParams;
    const uint64_t nwc = (nblk + kUpdBlocksPerWave - 1) / kUpdBlocksPerWave;
    // Many workgroups per CU: each builds its tables once and the persistent loop's tail
    // imbalance shrinks with the share per workgroup (measured: 154 ms at 4 per CU, 144 ms
    // from 16 per CU on, 30B bf16 params, n_pert = 160).
    static const int wg_per_cu = env_int("ZO_UPDATE_WG_PER_CU", 16);
    const uint64_t want = (nwc + kUpdWavesPerWG - 1) / kUpdWavesPerWG;
    const uint64_t cap = (uint64_t)num_cus * wg_per_cu;
    const uint32_t grid = (uint32_t)(want < cap ? want : cap);
    hipLaunchKernelGGL((k_update<kBF16, kBits, kRestore, kNG>), dim3(grid), dim3(kUpdThreads),
                       lds, stream, theta, n, blk0, step, key.k0, key.k1, c, npert, ngroups,
                       (double)eta, bits, (uint64_t)nblk * 16u, rprobe,
                       __builtin_bit_cast(uint32_t, ralpha));
    return hipGetLastError();
}

// Group counts with an unrolled kernel (probes regenerated): those of n_pert = 16, 32, 64 and
// 160.  Other counts, and stored bits (a streaming read that the unrolled form does not
// speed up), take the general kernel.  ZO_UPDATE_GENERIC=1 forces the general kernel.
template <bool kBF16, bool kBits, bool kRestore>
static hipError_t update_impl(void *theta, uint64_t n, uint64_t blk0, uint32_t step, Key key,
                              const float *c, uint32_t npert, float eta, const uint8_t *bits,
                              uint32_t rprobe, float ralpha, int num_cus, hipStream_t stream)
{
    static const bool generic = env_int("ZO_UPDATE_GENERIC", 0) == 1;
    const uint32_t ngroups = (npert + 7u) / 8u;
#define ZO_UPD(NG)                                                                           \
    update_launch<kBF16, kBits, kRestore, NG>(theta, n, blk0, step, key, c, npert, eta, bits, \
                                              rprobe, ralpha, num_cus, stream)
    if constexpr (!kBits) {
        if (!generic) {
            switch (ngroups) {
            case 2: return ZO_UPD(2);
            case 4: return ZO_UPD(4);
            case 8: return ZO_UPD(8);
            case 20: return ZO_UPD(20);
            default: break;
            }
        }
    }
    return ZO_UPD(0);
#undef ZO_UPD
}

template <bool kRestore>
static hipError_t update_dispatch(void *theta, bool bf16, uint64_t offset, uint64_t n, Key key,
                                  uint32_t step, const float *c, uint32_t npert, float eta,
                                  const uint8_t *bits, uint32_t rprobe, float ralpha,
                                  int num_cus, hipStream_t stream)
{
    const uint64_t blk0 = offset / kBlockParams;
    if (bf16)
        return bits ? update_impl<true, true, kRestore>(theta, n, blk0, step, key, c, npert, eta,
                                                        bits, rprobe, ralpha, num_cus, stream)
                    : update_impl<true, false, kRestore>(theta, n, blk0, step, key, c, npert,
                                                         eta, bits, rprobe, ralpha, num_cus,
                                                         stream);
    return bits ? update_impl<false, true, kRestore>(theta, n, blk0, step, key, c, npert, eta,
                                                     bits, rprobe, ralpha, num_cus, stream)
                : update_impl<false, false, kRestore>(theta, n, blk0, step, key, c, npert, eta,
                                                      bits, rprobe, ralpha, num_cus, stream);
}

template <bool kBF16, bool kBits, bool kRestore>
static hipError_t raise_lds_limit(int bytes)
{
    return hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_update<kBF16, kBits, kRestore, 0>),
        hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t prepare_update()
{
    const int bytes = (int)general_lds_bytes((kMaxNpert + 7u) / 8u);
    const hipError_t e[8] = {
        raise_lds_limit<false, false, false>(bytes), raise_lds_limit<false, false, true>(bytes),
        raise_lds_limit<false, true, false>(bytes),  raise_lds_limit<false, true, true>(bytes),
        raise_lds_limit<true, false, false>(bytes),  raise_lds_limit<true, false, true>(bytes),
        raise_lds_limit<true, true, false>(bytes),   raise_lds_limit<true, true, true>(bytes)};
    for (hipError_t x : e)
        if (x != hipSuccess) return x;
    return hipSuccess;
}

hipError_t launch_update(void *theta, bool bf16, uint64_t offset, uint64_t n, Key key,
                         uint32_t step, const float *c, uint32_t npert, float eta,
                         const uint8_t *bits, int num_cus, hipStream_t stream)
{
    return update_dispatch<false>(theta, bf16, offset, n, key, step, c, npert, eta, bits, 0u,
                                  0.0f, num_cus, stream);
}

hipError_t launch_restore_update(void *theta, bool bf16, uint64_t offset, uint64_t n, Key key,
                                 uint32_t step, uint32_t rprobe, float ralpha, const float *c,
                                 uint32_t npert, float eta, const uint8_t *bits, int num_cus,
                                 hipStream_t stream)
{
    return update_dispatch<true>(theta, bf16, offset, n, key, step, c, npert, eta, bits, rprobe,
                                 ralpha, num_cus, stream);
}

}  // namespace zo

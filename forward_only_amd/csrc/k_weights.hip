// k_weights.hip -- probe weights from the step's losses, the non-finite counter fill,
// and the diagonal-quadratic loss used by the synthetic workloads.
#include "zo_device.hpp"
#include "zo_launch.hpp"

namespace zo {

// Probe weights, fp64 ("How 1.5-SPSA Works" on "Stanford's 1.5-SPSA Trains OPT-30B Without
// Backpropagation" for the central difference; its "Probe-Space Preconditioning" section
// for the clean-pass curvature weight):
//   g = (L+ - L-) / (2 eps),  h = ((L+ + L-) - 2 L0) / eps^2,  c = g / max(|h|, delta).
// Division, add and multiply are the IEEE double operations (no contraction in this
// file), then one round-to-nearest-even to fp32.  A non-finite loss drops the probe
// (c = 0) and bumps the device counter.
// The other weight forms of the pages share the kernel (mode): 1 divides by
// max(|h|, delta)^power (the curvature-power weight of "Probe-Space Preconditioning", whose
// exponent the page gives as 0.1), 2 is the plain 1SPSA mean g / n_pert of "How 1.5-SPSA
// Works" (no clean pass; L0 is not read).
__global__ __launch_bounds__(256) void k_probe_weights(const double *__restrict__ Lp,
                                                       const double *__restrict__ Lm,
                                                       const double *__restrict__ L0p,
                                                       uint32_t npert, double eps, double delta,
                                                       int mode, double power,
                                                       float *__restrict__ c,
                                                       uint32_t *__restrict__ counter)
{
    const bool uses_l0 = mode != 2;
    const double L0 = uses_l0 ? *L0p : 0.0;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < npert;
         i += gridDim.x * blockDim.x) {
        const double lp = Lp[i], lm = Lm[i];
        if (!__builtin_isfinite(lp) || !__builtin_isfinite(lm) ||
            (uses_l0 && !__builtin_isfinite(L0))) {
            c[i] = 0.0f;
            atomicAdd(counter, 1u);
            continue;
        }
        const double g = (lp - lm) / (2.0 * eps);
        if (mode == 2) {
            c[i] = (float)(g / (double)npert);
            continue;
        }
        const double h = ((lp + lm) - 2.0 * L0) / (eps * eps);
        const double ah = __builtin_fabs(h);
        double den = ah > delta ? ah : delta;
        if (mode == 1) den = pow(den, power);
        c[i] = (float)(g / den);
    }
}

hipError_t launch_probe_weights(const double *Lp, const double *Lm, const double *L0,
                                uint32_t npert, double eps, double delta, int mode,
                                double power, float *c, uint32_t *counter, hipStream_t stream)
{
    const uint32_t grid = (npert + 255u) / 256u;
    const uint32_t g = grid < 64u ? grid : 64u;
    hipLaunchKernelGGL(k_probe_weights, dim3(g), dim3(256), 0, stream, Lp, Lm, L0, npert, eps,
                       delta, mode, power, c, counter);
    return hipGetLastError();
}

__global__ void k_zero_u32(uint32_t *__restrict__ p, uint32_t count)
{
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = 0u;
}

hipError_t launch_zero_u32(uint32_t *p, uint32_t count, hipStream_t stream)
{
    hipLaunchKernelGGL(k_zero_u32, dim3((count + 63u) / 64u), dim3(64), 0, stream, p, count);
    return hipGetLastError();
}

// ---- diagonal quadratic loss: 1/2 sum_j a_j theta_j^2 in fp64 ------------------------
// Pass 1: kLossPartials workgroups of four waves; wave w of the grid takes the chunks of
// kLossChunk params w, w + W, w + 2W, ... (W = total waves).  In a chunk, lane l reads
// params 256k + 4l .. 256k + 4l + 3 for k = 0 .. 7: every load instruction moves one
// contiguous KiB of a (and of fp32 theta; half a KiB of bf16 theta), and all sixteen of a
// chunk's loads are issued before any is used, so each wave keeps 12-16 KiB in flight.
// Then the ragged end (n mod kLossChunk params) one element per thread; each wave adds its
// lanes with a fixed butterfly and the workgroup adds its waves in order.  Pass 2: one
// workgroup adds the partials the same way.  The partition depends only on n, so the
// result is bit-reproducible.
constexpr uint32_t kLossChunk = 2048;

// One term of the sum, a_j t_j^2 added to acc with a single rounding: t is a widened fp32
// value, so t^2 (at most 48 significant bits) is exact in fp64 and fma(a, t^2, acc) rounds
// the exact a t^2 + acc once.  Spelled out so that every kernel accumulating this sum (the
// plain loss and the probes' losses below) rounds it identically.
__device__ __forceinline__ double quad_term_sq(double acc, double a, double t2)
{
    return __builtin_fma(a, t2, acc);
}
__device__ __forceinline__ double quad_term(double acc, float a, double t)
{
    return quad_term_sq(acc, (double)a, t * t);
}
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
    return v;
}

// Sum over the workgroup (256 threads = 4 waves), wave sums added in wave order.
__device__ __forceinline__ double block_sum256(double v, double *red)
{
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const double s = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return s;
}

template <bool kBF16>
__device__ __forceinline__ void theta8(const void *theta, uint64_t g, double (&t)[8])
{
    if constexpr (kBF16) {
        const u32x4_t w = static_cast<const u32x4_t *>(theta)[g];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            t[2 * q] = (double)bf16lo_to_f32(w[q]);
            t[2 * q + 1] = (double)bf16hi_to_f32(w[q]);
        }
    } else {
        const f32x4_t x0 = static_cast<const f32x4_t *>(theta)[2 * g];
        const f32x4_t x1 = static_cast<const f32x4_t *>(theta)[2 * g + 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            t[q] = (double)x0[q];
            t[4 + q] = (double)x1[q];
        }
    }
}

template <bool kBF16>
__device__ __forceinline__ double theta1(const void *theta, uint64_t j)
{
    if constexpr (kBF16)
        return (double)__uint_as_float((uint32_t)static_cast<const uint16_t *>(theta)[j] << 16);
    else
        return (double)static_cast<const float *>(theta)[j];
}

template <bool kBF16>
__global__ __launch_bounds__(256) void k_quad_loss_partial(const void *__restrict__ theta,
                                                           const float *__restrict__ a,
                                                           uint64_t n, double *__restrict__ part)
{
    __shared__ double red[4];
    double acc = 0.0;
    const uint64_t G = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t nwaves = (uint64_t)gridDim.x * (blockDim.x / 64u);
    const uint64_t nchunks = n / kLossChunk;
    for (uint64_t c = tid / 64u; c < nchunks; c += nwaves) {
        const uint64_t p0 = c * kLossChunk + 4u * lane;   // + 256 k
        const f32x4_t *ap = reinterpret_cast<const f32x4_t *>(a + p0);
        f32x4_t av[8];
        float tv[8][4];
        if constexpr (kBF16) {
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            const u32x2_t *tp =
                reinterpret_cast<const u32x2_t *>(static_cast<const uint16_t *>(theta) + p0);
            u32x2_t w[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) w[k] = __builtin_nontemporal_load(tp + 64 * k);
#pragma unroll
            for (int k = 0; k < 8; ++k) av[k] = __builtin_nontemporal_load(ap + 64 * k);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                tv[k][0] = bf16lo_to_f32(w[k][0]);
                tv[k][1] = bf16hi_to_f32(w[k][0]);
                tv[k][2] = bf16lo_to_f32(w[k][1]);
                tv[k][3] = bf16hi_to_f32(w[k][1]);
            }
        } else {
            const f32x4_t *tp = reinterpret_cast<const f32x4_t *>(static_cast<const float *>(theta) + p0);
            f32x4_t x[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = __builtin_nontemporal_load(tp + 64 * k);
#pragma unroll
            for (int k = 0; k < 8; ++k) av[k] = __builtin_nontemporal_load(ap + 64 * k);
#pragma unroll
            for (int k = 0; k < 8; ++k)
#pragma unroll
                for (int q = 0; q < 4; ++q) tv[k][q] = x[k][q];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = quad_term(acc, av[k][q], (double)tv[k][q]);
    }
    for (uint64_t j = nchunks * kLossChunk + tid; j < n; j += G)
        acc = quad_term(acc, a[j], theta1<kBF16>(theta, j));
    const double s = block_sum256(acc, red);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_sum_partials(const double *__restrict__ part,
                                                      uint32_t count, double scale,
                                                      double *__restrict__ out)
{
    __shared__ double red[4];
    double acc = 0.0;
    for (uint32_t i = threadIdx.x; i < count; i += blockDim.x) acc += part[i];
    const double s = block_sum256(acc, red);
    if (threadIdx.x == 0) *out = scale * s;
}

// ---- the same loss at theta +/- alpha z_i of several probes, theta read once ------------
// For each of up to kQuadProbes consecutive probes and both signs: the value an in-place
// zo_perturb would store (one fp32 add of the signed alpha; for bf16, widen, add, round to
// nearest even) squared into the sum -- theta itself is never written.  The partition into
// chunks, each lane's order of terms, the tail and both reductions are those of
// k_quad_loss_partial / k_sum_partials, per probe and sign, so each loss equals zo_perturb
// followed by zo_quad_loss bit for bit.  Signs: per chunk (16 blocks of 128 params) the
// wave's lanes produce the 16 x kQuadProbes blocks' bits once (one Philox call or one
// 16-byte row read per lane) into an LDS slice laid out [block][word][probe], and each lane
// reads, per group of 4 params, one 16-byte vector holding that word of every probe.
// m ? a : b for a lane mask m of all ones or all zeros, word by word.
__device__ __forceinline__ double select_f64(uint32_t m, double a, double b)
{
    const uint64_t ua = __builtin_bit_cast(uint64_t, a), ub = __builtin_bit_cast(uint64_t, b);
    const uint32_t lo = ((uint32_t)ua & m) | ((uint32_t)ub & ~m);
    const uint32_t hi = ((uint32_t)(ua >> 32) & m) | ((uint32_t)(ub >> 32) & ~m);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// The four params' terms for every probe and sign.  A perturbed value is one of two
// candidates, rnd(x + alpha) and rnd(x - alpha) (what zo_perturb stores for a set and for a
// clear sign bit under +alpha, and the other way round under -alpha), so both are formed
// and squared once per param and each probe's sign bit picks between them.  With kClean the
// last accumulator also takes the unperturbed terms, as the single-probe loss kernel forms
// them.
template <bool kBF16, bool kClean>
__device__ __forceinline__ void quad_terms4(double (&acc)[2 * kQuadProbes + kClean], const float (&x)[4],
                                            const float (&av)[4], const uint32_t (&w)[kQuadProbes],
                                            uint32_t sh, float alpha)
{
    float xa[4], xb[4];
    if constexpr (kBF16) {
#pragma unroll
        for (int q = 0; q < 4; q += 2) {
            const uint32_t pa = pack_bf16x2(x[q] + alpha, x[q + 1] + alpha);
            const uint32_t pb = pack_bf16x2(x[q] + (-alpha), x[q + 1] + (-alpha));
            xa[q] = bf16lo_to_f32(pa);
            xa[q + 1] = bf16hi_to_f32(pa);
            xb[q] = bf16lo_to_f32(pb);
            xb[q + 1] = bf16hi_to_f32(pb);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xa[q] = x[q] + alpha;
            xb[q] = x[q] + (-alpha);
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const double ta = (double)xa[q], tb = (double)xb[q];
        const double sa = ta * ta, sb = tb * tb, ad = (double)av[q];
        if constexpr (kClean) acc[2 * kQuadProbes] = quad_term(acc[2 * kQuadProbes], av[q], (double)x[q]);
#pragma unroll
        for (uint32_t i = 0; i < kQuadProbes; ++i) {
            // all ones where the probe's bit is set: one bit-field extract, then bitwise
            // selects of the two squares (a compare and two conditional moves per square
            // otherwise)
            const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)w[i], sh + (uint32_t)q, 1u);
            acc[2 * i] = quad_term_sq(acc[2 * i], ad, select_f64(m, sa, sb));
            acc[2 * i + 1] = quad_term_sq(acc[2 * i + 1], ad, select_f64(m, sb, sa));
        }
    }
}

template <bool kBF16, bool kBits, bool kClean>
__global__ __launch_bounds__(256) void k_quad_probes_partial(
    const void *__restrict__ theta, const float *__restrict__ a, uint64_t n, uint64_t blk0,
    uint32_t step, uint32_t probe0, uint32_t nvalid, uint32_t k0, uint32_t k1, float alpha,
    const uint8_t *__restrict__ bits, uint64_t stride, double *__restrict__ part)
{
    __shared__ double red[4];
    __shared__ __attribute__((aligned(16))) uint32_t xch[4][16 * 4 * kQuadProbes];
    constexpr uint32_t kNAcc = 2 * kQuadProbes + kClean;   // slot 2 kQuadProbes: the clean loss
    double acc[kNAcc];
#pragma unroll
    for (uint32_t s = 0; s < kNAcc; ++s) acc[s] = 0.0;
    const uint64_t G = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t *wx = xch[threadIdx.x >> 6];
    const uint64_t nwaves = (uint64_t)gridDim.x * (blockDim.x / 64u);
    const uint64_t nchunks = n / kLossChunk;
    const uint32_t sh = 4u * (lane & 7u);            // the lane's nibble in its sign word
    const uint32_t wsel = (lane & 31u) >> 3;          // which word of the block
    for (uint64_t c = tid / 64u; c < nchunks; c += nwaves) {
        const uint64_t p0 = c * kLossChunk + 4u * lane;   // + 256 k
        const f32x4_t *ap = reinterpret_cast<const f32x4_t *>(a + p0);
        f32x4_t av[8];
        float xv[8][4];
        if constexpr (kBF16) {
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            const u32x2_t *tp =
                reinterpret_cast<const u32x2_t *>(static_cast<const uint16_t *>(theta) + p0);
            u32x2_t w[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) w[k] = __builtin_nontemporal_load(tp + 64 * k);
#pragma unroll
            for (int k = 0; k < 8; ++k) av[k] = __builtin_nontemporal_load(ap + 64 * k);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                xv[k][0] = bf16lo_to_f32(w[k][0]);
                xv[k][1] = bf16hi_to_f32(w[k][0]);
                xv[k][2] = bf16lo_to_f32(w[k][1]);
                xv[k][3] = bf16hi_to_f32(w[k][1]);
            }
        } else {
            const f32x4_t *tp = reinterpret_cast<const f32x4_t *>(static_cast<const float *>(theta) + p0);
            f32x4_t x[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = __builtin_nontemporal_load(tp + 64 * k);
#pragma unroll
            for (int k = 0; k < 8; ++k) av[k] = __builtin_nontemporal_load(ap + 64 * k);
#pragma unroll
            for (int k = 0; k < 8; ++k)
#pragma unroll
                for (int q = 0; q < 4; ++q) xv[k][q] = x[k][q];
        }
        {   // the chunk's 16 blocks x kQuadProbes probes of sign bits: one per lane
            const uint32_t b = lane & 15u, i = lane >> 4;
            const uint64_t blk = c * (kLossChunk / kBlockParams) + b;   // local block
            uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
            if (i < nvalid) {
                if constexpr (kBits) {
                    const u32x4_t r = *reinterpret_cast<const u32x4_t *>(bits + (uint64_t)i * stride + blk * 16u);
                    w0 = r[0]; w1 = r[1]; w2 = r[2]; w3 = r[3];
                } else {
                    const U32x4 r = probe_block_bits(blk0 + blk, probe0 + i, step, k0, k1);
                    w0 = r.x; w1 = r.y; w2 = r.z; w3 = r.w;
                }
            }
            wave_lds_sync();   // the previous chunk's reads precede these writes
            wx[(b * 4u + 0u) * kQuadProbes + i] = w0;
            wx[(b * 4u + 1u) * kQuadProbes + i] = w1;
            wx[(b * 4u + 2u) * kQuadProbes + i] = w2;
            wx[(b * 4u + 3u) * kQuadProbes + i] = w3;
            wave_lds_sync();
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t blk = 2u * (uint32_t)k + (lane >> 5);   // block of params 256k + 4l
            const u32x4_t wq = *reinterpret_cast<const u32x4_t *>(wx + (blk * 4u + wsel) * kQuadProbes);
            const uint32_t w[kQuadProbes] = {wq[0], wq[1], wq[2], wq[3]};
            const float x[4] = {xv[k][0], xv[k][1], xv[k][2], xv[k][3]};
            const float aa[4] = {av[k][0], av[k][1], av[k][2], av[k][3]};
            quad_terms4<kBF16, kClean>(acc, x, aa, w, sh, alpha);
        }
    }
    for (uint64_t j = nchunks * kLossChunk + tid; j < n; j += G) {   // ragged end
        const float xj = (float)theta1<kBF16>(theta, j);
        if constexpr (kClean) acc[2 * kQuadProbes] = quad_term(acc[2 * kQuadProbes], a[j], (double)xj);
#pragma unroll
        for (uint32_t i = 0; i < kQuadProbes; ++i) {
            uint32_t bit = 0;
            if (i < nvalid) {
                if constexpr (kBits) {
                    bit = (bits[(uint64_t)i * stride + (j >> 3)] >> (j & 7u)) & 1u;
                } else {
                    const U32x4 r = probe_block_bits(blk0 + j / kBlockParams, probe0 + i, step, k0, k1);
                    const uint32_t wsl = (uint32_t)(j >> 5) & 3u;
                    const uint32_t word = wsl == 0 ? r.x : wsl == 1 ? r.y : wsl == 2 ? r.z : r.w;
                    bit = (word >> (j & 31u)) & 1u;
                }
            }
            float xa, xb;
            if constexpr (kBF16) {
                const uint32_t pab = pack_bf16x2(xj + alpha, xj + (-alpha));
                xa = bf16lo_to_f32(pab);
                xb = bf16hi_to_f32(pab);
            } else {
                xa = xj + alpha;
                xb = xj + (-alpha);
            }
            acc[2 * i] = quad_term(acc[2 * i], a[j], (double)(bit ? xa : xb));
            acc[2 * i + 1] = quad_term(acc[2 * i + 1], a[j], (double)(bit ? xb : xa));
        }
    }
#pragma unroll
    for (uint32_t s = 0; s < kNAcc; ++s) {
        const double v = block_sum256(acc[s], red);
        if (threadIdx.x == 0) part[(uint64_t)s * kLossPartials + blockIdx.x] = v;
    }
}

// Slot s < nprobe_slots of the fused pass (probe s / 2, sign s % 2), and for one more
// workgroup the clean slot 2 kQuadProbes: the partials summed exactly as k_sum_partials
// sums them, into out_plus / out_minus / out_clean.
__global__ __launch_bounds__(256) void k_sum_partials_slots(const double *__restrict__ part,
                                                            uint32_t count, double scale,
                                                            double *__restrict__ out_plus,
                                                            double *__restrict__ out_minus,
                                                            uint32_t nprobe_slots,
                                                            double *__restrict__ out_clean)
{
    __shared__ double red[4];
    const uint32_t s = blockIdx.x < nprobe_slots ? blockIdx.x : 2 * kQuadProbes;
    part += (uint64_t)s * count;
    double acc = 0.0;
    for (uint32_t i = threadIdx.x; i < count; i += blockDim.x) acc += part[i];
    const double v = block_sum256(acc, red);
    if (threadIdx.x == 0) {
        double *out = blockIdx.x >= nprobe_slots ? out_clean : (s & 1u) ? out_minus + (s >> 1)
                                                                        : out_plus + (s >> 1);
        *out = scale * v;
    }
}

hipError_t launch_quad_loss_probes(const void *theta, bool bf16, const float *a, uint64_t offset,
                                   uint64_t n, Key key, uint32_t step, uint32_t probe0,
                                   uint32_t nprobes, float alpha, const uint8_t *bits,
                                   double *partials, double *out_plus, double *out_minus,
                                   double *out_clean, hipStream_t stream)
{
    const uint64_t stride = (n + kBlockParams - 1) / kBlockParams * 16u;
    if (nprobes == 0 && out_clean) return launch_quad_loss(theta, bf16, a, n, partials, out_clean, stream);
    for (uint32_t done = 0; done < nprobes; done += kQuadProbes) {
        const uint32_t nvalid = nprobes - done < kQuadProbes ? nprobes - done : kQuadProbes;
        const uint8_t *b = bits ? bits + (uint64_t)done * stride : nullptr;
        const bool clean = out_clean && done == 0;   // the first pass also sums the clean loss
#define ZO_QP(BF, BI, CL)                                                                     \
    hipLaunchKernelGGL((k_quad_probes_partial<BF, BI, CL>), dim3(kLossPartials), dim3(256), 0, \
                       stream, theta, a, n, offset / kBlockParams, step, probe0 + done, nvalid, \
                       key.k0, key.k1, alpha, b, stride, partials)
#define ZO_QP2(BF, BI) do { if (clean) ZO_QP(BF, BI, true); else ZO_QP(BF, BI, false); } while (0)
        if (bf16) {
            if (b) ZO_QP2(true, true); else ZO_QP2(true, false);
        } else {
            if (b) ZO_QP2(false, true); else ZO_QP2(false, false);
        }
#undef ZO_QP2
#undef ZO_QP
        hipLaunchKernelGGL(k_sum_partials_slots, dim3(2 * nvalid + (clean ? 1u : 0u)), dim3(256),
                           0, stream, partials, kLossPartials, 0.5, out_plus + done,
                           out_minus + done, 2 * nvalid, out_clean);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_quad_loss(const void *theta, bool bf16, const float *a, uint64_t n,
                            double *partials, double *out, hipStream_t stream)
{
    if (bf16)
        hipLaunchKernelGGL(k_quad_loss_partial<true>, dim3(kLossPartials), dim3(256), 0, stream,
                           theta, a, n, partials);
    else
        hipLaunchKernelGGL(k_quad_loss_partial<false>, dim3(kLossPartials), dim3(256), 0, stream,
                           theta, a, n, partials);
    hipLaunchKernelGGL(k_sum_partials, dim3(1), dim3(256), 0, stream, partials, kLossPartials,
                       0.5, out);
    return hipGetLastError();
}

// ---- low-rank-plus-diagonal quadratic: 1/2 sum a_j theta_j^2 + 1/2 ||U theta||^2 -------
// One pass over theta, a and the r rows of U (row-major [r][n], each row contiguous, so
// every load is coalesced) accumulates the diagonal term and the r dot products in fp64;
// per-workgroup partials [block][kLowRankMax + 1], then one workgroup reduces each
// component in a fixed tree and squares the dot products.  Deterministic.
template <bool kBF16>
__global__ __launch_bounds__(256) void k_lowrank_partial(const void *__restrict__ theta,
                                                         const float *__restrict__ a,
                                                         const float *__restrict__ U, uint32_t r,
                                                         uint64_t n, double *__restrict__ part)
{
    __shared__ double red[4];
    double acc[kLowRankMax + 1];
#pragma unroll
    for (uint32_t q = 0; q <= kLowRankMax; ++q) acc[q] = 0.0;
    const uint64_t G = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool vec = (n % 8) == 0;    // rows of U stay 16-byte aligned only then
    const uint64_t ngroups = vec ? n / 8 : 0;
    const f32x4_t *a4 = reinterpret_cast<const f32x4_t *>(a);
    for (uint64_t g = tid; g < ngroups; g += G) {
        double t[8];
        theta8<kBF16>(theta, g, t);
        const f32x4_t a0 = a4[2 * g], a1 = a4[2 * g + 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[0] += (double)a0[q] * t[q] * t[q];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[0] += (double)a1[q] * t[4 + q] * t[4 + q];
#pragma unroll
        for (uint32_t k = 0; k < kLowRankMax; ++k) {
            if (k < r) {
                const f32x4_t *u4 = reinterpret_cast<const f32x4_t *>(U + (uint64_t)k * n);
                const f32x4_t u0 = u4[2 * g], u1 = u4[2 * g + 1];
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[1 + k] += (double)u0[q] * t[q];
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[1 + k] += (double)u1[q] * t[4 + q];
            }
        }
    }
    for (uint64_t j = ngroups * 8 + tid; j < n; j += G) {
        const double t = theta1<kBF16>(theta, j);
        acc[0] += (double)a[j] * t * t;
#pragma unroll
        for (uint32_t k = 0; k < kLowRankMax; ++k)
            if (k < r) acc[1 + k] += (double)U[(uint64_t)k * n + j] * t;
    }
    for (uint32_t q = 0; q <= r; ++q) {
        const double s = block_sum256(acc[q], red);
        if (threadIdx.x == 0) part[(uint64_t)blockIdx.x * (kLowRankMax + 1) + q] = s;
    }
}

__global__ __launch_bounds__(256) void k_lowrank_final(const double *__restrict__ part,
                                                       uint32_t blocks, uint32_t r,
                                                       double *__restrict__ out)
{
    // thread t adds the partial rows of blocks t, t + 256, ... (all its loads independent),
    // a fixed butterfly adds each component over the wave's lanes, and the four waves' sums
    // meet in LDS after one barrier
    __shared__ double wsum[4][kLowRankMax + 1];
    __shared__ double comp[kLowRankMax + 1];
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    double acc[kLowRankMax + 1];
#pragma unroll
    for (uint32_t q = 0; q <= kLowRankMax; ++q) acc[q] = 0.0;
    for (uint32_t b = threadIdx.x; b < blocks; b += blockDim.x) {
        const double *row = part + (uint64_t)b * (kLowRankMax + 1);
#pragma unroll
        for (uint32_t q = 0; q <= kLowRankMax; ++q)
            if (q <= r) acc[q] += row[q];
    }
#pragma unroll
    for (uint32_t q = 0; q <= kLowRankMax; ++q) {
        if (q <= r) {
            double v = acc[q];
#pragma unroll
            for (int w = 32; w >= 1; w >>= 1) v += __shfl_xor(v, w, 64);
            if (lane == 0) wsum[wave][q] = v;
        }
    }
    __syncthreads();
    if (threadIdx.x <= r)
        comp[threadIdx.x] = (wsum[0][threadIdx.x] + wsum[1][threadIdx.x]) +
                            (wsum[2][threadIdx.x] + wsum[3][threadIdx.x]);
    __syncthreads();
    if (threadIdx.x == 0) {
        double sq = 0.0;
        for (uint32_t k = 1; k <= r; ++k) sq += comp[k] * comp[k];
        *out = 0.5 * (comp[0] + sq);
    }
}

hipError_t launch_lowrank_loss(const void *theta, bool bf16, const float *a, const float *U,
                               uint32_t r, uint64_t n, double *partials, double *out,
                               hipStream_t stream)
{
    if (bf16)
        hipLaunchKernelGGL(k_lowrank_partial<true>, dim3(kLossPartials), dim3(256), 0, stream,
                           theta, a, U, r, n, partials);
    else
        hipLaunchKernelGGL(k_lowrank_partial<false>, dim3(kLossPartials), dim3(256), 0, stream,
                           theta, a, U, r, n, partials);
    hipLaunchKernelGGL(k_lowrank_final, dim3(1), dim3(256), 0, stream, partials, kLossPartials, r,
                       out);
    return hipGetLastError();
}

}  // namespace zo

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
// Pass 1: kLossPartials workgroups; thread i of the grid takes the 8-element groups
// i, i + G, i + 2G, ... (16-byte loads of theta and a; G = total threads), then the ragged
// end one element at a time; each wave adds its lanes with a fixed butterfly and the
// workgroup adds its waves in order.  Pass 2: one workgroup adds the partials the same
// way.  The partition depends only on n, so the result is bit-reproducible.
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
    const uint64_t ngroups = n / 8;
    const f32x4_t *a4 = reinterpret_cast<const f32x4_t *>(a);
    for (uint64_t g = tid; g < ngroups; g += G) {
        double t[8];
        theta8<kBF16>(theta, g, t);
        const f32x4_t a0 = a4[2 * g], a1 = a4[2 * g + 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc += (double)a0[q] * t[q] * t[q];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc += (double)a1[q] * t[4 + q] * t[4 + q];
    }
    for (uint64_t j = ngroups * 8 + tid; j < n; j += G) {
        const double t = theta1<kBF16>(theta, j);
        acc += (double)a[j] * t * t;
    }
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
    __shared__ double red[4];
    __shared__ double comp[kLowRankMax + 1];
    for (uint32_t q = 0; q <= r; ++q) {
        double acc = 0.0;
        for (uint32_t b = threadIdx.x; b < blocks; b += blockDim.x)
            acc += part[(uint64_t)b * (kLowRankMax + 1) + q];
        const double s = block_sum256(acc, red);
        if (threadIdx.x == 0) comp[q] = s;
    }
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

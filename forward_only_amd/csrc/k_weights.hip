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
// Pass 1: kLossPartials workgroups, fixed grid-stride partition, fixed-order LDS tree;
// pass 2: one workgroup sums the partials in a fixed tree.  Bit-reproducible run to run.
template <int kThreads>
__device__ __forceinline__ double block_sum(double v, double *red)
{
    red[threadIdx.x] = v;
    __syncthreads();
#pragma unroll
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    return red[0];
}

template <bool kBF16>
__global__ __launch_bounds__(256) void k_quad_loss_partial(const void *__restrict__ theta,
                                                           const float *__restrict__ a,
                                                           uint64_t n, double *__restrict__ part)
{
    __shared__ double red[256];
    double acc = 0.0;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
        double t;
        if constexpr (kBF16)
            t = (double)__uint_as_float((uint32_t)static_cast<const uint16_t *>(theta)[j] << 16);
        else
            t = (double)static_cast<const float *>(theta)[j];
        acc += (double)a[j] * t * t;
    }
    const double s = block_sum<256>(acc, red);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_sum_partials(const double *__restrict__ part,
                                                      uint32_t count, double scale,
                                                      double *__restrict__ out)
{
    __shared__ double red[256];
    double acc = 0.0;
    for (uint32_t i = threadIdx.x; i < count; i += blockDim.x) acc += part[i];
    const double s = block_sum<256>(acc, red);
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

}  // namespace zo

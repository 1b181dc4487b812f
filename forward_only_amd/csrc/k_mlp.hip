// k_mlp.hip -- loss of a two-layer MLP classifier (the "forward passes, loss only" box of
// the ZOO loop flowchart in "Pretraining Transformers Without Backprop: What Two
// Zero-Order Papers Actually Measure"), used as the small real forward pass of the path:
//   H = GELU(X W1^T + b1),  logits = H W2^T + b2,  loss = mean_b (logsumexp - logit[label]).
// Flat parameters: W1 [d_hid x d_in] row-major, b1 [d_hid], W2 [d_out x d_hid], b2 [d_out].
//
// Kernel 1 (k_mlp_tiles): one wave per 16x16 tile of H, v_mfma_f32_16x16x4f32 over K =
//   d_in (fp32 in, fp32 accumulate).  Lane l holds A = X[m0 + l%16][k], B = W1[n0 + l%16][k]
//   for k = k0 + 4*(l/16) + t, t = 0..3 (one float4 load per operand per 16 k; the order
//   of k inside an MFMA is free as long as both operands agree).  The accumulator gives
//   lane l rows m0 + 4*(l/16) + r (r = 0..3) of column n0 + l%16.  Epilogue: + b1, exact
//   GELU (erf), times W2[o][n], summed over the tile's 16 columns with a fixed butterfly,
//   written as fp64 partial logits at [row][output][tile column block].
//   Workgroups are remapped so that the tiles run by one XCD (workgroup id mod 8) are a
//   contiguous range of column blocks: each XCD's L2 then holds 1/8 of W1 plus X.
// Kernel 2 (k_mlp_rows): one wave per row; lane l sums the partial logits of column
//   blocks l, l+64, ... (coalesced), a fixed butterfly adds the lanes, + b2, logsumexp in
//   fp64: the row's loss.  Kernel 3 (k_mlp_mean): the batch mean by a fixed tree.
// Deterministic for a given shape.
//
// Perturbation-fused variant (kPert): every parameter is read as the fp32 value
// theta_j + (bit ? alpha : -alpha) of probe `probe` at `step` -- the value an in-place
// zo_perturb would have stored -- so the loss at theta +/- eps*z_i needs no pass over theta.
// Paired variant (kPair): the losses at +alpha and -alpha in one launch sequence; each W1
// operand is loaded once and feeds two accumulators (the second sees theta_j + (bit ?
// -alpha : alpha)), each with exactly the MFMA sequence of a single fused launch, so both
// losses equal the single fused results bit for bit.  Sign s (0: +alpha, 1: -alpha) writes
// its partial logits, row losses and loss to its own slots.
#include <stdlib.h>

#include "zo_device.hpp"
#include "zo_launch.hpp"

namespace zo {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Sign source for the fused variant: Philox of (global block, probe, step) or a plane.
struct PertArgs {
    uint64_t offset;      // global index of params[0] (multiple of 128)
    uint32_t step, probe, k0, k1;
    float alpha;
    const uint8_t *bits;  // packed row over the params, or nullptr
};

// Sign bits of the 4 consecutive params j .. j+3 (j % 4 == 0) in the low 4 bits.
__device__ __forceinline__ uint32_t quad_bits(const PertArgs &p, uint64_t j)
{
    if (p.bits) {
        return (uint32_t)(p.bits[j >> 3] >> (j & 4)) & 0xFu;
    }
    const uint64_t g = p.offset + j;
    const U32x4 r = probe_block_bits(g >> 7, p.probe, p.step, p.k0, p.k1);
    const uint32_t sel = (uint32_t)(g >> 5) & 3u;
    const uint32_t word = sel == 0 ? r.x : sel == 1 ? r.y : sel == 2 ? r.z : r.w;
    return (word >> (g & 31)) & 0xFu;
}

__device__ __forceinline__ float with_sign(float v, uint32_t bit, float alpha)
{
    return v + (bit ? alpha : -alpha);
}

__device__ __forceinline__ float param(const float *params, uint64_t j, const PertArgs &p,
                                       bool pert)
{
    const float v = params[j];
    if (!pert) return v;
    const uint32_t b = quad_bits(p, j & ~(uint64_t)3) >> (j & 3);
    return with_sign(v, b & 1u, p.alpha);
}

__device__ __forceinline__ float gelu_exact(float x)
{
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

template <bool kPert, bool kPair>
__global__ __launch_bounds__(64) void k_mlp_tiles(const float *__restrict__ X,
                                                  const float *__restrict__ params,
                                                  uint32_t batch, uint32_t d_in, uint32_t d_hid,
                                                  uint32_t d_out, double *__restrict__ partial,
                                                  PertArgs pa)
{
    const uint32_t lane = threadIdx.x;
    const uint32_t m_tiles = batch / 16, n_tiles = d_hid / 16;
    const uint32_t total = m_tiles * n_tiles;
    uint32_t t = blockIdx.x;
    if ((total & 7u) == 0) t = (t & 7u) * (total >> 3) + (t >> 3);  // XCD-contiguous tiles
    const uint32_t m0 = (t % m_tiles) * 16, nt = t / m_tiles, n0 = nt * 16;
    const uint32_t li = lane & 15u, kq = lane >> 4;

    const float *xrow = X + (uint64_t)(m0 + li) * d_in + 4u * kq;
    const uint64_t wrow = (uint64_t)(n0 + li) * d_in + 4u * kq;   // flat index in params
    const float *wptr = params + wrow;

    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4_t acc2 = {0.0f, 0.0f, 0.0f, 0.0f};   // kPair: the -alpha accumulator
    uint64_t cached_blk = ~(uint64_t)0;
    U32x4 cw = {0u, 0u, 0u, 0u};

    // Sign bits of the 4 params j .. j+3 of W1 (j a multiple of 4) in the low 4 bits.
    auto bits4 = [&](uint64_t j) -> uint32_t {
        uint32_t q;
        if (pa.bits) {
            q = (uint32_t)(pa.bits[j >> 3] >> (j & 4)) & 0xFu;
        } else {
            const uint64_t g = pa.offset + j;
            if ((g >> 7) != cached_blk) {
                cached_blk = g >> 7;
                cw = probe_block_bits(cached_blk, pa.probe, pa.step, pa.k0, pa.k1);
            }
            const uint32_t sel = (uint32_t)(g >> 5) & 3u;
            const uint32_t word = sel == 0 ? cw.x : sel == 1 ? cw.y : sel == 2 ? cw.z : cw.w;
            q = (word >> (g & 31)) & 0xFu;
        }
        return q;
    };
    auto mfma4 = [](f32x4_t &c, const f32x4_t &a, const f32x4_t &b) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    };
    // One 16-k group: operand a of X, operand b of W1 at flat index j.
    auto group = [&](const f32x4_t &a, const f32x4_t &b, uint64_t j) {
        if constexpr (!kPert) {
            mfma4(acc, a, b);
        } else {
            const uint32_t q = bits4(j);
            f32x4_t bp;
#pragma unroll
            for (int t = 0; t < 4; ++t) bp[t] = with_sign(b[t], (q >> t) & 1u, pa.alpha);
            mfma4(acc, a, bp);
            if constexpr (kPair) {
                f32x4_t bm;
#pragma unroll
                for (int t = 0; t < 4; ++t) bm[t] = with_sign(b[t], (q >> t) & 1u, -pa.alpha);
                mfma4(acc2, a, bm);
            }
        }
    };

    // Stages of kStage K-groups (16 k each): the loads of stage s+1 are in flight while
    // stage s runs through the MFMAs, so memory latency is paid once per kernel rather
    // than once per 16 k.
    constexpr uint32_t kStage = 8;
    const uint32_t kfull = (d_in / (16u * kStage)) * (16u * kStage);
    f32x4_t a0[kStage], b0[kStage], a1[kStage], b1[kStage];
    auto load_stage = [&](f32x4_t (&a)[kStage], f32x4_t (&b)[kStage], uint32_t kb) {
#pragma unroll
        for (uint32_t g = 0; g < kStage; ++g) {
            a[g] = *reinterpret_cast<const f32x4_t *>(xrow + kb + 16u * g);
            b[g] = *reinterpret_cast<const f32x4_t *>(wptr + kb + 16u * g);
        }
    };
    auto run_stage = [&](f32x4_t (&a)[kStage], f32x4_t (&b)[kStage], uint32_t kb) {
#pragma unroll
        for (uint32_t g = 0; g < kStage; ++g) group(a[g], b[g], wrow + kb + 16u * g);
    };
    if (kfull > 0) {
        load_stage(a0, b0, 0);
        uint32_t kb = 0;
        for (;;) {
            const uint32_t next = kb + 16u * kStage;
            if (next < kfull) load_stage(a1, b1, next);
            run_stage(a0, b0, kb);
            if (next >= kfull) break;
            kb = next;
            const uint32_t next2 = kb + 16u * kStage;
            if (next2 < kfull) load_stage(a0, b0, next2);
            run_stage(a1, b1, kb);
            if (next2 >= kfull) break;
            kb = next2;
        }
    }
    for (uint32_t k0 = kfull; k0 < d_in; k0 += 16) {      // K not a multiple of 128
        const f32x4_t a = *reinterpret_cast<const f32x4_t *>(xrow + k0);
        const f32x4_t b = *reinterpret_cast<const f32x4_t *>(wptr + k0);
        group(a, b, wrow + k0);
    }

    // epilogue: column n = n0 + li, rows m0 + 4*kq + r
    const uint64_t b1_at = (uint64_t)d_hid * d_in;
    const uint64_t w2_at = b1_at + d_hid;
    const uint64_t pset = (uint64_t)n_tiles * batch * d_out;   // one sign's partial logits
    const uint32_t n = n0 + li;
#pragma unroll
    for (int sgn = 0; sgn < (kPair ? 2 : 1); ++sgn) {
        PertArgs ps = pa;
        if (sgn) ps.alpha = -pa.alpha;
        const f32x4_t &c = sgn ? acc2 : acc;
        double *out = partial + (uint64_t)sgn * pset;
        const float bias = param(params, b1_at + n, ps, kPert);
        float g[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) g[r] = gelu_exact(c[r] + bias);
        for (uint32_t o = 0; o < d_out; ++o) {
            const float w2 = param(params, w2_at + (uint64_t)o * d_hid + n, ps, kPert);
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = g[r] * w2;
            // sum over the 16 columns of the tile (lanes with equal kq), fixed butterfly
#pragma unroll
            for (int s = 8; s >= 1; s >>= 1) {
#pragma unroll
                for (int r = 0; r < 4; ++r) p[r] = p[r] + __shfl_xor(p[r], s, 16);
            }
            if (li == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    out[((uint64_t)(m0 + 4u * kq + (uint32_t)r) * d_out + o) * n_tiles + nt] = (double)p[r];
            }
        }
    }
}

template <bool kPert>
__global__ __launch_bounds__(256) void k_mlp_rows(const double *__restrict__ partial,
                                                  const float *__restrict__ params,
                                                  const int64_t *__restrict__ labels,
                                                  uint32_t batch, uint32_t d_in, uint32_t d_hid,
                                                  uint32_t d_out, double *__restrict__ rowloss,
                                                  PertArgs pa)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t m = blockIdx.x * 4u + (threadIdx.x >> 6);
    if (m >= batch) return;
    const uint32_t n_tiles = d_hid / 16;
    // sign slot blockIdx.y (paired launch: 1 is the -alpha loss)
    if (blockIdx.y) pa.alpha = -pa.alpha;
    partial += (uint64_t)blockIdx.y * n_tiles * batch * d_out;
    rowloss += (uint64_t)blockIdx.y * batch;
    const uint64_t b2_at = (uint64_t)d_hid * d_in + d_hid + (uint64_t)d_out * d_hid;
    double z[16];
    double zmax = -__builtin_inf();
    for (uint32_t o = 0; o < d_out; ++o) {
        const double *row = partial + ((uint64_t)m * d_out + o) * n_tiles;
        double s = 0.0;
        for (uint32_t t = lane; t < n_tiles; t += 64) s += row[t];
#pragma unroll
        for (int w = 32; w >= 1; w >>= 1) s += __shfl_xor(s, w, 64);
        s += (double)param(params, b2_at + o, pa, kPert);
        z[o] = s;
        zmax = s > zmax ? s : zmax;
    }
    if (lane == 0) {
        double se = 0.0;
        for (uint32_t o = 0; o < d_out; ++o) se += exp(z[o] - zmax);
        const int64_t lab = labels[m];
        const double zl = (lab >= 0 && lab < (int64_t)d_out) ? z[lab] : __builtin_nan("");
        rowloss[m] = (zmax + log(se)) - zl;
    }
}

__global__ __launch_bounds__(256) void k_mlp_mean(const double *__restrict__ rowloss,
                                                  uint32_t batch, double *__restrict__ out,
                                                  double *__restrict__ out2)
{
    __shared__ double red[256];
    // sign slot blockIdx.x (paired launch: 1 is the -alpha loss, written to out2)
    rowloss += (uint64_t)blockIdx.x * batch;
    if (blockIdx.x) out = out2;
    double acc = 0.0;
    for (uint32_t m = threadIdx.x; m < batch; m += blockDim.x) acc += rowloss[m];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = red[0] / (double)batch;
}

template <bool kPert, bool kPair>
static void launch_chain(const float *params, const float *X, const int64_t *labels,
                         uint32_t batch, uint32_t d_in, uint32_t d_hid, uint32_t d_out,
                         double *partial, double *out, double *out2, const PertArgs &pa,
                         hipStream_t stream)
{
    const uint32_t tiles = (batch / 16) * (d_hid / 16);
    const uint32_t nsign = kPair ? 2u : 1u;
    double *rowloss = partial + (uint64_t)nsign * (d_hid / 16) * batch * d_out;
    hipLaunchKernelGGL((k_mlp_tiles<kPert, kPair>), dim3(tiles), dim3(64), 0, stream, X, params,
                       batch, d_in, d_hid, d_out, partial, pa);
    hipLaunchKernelGGL(k_mlp_rows<kPert>, dim3((batch + 3) / 4, nsign), dim3(256), 0, stream,
                       partial, params, labels, batch, d_in, d_hid, d_out, rowloss, pa);
    hipLaunchKernelGGL(k_mlp_mean, dim3(nsign), dim3(256), 0, stream, rowloss, batch, out, out2);
}

hipError_t launch_mlp_loss(const float *params, const float *X, const int64_t *labels,
                           uint32_t batch, uint32_t d_in, uint32_t d_hid, uint32_t d_out,
                           double *partial, double *out, const MlpPerturb *pert, Key key,
                           hipStream_t stream, double *out_minus)
{
    PertArgs pa{0, 0, 0, key.k0, key.k1, 0.0f, nullptr};
    if (pert) {
        pa.offset = pert->offset;
        pa.step = pert->step;
        pa.probe = pert->probe;
        pa.alpha = pert->alpha;
        pa.bits = pert->bits;
        if (out_minus)
            launch_chain<true, true>(params, X, labels, batch, d_in, d_hid, d_out, partial, out,
                                     out_minus, pa, stream);
        else
            launch_chain<true, false>(params, X, labels, batch, d_in, d_hid, d_out, partial, out,
                                      nullptr, pa, stream);
    } else {
        launch_chain<false, false>(params, X, labels, batch, d_in, d_hid, d_out, partial, out,
                                   nullptr, pa, stream);
    }
    return hipGetLastError();
}

}  // namespace zo

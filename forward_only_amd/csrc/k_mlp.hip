// k_mlp.hip -- loss of a two-layer MLP classifier (the "forward passes, loss only" box of
// the ZOO loop flowchart in "Pretraining Transformers Without Backprop: What Two
// Zero-Order Papers Actually Measure"), used as the small real forward pass of the path:
//   H = GELU(X W1^T + b1),  logits = H W2^T + b2,  loss = mean_b (logsumexp - logit[label]).
// Flat parameters: W1 [d_hid x d_in] row-major, b1 [d_hid], W2 [d_out x d_hid], b2 [d_out].
//
// Kernel 1 (k_mlp_tiles): one wave per kT x kT tile of H (kT = 32 with v_mfma_f32_32x32x2f32
//   where the batch and d_hid allow, else 16 with v_mfma_f32_16x16x4f32) over K = d_in (fp32
//   in, fp32 accumulate).  Lane l holds A = X[m0 + l%kT][k], B = W1[n0 + l%kT][k] for
//   k = k0 + (kT/4)*(l/kT) + e, e < kT/4 (one or two float4 loads per operand per 16 k;
//   the order of k inside an MFMA is free as long as both operands agree).  The
//   accumulator gives lane l rows of column n0 + l%kT.  Epilogue: + b1, exact GELU (erf),
//   times W2[o][n], summed over the tile's kT columns with a fixed reduce-scatter tree,
//   written as fp64 partial logits at [row][output][tile column block].  The 32-wide form
//   does twice the MFMA work per operand element a lane loads and perturbs.
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
// losses equal the single fused results bit for bit.
// Several probes (kNP > 1): each wave runs kNP probes, both signs each, so every X and W1
// operand it loads feeds 2*kNP accumulators, while each accumulator still runs exactly the
// single fused launch's MFMA sequence.  A launch covers kNP * gridDim.y probes: blockIdx.y
// picks the wave's group of kNP probes, so the tiles' waves come gridDim.y times over and
// each SIMD gets several to interleave (one 8-probe wave per tile left 1.5 waves per SIMD,
// which serialised every wave's sign arithmetic with its own MFMAs).  Slot s = 2i + sign
// (probe i of the launch; sign 0: +alpha, 1: -alpha) writes its partial logits, row losses
// and loss to its own places.  With a clean loss requested, one more group of waves
// (blockIdx.y == gridDim.y - 1) computes the unperturbed loss into the slot after the
// probes' -- the same tile code as the clean launch, staged like the probe waves (the
// staging depth does not change the k order), so its result equals the clean launch's.
#include <stdlib.h>

#include "zo_device.hpp"
#include "zo_launch.hpp"

namespace zo {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Sign source for the fused variant: Philox of (global block, probe, step) or stored rows.
struct PertArgs {
    uint64_t offset;      // global index of params[0] (multiple of 128)
    uint32_t step, probe, k0, k1;   // probe: the launch's first probe
    float alpha;
    const uint8_t *bits;  // packed rows over the params (row i: probe + i), or nullptr
    uint64_t bits_stride; // bytes per row
};

// Sign bits of the 4 consecutive params j .. j+3 (j % 4 == 0) of probe p.probe + i in the
// low 4 bits.
__device__ __forceinline__ uint32_t quad_bits(const PertArgs &p, uint32_t i, uint64_t j)
{
    if (p.bits) {
        return (uint32_t)(p.bits[(uint64_t)i * p.bits_stride + (j >> 3)] >> (j & 4)) & 0xFu;
    }
    const uint64_t g = p.offset + j;
    const U32x4 r = probe_block_bits(g >> 7, p.probe + i, p.step, p.k0, p.k1);
    const uint32_t sel = (uint32_t)(g >> 5) & 3u;
    const uint32_t word = sel == 0 ? r.x : sel == 1 ? r.y : sel == 2 ? r.z : r.w;
    return (word >> (g & 31)) & 0xFu;
}

__device__ __forceinline__ float with_sign(float v, uint32_t bit, float alpha)
{
    return v + (bit ? alpha : -alpha);
}

// The sign bit of parameter j under probe p.probe + i.
__device__ __forceinline__ uint32_t param_bit(const PertArgs &p, uint32_t i, uint64_t j)
{
    return (quad_bits(p, i, j & ~(uint64_t)3) >> (j & 3)) & 1u;
}

// Parameter j as the forward of probe p.probe + i with step `alpha` reads it.
__device__ __forceinline__ float param(const float *params, uint64_t j, const PertArgs &p,
                                       uint32_t i, float alpha, bool pert)
{
    const float v = params[j];
    return pert ? with_sign(v, param_bit(p, i, j), alpha) : v;
}

__device__ __forceinline__ float gelu_exact(float x)
{
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

// Tile shapes: one wave computes a kT x kT tile of H with v_mfma_f32_16x16x4f32 (kT = 16) or
// v_mfma_f32_32x32x2f32 (kT = 32).  Per 16-k group lane l loads kT/4 consecutive k of its X
// row and its W1 row (k = k0 + (kT/4)*(l/kT) + e), and MFMA e takes element e from every
// lane, so each k of the group enters exactly one MFMA.  The accumulator gives lane l the
// kT*kT/64 entries D[8*(r/4) + 4*(l/kT) + r%4][l%kT], r = 0 .. kT*kT/64 - 1 (for kT = 16
// that is rows 4*(l/16) + r).
template <int kT> struct TileAcc;
template <> struct TileAcc<16> { typedef f32x4_t type; };
template <> struct TileAcc<32> { typedef f32x16_t type; };

// Sum of v[.] over the kT lanes of a column group (equal lane / kT) by a fixed tree that
// scatters the rows while it adds: each halving stage passes the half of the values this
// lane does not keep to its partner at lane distance s and adds the partner's copy of the
// half it keeps; once one value is left the remaining stages add whole.  Lanes with
// li % (kT / kOut) == 0 end with row index li / (kT / kOut) in v[0].
template <int kT, int kOut, int kS = kT / 2, int kCnt = kOut>
__device__ __forceinline__ void sum_columns(float (&v)[kOut], uint32_t li)
{
    if constexpr (kS >= 1) {
        if constexpr (kCnt > 1) {
            constexpr int h = kCnt / 2;
            const bool up = (li & (uint32_t)kS) != 0;
#pragma unroll
            for (int r = 0; r < h; ++r) {
                const float send = up ? v[r] : v[r + h];
                const float keep = up ? v[r + h] : v[r];
                v[r] = keep + __shfl_xor(send, kS, kT);
            }
            sum_columns<kT, kOut, kS / 2, h>(v, li);
        } else {
            v[0] = v[0] + __shfl_xor(v[0], kS, kT);
            sum_columns<kT, kOut, kS / 2, 1>(v, li);
        }
    }
}

// K-groups per staging step of a wave with kNP probes (see tile_body).
template <int kT, int kNP>
constexpr uint32_t stage_groups()
{
    constexpr uint32_t s16 = kNP >= 8 ? 2 : kNP >= 2 ? 4 : 8;
    return kT == 16 ? s16 : s16 / 2;
}

// One wave's tile.  kNP: probes of the wave (0: the clean loss, no perturbation); kPair:
// both signs per probe; kStage: K-groups per staging step.  kNS accumulator slots, slot s =
// probe s / kPer, sign s % kPer, written from `partial` on (one slot of partial logits
// apart).
template <int kT, int kNP, bool kPair, uint32_t kStage>
__device__ __forceinline__ void tile_body(const float *__restrict__ X,
                                          const float *__restrict__ params, uint32_t batch,
                                          uint32_t d_in, uint32_t d_hid, uint32_t d_out,
                                          double *__restrict__ partial, PertArgs pa)
{
    constexpr int kE = kT / 4;          // k values per lane and 16-k group
    constexpr int kV = kE / 4;          // float4 loads per operand and group
    constexpr int kOut = kT * kT / 64;  // accumulator entries per lane
    typedef typename TileAcc<kT>::type acc_t;
    struct Op { f32x4_t v[kV]; };

    const uint32_t lane = threadIdx.x;
    const uint32_t m_tiles = batch / kT, n_tiles = d_hid / kT;
    const uint32_t total = m_tiles * n_tiles;
    uint32_t t = blockIdx.x;
    if ((total & 7u) == 0) t = (t & 7u) * (total >> 3) + (t >> 3);  // XCD-contiguous tiles
    const uint32_t m0 = (t % m_tiles) * kT, nt = t / m_tiles, n0 = nt * kT;
    const uint32_t li = lane % kT, kq = lane / kT;

    const float *xrow = X + (uint64_t)(m0 + li) * d_in + (uint32_t)kE * kq;
    const uint64_t wrow = (uint64_t)(n0 + li) * d_in + (uint32_t)kE * kq;   // flat index in params
    const float *wptr = params + wrow;

    constexpr bool kPert = kNP > 0;
    constexpr int kPer = kPair ? 2 : 1;
    constexpr int kNS = kPert ? kNP * kPer : 1;
    constexpr int kNB = kPert ? kNP : 1;
    acc_t acc[kNS];
#pragma unroll
    for (int s = 0; s < kNS; ++s) acc[s] = acc_t{};
    uint64_t cached_blk = ~(uint64_t)0;
    // the four Philox words of the cached block, one array per word (an array of 4-word
    // structs picked by a run-time word index ends up in scratch memory)
    uint32_t cwx[kNB], cwy[kNB], cwz[kNB], cww[kNB];
#pragma unroll
    for (int i = 0; i < kNB; ++i) cwx[i] = cwy[i] = cwz[i] = cww[i] = 0u;

    // Sign bits of the kE params j .. j+kE-1 of W1 (j a multiple of kE) of each probe of
    // the launch, in the low kE bits of q[i].  The probes share the parameters, so one
    // block change refreshes all their Philox words.
    constexpr uint32_t kMask = (1u << kE) - 1u;
    auto bits_of = [&](uint64_t j, uint32_t (&q)[kNB]) {
        if (pa.bits) {
#pragma unroll
            for (int i = 0; i < kNB; ++i) {
                const uint32_t byte = pa.bits[(uint64_t)i * pa.bits_stride + (j >> 3)];
                q[i] = kE == 8 ? byte : (byte >> (j & 4)) & kMask;
            }
            return;
        }
        const uint64_t g = pa.offset + j;
        if ((g >> 7) != cached_blk) {
            cached_blk = g >> 7;
#pragma unroll
            for (int i = 0; i < kNB; ++i) {
                const U32x4 w = probe_block_bits(cached_blk, pa.probe + (uint32_t)i, pa.step,
                                                 pa.k0, pa.k1);
                cwx[i] = w.x;
                cwy[i] = w.y;
                cwz[i] = w.z;
                cww[i] = w.w;
            }
        }
        const bool odd = (g >> 5) & 1u, high = (g >> 6) & 1u;   // word (g >> 5) & 3
#pragma unroll
        for (int i = 0; i < kNB; ++i) {
            const uint32_t lo = odd ? cwy[i] : cwx[i];
            const uint32_t hi = odd ? cww[i] : cwz[i];
            q[i] = ((high ? hi : lo) >> (g & 31)) & kMask;
        }
    };
    auto mfma_group = [](acc_t &c, const Op &a, const Op &b) {
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            if constexpr (kT == 16)
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e / 4][e % 4], b.v[e / 4][e % 4],
                                                         c, 0, 0, 0);
            else
                c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[e / 4][e % 4], b.v[e / 4][e % 4],
                                                         c, 0, 0, 0);
        }
    };
    // One 16-k group: operand a of X, operand b of W1 at flat index j.
    auto group = [&](const Op &a, const Op &b, uint64_t j) {
        if constexpr (!kPert) {
            mfma_group(acc[0], a, b);
        } else {
            uint32_t q[kNB];
            bits_of(j, q);
            const uint32_t abits = __builtin_bit_cast(uint32_t, pa.alpha);
#pragma unroll
            for (int i = 0; i < kNP; ++i) {
                // d = +alpha where the bit is set, -alpha where clear (alpha's sign bit
                // flipped): w + d is with_sign(w, bit, alpha), w + (-d) the -alpha value
                const uint32_t nq = ~q[i];
                float d[kE];
                Op bp;
#pragma unroll
                for (int e = 0; e < kE; ++e) {
                    d[e] = signed_alpha(nq, e, abits);
                    bp.v[e / 4][e % 4] = b.v[e / 4][e % 4] + d[e];
                }
                mfma_group(acc[kPer * i], a, bp);
                if constexpr (kPair) {
                    Op bm;
#pragma unroll
                    for (int e = 0; e < kE; ++e) bm.v[e / 4][e % 4] = b.v[e / 4][e % 4] + (-d[e]);
                    mfma_group(acc[kPer * i + 1], a, bm);
                }
            }
        }
    };

    // Stages of kStage K-groups (16 k each): the loads of stage s+1 are in flight while
    // stage s runs through the MFMAs, so memory latency is paid once per kernel rather
    // than once per 16 k.  With several probes each stage carries 2*kNP times the MFMA work,
    // and wide tiles load twice the operands per group, so shorter stages suffice (and keep
    // the registers from spilling).  The k order, and with it every accumulator's sequence,
    // does not depend on the staging.
    const uint32_t kfull = (d_in / (16u * kStage)) * (16u * kStage);
    Op a0[kStage], b0[kStage], a1[kStage], b1[kStage];
    auto load_op = [](Op &o, const float *p) {
#pragma unroll
        for (int v = 0; v < kV; ++v) o.v[v] = *reinterpret_cast<const f32x4_t *>(p + 4 * v);
    };
    auto load_stage = [&](Op (&a)[kStage], Op (&b)[kStage], uint32_t kb) {
#pragma unroll
        for (uint32_t g = 0; g < kStage; ++g) {
            load_op(a[g], xrow + kb + 16u * g);
            load_op(b[g], wptr + kb + 16u * g);
        }
    };
    auto run_stage = [&](Op (&a)[kStage], Op (&b)[kStage], uint32_t kb) {
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
    for (uint32_t k0 = kfull; k0 < d_in; k0 += 16) {      // K not a multiple of the stage
        Op a, b;
        load_op(a, xrow + k0);
        load_op(b, wptr + k0);
        group(a, b, wrow + k0);
    }

    // epilogue: column n = n0 + li; the row of entry r is m0 + 8*(r/4) + 4*kq + r%4
    const uint64_t b1_at = (uint64_t)d_hid * d_in;
    const uint64_t w2_at = b1_at + d_hid;
    const uint64_t pset = (uint64_t)n_tiles * batch * d_out;   // one slot's partial logits
    const uint32_t n = n0 + li;
    const float b1v = params[b1_at + n];
    // after sum_columns: the lanes that write, and the row each holds
    constexpr uint32_t kRep = (uint32_t)(kT / kOut);
    const uint32_t ridx = li / kRep;
    const uint32_t row = m0 + 8u * (ridx / 4u) + 4u * kq + ridx % 4u;
    uint32_t sb1[kNB], sw2[kNB];   // per probe: the sign bits of b1[n] and of W2[.][n]
#pragma unroll
    for (int slot = 0; slot < kNS; ++slot) {
        const uint32_t pi = (uint32_t)(slot / kPer);
        const float alpha = (slot % kPer) ? -pa.alpha : pa.alpha;
        const acc_t &c = acc[slot];
        double *out = partial + (uint64_t)slot * pset;
        // the sign bits of b1[n] and of W2[o][n] (bit o), once per probe for both signs
        uint32_t b1bit = 0, w2bits = 0;
        if constexpr (kPert) {
            if (slot % kPer == 0) {
                b1bit = param_bit(pa, pi, b1_at + n);
                for (uint32_t o = 0; o < d_out; ++o)
                    w2bits |= param_bit(pa, pi, w2_at + (uint64_t)o * d_hid + n) << o;
                sb1[pi] = b1bit;
                sw2[pi] = w2bits;
            } else {
                b1bit = sb1[pi];
                w2bits = sw2[pi];
            }
        }
        const float bias = kPert ? with_sign(b1v, b1bit, alpha) : b1v;
        float g[kOut];
#pragma unroll
        for (int r = 0; r < kOut; ++r) g[r] = gelu_exact(c[r] + bias);
        for (uint32_t o = 0; o < d_out; ++o) {
            const float w2v = params[w2_at + (uint64_t)o * d_hid + n];
            const float w2 = kPert ? with_sign(w2v, (w2bits >> o) & 1u, alpha) : w2v;
            float p[kOut];
#pragma unroll
            for (int r = 0; r < kOut; ++r) p[r] = g[r] * w2;
            sum_columns<kT, kOut>(p, li);      // over the tile's kT columns
            if (li % kRep == 0)
                out[((uint64_t)row * d_out + o) * n_tiles + nt] = (double)p[0];
        }
    }
}

// Tiles of kNP probes per wave (gridDim.y groups of them: group y takes probes pa.probe +
// y kNP onwards and slots y kNS onwards); the workgroups with blockIdx.y == clean_group
// compute the clean loss into the slot after the probes' (kNP = 0: every wave does).
template <int kT, int kNP, bool kPair>
__global__ __launch_bounds__(64) void k_mlp_tiles(const float *__restrict__ X,
                                                  const float *__restrict__ params,
                                                  uint32_t batch, uint32_t d_in, uint32_t d_hid,
                                                  uint32_t d_out, double *__restrict__ partial,
                                                  PertArgs pa, uint32_t clean_group)
{
    if constexpr (kNP > 0) {
        constexpr uint32_t kNS = (uint32_t)kNP * (kPair ? 2u : 1u);
        const uint64_t pset = (uint64_t)(d_hid / kT) * batch * d_out;
        if (blockIdx.y == clean_group) {   // staged like the probes' waves: same registers
            tile_body<kT, 0, false, stage_groups<kT, kNP>()>(
                X, params, batch, d_in, d_hid, d_out,
                partial + (uint64_t)clean_group * kNS * pset, pa);
            return;
        }
        pa.probe += blockIdx.y * (uint32_t)kNP;
        if (pa.bits) pa.bits += (uint64_t)blockIdx.y * kNP * pa.bits_stride;
        tile_body<kT, kNP, kPair, stage_groups<kT, kNP>()>(
            X, params, batch, d_in, d_hid, d_out, partial + (uint64_t)blockIdx.y * kNS * pset,
            pa);
    } else {
        tile_body<kT, 0, false, stage_groups<kT, 0>()>(X, params, batch, d_in, d_hid, d_out,
                                                        partial, pa);
    }
}

template <bool kPert>
__global__ __launch_bounds__(256) void k_mlp_rows(const double *__restrict__ partial,
                                                  const float *__restrict__ params,
                                                  const int64_t *__restrict__ labels,
                                                  uint32_t batch, uint32_t d_in, uint32_t d_hid,
                                                  uint32_t d_out, uint32_t n_tiles,
                                                  double *__restrict__ rowloss, PertArgs pa,
                                                  uint32_t per, uint32_t nprobe_slots)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t m = blockIdx.x * 4u + (threadIdx.x >> 6);
    if (m >= batch) return;
    // slot blockIdx.y: probe pa.probe + blockIdx.y / per, -alpha for the odd slots of pairs;
    // the slot after the probes' (if any) is the clean loss
    const bool pert = kPert && blockIdx.y < nprobe_slots;
    const uint32_t pi = blockIdx.y / per;
    const float alpha = (blockIdx.y % per) ? -pa.alpha : pa.alpha;
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
        s += (double)param(params, b2_at + o, pa, pi, alpha, pert);
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
                                                  double *__restrict__ out2, uint32_t per,
                                                  uint32_t nprobe_slots,
                                                  double *__restrict__ out_clean)
{
    __shared__ double red[256];
    // slot blockIdx.x: probe blockIdx.x / per; the -alpha slot of a pair writes to out2; the
    // slot after the probes' writes out_clean
    rowloss += (uint64_t)blockIdx.x * batch;
    out = blockIdx.x >= nprobe_slots ? out_clean
                                     : ((blockIdx.x % per) ? out2 : out) + blockIdx.x / per;
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

// One launch sequence: tiles (kNP probes per wave, `groups` probe groups, and with
// out_clean one more group for the clean loss), row losses, means.
template <int kT, int kNP, bool kPair>
static void launch_chain(const float *params, const float *X, const int64_t *labels,
                         uint32_t batch, uint32_t d_in, uint32_t d_hid, uint32_t d_out,
                         double *partial, double *out, double *out2, const PertArgs &pa,
                         hipStream_t stream, uint32_t groups = 1, double *out_clean = nullptr)
{
    const uint32_t n_tiles = d_hid / kT;
    const uint32_t tiles = (batch / kT) * n_tiles;
    const uint32_t per = kPair ? 2u : 1u;
    const uint32_t nslot = kNP > 0 ? (uint32_t)kNP * per * groups : 1u;   // probe slots
    const uint32_t clean = (kNP > 0 && out_clean) ? 1u : 0u;
    double *rowloss = partial + (uint64_t)(nslot + clean) * n_tiles * batch * d_out;
    hipLaunchKernelGGL((k_mlp_tiles<kT, kNP, kPair>), dim3(tiles, groups + clean), dim3(64), 0,
                       stream, X, params, batch, d_in, d_hid, d_out, partial, pa,
                       clean ? groups : 0xFFFFFFFFu);
    hipLaunchKernelGGL(k_mlp_rows<(kNP > 0)>, dim3((batch + 3) / 4, nslot + clean), dim3(256), 0,
                       stream, partial, params, labels, batch, d_in, d_hid, d_out, n_tiles,
                       rowloss, pa, per, nslot);
    hipLaunchKernelGGL(k_mlp_mean, dim3(nslot + clean), dim3(256), 0, stream, rowloss, batch, out,
                       out2, per, nslot, out_clean);
}

// Every launch for one shape uses the same tile kernel, so the k order of each hidden unit's
// accumulation, and with it every loss, is the same in all the MLP entry points: 32 x 32
// tiles where the batch and the hidden width allow (half the operand arithmetic and loads
// per MFMA flop of the 16 x 16 form), 16 x 16 tiles otherwise.
static bool wide_tiles(uint32_t batch, uint32_t d_hid)
{
    return batch % 32u == 0 && d_hid % 32u == 0;
}

static PertArgs pert_args(const MlpPerturb *pert, Key key, uint64_t nparams)
{
    PertArgs pa{0, 0, 0, key.k0, key.k1, 0.0f, nullptr, 0};
    if (pert) {
        pa.offset = pert->offset;
        pa.step = pert->step;
        pa.probe = pert->probe;
        pa.alpha = pert->alpha;
        pa.bits = pert->bits;
        pa.bits_stride = (nparams + 127) / 128 * 16;
    }
    return pa;
}

static uint64_t mlp_params(uint32_t d_in, uint32_t d_hid, uint32_t d_out)
{
    return (uint64_t)d_hid * d_in + d_hid + (uint64_t)d_out * d_hid + d_out;
}

template <int kT>
static void launch_mlp_loss_t(const float *params, const float *X, const int64_t *labels,
                              uint32_t batch, uint32_t d_in, uint32_t d_hid, uint32_t d_out,
                              double *partial, double *out, const PertArgs &pa, bool pert,
                              hipStream_t stream, double *out_minus)
{
    if (pert) {
        if (out_minus)
            launch_chain<kT, 1, true>(params, X, labels, batch, d_in, d_hid, d_out, partial,
                                      out, out_minus, pa, stream);
        else
            launch_chain<kT, 1, false>(params, X, labels, batch, d_in, d_hid, d_out, partial,
                                       out, nullptr, pa, stream);
    } else {
        launch_chain<kT, 0, false>(params, X, labels, batch, d_in, d_hid, d_out, partial, out,
                                   nullptr, pa, stream);
    }
}

hipError_t launch_mlp_loss(const float *params, const float *X, const int64_t *labels,
                           uint32_t batch, uint32_t d_in, uint32_t d_hid, uint32_t d_out,
                           double *partial, double *out, const MlpPerturb *pert, Key key,
                           hipStream_t stream, double *out_minus)
{
    const PertArgs pa = pert_args(pert, key, mlp_params(d_in, d_hid, d_out));
    if (wide_tiles(batch, d_hid))
        launch_mlp_loss_t<32>(params, X, labels, batch, d_in, d_hid, d_out, partial, out, pa,
                              pert != nullptr, stream, out_minus);
    else
        launch_mlp_loss_t<16>(params, X, labels, batch, d_in, d_hid, d_out, partial, out, pa,
                              pert != nullptr, stream, out_minus);
    return hipGetLastError();
}

// Probes per wave of the batched MLP forward, from the environment (read once per process):
// 1, 2, 4 or 8; anything else keeps the default.  Results do not depend on it.
static uint32_t mlp_probes_per_wave()
{
    static const uint32_t v = [] {
        const char *s = getenv("ZO_MLP_PROBES_PER_WAVE");
        const int x = (s && *s) ? atoi(s) : 0;
        return (x == 1 || x == 2 || x == 4 || x == 8) ? (uint32_t)x : kMlpProbesPerWave;
    }();
    return v;
}

hipError_t launch_mlp_loss_probes(const float *params, const float *X, const int64_t *labels,
                                  uint32_t batch, uint32_t d_in, uint32_t d_hid, uint32_t d_out,
                                  double *partial, const MlpPerturb &pert, uint32_t nprobes,
                                  Key key, double *out_plus, double *out_minus,
                                  double *out_clean, hipStream_t stream)
{
    const uint64_t nparams = mlp_params(d_in, d_hid, d_out);
    const uint32_t pw = mlp_probes_per_wave();
    if (nprobes == 0 && out_clean)
        return launch_mlp_loss(params, X, labels, batch, d_in, d_hid, d_out, partial, out_clean,
                               nullptr, key, stream);
    // launch sequences of 64 probes, then 32, 16, ..., 1 for the rest, each with min(pw, size)
    // probes per wave; each reuses the workspace from its start (they run in stream order)
    for (uint32_t done = 0; done < nprobes;) {
        const uint32_t left = nprobes - done;
        uint32_t k = kMlpProbesPerLaunch;
        while (k > left) k >>= 1;
        const uint32_t w = pw < k ? pw : k;
        MlpPerturb p = pert;
        p.probe = pert.probe + done;
        if (pert.bits) p.bits = pert.bits + (uint64_t)done * ((nparams + 127) / 128 * 16);
        const PertArgs pa = pert_args(&p, key, nparams);
        double *op = out_plus + done, *om = out_minus + done;
        double *oc = done == 0 ? out_clean : nullptr;   // the first sequence adds the clean loss
        if (wide_tiles(batch, d_hid)) {
            // at most 4 probes per wave: 8 would hold 256 accumulator registers
            switch (w) {
            case 8:
            case 4: launch_chain<32, 4, true>(params, X, labels, batch, d_in, d_hid, d_out, partial, op, om, pa, stream, k / 4, oc); break;
            case 2: launch_chain<32, 2, true>(params, X, labels, batch, d_in, d_hid, d_out, partial, op, om, pa, stream, k / 2, oc); break;
            default: launch_chain<32, 1, true>(params, X, labels, batch, d_in, d_hid, d_out, partial, op, om, pa, stream, k, oc); break;
            }
        } else {
            switch (w) {
            case 8: launch_chain<16, 8, true>(params, X, labels, batch, d_in, d_hid, d_out, partial, op, om, pa, stream, k / 8, oc); break;
            case 4: launch_chain<16, 4, true>(params, X, labels, batch, d_in, d_hid, d_out, partial, op, om, pa, stream, k / 4, oc); break;
            case 2: launch_chain<16, 2, true>(params, X, labels, batch, d_in, d_hid, d_out, partial, op, om, pa, stream, k / 2, oc); break;
            default: launch_chain<16, 1, true>(params, X, labels, batch, d_in, d_hid, d_out, partial, op, om, pa, stream, k, oc); break;
            }
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        done += k;
    }
    return hipSuccess;
}

}  // namespace zo

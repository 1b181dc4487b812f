// zo_launch.hpp -- host-side launchers of the gfx950 kernels (internal to libzo).
// Arguments are validated by the C ABI layer (api.hip) before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zo {

struct Key {
    uint32_t k0, k1;  // Philox key = (seed_lo, seed_hi)
};

// Packed sign rows: rows of ceil(n/128)*16 bytes for probes probe0 .. probe0+nprobes-1.
hipError_t launch_gen_probes(Key key, uint32_t step, uint32_t probe0, uint32_t nprobes,
                             uint64_t offset, uint64_t n, uint8_t *bits, int num_cus,
                             hipStream_t stream);

// Slice lengths of the perturb passes are multiples of this many params (a whole number of
// the kernel's chunks: 4096 bf16 or 2048 fp32 params, 8 KiB each).
constexpr uint64_t kPerturbChunkParams = 4096;

// Workgroups of a non-persistent XCD-range launch (xcd_range_chunk) over n chunks with
// `waves` waves per workgroup: eight times those of the longest range (ranges differ by at
// most one chunk, so the longest holds ceil(n / 8)).  Launches cover at most
// kMaxChunksPerLaunch chunks, which keeps the grid below 2^31 workgroups even with one wave
// per workgroup.
constexpr uint64_t kMaxChunksPerLaunch = (uint64_t)1 << 30;
inline uint32_t xcd_range_grid(uint64_t n, uint32_t waves)
{
    return (uint32_t)(8 * (((n + 7) / 8 + waves - 1) / waves));
}

// theta[0..n) += alpha * z (fp32 or bf16), bits == nullptr regenerates.  slice > 0 (a
// multiple of kPerturbChunkParams) issues the pass as one launch per slice of that many
// params; 0 is one launch.
hipError_t launch_perturb(void *theta, bool bf16, uint64_t offset, uint64_t n, Key key,
                          uint32_t step, uint32_t probe, float alpha, const uint8_t *bits,
                          int num_cus, hipStream_t stream, uint64_t slice = 0);

// theta[0..n) += (+/-alpha_a) + (+/-alpha_b) in one pass (probes a and b); bits_a and
// bits_b are both given or both nullptr.  slice as launch_perturb.
hipError_t launch_perturb2(void *theta, bool bf16, uint64_t offset, uint64_t n, Key key,
                           uint32_t step, uint32_t probe_a, float alpha_a, uint32_t probe_b,
                           float alpha_b, const uint8_t *bits_a, const uint8_t *bits_b,
                           int num_cus, hipStream_t stream, uint64_t slice = 0);

// c[i] from (L+, L-, L0) in fp64; non-finite probes counted into *counter.
// mode 0: g / max(|h|, delta); 1: g / max(|h|, delta)^power; 2: g / npert (L0 unused).
hipError_t launch_probe_weights(const double *Lp, const double *Lm, const double *L0,
                                uint32_t npert, double eps, double delta, int mode,
                                double power, float *c, uint32_t *counter, hipStream_t stream);

// Largest probe count of one update (its sign tables live in LDS).
constexpr uint32_t kMaxNpert = 512;

// Raise the dynamic-LDS limit of the general update kernels to what kMaxNpert needs, on the
// current device (once per context, from zo_init; launches then call no attribute setter).
hipError_t prepare_update();

// theta[0..n) -= eta * sum_i c_i z_i through per-8-probe LDS tables.
hipError_t launch_update(void *theta, bool bf16, uint64_t offset, uint64_t n, Key key,
                         uint32_t step, const float *c, uint32_t npert, float eta,
                         const uint8_t *bits, int num_cus, hipStream_t stream);
// The update preceded, in the same pass, by the move theta + alpha_r * z_rprobe rounded as
// launch_perturb rounds it (rprobe < npert).
hipError_t launch_restore_update(void *theta, bool bf16, uint64_t offset, uint64_t n, Key key,
                                 uint32_t step, uint32_t rprobe, float ralpha, const float *c,
                                 uint32_t npert, float eta, const uint8_t *bits, int num_cus,
                                 hipStream_t stream);

// counter[0] = 0 with a fill kernel (no memset node if the caller captures a graph).
hipError_t launch_zero_u32(uint32_t *p, uint32_t count, hipStream_t stream);

// 1/2 sum a_j theta_j^2 in fp64, two deterministic passes through `partials`.
constexpr uint32_t kLossPartials = 1024;
hipError_t launch_quad_loss(const void *theta, bool bf16, const float *a, uint64_t n,
                            double *partials, double *out, hipStream_t stream);
constexpr uint32_t kQuadProbes = 4;   // probes per pass of the fused quadratic losses
// The same loss at theta +/- alpha z_i for n_probes consecutive probes from probe0, theta
// read once per kQuadProbes probes and never written; each loss bit-equal to zo_perturb
// followed by launch_quad_loss.  With out_clean the first pass also sums the loss at theta
// itself, bit-equal to launch_quad_loss.  `partials` as for launch_quad_loss (2 kQuadProbes
// + 1 slots).
hipError_t launch_quad_loss_probes(const void *theta, bool bf16, const float *a, uint64_t offset,
                                   uint64_t n, Key key, uint32_t step, uint32_t probe0,
                                   uint32_t nprobes, float alpha, const uint8_t *bits,
                                   double *partials, double *out_plus, double *out_minus,
                                   double *out_clean, hipStream_t stream);

// 1/2 sum a_j theta_j^2 + 1/2 ||U theta||^2, U row-major [r][n], r <= kLowRankMax;
// `partials` holds kLossPartials * (kLowRankMax + 1) doubles.
constexpr uint32_t kLowRankMax = 16;
hipError_t launch_lowrank_loss(const void *theta, bool bf16, const float *a, const float *U,
                               uint32_t r, uint64_t n, double *partials, double *out,
                               hipStream_t stream);

// Two-layer MLP classifier loss (fp32 parameters, MFMA GEMM, fp64 reduction); with
// `pert` the parameters are read as theta + alpha * z_probe without being written, and with
// `pert` and `out_minus` the loss at theta - alpha * z_probe goes to out_minus as well (the
// workspace then holds both signs' partials).
struct MlpPerturb {
    uint64_t offset;
    uint32_t step, probe;
    float alpha;
    const uint8_t *bits;
};
hipError_t launch_mlp_loss(const float *params, const float *X, const int64_t *labels,
                           uint32_t batch, uint32_t d_in, uint32_t d_hid, uint32_t d_out,
                           double *partial, double *out, const MlpPerturb *pert, Key key,
                           hipStream_t stream, double *out_minus = nullptr);

// Both losses of probes pert.probe .. pert.probe + nprobes - 1 (out_plus[i], out_minus[i]),
// up to kMlpProbesPerLaunch probes per launch sequence, kMlpProbesPerWave of them per wave
// sharing every operand load (ZO_MLP_PROBES_PER_WAVE overrides: 1, 2, 4, 8; 4 at most on 32-wide tiles); pert.bits (if
// given) holds nprobes packed rows.  With out_clean the first launch sequence also computes
// the loss at the unperturbed parameters (bit-equal to launch_mlp_loss without pert).  The
// workspace holds 2 * min(nprobes, kMlpProbesPerLaunch) + 1 slots of partial logits and row
// losses.
constexpr uint32_t kMlpProbesPerLaunch = 64;
constexpr uint32_t kMlpProbesPerWave = 2;
hipError_t launch_mlp_loss_probes(const float *params, const float *X, const int64_t *labels,
                                  uint32_t batch, uint32_t d_in, uint32_t d_hid, uint32_t d_out,
                                  double *partial, const MlpPerturb &pert, uint32_t nprobes,
                                  Key key, double *out_plus, double *out_minus,
                                  double *out_clean, hipStream_t stream);

// Diagnostic: every 16-byte word of buf (bytes % 16 == 0) <- word ^ mask, in place;
// slice_bytes > 0 (a multiple of 8 KiB) issues it as one launch per slice of that size.
hipError_t launch_stream_rmw(void *buf, uint64_t bytes, uint32_t mask, int num_cus,
                             hipStream_t stream, uint64_t slice_bytes = 0);

}  // namespace zo

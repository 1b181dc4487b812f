// api.hip -- the extern "C" boundary of libzo: context, argument validation, launches.
// Every check happens before any launch; a rejected call touches no device memory.
#include <mutex>
#include <new>

#include "../../include/zo.h"
#include "../../include/zo_placement.h"
#include "zo_launch.hpp"

static_assert(ZO_MAX_NPERT == zo::kMaxNpert, "one probe-count limit");
static_assert(2 * zo::kQuadProbes + 1 <= zo::kLowRankMax + 1,
              "the loss partials hold both signs of every probe of a fused pass and the clean loss");

// Scratch of zo_mlp_loss_pair_noalloc: the partial logits and row losses of both signs,
// ZO_NOALLOC_SCRATCH_BYTES per device, held until the process ends.  Host code never
// passes this name to a kernel (on the host it is only a stand-in symbol): kernels get the
// device address that hipGetSymbolAddress returns for the current device (scratch_on).
static __device__ __align__(256) unsigned char scratch[ZO_NOALLOC_SCRATCH_BYTES];

struct zo_ctx {
    uint64_t seed;
    int device;
    int num_cus;
    uint32_t *d_counter;   // non-finite probe counter
    double *d_partials;    // loss partial sums (zo::kLossPartials * (kLowRankMax + 1) doubles)
    uint64_t slice_bytes;  // perturb passes issued per slice of this many bytes (0: whole)
    void *d_scratch;       // this device's copy of `scratch`
};

namespace {

// Device address of `scratch` on device `dev` (which must be current), looked up once per
// device and kept; nullptr if the lookup fails.
void *scratch_on(int dev)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        addr[dev] = p;
    }
    return addr[dev];
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline zo::Key key_of(const zo_ctx *c) { return {(uint32_t)c->seed, (uint32_t)(c->seed >> 32)}; }

inline hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

// A usable context: non-null, and its device is the current one (its counter and scratch
// live there; a launch on another device would address them on the wrong GPU).
inline bool ctx_ok(const zo_ctx *c)
{
    int dev = -1;
    return c && hipGetDevice(&dev) == hipSuccess && dev == c->device;
}

inline zo_status from_hip(hipError_t e) { return e == hipSuccess ? ZO_OK : ZO_EHIP; }

// Params per slice for the context's slice setting and an element size: a whole number of
// streaming chunks, or 0 (one launch per pass).
inline uint64_t slice_params(const zo_ctx *c, uint64_t elem)
{
    const uint64_t p = c->slice_bytes / elem;
    return p / zo::kPerturbChunkParams * zo::kPerturbChunkParams;
}

// Slice size zo_tune_placement tries against one whole launch: on 60 GB and 25.7 GB
// buffers, 1 GiB slices gave the perturb pass its best sliced rate (256 MiB - 8 GiB tried).
constexpr uint64_t kTuneSliceBytes = (uint64_t)1 << 30;

// Common checks for a parameter range [offset, offset + n).
inline bool range_ok(uint64_t offset, uint64_t n)
{
    if (offset % 128u != 0) return false;
    if (n > UINT64_MAX - offset) return false;
    return true;
}

}  // namespace

extern "C" {

const char *zo_strerror(zo_status s)
{
    switch (s) {
    case ZO_OK: return "ok";
    case ZO_EINVAL: return "invalid argument";
    case ZO_EHIP: return "HIP runtime error";
    case ZO_ENOMEM: return "out of memory";
    case ZO_EUNSUPPORTED: return "unsupported request (beyond a documented limit)";
    }
    return "unknown status";
}

size_t zo_bits_stride(uint64_t n) { return (size_t)(((n + 127u) / 128u) * 16u); }

zo_status zo_init(uint64_t seed, zo_ctx **out)
{
    if (!out) return ZO_EINVAL;
    zo_ctx *c = new (std::nothrow) zo_ctx{};
    if (!c) return ZO_ENOMEM;
    c->seed = seed;
    if (hipGetDevice(&c->device) != hipSuccess ||
        hipDeviceGetAttribute(&c->num_cus, hipDeviceAttributeMultiprocessorCount, c->device) !=
            hipSuccess ||
        c->num_cus <= 0) {
        delete c;
        (void)hipGetLastError();
        return ZO_EHIP;
    }
    if (hipMalloc(reinterpret_cast<void **>(&c->d_counter), 256) != hipSuccess) {
        delete c;
        (void)hipGetLastError();
        return ZO_ENOMEM;
    }
    if (hipMalloc(reinterpret_cast<void **>(&c->d_partials),
                  (size_t)zo::kLossPartials * (zo::kLowRankMax + 1) * sizeof(double)) != hipSuccess) {
        (void)hipFree(c->d_counter);
        delete c;
        (void)hipGetLastError();
        return ZO_ENOMEM;
    }
    c->d_scratch = scratch_on(c->device);
    if (!c->d_scratch || zo::prepare_update() != hipSuccess ||
        zo::launch_zero_u32(c->d_counter, 64, nullptr) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(c->d_partials);
        (void)hipFree(c->d_counter);
        delete c;
        return ZO_EHIP;
    }
    *out = c;
    return ZO_OK;
}

zo_status zo_destroy(zo_ctx *c)
{
    if (!c) return ZO_OK;
    hipError_t e = hipDeviceSynchronize();
    if (c->d_partials) (void)hipFree(c->d_partials);
    if (c->d_counter) (void)hipFree(c->d_counter);
    delete c;
    return from_hip(e);
}

uint64_t zo_get_seed(const zo_ctx *c) { return c ? c->seed : 0; }

zo_status zo_gen_probes(zo_ctx *c, uint32_t step, uint32_t probe0, uint32_t n_probes,
                        uint64_t offset, uint64_t n, uint8_t *d_bits, void *stream)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    if (!range_ok(offset, n)) return ZO_EINVAL;
    if (n == 0 || n_probes == 0) return ZO_OK;
    if (!d_bits || !aligned16(d_bits)) return ZO_EINVAL;
    return from_hip(zo::launch_gen_probes(key_of(c), step, probe0, n_probes, offset, n, d_bits,
                                          c->num_cus, as_stream(stream)));
}

zo_status zo_perturb(zo_ctx *c, void *d_theta, zo_dtype dtype, uint64_t offset, uint64_t n,
                     uint32_t step, uint32_t probe, float alpha, const uint8_t *d_bits,
                     void *stream)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    if (dtype != ZO_FP32 && dtype != ZO_BF16) return ZO_EINVAL;
    if (!range_ok(offset, n)) return ZO_EINVAL;
    if (n == 0) return ZO_OK;
    if (!d_theta || !aligned16(d_theta)) return ZO_EINVAL;
    if (d_bits && !aligned16(d_bits)) return ZO_EINVAL;
    return from_hip(zo::launch_perturb(d_theta, dtype == ZO_BF16, offset, n, key_of(c), step,
                                       probe, alpha, d_bits, c->num_cus, as_stream(stream),
                                       slice_params(c, dtype == ZO_BF16 ? 2 : 4)));
}

zo_status zo_perturb2(zo_ctx *c, void *d_theta, zo_dtype dtype, uint64_t offset, uint64_t n,
                      uint32_t step, uint32_t probe_a, float alpha_a, uint32_t probe_b,
                      float alpha_b, const uint8_t *d_bits_a, const uint8_t *d_bits_b,
                      void *stream)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    if (dtype != ZO_FP32 && dtype != ZO_BF16) return ZO_EINVAL;
    if (!range_ok(offset, n)) return ZO_EINVAL;
    if ((d_bits_a == nullptr) != (d_bits_b == nullptr)) return ZO_EINVAL;
    if (n == 0) return ZO_OK;
    if (!d_theta || !aligned16(d_theta)) return ZO_EINVAL;
    if (d_bits_a && (!aligned16(d_bits_a) || !aligned16(d_bits_b))) return ZO_EINVAL;
    return from_hip(zo::launch_perturb2(d_theta, dtype == ZO_BF16, offset, n, key_of(c), step,
                                        probe_a, alpha_a, probe_b, alpha_b, d_bits_a, d_bits_b,
                                        c->num_cus, as_stream(stream),
                                        slice_params(c, dtype == ZO_BF16 ? 2 : 4)));
}

zo_status zo_probe_weights(zo_ctx *c, const double *d_Lp, const double *d_Lm,
                           const double *d_L0, uint32_t n_pert, double eps, double delta,
                           float *d_c, void *stream)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    if (!(eps == eps) || eps == 0.0 || eps - eps != 0.0) return ZO_EINVAL;       // NaN/0/inf
    if (!(delta >= 0.0) || delta - delta != 0.0) return ZO_EINVAL;               // <0/NaN/inf
    if (n_pert == 0) return ZO_OK;
    if (!d_Lp || !d_Lm || !d_L0 || !d_c) return ZO_EINVAL;
    return from_hip(zo::launch_probe_weights(d_Lp, d_Lm, d_L0, n_pert, eps, delta, 0, 1.0, d_c,
                                             c->d_counter, as_stream(stream)));
}

zo_status zo_probe_weights_ex(zo_ctx *c, const double *d_Lp, const double *d_Lm,
                              const double *d_L0, uint32_t n_pert, double eps, double delta,
                              zo_weights_mode mode, double power, float *d_c, void *stream)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    if (mode != ZO_WEIGHTS_PRECOND && mode != ZO_WEIGHTS_POWER && mode != ZO_WEIGHTS_SPSA_MEAN)
        return ZO_EINVAL;
    if (!(eps == eps) || eps == 0.0 || eps - eps != 0.0) return ZO_EINVAL;
    if (mode != ZO_WEIGHTS_SPSA_MEAN && (!(delta >= 0.0) || delta - delta != 0.0))
        return ZO_EINVAL;
    if (mode == ZO_WEIGHTS_POWER && (!(power >= 0.0) || power - power != 0.0)) return ZO_EINVAL;
    if (n_pert == 0) return ZO_OK;
    if (!d_Lp || !d_Lm || !d_c || (mode != ZO_WEIGHTS_SPSA_MEAN && !d_L0)) return ZO_EINVAL;
    return from_hip(zo::launch_probe_weights(d_Lp, d_Lm, d_L0, n_pert, eps, delta, (int)mode,
                                             power, d_c, c->d_counter, as_stream(stream)));
}

zo_status zo_update(zo_ctx *c, void *d_theta, zo_dtype dtype, uint64_t offset, uint64_t n,
                    uint32_t step, const float *d_c, uint32_t n_pert, float eta,
                    const uint8_t *d_bits, void *stream)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    if (dtype != ZO_FP32 && dtype != ZO_BF16) return ZO_EINVAL;
    if (!range_ok(offset, n)) return ZO_EINVAL;
    if (n_pert > ZO_MAX_NPERT) return ZO_EUNSUPPORTED;
    if (n == 0 || n_pert == 0) return ZO_OK;
    if (!d_theta || !aligned16(d_theta) || !d_c) return ZO_EINVAL;
    if (d_bits && !aligned16(d_bits)) return ZO_EINVAL;
    return from_hip(zo::launch_update(d_theta, dtype == ZO_BF16, offset, n, key_of(c), step, d_c,
                                      n_pert, eta, d_bits, c->num_cus, as_stream(stream)));
}

zo_status zo_restore_update(zo_ctx *c, void *d_theta, zo_dtype dtype, uint64_t offset,
                            uint64_t n, uint32_t step, uint32_t restore_probe,
                            float restore_alpha, const float *d_c, uint32_t n_pert, float eta,
                            const uint8_t *d_bits, void *stream)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    if (dtype != ZO_FP32 && dtype != ZO_BF16) return ZO_EINVAL;
    if (!range_ok(offset, n)) return ZO_EINVAL;
    if (n_pert > ZO_MAX_NPERT) return ZO_EUNSUPPORTED;
    if (restore_probe >= n_pert) return ZO_EINVAL;
    if (n == 0) return ZO_OK;
    if (!d_theta || !aligned16(d_theta) || !d_c) return ZO_EINVAL;
    if (d_bits && !aligned16(d_bits)) return ZO_EINVAL;
    return from_hip(zo::launch_restore_update(d_theta, dtype == ZO_BF16, offset, n, key_of(c),
                                              step, restore_probe, restore_alpha, d_c, n_pert,
                                              eta, d_bits, c->num_cus, as_stream(stream)));
}

zo_status zo_nonfinite_count(zo_ctx *c, void *stream, uint32_t *out)
{
    if (!ctx_ok(c) || !out) return ZO_EINVAL;
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return ZO_EHIP;
    uint32_t v = 0;
    if (hipMemcpy(&v, c->d_counter, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess)
        return ZO_EHIP;
    *out = v;
    return ZO_OK;
}

zo_status zo_reset_nonfinite(zo_ctx *c, void *stream)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    return from_hip(zo::launch_zero_u32(c->d_counter, 1, as_stream(stream)));
}

zo_status zo_quad_loss(zo_ctx *c, const void *d_theta, zo_dtype dtype, const float *d_a,
                       uint64_t n, double *d_out, void *stream)
{
    if (!ctx_ok(c) || !d_out) return ZO_EINVAL;
    if (dtype != ZO_FP32 && dtype != ZO_BF16) return ZO_EINVAL;
    if (n > 0 && (!d_theta || !d_a || !aligned16(d_theta) || !aligned16(d_a))) return ZO_EINVAL;
    return from_hip(zo::launch_quad_loss(d_theta, dtype == ZO_BF16, d_a, n, c->d_partials, d_out,
                                         as_stream(stream)));
}

zo_status zo_quad_loss_probes(zo_ctx *c, const void *d_theta, zo_dtype dtype, const float *d_a,
                              uint64_t offset, uint64_t n, uint32_t step, uint32_t probe0,
                              uint32_t n_probes, float alpha, const uint8_t *d_bits,
                              double *d_out_plus, double *d_out_minus, double *d_out_clean,
                              void *stream)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    if (dtype != ZO_FP32 && dtype != ZO_BF16) return ZO_EINVAL;
    if (n_probes == 0 && !d_out_clean) return ZO_OK;
    if (n_probes > 0 && (!d_out_plus || !d_out_minus)) return ZO_EINVAL;
    if (n_probes > 0 && n_probes - 1 > UINT32_MAX - probe0) return ZO_EINVAL;   // indices wrap
    if (!range_ok(offset, n)) return ZO_EINVAL;
    if (n > 0 && (!d_theta || !d_a || !aligned16(d_theta) || !aligned16(d_a))) return ZO_EINVAL;
    if (d_bits && !aligned16(d_bits)) return ZO_EINVAL;
    return from_hip(zo::launch_quad_loss_probes(d_theta, dtype == ZO_BF16, d_a, offset, n,
                                                key_of(c), step, probe0, n_probes, alpha,
                                                n > 0 ? d_bits : nullptr, c->d_partials,
                                                d_out_plus, d_out_minus, d_out_clean,
                                                as_stream(stream)));
}

zo_status zo_lowrank_quad_loss(zo_ctx *c, const void *d_theta, zo_dtype dtype,
                               const float *d_a, const float *d_U, uint32_t r, uint64_t n,
                               double *d_out, void *stream)
{
    if (!ctx_ok(c) || !d_out) return ZO_EINVAL;
    if (dtype != ZO_FP32 && dtype != ZO_BF16) return ZO_EINVAL;
    if (r > zo::kLowRankMax) return ZO_EUNSUPPORTED;
    if (n > 0 && (!d_theta || !d_a || !aligned16(d_theta) || !aligned16(d_a))) return ZO_EINVAL;
    if (n > 0 && r > 0 && (!d_U || !aligned16(d_U))) return ZO_EINVAL;
    return from_hip(zo::launch_lowrank_loss(d_theta, dtype == ZO_BF16, d_a, d_U, r, n,
                                            c->d_partials, d_out, as_stream(stream)));
}

uint64_t zo_mlp_workspace_bytes(uint32_t batch, uint32_t d_in, uint32_t d_hid, uint32_t d_out)
{
    (void)d_in;
    // partial logits and row losses of two signs (zo_mlp_loss_pair); one-sign calls use half
    return 2u * ((uint64_t)(d_hid / 16u) * batch * d_out + batch) * sizeof(double);
}

uint64_t zo_mlp_probes_workspace_bytes(uint32_t batch, uint32_t d_in, uint32_t d_hid,
                                       uint32_t d_out, uint32_t n_probes)
{
    (void)d_in;
    // partial logits and row losses of both signs of up to kMlpProbesPerLaunch probes and of
    // the clean loss
    const uint64_t k = n_probes < zo::kMlpProbesPerLaunch ? n_probes : zo::kMlpProbesPerLaunch;
    return (2u * k + 1u) * ((uint64_t)(d_hid / 16u) * batch * d_out + batch) * sizeof(double);
}

static zo_status mlp_checks(zo_ctx *c, const float *d_params, const float *d_X,
                            const int64_t *d_labels, uint32_t batch, uint32_t d_in,
                            uint32_t d_hid, uint32_t d_out, void *d_workspace,
                            uint64_t workspace_bytes, double *d_loss)
{
    if (!ctx_ok(c) || !d_params || !d_X || !d_labels || !d_workspace || !d_loss)
        return ZO_EINVAL;
    if (batch == 0 || d_in == 0 || d_hid == 0 || batch % 16u || d_in % 16u || d_hid % 16u)
        return ZO_EINVAL;
    if (d_out == 0 || d_out > 16u) return ZO_EINVAL;
    if (!aligned16(d_params) || !aligned16(d_X) || (reinterpret_cast<uintptr_t>(d_workspace) & 7u))
        return ZO_EINVAL;
    if (workspace_bytes < zo_mlp_workspace_bytes(batch, d_in, d_hid, d_out)) return ZO_EINVAL;
    return ZO_OK;
}

zo_status zo_mlp_loss(zo_ctx *c, const float *d_params, const float *d_X,
                      const int64_t *d_labels, uint32_t batch, uint32_t d_in, uint32_t d_hid,
                      uint32_t d_out, void *d_workspace, uint64_t workspace_bytes,
                      double *d_loss, void *stream)
{
    const zo_status st = mlp_checks(c, d_params, d_X, d_labels, batch, d_in, d_hid, d_out,
                                    d_workspace, workspace_bytes, d_loss);
    if (st != ZO_OK) return st;
    return from_hip(zo::launch_mlp_loss(d_params, d_X, d_labels, batch, d_in, d_hid, d_out,
                                        static_cast<double *>(d_workspace), d_loss, nullptr,
                                        key_of(c), as_stream(stream)));
}

zo_status zo_mlp_loss_perturbed(zo_ctx *c, const float *d_params, uint64_t offset,
                                uint32_t step, uint32_t probe, float alpha,
                                const uint8_t *d_bits, const float *d_X,
                                const int64_t *d_labels, uint32_t batch, uint32_t d_in,
                                uint32_t d_hid, uint32_t d_out, void *d_workspace,
                                uint64_t workspace_bytes, double *d_loss, void *stream)
{
    const zo_status st = mlp_checks(c, d_params, d_X, d_labels, batch, d_in, d_hid, d_out,
                                    d_workspace, workspace_bytes, d_loss);
    if (st != ZO_OK) return st;
    const uint64_t nparams = (uint64_t)d_hid * d_in + d_hid + (uint64_t)d_out * d_hid + d_out;
    if (!range_ok(offset, nparams)) return ZO_EINVAL;
    const zo::MlpPerturb pert{offset, step, probe, alpha, d_bits};
    return from_hip(zo::launch_mlp_loss(d_params, d_X, d_labels, batch, d_in, d_hid, d_out,
                                        static_cast<double *>(d_workspace), d_loss, &pert,
                                        key_of(c), as_stream(stream)));
}

zo_status zo_mlp_loss_pair(zo_ctx *c, const float *d_params, uint64_t offset, uint32_t step,
                           uint32_t probe, float alpha, const uint8_t *d_bits, const float *d_X,
                           const int64_t *d_labels, uint32_t batch, uint32_t d_in,
                           uint32_t d_hid, uint32_t d_out, void *d_workspace,
                           uint64_t workspace_bytes, double *d_loss_plus, double *d_loss_minus,
                           void *stream)
{
    const zo_status st = mlp_checks(c, d_params, d_X, d_labels, batch, d_in, d_hid, d_out,
                                    d_workspace, workspace_bytes, d_loss_plus);
    if (st != ZO_OK) return st;
    if (!d_loss_minus) return ZO_EINVAL;
    const uint64_t nparams = (uint64_t)d_hid * d_in + d_hid + (uint64_t)d_out * d_hid + d_out;
    if (!range_ok(offset, nparams)) return ZO_EINVAL;
    const zo::MlpPerturb pert{offset, step, probe, alpha, d_bits};
    return from_hip(zo::launch_mlp_loss(d_params, d_X, d_labels, batch, d_in, d_hid, d_out,
                                        static_cast<double *>(d_workspace), d_loss_plus, &pert,
                                        key_of(c), as_stream(stream), d_loss_minus));
}

zo_status zo_mlp_loss_probes(zo_ctx *c, const float *d_params, uint64_t offset, uint32_t step,
                             uint32_t probe0, uint32_t n_probes, float alpha,
                             const uint8_t *d_bits, const float *d_X, const int64_t *d_labels,
                             uint32_t batch, uint32_t d_in, uint32_t d_hid, uint32_t d_out,
                             void *d_workspace, uint64_t workspace_bytes, double *d_loss_plus,
                             double *d_loss_minus, double *d_loss_clean, void *stream)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    if (n_probes == 0 && !d_loss_clean) return ZO_OK;
    const zo_status st = mlp_checks(c, d_params, d_X, d_labels, batch, d_in, d_hid, d_out,
                                    d_workspace, UINT64_MAX,
                                    n_probes > 0 ? d_loss_plus : d_loss_clean);
    if (st != ZO_OK) return st;
    if (n_probes > 0 && !d_loss_minus) return ZO_EINVAL;
    if (workspace_bytes < zo_mlp_probes_workspace_bytes(batch, d_in, d_hid, d_out, n_probes))
        return ZO_EINVAL;
    if (n_probes > 0 && n_probes - 1 > UINT32_MAX - probe0) return ZO_EINVAL;   // indices wrap
    if (d_bits && !aligned16(d_bits)) return ZO_EINVAL;
    const uint64_t nparams = (uint64_t)d_hid * d_in + d_hid + (uint64_t)d_out * d_hid + d_out;
    if (!range_ok(offset, nparams)) return ZO_EINVAL;
    const zo::MlpPerturb pert{offset, step, probe0, alpha, d_bits};
    return from_hip(zo::launch_mlp_loss_probes(d_params, d_X, d_labels, batch, d_in, d_hid, d_out,
                                               static_cast<double *>(d_workspace), pert, n_probes,
                                               key_of(c), d_loss_plus, d_loss_minus,
                                               d_loss_clean, as_stream(stream)));
}

zo_status zo_mlp_loss_pair_noalloc(zo_ctx *c, const float *d_params, uint64_t offset,
                                   uint32_t step, uint32_t probe, float alpha,
                                   const uint8_t *d_bits, const float *d_X,
                                   const int64_t *d_labels, uint32_t batch, uint32_t d_in,
                                   uint32_t d_hid, uint32_t d_out, double *d_loss_plus,
                                   double *d_loss_minus, void *stream)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    // the workspace check below compares the library's own size with the scratch size;
    // shapes whose pair workspace exceeds it are refused before anything is launched
    if (batch != 0 && d_hid != 0 &&
        zo_mlp_workspace_bytes(batch, d_in, d_hid, d_out) > ZO_NOALLOC_SCRATCH_BYTES)
        return ZO_EUNSUPPORTED;
    const zo_status st = mlp_checks(c, d_params, d_X, d_labels, batch, d_in, d_hid, d_out,
                                    c->d_scratch, ZO_NOALLOC_SCRATCH_BYTES, d_loss_plus);
    if (st != ZO_OK) return st;
    if (!d_loss_minus) return ZO_EINVAL;
    const uint64_t nparams = (uint64_t)d_hid * d_in + d_hid + (uint64_t)d_out * d_hid + d_out;
    if (!range_ok(offset, nparams)) return ZO_EINVAL;
    const zo::MlpPerturb pert{offset, step, probe, alpha, d_bits};
    return from_hip(zo::launch_mlp_loss(d_params, d_X, d_labels, batch, d_in, d_hid, d_out,
                                        static_cast<double *>(c->d_scratch), d_loss_plus, &pert,
                                        key_of(c), as_stream(stream), d_loss_minus));
}

zo_status zo_stream_rmw(zo_ctx *c, void *d_buf, uint64_t bytes, uint32_t mask, void *stream)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    if (bytes == 0) return ZO_OK;
    if (!d_buf || !aligned16(d_buf) || bytes % 16u) return ZO_EINVAL;
    return from_hip(zo::launch_stream_rmw(d_buf, bytes, mask, c->num_cus, as_stream(stream),
                                          c->slice_bytes));
}

zo_status zo_set_slice_bytes(zo_ctx *c, uint64_t slice_bytes)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    if (slice_bytes % ((uint64_t)1 << 20)) return ZO_EINVAL;
    c->slice_bytes = slice_bytes;
    return ZO_OK;
}

uint64_t zo_get_slice_bytes(const zo_ctx *c) { return c ? c->slice_bytes : 0; }

zo_status zo_tune_placement(zo_ctx *c, void *d_buf, uint64_t bytes, void *stream,
                            uint64_t *out_slice_bytes, double *out_gbps_whole,
                            double *out_gbps_sliced)
{
    if (!ctx_ok(c)) return ZO_EINVAL;
    if (!d_buf || !aligned16(d_buf) || bytes % 16u) return ZO_EINVAL;
    const hipStream_t s = as_stream(stream);
    double gbps[2] = {0.0, 0.0};                 // whole, sliced
    const bool try_slices = bytes >= 2 * kTuneSliceBytes;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        (void)hipGetLastError();
        return ZO_EHIP;
    }
    zo_status st = ZO_OK;
    for (int mode = 0; mode < (try_slices ? 2 : 1) && st == ZO_OK; ++mode) {
        const uint64_t sl = mode ? kTuneSliceBytes : 0;
        // mask 0: every word is written back unchanged
        if (zo::launch_stream_rmw(d_buf, bytes, 0u, c->num_cus, s, sl) != hipSuccess ||
            hipEventRecord(e0, s) != hipSuccess) {
            st = ZO_EHIP;
            break;
        }
        for (int r = 0; r < 2; ++r)
            if (zo::launch_stream_rmw(d_buf, bytes, 0u, c->num_cus, s, sl) != hipSuccess)
                st = ZO_EHIP;
        float ms = 0.0f;
        if (st != ZO_OK || hipEventRecord(e1, s) != hipSuccess ||
            hipEventSynchronize(e1) != hipSuccess ||
            hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
            st = ZO_EHIP;
            break;
        }
        gbps[mode] = ms > 0.0f ? 2.0 * 2.0 * (double)bytes / (ms * 1e-3) / 1e9 : 0.0;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (st != ZO_OK) {
        (void)hipGetLastError();
        return st;
    }
    // slices only when clearly faster than one launch
    c->slice_bytes = (try_slices && gbps[1] > 1.02 * gbps[0]) ? kTuneSliceBytes : 0;
    if (out_slice_bytes) *out_slice_bytes = c->slice_bytes;
    if (out_gbps_whole) *out_gbps_whole = gbps[0];
    if (out_gbps_sliced) *out_gbps_sliced = gbps[1];
    return ZO_OK;
}

}  // extern "C"

/* capi_check.c -- the library driven from plain C through include/zo.h alone: device
 * buffers from hipMalloc, no torch, no Python.  Seeded inputs; every result is compared
 * with the C oracle (liboracle.so) computed here on the same inputs: packed planes,
 * in-place passes (one and two probes), probe weights bit for bit; the update within the
 * update bar (fp32: 1e-5 * max(|theta|, eta * sum|c|); bf16: one ulp); plus the argument
 * errors the header documents.  Test infrastructure: prints "capi ok" and exits 0 when
 * every check holds, names the first failing check and exits 1 otherwise. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zo.h"

/* The oracle's entry points (oracle/zo_oracle.c), declared here: the test links the two
 * libraries side by side; neither includes the other. */
uint64_t ora_plane_bytes(uint64_t n);
void ora_gen_plane(uint64_t seed, uint32_t step, uint32_t probe, uint64_t offset, uint64_t n,
                   uint8_t *out);
void ora_perturb_f32(float *th, uint64_t n, uint64_t offset, uint64_t seed, uint32_t step,
                     uint32_t probe, float alpha, const uint8_t *bits);
void ora_perturb2_bf16(uint16_t *th, uint64_t n, uint64_t offset, uint64_t seed, uint32_t step,
                       uint32_t probe_a, float alpha_a, uint32_t probe_b, float alpha_b,
                       const uint8_t *bits_a, const uint8_t *bits_b);
uint32_t ora_probe_weights(const double *Lp, const double *Lm, double L0, uint32_t n,
                           double eps, double delta, float *c);
void ora_update_f32(float *th, uint64_t n, uint64_t offset, uint64_t seed, uint32_t step,
                    const float *c, uint32_t npert, float eta, const uint8_t *bits);
void ora_update_bf16(uint16_t *th, uint64_t n, uint64_t offset, uint64_t seed, uint32_t step,
                     const float *c, uint32_t npert, float eta, const uint8_t *bits);
float ora_bf16_to_f32(uint16_t h);
double ora_quad_loss_f32(const float *th, const float *a, uint64_t n);
uint16_t ora_f32_to_bf16(float f);

#define FAIL(...)                                     \
    do {                                              \
        fprintf(stdout, "FAIL: " __VA_ARGS__);        \
        fprintf(stdout, "\n");                        \
        fflush(stdout);                               \
        exit(1);                                      \
    } while (0)
#define HIPCHK(x)                                                            \
    do {                                                                     \
        hipError_t e_ = (x);                                                 \
        if (e_ != hipSuccess) FAIL("%s: %s", #x, hipGetErrorString(e_));     \
    } while (0)
#define ZOCHK(x)                                                             \
    do {                                                                     \
        zo_status s_ = (x);                                                  \
        if (s_ != ZO_OK) FAIL("%s: %s", #x, zo_strerror(s_));                \
    } while (0)

/* splitmix64: seeded test inputs */
static uint64_t sm_state;
static uint64_t sm_next(void)
{
    uint64_t z = (sm_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double sm_uniform(void) { return (double)(sm_next() >> 11) * (1.0 / 9007199254740992.0); }

static double bf16_ulp(double v)
{
    double a = fabs(v);
    if (a < ldexp(1.0, -126)) return ldexp(1.0, -133);
    return ldexp(1.0, (int)floor(log2(a)) - 7);
}

int main(void)
{
    const uint64_t seed = 0x0123456789ABCDEFull;
    sm_state = 20261203u;
    zo_ctx *ctx = NULL;
    ZOCHK(zo_init(seed, &ctx));
    if (zo_get_seed(ctx) != seed) FAIL("zo_get_seed");

    /* 1. packed planes: three probes over a ragged range at a non-zero offset */
    {
        const uint64_t n = 10033, offset = 128 * 3;
        const uint32_t step = 2, probe0 = 1, np = 3;
        const uint64_t stride = zo_bits_stride(n);
        if (stride != ora_plane_bytes(n)) FAIL("zo_bits_stride");
        uint8_t *d = NULL, *h = malloc(stride * np), *r = malloc(stride);
        HIPCHK(hipMalloc((void **)&d, stride * np));
        ZOCHK(zo_gen_probes(ctx, step, probe0, np, offset, n, d, NULL));
        HIPCHK(hipMemcpy(h, d, stride * np, hipMemcpyDeviceToHost));
        for (uint32_t p = 0; p < np; ++p) {
            ora_gen_plane(seed, step, probe0 + p, offset, n, r);
            if (memcmp(h + p * stride, r, stride) != 0) FAIL("plane of probe %u", probe0 + p);
        }
        HIPCHK(hipFree(d));
        free(h);
        free(r);
    }

    /* 2. fp32 in-place pass, signs regenerated */
    {
        const uint64_t n = 20007, offset = 128;
        float *h = malloc(n * 4), *g = malloc(n * 4), *d = NULL;
        for (uint64_t i = 0; i < n; ++i) h[i] = (float)((sm_uniform() - 0.5) * 0.04);
        HIPCHK(hipMalloc((void **)&d, n * 4));
        HIPCHK(hipMemcpy(d, h, n * 4, hipMemcpyHostToDevice));
        ZOCHK(zo_perturb(ctx, d, ZO_FP32, offset, n, 5, 4, 0x1p-10f, NULL, NULL));
        HIPCHK(hipMemcpy(g, d, n * 4, hipMemcpyDeviceToHost));
        ora_perturb_f32(h, n, offset, seed, 5, 4, 0x1p-10f, NULL);
        if (memcmp(g, h, n * 4) != 0) FAIL("fp32 perturb");
        HIPCHK(hipFree(d));
        free(h);
        free(g);
    }

    /* 3. bf16 fused two-probe pass (restore of one probe, move to the next) */
    {
        const uint64_t n = 8192 * 3 + 999, offset = 0;
        uint16_t *h = malloc(n * 2), *g = malloc(n * 2), *d = NULL;
        for (uint64_t i = 0; i < n; ++i)
            h[i] = ora_f32_to_bf16((float)((sm_uniform() - 0.5) * 0.04));
        HIPCHK(hipMalloc((void **)&d, n * 2));
        HIPCHK(hipMemcpy(d, h, n * 2, hipMemcpyHostToDevice));
        ZOCHK(zo_perturb2(ctx, d, ZO_BF16, offset, n, 7, 2, 1e-3f, 3, 1e-3f, NULL, NULL, NULL));
        HIPCHK(hipMemcpy(g, d, n * 2, hipMemcpyDeviceToHost));
        ora_perturb2_bf16(h, n, offset, seed, 7, 2, 1e-3f, 3, 1e-3f, NULL, NULL);
        if (memcmp(g, h, n * 2) != 0) FAIL("bf16 fused pass");
        HIPCHK(hipFree(d));
        free(h);
        free(g);
    }

    /* 4. probe weights, then 5. the update with them (fp32 and bf16) */
    {
        const uint32_t npert = 16;
        const double eps = (double)1e-3f, delta = 1e-6;
        double Lp[16], Lm[16], L0 = 0.693;
        for (uint32_t i = 0; i < npert; ++i) {
            const double u = (sm_uniform() - 0.5) * 0.02;
            Lp[i] = L0 + u + 0.002 + (sm_uniform() - 0.5) * 0.002;
            Lm[i] = L0 - u + 0.002 + (sm_uniform() - 0.5) * 0.002;
        }
        double *dl = NULL;
        float *dc = NULL, c_gpu[16], c_ora[16];
        HIPCHK(hipMalloc((void **)&dl, (2 * npert + 1) * sizeof(double)));
        HIPCHK(hipMalloc((void **)&dc, npert * sizeof(float)));
        HIPCHK(hipMemcpy(dl, Lp, npert * sizeof(double), hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(dl + npert, Lm, npert * sizeof(double), hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(dl + 2 * npert, &L0, sizeof(double), hipMemcpyHostToDevice));
        ZOCHK(zo_probe_weights(ctx, dl, dl + npert, dl + 2 * npert, npert, eps, delta, dc, NULL));
        HIPCHK(hipMemcpy(c_gpu, dc, sizeof(c_gpu), hipMemcpyDeviceToHost));
        ora_probe_weights(Lp, Lm, L0, npert, eps, delta, c_ora);
        if (memcmp(c_gpu, c_ora, sizeof(c_gpu)) != 0) FAIL("probe weights");
        double csum = 0.0;
        for (uint32_t i = 0; i < npert; ++i) csum += fabs((double)c_ora[i]);

        const uint64_t n = 8192 * 2 + 333, offset = 128 * 9;
        const float eta = 1e-2f;
        float *h = malloc(n * 4), *g = malloc(n * 4), *d = NULL;
        for (uint64_t i = 0; i < n; ++i) h[i] = (float)((sm_uniform() - 0.5) * 0.04);
        HIPCHK(hipMalloc((void **)&d, n * 4));
        HIPCHK(hipMemcpy(d, h, n * 4, hipMemcpyHostToDevice));
        ZOCHK(zo_update(ctx, d, ZO_FP32, offset, n, 9, dc, npert, eta, NULL, NULL));
        HIPCHK(hipMemcpy(g, d, n * 4, hipMemcpyDeviceToHost));
        ora_update_f32(h, n, offset, seed, 9, c_ora, npert, eta, NULL);
        for (uint64_t i = 0; i < n; ++i) {
            const double tol = 1e-5 * fmax(fabs((double)h[i]), (double)eta * csum);
            if (fabs((double)g[i] - (double)h[i]) > tol) FAIL("fp32 update at %llu", (unsigned long long)i);
        }
        HIPCHK(hipFree(d));
        free(h);
        free(g);

        uint16_t *hb = malloc(n * 2), *gb = malloc(n * 2), *db = NULL;
        for (uint64_t i = 0; i < n; ++i)
            hb[i] = ora_f32_to_bf16((float)((sm_uniform() - 0.5) * 0.04));
        HIPCHK(hipMalloc((void **)&db, n * 2));
        HIPCHK(hipMemcpy(db, hb, n * 2, hipMemcpyHostToDevice));
        ZOCHK(zo_update(ctx, db, ZO_BF16, offset, n, 9, dc, npert, 1.0f, NULL, NULL));
        HIPCHK(hipMemcpy(gb, db, n * 2, hipMemcpyDeviceToHost));
        ora_update_bf16(hb, n, offset, seed, 9, c_ora, npert, 1.0f, NULL);
        for (uint64_t i = 0; i < n; ++i) {
            const double v = ora_bf16_to_f32(hb[i]), w = ora_bf16_to_f32(gb[i]);
            if (fabs(w - v) > bf16_ulp(v)) FAIL("bf16 update at %llu", (unsigned long long)i);
        }
        HIPCHK(hipFree(db));
        free(hb);
        free(gb);
        HIPCHK(hipFree(dl));
        HIPCHK(hipFree(dc));
    }

    /* 6. the quadratic loss at theta +/- alpha z_i of three probes, theta read once and not
     *    written: each loss within the fp64 summation bound of the oracle's perturb + loss;
     *    the clean loss from the same pass equal to zo_quad_loss and within that bound of
     *    the oracle's loss at theta */
    {
        const uint64_t n = 30011, offset = 256;
        const uint32_t np = 3, step = 4, probe0 = 6;
        const float alpha = 0x1p-10f;
        float *h = malloc(n * 4), *a = malloc(n * 4), *w = malloc(n * 4), *g = malloc(n * 4);
        float *dt = NULL, *da = NULL;
        double *dp = NULL, *dm = NULL, *dc = NULL, *dq = NULL, lp[3], lm[3], lc, lq;
        for (uint64_t i = 0; i < n; ++i) {
            h[i] = (float)((sm_uniform() - 0.5) * 2.0);
            a[i] = (float)(0.1 + sm_uniform());
        }
        HIPCHK(hipMalloc((void **)&dt, n * 4));
        HIPCHK(hipMalloc((void **)&da, n * 4));
        HIPCHK(hipMalloc((void **)&dp, np * 8));
        HIPCHK(hipMalloc((void **)&dm, np * 8));
        HIPCHK(hipMalloc((void **)&dc, 8));
        HIPCHK(hipMalloc((void **)&dq, 8));
        HIPCHK(hipMemcpy(dt, h, n * 4, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(da, a, n * 4, hipMemcpyHostToDevice));
        ZOCHK(zo_quad_loss_probes(ctx, dt, ZO_FP32, da, offset, n, step, probe0, np, alpha, NULL,
                                  dp, dm, dc, NULL));
        ZOCHK(zo_quad_loss(ctx, dt, ZO_FP32, da, n, dq, NULL));
        HIPCHK(hipMemcpy(&lc, dc, 8, hipMemcpyDeviceToHost));
        HIPCHK(hipMemcpy(&lq, dq, 8, hipMemcpyDeviceToHost));
        if (memcmp(&lc, &lq, 8) != 0) FAIL("fused clean loss differs from zo_quad_loss");
        {
            const double ref = ora_quad_loss_f32(h, a, n);
            if (fabs(lc - ref) > 4.0 * (double)n * 0x1p-53 * fabs(ref)) FAIL("fused clean loss");
        }
        HIPCHK(hipMemcpy(lp, dp, np * 8, hipMemcpyDeviceToHost));
        HIPCHK(hipMemcpy(lm, dm, np * 8, hipMemcpyDeviceToHost));
        HIPCHK(hipMemcpy(g, dt, n * 4, hipMemcpyDeviceToHost));
        if (memcmp(g, h, n * 4) != 0) FAIL("fused losses wrote theta");
        for (uint32_t i = 0; i < np; ++i) {
            for (int sgn = 0; sgn < 2; ++sgn) {
                memcpy(w, h, n * 4);
                ora_perturb_f32(w, n, offset, seed, step, probe0 + i, sgn ? -alpha : alpha, NULL);
                const double ref = ora_quad_loss_f32(w, a, n), got = sgn ? lm[i] : lp[i];
                if (fabs(got - ref) > 4.0 * (double)n * 0x1p-53 * fabs(ref))
                    FAIL("fused quadratic loss");
            }
        }
        HIPCHK(hipFree(dt));
        HIPCHK(hipFree(da));
        HIPCHK(hipFree(dp));
        HIPCHK(hipFree(dm));
        HIPCHK(hipFree(dc));
        HIPCHK(hipFree(dq));
        free(h);
        free(a);
        free(w);
        free(g);
    }

    /* 7. documented argument errors (nothing launched) */
    {
        float *d = NULL;
        HIPCHK(hipMalloc((void **)&d, 1024 * 4));
        if (zo_perturb(ctx, d, ZO_FP32, 64, 256, 0, 0, 1.0f, NULL, NULL) != ZO_EINVAL)
            FAIL("offset %% 128 != 0 accepted");
        if (zo_perturb(ctx, NULL, ZO_FP32, 0, 256, 0, 0, 1.0f, NULL, NULL) != ZO_EINVAL)
            FAIL("null theta accepted");
        if (zo_perturb(ctx, (char *)d + 4, ZO_FP32, 0, 256, 0, 0, 1.0f, NULL, NULL) != ZO_EINVAL)
            FAIL("misaligned theta accepted");
        if (zo_perturb(NULL, d, ZO_FP32, 0, 256, 0, 0, 1.0f, NULL, NULL) != ZO_EINVAL)
            FAIL("null context accepted");
        if (zo_perturb(ctx, d, ZO_FP32, 0, 0, 0, 0, 1.0f, NULL, NULL) != ZO_OK)
            FAIL("empty call rejected");
        if (!zo_strerror(ZO_EINVAL) || !zo_strerror(ZO_EHIP)) FAIL("zo_strerror");
        HIPCHK(hipFree(d));
    }
    HIPCHK(hipDeviceSynchronize());
    ZOCHK(zo_destroy(ctx));
    printf("capi ok\n");
    return 0;
}

/*
 * zo_oracle.c -- plain, slow CPU oracle for the 1.5-SPSA perturb / probe-weight /
 * update path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file; only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or constant generator with the HIP library: every
 * constant below is written out here from its published definition.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC (no FMA
 * contraction, no flush-to-zero: x86-64 SSE arithmetic, FLT_EVAL_METHOD == 0).
 *
 * Sources, by the title of the page they come from:
 *  - "Stanford's 1.5-SPSA Trains OPT-30B Without Backpropagation", section
 *    "How 1.5-SPSA Works": Rademacher probes z_i, the loss at theta +/- eps*z_i, and the
 *    central difference divided by 2*eps (the displayed estimator, which is garbled; the
 *    standard SPSA reading is taken).
 *  - the same page, section "Probe-Space Preconditioning": one clean (unperturbed) loss
 *    per step feeding a diagonal weight per probe that shrinks high-curvature probes.
 *    The page stops before the formula; the form used here is
 *    c_i = g_i / max(|h_i|, delta) with h_i the second difference through the clean loss.
 *  - "Pretraining Transformers Without Backprop: What Two Zero-Order Papers Actually
 *    Measure", the ZOO training-loop flowchart: weights move by W <- W - eta * g_hat.
 *  - "Probe-Space Preconditioning for Fast and Stable Zero-Order Training" (abstract):
 *    in-place, inference-mode training, probes produced by an 8-bit-packing generator
 *    (read as 8 sign bits per byte) and applied by fused unpack/apply kernels.
 *  - Philox4x32-10: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random
 *    Numbers: As Easy as 1, 2, 3", SC'11, section 4 (the Philox bijection).
 *
 * Conventions fixed where the pages are silent (each is a reading, not a page fact):
 *  - probe j of (seed, step, probe): counter = (blk_lo, blk_hi, probe, step) with
 *    blk = j / 128, key = (seed_lo, seed_hi); bit (j % 32) of output word (j / 32) % 4;
 *    z = +1 for bit 1, -1 for bit 0.
 *  - packed plane: the four output words of each block stored little-endian, so byte m
 *    holds params 8m .. 8m+7, least significant bit first.
 *  - bf16 perturb: widen to fp32 (exact), one fp32 add, round to nearest even to bf16.
 *  - update: s_j = sum_i c_i z_ij in fp64 (i ascending), t = theta_j - eta*s_j in fp64,
 *    one rounding of t to the storage type.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------------------------- */
/* Philox4x32-10 (Salmon et al., SC'11, section 4).                                   */
/* One round maps (c0,c1,c2,c3) with key (k0,k1) to                                   */
/*   (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0));             */
/* the key is bumped by the Weyl constants between rounds; ten rounds.                */
/* ---------------------------------------------------------------------------------- */
static const uint32_t ORA_PHILOX_M0 = 0xD2511F53u;
static const uint32_t ORA_PHILOX_M1 = 0xCD9E8D57u;
static const uint32_t ORA_PHILOX_W0 = 0x9E3779B9u; /* golden ratio */
static const uint32_t ORA_PHILOX_W1 = 0xBB67AE85u; /* sqrt(3) - 1 */

void ora_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += ORA_PHILOX_W0;
            k1 += ORA_PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)ORA_PHILOX_M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)ORA_PHILOX_M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 128 sign bits of block `blk` of probe `probe` at `step` under `seed`. */
static void ora_block_words(uint64_t seed, uint32_t step, uint32_t probe, uint64_t blk,
                            uint32_t words[4])
{
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), probe, step};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    ora_philox4x32_10(ctr, key, words);
}

/* Rademacher sign z_j in {-1, +1} of global parameter index j (plain definition). */
int ora_sign(uint64_t seed, uint32_t step, uint32_t probe, uint64_t j)
{
    uint32_t w[4];
    ora_block_words(seed, step, probe, j >> 7, w);
    uint32_t bit = (w[(j >> 5) & 3u] >> (j & 31u)) & 1u;
    return bit ? +1 : -1;
}

/* Bytes per packed probe row covering n parameters: whole 128-param blocks. */
uint64_t ora_plane_bytes(uint64_t n) { return ((n + 127u) / 128u) * 16u; }

/* Packed sign plane of one probe over global params [offset, offset + n),
 * offset % 128 == 0.  Byte m holds params offset + 8m .. +7, LSB first. */
void ora_gen_plane(uint64_t seed, uint32_t step, uint32_t probe, uint64_t offset,
                   uint64_t n, uint8_t *out)
{
    uint64_t nblk = (n + 127u) / 128u;
    for (uint64_t b = 0; b < nblk; ++b) {
        uint32_t w[4];
        ora_block_words(seed, step, probe, (offset >> 7) + b, w);
        for (int k = 0; k < 4; ++k)
            for (int byte = 0; byte < 4; ++byte)
                out[b * 16u + (uint64_t)k * 4u + (uint64_t)byte] = (uint8_t)(w[k] >> (8 * byte));
    }
}

/* Sign bit of local element e (0 <= e < n) from a packed row. */
static int ora_plane_bit(const uint8_t *row, uint64_t e)
{
    return (row[e >> 3] >> (e & 7u)) & 1;
}

/* ---------------------------------------------------------------------------------- */
/* bfloat16: 1 sign, 8 exponent, 7 stored mantissa bits (the top half of an fp32).   */
/* ---------------------------------------------------------------------------------- */
float ora_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a double to the nearest bf16, ties to even, straight from the definition:
 * the representable bf16 values of magnitude in [2^E, 2^(E+1)) are spaced q = 2^(E-7)
 * (normal) and the subnormals are spaced 2^-133; the result is rint(|x|/q)*q (rint
 * rounds half to even), and anything that rounds to 2^128 or above is infinity.
 * NaN maps to the quiet NaN 0x7FC0 with the input's sign. */
uint16_t ora_f64_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    int ex;
    (void)frexp(a, &ex);          /* a = m * 2^ex, m in [0.5, 1)  => a in [2^(ex-1), 2^ex) */
    int E = ex - 1;
    int qexp = (E >= -126) ? (E - 7) : -133;
    double k = rint(ldexp(a, -qexp)); /* exact scaling, then round half to even */
    double v = ldexp(k, qexp);        /* exact */
    if (v >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    float f = (float)v;               /* exact: v is a bf16 value, hence an fp32 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFFu));
}

/* fp32 -> bf16 nearest-even: the fp32 value is exact in double. */
uint16_t ora_f32_to_bf16(float f) { return ora_f64_to_bf16((double)f); }

/* ---------------------------------------------------------------------------------- */
/* Perturb: theta_j <- theta_j + alpha * z_j in place ("How 1.5-SPSA Works": losses are */
/* taken at theta +/- eps*z_i; the abstract: parameters are changed in place).        */
/* bits == NULL regenerates the signs from (seed, step, probe); otherwise `bits` is the */
/* packed row of this probe over the same [offset, offset+n).                         */
/* ---------------------------------------------------------------------------------- */
void ora_perturb_f32(float *th, uint64_t n, uint64_t offset, uint64_t seed, uint32_t step,
                     uint32_t probe, float alpha, const uint8_t *bits)
{
    for (uint64_t e = 0; e < n; ++e) {
        int bit = bits ? ora_plane_bit(bits, e)
                       : (ora_sign(seed, step, probe, offset + e) > 0);
        float d = bit ? alpha : -alpha;
        th[e] = th[e] + d;
    }
}

void ora_perturb_bf16(uint16_t *th, uint64_t n, uint64_t offset, uint64_t seed,
                      uint32_t step, uint32_t probe, float alpha, const uint8_t *bits)
{
    for (uint64_t e = 0; e < n; ++e) {
        int bit = bits ? ora_plane_bit(bits, e)
                       : (ora_sign(seed, step, probe, offset + e) > 0);
        float d = bit ? alpha : -alpha;
        float t = ora_bf16_to_f32(th[e]) + d;   /* one fp32 rounding */
        th[e] = ora_f32_to_bf16(t);              /* one bf16 rounding */
    }
}

/* Fused move of two probes in one pass: theta_j <- round(theta_j + d_j) with
 * d_j = (+/-alpha_a) + (+/-alpha_b) formed in fp32 (exact when |alpha_a| == |alpha_b|,
 * the case of a restore of probe a fused with the next probe b), then the same fp32 add
 * (and for bf16 the same nearest-even narrow) as a single-probe perturb.  The restore of
 * one probe and the +eps move of the next ("How 1.5-SPSA Works": losses at theta +/-
 * eps*z_i, restoring in between) thereby take one pass instead of two. */
static float ora_fused_delta(int bit_a, float alpha_a, int bit_b, float alpha_b)
{
    float da = bit_a ? alpha_a : -alpha_a;
    float db = bit_b ? alpha_b : -alpha_b;
    return da + db;
}

void ora_perturb2_f32(float *th, uint64_t n, uint64_t offset, uint64_t seed, uint32_t step,
                      uint32_t probe_a, float alpha_a, uint32_t probe_b, float alpha_b,
                      const uint8_t *bits_a, const uint8_t *bits_b)
{
    for (uint64_t e = 0; e < n; ++e) {
        int ba = bits_a ? ora_plane_bit(bits_a, e)
                        : (ora_sign(seed, step, probe_a, offset + e) > 0);
        int bb = bits_b ? ora_plane_bit(bits_b, e)
                        : (ora_sign(seed, step, probe_b, offset + e) > 0);
        th[e] = th[e] + ora_fused_delta(ba, alpha_a, bb, alpha_b);
    }
}

void ora_perturb2_bf16(uint16_t *th, uint64_t n, uint64_t offset, uint64_t seed, uint32_t step,
                       uint32_t probe_a, float alpha_a, uint32_t probe_b, float alpha_b,
                       const uint8_t *bits_a, const uint8_t *bits_b)
{
    for (uint64_t e = 0; e < n; ++e) {
        int ba = bits_a ? ora_plane_bit(bits_a, e)
                        : (ora_sign(seed, step, probe_a, offset + e) > 0);
        int bb = bits_b ? ora_plane_bit(bits_b, e)
                        : (ora_sign(seed, step, probe_b, offset + e) > 0);
        float t = ora_bf16_to_f32(th[e]) + ora_fused_delta(ba, alpha_a, bb, alpha_b);
        th[e] = ora_f32_to_bf16(t);
    }
}

/* ---------------------------------------------------------------------------------- */
/* Probe weights ("How 1.5-SPSA Works" for g; "Probe-Space Preconditioning" for the   */
/* clean-pass curvature weighting), in double:                                       */
/*   g_i = (L+_i - L-_i) / (2 eps)                                                    */
/*   h_i = ((L+_i + L-_i) - 2 L0) / (eps*eps)                                          */
/*   c_i = g_i / max(|h_i|, delta), rounded once to fp32.                             */
/* A probe with a non-finite L+_i, L-_i or L0 gets c_i = 0 and is counted.            */
/* Returns the number of such probes.                                                 */
/* ---------------------------------------------------------------------------------- */
uint32_t ora_probe_weights(const double *Lp, const double *Lm, double L0, uint32_t n,
                           double eps, double delta, float *c)
{
    uint32_t bad = 0;
    for (uint32_t i = 0; i < n; ++i) {
        if (!isfinite(Lp[i]) || !isfinite(Lm[i]) || !isfinite(L0)) {
            c[i] = 0.0f;
            ++bad;
            continue;
        }
        double g = (Lp[i] - Lm[i]) / (2.0 * eps);
        double h = ((Lp[i] + Lm[i]) - 2.0 * L0) / (eps * eps);
        double den = fabs(h) > delta ? fabs(h) : delta;
        c[i] = (float)(g / den);
    }
    return bad;
}

/* Other weight forms of the pages, in double, one rounding to fp32:
 *  mode 0  c_i = g_i / max(|h_i|, delta)            (as ora_probe_weights)
 *  mode 1  c_i = g_i / max(|h_i|, delta)^power      ("Probe-Space Preconditioning": a
 *          curvature weight |c_hat_i|^alpha from the clean and perturbed losses that
 *          shrinks high-curvature probes; the pages' alpha is 0.1)
 *  mode 2  c_i = g_i / n                            (plain 1SPSA mean of "How 1.5-SPSA
 *          Works": no clean pass; L0 is not read)
 * A probe with a non-finite loss it reads gets c_i = 0 and is counted. */
uint32_t ora_probe_weights_ex(const double *Lp, const double *Lm, double L0, uint32_t n,
                              double eps, double delta, int mode, double power, float *c)
{
    uint32_t bad = 0;
    for (uint32_t i = 0; i < n; ++i) {
        int uses_l0 = (mode != 2);
        if (!isfinite(Lp[i]) || !isfinite(Lm[i]) || (uses_l0 && !isfinite(L0))) {
            c[i] = 0.0f;
            ++bad;
            continue;
        }
        double g = (Lp[i] - Lm[i]) / (2.0 * eps);
        if (mode == 2) {
            c[i] = (float)(g / (double)n);
            continue;
        }
        double h = ((Lp[i] + Lm[i]) - 2.0 * L0) / (eps * eps);
        double den = fabs(h) > delta ? fabs(h) : delta;
        if (mode == 1) den = pow(den, power);
        c[i] = (float)(g / den);
    }
    return bad;
}

/* ---------------------------------------------------------------------------------- */
/* Multi-probe update theta <- theta - eta * sum_i c_i z_i (the loop's update box in   */
/* the ZOO training-loop flowchart; "How 1.5-SPSA Works" for the probe sum).          */
/* Per element: s = sum over i ascending of (double)c_i * z_ij in fp64, then          */
/* t = (double)theta - (double)eta * s, rounded once.  bits == NULL regenerates; else */
/* `bits` holds npert packed rows of ora_plane_bytes(n) bytes each.                   */
/* ---------------------------------------------------------------------------------- */
static void ora_block_sums(double *s, uint64_t e0, uint64_t cnt, uint64_t offset,
                           uint64_t seed, uint32_t step, const float *c, uint32_t npert,
                           const uint8_t *bits, uint64_t stride)
{
    for (uint64_t k = 0; k < cnt; ++k) s[k] = 0.0;
    for (uint32_t i = 0; i < npert; ++i) {
        uint32_t w[4];
        if (!bits) ora_block_words(seed, step, i, (offset + e0) >> 7, w);
        for (uint64_t k = 0; k < cnt; ++k) {
            uint64_t e = e0 + k;
            int bit = bits ? ora_plane_bit(bits + (uint64_t)i * stride, e)
                           : (int)((w[(e >> 5) & 3u] >> (e & 31u)) & 1u);
            double z = bit ? 1.0 : -1.0;
            s[k] += (double)c[i] * z;
        }
    }
}

void ora_update_f32(float *th, uint64_t n, uint64_t offset, uint64_t seed, uint32_t step,
                    const float *c, uint32_t npert, float eta, const uint8_t *bits)
{
    uint64_t stride = ora_plane_bytes(n);
    double s[128];
    for (uint64_t e0 = 0; e0 < n; e0 += 128) {
        uint64_t cnt = (n - e0) < 128 ? (n - e0) : 128;
        ora_block_sums(s, e0, cnt, offset, seed, step, c, npert, bits, stride);
        for (uint64_t k = 0; k < cnt; ++k) {
            double t = (double)th[e0 + k] - (double)eta * s[k];
            th[e0 + k] = (float)t;
        }
    }
}

void ora_update_bf16(uint16_t *th, uint64_t n, uint64_t offset, uint64_t seed, uint32_t step,
                     const float *c, uint32_t npert, float eta, const uint8_t *bits)
{
    uint64_t stride = ora_plane_bytes(n);
    double s[128];
    for (uint64_t e0 = 0; e0 < n; e0 += 128) {
        uint64_t cnt = (n - e0) < 128 ? (n - e0) : 128;
        ora_block_sums(s, e0, cnt, offset, seed, step, c, npert, bits, stride);
        for (uint64_t k = 0; k < cnt; ++k) {
            double t = (double)ora_bf16_to_f32(th[e0 + k]) - (double)eta * s[k];
            th[e0 + k] = ora_f64_to_bf16(t);
        }
    }
}

/* The probe sums s_j alone (fp64), for diagnostics of the update's summation error. */
void ora_probe_sums(double *s_out, uint64_t n, uint64_t offset, uint64_t seed, uint32_t step,
                    const float *c, uint32_t npert, const uint8_t *bits)
{
    uint64_t stride = ora_plane_bytes(n);
    for (uint64_t e0 = 0; e0 < n; e0 += 128) {
        uint64_t cnt = (n - e0) < 128 ? (n - e0) : 128;
        ora_block_sums(s_out + e0, e0, cnt, offset, seed, step, c, npert, bits, stride);
    }
}

/* ---------------------------------------------------------------------------------- */
/* Diagonal quadratic loss L = 1/2 sum_j a_j theta_j^2, accumulated in fp64 with j     */
/* ascending (a stand-in for the model's forward pass on the synthetic workloads).    */
/* ---------------------------------------------------------------------------------- */
double ora_quad_loss_f32(const float *th, const float *a, uint64_t n)
{
    double acc = 0.0;
    for (uint64_t j = 0; j < n; ++j) {
        double t = (double)th[j];
        acc += (double)a[j] * t * t;
    }
    return 0.5 * acc;
}

double ora_quad_loss_bf16(const uint16_t *th, const float *a, uint64_t n)
{
    double acc = 0.0;
    for (uint64_t j = 0; j < n; ++j) {
        double t = (double)ora_bf16_to_f32(th[j]);
        acc += (double)a[j] * t * t;
    }
    return 0.5 * acc;
}

/* Array helpers for the tests: element-wise roundings with the definitions above. */
void ora_f64_to_bf16_array(const double *x, uint16_t *out, uint64_t n)
{
    for (uint64_t j = 0; j < n; ++j) out[j] = ora_f64_to_bf16(x[j]);
}

void ora_f32_to_bf16_array(const float *x, uint16_t *out, uint64_t n)
{
    for (uint64_t j = 0; j < n; ++j) out[j] = ora_f32_to_bf16(x[j]);
}

/*
 * fp4_oracle.c -- plain, slow, scalar CPU oracle for block-scaled FP4
 * quantization.  TEST INFRASTRUCTURE ONLY: it is loaded by the test suite,
 * by the smoke check and by the CPU-baseline leg of the benchmark, never by
 * the GPU library.  It shares no code, header, table or constant generator
 * with the HIP path.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared fp4_oracle.c -lm
 * (no -ffast-math: every double and float operation below must be IEEE
 * round-to-nearest-even with gradual underflow).
 *
 * Sources (cited by page title and section):
 *  [MXA] "MXFP4 Quantization: Audit the 4.25-Bit Blocks"
 *        sections "Read the FP4 E2M1 value lattice", "Read the shared E8M0
 *        scale", "Encode one MXFP4 block step by step", "Expose outlier and
 *        dead-zone damage", "Publish the MXFP4 audit receipt".
 *  [SUB4] "Sub-4-Bit Microscaling (NVFP4, MXFP4 & Walsh-Hadamard Rotation)"
 *        sections 1 (E2M1), 2 (MXFP4 vs NVFP4 two-level scaling), 3 (FWHT).
 *  [EXEC] metrale_circuit "hardware::exec" module description (the exact
 *        E2M1 -> E4M3 bit conversion).
 *  [ABS] "Adaptive Block-Scaled Data Types" podcast transcript, cue 8
 *        (random Hadamard transform, stochastic rounding), cue 10
 *        (Four Over Six), cues 14 and 17 (IF4: FP4 or scaled INT4 per
 *        16-block, flagged in the sign bit of the block scale).
 * Where the pages leave a step open, the reading taken is named R-n; the
 * list of readings lives with the design notes of this repository.
 *
 * Parity status: every exported function is pinned by the host test suite
 * (worked examples, library routines, exact-rational brute force, closed
 * forms).  Parity unpinned: the exact Philox bit stream beyond the rocRAND
 * cross-check, and Four-Over-Six and IF4 choices on blocks whose two sums of
 * squared errors are within fp32 rounding of each other (the frozen
 * summation order R-14 decides those).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_BAD 1

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* E2M1 element, [SUB4] section 1 and [MXA] "Read the FP4 E2M1 value
 * lattice": 1 sign bit (bit 3), 2 exponent bits (bits 2..1), 1 mantissa bit
 * (bit 0), exponent bias 1, exponent field 0 is subnormal, no Inf/NaN. */
double oracle_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E8M0 scale byte, [MXA] "Read the shared E8M0 scale": 2^(b-127),
 * byte 255 reserved for NaN. */
double oracle_e8m0_value(int byte)
{
    if (byte == 255) return NAN;
    return ldexp(1.0, byte - 127);
}

/* E4M3 (FN flavour: bias 7, subnormals k * 2^-9, max 448, S.1111.111 NaN),
 * the NVFP4 block scale of [SUB4] section 2.  Reading R-11. */
double oracle_e4m3_value(int byte)
{
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Round t >= 0 to the nearest E4M3 value, ties to the even code, values
 * above the largest finite value saturate to 448 (R-11).  Enumerates every
 * finite non-negative code. */
int oracle_e4m3_encode(double t)
{
    int best = 0, c;
    double bd = INFINITY;
    if (!(t >= 0)) return 0x7F;      /* NaN / negative never requested */
    if (t >= 448.0) return 0x7E;
    for (c = 0; c <= 0x7E; c++) {
        double d = fabs(t - oracle_e4m3_value(c));
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            bd = d;
            best = c;
        }
    }
    return best;
}

/* Nearest point of the E2M1 magnitude lattice to a = |q|, ties to the even
 * code ([MXA] "Read the FP4 E2M1 value lattice": round to nearest, ties to
 * even, magnitudes above 6 clamp to 6 and count as saturated; reading R-3:
 * exactly 6 is not counted).  Returns the magnitude code 0..7. */
static int e2m1_nearest_mag(double a, int *sat)
{
    int k, best = 0;
    double bd = INFINITY;
    *sat = 0;
    if (a > 6.0) {
        *sat = 1;
        return 7;
    }
    for (k = 0; k < 8; k++) {
        double d = fabs(a - oracle_e2m1_value(k));
        if (d < bd || (d == bd && (k & 1) == 0 && (best & 1) == 1)) {
            bd = d;
            best = k;
        }
    }
    return best;
}

/* Stochastic rounding onto the E2M1 lattice (reading R-17): with lo <= a <
 * hi the neighbouring lattice points, round up iff a - lo > (u / 65536) *
 * (hi - lo), u a 16-bit uniform draw.  Lattice points never move; a > 6
 * saturates.  The comparison is exact: t = lo + u * 2^-16 * (hi - lo) has at
 * most 19 significant bits. */
static int e2m1_stochastic_mag(double a, unsigned u, int *sat)
{
    int k;
    *sat = 0;
    if (a > 6.0) {
        *sat = 1;
        return 7;
    }
    if (a == 6.0) return 7;
    for (k = 0; k < 7; k++) {
        double lo = oracle_e2m1_value(k), hi = oracle_e2m1_value(k + 1);
        if (a >= lo && a < hi) {
            double t = lo + ldexp((double)u, -16) * (hi - lo);
            return (a > t) ? k + 1 : k;
        }
    }
    return 7; /* unreachable for finite a */
}

/* Signed E2M1 code for a normalised value q (the sign of q, including the
 * sign of zero, is kept: reading R-5). */
int oracle_e2m1_round(double q, int rounding, unsigned u, int *sat)
{
    int s = signbit(q) ? 8 : 0;
    double a = fabs(q);
    int mag = rounding ? e2m1_stochastic_mag(a, u, sat) : e2m1_nearest_mag(a, sat);
    return s | mag;
}

/* Scaled-INT4 element of IF4 ([ABS] cues 14 and 17; reading R-22): the
 * integer k nearest to q with ties to the even integer, |k| <= 7; |q| > 7
 * clamps to 7 and counts as saturated.  The nibble is sign-magnitude like
 * an E2M1 code, sign << 3 | |k|, keeping the sign of q (also of zero). */
int oracle_int4_round(double q, int *sat)
{
    int s = signbit(q) ? 8 : 0, k;
    double a = fabs(q), fl;
    *sat = 0;
    if (a > 7.0) {
        *sat = 1;
        return s | 7;
    }
    fl = floor(a);
    k = (int)fl;
    if (a - fl > 0.5 || (a - fl == 0.5 && (k & 1))) k++; /* a - fl is exact */
    return s | k;
}

/* OCP max-based E8M0 exponent, [MXA] "Read the shared E8M0 scale":
 * e = floor(log2(amax / 4)), clamped to [-127, 127]; the all-zero block
 * takes exponent 0.  floor(log2) is read off frexp (exact), never libm log2
 * (reading R-6). */
int oracle_mx_exponent(double amax)
{
    int p, e;
    if (amax == 0.0) return 0;
    (void)frexp(amax, &p);  /* amax = f * 2^p, f in [0.5, 1) */
    e = (p - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: */
/* As Easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies, */
/* a word permutation and a Weyl-sequence key schedule (reading R-18).  */
/* ------------------------------------------------------------------ */
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    int r;
    for (r = 0; r < 10; r++) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* 16-bit stochastic-rounding draw for flat element index i (reading R-17):
 * field (i mod 8) of Philox(key = seed, counter = (i/8, 0, 0)) where field f
 * is bits 16*(f&1)..+15 of word f>>1. */
unsigned oracle_sr_draw(uint64_t seed, uint64_t i)
{
    uint32_t ctr[4], key[2], out[4];
    uint64_t g = i >> 3;
    int f = (int)(i & 7);
    ctr[0] = (uint32_t)g; ctr[1] = (uint32_t)(g >> 32); ctr[2] = 0; ctr[3] = 0;
    key[0] = (uint32_t)seed; key[1] = (uint32_t)(seed >> 32);
    oracle_philox4x32_10(ctr, key, out);
    return (out[f >> 1] >> (16 * (f & 1))) & 0xFFFFu;
}

/* Random sign for position j of a Hadamard block (readings R-16): bit
 * (j mod 32) of word (j/32 mod 4) of Philox(key = seed, counter =
 * (j/128, 0, 1, 0)); a set bit means -1. */
int oracle_rht_sign_negative(uint64_t seed, int64_t j)
{
    uint32_t ctr[4], key[2], out[4];
    ctr[0] = (uint32_t)(j >> 7); ctr[1] = 0; ctr[2] = 1; ctr[3] = 0;
    key[0] = (uint32_t)seed; key[1] = (uint32_t)(seed >> 32);
    oracle_philox4x32_10(ctr, key, out);
    return (int)((out[(j >> 5) & 3] >> (j & 31)) & 1u);
}

/* ------------------------------------------------------------------ */
/* Inputs                                                              */
/* ------------------------------------------------------------------ */
/* dtype 0: fp32, dtype 1: bf16 stored as its 16 raw bits, dtype 2: fp64. */
static double load_elem(const void *x, int dtype, int64_t idx)
{
    if (dtype == 0) return (double)((const float *)x)[idx];
    if (dtype == 2) return ((const double *)x)[idx];
    {
        uint32_t b = (uint32_t)((const uint16_t *)x)[idx] << 16;
        float f;
        memcpy(&f, &b, 4);
        return (double)f;
    }
}

static float load_elem_f32(const void *x, int dtype, int64_t idx)
{
    return (float)load_elem(x, dtype, idx);
}

static void counters_zero(uint64_t *c)
{
    if (c) c[0] = c[1] = c[2] = 0;
}

/* ------------------------------------------------------------------ */
/* MXFP4 quantize                                                      */
/* ------------------------------------------------------------------ */
/* [MXA] "Encode one MXFP4 block step by step": per block of 32 values along
 * a row, amax -> exponent -> scale byte e + 127 -> each value divided by
 * 2^e, rounded on the E2M1 lattice -> nibble; element 2k in the low half of
 * byte k ([MXA], same section, nibble packing).  Counters: [0] saturated,
 * [1] underflowed (a nonzero source reconstructs as zero), [2] non-finite
 * inputs; a block holding a non-finite value gets scale byte 0xFF and zero
 * codes (reading R-8).  policy 0 = OCP max rule, 1 = manual exponent.
 * rounding 0 = nearest-even, 1 = stochastic with draws keyed by the flat
 * element index r*cols + c. */
int oracle_quantize_mx(int64_t rows, int64_t cols, int64_t stride, int dtype, const void *x,
                       int policy, int manual_exponent, int rounding, uint64_t seed,
                       uint8_t *codes, uint8_t *scales, uint64_t *counters)
{
    int64_t r, b, i;
    const int B = 32;
    if (rows < 0 || cols < 0 || cols % B != 0 || stride < cols) return OR_BAD;
    if (policy == 1 && (manual_exponent < -127 || manual_exponent > 127)) return OR_BAD;
    counters_zero(counters);
    memset(codes, 0, (size_t)(rows * cols / 2));
    for (r = 0; r < rows; r++) {
        for (b = 0; b < cols / B; b++) {
            double v[32], amax = 0.0;
            int nonfinite = 0, e;
            for (i = 0; i < B; i++) {
                v[i] = load_elem(x, dtype, r * stride + b * B + i);
                if (!isfinite(v[i])) nonfinite++;
                else if (fabs(v[i]) > amax) amax = fabs(v[i]);
            }
            if (nonfinite) {
                scales[r * (cols / B) + b] = 0xFF;
                if (counters) counters[2] += (uint64_t)nonfinite;
                continue; /* codes stay 0 */
            }
            e = (policy == 1) ? manual_exponent : oracle_mx_exponent(amax);
            scales[r * (cols / B) + b] = (uint8_t)(e + 127);
            for (i = 0; i < B; i++) {
                int64_t flat = r * cols + b * B + i;
                double q = ldexp(v[i], -e); /* exact: power-of-two scaling */
                int sat;
                unsigned u = rounding ? oracle_sr_draw(seed, (uint64_t)flat) : 0;
                int code = oracle_e2m1_round(q, rounding, u, &sat);
                if (counters) {
                    counters[0] += (uint64_t)sat;
                    if (v[i] != 0.0 && (code & 7) == 0) counters[1]++;
                }
                codes[flat >> 1] |= (uint8_t)(code << (4 * (flat & 1)));
            }
        }
    }
    return OR_OK;
}

/* Largest finite |x| of a tensor (the NVFP4 per-tensor amax, reading R-10:
 * non-finite values are excluded). */
float oracle_tensor_amax(int64_t rows, int64_t cols, int64_t stride, int dtype, const void *x)
{
    int64_t r, i;
    float amax = 0.0f;
    for (r = 0; r < rows; r++)
        for (i = 0; i < cols; i++) {
            float f = load_elem_f32(x, dtype, r * stride + i);
            if (isfinite(f) && fabsf(f) > amax) amax = fabsf(f);
        }
    return amax;
}

/* ------------------------------------------------------------------ */
/* NVFP4 quantize (two-level) and Four-Over-Six                        */
/* ------------------------------------------------------------------ */
/* One candidate encoding of a 16-block under E4M3 scale byte sb and global
 * scale g.  The element quotient x / (s_dec * g) is evaluated in fp64,
 * which decides the nearest-even and stochastic roundings exactly (reading
 * R-12: s_dec * g is exact in fp64 and a non-tie quotient is at least
 * 2^-47 away, relatively, from any decision point).  Returns the codes and
 * per-block saturation / underflow counts. */
static void nv_encode_block(const double *v, int sb, float g, int rounding, uint64_t seed,
                            int64_t flat0, int *codes16, uint64_t *nsat, uint64_t *nunder)
{
    double sdec = oracle_e4m3_value(sb);
    double denom = sdec * (double)g; /* exact: 4 x 24 significant bits */
    int i;
    *nsat = 0;
    *nunder = 0;
    for (i = 0; i < 16; i++) {
        int sat = 0, code;
        if (sdec == 0.0) {
            code = signbit(v[i]) ? 8 : 0; /* a zero scale maps the block to signed zero */
        } else {
            unsigned u = rounding ? oracle_sr_draw(seed, (uint64_t)(flat0 + i)) : 0;
            code = oracle_e2m1_round(v[i] / denom, rounding, u, &sat);
        }
        codes16[i] = code;
        *nsat += (uint64_t)sat;
        if (v[i] != 0.0 && (code & 7) == 0) (*nunder)++;
    }
}

/* Block sum of squared reconstruction errors in the frozen fp32 order of
 * reading R-14: dq = fl32(fl32(value * s_dec) * g), d = fl32(x - dq),
 * S_lo = sequential fl32 sum of fl32(d*d) over elements 0..7, S_hi over
 * 8..15, SSE = fl32(S_lo + S_hi). */
static float block_sse_f32(const double *v, const int *codes16, int sb, float g)
{
    float sdec = (float)oracle_e4m3_value(sb);
    float slo = 0.0f, shi = 0.0f;
    int i;
    for (i = 0; i < 16; i++) {
        float vs = (float)oracle_e2m1_value(codes16[i]) * sdec;
        float dq = vs * g;
        float d = (float)v[i] - dq;
        float sq = d * d;
        if (i < 8) slo = slo + sq;
        else shi = shi + sq;
    }
    return slo + shi;
}

/* IF4's scaled-INT4 candidate ([ABS] cue 17; reading R-22) of a 16-block
 * under the block's NVFP4 scale byte sb: the element is the integer nearest
 * to q = x * 7 / (6 * s_dec * g), i.e. the INT4 grid is stretched by 7/6 so
 * that 7 lands where FP4's 6 does.  fp64 decides the rounding exactly: 7x
 * has at most 27 significant bits and 6 * s_dec * g at most 30, so a
 * quotient that is not a tie stays at least 2^-40 (relatively) away from
 * every half-integer.  A zero scale maps the block to signed zeros. */
static void int4_encode_block(const double *v, int sb, float g, int *codes16, uint64_t *nsat, uint64_t *nunder)
{
    double sdec = oracle_e4m3_value(sb);
    double denom = 6.0 * sdec * (double)g; /* exact */
    int i;
    *nsat = 0;
    *nunder = 0;
    for (i = 0; i < 16; i++) {
        int sat = 0, code;
        if (sdec == 0.0) code = signbit(v[i]) ? 8 : 0;
        else code = oracle_int4_round(7.0 * v[i] / denom, &sat);
        codes16[i] = code;
        *nsat += (uint64_t)sat;
        if (v[i] != 0.0 && (code & 7) == 0) (*nunder)++;
    }
}

/* Reconstruction of an INT4 nibble, k * 6 * s_dec * g / 7 (reading R-23).
 * The product is exact in fp64 (at most 33 significant bits); the fp64
 * quotient is never within 2^-33 (relatively) of an fp32 or bf16 rounding
 * boundary unless the exact value lies on it, so rounding it once more to
 * fp32 or bf16 gives the single rounding of the exact value. */
static double int4_recon(int code, double sdec, float g)
{
    double m = (double)(code & 7) * 6.0 * sdec * (double)g / 7.0;
    return (code & 8) ? -m : m;
}

/* The INT4 candidate's block SSE in the order of reading R-14, with
 * dq = fl32(k * 6 * s_dec * g / 7) in place of the FP4 reconstruction. */
static float block_sse_int4_f32(const double *v, const int *codes16, int sb, float g)
{
    double sdec = oracle_e4m3_value(sb);
    float slo = 0.0f, shi = 0.0f;
    int i;
    for (i = 0; i < 16; i++) {
        float dq = (float)int4_recon(codes16[i], sdec, g);
        float d = (float)v[i] - dq;
        float sq = d * d;
        if (i < 8) slo = slo + sq;
        else shi = shi + sq;
    }
    return slo + shi;
}

/* [SUB4] section 2: per-tensor fp32 scale g = amax / (6 * 448) and per 16-
 * block E4M3 scale s = RNE_E4M3(bamax / (6 g)); elements round to E2M1 after
 * dividing by s * g.  policy 2 = max->6, policy 3 = Four Over Six ([ABS]
 * cue 10): g = amax / (4 * 448), each block is encoded with both
 * s6 = RNE_E4M3(bamax / (6 g)) and s4 = RNE_E4M3(bamax / (4 g)) and keeps the
 * candidate with the lower block SSE (ties keep max->6); the choice bit of
 * flat block b = r * (cols/16) + j is bit (b mod 8) of byte b/8, 1 = max->4.
 * policy 4 = IF4 ([ABS] cues 14 and 17): g and s as for max->6; each
 * block is also encoded as scaled INT4 (int4_encode_block) and keeps the
 * candidate with the lower block SSE, ties keeping FP4 (reading R-24); an
 * INT4 block sets bit 7 of its scale byte.  Round to nearest only.
 * global_amax (optional) replaces the in-call tensor amax.  amax excludes
 * non-finite values; amax 0 gives g = 1 (reading R-10); a nonzero amax whose
 * g would underflow to 0 takes g = 2^-149 (reading R-21).  A block holding a
 * non-finite value gets scale byte 0x7F, zero codes and choice bit 0. */
int oracle_quantize_nv(int64_t rows, int64_t cols, int64_t stride, int dtype, const void *x,
                       int policy, int rounding, uint64_t seed, const float *global_amax,
                       uint8_t *codes, uint8_t *scales, float *global_scale,
                       uint8_t *choice_bits, uint64_t *counters)
{
    int64_t r, b, i, nb = cols / 16;
    float amax = 0.0f, g, denom_mult;
    const int fos = (policy == 3), if4 = (policy == 4);
    if (rows < 0 || cols < 0 || cols % 16 != 0 || stride < cols) return OR_BAD;
    if (policy != 2 && policy != 3 && policy != 4) return OR_BAD;
    if (if4 && rounding) return OR_BAD;
    if (fos && !choice_bits) return OR_BAD;
    counters_zero(counters);
    memset(codes, 0, (size_t)(rows * cols / 2));
    if (fos) memset(choice_bits, 0, (size_t)((rows * nb + 7) / 8));
    amax = global_amax ? *global_amax : oracle_tensor_amax(rows, cols, stride, dtype, x);
    denom_mult = fos ? 4.0f : 6.0f;
    if (amax == 0.0f) {
        g = 1.0f;
    } else {
        g = amax / (denom_mult * 448.0f); /* correctly rounded fp32 division */
        if (g == 0.0f) g = ldexpf(1.0f, -149);
    }
    *global_scale = g;
    for (r = 0; r < rows; r++) {
        for (b = 0; b < nb; b++) {
            double v[16], bamax = 0.0;
            int nonfinite = 0, c6[16], c4[16], ci[16], *chosen, sb, sb6, sb4, pick4 = 0;
            uint64_t sat6, und6, sat4 = 0, und4 = 0, sat, und;
            int64_t flat0 = r * cols + b * 16, fb = r * nb + b;
            for (i = 0; i < 16; i++) {
                v[i] = load_elem(x, dtype, r * stride + b * 16 + i);
                if (!isfinite(v[i])) nonfinite++;
                else if (fabs(v[i]) > bamax) bamax = fabs(v[i]);
            }
            if (nonfinite) {
                scales[fb] = 0x7F;
                if (counters) counters[2] += (uint64_t)nonfinite;
                continue;
            }
            /* bamax / (6 g) in fp64: 6 g is exact and the E4M3 decision
             * points are at least 2^-31 away (relatively) from a non-tie
             * quotient, so fp64 division decides the rounding exactly. */
            sb6 = oracle_e4m3_encode(bamax / (6.0 * (double)g));
            nv_encode_block(v, sb6, g, rounding, seed, flat0, c6, &sat6, &und6);
            chosen = c6; sb = sb6; sat = sat6; und = und6;
            if (fos) {
                float sse6, sse4;
                sb4 = oracle_e4m3_encode(bamax / (4.0 * (double)g));
                nv_encode_block(v, sb4, g, rounding, seed, flat0, c4, &sat4, &und4);
                sse6 = block_sse_f32(v, c6, sb6, g);
                sse4 = block_sse_f32(v, c4, sb4, g);
                if (sse4 < sse6) {
                    pick4 = 1;
                    chosen = c4; sb = sb4; sat = sat4; und = und4;
                }
                if (pick4) choice_bits[fb >> 3] |= (uint8_t)(1u << (fb & 7));
            }
            if (if4) {
                uint64_t sati, undi;
                float ssef, ssei;
                int4_encode_block(v, sb6, g, ci, &sati, &undi);
                ssef = block_sse_f32(v, c6, sb6, g);
                ssei = block_sse_int4_f32(v, ci, sb6, g);
                if (ssei < ssef) {
                    chosen = ci; sb = sb6 | 0x80; sat = sati; und = undi;
                }
            }
            scales[fb] = (uint8_t)sb;
            if (counters) {
                counters[0] += sat;
                counters[1] += und;
            }
            for (i = 0; i < 16; i++) {
                int64_t flat = flat0 + i;
                codes[flat >> 1] |= (uint8_t)(chosen[i] << (4 * (flat & 1)));
            }
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Walsh-Hadamard rotation                                             */
/* ------------------------------------------------------------------ */
/* [SUB4] section 3: y = x * H_t / sqrt(t) with H_t the Sylvester Hadamard
 * matrix (entries +-1, H[i][j] = (-1)^popcount(i & j)), applied to each
 * consecutive t-chunk of every row (t = d: full-row FWHT; t = 16: the
 * 16-point block transform).  With random_signs, x is first multiplied by
 * the seeded +-1 diagonal ([ABS] cue 8, reading R-16).  fp64 butterfly; the
 * output is fp64. */
int oracle_fwht(int64_t rows, int64_t d, int64_t stride, int dtype, const void *x,
                double *y, int64_t t, int random_signs, uint64_t seed)
{
    int64_t r, c0, i, h, j;
    double norm;
    if (rows < 0 || d <= 0 || t <= 0 || (t & (t - 1)) != 0 || d % t != 0 || stride < d) return OR_BAD;
    norm = 1.0 / sqrt((double)t);
    for (r = 0; r < rows; r++) {
        for (c0 = 0; c0 < d; c0 += t) {
            double *w = y + r * d + c0;
            for (i = 0; i < t; i++) {
                double v = load_elem(x, dtype, r * stride + c0 + i);
                if (random_signs && oracle_rht_sign_negative(seed, i)) v = -v;
                w[i] = v;
            }
            for (h = 1; h < t; h <<= 1)
                for (i = 0; i < t; i += 2 * h)
                    for (j = i; j < i + h; j++) {
                        double a = w[j], bb = w[j + h];
                        w[j] = a + bb;
                        w[j + h] = a - bb;
                    }
            for (i = 0; i < t; i++) w[i] *= norm;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* MXFP4 GEMM                                                          */
/* ------------------------------------------------------------------ */
/* The consumer of two MXFP4 tensors ([SUB4] section 3: Y = X W^T with both
 * operands quantized): C[m][n] = sum_k A[m][k] B[n][k] over the
 * reconstructed values (value * 2^(b - 127), [MXA] "Encode one MXFP4 block
 * step by step"), A [M][K] and B [N][K] in the quantizer's layout (codes
 * [rows][K/2], scales [rows][K/32]).  Every product is exact in fp64 and the
 * sum is taken in fp64 in k order (reading R-27); absc[m][n] = sum_k
 * |A[m][k] B[n][k]| bounds the rounding of any other summation order.  A NaN
 * scale code (255) makes its terms NaN.  rows0/nrows select the rows of A
 * (and of C) to compute. */
int oracle_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t *a_codes, const uint8_t *a_scales,
                   const uint8_t *b_codes, const uint8_t *b_scales, int64_t row0, int64_t nrows,
                   double *c, double *absc)
{
    int64_t m, n, k;
    double *arow, *brow;
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || row0 < 0 || nrows < 0 || row0 + nrows > M) return OR_BAD;
    arow = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    brow = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    if (!arow || !brow) {
        free(arow);
        free(brow);
        return OR_BAD;
    }
    for (m = row0; m < row0 + nrows; m++) {
        for (k = 0; k < K; k++) {
            int code = (a_codes[m * (K / 2) + k / 2] >> (4 * (k & 1))) & 15;
            int sb = a_scales[m * (K / 32) + k / 32];
            arow[k] = sb == 255 ? NAN : oracle_e2m1_value(code) * oracle_e8m0_value(sb);
        }
        for (n = 0; n < N; n++) {
            double s = 0.0, sa = 0.0;
            for (k = 0; k < K; k++) {
                int code = (b_codes[n * (K / 2) + k / 2] >> (4 * (k & 1))) & 15;
                int sb = b_scales[n * (K / 32) + k / 32];
                brow[k] = sb == 255 ? NAN : oracle_e2m1_value(code) * oracle_e8m0_value(sb);
                s += arow[k] * brow[k];
                sa += fabs(arow[k] * brow[k]);
            }
            c[(m - row0) * N + n] = s;
            if (absc) absc[(m - row0) * N + n] = sa;
        }
    }
    free(arow);
    free(brow);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* SiLU_and_Mul                                                        */
/* ------------------------------------------------------------------ */
/* [SUB4] section 3, the online rotation fused into the SwiGLU epilogue
 * before down_proj: the activation is h = SiLU(gate) * up with
 * SiLU(g) = g / (1 + e^-g) (reading R-25), here in fp64 with libm exp, one
 * value per (row, column) of two [rows][stride] inputs of dtype 0/1; the
 * result is a dense [rows][cols] fp64 array. */
int oracle_silu_mul(int64_t rows, int64_t cols, int64_t stride, int dtype, const void *gate,
                    const void *up, double *out)
{
    int64_t r, c;
    if (rows < 0 || cols < 0 || stride < cols || (dtype != 0 && dtype != 1)) return OR_BAD;
    for (r = 0; r < rows; r++)
        for (c = 0; c < cols; c++) {
            double g = load_elem(gate, dtype, r * stride + c);
            double u = load_elem(up, dtype, r * stride + c);
            out[r * cols + c] = g / (1.0 + exp(-g)) * u;
        }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Dequantize                                                          */
/* ------------------------------------------------------------------ */
/* Round a double to the nearest bf16 (8 significant bits, min normal
 * 2^-126, min subnormal 2^-133), ties to even; returns the 16 bits. */
static uint16_t to_bf16_bits(double v)
{
    double r;
    float f;
    uint32_t u;
    if (isnan(v)) return 0x7FC0;
    if (v == 0.0 || isinf(v)) {
        r = v;
    } else {
        int e;
        (void)frexp(v, &e); /* |v| in [2^(e-1), 2^e) */
        if (e - 1 >= -126) r = ldexp(rint(ldexp(v, 8 - e)), e - 8);
        else r = ldexp(rint(ldexp(v, 133)), -133);
        if (fabs(r) >= ldexp(1.0, 128)) r = copysign(INFINITY, v);
    }
    f = (float)r; /* exact: r is a bf16 value */
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* [MXA] "Encode one MXFP4 block step by step": reconstruction multiplies
 * the lattice value back by the scale.  MX: value * 2^(b - 127) (exact).
 * NV: value * s_dec * g, exact in fp64, rounded once to the output type
 * (reading R-13).  IF4 (format 2): a scale byte with bit 7 set marks an
 * INT4 block, whose value is k * 6 * s_dec * g / 7 rounded once (reading
 * R-23), s_dec from the low 7 bits; otherwise as NV.  A NaN scale code
 * yields NaN for its block.  format 0 = MX (block 32), 1 = NV and 2 = IF4
 * (block 16); out_dtype 0 fp32, 1 bf16. */
int oracle_dequantize(int format, int64_t rows, int64_t cols, int block,
                      const uint8_t *codes, const uint8_t *scales, const float *global_scale,
                      int out_dtype, void *out)
{
    int64_t r, c;
    if (rows < 0 || cols < 0 || block <= 0 || cols % block != 0) return OR_BAD;
    if (format < 0 || format > 2) return OR_BAD;
    if ((format == 0 && block != 32) || (format != 0 && (block != 16 || !global_scale))) return OR_BAD;
    for (r = 0; r < rows; r++)
        for (c = 0; c < cols; c++) {
            int64_t flat = r * cols + c;
            int code = (codes[flat >> 1] >> (4 * (flat & 1))) & 15;
            int sb = scales[r * (cols / block) + c / block];
            double v;
            if (format == 0) {
                v = (sb == 255) ? NAN : oracle_e2m1_value(code) * oracle_e8m0_value(sb);
            } else if (format == 2 && (sb & 0x80)) {
                double sdec = oracle_e4m3_value(sb & 0x7F);
                v = isnan(sdec) ? NAN : int4_recon(code, sdec, *global_scale);
            } else {
                double sdec = oracle_e4m3_value(format == 2 ? (sb & 0x7F) : sb);
                v = isnan(sdec) ? NAN : oracle_e2m1_value(code) * sdec * (double)(*global_scale);
            }
            if (out_dtype == 0) ((float *)out)[flat] = (float)v;
            else ((uint16_t *)out)[flat] = to_bf16_bits(v);
        }
    return OR_OK;
}

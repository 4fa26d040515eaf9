/*
 * oracle.c -- plain, slow CPU reference for the routed-expert forward of an MXFP4 Stable
 * LatentMoE layer (Kimi K3 / K3.1).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls this file; only
 * the tests, the smoke check and the bench's CPU-baseline leg do. It shares no code, header,
 * table or constant with the HIP library.
 *
 * Arithmetic: every sum is accumulated in IEEE double in index order; BF16 rounding is a
 * single round-to-nearest-even from the double value; no fast-math, no FMA contraction
 * (built with -ffp-contract=off). OpenMP splits work over tokens (or token/expert pairs);
 * each output element is produced by one thread in a fixed order, so results do not depend
 * on the thread count.
 *
 * Sources (cited by page title and section):
 *  [K31] "Kimi K3.1 Pro on AMD Instinct GPUs", section "Kimi K3.1 Pro at a glance": 896 routed
 *        experts, 16 active per token, plus two shared experts; sigmoid routing; routed experts
 *        work in a 3584-wide latent (half of the 7168 hidden width) with a GLU activation;
 *        routed experts in MXFP4 with one E8M0 scale per 32 values; router, shared experts and
 *        latent up/down projections in BF16.
 *  [K3A] "Day 0 Kimi-K3 Inference Deployment with ATOM on AMD Instinct MI355X GPUs",
 *        section "Model Architecture": Stable LatentMoE projects the 7168-wide hidden state
 *        down to 3584 before the experts; expert intermediate 3072.
 *  [K3W] same article, section "HBM Usage Under TP8": every rank keeps all expert IDs, each
 *        expert's matrices are split (gate/up by column, down by row), router and latent
 *        down/up are replicated.
 * Readings where the pages are silent (each also listed in the design notes):
 *  R1  E2M1 bit map and nibble order follow the OCP Microscaling (MX) v1.0 format: bit 3 sign,
 *      bits 2..1 exponent with bias 1, bit 0 mantissa; element 2i is the low nibble of byte i.
 *  R2  The 32-value scale block runs along each weight row's reduction (input) axis.
 *  R3  "SiTU-GLU" is not defined on the pages; the GLU reads h = silu(g) * u, silu(g) = g*sigmoid(g).
 *  R4  Selection ranks experts by the FP32/FP64 router logit (plus optional per-expert bias),
 *      descending, ties to the lower expert index; gate weights are the sigmoid of the selected
 *      logits divided by their sum; no scaling factor, no capacity limit, no dropped tokens.
 *  R5  Shared experts read the hidden state x and add to the output after the up-projection.
 *  R6  BF16 rounding points: z, h, y (unweighted expert output), the combined latent zc,
 *      the shared-expert GLU output h_s and the final output; y_s is not rounded.
 *  R7  "Stable" adds nothing to the arithmetic: the down and up projections are plain linears.
 *
 * Parity status per function is stated in the design notes; the function-level pins live in
 * tests/test_oracle_*.py.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads an OpenMP region of the oracle uses (reported with its timings). */
int or_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- number formats ---------- */

/* BF16 bit pattern -> exact double. */
double or_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* double -> BF16 bit pattern, one round-to-nearest-even step from the double value.
 * BF16 keeps 8 significant bits, normal exponents -126..127, subnormal quantum 2^-133. */
uint16_t or_double_to_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    if (v == 0.0)
        return signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v), r;
    if (isinf(a)) {
        r = a;
    } else {
        int e;
        frexp(a, &e);                    /* a = m * 2^e, 0.5 <= m < 1 */
        int q = e - 8;                   /* quantum exponent for 8 significant bits */
        if (q < -133)
            q = -133;                    /* subnormal range */
        r = ldexp(nearbyint(ldexp(a, -q)), q);   /* exact scaling, RNE at the quantum */
        if (r >= ldexp(1.0, 128))
            r = INFINITY;                /* overflow past the largest finite BF16 */
    }
    float f = (float)r;                  /* r is a BF16 value, hence exact in float */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t b = (uint16_t)(u >> 16);
    return signbit(v) ? (uint16_t)(b | 0x8000) : b;
}

/* O1a. E2M1 value of a 4-bit code (R1). */
double or_e2m1(int code)
{
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

/* O1b. E8M0 scale: 2^(e-127); the code 255 is NaN. */
double or_e8m0(int e)
{
    if (e == 255)
        return NAN;
    return ldexp(1.0, e - 127);
}

/* Element k of row n of an MX matrix with K columns: codes [N, K/2], scales [N, K/32]. */
static double mx_elem(const uint8_t *codes, const uint8_t *scales, int64_t K, int64_t n, int64_t k)
{
    uint8_t byte = codes[n * (K / 2) + k / 2];
    int code = (k & 1) ? (byte >> 4) : (byte & 0xF);
    return or_e2m1(code) * or_e8m0(scales[n * (K / 32) + k / 32]);
}

/* O1. Dequantise an MX matrix [N, K] to double. */
void or_dequant(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K, double *out)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            out[n * K + k] = mx_elem(codes, scales, K, n, k);
}

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* ---------------------------------------------------------------- routing ----------------- */

/* O2. Router logits: l[t,e] = sum_k x[t,k] * Wr[e,k] (+ bias[e]).  x [T,Hin], Wr [E,Hin]. */
void or_logits(const uint16_t *x, int64_t T, int64_t Hin, const uint16_t *wr, int64_t E,
               const float *bias, double *logits)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++)
        for (int64_t e = 0; e < E; e++) {
            double acc = 0.0;
            for (int64_t k = 0; k < Hin; k++)
                acc += or_bf16_to_double(x[t * Hin + k]) * or_bf16_to_double(wr[e * Hin + k]);
            if (bias)
                acc += (double)bias[e];
            logits[t * E + e] = acc;
        }
}

/* O3. Top-K selection (R4): K passes, each taking the largest remaining logit, ties to the
 * lower index. ids[t, j] is the expert of rank j. */
void or_select(const double *logits, int64_t T, int64_t E, int64_t K, int32_t *ids)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        const double *l = logits + t * E;
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        for (int64_t j = 0; j < K; j++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++) {
                if (taken[e])
                    continue;
                if (best < 0 || l[e] > l[best])   /* strict: an equal later index never wins */
                    best = e;
            }
            taken[best] = 1;
            ids[t * K + j] = (int32_t)best;
        }
        free(taken);
    }
}

/* O4. Gate weights: s_j = sigmoid(l[t, ids[t,j]]), w_j = s_j / sum_i s_i. */
void or_route_weights(const double *logits, const int32_t *ids, int64_t T, int64_t E, int64_t K,
                      double *w)
{
    for (int64_t t = 0; t < T; t++) {
        double sum = 0.0;
        for (int64_t j = 0; j < K; j++)
            sum += sigmoid(logits[t * E + ids[t * K + j]]);
        for (int64_t j = 0; j < K; j++)
            w[t * K + j] = sigmoid(logits[t * E + ids[t * K + j]]) / sum;
    }
}

/* O5. Group token/expert pairs by expert. Pair p = t*K + j. counts[e] = pairs routed to e;
 * offsets = exclusive prefix sum (offsets[E] = T*K); sorted_pairs lists pair ids grouped by
 * expert, ascending within an expert; inv[p] = row of p in sorted_pairs. */
void or_permute(const int32_t *ids, int64_t T, int64_t K, int64_t E, int32_t *counts,
                int32_t *offsets, int32_t *sorted_pairs, int32_t *inv)
{
    int64_t P = T * K;
    memset(counts, 0, (size_t)E * sizeof(int32_t));
    for (int64_t p = 0; p < P; p++)
        counts[ids[p]]++;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; e++)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int64_t p = 0; p < P; p++) {
        int32_t e = ids[p];
        int32_t row = offsets[e] + fill[e]++;
        sorted_pairs[row] = (int32_t)p;
        inv[p] = row;
    }
    free(fill);
}

/* ---------------------------------------------------------------- dense parts ------------- */

/* O6. Latent down-projection: z = bf16(x . Wdn^T).  x [T,H], Wdn [Lt,H], z [T,Lt]. */
void or_latent_down(const uint16_t *x, int64_t T, int64_t H, const uint16_t *wdn, int64_t Lt,
                    uint16_t *z)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++)
        for (int64_t n = 0; n < Lt; n++) {
            double acc = 0.0;
            for (int64_t k = 0; k < H; k++)
                acc += or_bf16_to_double(x[t * H + k]) * or_bf16_to_double(wdn[n * H + k]);
            z[t * Lt + n] = or_double_to_bf16(acc);
        }
}

/* O9. Shared experts (R3, R5, R6): h_s = bf16(silu(x.Wg_s^T) * (x.Wu_s^T)), y_s = h_s . Wd_s^T.
 * x [T,H]; sg, su [S,Is,H]; sd [S,H,Is]. hs [T, S*Is] (bf16, nullable); ys [T,H] = sum_s y_s. */
void or_shared(const uint16_t *x, int64_t T, int64_t H, const uint16_t *sg, const uint16_t *su,
               const uint16_t *sd, int64_t S, int64_t Is, uint16_t *hs, double *ys)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        double *h = (double *)malloc((size_t)(S * Is) * sizeof(double));
        for (int64_t s = 0; s < S; s++)
            for (int64_t j = 0; j < Is; j++) {
                double g = 0.0, u = 0.0;
                for (int64_t k = 0; k < H; k++) {
                    double xv = or_bf16_to_double(x[t * H + k]);
                    g += xv * or_bf16_to_double(sg[(s * Is + j) * H + k]);
                    u += xv * or_bf16_to_double(su[(s * Is + j) * H + k]);
                }
                uint16_t hb = or_double_to_bf16(g * sigmoid(g) * u);
                if (hs)
                    hs[t * S * Is + s * Is + j] = hb;
                h[s * Is + j] = or_bf16_to_double(hb);
            }
        for (int64_t n = 0; n < H; n++) {
            double acc = 0.0;
            for (int64_t s = 0; s < S; s++)
                for (int64_t j = 0; j < Is; j++)
                    acc += h[s * Is + j] * or_bf16_to_double(sd[(s * H + n) * Is + j]);
            ys[t * H + n] = acc;
        }
        free(h);
    }
}

/* O10. Output: out = bf16(zc . Wup^T + ys).  zc [T,Lt], Wup [H,Lt], ys [T,H] (nullable). */
void or_output(const uint16_t *zc, int64_t T, int64_t Lt, const uint16_t *wup, int64_t H,
               const double *ys, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++)
        for (int64_t n = 0; n < H; n++) {
            double acc = 0.0;
            for (int64_t k = 0; k < Lt; k++)
                acc += or_bf16_to_double(zc[t * Lt + k]) * or_bf16_to_double(wup[n * Lt + k]);
            if (ys)
                acc += ys[t * H + n];
            out[t * H + n] = or_double_to_bf16(acc);
        }
}

/* ---------------------------------------------------------------- routed experts ---------- */

/* O7. Routed GLU experts for every pair p = t*K + j with e = ids[p] (R2, R3, R6):
 *   g = z_t . Wg_e^T, u = z_t . Wu_e^T, h = bf16(silu(g) * u), y_p = bf16(h . Wd_e^T).
 * z [T,Lt] bf16; gate/up codes [E,I,Lt/2], scales [E,I,Lt/32]; down codes [E,Lt,I/2],
 * scales [E,Lt,I/32]. h [T*K, I] (nullable) and y [T*K, Lt], both indexed by pair id. */
void or_experts(const uint16_t *z, int64_t T, int64_t Lt, const int32_t *ids, int64_t K,
                int64_t I, const uint8_t *gate_codes, const uint8_t *gate_scales,
                const uint8_t *up_codes, const uint8_t *up_scales, const uint8_t *down_codes,
                const uint8_t *down_scales, uint16_t *h_out, uint16_t *y_out)
{
    const int64_t gcb = I * (Lt / 2), gsb = I * (Lt / 32);   /* per-expert bytes, gate/up */
    const int64_t dcb = Lt * (I / 2), dsb = Lt * (I / 32);   /* per-expert bytes, down */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < T * K; p++) {
        int64_t t = p / K, e = ids[p];
        double *zt = (double *)malloc((size_t)Lt * sizeof(double));
        double *h = (double *)malloc((size_t)I * sizeof(double));
        for (int64_t k = 0; k < Lt; k++)
            zt[k] = or_bf16_to_double(z[t * Lt + k]);
        for (int64_t j = 0; j < I; j++) {
            double g = 0.0, u = 0.0;
            for (int64_t k = 0; k < Lt; k++) {
                g += zt[k] * mx_elem(gate_codes + e * gcb, gate_scales + e * gsb, Lt, j, k);
                u += zt[k] * mx_elem(up_codes + e * gcb, up_scales + e * gsb, Lt, j, k);
            }
            uint16_t hb = or_double_to_bf16(g * sigmoid(g) * u);
            if (h_out)
                h_out[p * I + j] = hb;
            h[j] = or_bf16_to_double(hb);
        }
        for (int64_t n = 0; n < Lt; n++) {
            double acc = 0.0;
            for (int64_t j = 0; j < I; j++)
                acc += h[j] * mx_elem(down_codes + e * dcb, down_scales + e * dsb, I, n, j);
            y_out[p * Lt + n] = or_double_to_bf16(acc);
        }
        free(zt);
        free(h);
    }
}

/* O7b. The down half of O7 on given h: y_p = bf16(h_p . Wd_e^T) for every pair p with e = ids[p].
 * h [T*K, I] bf16 by pair id; y [T*K, Lt]. (Used to check a down product on its own inputs.) */
void or_expert_down(const uint16_t *h, int64_t T, int64_t K, int64_t I, int64_t Lt, const int32_t *ids,
                    const uint8_t *down_codes, const uint8_t *down_scales, uint16_t *y_out)
{
    const int64_t dcb = Lt * (I / 2), dsb = Lt * (I / 32);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < T * K; p++) {
        const int64_t e = ids[p];
        for (int64_t n = 0; n < Lt; n++) {
            double acc = 0.0;
            for (int64_t j = 0; j < I; j++)
                acc += or_bf16_to_double(h[p * I + j]) * mx_elem(down_codes + e * dcb, down_scales + e * dsb, I, n, j);
            y_out[p * Lt + n] = or_double_to_bf16(acc);
        }
    }
}

/* ---------------------------------------------------- FP8 second stage (opt-in mode) ---------
 * [K31-opt] ("Kimi K3.1 Pro on AMD Instinct GPUs", section "What we optimized", and its
 * "Appendix: environment variables") runs the routed experts' second stage -- the down
 * product -- in FP8. The pages fix neither the FP8 format nor the scale granularity; reading F1:
 *  F1  h is quantised per pair row in blocks of 32 consecutive values along I (the down
 *      product's input axis, the same blocks as the weights' scales) to OCP MX FP8: E4M3
 *      elements with one E8M0 block scale 2^X. X follows the OCP MX v1.0 conversion rule,
 *      X = floor(log2(max |h| over the block)) - 8 (8 = exponent of E4M3's largest normal),
 *      clamped to [-127, 127]; an all-zero block takes X = -127. Each element h / 2^X is
 *      rounded to nearest even at E4M3's precision (4 significant bits, subnormal quantum 2^-9)
 *      and saturates at +-448; its sign bit is kept (also for zero).
 *  F2  The down product then reads the dequantised values: y_p = bf16(sum_j q_j 2^X_j . Wd[n][j]).
 */

/* O10a. E4M3 (OCP, "FN": no infinities) value of an 8-bit code: bit 7 sign, bits 6..3 exponent
 * (bias 7), bits 2..0 mantissa; exponent field 0 is subnormal (m/8 . 2^-6); S.1111.111 is NaN. */
double or_e4m3(int code)
{
    int sign = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7)
        return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* E4M3 code of |a| (a >= 0, finite) rounded to nearest even, saturating at 448; sign added by caller. */
static int e4m3_round(double a)
{
    if (a == 0.0)
        return 0;
    int ex;
    frexp(a, &ex);                       /* a = m 2^ex, 0.5 <= m < 1: leading bit at 2^(ex-1) */
    int q = ex - 1 - 3;                  /* quantum for 4 significant bits */
    if (q < -9)
        q = -9;                          /* subnormal range */
    double r = ldexp(nearbyint(ldexp(a, -q)), q);
    if (r > 448.0)
        r = 448.0;
    /* encode r: find the code whose value is r (codes are monotone in magnitude) */
    for (int c = 0; c <= 0x7E; c++)
        if (or_e4m3(c) == r)
            return c;
    return -1;                           /* unreachable: r is an E4M3 value */
}

/* O10b. MX FP8 quantisation of h [R, I] bf16 (I a multiple of 32) per F1: codes u8 [R, I] and
 * scale bytes u8 [R, I/32] (E8M0, 2^(code-127)). */
void or_fp8_quant(const uint16_t *h, int64_t R, int64_t I, uint8_t *codes, uint8_t *scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++)
        for (int64_t b = 0; b < I / 32; b++) {
            const uint16_t *v = h + r * I + b * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; i++) {
                double a = fabs(or_bf16_to_double(v[i]));
                if (a > amax)
                    amax = a;
            }
            int X = -127;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);        /* floor(log2 amax) = ex - 1 */
                X = ex - 1 - 8;
                if (X < -127)
                    X = -127;
                if (X > 127)
                    X = 127;
            }
            scales[r * (I / 32) + b] = (uint8_t)(X + 127);
            for (int i = 0; i < 32; i++) {
                double x = or_bf16_to_double(v[i]);
                int c = e4m3_round(ldexp(fabs(x), -X));
                codes[r * I + b * 32 + i] = (uint8_t)(c | ((v[i] & 0x8000) ? 0x80 : 0));
            }
        }
}

/* O10c. The FP8 second stage on given quantised h (F2): y_p = bf16(sum_j q_pj 2^X . Wd_e[n][j]) for
 * every pair p with e = ids[p]. codes [T*K, I], scales [T*K, I/32] by pair id; y [T*K, Lt]. */
void or_expert_down_fp8(const uint8_t *hq, const uint8_t *hs, int64_t T, int64_t K, int64_t I, int64_t Lt,
                        const int32_t *ids, const uint8_t *down_codes, const uint8_t *down_scales, uint16_t *y_out)
{
    const int64_t dcb = Lt * (I / 2), dsb = Lt * (I / 32);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < T * K; p++) {
        const int64_t e = ids[p];
        double *hv = (double *)malloc((size_t)I * sizeof(double));
        for (int64_t j = 0; j < I; j++)
            hv[j] = or_e4m3(hq[p * I + j]) * or_e8m0(hs[p * (I / 32) + j / 32]);
        for (int64_t n = 0; n < Lt; n++) {
            double acc = 0.0;
            for (int64_t j = 0; j < I; j++)
                acc += hv[j] * mx_elem(down_codes + e * dcb, down_scales + e * dsb, I, n, j);
            y_out[p * Lt + n] = or_double_to_bf16(acc);
        }
        free(hv);
    }
}

/* ------------------------------------------------- MXFP4 first stage (opt-in mode, A4W4) -------
 * [K31-opt] ("Kimi K3.1 Pro on AMD Instinct GPUs", section "What we optimized", and its appendix of
 * environment variables) names an A4W4 mode of the grouped MoE: activations in 4-bit MX as well as
 * the weights. The pages fix neither the activation format's scale rule nor its rounding; reading
 * A1, the same conversion rule as F1 with the E2M1 element:
 *  A1  z is quantised per token row in blocks of 32 consecutive values along Lt (the first stage's
 *      input axis, the same blocks as the gate/up weights' scales) to OCP MX FP4: E2M1 elements
 *      with one E8M0 block scale 2^X, X = floor(log2(max |z| over the block)) - 2 (2 = exponent of
 *      E2M1's largest normal, 6 = 1.5 . 2^2), clamped to [-127, 127]; an all-zero block takes
 *      X = -127. Each element z / 2^X is rounded to nearest even at E2M1's precision (2 significant
 *      bits, subnormal quantum 1/2) and saturates at +-6; its sign bit is kept (also for zero).
 *      Codes are packed as the weights are: element 2i in the low nibble of byte i.
 *  A2  The gate/up product then reads the dequantised values: g = sum_k q_k 2^X_k . Wg[j][k] (and
 *      u likewise), h = bf16(silu(g) u); everything after h is unchanged.
 */

/* E2M1 code of |a| (a >= 0, finite) rounded to nearest even, saturating at 6; sign added by caller. */
static int e2m1_round(double a)
{
    if (a == 0.0)
        return 0;
    int ex;
    frexp(a, &ex);                       /* leading bit of a at 2^(ex-1) */
    int q = ex - 1 - 1;                  /* quantum for 2 significant bits */
    if (q < -1)
        q = -1;                          /* subnormal range: quantum 1/2 */
    double r = ldexp(nearbyint(ldexp(a, -q)), q);
    if (r > 6.0)
        r = 6.0;
    for (int c = 0; c <= 7; c++)         /* codes 0..7 are monotone in magnitude */
        if (or_e2m1(c) == r)
            return c;
    return -1;                           /* unreachable: r is an E2M1 value */
}

/* O11a. MX FP4 quantisation of z [R, L] bf16 (L a multiple of 32) per A1: codes u8 [R, L/2] (two
 * per byte, element 2i low) and scale bytes u8 [R, L/32]. */
void or_fp4_quant(const uint16_t *z, int64_t R, int64_t L, uint8_t *codes, uint8_t *scales)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++)
        for (int64_t b = 0; b < L / 32; b++) {
            const uint16_t *v = z + r * L + b * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; i++) {
                double a = fabs(or_bf16_to_double(v[i]));
                if (a > amax)
                    amax = a;
            }
            int X = -127;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);        /* floor(log2 amax) = ex - 1 */
                X = ex - 1 - 2;
                if (X < -127)
                    X = -127;
                if (X > 127)
                    X = 127;
            }
            scales[r * (L / 32) + b] = (uint8_t)(X + 127);
            for (int i = 0; i < 32; i += 2) {
                int c0 = e2m1_round(ldexp(fabs(or_bf16_to_double(v[i])), -X)) | ((v[i] & 0x8000) ? 8 : 0);
                int c1 = e2m1_round(ldexp(fabs(or_bf16_to_double(v[i + 1])), -X)) | ((v[i + 1] & 0x8000) ? 8 : 0);
                codes[r * (L / 2) + (b * 32 + i) / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
}

/* O11b. The A4W4 first stage on given quantised z (A2): for every pair p = t*K + j with
 * e = ids[p], h_p = bf16(silu(g) u), g = zq_t . Wg_e^T, u = zq_t . Wu_e^T, zq the dequantised
 * MX FP4 row of token t. zc codes [T, Lt/2], scales [T, Lt/32]; h [T*K, I] by pair id. */
void or_expert_gateup_a4(const uint8_t *zq, const uint8_t *zs, int64_t T, int64_t Lt, const int32_t *ids, int64_t K,
                         int64_t I, const uint8_t *gate_codes, const uint8_t *gate_scales, const uint8_t *up_codes,
                         const uint8_t *up_scales, uint16_t *h_out)
{
    const int64_t gcb = I * (Lt / 2), gsb = I * (Lt / 32);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < T * K; p++) {
        const int64_t t = p / K, e = ids[p];
        double *zt = (double *)malloc((size_t)Lt * sizeof(double));
        for (int64_t k = 0; k < Lt; k++)
            zt[k] = mx_elem(zq, zs, Lt, t, k);
        for (int64_t j = 0; j < I; j++) {
            double g = 0.0, u = 0.0;
            for (int64_t k = 0; k < Lt; k++) {
                g += zt[k] * mx_elem(gate_codes + e * gcb, gate_scales + e * gsb, Lt, j, k);
                u += zt[k] * mx_elem(up_codes + e * gcb, up_scales + e * gsb, Lt, j, k);
            }
            h_out[p * I + j] = or_double_to_bf16(g * sigmoid(g) * u);
        }
        free(zt);
    }
}

/* O9b. The down half of O9 on given h_s: ys[t] = sum_s h_s[t] . Wd_s^T (FP64, not rounded).
 * hs [T, S*Is] bf16; sd [S,H,Is]; ys [T,H]. */
void or_shared_down(const uint16_t *hs, int64_t T, int64_t S, int64_t Is, const uint16_t *sd, int64_t H, double *ys)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++)
        for (int64_t n = 0; n < H; n++) {
            double acc = 0.0;
            for (int64_t s = 0; s < S; s++)
                for (int64_t j = 0; j < Is; j++)
                    acc += or_bf16_to_double(hs[t * S * Is + s * Is + j]) * or_bf16_to_double(sd[(s * H + n) * Is + j]);
            ys[t * H + n] = acc;
        }
}

/* O8. Gate-weighted combine in slot order: zc[t] = bf16(sum_j w[t,j] * y[t*K + j]).
 * y [T*K, Lt] by pair id; w [T,K]; zc [T,Lt]. */
void or_combine(const uint16_t *y, const double *w, int64_t T, int64_t K, int64_t Lt, uint16_t *zc)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++)
        for (int64_t c = 0; c < Lt; c++) {
            double acc = 0.0;
            for (int64_t j = 0; j < K; j++)
                acc += w[t * K + j] * or_bf16_to_double(y[(t * K + j) * Lt + c]);
            zc[t * Lt + c] = or_double_to_bf16(acc);
        }
}

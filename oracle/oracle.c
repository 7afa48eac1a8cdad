/*
 * CPU oracle for the FP4 routed mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file: only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark use it. It shares no code, header, table or constant generator
 * with the HIP library; both sides take their inputs from the seeded generators
 * and nothing else.
 *
 * What it computes (the routed mixture of experts with FP4 packed expert
 * weights and int8-quantized decode activations of DeepSeek-V4-Flash on AMD
 * gfx90a: Correctness Recovery and Inference Performance Engineering,
 * abstract; 256 routed experts with 6 active per token from DeepSeek V4
 * Flash on 8x AMD gfx1201: packaged TP=8 deployment, What we set out to do):
 *
 *   1. router logits  l[t,e] = <x[t,:], Wr[e,:]> (+ b[e])            fp32
 *   2. scores s = sigmoid(l); the k largest (ties -> lower expert);
 *      weights w_j = s_j / sum_j s_j                                     fp32
 *   3. expert sort: stable counting sort of the T*k (token, slot) pairs by
 *      expert, each expert segment padded to a multiple of block_m
 *   4. activation quantization: per-row symmetric int8, or MXFP4 (E2M1
 *      codes with one E8M0 scale per 32 along K, OCP Microscaling v1.0)
 *   5. gate/up GEMM against packed E2M1 weights with block-32 E8M0 scales,
 *      a = silu(g) * u, requantized like step 4
 *   6. down GEMM against W2
 *   7. out[t] = sum_j w_j * y[pair(t, j)]
 *
 * Floating point is fp32 where the layer fixes fp32 (router, accumulation
 * over scale blocks, activation), with every reduction in one written-down
 * order so that a second implementation can reproduce the bits. Block sums
 * of code products are exact integers. The readings taken where the pages
 * leave a step open are stated beside each function.
 *
 * Build: gcc -O3 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 * -ffp-contract=off matters: every fused multiply-add below is written as
 * fmaf() and every other product/sum must round on its own.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Formats (OCP Microscaling Formats v1.0: E2M1 element, E8M0 scale)        */
/* ------------------------------------------------------------------------ */

/* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent field 0 is subnormal: value = m * 2^(1-1) * 0.5. */
float or_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    float mag = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return s ? -mag : mag;
}

/* E8M0: an unsigned biased exponent, value 2^(b-127); 0xFF encodes NaN. */
float or_e8m0_value(int b)
{
    if (b == 255) return NAN;
    return ldexpf(1.0f, b - 127);
}

/* Twice an E2M1 value is an integer in {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}. */
static int twice_e2m1(int code) { return (int)(2.0f * or_e2m1_value(code)); }

static int nibble(const uint8_t* row, int k) { return (row[k >> 1] >> ((k & 1) * 4)) & 15; }

/* ------------------------------------------------------------------------ */
/* exp and sigmoid in fp32, from the mathematics                            */
/* ------------------------------------------------------------------------ */
/* exp(z) = 2^n * exp(r), n = rint(z * log2 e), r = z - n ln2 by a two-term
 * Cody-Waite split of ln 2 (the high part keeps 15 significant bits so n*hi
 * is exact for |n| <= 256), exp(r) by its Taylor series to degree 7 in
 * Horner form with fused multiply-adds, then an exact power-of-two scaling.
 * Only IEEE operations with one rounding each are used (mul, fma, rint,
 * ldexp, add, div), so any conforming fp32 implementation gets the same bits.
 * The Taylor remainder on |r| <= ln2/2 is below 0.1 ulp. */
#define OR_LOG2E 0x1.715476p+0f   /* fp32(log2 e) */
#define OR_LN2_HI 0x1.62e4p-1f    /* ln 2 truncated to 15 significant bits */
#define OR_LN2_LO 0x1.7f7d1cp-20f /* fp32(ln 2 - OR_LN2_HI) */
#define OR_EXP_HI 0x1.62e42ep+6f  /* largest z with finite fp32 exp(z) */
#define OR_EXP_LO (-0x1.9fe36ap+6f) /* fp32 just below ln(2^-150): exp rounds to 0 */

float or_expf(float z)
{
    if (z != z) return z;
    if (z > OR_EXP_HI) return INFINITY;
    if (z < OR_EXP_LO) return 0.0f;
    float n = rintf(z * OR_LOG2E);
    float r = fmaf(-n, OR_LN2_HI, z);
    r = fmaf(-n, OR_LN2_LO, r);
    /* 1/k! for k = 7..0 */
    float p = 0x1.a01a02p-13f;        /* 1/5040 */
    p = fmaf(p, r, 0x1.6c16c2p-10f);  /* 1/720 */
    p = fmaf(p, r, 0x1.111112p-7f);   /* 1/120 */
    p = fmaf(p, r, 0x1.555556p-5f);   /* 1/24 */
    p = fmaf(p, r, 0x1.555556p-3f);   /* 1/6 */
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);
}

float or_sigmoidf(float z) { return 1.0f / (1.0f + or_expf(-z)); }

/* ------------------------------------------------------------------------ */
/* Ordered fp32 dot product                                                  */
/* ------------------------------------------------------------------------ */
/* Reading of the reduction order (the pages give none; bit-exact routing
 * needs one): split the length-H vectors into 64 contiguous chunks of
 * L = H/64; each chunk is a chain p = fma(a_i, b_i, p) from p = 0 over
 * ascending i; the 64 partials are then summed as a perfect pairwise tree in
 * index order (level 1: p0+p1, p2+p3, ...; six levels). */
static float ordered_dot(int H, const float* a, const float* b)
{
    float part[64];
    int L = H / 64;
    for (int c = 0; c < 64; ++c) {
        float p = 0.0f;
        for (int i = 0; i < L; ++i) p = fmaf(a[c * L + i], b[c * L + i], p);
        part[c] = p;
    }
    for (int width = 64; width > 1; width /= 2)
        for (int j = 0; j < width / 2; ++j) part[j] = part[2 * j] + part[2 * j + 1];
    return part[0];
}

/* x arrives as fp32 or as bf16 bit patterns; bf16 -> fp32 is exact. */
void or_x_to_f32(int T, int H, int x_dtype, const void* x, float* xf)
{
    if (x_dtype == 0) {
        memcpy(xf, x, (size_t)T * H * sizeof(float));
        return;
    }
    const uint16_t* xb = (const uint16_t*)x;
    for (size_t i = 0; i < (size_t)T * H; ++i) {
        uint32_t u = (uint32_t)xb[i] << 16;
        memcpy(&xf[i], &u, 4);
    }
}

/* ------------------------------------------------------------------------ */
/* Router: logits, sigmoid, top-k, renormalization                          */
/* ------------------------------------------------------------------------ */
/* Router logits on unquantized x (fp32). The optional bias is added to the
 * finished dot product as one fp32 add, before the sigmoid, so it moves both
 * the selection and the weights. */
void or_router_logits(int T, int H, int E, const float* xf, const float* wr,
                      const float* bias, float* logits)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            float l = ordered_dot(H, xf + (size_t)t * H, wr + (size_t)e * H);
            if (bias) l = l + bias[e];
            logits[(size_t)t * E + e] = l;
        }
}

/* Sigmoid scores; pick the k largest scores, ties to the lower expert index,
 * slot j holding the j-th pick; renormalize: S = ((s_0 + s_1) + s_2) + ...
 * in slot order and w_j = s_j / S (w_j = 1/k if S == 0). No group-limited
 * routing and a routed scaling factor of 1. */
void or_topk(int T, int E, int k, const float* logits, int32_t* ids, float* w, float* scores_out)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        float* s = (float*)malloc((size_t)E * sizeof(float));
        char* taken = (char*)calloc((size_t)E, 1);
        for (int e = 0; e < E; ++e) s[e] = or_sigmoidf(logits[(size_t)t * E + e]);
        if (scores_out) memcpy(scores_out + (size_t)t * E, s, (size_t)E * sizeof(float));
        float S = 0.0f;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || s[e] > s[best])) best = e;
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
            S = S + s[best];
        }
        for (int j = 0; j < k; ++j) {
            float sj = s[ids[(size_t)t * k + j]];
            w[(size_t)t * k + j] = (S == 0.0f) ? 1.0f / (float)k : sj / S;
        }
        free(s);
        free(taken);
    }
}

/* ------------------------------------------------------------------------ */
/* Expert sort (retuned for prefill in the gfx90a paper, abstract)         */
/* ------------------------------------------------------------------------ */
/* Pairs are numbered i = t*k + j. counts[e] = pairs routed to e. Each
 * expert's segment is padded up to a multiple of block_m; offsets[e] is the
 * segment start (offsets[E] = padded total). sorted[p] is the pair index at
 * padded position p (pairs of one expert in ascending i), or the sentinel P
 * in padding. pos[i] is where pair i landed. tile_expert[q] is the expert of
 * the q-th block of block_m positions; *n_tiles = offsets[E] / block_m.
 * Returns the padded total. */
int or_sort(int P, int E, int block_m, const int32_t* ids, int32_t* counts, int32_t* offsets,
            int32_t* sorted, int32_t* pos, int32_t* tile_expert, int32_t* n_tiles)
{
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int i = 0; i < P; ++i) counts[ids[i]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        int padded = (counts[e] + block_m - 1) / block_m * block_m;
        offsets[e + 1] = offsets[e] + padded;
    }
    int total = offsets[E];
    for (int p = 0; p < total; ++p) sorted[p] = P;
    int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (int i = 0; i < P; ++i) {
        int e = ids[i];
        int p = offsets[e] + fill[e]++;
        sorted[p] = i;
        pos[i] = p;
    }
    free(fill);
    int nt = 0;
    for (int e = 0; e < E; ++e)
        for (int p = offsets[e]; p < offsets[e + 1]; p += block_m) tile_expert[nt++] = e;
    *n_tiles = nt;
    return total;
}

/* ------------------------------------------------------------------------ */
/* Activation quantization                                                   */
/* ------------------------------------------------------------------------ */
/* Symmetric int8 per row: amax = max |v|, s = amax / 127,
 * q = clamp(rint(v / s), -127, 127) with ties to even; amax = 0 gives s = 0
 * and q = 0. */
void or_quant_int8(int R, int K, const float* v, int8_t* q, float* s)
{
    for (int r = 0; r < R; ++r) {
        const float* row = v + (size_t)r * K;
        float amax = 0.0f;
        for (int i = 0; i < K; ++i) amax = fmaxf(amax, fabsf(row[i]));
        float sc = amax / 127.0f;
        s[r] = sc;
        for (int i = 0; i < K; ++i) {
            float qq = (amax == 0.0f) ? 0.0f : rintf(row[i] / sc);
            if (qq > 127.0f) qq = 127.0f;
            if (qq < -127.0f) qq = -127.0f;
            q[(size_t)r * K + i] = (int8_t)qq;
        }
    }
}

/* Nearest E2M1 magnitude code for a >= 0, ties to the code with mantissa bit
 * 0; everything above 6 saturates to 6. Written as a scan over the eight
 * magnitudes, which is the definition of round-to-nearest-even on this grid. */
static int e2m1_nearest_mag(float a)
{
    int best = 0;
    float bestd = INFINITY;
    for (int m = 0; m < 8; ++m) {
        float d = fabsf(a - or_e2m1_value(m));
        if (d < bestd || (d == bestd && (m & 1) == 0 && (best & 1) == 1)) {
            best = m;
            bestd = d;
        }
    }
    return best;
}

/* MXFP4 per block of 32 along K (OCP MX v1.0 conversion): the shared scale
 * exponent is floor(log2 amax) - 2 (2 = the largest E2M1 exponent), stored
 * biased by 127 and clamped to [0, 254]; elements are scaled exactly by
 * 2^(127 - e) and rounded to nearest-even on the E2M1 grid with saturation at
 * 6. The code's sign bit is the sign bit of the element (so -0 may appear).
 * A block with amax = 0 gets scale byte 0 and codes 0.
 * codes: [R][K/2] (low nibble = even k); scales: [R][K/32]. */
void or_quant_mxfp4(int R, int K, const float* v, uint8_t* codes, uint8_t* scales)
{
    memset(codes, 0, (size_t)R * K / 2);
    for (int r = 0; r < R; ++r)
        for (int b = 0; b < K / 32; ++b) {
            const float* blk = v + (size_t)r * K + 32 * b;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(blk[i]));
            int e = 0;
            if (amax > 0.0f) {
                int ex;
                frexpf(amax, &ex); /* amax = m * 2^ex, m in [0.5, 1): floor(log2) = ex - 1 */
                e = (ex - 1) - 2 + 127;
                if (e < 0) e = 0;
                if (e > 254) e = 254;
            }
            scales[(size_t)r * (K / 32) + b] = (uint8_t)e;
            for (int i = 0; i < 32; ++i) {
                int code = 0;
                if (amax > 0.0f) {
                    float vs = ldexpf(blk[i], 127 - e);
                    code = e2m1_nearest_mag(fabsf(vs)) | (signbit(vs) ? 8 : 0);
                }
                int k = 32 * b + i;
                codes[(size_t)r * (K / 2) + k / 2] |= (uint8_t)(code << ((k & 1) * 4));
            }
        }
}

/* ------------------------------------------------------------------------ */
/* One output row of a block-scaled FP4 GEMM                                 */
/* ------------------------------------------------------------------------ */
/* Weights W[N][K]: codes [N][K/2], E8M0 scales [N][K/32], block 32 along K.
 * int8 activations (q, s):
 *   isum_b = sum_{i in b} q_i * (2 c_i)                     exact int32
 *   acc    = acc + isum_b * 2^(e_b - 128)  over ascending b  fp32
 *   out_n  = s * acc
 * MXFP4 activations (codes cx, scales ex):
 *   isum_b = sum (2 cx_i)(2 cw_i);  acc = acc + isum_b * 2^(ex_b + ew_b - 256)
 *   out_n  = acc
 * (Each term isum_b * 2^m is one correctly rounded operation, exact while it
 * stays in the normal range; only the fp32 additions round.) */
static void twice_table(int t[16])
{
    for (int c = 0; c < 16; ++c) t[c] = twice_e2m1(c);
}

/* Twice the E2M1 value of each of the K codes of a row, as small integers. */
static void twice_row(int K, const uint8_t* codes, int8_t* out)
{
    int t2[16];
    twice_table(t2);
    for (int k = 0; k < K; ++k) out[k] = (int8_t)t2[nibble(codes, k)];
}

/* isum * 2^m rounded once to fp32, as ldexpf((float)isum, m) gives it
 * (|isum| < 2^24, so (float)isum is exact). Where 2^m is itself an fp32 value
 * the product with it is that same single rounding. */
static float times_pow2(int32_t isum, int m)
{
    if (m >= -149 && m <= 127) {
        uint32_t bits = m >= -126 ? (uint32_t)(m + 127) << 23 : 1u << (m + 149);
        float p;
        memcpy(&p, &bits, 4);
        return (float)isum * p;
    }
    return ldexpf((float)isum, m);
}

/* Rows of activations against decoded weights: xv[R][K] are the activation
 * integers of R rows (q for int8, twice the E2M1 value for MXFP4), wd[N][K]
 * twice the weight values. xs = NULL selects int8 (exponent e_b - 128, each
 * row times its s[r] at the end); otherwise xs[R][K/32] are the activation
 * E8M0 bytes (exponent ex_b + ew_b - 256). out[R][N]. Each output is the
 * single-row formula above; the rows share the reads of a weight row. */
static void gemm_rows_decoded(int K, int N, int R, const int8_t* xv, const uint8_t* xs, const float* s,
                              const int8_t* wd, const uint8_t* ws, float* out)
{
    for (int n = 0; n < N; ++n) {
        const int8_t* row = wd + (size_t)n * K;
        const uint8_t* sc = ws + (size_t)n * (K / 32);
        for (int r = 0; r < R; ++r) {
            const int8_t* x = xv + (size_t)r * K;
            float acc = 0.0f;
            for (int b = 0; b < K / 32; ++b) {
                int32_t isum = 0;
                for (int i = 0; i < 32; ++i) isum += (int32_t)x[32 * b + i] * (int32_t)row[32 * b + i];
                int m = xs ? (int)xs[(size_t)r * (K / 32) + b] + (int)sc[b] - 256 : (int)sc[b] - 128;
                acc = acc + times_pow2(isum, m);
            }
            out[(size_t)r * N + n] = xs ? acc : s[r] * acc;
        }
    }
}

static void gemm_row_int8(int K, int N, const int8_t* q, float s, const uint8_t* wc,
                          const uint8_t* ws, float* out)
{
    int8_t* wd = (int8_t*)malloc((size_t)N * K);
    for (int n = 0; n < N; ++n) twice_row(K, wc + (size_t)n * (K / 2), wd + (size_t)n * K);
    gemm_rows_decoded(K, N, 1, q, NULL, &s, wd, ws, out);
    free(wd);
}

static void gemm_row_mxfp4(int K, int N, const uint8_t* xc, const uint8_t* xs, const uint8_t* wc,
                           const uint8_t* ws, float* out)
{
    int8_t* xv = (int8_t*)malloc((size_t)K);
    int8_t* wd = (int8_t*)malloc((size_t)N * K);
    twice_row(K, xc, xv);
    for (int n = 0; n < N; ++n) twice_row(K, wc + (size_t)n * (K / 2), wd + (size_t)n * K);
    gemm_rows_decoded(K, N, 1, xv, xs, NULL, wd, ws, out);
    free(xv);
    free(wd);
}

/* a = (g * sigmoid(g)) * u, two fp32 multiplies in that order; g = h[0:I],
 * u = h[I:2I] (gate rows first in W13). */
static void silu_mul(int I, const float* h, float* a)
{
    for (int n = 0; n < I; ++n) {
        float g = h[n], u = h[I + n];
        a[n] = (g * or_sigmoidf(g)) * u;
    }
}

/* Public single-row entry points (used by tests on intermediates). */
void or_gemm_row_int8(int K, int N, const int8_t* q, float s, const uint8_t* wc, const uint8_t* ws, float* out)
{
    gemm_row_int8(K, N, q, s, wc, ws, out);
}
void or_gemm_row_mxfp4(int K, int N, const uint8_t* xc, const uint8_t* xs, const uint8_t* wc,
                       const uint8_t* ws, float* out)
{
    gemm_row_mxfp4(K, N, xc, xs, wc, ws, out);
}
void or_silu_mul(int I, const float* h, float* a) { silu_mul(I, h, a); }

/* ------------------------------------------------------------------------ */
/* The whole layer for a list of tokens                                      */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t T, H, I, E, top_k, x_dtype, act_mode;
} or_config;

/* Every output of the layer depends only on its own token, so the oracle
 * computes any subset of tokens exactly as it would inside the whole batch.
 * x: [T][H] (fp32 or bf16 bits) of the tokens to compute. Weights are given
 * per expert (arrays of E pointers, canonical layout: W13 [2I][H/2] codes,
 * [2I][H/32] scales; W2 [H][I/2], [H][I/32]); a NULL entry is allowed for an
 * expert that no token selects. Optional outputs (NULL to skip), pair p =
 * t*k + j: ids/w [T][k]; xq (int8 [T][H] or codes [T][H/2]) and xs (fp32 [T]
 * or bytes [T][H/32]); h [P][2I]; aq/as like xq/xs with K = I; y [P][H].
 * Returns 0, or -1 if a needed expert pointer is NULL. */
/* The layer's expert part for given routing: quantize x, per pair the
 * gate/up row, SiLU-mul, requantization and the down row, then the combine.
 * ids/wts [T][k] are the routing (ids in [0, E)); xf is x in fp32. */
static int layer_given_routing(const or_config* c, const float* xf, const int32_t* ids, const float* wts,
                               const uint8_t* const* w13, const uint8_t* const* w13s,
                               const uint8_t* const* w2, const uint8_t* const* w2s, float* out,
                               void* xq_out, void* xs_out, float* h_out, void* aq_out, void* as_out, float* y_out)
{
    const int T = c->T, H = c->H, I = c->I, k = c->top_k;
    const int mx = c->act_mode == 1;
    const int P = T * k;
    for (int p = 0; p < P; ++p)
        if (ids[p] < 0 || ids[p] >= c->E || !w13[ids[p]] || !w13s[ids[p]] || !w2[ids[p]] || !w2s[ids[p]])
            return -1;

    /* activation quantization of x (per token) */
    size_t xq_row = mx ? (size_t)H / 2 : (size_t)H;
    size_t xs_row = mx ? (size_t)H / 32 : sizeof(float);
    uint8_t* xq = (uint8_t*)malloc((size_t)T * xq_row);
    uint8_t* xs = (uint8_t*)malloc((size_t)T * xs_row);
    if (mx) or_quant_mxfp4(T, H, xf, xq, xs);
    else or_quant_int8(T, H, xf, (int8_t*)xq, (float*)xs);
    if (xq_out) memcpy(xq_out, xq, (size_t)T * xq_row);
    if (xs_out) memcpy(xs_out, xs, (size_t)T * xs_row);

    size_t aq_row = mx ? (size_t)I / 2 : (size_t)I;
    size_t as_row = mx ? (size_t)I / 32 : sizeof(float);
    float* y = (float*)malloc((size_t)P * H * sizeof(float));

    /* Activation integers of x per token: q itself (int8) or twice the E2M1
     * values of the codes (MXFP4). */
    int8_t* xv = (int8_t*)malloc((size_t)T * H);
    for (int t = 0; t < T; ++t) {
        if (mx) twice_row(H, xq + (size_t)t * xq_row, xv + (size_t)t * H);
        else memcpy(xv + (size_t)t * H, xq + (size_t)t * xq_row, (size_t)H);
    }

    /* The pairs are taken expert by expert (ascending pair index within an
     * expert) in blocks of up to PB, after each used expert's codes have been
     * decoded to integers once; a block's rows share the reads of the decoded
     * weights. The arithmetic of every pair is the same whatever the order. */
    enum { PB = 8 };
    int32_t* order = (int32_t*)malloc((size_t)P * sizeof(int32_t));
    int32_t* start = (int32_t*)calloc((size_t)c->E + 1, sizeof(int32_t));
    for (int p = 0; p < P; ++p) start[ids[p] + 1]++;
    for (int e = 0; e < c->E; ++e) start[e + 1] += start[e];
    {
        int32_t* fill = (int32_t*)calloc((size_t)c->E, sizeof(int32_t));
        for (int p = 0; p < P; ++p) order[start[ids[p]] + fill[ids[p]]++] = p;
        free(fill);
    }
    /* decoded weights of the used experts: slot[e] = index into dec, or -1 */
    int32_t* slot = (int32_t*)malloc((size_t)c->E * sizeof(int32_t));
    int nused = 0;
    for (int e = 0; e < c->E; ++e) slot[e] = start[e + 1] > start[e] ? nused++ : -1;
    const size_t d13 = (size_t)2 * I * H, d2 = (size_t)H * I;
    int8_t* dec = (int8_t*)malloc((size_t)nused * (d13 + d2));
#pragma omp parallel for schedule(dynamic, 64)
    for (long long i = 0; i < (long long)c->E * (2 * I + H); ++i) {
        int e = (int)(i / (2 * I + H)), n = (int)(i % (2 * I + H));
        if (slot[e] < 0) continue;
        int8_t* base = dec + (size_t)slot[e] * (d13 + d2);
        if (n < 2 * I) twice_row(H, w13[e] + (size_t)n * (H / 2), base + (size_t)n * H);
        else twice_row(I, w2[e] + (size_t)(n - 2 * I) * (I / 2), base + d13 + (size_t)(n - 2 * I) * I);
    }
    /* task list: (expert, first index into order) per block */
    int ntask = 0;
    for (int e = 0; e < c->E; ++e) ntask += (start[e + 1] - start[e] + PB - 1) / PB;
    int32_t* task = (int32_t*)malloc((size_t)(ntask + 1) * sizeof(int32_t));
    int32_t* task_e = (int32_t*)malloc((size_t)(ntask + 1) * sizeof(int32_t));
    ntask = 0;
    for (int e = 0; e < c->E; ++e)
        for (int i = start[e]; i < start[e + 1]; i += PB) {
            task[ntask] = i;
            task_e[ntask++] = e;
        }

#pragma omp parallel for schedule(dynamic, 1)
    for (int tk = 0; tk < ntask; ++tk) {
        const int e = task_e[tk], i0 = task[tk];
        const int R = (start[e + 1] - i0) < PB ? (start[e + 1] - i0) : PB;
        const int8_t* wd13 = dec + (size_t)slot[e] * (d13 + d2);
        const int8_t* wd2 = wd13 + d13;
        int8_t* xr = (int8_t*)malloc((size_t)PB * H);
        uint8_t* xsr = (uint8_t*)malloc((size_t)PB * (H / 32));
        float sr[PB], sa[PB];
        float* h = (float*)malloc((size_t)PB * 2 * I * sizeof(float));
        float* a = (float*)malloc((size_t)I * sizeof(float));
        uint8_t* aq = (uint8_t*)malloc((size_t)PB * aq_row);
        uint8_t* asp = (uint8_t*)malloc((size_t)PB * (I / 32 + 4));
        int8_t* av = (int8_t*)malloc((size_t)PB * I);
        float* yb = (float*)malloc((size_t)PB * H * sizeof(float));
        /* gather the block's activation rows */
        for (int r = 0; r < R; ++r) {
            int t = order[i0 + r] / k;
            memcpy(xr + (size_t)r * H, xv + (size_t)t * H, (size_t)H);
            if (mx) memcpy(xsr + (size_t)r * (H / 32), xs + (size_t)t * xs_row, (size_t)H / 32);
            else sr[r] = ((const float*)xs)[t];
        }
        /* gate/up, SiLU-mul, requantization */
        gemm_rows_decoded(H, 2 * I, R, xr, mx ? xsr : NULL, sr, wd13, w13s[e], h);
        for (int r = 0; r < R; ++r) {
            silu_mul(I, h + (size_t)r * 2 * I, a);
            if (mx) {
                or_quant_mxfp4(1, I, a, aq + (size_t)r * aq_row, asp + (size_t)r * (I / 32));
                twice_row(I, aq + (size_t)r * aq_row, av + (size_t)r * I);
            } else {
                or_quant_int8(1, I, a, (int8_t*)aq + (size_t)r * aq_row, &sa[r]);
                memcpy(av + (size_t)r * I, aq + (size_t)r * aq_row, (size_t)I);
            }
        }
        /* down */
        gemm_rows_decoded(I, H, R, av, mx ? asp : NULL, sa, wd2, w2s[e], yb);
        for (int r = 0; r < R; ++r) {
            int p = order[i0 + r];
            memcpy(y + (size_t)p * H, yb + (size_t)r * H, (size_t)H * sizeof(float));
            if (h_out) memcpy(h_out + (size_t)p * 2 * I, h + (size_t)r * 2 * I, (size_t)2 * I * sizeof(float));
            if (aq_out) memcpy((uint8_t*)aq_out + (size_t)p * aq_row, aq + (size_t)r * aq_row, aq_row);
            if (as_out) {
                if (mx) memcpy((uint8_t*)as_out + (size_t)p * as_row, asp + (size_t)r * (I / 32), as_row);
                else memcpy((uint8_t*)as_out + (size_t)p * as_row, &sa[r], as_row);
            }
        }
        free(xr); free(xsr); free(h); free(a); free(aq); free(asp); free(av); free(yb);
    }
    free(task); free(task_e); free(dec); free(slot); free(order); free(start); free(xv);

    /* combine: acc = fma(w_j, y_j, acc) over ascending slots, from 0 */
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int n = 0; n < H; ++n) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j)
                acc = fmaf(wts[(size_t)t * k + j], y[((size_t)t * k + j) * H + n], acc);
            out[(size_t)t * H + n] = acc;
        }

    if (y_out) memcpy(y_out, y, (size_t)P * H * sizeof(float));
    free(xq); free(xs); free(y);
    return 0;
}

/* Every output of the layer depends only on its own token, so the oracle
 * computes any subset of tokens exactly as it would inside the whole batch.
 * x: [T][H] (fp32 or bf16 bits) of the tokens to compute. Weights are given
 * per expert (arrays of E pointers, canonical layout: W13 [2I][H/2] codes,
 * [2I][H/32] scales; W2 [H][I/2], [H][I/32]); a NULL entry is allowed for an
 * expert that no token selects. Optional outputs (NULL to skip), pair p =
 * t*k + j: ids/w [T][k]; xq (int8 [T][H] or codes [T][H/2]) and xs (fp32 [T]
 * or bytes [T][H/32]); h [P][2I]; aq/as like xq/xs with K = I; y [P][H].
 * Returns 0, or -1 if a needed expert pointer is NULL. */
int or_moe_layer(const or_config* c, const void* x, const float* wr, const float* bias,
                 const uint8_t* const* w13, const uint8_t* const* w13s,
                 const uint8_t* const* w2, const uint8_t* const* w2s,
                 float* out, int32_t* ids_out, float* w_out,
                 void* xq_out, void* xs_out, float* h_out, void* aq_out, void* as_out, float* y_out)
{
    const int T = c->T, H = c->H, E = c->E, k = c->top_k;
    const int P = T * k;
    float* xf = (float*)malloc((size_t)T * H * sizeof(float));
    float* logits = (float*)malloc((size_t)T * E * sizeof(float));
    int32_t* ids = (int32_t*)malloc((size_t)P * sizeof(int32_t));
    float* wts = (float*)malloc((size_t)P * sizeof(float));
    or_x_to_f32(T, H, c->x_dtype, x, xf);
    or_router_logits(T, H, E, xf, wr, bias, logits);
    or_topk(T, E, k, logits, ids, wts, NULL);
    const int r = layer_given_routing(c, xf, ids, wts, w13, w13s, w2, w2s, out, xq_out, xs_out, h_out, aq_out,
                                      as_out, y_out);
    if (r == 0 && ids_out) memcpy(ids_out, ids, (size_t)P * sizeof(int32_t));
    if (r == 0 && w_out) memcpy(w_out, wts, (size_t)P * sizeof(float));
    free(xf); free(logits); free(ids); free(wts);
    return r;
}

/* The layer without its router: the expert part for routing given by the
 * caller (ids [T][k] in [0, E), weights [T][k]), as a rank of an
 * expert-parallel deployment computes its dispatched pairs. Same outputs as
 * or_moe_layer after the routing. Returns 0, or -1 for an id out of range or
 * a NULL expert pointer it needs. */
int or_moe_layer_routed(const or_config* c, const void* x, const int32_t* ids, const float* wts,
                        const uint8_t* const* w13, const uint8_t* const* w13s,
                        const uint8_t* const* w2, const uint8_t* const* w2s, float* out,
                        void* xq_out, void* xs_out, float* h_out, void* aq_out, void* as_out, float* y_out)
{
    float* xf = (float*)malloc((size_t)c->T * c->H * sizeof(float));
    or_x_to_f32(c->T, c->H, c->x_dtype, x, xf);
    const int r = layer_given_routing(c, xf, ids, wts, w13, w13s, w2, w2s, out, xq_out, xs_out, h_out, aq_out,
                                      as_out, y_out);
    free(xf);
    return r;
}

/* ------------------------------------------------------------------------ */
/* Block-scaled FP8 dense projection (the model's FP8 dense projections: the  */
/* gfx90a paper, abstract; FP8 block quantization: the gfx1201 blog, What we  */
/* set out to do). Format (reading; the pages name no layout): OCP MX v1.0    */
/* MXFP8, E4M3 elements with one E8M0 scale per 32 consecutive elements      */
/* along K, for the weights [N][K] and for the activations quantized per     */
/* token.                                                                    */
/* ------------------------------------------------------------------------ */

/* E4M3 (OCP FP8, no infinities): bit 7 sign, bits 6..3 exponent (bias 7),
 * bits 2..0 mantissa; exponent 0 is subnormal (m * 2^-9); exponent 15 with
 * mantissa 7 is NaN. The largest finite magnitude is 1.75 * 2^8 = 448. */
float or_e4m3_value(int code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    float mag = (e == 0) ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -mag : mag;
}

/* Nearest E4M3 magnitude code (0..126) for a >= 0: a scan over the finite
 * magnitudes, ties to the code whose mantissa bit 0 is clear; anything above
 * the largest magnitude saturates to 448 (code 126). */
static int e4m3_nearest_mag(float a)
{
    if (a >= 448.0f) return 126;
    int best = 0;
    float bestd = INFINITY;
    for (int c = 0; c < 127; ++c) {
        float d = fabsf(a - or_e4m3_value(c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* MXFP8 per block of 32 along K: the shared scale exponent is
 * floor(log2 amax) - 8 (8 = the largest E4M3 exponent), stored biased by 127
 * and clamped to [0, 254]; elements are scaled exactly by 2^(127 - e),
 * rounded to the nearest E4M3 value with ties to even and saturated at 448.
 * The code's sign bit is the element's sign bit. A block with amax = 0 gets
 * scale byte 0 and codes 0. codes: [R][K]; scales: [R][K/32]. */
void or_quant_mxfp8(int R, int K, const float* v, uint8_t* codes, uint8_t* scales)
{
#pragma omp parallel for schedule(static)
    for (int r = 0; r < R; ++r)
        for (int b = 0; b < K / 32; ++b) {
            const float* blk = v + (size_t)r * K + 32 * b;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(blk[i]));
            int e = 0;
            if (amax > 0.0f) {
                int ex;
                frexpf(amax, &ex); /* floor(log2 amax) = ex - 1 */
                e = (ex - 1) - 8 + 127;
                if (e < 0) e = 0;
                if (e > 254) e = 254;
            }
            scales[(size_t)r * (K / 32) + b] = (uint8_t)e;
            for (int i = 0; i < 32; ++i) {
                int code = 0;
                if (amax > 0.0f) {
                    float vs = ldexpf(blk[i], 127 - e);
                    code = e4m3_nearest_mag(fabsf(vs)) | (signbit(vs) ? 0x80 : 0);
                }
                codes[(size_t)r * K + 32 * b + i] = (uint8_t)code;
            }
        }
}

/* Y[m][n] = sum_b 2^(ex[m][b] + ew[n][b] - 254) * sum_{k in b} x_k w_k with the
 * E4M3 values x, w. The products are exact in float64 and so is each block
 * sum (at most 32 products spanning under 48 significant bits); the block
 * terms are added in float64 in ascending b and the result rounded once to
 * fp32. absbound (nullable) receives sum_b 2^(...) sum_k |x_k w_k| in float64:
 * any fp32 evaluation that adds the K products in some order stays within
 * K * 2^-24 * absbound of the exact value. x: codes [M][K], scales [M][K/32];
 * w: codes [N][K], scales [N][K/32]. */
void or_dense_mxfp8(int M, int N, int K, const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                    const uint8_t* ws, float* out, double* absbound)
{
    double tab[256];
    for (int c = 0; c < 256; ++c) tab[c] = (double)or_e4m3_value(c);
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0, bound = 0.0;
            for (int b = 0; b < K / 32; ++b) {
                double bs = 0.0, ba = 0.0;
                for (int i = 0; i < 32; ++i) {
                    double p = tab[xq[(size_t)m * K + 32 * b + i]] * tab[wq[(size_t)n * K + 32 * b + i]];
                    bs += p;
                    ba += fabs(p);
                }
                double sc = ldexp(1.0, (int)xs[(size_t)m * (K / 32) + b] + (int)ws[(size_t)n * (K / 32) + b] - 254);
                acc += bs * sc;
                bound += ba * sc;
            }
            out[(size_t)m * N + n] = (float)acc;
            if (absbound) absbound[(size_t)m * N + n] = bound;
        }
}

/* ------------------------------------------------------------------------ */
/* RMSNorm for the stacked-layer residual stream                             */
/* ------------------------------------------------------------------------ */
/* Unit-gain RMSNorm between stacked layers (x_{l+1} = x_l + moe(rmsnorm(x_l))):
 * ss = ordered_dot(x, x) in the same chunked order as the router,
 * r = sqrt(ss / H + 1e-6) with IEEE sqrt and division, out = x / r. */
void or_rmsnorm(int T, int H, const float* x, float* out)
{
    for (int t = 0; t < T; ++t) {
        const float* row = x + (size_t)t * H;
        float ss = ordered_dot(H, row, row);
        float r = sqrtf(ss / (float)H + 1e-6f);
        for (int i = 0; i < H; ++i) out[(size_t)t * H + i] = row[i] / r;
    }
}

int or_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void or_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Array forms for the tests. */
void or_expf_n(int n, const float* z, float* out)
{
    for (int i = 0; i < n; ++i) out[i] = or_expf(z[i]);
}
void or_sigmoidf_n(int n, const float* z, float* out)
{
    for (int i = 0; i < n; ++i) out[i] = or_sigmoidf(z[i]);
}
void or_e2m1_table(float* out16)
{
    for (int c = 0; c < 16; ++c) out16[c] = or_e2m1_value(c);
}

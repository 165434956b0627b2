/*
 * MosaicQuant CPU oracle -- TEST INFRASTRUCTURE, NOT PART OF THE LIBRARY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this file's library. The HIP library never calls it, and the two share no
 * code: this file has its own fp16/bf16 conversions, its own nibble packing and
 * no include of the library's headers.
 *
 * It is a plain, slow, single-threaded statement of what the fused
 * W4A4 + sparse 4-bit residual path computes, following the MosaicQuant
 * technical summary ("MosaicQuant: Inlier-Outlier Disaggregation for Unified
 * 4-Bit LLM Quantization", gist.science):
 *   Methodology 1 "Inlier-Outlier Disaggregation": W^ ~ Q(W^) + R, a dense 4-bit
 *     base plus a sparse 4-bit residual, both 4-bit;
 *   Methodology 2 "Block-wise Residual Allocation": a Hessian-guided Delta-score
 *     (residual error weighted by the diagonal-Hessian activation sensitivity of
 *     the input channels) ranks blocks, and the top-K blocks get the residual;
 *   Methodology 3 "ZipperEngine": the residual product is computed inside the
 *     dense 4-bit GEMM; Experimental Results: W4A4 setting.
 * The pages fix no quantizer, scale format, score formula or summation order.
 * The readings used here (each one listed in the design notes) are:
 *   - symmetric round-to-nearest int4 in [-7, 7], ties to even; weights per
 *     (row, 128-wide group along K) with an fp16 scale (round-to-nearest-even of
 *     absmax/7 in fp32); activations per token with an fp32 scale;
 *   - residual R = int4 RTN of the base error E = W - s*q on the grid
 *     s_r = s/14 (= s / (2*qmax)), clamp [-7, 7], stored only for chosen blocks;
 *   - h_k = mean over tokens of x_k^2 (fp64 sum over tokens in ascending order,
 *     divided by M, rounded to fp32);
 *   - Delta_b = sum over the block's rows (ascending) of the row sums over the
 *     block's columns (ascending) of h_k * (e^2 - e'^2), every fp64 operation
 *     rounded separately; e' = E - s_r*r;
 *   - top-K by (Delta descending, block id ascending), id = row_block*(K/bk)+col_block;
 *   - Y = s_x * sum_g (s*P_g + s_r*Pr_g) in fp64 with exact integer P, Pr.
 *
 * fp32 steps are written with IEEE single operations (correctly rounded division,
 * rintf under round-to-nearest-even, fmaf). Build with -ffp-contract=off and no
 * fast-math so that no other contraction or reassociation happens.
 *
 * All pointers are host pointers. Functions return 0 on success, a negative
 * value on bad arguments.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_QMAX 7

/* Planted-mistake switch for the test suite's mutation check: the default build
 * (OR_MUTANT == 0) is the oracle; each non-zero value plants one plausible slip
 * so the tests can show that some pin catches it. */
#ifndef OR_MUTANT
#define OR_MUTANT 0
#endif
#define MUT(k) (OR_MUTANT == (k))

/* ------------------------------------------------------------------------- */
/* scalar conversions (from the IEEE 754 binary16 / bfloat16 definitions)     */
/* ------------------------------------------------------------------------- */

/* bfloat16 is the top half of a binary32, so widening is exact. */
static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Nearest binary16 value to f (ties to even), as its bit pattern.
 * All binary16 values are exact in double, so the rounding is done on the
 * integer count of quanta of the binade that holds |f|. */
uint16_t or_f32_to_f16_bits(float f) {
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    double a = fabs((double)f);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u); /* 65520 ties to the overflow side */
    int e;                                                 /* a in [2^e, 2^(e+1)) */
    if (a < 0x1p-14) {
        e = -14;                                           /* subnormal quantum 2^-24 */
    } else {
        (void)frexp(a, &e);
        e -= 1;
    }
    double quantum = ldexp(1.0, e - 10);
    double n = MUT(1) ? floor(a / quantum) : nearbyint(a / quantum); /* exact scaling, ties to even */
    double v = n * quantum;
    if (v == 0.0) return sign;
    if (v < 0x1p-14) return (uint16_t)(sign | (uint16_t)(v / 0x1p-24));
    int ev;
    (void)frexp(v, &ev);
    int E = ev - 1;                                        /* v in [2^E, 2^(E+1)) */
    uint16_t mant = (uint16_t)((v / ldexp(1.0, E) - 1.0) * 1024.0);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | mant);
}

float or_f16_bits_to_f32(uint16_t b) {
    int sign = (b >> 15) & 1, ex = (b >> 10) & 0x1f, mant = b & 0x3ff;
    double v;
    if (ex == 0x1f) v = mant ? NAN : INFINITY;
    else if (ex == 0) v = ldexp((double)mant, -24);
    else v = ldexp(1.0 + mant / 1024.0, ex - 15);
    return (float)(sign ? -v : v);
}

/* ------------------------------------------------------------------------- */
/* int4 helpers: two's-complement nibbles, low nibble = even index            */
/* ------------------------------------------------------------------------- */

static int nib_get(const uint8_t* row, int64_t k) {
    int v = ((k & 1) ^ MUT(2)) ? (row[k >> 1] >> 4) : (row[k >> 1] & 0xf);
    return v >= 8 ? v - 16 : v;
}

static void nib_put(uint8_t* row, int64_t k, int v) {
    uint8_t n = (uint8_t)(v & 0xf);
    if ((k & 1) ^ MUT(2)) row[k >> 1] = (uint8_t)((row[k >> 1] & 0x0f) | (n << 4));
    else row[k >> 1] = (uint8_t)((row[k >> 1] & 0xf0) | n);
}

/* symmetric RTN code of v on scale s: 0 if s == 0, else clamp(rint(v/s), lo, hi) */
static int rtn_code(float v, float s, int lo, int hi) {
    if (s == 0.0f) return 0;
    float t = MUT(3) ? roundf(v / s) : rintf(v / s);
    if (t < (float)lo) t = (float)lo;
    if (t > (float)hi) t = (float)hi;
    return (int)t;
}

static float load_x(const void* x, int x_dtype, int64_t i) {
    return x_dtype == 1 ? bf16_to_f32(((const uint16_t*)x)[i]) : ((const float*)x)[i];
}

/* ------------------------------------------------------------------------- */
/* O1: per-token symmetric int4 activation quantization (W4A4 setting)        */
/* ------------------------------------------------------------------------- */
int or_quantize_act(const void* x, int x_dtype, int64_t M, int64_t K, uint8_t* xq, float* sx) {
    if (M < 0 || K <= 0 || (K & 1) || (x_dtype != 0 && x_dtype != 1)) return -1;
    for (int64_t m = 0; m < M; ++m) {
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(load_x(x, x_dtype, m * K + k));
            if (v > a) a = v;
        }
        float s = a / (MUT(13) ? 8.0f : 7.0f);
        sx[m] = s;
        uint8_t* row = xq + m * (K / 2);
        memset(row, 0, (size_t)(K / 2));
        for (int64_t k = 0; k < K; ++k)
            nib_put(row, k, rtn_code(load_x(x, x_dtype, m * K + k), s, -OR_QMAX, OR_QMAX));
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O0: migration of activation outliers into the weights by an equivalent      */
/* per-channel transform (Methodology 1 starts with one, naming SmoothQuant as */
/* an example; the pages fix no exponent, the reading here is alpha = 1/2):    */
/*   a_k = max_m |x_mk|, b_k = max_n |w_nk|,                                   */
/*   s_k = sqrt(a_k) / sqrt(b_k)   (fp32 square roots and division),           */
/*   s_k = 1 when a_k or b_k is 0 (a dead channel is left alone), r_k = 1/s_k. */
/* The migrated layer is W^ = W diag(s) and X^ = X diag(r) (both fp32, one     */
/* rounding per element): X^ W^T = X W^T up to those roundings.                */
/* ------------------------------------------------------------------------- */
int or_smooth_factors(const void* x, int x_dtype, int64_t M, int64_t K, const float* w, int64_t N,
                      float* s, float* r) {
    if (M <= 0 || N <= 0 || K <= 0 || (x_dtype != 0 && x_dtype != 1)) return -1;
    for (int64_t k = 0; k < K; ++k) {
        float a = 0.0f, b = 0.0f;
        for (int64_t m = 0; m < M; ++m) {
            float v = fabsf(load_x(x, x_dtype, m * K + k));
            if (v > a) a = v;
        }
        for (int64_t n = 0; n < N; ++n) {
            float v = fabsf(w[n * K + k]);
            if (v > b) b = v;
        }
        float sk = 1.0f;
        if (a > 0.0f && b > 0.0f) sk = MUT(14) ? sqrtf(b) / sqrtf(a) : sqrtf(a) / sqrtf(b);
        s[k] = sk;
        r[k] = 1.0f / sk;
    }
    return 0;
}

/* out[i][k] = fp32(in[i][k] * c[k]) for an fp32 or bf16 input (rows x K) */
int or_scale_columns(const void* in, int in_dtype, int64_t rows, int64_t K, const float* c, float* out) {
    if (rows < 0 || K <= 0 || (in_dtype != 0 && in_dtype != 1)) return -1;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t k = 0; k < K; ++k) out[i * K + k] = load_x(in, in_dtype, i * K + k) * c[k];
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O4: diagonal-Hessian estimate of the input channels, h_k = mean_m x_mk^2   */
/* ------------------------------------------------------------------------- */
int or_hessian_diag(const void* x, int x_dtype, int64_t M, int64_t K, float* h) {
    if (M <= 0 || K <= 0 || (x_dtype != 0 && x_dtype != 1)) return -1;
    for (int64_t k = 0; k < K; ++k) {
        double acc = 0.0;
        for (int64_t m = 0; m < M; ++m) {
            double v = (double)load_x(x, x_dtype, m * K + k);
            acc = acc + v * v;
        }
        h[k] = (float)(acc / (double)(MUT(4) ? M - 1 + (M == 1) : M));
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O2 + O3: base Q(W) and residual R for one element                          */
/* ------------------------------------------------------------------------- */

/* fp16 base scale of row n, group g */
static uint16_t group_scale_bits(const float* w, int64_t K, int group, int64_t n, int64_t g) {
    float a = 0.0f;
    for (int64_t k = g * group; k < (g + 1) * group; ++k) {
        float v = fabsf(w[n * K + k]);
        if (v > a) a = v;
    }
    return or_f32_to_f16_bits(a / 7.0f);
}

typedef struct {
    int q;     /* base code in [-7, 7] */
    int r;     /* residual code in [-7, 7] */
    float e;   /* base error  E  = w - s*q   */
    float ep;  /* after residual e' = E - s_r*r */
} elem_t;

static elem_t quant_elem(float w, float s) {
    elem_t o;
    o.q = rtn_code(w, s, -OR_QMAX, OR_QMAX);
    o.e = MUT(12) ? fmaf(s, (float)o.q, w) : fmaf(-s, (float)o.q, w);
    float sr = MUT(5) ? s / 16.0f : s / 14.0f;
    o.r = rtn_code(o.e, sr, -OR_QMAX, OR_QMAX);
    o.ep = fmaf(-sr, (float)o.r, o.e);
    return o;
}

/* Unpacked element-wise view of the decomposition, for tests:
 * q, r int8 [N][K]; sw fp16 bits [N][K/group]; e, ep fp32 [N][K] (any may be NULL). */
int or_quantize_weights(const float* w, int64_t N, int64_t K, int group,
                        int8_t* q, uint16_t* sw, int8_t* r, float* e, float* ep) {
    if (N <= 0 || K <= 0 || group <= 0 || K % group) return -1;
    int64_t G = K / group;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < G; ++g) {
            uint16_t sb = group_scale_bits(w, K, group, n, g);
            float s = or_f16_bits_to_f32(sb);
            if (sw) sw[n * G + g] = sb;
            for (int64_t k = g * group; k < (g + 1) * group; ++k) {
                elem_t o = quant_elem(w[n * K + k], s);
                if (q) q[n * K + k] = (int8_t)o.q;
                if (r) r[n * K + k] = (int8_t)o.r;
                if (e) e[n * K + k] = o.e;
                if (ep) ep[n * K + k] = o.ep;
            }
        }
    return 0;
}

static int check_blocks(int64_t N, int64_t K, int group, int bn, int bk) {
    if (N <= 0 || K <= 0 || group <= 0 || bn <= 0 || bk <= 0) return -1;
    if (K % group || N % bn || K % bk) return -1;
    /* a block must lie inside one quantization group */
    if (group % bk) return -1;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O5: Hessian-guided Delta-score of every (bn x bk) block                    */
/* ------------------------------------------------------------------------- */
int or_delta_scores(const float* w, const float* h, int64_t N, int64_t K, int group,
                    int bn, int bk, double* delta) {
    if (check_blocks(N, K, group, bn, bk)) return -1;
    int64_t nbr = N / bn, nbc = K / bk;
    for (int64_t i = 0; i < nbr; ++i)
        for (int64_t j = 0; j < nbc; ++j) {
            int64_t g = (j * bk) / group;
            double total = 0.0;
            for (int64_t n = i * bn; n < (i + 1) * bn; ++n) {
                float s = or_f16_bits_to_f32(group_scale_bits(w, K, group, n, g));
                double row = 0.0;
                for (int64_t k = j * bk; k < (j + 1) * bk; ++k) {
                    elem_t o = quant_elem(w[n * K + k], s);
                    double e = (double)o.e, ep = (double)o.ep;
                    double reduction = MUT(6) ? e * e : e * e - ep * ep;
                    row = row + (MUT(7) ? 1.0 : (double)h[k]) * reduction;
                }
                total = total + row;
            }
            delta[i * nbc + j] = total;
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O6: global top-K blocks by Delta, emitted as CSR over block rows           */
/* ------------------------------------------------------------------------- */
static const double* g_sort_delta;

static int cmp_block(const void* a, const void* b) {
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    double dx = g_sort_delta[x], dy = g_sort_delta[y];
    if (dx > dy) return -1;
    if (dx < dy) return 1;
    if (MUT(8)) return x > y ? -1 : (x < y ? 1 : 0);
    return x < y ? -1 : (x > y ? 1 : 0);
}

/* delta [nbr*nbc] -> row_ptr [nbr+1], col_idx [k_blocks] (column-block index,
 * ascending within a row); sel (optional) [nbr*nbc] 0/1 mask. */
int or_select_topk(const double* delta, int64_t nbr, int64_t nbc, int64_t k_blocks,
                   int32_t* row_ptr, int32_t* col_idx, uint8_t* sel) {
    int64_t nb = nbr * nbc;
    if (nbr <= 0 || nbc <= 0 || k_blocks < 0 || k_blocks > nb) return -1;
    int64_t* order = (int64_t*)malloc((size_t)nb * sizeof(int64_t));
    uint8_t* mask = (uint8_t*)calloc((size_t)nb, 1);
    if (!order || !mask) { free(order); free(mask); return -2; }
    for (int64_t b = 0; b < nb; ++b) order[b] = b;
    g_sort_delta = delta;
    qsort(order, (size_t)nb, sizeof(int64_t), cmp_block);
    for (int64_t t = 0; t < k_blocks; ++t) mask[order[t]] = 1;
    int64_t p = 0;
    for (int64_t i = 0; i < nbr; ++i) {
        row_ptr[i] = (int32_t)p;
        for (int64_t j = 0; j < nbc; ++j)
            if (mask[i * nbc + j]) col_idx[p++] = (int32_t)j;
    }
    row_ptr[nbr] = (int32_t)p;
    if (sel) memcpy(sel, mask, (size_t)nb);
    free(order);
    free(mask);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O7: packed base (all groups) and residual payload (chosen blocks, CSR order)*/
/* ------------------------------------------------------------------------- */
int or_pack_weights(const float* w, int64_t N, int64_t K, int group, int bn, int bk,
                    const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                    uint8_t* wq, uint16_t* sw, uint8_t* rq) {
    if (check_blocks(N, K, group, bn, bk) || (bk & 1) || (K & 1)) return -1;
    int64_t G = K / group, nbr = N / bn;
    memset(wq, 0, (size_t)(N * (K / 2)));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < G; ++g) {
            uint16_t sb = group_scale_bits(w, K, group, n, g);
            sw[n * G + g] = sb;
            float s = or_f16_bits_to_f32(sb);
            for (int64_t k = g * group; k < (g + 1) * group; ++k)
                nib_put(wq + n * (K / 2), k, quant_elem(w[n * K + k], s).q);
        }
    if (nnz) memset(rq, 0, (size_t)(nnz * bn * (bk / 2)));
    for (int64_t i = 0; i < nbr; ++i)
        for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
            if (p < 0 || p >= nnz) return -1;
            int64_t j = col_idx[p], g = (j * bk) / group;
            for (int64_t rr = 0; rr < bn; ++rr) {
                int64_t n = i * bn + rr;
                float s = or_f16_bits_to_f32(sw[n * G + g]);
                uint8_t* dst = rq + (p * bn + rr) * (bk / 2);
                for (int64_t c = 0; c < bk; ++c)
                    nib_put(dst, c, quant_elem(w[n * K + j * bk + c], s).r);
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O8: exact integer partial sums per (token, output, group)                  */
/*   P [m][n][g]  = sum_{k in g} xq[m,k] * q[n,k]                             */
/*   Pr[m][n][g]  = sum over chosen blocks b in row n, group g of             */
/*                  sum_{k in cols(b)} xq[m,k] * r[n,k]                       */
/* ------------------------------------------------------------------------- */
int or_accumulators(const uint8_t* xq, const uint8_t* wq, const int32_t* row_ptr,
                    const int32_t* col_idx, const uint8_t* rq, int64_t nnz,
                    int64_t M, int64_t N, int64_t K, int group, int bn, int bk,
                    int32_t* P, int32_t* Pr) {
    if (check_blocks(N, K, group, bn, bk) || M < 0) return -1;
    int64_t G = K / group, nbr = N / bn;
    /* decode the codes once, so the dot products below are plain integer loops */
    int8_t* xs = (int8_t*)malloc((size_t)(M * K) + 1);
    int8_t* ws = (int8_t*)malloc((size_t)K);
    int8_t* rs = (int8_t*)malloc((size_t)bk);
    if (!xs || !ws || !rs) { free(xs); free(ws); free(rs); return -2; }
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) xs[m * K + k] = (int8_t)nib_get(xq + m * (K / 2), k);
    int rc = 0;
    for (int64_t n = 0; n < N && !rc; ++n) {
        for (int64_t k = 0; k < K; ++k) ws[k] = (int8_t)nib_get(wq + n * (K / 2), k);
        for (int64_t m = 0; m < M; ++m)
            for (int64_t g = 0; g < G; ++g) {
                int64_t acc = 0;
                for (int64_t k = g * group; k < (g + 1) * group; ++k)
                    acc += (int64_t)xs[m * K + k] * ws[MUT(11) ? (k ^ 1) : k];
                if (acc > INT32_MAX || acc < INT32_MIN) rc = -3;
                P[(m * N + n) * G + g] = (int32_t)acc;
            }
    }
    if (!rc) memset(Pr, 0, (size_t)(M * N * G) * sizeof(int32_t));
    for (int64_t i = 0; i < nbr && !rc; ++i)
        for (int64_t p = row_ptr[i]; p < row_ptr[i + 1] && !rc; ++p) {
            if (p < 0 || p >= nnz) { rc = -1; break; }
            int64_t j = col_idx[p], g = (j * bk) / group;
            if (MUT(9)) g = (g + 1) % G;
            for (int64_t rr = 0; rr < bn; ++rr) {
                int64_t n = i * bn + rr;
                const uint8_t* rrow = rq + (p * bn + rr) * (bk / 2);
                for (int64_t c = 0; c < bk; ++c) rs[c] = (int8_t)nib_get(rrow, c);
                for (int64_t m = 0; m < M; ++m) {
                    int64_t acc = Pr[(m * N + n) * G + g];
                    for (int64_t c = 0; c < bk; ++c) acc += (int64_t)xs[m * K + j * bk + c] * rs[c];
                    if (acc > INT32_MAX || acc < INT32_MIN) rc = -3;
                    Pr[(m * N + n) * G + g] = (int32_t)acc;
                }
            }
        }
    free(xs);
    free(ws);
    free(rs);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* O9: output Y[m][n] = s_x[m] * sum_g (s[n,g]*P + s_r[n,g]*Pr), fp64         */
/* ------------------------------------------------------------------------- */
int or_output(const float* sx, const uint16_t* sw, const int32_t* P, const int32_t* Pr,
              int64_t M, int64_t N, int64_t G, double* y) {
    if (M < 0 || N <= 0 || G <= 0) return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                float s = or_f16_bits_to_f32(sw[n * G + g]);
                float sr = s / 14.0f;
                int64_t t = (m * N + n) * G + g;
                acc = acc + (double)s * (double)P[t] + (MUT(10) ? 0.0 : (double)sr * (double)Pr[t]);
            }
            y[m * N + n] = (double)sx[m] * acc;
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O10: output distortion of a block selection S (mask over blocks), fp64     */
/*   W_S = s*q + s_r*r on blocks in S, s*q elsewhere; D = W^ - W_S            */
/*   exact: || X D^T ||_F^2      diag: M * sum_{n,k} h_k D_nk^2               */
/* ------------------------------------------------------------------------- */
static void selection_error(const float* w, int64_t N, int64_t K, int group, int bn, int bk,
                            const uint8_t* mask, double* D) {
    int64_t G = K / group, nbc = K / bk;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < G; ++g) {
            float s = or_f16_bits_to_f32(group_scale_bits(w, K, group, n, g));
            for (int64_t k = g * group; k < (g + 1) * group; ++k) {
                elem_t o = quant_elem(w[n * K + k], s);
                int chosen = mask[(n / bn) * nbc + k / bk];
                D[n * K + k] = chosen ? (double)o.ep : (double)o.e;
            }
        }
}

int or_distortion(const float* x, int64_t M, const float* w, const float* h, int64_t N,
                  int64_t K, int group, int bn, int bk, const uint8_t* mask,
                  double* d_exact, double* d_diag) {
    if (check_blocks(N, K, group, bn, bk) || M <= 0) return -1;
    double* D = (double*)malloc((size_t)(N * K) * sizeof(double));
    if (!D) return -2;
    selection_error(w, N, K, group, bn, bk, mask, D);
    if (d_exact) {
        double tot = 0.0;
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < N; ++n) {
                double dot = 0.0;
                for (int64_t k = 0; k < K; ++k) dot = dot + (double)x[m * K + k] * D[n * K + k];
                tot = tot + dot * dot;
            }
        *d_exact = tot;
    }
    if (d_diag) {
        double tot = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t k = 0; k < K; ++k) tot = tot + (double)h[k] * D[n * K + k] * D[n * K + k];
        *d_diag = (double)M * tot;
    }
    free(D);
    return 0;
}

/* Drives every step of the CPU oracle (oracle/oracle.c) once on a small random
 * layer, for a build with AddressSanitizer and UndefinedBehaviorSanitizer: any
 * out-of-bounds access, use after free, leak, signed overflow or misaligned
 * access in the oracle aborts the run. Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int or_quantize_act(const void* x, int x_dtype, int64_t M, int64_t K, uint8_t* xq, float* sx);
int or_smooth_factors(const void* x, int x_dtype, int64_t M, int64_t K, const float* w, int64_t N,
                      float* s, float* r);
int or_scale_columns(const void* in, int in_dtype, int64_t rows, int64_t K, const float* c, float* out);
int or_hessian_diag(const void* x, int x_dtype, int64_t M, int64_t K, float* h);
int or_quantize_weights(const float* w, int64_t N, int64_t K, int group, int8_t* q, uint16_t* sw,
                        int8_t* r, float* e, float* ep);
int or_delta_scores(const float* w, const float* h, int64_t N, int64_t K, int group, int bn, int bk,
                    double* delta);
int or_select_topk(const double* delta, int64_t nbr, int64_t nbc, int64_t k_blocks, int32_t* row_ptr,
                   int32_t* col_idx, uint8_t* sel);
int or_pack_weights(const float* w, int64_t N, int64_t K, int group, int bn, int bk,
                    const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz, uint8_t* wq,
                    uint16_t* sw, uint8_t* rq);
int or_accumulators(const uint8_t* xq, const uint8_t* wq, const int32_t* row_ptr, const int32_t* col_idx,
                    const uint8_t* rq, int64_t nnz, int64_t M, int64_t N, int64_t K, int group, int bn,
                    int bk, int32_t* P, int32_t* Pr);
int or_output(const float* sx, const uint16_t* sw, const int32_t* P, const int32_t* Pr, int64_t M,
              int64_t N, int64_t G, double* y);
int or_distortion(const float* x, int64_t M, const float* w, const float* h, int64_t N, int64_t K,
                  int group, int bn, int bk, const uint8_t* mask, double* d_exact, double* d_diag);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static float rnd(void) {   /* xorshift64*, uniform in [-1, 1) */
    state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
    return (float)((state * 0x2545f4914f6cdd1dull) >> 40) / (float)(1u << 23) - 1.0f;
}

#define CHECK(call) do { int rc_ = (call); if (rc_) { fprintf(stderr, "%s -> %d\n", #call, rc_); return 1; } } while (0)

int main(void) {
    const int64_t M = 5, N = 96, K = 256, group = 128, bn = 32, bk = 64, kb = 5;
    const int64_t G = K / group, nbr = N / bn, nbc = K / bk, nb = nbr * nbc;
    float* x = malloc(sizeof(float) * M * K);
    float* w = malloc(sizeof(float) * N * K);
    for (int64_t i = 0; i < M * K; ++i) x[i] = 3.0f * rnd();
    for (int64_t i = 0; i < N * K; ++i) w[i] = 0.02f * rnd();
    x[7] = 90.0f;       /* an outlier channel entry */
    for (int64_t k = 0; k < K; ++k) w[3 * K + k] = 0.0f;   /* an all-zero row */

    uint8_t* xq = calloc(M * K / 2, 1);
    float* sx = malloc(sizeof(float) * M);
    float* s = malloc(sizeof(float) * K);
    float* r = malloc(sizeof(float) * K);
    float* wh = malloc(sizeof(float) * N * K);
    float* xh = malloc(sizeof(float) * M * K);
    float* h = malloc(sizeof(float) * K);
    int8_t* q = calloc(N * K, 1);
    uint16_t* sw = malloc(sizeof(uint16_t) * N * G);
    int8_t* rr = calloc(N * K, 1);
    float* e = malloc(sizeof(float) * N * K);
    float* ep = malloc(sizeof(float) * N * K);
    double* delta = malloc(sizeof(double) * nb);
    int32_t* row_ptr = malloc(sizeof(int32_t) * (nbr + 1));
    int32_t* col_idx = malloc(sizeof(int32_t) * kb);
    uint8_t* sel = calloc(nb, 1);
    uint8_t* wq = calloc(N * K / 2, 1);
    uint16_t* sw2 = malloc(sizeof(uint16_t) * N * G);
    uint8_t* rq = calloc(kb * bn * bk / 2, 1);
    int32_t* P = malloc(sizeof(int32_t) * M * N * G);
    int32_t* Pr = malloc(sizeof(int32_t) * M * N * G);
    double* y = malloc(sizeof(double) * M * N);
    double dex = 0.0, ddi = 0.0;

    CHECK(or_smooth_factors(x, 0, M, K, w, N, s, r));
    CHECK(or_scale_columns(w, 0, N, K, s, wh));
    CHECK(or_scale_columns(x, 0, M, K, r, xh));
    CHECK(or_quantize_act(xh, 0, M, K, xq, sx));
    CHECK(or_hessian_diag(xh, 0, M, K, h));
    CHECK(or_quantize_weights(wh, N, K, group, q, sw, rr, e, ep));
    CHECK(or_delta_scores(wh, h, N, K, group, bn, bk, delta));
    CHECK(or_select_topk(delta, nbr, nbc, kb, row_ptr, col_idx, sel));
    CHECK(or_pack_weights(wh, N, K, group, bn, bk, row_ptr, col_idx, kb, wq, sw2, rq));
    CHECK(or_accumulators(xq, wq, row_ptr, col_idx, rq, kb, M, N, K, group, bn, bk, P, Pr));
    CHECK(or_output(sx, sw2, P, Pr, M, N, G, y));
    CHECK(or_distortion(xh, M, wh, h, N, K, group, bn, bk, sel, &dex, &ddi));
    printf("ok y[0]=%.6e d_exact=%.6e d_diag=%.6e\n", y[0], dex, ddi);

    free(x); free(w); free(xq); free(sx); free(s); free(r); free(wh); free(xh); free(h); free(q);
    free(sw); free(rr); free(e); free(ep); free(delta); free(row_ptr); free(col_idx); free(sel);
    free(wq); free(sw2); free(rq); free(P); free(Pr); free(y);
    return 0;
}

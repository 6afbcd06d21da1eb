/* Runs the fp64 oracles (oracle/gdn2_oracle.c, oracle/gdn2_oracle_bwd.c) on
 * small seeded inputs in every storage dtype, both erase readings, dense and
 * packed batches (with empty and one-token sequences) and their argument
 * errors, built with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py).  Exit status 0 when every call returns its
 * expected status and every output is finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdn2_oracle_fwd_ex(const void* q, const void* k, const void* v, const void* alpha,
                       const void* b, const void* w, int dtype, const double* S0,
                       double* o, double* S_T, const int32_t* cu_seqlens, int32_t num_seqs,
                       int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                       const uint8_t* pair_mask, int32_t nthreads, int32_t erase_rows);
int gdn2_oracle_bwd(const void* q, const void* k, const void* v, const void* alpha,
                    const void* b, const void* w, int dtype, const double* S0,
                    const void* dout, int do_dtype, const double* dS_T, double* dq, double* dk,
                    double* dv, double* dalpha, double* db, double* dw, double* dS0,
                    const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                    int32_t dkd, int32_t dvd, int32_t nthreads);

static int failures = 0;
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

static double urand(void) {   /* xorshift64*, in (0, 1) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return ((double)((rng_state * 2685821657736338717ull) >> 11) + 0.5) / 9007199254740992.0;
}

static void expect(int cond, const char* what) {
    if (!cond) {
        printf("FAIL %s\n", what);
        ++failures;
    }
}

static int all_finite(const double* x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

/* Fills n values of a storage dtype (0 fp32, 1 bf16 bits, 2 fp64) with
 * lo + (hi - lo) u. */
static void* fill(int dtype, size_t n, double lo, double hi) {
    if (n == 0) n = 1;
    if (dtype == 0) {
        float* p = malloc(n * sizeof(float));
        for (size_t i = 0; i < n; ++i) p[i] = (float)(lo + (hi - lo) * urand());
        return p;
    }
    if (dtype == 1) {
        uint16_t* p = malloc(n * sizeof(uint16_t));
        for (size_t i = 0; i < n; ++i) {
            float f = (float)(lo + (hi - lo) * urand());
            uint32_t u;
            memcpy(&u, &f, 4);
            p[i] = (uint16_t)(u >> 16);   /* truncation is fine for test data */
        }
        return p;
    }
    double* p = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * urand();
    return p;
}

static void run_case(int dtype, int erase, int packed, int nthreads) {
    const int32_t H = 2, dk = 8, dv = 12;
    int32_t lens[] = {5, 0, 70, 1, 64};
    const int32_t nseq = packed ? 5 : 3;
    int32_t cu[6] = {0};
    int32_t B, T;
    if (packed) {
        for (int i = 0; i < nseq; ++i) cu[i + 1] = cu[i] + lens[i];
        B = 1;
        T = cu[nseq];
    } else {
        B = nseq;
        T = 67;
    }
    const int32_t N = packed ? nseq : B;
    const size_t rows = (size_t)B * T;
    void* q = fill(dtype, rows * H * dk, -1, 1);
    void* k = fill(dtype, rows * H * dk, -0.4, 0.4);
    void* v = fill(dtype, rows * H * dv, -1, 1);
    void* al = fill(dtype, rows * H * dk, 0.6, 1.0);
    void* b = fill(dtype, rows * H * dk, 0.0, 1.0);
    void* w = fill(dtype, rows * H * dv, 0.0, 1.0);
    double* S0 = fill(2, (size_t)N * H * dk * dv, -0.1, 0.1);
    double* o = calloc(rows * H * dv + 1, sizeof(double));
    double* ST = calloc((size_t)N * H * dk * dv, sizeof(double));
    const int32_t* cup = packed ? cu : NULL;
    int r = gdn2_oracle_fwd_ex(q, k, v, al, b, w, dtype, S0, o, ST, cup, packed ? nseq : 0, B, T,
                               H, dk, dv, NULL, nthreads, erase);
    expect(r >= 1, "fwd status");
    expect(all_finite(o, rows * H * dv) && all_finite(ST, (size_t)N * H * dk * dv), "fwd finite");
    if (erase == 0) {
        void* dout = fill(dtype, rows * H * dv, -1, 1);
        double* dST = fill(2, (size_t)N * H * dk * dv, -1, 1);
        double* g[7];
        const size_t gn[7] = {rows * H * dk, rows * H * dk, rows * H * dv, rows * H * dk,
                              rows * H * dk, rows * H * dv, (size_t)N * H * dk * dv};
        for (int i = 0; i < 7; ++i) g[i] = calloc(gn[i] + 1, sizeof(double));
        r = gdn2_oracle_bwd(q, k, v, al, b, w, dtype, S0, dout, dtype, dST, g[0], g[1], g[2], g[3],
                            g[4], g[5], g[6], cup, packed ? nseq : 0, B, T, H, dk, dv, nthreads);
        expect(r >= 1, "bwd status");
        for (int i = 0; i < 7; ++i) expect(all_finite(g[i], gn[i]), "bwd finite");
        /* without S0 and dS_T */
        r = gdn2_oracle_bwd(q, k, v, al, b, w, dtype, NULL, dout, dtype, NULL, g[0], g[1], g[2],
                            g[3], g[4], g[5], NULL, cup, packed ? nseq : 0, B, T, H, dk, dv,
                            nthreads);
        expect(r >= 1, "bwd status without S0, dS_T");
        for (int i = 0; i < 7; ++i) free(g[i]);
        free(dout);
        free(dST);
    }
    free(q); free(k); free(v); free(al); free(b); free(w);
    free(S0); free(o); free(ST);
}

int main(void) {
    for (int dtype = 0; dtype < 3; ++dtype)
        for (int erase = 0; erase < 2; ++erase)
            for (int packed = 0; packed < 2; ++packed) run_case(dtype, erase, packed, 1 + packed);
    /* argument errors */
    double o[4], S[4], g[4];
    float x[4] = {0};
    expect(gdn2_oracle_fwd_ex(NULL, x, x, x, x, x, 0, NULL, o, S, NULL, 0, 1, 1, 1, 1, 1, NULL, 1, 0) == -1,
           "fwd null q");
    expect(gdn2_oracle_fwd_ex(x, x, x, x, x, x, 7, NULL, o, S, NULL, 0, 1, 1, 1, 1, 1, NULL, 1, 0) == -1,
           "fwd bad dtype");
    expect(gdn2_oracle_fwd_ex(x, x, x, x, x, x, 0, NULL, o, S, NULL, 0, 0, 1, 1, 1, 1, NULL, 1, 0) == -1,
           "fwd B = 0");
    expect(gdn2_oracle_bwd(x, x, x, x, x, x, 0, NULL, NULL, 0, NULL, g, g, g, g, g, g, NULL, NULL, 0,
                           1, 1, 1, 1, 1, 1) == -1, "bwd null dout");
    expect(gdn2_oracle_bwd(x, x, x, x, x, x, 0, NULL, x, 9, NULL, g, g, g, g, g, g, NULL, NULL, 0,
                           1, 1, 1, 1, 1, 1) == -1, "bwd bad dout dtype");
    /* zero tokens: S_T = S0 */
    double s0[4] = {1, 2, 3, 4}, st[4] = {0};
    int r = gdn2_oracle_fwd_ex(x, x, x, x, x, x, 0, s0, o, st, NULL, 0, 1, 0, 1, 2, 2, NULL, 1, 0);
    expect(r >= 1 && st[0] == 1 && st[3] == 4, "zero tokens pass the state through");
    if (failures == 0) printf("OK\n");
    return failures == 0 ? 0 : 1;
}

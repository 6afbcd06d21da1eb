/*
 * gdn2_oracle.c -- plain, slow, fp64 CPU oracle of the Gated Delta Rule-2
 * recurrence.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * bench's CPU-baseline leg may load it; the product path never does.  It shares
 * no code, header or constant with the HIP library.
 *
 * What it computes (per sequence n, head h, token t = 1..L), following the
 * Gated DeltaNet-2 pages:
 *
 *   step 1  S' = Diag(alpha_t) S_{t-1}
 *           The per-key-channel decay inherited from KDA is applied before the
 *           active edit (Japanese article, "core" section; Spanish blog, gate
 *           table in "Gated DeltaNet-2: La Solucion").
 *   step 2  r  = S'^T (b_t (.) k_t)
 *           The erase gate b_t acts per key channel (Korean summary, "method"
 *           step 2; Spanish blog gate table, "lado key").  Reading adopted: the
 *           gate sits on the read key of the delta rule's prediction.
 *   step 3  delta = w_t (.) v_t - r
 *           The write gate w_t acts per value channel (same passages): gated
 *           target minus gated prediction, the fast-weight view of the update
 *           (Spanish blog, "Innovaciones Tecnicas" item 3).
 *   step 4  S_t = S' + k_t delta^T
 *   step 5  o_t = S_t^T q_t
 *           Read the memory with a linear-attention query (Korean summary,
 *           "method" step 1), from the post-update state, no scale.
 *
 * Closed form: S_t = (I - k_t (b_t (.) k_t)^T) Diag(alpha_t) S_{t-1}
 *                    + k_t (w_t (.) v_t)^T.
 *
 * The pages do not settle which side of the erase product carries b_t (the
 * Spanish blog's gate table only puts b on the key side).  The reading above
 * gates the key that reads the prediction.  gdn2_oracle_fwd_ex with
 * erase_rows = 1 takes the other reading, which gates the erased rows:
 *   step 2' r = S'^T k_t                  (prediction read with the key)
 *   step 4' S_t = S' - (b_t (.) k_t) r^T + k_t (w_t (.) v_t)^T
 *   i.e. S_t = (I - (b_t (.) k_t) k_t^T) Diag(alpha_t) S_{t-1} + k_t (w_t (.) v_t)^T.
 * Both readings coincide when b_t is a scalar times 1 (Kimi Delta Attention
 * and Gated DeltaNet).
 * With b_t = w_t = beta_t * 1 it is KDA; with alpha_t also a scalar it is Gated
 * DeltaNet (Spanish blog, "Jerarquia de Generalizacion").
 *
 * Layouts (row-major, contiguous):
 *   q, k, alpha, b : [rows, H, dk]      v, w : [rows, H, dv]
 *   rows = B*T (sequence n = batch n, rows n*T .. n*T+T-1), or, with
 *   cu_seqlens (B must be 1), sequence n = rows cu[n] .. cu[n+1]-1.
 *   Storage dtype: 0 = fp32, 1 = bf16 (raw 16-bit patterns), 2 = fp64 (used
 *   by the finite-difference pins of the gradient oracle); every element is
 *   widened exactly to double.
 *   S0, S_T : [N, H, dk, dv] double (S0 may be NULL = zeros; S0 may equal S_T).
 *   o : [rows, H, dv] double.
 *
 * Work is spread over threads by independent (sequence, head) pairs only; the
 * token loop of each pair runs exactly as written above.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

static double widen(const void* p, int dtype, size_t idx) {
    if (dtype == ORC_F64) return ((const double*)p)[idx];
    if (dtype == ORC_F32) return (double)((const float*)p)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)p)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    const void *q, *k, *v, *alpha, *b, *w;
    int dtype;
    const double* S0;
    double* o;
    double* S_T;
    const int32_t* cu;
    int32_t N, T, H, dk, dv;
    const uint8_t* pair_mask;
    int erase_rows;          /* 0: b on the read key; 1: b on the erased rows */
    int32_t next;            /* next (n, h) pair to take */
    pthread_mutex_t lock;
    int failed;
} job_t;

/* One (sequence, head) pair: the five steps above, token by token. */
static int run_pair(job_t* J, int32_t n, int32_t h) {
    const int32_t H = J->H, dk = J->dk, dv = J->dv;
    const int64_t row0 = J->cu ? (int64_t)J->cu[n] : (int64_t)n * J->T;
    const int64_t len = J->cu ? (int64_t)J->cu[n + 1] - J->cu[n] : (int64_t)J->T;
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* r = (double*)malloc(sizeof(double) * (size_t)dv);
    double* delta = (double*)malloc(sizeof(double) * (size_t)dv);
    double* kv = (double*)malloc(sizeof(double) * (size_t)dk * 4);
    if (!S || !r || !delta || !kv) {
        free(S); free(r); free(delta); free(kv);
        return -1;
    }
    double *qt = kv, *kt = kv + dk, *at = kv + 2 * dk, *bt = kv + 3 * dk;
    const size_t sbase = ((size_t)n * H + h) * (size_t)dk * dv;
    for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] = J->S0 ? J->S0[sbase + e] : 0.0;

    for (int64_t t = 0; t < len; ++t) {
        const size_t row = (size_t)(row0 + t);
        const size_t kb = (row * H + h) * (size_t)dk;
        const size_t vb = (row * H + h) * (size_t)dv;
        for (int32_t i = 0; i < dk; ++i) {
            qt[i] = widen(J->q, J->dtype, kb + i);
            kt[i] = widen(J->k, J->dtype, kb + i);
            at[i] = widen(J->alpha, J->dtype, kb + i);
            bt[i] = widen(J->b, J->dtype, kb + i);
        }
        /* step 1: decay every key row of the state */
        for (int32_t i = 0; i < dk; ++i)
            for (int32_t j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= at[i];
        if (!J->erase_rows) {
            /* step 2: gated erase read r = S'^T (b (.) k) */
            for (int32_t j = 0; j < dv; ++j) r[j] = 0.0;
            for (int32_t i = 0; i < dk; ++i) {
                const double bk = bt[i] * kt[i];
                for (int32_t j = 0; j < dv; ++j) r[j] += bk * S[(size_t)i * dv + j];
            }
            /* step 3: gated write target minus prediction */
            for (int32_t j = 0; j < dv; ++j)
                delta[j] = widen(J->w, J->dtype, vb + j) * widen(J->v, J->dtype, vb + j) - r[j];
            /* step 4: rank-one edit along k */
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * delta[j];
        } else {
            /* step 2': prediction read with the key, r = S'^T k */
            for (int32_t j = 0; j < dv; ++j) r[j] = 0.0;
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j) r[j] += kt[i] * S[(size_t)i * dv + j];
            /* step 4': erase the gated rows, write along k */
            for (int32_t j = 0; j < dv; ++j)
                delta[j] = widen(J->w, J->dtype, vb + j) * widen(J->v, J->dtype, vb + j);
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j)
                    S[(size_t)i * dv + j] += kt[i] * delta[j] - (bt[i] * kt[i]) * r[j];
        }
        /* step 5: query readout from the updated state */
        for (int32_t j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int32_t i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * qt[i];
            J->o[vb + j] = acc;
        }
    }
    if (J->S_T)
        for (size_t e = 0; e < (size_t)dk * dv; ++e) J->S_T[sbase + e] = S[e];
    free(S); free(r); free(delta); free(kv);
    return 0;
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    const int32_t pairs = J->N * J->H;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int32_t p = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (p >= pairs) break;
        if (J->pair_mask && !J->pair_mask[p]) continue;
        if (run_pair(J, p / J->H, p % J->H) != 0) {
            pthread_mutex_lock(&J->lock);
            J->failed = 1;
            pthread_mutex_unlock(&J->lock);
        }
    }
    return NULL;
}

/* Returns the number of threads used (>= 1), or a negative value on bad
 * arguments (-1) or allocation failure (-2).  pair_mask (uint8 [N*H], may be
 * NULL) restricts the work to selected (sequence, head) pairs; the outputs of
 * the other pairs are left untouched.  erase_rows selects the reading of the
 * erase gate (see the top of this file). */
int gdn2_oracle_fwd_ex(const void* q, const void* k, const void* v, const void* alpha,
                       const void* b, const void* w, int dtype, const double* S0,
                       double* o, double* S_T, const int32_t* cu_seqlens, int32_t num_seqs,
                       int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                       const uint8_t* pair_mask, int32_t nthreads, int32_t erase_rows) {
    if (!q || !k || !v || !alpha || !b || !w || !o) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_F64) return -1;
    if (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1) return -1;
    if (cu_seqlens && (B != 1 || num_seqs < 0)) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.b = b; J.w = w;
    J.dtype = dtype; J.S0 = S0; J.o = o; J.S_T = S_T; J.cu = cu_seqlens;
    J.N = cu_seqlens ? num_seqs : B;
    J.T = T; J.H = H; J.dk = dk; J.dv = dv; J.pair_mask = pair_mask;
    J.erase_rows = erase_rows != 0;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads <= 0) {
        long nc = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = nc > 0 ? (int32_t)nc : 1;
    }
    const int32_t pairs = J.N * J.H;
    if (nthreads > pairs) nthreads = pairs > 0 ? pairs : 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -2;
    int32_t started = 0;
    for (int32_t i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, worker, &J) == 0) ++started;
    worker(&J);
    for (int32_t i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return J.failed ? -2 : started + 1;
}

int gdn2_oracle_fwd(const void* q, const void* k, const void* v, const void* alpha,
                    const void* b, const void* w, int dtype, const double* S0,
                    double* o, double* S_T, const int32_t* cu_seqlens, int32_t num_seqs,
                    int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                    const uint8_t* pair_mask, int32_t nthreads) {
    return gdn2_oracle_fwd_ex(q, k, v, alpha, b, w, dtype, S0, o, S_T, cu_seqlens, num_seqs, B,
                              T, H, dk, dv, pair_mask, nthreads, 0);
}

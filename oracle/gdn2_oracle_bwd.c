/*
 * gdn2_oracle_bwd.c -- plain, slow, fp64 CPU oracle of the gradients of the
 * Gated Delta Rule-2 recurrence.  TEST INFRASTRUCTURE ONLY: the tests, the
 * smoke check and the bench's CPU-baseline leg may load it; the product path
 * never does.  It shares no code, header or constant with the HIP library.
 *
 * The pages name a gate-aware backward that keeps the gradient flowing
 * through both the erase and the write gate (Spanish blog, "Innovaciones
 * Tecnicas" item 2; Korean summary, "method", closing paragraph; Japanese
 * article, "architecture and benchmarks", last paragraph).  Whatever the
 * kernel, the gradient it must produce is that of the forward recurrence
 * (gdn2_oracle.c), per sequence n, head h, token t:
 *
 *   step 1  S' = Diag(alpha_t) S_{t-1}
 *   step 2  r  = S'^T (b_t (.) k_t)
 *   step 3  delta = w_t (.) v_t - r
 *   step 4  S_t = S' + k_t delta^T
 *   step 5  o_t = S_t^T q_t
 *
 * for the scalar loss  L = sum_t <do_t, o_t> + <dS_T, S_T>  (do, dS_T given).
 * This file takes the adjoint of those five steps, token by token from the
 * last token to the first, with G = dL/dS_t carried backwards:
 *
 *   adjoint of 5:  dq_t = S_t do_t;            G += q_t do_t^T
 *   adjoint of 4:  dk_t = G delta;             d(delta) = G^T k_t;   dS' = G
 *   adjoint of 3:  dw_t = d(delta) (.) v_t;    dv_t = d(delta) (.) w_t;
 *                  dr = -d(delta)
 *   adjoint of 2:  dS' += (b_t (.) k_t) dr^T;  with e = S' dr:
 *                  db_t = e (.) k_t;           dk_t += e (.) b_t
 *   adjoint of 1:  dalpha_t[i] = sum_j dS'[i][j] S_{t-1}[i][j];
 *                  G <- Diag(alpha_t) dS'
 *
 * and dS0 = G after the first token.  The states S_{t-1} and S_t each step
 * needs are recomputed forward from checkpoints taken every 64 tokens (the
 * forward steps above, restated), so memory stays at (L/64 + 65) states per
 * (sequence, head).
 *
 * Layouts as in gdn2_oracle.c.  Storage dtypes: 0 = fp32, 1 = bf16 (raw
 * 16-bit patterns), 2 = fp64; every element is widened exactly to double.
 * do has the inputs' layout [rows, H, dv] and its own storage dtype; dS_T is
 * [N, H, dk, dv] double or NULL (= zeros); S0 as in the forward oracle.
 * Outputs (double): dq, dk, dalpha, db [rows, H, dk]; dv, dw [rows, H, dv];
 * dS0 [N, H, dk, dv] (may be NULL).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORB_F32 = 0, ORB_BF16 = 1, ORB_F64 = 2 };
enum { ORB_CKPT = 64 };

static double bwiden(const void* p, int dtype, size_t idx) {
    if (dtype == ORB_F64) return ((const double*)p)[idx];
    if (dtype == ORB_F32) return (double)((const float*)p)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)p)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    const void *q, *k, *v, *alpha, *b, *w, *dout;
    int dtype, do_dtype;
    const double *S0, *dS_T;
    double *dq, *dk, *dv, *dalpha, *db, *dw, *dS0;
    const int32_t* cu;
    int32_t N, T, H, dk_, dv_;
    int32_t next;
    pthread_mutex_t lock;
    int failed;
} bjob_t;

typedef struct {
    double *q, *k, *a, *b, *v, *w;   /* one token's inputs, widened */
} tok_t;

static void load_token(const bjob_t* J, size_t row, int32_t h, tok_t* x) {
    const size_t kb = (row * J->H + h) * (size_t)J->dk_;
    const size_t vb = (row * J->H + h) * (size_t)J->dv_;
    for (int32_t i = 0; i < J->dk_; ++i) {
        x->q[i] = bwiden(J->q, J->dtype, kb + i);
        x->k[i] = bwiden(J->k, J->dtype, kb + i);
        x->a[i] = bwiden(J->alpha, J->dtype, kb + i);
        x->b[i] = bwiden(J->b, J->dtype, kb + i);
    }
    for (int32_t j = 0; j < J->dv_; ++j) {
        x->v[j] = bwiden(J->v, J->dtype, vb + j);
        x->w[j] = bwiden(J->w, J->dtype, vb + j);
    }
}

/* forward steps 1-4 on S in place (the output of step 5 is not needed) */
static void fwd_step(int32_t dk, int32_t dv, const tok_t* x, double* S, double* r) {
    for (int32_t i = 0; i < dk; ++i)
        for (int32_t j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= x->a[i];
    for (int32_t j = 0; j < dv; ++j) r[j] = 0.0;
    for (int32_t i = 0; i < dk; ++i) {
        const double bk = x->b[i] * x->k[i];
        for (int32_t j = 0; j < dv; ++j) r[j] += bk * S[(size_t)i * dv + j];
    }
    for (int32_t j = 0; j < dv; ++j) r[j] = x->w[j] * x->v[j] - r[j];   /* delta */
    for (int32_t i = 0; i < dk; ++i)
        for (int32_t j = 0; j < dv; ++j) S[(size_t)i * dv + j] += x->k[i] * r[j];
}

static int run_pair_bwd(bjob_t* J, int32_t n, int32_t h) {
    const int32_t H = J->H, dk = J->dk_, dv = J->dv_;
    const int64_t row0 = J->cu ? (int64_t)J->cu[n] : (int64_t)n * J->T;
    const int64_t len = J->cu ? (int64_t)J->cu[n + 1] - J->cu[n] : (int64_t)J->T;
    const size_t SS = (size_t)dk * dv;
    const int64_t nblk = (len + ORB_CKPT - 1) / ORB_CKPT;
    double* ck = (double*)malloc(sizeof(double) * SS * (size_t)(nblk > 0 ? nblk : 1));
    double* st = (double*)malloc(sizeof(double) * SS * (ORB_CKPT + 1));
    double* G = (double*)malloc(sizeof(double) * SS);
    double* dSp = (double*)malloc(sizeof(double) * SS);
    double* buf = (double*)malloc(sizeof(double) * (size_t)(6 * dk + 8 * dv));
    if (!ck || !st || !G || !dSp || !buf) {
        free(ck); free(st); free(G); free(dSp); free(buf);
        return -1;
    }
    tok_t x = {buf, buf + dk, buf + 2 * dk, buf + 3 * dk, buf + 4 * dk, buf + 4 * dk + dv};
    double* e = buf + 4 * dk + 2 * dv;          /* dk */
    double* u = e + dk;                          /* dk: b (.) k */
    double* delta = u + dk;                      /* dv */
    double* ddelta = delta + dv;                 /* dv */
    double* dout = ddelta + dv;                  /* dv */
    double* r = dout + dv;                       /* dv */
    const size_t sbase = ((size_t)n * H + h) * SS;

    /* forward with a checkpoint before every block of ORB_CKPT tokens */
    double* S = st;
    for (size_t q = 0; q < SS; ++q) S[q] = J->S0 ? J->S0[sbase + q] : 0.0;
    for (int64_t t = 0; t < len; ++t) {
        if (t % ORB_CKPT == 0) memcpy(ck + (size_t)(t / ORB_CKPT) * SS, S, sizeof(double) * SS);
        load_token(J, (size_t)(row0 + t), h, &x);
        fwd_step(dk, dv, &x, S, r);
    }
    for (size_t q = 0; q < SS; ++q) G[q] = J->dS_T ? J->dS_T[sbase + q] : 0.0;

    for (int64_t blk = nblk - 1; blk >= 0; --blk) {
        const int64_t t0 = blk * ORB_CKPT;
        const int64_t t1 = t0 + ORB_CKPT < len ? t0 + ORB_CKPT : len;
        /* st[m] = S_{t0 + m - 1}: the block's states, recomputed forward */
        memcpy(st, ck + (size_t)blk * SS, sizeof(double) * SS);
        for (int64_t t = t0; t < t1; ++t) {
            memcpy(st + (size_t)(t - t0 + 1) * SS, st + (size_t)(t - t0) * SS, sizeof(double) * SS);
            load_token(J, (size_t)(row0 + t), h, &x);
            fwd_step(dk, dv, &x, st + (size_t)(t - t0 + 1) * SS, r);
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const double* Sp = st + (size_t)(t - t0) * SS;      /* S_{t-1} */
            const double* Sc = st + (size_t)(t - t0 + 1) * SS;  /* S_t */
            const size_t row = (size_t)(row0 + t);
            const size_t kb = (row * H + h) * (size_t)dk;
            const size_t vb = (row * H + h) * (size_t)dv;
            load_token(J, row, h, &x);
            for (int32_t j = 0; j < dv; ++j) dout[j] = bwiden(J->dout, J->do_dtype, vb + j);
            /* recompute delta = w (.) v - S'^T (b (.) k) */
            for (int32_t i = 0; i < dk; ++i) u[i] = x.b[i] * x.k[i];
            for (int32_t j = 0; j < dv; ++j) r[j] = 0.0;
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j) r[j] += u[i] * (x.a[i] * Sp[(size_t)i * dv + j]);
            for (int32_t j = 0; j < dv; ++j) delta[j] = x.w[j] * x.v[j] - r[j];
            /* adjoint of step 5 */
            for (int32_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) acc += Sc[(size_t)i * dv + j] * dout[j];
                J->dq[kb + i] = acc;
            }
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j) G[(size_t)i * dv + j] += x.q[i] * dout[j];
            /* adjoint of step 4 */
            for (int32_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) acc += G[(size_t)i * dv + j] * delta[j];
                J->dk[kb + i] = acc;
            }
            for (int32_t j = 0; j < dv; ++j) ddelta[j] = 0.0;
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j) ddelta[j] += G[(size_t)i * dv + j] * x.k[i];
            /* adjoint of step 3 (dr = -ddelta) */
            for (int32_t j = 0; j < dv; ++j) {
                J->dw[vb + j] = ddelta[j] * x.v[j];
                J->dv[vb + j] = ddelta[j] * x.w[j];
            }
            /* adjoint of step 2: dS' = G + u dr^T, e = S' dr */
            for (int32_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j)
                    acc += (x.a[i] * Sp[(size_t)i * dv + j]) * (-ddelta[j]);
                e[i] = acc;
            }
            for (int32_t i = 0; i < dk; ++i) {
                J->db[kb + i] = e[i] * x.k[i];
                J->dk[kb + i] += e[i] * x.b[i];
            }
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j)
                    dSp[(size_t)i * dv + j] = G[(size_t)i * dv + j] + u[i] * (-ddelta[j]);
            /* adjoint of step 1 */
            for (int32_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int32_t j = 0; j < dv; ++j) acc += dSp[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];
                J->dalpha[kb + i] = acc;
            }
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dv; ++j)
                    G[(size_t)i * dv + j] = x.a[i] * dSp[(size_t)i * dv + j];
        }
    }
    if (J->dS0)
        for (size_t q = 0; q < SS; ++q) J->dS0[sbase + q] = G[q];
    free(ck); free(st); free(G); free(dSp); free(buf);
    return 0;
}

static void* bworker(void* arg) {
    bjob_t* J = (bjob_t*)arg;
    const int32_t pairs = J->N * J->H;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int32_t p = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (p >= pairs) break;
        if (run_pair_bwd(J, p / J->H, p % J->H) != 0) {
            pthread_mutex_lock(&J->lock);
            J->failed = 1;
            pthread_mutex_unlock(&J->lock);
        }
    }
    return NULL;
}

/* Returns the number of threads used (>= 1), or -1 on bad arguments, -2 on
 * allocation failure. */
int gdn2_oracle_bwd(const void* q, const void* k, const void* v, const void* alpha,
                    const void* b, const void* w, int dtype, const double* S0,
                    const void* dout, int do_dtype, const double* dS_T, double* dq, double* dk,
                    double* dv, double* dalpha, double* db, double* dw, double* dS0,
                    const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                    int32_t dkd, int32_t dvd, int32_t nthreads) {
    if (!q || !k || !v || !alpha || !b || !w || !dout) return -1;
    if (!dq || !dk || !dv || !dalpha || !db || !dw) return -1;
    if (dtype < ORB_F32 || dtype > ORB_F64 || do_dtype < ORB_F32 || do_dtype > ORB_F64) return -1;
    if (B < 1 || T < 0 || H < 1 || dkd < 1 || dvd < 1) return -1;
    if (cu_seqlens && (B != 1 || num_seqs < 0)) return -1;
    bjob_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.b = b; J.w = w; J.dout = dout;
    J.dtype = dtype; J.do_dtype = do_dtype; J.S0 = S0; J.dS_T = dS_T;
    J.dq = dq; J.dk = dk; J.dv = dv; J.dalpha = dalpha; J.db = db; J.dw = dw; J.dS0 = dS0;
    J.cu = cu_seqlens;
    J.N = cu_seqlens ? num_seqs : B;
    J.T = T; J.H = H; J.dk_ = dkd; J.dv_ = dvd;
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
        if (pthread_create(&th[started], NULL, bworker, &J) == 0) ++started;
    bworker(&J);
    for (int32_t i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return J.failed ? -2 : started + 1;
}

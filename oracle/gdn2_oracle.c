/*
 * gdn2_oracle.c -- plain fp64 CPU reference for the Gated DeltaNet-2 recurrence.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this file's library. The product path (the HIP
 * library and its Python binding) never does, and shares no code with it.
 *
 * Sources (pages, cited by title and paragraph):
 *   [GDN2-summary] "NVIDIA представила Gated DeltaNet-2 с канал-wise гейтами для
 *                  раздельного стирания и записи в линейном внимании" (edge.aivizor.me)
 *   [GDN2-news]    "NVIDIA улучшила память LLM без роста затрат на контекст" (arddev.tech)
 *
 * What is computed, for every (batch b, head h) independently, token by token:
 *
 *   S_t = (I - k_t (b_t (.) k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t (.) v_t)^T
 *
 * [GDN2-summary, paragraph "Техническая схема ...", the state-update equation; D_t =
 * Diag(alpha_t) is the channel-wise decay]. The erase gate b_t lives on the key axis and
 * chooses which state coordinates are read and cleared; the write gate w_t lives on the
 * value axis and chooses which coordinates of the new content are committed
 * [GDN2-news, section "Аналитика", the paragraph on the key idea].
 *
 * The readout o_t = S_t^T q_t is taken on the updated state. The pages print no readout
 * formula; this is the plain reading of "the whole history is compressed into a fixed
 * recurrent state" [GDN2-news, section "Контекст"] for a linear-attention layer.
 *
 * The steps below are the equation applied right to left, each written out on its own:
 *   1. decay        S <- Diag(alpha_t) S
 *   2. erase read   r <- S^T (b_t (.) k_t)
 *   3. erase        S <- S - k_t r^T          (together: (I - k_t (b_t(.)k_t)^T) D_t S_{t-1})
 *   4. write        S <- S + k_t (w_t (.) v_t)^T
 *   5. readout      o_t <- S^T q_t
 *
 * Layouts (row-major, contiguous): q, k, alpha, b are [B, T, H, d_k]; v, w and o are
 * [B, T, H, d_v]; S0 and S_out are [B, H, d_k, d_v]. All arrays are float64. S0 == NULL
 * means a zero initial state; S_out == NULL means the final state is not stored.
 *
 * A decode step is the same loop with T = 1 (a [B, H, d] array is a [B, 1, H, d] array).
 * Parallelism: the (b, h) sequences are independent; they are spread over POSIX threads.
 */
#include <pthread.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *alpha, *b, *w, *S0;
    double *o, *S_out;
    long B, T, H, dk, dv;
    long first, stride; /* this worker's (b,h) items: first, first+stride, ... */
    int status;
} oracle_job;

static void run_one_sequence(const oracle_job *j, long bh, double *S, double *r) {
    const long bb = bh / j->H, hh = bh % j->H;
    const long dk = j->dk, dv = j->dv;

    /* initial state */
    if (j->S0) {
        memcpy(S, j->S0 + bh * dk * dv, sizeof(double) * (size_t)(dk * dv));
    } else {
        memset(S, 0, sizeof(double) * (size_t)(dk * dv));
    }

    for (long t = 0; t < j->T; ++t) {
        const long tok = (bb * j->T + t) * j->H + hh; /* index of (b, t, h) */
        const double *q = j->q + tok * dk;
        const double *k = j->k + tok * dk;
        const double *a = j->alpha + tok * dk;
        const double *be = j->b + tok * dk;
        const double *v = j->v + tok * dv;
        const double *w = j->w + tok * dv;
        double *o = j->o ? j->o + tok * dv : NULL;

        /* 1. decay: row i of S (key channel i) is scaled by alpha_t[i] */
        for (long i = 0; i < dk; ++i)
            for (long c = 0; c < dv; ++c) S[i * dv + c] *= a[i];

        /* 2. erase read: r = S^T (b_t (.) k_t) */
        for (long c = 0; c < dv; ++c) r[c] = 0.0;
        for (long i = 0; i < dk; ++i) {
            const double e = be[i] * k[i];
            for (long c = 0; c < dv; ++c) r[c] += e * S[i * dv + c];
        }

        /* 3. erase: S <- S - k_t r^T */
        for (long i = 0; i < dk; ++i)
            for (long c = 0; c < dv; ++c) S[i * dv + c] -= k[i] * r[c];

        /* 4. write: S <- S + k_t (w_t (.) v_t)^T */
        for (long i = 0; i < dk; ++i)
            for (long c = 0; c < dv; ++c) S[i * dv + c] += k[i] * (w[c] * v[c]);

        /* 5. readout on the updated state: o_t = S^T q_t */
        if (o) {
            for (long c = 0; c < dv; ++c) o[c] = 0.0;
            for (long i = 0; i < dk; ++i)
                for (long c = 0; c < dv; ++c) o[c] += q[i] * S[i * dv + c];
        }
    }

    if (j->S_out) memcpy(j->S_out + bh * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
}

static void *worker(void *arg) {
    oracle_job *j = (oracle_job *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)(j->dk * j->dv));
    double *r = (double *)malloc(sizeof(double) * (size_t)j->dv);
    if (!S || !r) {
        free(S);
        free(r);
        j->status = 2;
        return NULL;
    }
    for (long bh = j->first; bh < j->B * j->H; bh += j->stride) run_one_sequence(j, bh, S, r);
    free(S);
    free(r);
    j->status = 0;
    return NULL;
}

/*
 * Runs the recurrence over all (b, h). Returns 0 on success, 1 on bad arguments,
 * 2 when memory or threads could not be obtained. `threads` <= 0 means one thread.
 * S_out may alias S0 (each sequence reads its S0 slice before writing its S_out slice,
 * and no two sequences share a slice).
 */
int gdn2_oracle_forward(const double *q, const double *k, const double *v, const double *alpha,
                        const double *b, const double *w, const double *S0, double *o,
                        double *S_out, long B, long T, long H, long dk, long dv, int threads) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return 1;
    if (T > 0 && (!q || !k || !v || !alpha || !b || !w)) return 1;
    const long items = B * H;
    if (items == 0) return 0;
    if (threads <= 0) threads = 1;
    if (threads > items) threads = (int)items;

    oracle_job *jobs = (oracle_job *)calloc((size_t)threads, sizeof(oracle_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return 2;
    }
    int rc = 0, started = 0;
    for (int i = 0; i < threads; ++i) {
        oracle_job j = {q, k, v, alpha, b, w, S0, o, S_out, B, T, H, dk, dv, i, threads, 2};
        jobs[i] = j;
        if (pthread_create(&tid[i], NULL, worker, &jobs[i]) != 0) {
            rc = 2;
            break;
        }
        ++started;
    }
    for (int i = 0; i < started; ++i) {
        pthread_join(tid[i], NULL);
        if (jobs[i].status != 0) rc = 2;
    }
    free(jobs);
    free(tid);
    return rc;
}

/*
 * Backward: the reverse mode of the same recurrence, for the scalar loss
 *
 *   L = sum_t <dO_t, o_t> + <dS_T, S_T>
 *
 * (dO = [B, T, H, d_v] output cotangents, dS_T = [B, H, d_k, d_v] final-state cotangent,
 * NULL = zeros). It returns dL/dq, dL/dk, dL/dalpha, dL/db ([B, T, H, d_k]), dL/dv, dL/dw
 * ([B, T, H, d_v]) and dL/dS0 ([B, H, d_k, d_v]). The derivative of the recurrence is the plain
 * definition: each of the five forward steps above is replaced by its adjoint, and the
 * adjoints run in the reverse order over the tokens, with G = dL/dS carried backwards.
 * For token t with P = S_{t-1} (the state before it):
 *   recompute  X = Diag(alpha) P,  c = b (.) k,  r = X^T c,  u = w (.) v,  S_t = X - k r^T + k u^T
 *   5'. readout      dq = S_t dO_t;                  G += q dO_t^T
 *   4'. write        dk += G u;  du = G^T k;         dv = w (.) du,  dw = v (.) du
 *   3'. erase        dk -= G r;  dr = -G^T k;        (dX = G so far)
 *   2'. erase read   dX = G + c dr^T;  dc = X dr;    db = k (.) dc,  dk += b (.) dc
 *   1'. decay        dalpha_i = sum_c P_ic dX_ic;    G <- Diag(alpha) dX   (= dL/dS_{t-1})
 * The states before each token are recomputed forward from checkpoints kept every 64 tokens,
 * so a sequence needs (T / 64 + 64) states of memory.
 */
enum { BWD_SEG = 64 };

typedef struct {
    const double *q, *k, *v, *alpha, *b, *w, *S0, *dO, *dST;
    double *dq, *dk, *dalpha, *db, *dv, *dw, *dS0;
    long B, T, H, dk_, dv_;
    long first, stride;
    int status;
} bwd_job;

/* one forward token step on S (in place), the five steps above without the readout */
static void step_forward(double *S, const double *k, const double *a, const double *be,
                         const double *v, const double *w, long dk, long dv, double *r) {
    for (long i = 0; i < dk; ++i)
        for (long c = 0; c < dv; ++c) S[i * dv + c] *= a[i];
    for (long c = 0; c < dv; ++c) r[c] = 0.0;
    for (long i = 0; i < dk; ++i) {
        const double e = be[i] * k[i];
        for (long c = 0; c < dv; ++c) r[c] += e * S[i * dv + c];
    }
    for (long i = 0; i < dk; ++i)
        for (long c = 0; c < dv; ++c) S[i * dv + c] += k[i] * (w[c] * v[c] - r[c]);
}

static int backward_one_sequence(const bwd_job *j, long bh) {
    const long bb = bh / j->H, hh = bh % j->H;
    const long dk = j->dk_, dv = j->dv_, T = j->T, n = dk * dv;
    const long nseg = (T + BWD_SEG - 1) / BWD_SEG;
    double *ck = (double *)malloc(sizeof(double) * (size_t)(n * (nseg > 0 ? nseg : 1)));
    double *seg = (double *)malloc(sizeof(double) * (size_t)(n * (BWD_SEG + 1)));
    double *G = (double *)malloc(sizeof(double) * (size_t)n);
    double *X = (double *)malloc(sizeof(double) * (size_t)n);
    double *St = (double *)malloc(sizeof(double) * (size_t)n);
    double *vec = (double *)malloc(sizeof(double) * (size_t)(3 * dv + 2 * dk));
    if (!ck || !seg || !G || !X || !St || !vec) {
        free(ck); free(seg); free(G); free(X); free(St); free(vec);
        return 2;
    }
    double *r = vec, *du = vec + dv, *dr = vec + 2 * dv, *cvec = vec + 3 * dv, *dc = cvec + dk;

    /* checkpoints: the state before token 64 m */
    double *S = seg; /* scratch for the forward sweep */
    if (j->S0) memcpy(S, j->S0 + bh * n, sizeof(double) * (size_t)n);
    else memset(S, 0, sizeof(double) * (size_t)n);
    for (long t = 0; t < T; ++t) {
        if (t % BWD_SEG == 0) memcpy(ck + (t / BWD_SEG) * n, S, sizeof(double) * (size_t)n);
        const long tok = (bb * T + t) * j->H + hh;
        step_forward(S, j->k + tok * dk, j->alpha + tok * dk, j->b + tok * dk, j->v + tok * dv,
                     j->w + tok * dv, dk, dv, r);
    }

    /* G = dL/dS_T */
    if (j->dST) memcpy(G, j->dST + bh * n, sizeof(double) * (size_t)n);
    else memset(G, 0, sizeof(double) * (size_t)n);

    for (long m = nseg - 1; m >= 0; --m) {
        const long t0 = m * BWD_SEG, t1 = (t0 + BWD_SEG < T) ? t0 + BWD_SEG : T;
        /* states before tokens t0 .. t1-1 */
        memcpy(seg, ck + m * n, sizeof(double) * (size_t)n);
        for (long t = t0; t + 1 < t1; ++t) {
            const long tok = (bb * T + t) * j->H + hh;
            memcpy(seg + (t - t0 + 1) * n, seg + (t - t0) * n, sizeof(double) * (size_t)n);
            step_forward(seg + (t - t0 + 1) * n, j->k + tok * dk, j->alpha + tok * dk,
                         j->b + tok * dk, j->v + tok * dv, j->w + tok * dv, dk, dv, r);
        }
        for (long t = t1 - 1; t >= t0; --t) {
            const long tok = (bb * T + t) * j->H + hh;
            const double *P = seg + (t - t0) * n;
            const double *q = j->q + tok * dk, *k = j->k + tok * dk, *a = j->alpha + tok * dk;
            const double *be = j->b + tok * dk, *v = j->v + tok * dv, *w = j->w + tok * dv;
            const double *dO = j->dO ? j->dO + tok * dv : NULL;
            double *dq = j->dq + tok * dk, *dk_o = j->dk + tok * dk, *da = j->dalpha + tok * dk;
            double *db = j->db + tok * dk, *dv_o = j->dv + tok * dv, *dw = j->dw + tok * dv;

            /* recompute X, c, r and S_t */
            for (long i = 0; i < n; ++i) X[i] = 0.0;
            for (long i = 0; i < dk; ++i)
                for (long c = 0; c < dv; ++c) X[i * dv + c] = a[i] * P[i * dv + c];
            for (long i = 0; i < dk; ++i) cvec[i] = be[i] * k[i];
            for (long c = 0; c < dv; ++c) r[c] = 0.0;
            for (long i = 0; i < dk; ++i)
                for (long c = 0; c < dv; ++c) r[c] += cvec[i] * X[i * dv + c];
            for (long i = 0; i < dk; ++i)
                for (long c = 0; c < dv; ++c)
                    St[i * dv + c] = X[i * dv + c] - k[i] * r[c] + k[i] * (w[c] * v[c]);

            /* 5'. readout: dq = S_t dO_t, G += q dO_t^T */
            for (long i = 0; i < dk; ++i) {
                double acc = 0.0;
                if (dO)
                    for (long c = 0; c < dv; ++c) acc += St[i * dv + c] * dO[c];
                dq[i] = acc;
            }
            if (dO)
                for (long i = 0; i < dk; ++i)
                    for (long c = 0; c < dv; ++c) G[i * dv + c] += q[i] * dO[c];

            /* 4'. write: dk = G u, du = G^T k, dv = w du, dw = v du */
            for (long i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (long c = 0; c < dv; ++c) acc += G[i * dv + c] * (w[c] * v[c]);
                dk_o[i] = acc;
            }
            for (long c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (long i = 0; i < dk; ++i) acc += G[i * dv + c] * k[i];
                du[c] = acc;
                dv_o[c] = w[c] * acc;
                dw[c] = v[c] * acc;
            }

            /* 3'. erase: dk -= G r, dr = -G^T k */
            for (long i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (long c = 0; c < dv; ++c) acc += G[i * dv + c] * r[c];
                dk_o[i] -= acc;
            }
            for (long c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (long i = 0; i < dk; ++i) acc += G[i * dv + c] * k[i];
                dr[c] = -acc;
            }

            /* 2'. erase read: dX = G + c dr^T (in G), dc = X dr, db = k dc, dk += b dc */
            for (long i = 0; i < dk; ++i)
                for (long c = 0; c < dv; ++c) G[i * dv + c] += cvec[i] * dr[c];
            for (long i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (long c = 0; c < dv; ++c) acc += X[i * dv + c] * dr[c];
                dc[i] = acc;
                db[i] = k[i] * acc;
                dk_o[i] += be[i] * acc;
            }

            /* 1'. decay: dalpha_i = sum_c P_ic dX_ic, G <- Diag(alpha) dX */
            for (long i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (long c = 0; c < dv; ++c) acc += P[i * dv + c] * G[i * dv + c];
                da[i] = acc;
                for (long c = 0; c < dv; ++c) G[i * dv + c] *= a[i];
            }
        }
    }
    if (j->dS0) memcpy(j->dS0 + bh * n, G, sizeof(double) * (size_t)n);
    free(ck); free(seg); free(G); free(X); free(St); free(vec);
    return 0;
}

static void *bwd_worker(void *arg) {
    bwd_job *j = (bwd_job *)arg;
    j->status = 0;
    for (long bh = j->first; bh < j->B * j->H; bh += j->stride)
        if (backward_one_sequence(j, bh) != 0) {
            j->status = 2;
            break;
        }
    return NULL;
}

/*
 * Gradients of L over all (b, h). Returns 0 on success, 1 on bad arguments, 2 when memory or
 * threads could not be obtained. dO, dS_T and S0 may be NULL (zeros); dS0 may be NULL (not
 * stored). Every other output must be given.
 */
int gdn2_oracle_backward(const double *q, const double *k, const double *v, const double *alpha,
                         const double *b, const double *w, const double *S0, const double *dO,
                         const double *dS_T, double *dq, double *dk, double *dalpha, double *db,
                         double *dv, double *dw, double *dS0, long B, long T, long H, long dk_,
                         long dv_, int threads) {
    if (B < 0 || T < 0 || H < 0 || dk_ <= 0 || dv_ <= 0) return 1;
    if (T > 0 && (!q || !k || !v || !alpha || !b || !w || !dq || !dk || !dalpha || !db || !dv || !dw))
        return 1;
    const long items = B * H;
    if (items == 0) return 0;
    if (threads <= 0) threads = 1;
    if (threads > items) threads = (int)items;
    bwd_job *jobs = (bwd_job *)calloc((size_t)threads, sizeof(bwd_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return 2;
    }
    int rc = 0, started = 0;
    for (int i = 0; i < threads; ++i) {
        bwd_job jb = {q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk, dalpha, db, dv, dw, dS0,
                      B, T, H, dk_, dv_, i, threads, 2};
        jobs[i] = jb;
        if (pthread_create(&tid[i], NULL, bwd_worker, &jobs[i]) != 0) {
            rc = 2;
            break;
        }
        ++started;
    }
    for (int i = 0; i < started; ++i) {
        pthread_join(tid[i], NULL);
        if (jobs[i].status != 0) rc = 2;
    }
    free(jobs);
    free(tid);
    return rc;
}

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

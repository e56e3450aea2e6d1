/*
 * lcd_oracle_bench.c -- times the CPU oracle on the host's cores.
 *
 * TEST INFRASTRUCTURE ONLY (the CPU-baseline leg of the benchmark).  It calls
 * the oracle's own exported functions unchanged -- lookup, fusion, greedy
 * acceptance and the scheduler, one request at a time -- and adds nothing to
 * their arithmetic: it only spreads the requests of each decode step over
 * native threads and measures wall and CPU time.
 *
 * Two workloads, one runner.  A greedy decode step (oracle_bench_steps) is
 * every request of the batch once: lookup on its history, fusion of the draft
 * with the draft model's proposal, greedy acceptance against the target
 * tokens (no append, so every step sees the same histories) and one scheduler
 * update.  A sampled-verification step (oracle_bench_rejection) is the
 * oracle's rejection_accept on every request once (no append).  Threads take
 * requests from a shared counter (largest first, so the step's tail is short)
 * and meet at a barrier after each step; the main thread stops after the first
 * step that ends past the time budget.
 */
#define _GNU_SOURCE
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#define ORACLE_DRAFT_STRIDE 15
#define ORACLE_Q_STRIDE 7
#define ORACLE_TARGET_STRIDE 16

typedef struct oracle_params {
    int32_t l_min, l_max, k_max;
    int32_t n_head, n_block;
    int32_t head_full, head_agree, agree_n, tail_min;
    int32_t entry_steps, sticky, near_full_slack;
} oracle_params;

int oracle_lookup_propose(const int32_t *hist, const int64_t *row_off, const int32_t *len,
                          int32_t B, const oracle_params *p, int32_t *match_len,
                          int32_t *match_end, int32_t *draft);
int oracle_fuse_verify_block(const int32_t *draft, const int32_t *match_len, const int32_t *q,
                             const int32_t *long_mode, int32_t B, const oracle_params *p,
                             int32_t *block, int32_t *block_len, uint32_t *model_mask);
int oracle_greedy_accept(const int32_t *block, const int32_t *block_len, const int32_t *target,
                         int32_t B, int32_t *accept, int32_t *hist, const int64_t *row_off,
                         int32_t *len, const int32_t *cap);
int oracle_lookup_schedule_step(int32_t *state, const int32_t *match_len, const int32_t *accept,
                                const int32_t *block_len, int32_t B, const oracle_params *p,
                                int32_t *long_next);
int oracle_rejection_accept(const int32_t *block, const int32_t *block_len,
                            const uint32_t *model_mask, const float *target_probs,
                            const float *model_probs, int32_t V, const double *u_accept,
                            const uint64_t *u_sample, int32_t B, int32_t *accept,
                            int32_t *emitted, int32_t *hist, const int64_t *row_off,
                            int32_t *len, const int32_t *cap);

/* One request's share of a step: adds what it computed to *sum (a checksum
 * that keeps the results live). */
typedef void (*request_fn)(const void *ctx, int32_t r, int64_t *sum);

typedef struct {
    request_fn fn;
    const void *ctx;
    const int32_t *order;          /* requests, largest first */
    int32_t B;
    int32_t nthreads;
    volatile int stop;
    int next;                      /* next entry of `order` this step (atomic) */
    pthread_mutex_t gate;          /* held by the main thread until the barriers exist */
    pthread_barrier_t start, done;
    int64_t checksum;
} shared_t;

typedef struct {
    const int32_t *hist;
    const int64_t *row_off;
    const int32_t *len;
    const int32_t *q;
    const int32_t *target;
    const oracle_params *p;
} lookup_ctx;

/* lookup, fusion, greedy acceptance and scheduler of request r */
static void lookup_request(const void *ctx, int32_t r, int64_t *sum) {
    const lookup_ctx *c = (const lookup_ctx *)ctx;
    int32_t m, e, d[ORACLE_DRAFT_STRIDE], blk[ORACLE_DRAFT_STRIDE], bl, acc, st[3] = {0, 0, 0};
    int32_t lmode = 0, ln;
    oracle_lookup_propose(c->hist, c->row_off + r, c->len + r, 1, c->p, &m, &e, d);
    oracle_fuse_verify_block(d, &m, c->q + (int64_t)r * ORACLE_Q_STRIDE, &lmode, 1, c->p, blk, &bl,
                             NULL);
    oracle_greedy_accept(blk, &bl, c->target + (int64_t)r * ORACLE_TARGET_STRIDE, 1, &acc, NULL,
                         NULL, NULL, NULL);
    oracle_lookup_schedule_step(st, &m, &acc, &bl, 1, c->p, &ln);
    *sum += m + acc + ln;
}

typedef struct {
    const int32_t *block, *block_len;
    const uint32_t *model_mask;    /* nullable */
    const float *target_probs, *model_probs;   /* model_probs nullable */
    int32_t V;
    const double *u_accept;
    const uint64_t *u_sample;
} rejection_ctx;

/* sampled verification of request r (no append) */
static void rejection_request(const void *ctx, int32_t r, int64_t *sum) {
    const rejection_ctx *c = (const rejection_ctx *)ctx;
    int32_t acc, em[ORACLE_TARGET_STRIDE];
    oracle_rejection_accept(c->block + (int64_t)r * ORACLE_DRAFT_STRIDE, c->block_len + r,
                            c->model_mask ? c->model_mask + r : NULL,
                            c->target_probs + (int64_t)r * ORACLE_TARGET_STRIDE * c->V,
                            c->model_probs ? c->model_probs + (int64_t)r * ORACLE_Q_STRIDE * c->V : NULL,
                            c->V, c->u_accept + (int64_t)r * ORACLE_DRAFT_STRIDE, c->u_sample + r, 1,
                            &acc, em, NULL, NULL, NULL, NULL);
    *sum += acc;
    for (int k = 0; k < ORACLE_TARGET_STRIDE; ++k) *sum += em[k];
}

static void *worker(void *arg) {
    shared_t *s = (shared_t *)arg;
    int64_t sum = 0;
    pthread_mutex_lock(&s->gate);
    pthread_mutex_unlock(&s->gate);
    for (;;) {
        pthread_barrier_wait(&s->start);
        if (s->stop) break;
        for (;;) {
            const int i = __atomic_fetch_add(&s->next, 1, __ATOMIC_RELAXED);
            if (i >= s->B) break;
            s->fn(s->ctx, s->order[i], &sum);
        }
        pthread_barrier_wait(&s->done);
    }
    __atomic_fetch_add(&s->checksum, sum, __ATOMIC_RELAXED);
    return NULL;
}

static double now(clockid_t c) {
    struct timespec ts;
    clock_gettime(c, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

static int by_len_desc(const void *a, const void *b, void *len) {
    const int32_t *l = (const int32_t *)len;
    const int32_t x = l[*(const int32_t *)a], y = l[*(const int32_t *)b];
    return (x < y) - (x > y);
}

/*
 * Runs whole steps (fn over every request of `order`) on `nthreads` threads
 * until `min_seconds` of wall time have passed (at least one step, at most
 * max_steps).  Takes ownership of `order`.  Outputs: steps run, wall seconds,
 * process CPU seconds and a checksum of the results (so nothing is optimised
 * away).  Returns 0, or -1 when threads cannot be created.
 */
static int run_steps(request_fn fn, const void *ctx, int32_t *order, int32_t B, int32_t nthreads,
                     double min_seconds, int32_t max_steps, int64_t *steps_out, double *wall_out,
                     double *cpu_out, int64_t *checksum) {
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) {
        free(order);
        return -1;
    }
    shared_t s;
    memset(&s, 0, sizeof(s));
    s.fn = fn;
    s.ctx = ctx;
    s.order = order;
    s.B = B;
    pthread_mutex_init(&s.gate, NULL);
    pthread_mutex_lock(&s.gate);
    int made = 0;
    for (; made < nthreads; ++made)
        if (pthread_create(&th[made], NULL, worker, &s) != 0) break;
    /* the workers wait at the gate until the barriers are sized to them */
    s.nthreads = made;
    const int rc = made == nthreads ? 0 : -1;
    pthread_barrier_init(&s.start, NULL, (unsigned)made + 1);
    pthread_barrier_init(&s.done, NULL, (unsigned)made + 1);
    s.stop = rc != 0;                  /* a short pool runs no step */
    pthread_mutex_unlock(&s.gate);
    const double w0 = now(CLOCK_MONOTONIC), c0 = now(CLOCK_PROCESS_CPUTIME_ID);
    int64_t steps = 0;
    while (!s.stop) {
        s.next = 0;
        pthread_barrier_wait(&s.start);
        pthread_barrier_wait(&s.done);
        ++steps;
        if (now(CLOCK_MONOTONIC) - w0 >= min_seconds || steps >= max_steps) s.stop = 1;
    }
    pthread_barrier_wait(&s.start);    /* releases the workers, which see stop */
    const double w1 = now(CLOCK_MONOTONIC), c1 = now(CLOCK_PROCESS_CPUTIME_ID);
    for (int i = 0; i < made; ++i) pthread_join(th[i], NULL);
    pthread_barrier_destroy(&s.start);
    pthread_barrier_destroy(&s.done);
    pthread_mutex_destroy(&s.gate);
    *steps_out = steps;
    *wall_out = w1 - w0;
    *cpu_out = c1 - c0;
    *checksum = s.checksum;
    free(order);
    free(th);
    return rc;
}

/*
 * Greedy decode steps of the batch (see the top of the file): requests by
 * history length, largest first.  Returns 0, or -1 for bad arguments or when
 * threads cannot be created.
 */
int oracle_bench_steps(const int32_t *hist, const int64_t *row_off, const int32_t *len, int32_t B,
                       const int32_t *q, const int32_t *target, const oracle_params *p,
                       int32_t nthreads, double min_seconds, int32_t max_steps,
                       int64_t *steps_out, double *wall_out, double *cpu_out, int64_t *checksum) {
    if (B <= 0 || nthreads <= 0 || max_steps <= 0 || !hist || !row_off || !len || !q || !target ||
        !p || !steps_out || !wall_out || !cpu_out || !checksum)
        return -1;
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)B);
    if (!order) return -1;
    for (int32_t r = 0; r < B; ++r) order[r] = r;
    qsort_r(order, (size_t)B, sizeof(int32_t), by_len_desc, (void *)len);
    const lookup_ctx c = {hist, row_off, len, q, target, p};
    return run_steps(lookup_request, &c, order, B, nthreads, min_seconds, max_steps, steps_out,
                     wall_out, cpu_out, checksum);
}

/*
 * Sampled-verification steps of the batch: oracle_rejection_accept on every
 * request (no append), requests with a draft-model row first (their draw may
 * read two rows).  Returns 0, or -1 for bad arguments or when threads cannot
 * be created.
 */
int oracle_bench_rejection(const int32_t *block, const int32_t *block_len,
                           const uint32_t *model_mask, const float *target_probs,
                           const float *model_probs, int32_t V, const double *u_accept,
                           const uint64_t *u_sample, int32_t B, int32_t nthreads,
                           double min_seconds, int32_t max_steps, int64_t *steps_out,
                           double *wall_out, double *cpu_out, int64_t *checksum) {
    if (B <= 0 || V <= 0 || nthreads <= 0 || max_steps <= 0 || !block || !block_len ||
        !target_probs || !u_accept || !u_sample || !steps_out || !wall_out || !cpu_out || !checksum)
        return -1;
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)B);
    if (!order) return -1;
    int32_t k = 0;
    for (int pass = 0; pass < 2; ++pass)
        for (int32_t r = 0; r < B; ++r) {
            const int with_model = model_mask && model_probs && model_mask[r] != 0;
            if (with_model == (pass == 0)) order[k++] = r;
        }
    const rejection_ctx c = {block, block_len, model_mask, target_probs, model_probs, V, u_accept,
                             u_sample};
    return run_steps(rejection_request, &c, order, B, nthreads, min_seconds, max_steps, steps_out,
                     wall_out, cpu_out, checksum);
}

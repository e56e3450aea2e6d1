/*
 * oracle_sanitize_main.c -- drives every function of the CPU oracle
 * (oracle/lcd_oracle.c, oracle/lcd_oracle_bench.c) over seeded random and
 * edge-case inputs held in heap buffers of exactly the size each call may
 * touch, and prints a checksum of all outputs.  tests/test_oracle_sanitized.py
 * builds it twice -- plain, and with AddressSanitizer and UndefinedBehavior
 * Sanitizer -- and requires a clean sanitized run with the same checksum.
 *
 * Inputs: histories over alphabets of 1..6 ids (so matches of every length
 * occur) with lengths 0..400 and some negative lengths, every parameter at its
 * edges (l_min 1..4, l_max up to 16, k_max 0..15, short and long blocks),
 * appends that fit and that overflow their row, scheduler states in both
 * modes, telemetry classes outside the range, and probability rows with NaN,
 * negative, infinite, above-one and all-zero entries.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct oracle_params {
    int32_t l_min, l_max, k_max;
    int32_t n_head, n_block;
    int32_t head_full, head_agree, agree_n, tail_min;
    int32_t entry_steps, sticky, near_full_slack;
} oracle_params;

int oracle_lookup_propose(const int32_t *, const int64_t *, const int32_t *, int32_t,
                          const oracle_params *, int32_t *, int32_t *, int32_t *);
int oracle_fuse_verify_block(const int32_t *, const int32_t *, const int32_t *, const int32_t *,
                             int32_t, const oracle_params *, int32_t *, int32_t *, uint32_t *);
int oracle_greedy_accept(const int32_t *, const int32_t *, const int32_t *, int32_t, int32_t *,
                         int32_t *, const int64_t *, int32_t *, const int32_t *);
int oracle_rejection_accept(const int32_t *, const int32_t *, const uint32_t *, const float *,
                            const float *, int32_t, const double *, const uint64_t *, int32_t,
                            int32_t *, int32_t *, int32_t *, const int64_t *, int32_t *,
                            const int32_t *);
int oracle_lookup_schedule_step(int32_t *, const int32_t *, const int32_t *, const int32_t *,
                                int32_t, const oracle_params *, int32_t *);
int oracle_telemetry_update(uint32_t *, const int32_t *, const int32_t *, const int32_t *,
                            const int32_t *, const int32_t *, const int32_t *, const int32_t *,
                            int32_t, const oracle_params *);
int oracle_telemetry_reduce(const uint32_t *, const int32_t *, int32_t, int32_t, uint64_t *);
int oracle_bench_steps(const int32_t *, const int64_t *, const int32_t *, int32_t, const int32_t *,
                       const int32_t *, const oracle_params *, int32_t, double, int32_t, int64_t *,
                       double *, double *, int64_t *);
int oracle_bench_rejection(const int32_t *, const int32_t *, const uint32_t *, const float *,
                           const float *, int32_t, const double *, const uint64_t *, int32_t,
                           int32_t, double, int32_t, int64_t *, double *, double *, int64_t *);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {                 /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int32_t uni(int32_t lo, int32_t hi) { /* [lo, hi] */
    return lo + (int32_t)(next_u64() % (uint64_t)(hi - lo + 1));
}

static uint64_t sum = 1469598103934665603ull;     /* FNV-1a over all outputs */
static void mix(const void *p, size_t n) {
    const unsigned char *c = (const unsigned char *)p;
    for (size_t i = 0; i < n; ++i) sum = (sum ^ c[i]) * 1099511628211ull;
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

static oracle_params random_params(void) {
    oracle_params p;
    p.l_min = uni(1, 4);
    p.l_max = uni(p.l_min, 16);
    p.k_max = uni(0, 15);
    p.n_head = uni(1, 7);
    p.n_block = uni(p.n_head, 15);
    p.head_full = uni(1, 16);
    p.head_agree = uni(1, 16);
    p.agree_n = uni(0, p.n_head);
    p.tail_min = uni(1, 16);
    p.entry_steps = uni(1, 4);
    p.sticky = uni(0, 4);
    p.near_full_slack = uni(0, 3);
    return p;
}

/* One round of lookup, fusion, acceptance with append, scheduling and
 * telemetry on a fresh random batch. */
static void step_round(void) {
    const int32_t B = uni(1, 24);
    const oracle_params p = random_params();
    const int32_t alpha = uni(1, 6);
    int32_t *len = (int32_t *)xmalloc(sizeof(int32_t) * B);
    int32_t *cap = (int32_t *)xmalloc(sizeof(int32_t) * B);
    int64_t *row_off = (int64_t *)xmalloc(sizeof(int64_t) * B);
    int64_t total = 0;
    for (int32_t r = 0; r < B; ++r) {
        const int32_t n = uni(0, 400);
        len[r] = (uni(0, 9) == 0) ? -uni(1, 5) : n;          /* some negative lengths */
        const int32_t have = len[r] > 0 ? len[r] : 0;
        cap[r] = have + uni(0, 20);                          /* some appends overflow */
        row_off[r] = total;
        total += cap[r];
    }
    int32_t *hist = (int32_t *)xmalloc(sizeof(int32_t) * (size_t)total);
    for (int64_t i = 0; i < total; ++i) hist[i] = uni(0, alpha - 1);
    int32_t *m = (int32_t *)xmalloc(sizeof(int32_t) * B), *e = (int32_t *)xmalloc(sizeof(int32_t) * B);
    int32_t *d = (int32_t *)xmalloc(sizeof(int32_t) * B * 15);
    oracle_lookup_propose(hist, row_off, len, B, &p, m, e, d);
    mix(m, sizeof(int32_t) * B); mix(e, sizeof(int32_t) * B); mix(d, sizeof(int32_t) * B * 15);

    int32_t *q = (int32_t *)xmalloc(sizeof(int32_t) * B * 7);
    int32_t *lm = (int32_t *)xmalloc(sizeof(int32_t) * B);
    int32_t *tgt = (int32_t *)xmalloc(sizeof(int32_t) * B * 16);
    for (int32_t i = 0; i < B * 7; ++i) q[i] = uni(0, alpha - 1);
    for (int32_t i = 0; i < B * 16; ++i) tgt[i] = uni(0, alpha - 1);
    for (int32_t r = 0; r < B; ++r) lm[r] = uni(0, 1);
    int32_t *blk = (int32_t *)xmalloc(sizeof(int32_t) * B * 15), *bl = (int32_t *)xmalloc(sizeof(int32_t) * B);
    uint32_t *mm = (uint32_t *)xmalloc(sizeof(uint32_t) * B);
    oracle_fuse_verify_block(d, m, q, lm, B, &p, blk, bl, mm);
    mix(blk, sizeof(int32_t) * B * 15); mix(bl, sizeof(int32_t) * B); mix(mm, sizeof(uint32_t) * B);

    int32_t *acc = (int32_t *)xmalloc(sizeof(int32_t) * B);
    oracle_greedy_accept(blk, bl, tgt, B, acc, NULL, NULL, NULL, NULL);
    mix(acc, sizeof(int32_t) * B);
    oracle_greedy_accept(blk, bl, tgt, B, acc, hist, row_off, len, cap);
    mix(acc, sizeof(int32_t) * B); mix(len, sizeof(int32_t) * B); mix(hist, sizeof(int32_t) * (size_t)total);

    int32_t *st = (int32_t *)xmalloc(sizeof(int32_t) * B * 3), *ln = (int32_t *)xmalloc(sizeof(int32_t) * B);
    for (int32_t r = 0; r < B; ++r) {
        st[3 * r] = uni(0, 1); st[3 * r + 1] = uni(0, 3); st[3 * r + 2] = uni(0, 5);
    }
    oracle_lookup_schedule_step(st, m, acc, bl, B, &p, ln);
    mix(st, sizeof(int32_t) * B * 3); mix(ln, sizeof(int32_t) * B);

    uint32_t *tele = (uint32_t *)xmalloc(sizeof(uint32_t) * B * 32);
    memset(tele, 0, sizeof(uint32_t) * B * 32);
    oracle_telemetry_update(tele, m, d, q, lm, bl, acc, ln, B, &p);
    mix(tele, sizeof(uint32_t) * B * 32);
    const int32_t K = uni(1, 3);
    int32_t *cls = (int32_t *)xmalloc(sizeof(int32_t) * B);
    for (int32_t r = 0; r < B; ++r) cls[r] = uni(-1, K);         /* some outside [0, K) */
    uint64_t *tot = (uint64_t *)xmalloc(sizeof(uint64_t) * K * 32);
    oracle_telemetry_reduce(tele, cls, B, K, tot);
    mix(tot, sizeof(uint64_t) * K * 32);

    free(len); free(cap); free(row_off); free(hist); free(m); free(e); free(d); free(q); free(lm);
    free(tgt); free(blk); free(bl); free(mm); free(acc); free(st); free(ln); free(tele); free(cls);
    free(tot);
}

static float special_prob(void) {
    switch (uni(0, 9)) {
    case 0: return NAN;
    case 1: return -0.25f;
    case 2: return INFINITY;
    case 3: return 1.5f;
    case 4: return 0.0f;
    default: return (float)(next_u64() >> 40) / (float)(1 << 24);
    }
}

static void rejection_round(void) {
    const int32_t B = uni(1, 6);
    const int32_t V = 4 * uni(1, 300);
    int32_t *blk = (int32_t *)xmalloc(sizeof(int32_t) * B * 15), *bl = (int32_t *)xmalloc(sizeof(int32_t) * B);
    uint32_t *mm = (uint32_t *)xmalloc(sizeof(uint32_t) * B);
    for (int32_t i = 0; i < B * 15; ++i) blk[i] = uni(-1, V);       /* PAD and out-of-vocabulary too */
    for (int32_t r = 0; r < B; ++r) { bl[r] = uni(-2, 17); mm[r] = (uint32_t)next_u64(); }
    float *tp = (float *)xmalloc(sizeof(float) * (size_t)B * 16 * V);
    float *mp = (float *)xmalloc(sizeof(float) * (size_t)B * 7 * V);
    const int zero_rows = uni(0, 3) == 0;
    for (int64_t i = 0; i < (int64_t)B * 16 * V; ++i) tp[i] = zero_rows ? 0.0f : special_prob();
    for (int64_t i = 0; i < (int64_t)B * 7 * V; ++i) mp[i] = special_prob();
    double *ua = (double *)xmalloc(sizeof(double) * B * 15);
    uint64_t *us = (uint64_t *)xmalloc(sizeof(uint64_t) * B);
    for (int32_t i = 0; i < B * 15; ++i) ua[i] = (double)(next_u64() >> 11) / 9007199254740992.0;
    for (int32_t r = 0; r < B; ++r) us[r] = next_u64();
    int32_t *acc = (int32_t *)xmalloc(sizeof(int32_t) * B), *em = (int32_t *)xmalloc(sizeof(int32_t) * B * 16);
    oracle_rejection_accept(blk, bl, uni(0, 1) ? mm : NULL, tp, uni(0, 1) ? mp : NULL, V, ua, us, B, acc,
                            em, NULL, NULL, NULL, NULL);
    mix(acc, sizeof(int32_t) * B); mix(em, sizeof(int32_t) * B * 16);
    /* with the append */
    int32_t *len = (int32_t *)xmalloc(sizeof(int32_t) * B), *cap = (int32_t *)xmalloc(sizeof(int32_t) * B);
    int64_t *ro = (int64_t *)xmalloc(sizeof(int64_t) * B);
    int64_t total = 0;
    for (int32_t r = 0; r < B; ++r) {
        len[r] = uni(-2, 10);
        cap[r] = (len[r] > 0 ? len[r] : 0) + uni(0, 17);
        ro[r] = total;
        total += cap[r];
    }
    int32_t *hist = (int32_t *)xmalloc(sizeof(int32_t) * (size_t)total);
    for (int64_t i = 0; i < total; ++i) hist[i] = 7;
    oracle_rejection_accept(blk, bl, mm, tp, mp, V, ua, us, B, acc, em, hist, ro, len, cap);
    mix(acc, sizeof(int32_t) * B); mix(em, sizeof(int32_t) * B * 16);
    mix(hist, sizeof(int32_t) * (size_t)total); mix(len, sizeof(int32_t) * B);
    /* the benchmark harness over the same batch, with and without model rows */
    int64_t steps, chk;
    double wall, cpu;
    const int with_model = uni(0, 1);
    if (oracle_bench_rejection(blk, bl, with_model ? mm : NULL, tp, with_model ? mp : NULL, V, ua,
                               us, B, uni(1, 3), 0.0, 2, &steps, &wall, &cpu, &chk) != 0) {
        fprintf(stderr, "oracle_bench_rejection failed\n");
        exit(3);
    }
    mix(&steps, sizeof steps); mix(&chk, sizeof chk);
    free(blk); free(bl); free(mm); free(tp); free(mp); free(ua); free(us); free(acc); free(em);
    free(len); free(cap); free(ro); free(hist);
}

static void bench_round(void) {
    const int32_t B = 5;
    int32_t len[5] = {0, 3, 100, 257, 31};
    int64_t ro[5];
    int64_t total = 0;
    for (int r = 0; r < B; ++r) { ro[r] = total; total += len[r]; }
    int32_t *hist = (int32_t *)xmalloc(sizeof(int32_t) * (size_t)total);
    for (int64_t i = 0; i < total; ++i) hist[i] = uni(0, 2);
    int32_t *q = (int32_t *)xmalloc(sizeof(int32_t) * B * 7), *t = (int32_t *)xmalloc(sizeof(int32_t) * B * 16);
    for (int i = 0; i < B * 7; ++i) q[i] = uni(0, 2);
    for (int i = 0; i < B * 16; ++i) t[i] = uni(0, 2);
    oracle_params p = {4, 12, 15, 7, 15, 8, 6, 2, 4, 2, 3, 1};
    int64_t steps, chk;
    double wall, cpu;
    if (oracle_bench_steps(hist, ro, len, B, q, t, &p, 3, 0.0, 2, &steps, &wall, &cpu, &chk) != 0) {
        fprintf(stderr, "oracle_bench_steps failed\n");
        exit(3);
    }
    mix(&steps, sizeof steps); mix(&chk, sizeof chk);
    free(hist); free(q); free(t);
}

int main(int argc, char **argv) {
    const int rounds = argc > 1 ? atoi(argv[1]) : 300;
    for (int i = 0; i < rounds; ++i) step_round();
    for (int i = 0; i < rounds / 10 + 1; ++i) rejection_round();
    bench_round();
    printf("%016llx\n", (unsigned long long)sum);
    return 0;
}

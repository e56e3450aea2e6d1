/*
 * lcd_oracle.c -- plain CPU oracle for context-lookup drafting.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, literal statement of what
 * the drafting hot path computes.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load it; the product path never does, and it
 * shares no source, header, table or helper with the HIP library.
 *
 * Source of the method: the HyperQwen lookup-drafting article (page titled
 * "HyperQwen 上下文复述加速：lookup 草稿如何把 25k 文档复读推到 381 tok/s"),
 * sections "第 1 步" (search the request's own history), "第 2 步" (fuse with the
 * draft model's proposal), "第 3 步" (schedule the long block only while a copy
 * is in progress) and the closing paragraph on losslessness (greedy verification
 * never reads the draft distribution).  Where the article leaves a step open the
 * reading taken is stated at the function.
 *
 * Conventions: token ids are int32; PAD = -1 marks an empty draft or block slot.
 * Every array is host memory owned by the caller.  Nothing here allocates.
 * Each function handles B requests with a plain loop; no blocking, no early
 * termination beyond what the definition itself implies.
 */
#include <stdint.h>
#include <stddef.h>

#define ORACLE_PAD (-1)
#define ORACLE_DRAFT_STRIDE 15   /* draft and block rows */
#define ORACLE_Q_STRIDE 7        /* draft-model proposal rows */
#define ORACLE_TARGET_STRIDE 16  /* target argmax rows */

/* Method parameters; the defaults are the article's numbers (4..12-token
 * suffixes, up to 15 drafted tokens, 7-slot draft-model head, head thresholds
 * 8 and 6-with-2-agreeing, tail threshold 4, two-step entry, sticky exit 3). */
typedef struct oracle_params {
    int32_t l_min, l_max, k_max;
    int32_t n_head, n_block;
    int32_t head_full, head_agree, agree_n, tail_min;
    int32_t entry_steps, sticky, near_full_slack;
} oracle_params;

/*
 * Lookup for one request (article, "第 1 步").
 *
 * The longest current suffix of l_max..l_min tokens is searched for, longest
 * length first; for a given length the most recent earlier occurrence wins
 * (positions scanned from latest to earliest).  "Earlier occurrence" is read as
 * an occurrence that ends at most at index n-2, so that at least one following
 * token exists; it may overlap the suffix itself (the article allows a match to
 * overlap the suffix so periodic text matches at its own period).
 *
 * Draft: the tokens that follow the occurrence, read LZ77-style from the history
 * extended by the draft itself, so when the occurrence overlaps the suffix the
 * copy runs past the end of the history and repeats with period n-1-e.  Up to
 * k_max tokens; the remaining slots of the 15-slot row are PAD.  No match:
 * m = 0, e = -1, all PAD.
 */
static void lookup_one(const int32_t *h, int64_t n, const oracle_params *p,
                       int32_t *m_out, int32_t *e_out, int32_t *draft)
{
    int32_t m = 0;
    int64_t e = -1;
    for (int32_t L = p->l_max; L >= p->l_min && m == 0; --L) {
        /* the occurrence h[q..q+L-1] must end at q+L-1 <= n-2 */
        for (int64_t q = n - L - 1; q >= 0; --q) {
            int same = 1;
            for (int32_t j = 0; j < L; ++j) {
                if (h[q + j] != h[n - L + j]) { same = 0; break; }
            }
            if (same) { m = L; e = q + L - 1; break; }
        }
    }
    for (int k = 0; k < ORACLE_DRAFT_STRIDE; ++k) draft[k] = ORACLE_PAD;
    if (m > 0) {
        /* append one token at a time: source index e+1+k in (history ++ draft) */
        for (int32_t k = 0; k < p->k_max; ++k) {
            int64_t src = e + 1 + k;
            draft[k] = (src < n) ? h[src] : draft[src - n];
        }
    }
    *m_out = m;
    *e_out = (int32_t)e;
}

int oracle_lookup_propose(const int32_t *hist, const int64_t *row_off, const int32_t *len,
                          int32_t B, const oracle_params *p,
                          int32_t *match_len, int32_t *match_end, int32_t *draft)
{
    for (int32_t r = 0; r < B; ++r) {
        int64_t n = len[r] > 0 ? len[r] : 0;
        lookup_one(hist + row_off[r], n, p, &match_len[r], &match_end[r],
                   draft + (int64_t)r * ORACLE_DRAFT_STRIDE);
    }
    return 0;
}

/*
 * Fusion into the verify block (article, "第 2 步").
 *
 * The verify block is the input token plus n_block draft slots when long and
 * n_head slots when short.  Head slots 0..n_head-1 already hold the draft
 * model's proposal; they are all replaced by the lookup draft when the match is
 * at least head_full tokens, or at least head_agree tokens and the draft model
 * independently proposed the same first agree_n tokens.  Tail slots
 * n_head..blk-1 were proposed by nobody; in a long block they take the lookup
 * draft whenever the match is at least tail_min tokens, independently of the
 * head decision, and PAD otherwise.  Slots beyond the verified length, and
 * draft slots at or past k_max, are never taken from the lookup.
  *
 * model_mask (may be NULL): bit i is set when slot i holds the draft model's own
 * token q[i] (a head slot the lookup did not replace), so that a sampled
 * verifier knows which slots carry the draft model's distribution; every other
 * non-PAD slot is a lookup token.
 */
int oracle_fuse_verify_block(const int32_t *draft, const int32_t *match_len,
                             const int32_t *q, const int32_t *long_mode, int32_t B,
                             const oracle_params *p, int32_t *block, int32_t *block_len,
                             uint32_t *model_mask)
{
    for (int32_t r = 0; r < B; ++r) {
        const int32_t *d = draft + (int64_t)r * ORACLE_DRAFT_STRIDE;
        const int32_t *qr = q + (int64_t)r * ORACLE_Q_STRIDE;
        int32_t *out = block + (int64_t)r * ORACLE_DRAFT_STRIDE;
        int32_t m = match_len[r];
        int is_long = long_mode[r] != 0;

        int agree = 1;
        for (int32_t i = 0; i < p->agree_n; ++i)
            if (qr[i] != d[i]) agree = 0;
        int head = (m >= p->head_full) || (m >= p->head_agree && agree);
        int tail = is_long && (m >= p->tail_min);
        int32_t blk = is_long ? p->n_block : p->n_head;

        uint32_t from_model = 0;   /* bit i: slot i holds the draft model's proposal */
        for (int32_t i = 0; i < ORACLE_DRAFT_STRIDE; ++i) {
            int32_t v;
            if (i >= blk) {
                v = ORACLE_PAD;
            } else if (i < p->n_head) {
                if (head && i < p->k_max) {
                    v = d[i];
                } else {
                    v = qr[i];
                    from_model |= 1u << i;
                }
            } else {
                v = (tail && i < p->k_max) ? d[i] : ORACLE_PAD;
            }
            out[i] = v;
        }
        block_len[r] = blk;
        if (model_mask != NULL)
            model_mask[r] = from_model;
    }
    return 0;
}

/*
 * Greedy acceptance (article, closing paragraph on losslessness; the Polish
 * speculative-decoding post, section on why token-by-token generation is
 * expensive: the first rejected proposal ends the run).
 *
 * a = length of the longest prefix of the block equal to the target's argmax
 * tokens, at most blk.  The step emits target[0..a] (a+1 tokens: the accepted
 * drafts plus the target's own token at the first mismatch, or its bonus token).
 * Optional append: when hist is non-NULL, target[0..a] is written at
 * row_off[r]+n with n = max(len[r], 0) and len[r] becomes n+a+1; if that would
 * exceed cap[r] the request is flagged with accept = -1 and nothing is written.
 */
int oracle_greedy_accept(const int32_t *block, const int32_t *block_len,
                         const int32_t *target, int32_t B, int32_t *accept,
                         int32_t *hist, const int64_t *row_off, int32_t *len,
                         const int32_t *cap)
{
    for (int32_t r = 0; r < B; ++r) {
        const int32_t *blkr = block + (int64_t)r * ORACLE_DRAFT_STRIDE;
        const int32_t *t = target + (int64_t)r * ORACLE_TARGET_STRIDE;
        int32_t blk = block_len[r];
        int32_t a = 0;
        while (a < blk && blkr[a] == t[a]) a++;
        if (hist != NULL) {
            int64_t have = len[r] > 0 ? len[r] : 0;   /* a negative length reads as an empty row */
            if (have + a + 1 > (int64_t)cap[r]) {
                accept[r] = -1;
                continue;
            }
            for (int32_t i = 0; i <= a; ++i)
                hist[row_off[r] + have + i] = t[i];
            len[r] = (int32_t)(have + a + 1);
        }
        accept[r] = a;
    }
    return 0;
}

/*
 * Sampled verification with point-mass lookup proposals (article, closing
 * paragraph on losslessness: for sampled requests each lookup-filled slot is
 * rewritten as a point mass on its token, a legal proposal distribution for the
 * speculative rejection sampler, so the output distribution is unchanged; the
 * Polish speculative-decoding post, on verification: the first rejected
 * proposal ends the run).
 *
 * Per request, the verified slots are i < L, L = block_len clamped to 0..15.
 * target_probs holds 16 rows of V probabilities, row i being the target's
 * distribution for the token after the block's first i slots; model_probs (may
 * be NULL) holds the draft model's 7 head rows.  Slot i's proposal
 * distribution is the draft model's row i when bit i of model_mask is set, i < 7
 * and model_probs is given; otherwise (lookup slots, or a draft model that gives
 * no distribution) it is the point mass on block[i].
 *
 * Walking i = 0, 1, ...: a slot whose token is PAD or outside [0, V) ends the
 * run with nothing proposed there.  Otherwise, with P = p_i(x) and Q = q_i(x)
 * (Q = 1 for a point mass), the slot is accepted iff u_i * Q < P, i.e. with
 * probability min(1, P/Q) for u_i uniform on [0,1).  The first rejection ends
 * the run; its token is drawn from the residual max(p_i - q_i, 0) renormalised
 * (for a point mass: p_i with x removed).  When the run ends without a
 * rejection (all L slots accepted, or a slot with nothing proposed), the token
 * is drawn from p_a itself (the bonus token).  So a = accepted slots, and the
 * step emits block[0..a-1] followed by the drawn token.
 *
 * Precision (the token is an integer decided by floating point, so the
 * arithmetic is fixed here and the kernel takes the same decisions):
 *  - probabilities are read as fp32 and clamped into [0, 1] (NaN reads as 0);
 *  - the acceptance test is evaluated in fp64 (u_i is fp64; u_i * Q is the only
 *    rounding step);
 *  - the residual difference p - q is an fp32 subtraction, negative -> 0;
 *  - drawing: each weight w_j becomes the integer W_j = floor(w_j * 2^40), the
 *    total S = sum W_j is exact in 64 bits (V < 2^23), t = floor(u_s * S / 2^64)
 *    for the request's 64-bit uniform word u_s, and the token is the smallest j
 *    whose running total W_0 + ... + W_j exceeds t.  A probability below 2^-40
 *    gets weight 0; the drawn distribution is W_j / S.
 * An all-zero residual falls back to p_a; if that is all zero too the request
 * emits nothing: accept = -1, the emitted row is all PAD and nothing is appended.
 *
 * emitted int32 [B*16]: the a+1 emitted tokens, then PAD.  With hist non-NULL
 * the emitted tokens are appended exactly as greedy_accept appends them.
 */
static float prob01(float x)
{
    if (!(x > 0.0f)) return 0.0f;   /* negative, zero or NaN */
    if (x > 1.0f) return 1.0f;
    return x;
}

static uint64_t fixed40(float w)   /* floor(w * 2^40) for w in [0, 1] */
{
    return (uint64_t)((double)w * 1099511627776.0);
}

int oracle_rejection_accept(const int32_t *block, const int32_t *block_len,
                            const uint32_t *model_mask, const float *target_probs,
                            const float *model_probs, int32_t V, const double *u_accept,
                            const uint64_t *u_sample, int32_t B, int32_t *accept,
                            int32_t *emitted, int32_t *hist, const int64_t *row_off,
                            int32_t *len, const int32_t *cap)
{
    for (int32_t r = 0; r < B; ++r) {
        const int32_t *blkr = block + (int64_t)r * ORACLE_DRAFT_STRIDE;
        int32_t *em = emitted + (int64_t)r * ORACLE_TARGET_STRIDE;
        int32_t L = block_len[r];
        if (L < 0) L = 0;
        if (L > ORACLE_DRAFT_STRIDE) L = ORACLE_DRAFT_STRIDE;

        /* 1. walk the slots */
        int32_t a = 0;
        int rejected = 0;
        int rej_model = 0;   /* the rejected slot's proposal was the draft model's row */
        int32_t rej_tok = 0;
        while (a < L) {
            int32_t x = blkr[a];
            if (x < 0 || x >= V)
                break;
            const float *pr = target_probs + ((int64_t)r * ORACLE_TARGET_STRIDE + a) * V;
            int use_model = model_probs != NULL && model_mask != NULL &&
                            a < ORACLE_Q_STRIDE && ((model_mask[r] >> a) & 1u);
            double P = prob01(pr[x]);
            double Q = 1.0;
            if (use_model)
                Q = prob01(model_probs[((int64_t)r * ORACLE_Q_STRIDE + a) * V + x]);
            if (u_accept[(int64_t)r * ORACLE_DRAFT_STRIDE + a] * Q < P) {
                a++;
                continue;
            }
            rejected = 1;
            rej_model = use_model;
            rej_tok = x;
            break;
        }

        /* 2. the distribution the last token is drawn from, as integer weights */
        const float *pr = target_probs + ((int64_t)r * ORACLE_TARGET_STRIDE + a) * V;
        const float *qr = rej_model
            ? model_probs + ((int64_t)r * ORACLE_Q_STRIDE + a) * V : NULL;
        uint64_t S = 0;
        if (rejected) {
            for (int32_t j = 0; j < V; ++j) {
                float w;
                if (qr != NULL) {
                    w = prob01(pr[j]) - prob01(qr[j]);
                    if (!(w > 0.0f)) w = 0.0f;
                } else {
                    w = (j == rej_tok) ? 0.0f : prob01(pr[j]);
                }
                S += fixed40(w);
            }
        }
        int plain = !rejected || S == 0;
        if (plain) {
            S = 0;
            for (int32_t j = 0; j < V; ++j)
                S += fixed40(prob01(pr[j]));
        }
        for (int32_t i = 0; i < ORACLE_TARGET_STRIDE; ++i)
            em[i] = ORACLE_PAD;
        if (S == 0) {
            accept[r] = -1;
            continue;
        }

        /* 3. inverse-CDF draw on the integer weights */
        uint64_t t = (uint64_t)(((unsigned __int128)u_sample[r] * S) >> 64);
        uint64_t run = 0;
        int32_t z = -1;
        for (int32_t j = 0; j < V; ++j) {
            float w;
            if (plain) {
                w = prob01(pr[j]);
            } else if (qr != NULL) {
                w = prob01(pr[j]) - prob01(qr[j]);
                if (!(w > 0.0f)) w = 0.0f;
            } else {
                w = (j == rej_tok) ? 0.0f : prob01(pr[j]);
            }
            run += fixed40(w);
            if (run > t) {
                z = j;
                break;
            }
        }

        /* 4. emit, and append as the greedy verifier does */
        for (int32_t i = 0; i < a; ++i)
            em[i] = blkr[i];
        em[a] = z;
        if (hist != NULL) {
            int64_t have = len[r] > 0 ? len[r] : 0;
            if (have + a + 1 > (int64_t)cap[r]) {
                accept[r] = -1;
                continue;
            }
            for (int32_t i = 0; i <= a; ++i)
                hist[row_off[r] + have + i] = em[i];
            len[r] = (int32_t)(have + a + 1);
        }
        accept[r] = a;
    }
    return 0;
}

/*
 * Long-block scheduler (article, "第 3 步").
 *
 * Per request the state is {long_mode, streak, down}.  This step's flag is
 * "the lookup match could fill the tail" (m >= tail_min) and "the step came out
 * nearly full" (a >= blk - near_full_slack, reading "nearly full" as at most
 * near_full_slack short of the verified length; a failed append, a = -1, never
 * counts).  In short mode the flag must hold on entry_steps consecutive steps to
 * switch to the long block; in long mode the block is kept while the flag has
 * been down for at most `sticky` consecutive steps and dropped on the next one,
 * after which entry has to be earned again from zero.  The returned mode is the
 * one the next step uses.
 */
int oracle_lookup_schedule_step(int32_t *state /* B x 3 */, const int32_t *match_len,
                                const int32_t *accept, const int32_t *block_len, int32_t B,
                                const oracle_params *p, int32_t *long_next)
{
    for (int32_t r = 0; r < B; ++r) {
        int32_t *st = state + (int64_t)r * 3;
        int32_t is_long = st[0], streak = st[1], down = st[2];
        int32_t a = accept[r];
        int flag = (match_len[r] >= p->tail_min) && (a >= 0) &&
                   (a >= block_len[r] - p->near_full_slack);
        if (!is_long) {
            streak = flag ? streak + 1 : 0;
            if (streak >= p->entry_steps) { is_long = 1; streak = 0; down = 0; }
        } else {
            if (flag) {
                down = 0;
            } else {
                down = down + 1;
                if (down > p->sticky) { is_long = 0; down = 0; streak = 0; }
            }
        }
        st[0] = is_long; st[1] = streak; st[2] = down;
        long_next[r] = is_long;
    }
    return 0;
}


/*
 * Acceptance telemetry (the forum thread on the article: wire up hit rate and
 * mean accepted length before drawing conclusions, and print the accepted-
 * length distribution; the Polish post, "Jak testować bez mylenia prędkości z
 * jakością", item 5: measure acceptance per task class).
 *
 * Per request r, tele[r*32 + k] are unsigned 32-bit counters that one decode
 * step updates once:
 *   0 steps            1 hits (m > 0)
 *   2 steps whose head slots took the lookup draft (the fusion head decision)
 *   3 steps whose tail slots took the lookup draft (the fusion tail decision)
 *   4 steps verified as a long block (the mode the step used)
 *   5 entries into the long block (this step short, the next one long)
 *   6 exits from it (this step long, the next one short)
 *   7 tokens emitted (a+1 summed over steps with a >= 0)
 *   8 failed appends (a = -1)
 *   9 + i, i = 0..15: steps that accepted exactly i draft slots
 *   25..31 unused (zero)
 * The head and tail decisions are recomputed from the step's match length,
 * draft, draft-model proposal and mode with the fusion rule above.
 */
int oracle_telemetry_update(uint32_t *tele, const int32_t *match_len, const int32_t *draft,
                            const int32_t *q, const int32_t *long_mode,
                            const int32_t *block_len, const int32_t *accept,
                            const int32_t *long_next, int32_t B, const oracle_params *p)
{
    for (int32_t r = 0; r < B; ++r) {
        uint32_t *t = tele + (int64_t)r * 32;
        const int32_t *d = draft + (int64_t)r * ORACLE_DRAFT_STRIDE;
        const int32_t *qr = q + (int64_t)r * ORACLE_Q_STRIDE;
        int32_t m = match_len[r];
        int is_long = long_mode[r] != 0;
        int agree = 1;
        for (int32_t i = 0; i < p->agree_n; ++i)
            if (qr[i] != d[i]) agree = 0;
        int head = (m >= p->head_full) || (m >= p->head_agree && agree);
        int tail = is_long && (m >= p->tail_min);
        int32_t a = accept[r];
        (void)block_len;
        t[0] += 1;
        if (m > 0) t[1] += 1;
        if (head) t[2] += 1;
        if (tail) t[3] += 1;
        if (is_long) t[4] += 1;
        if (!is_long && long_next[r]) t[5] += 1;
        if (is_long && !long_next[r]) t[6] += 1;
        if (a >= 0) {
            t[7] += (uint32_t)(a + 1);
            if (a < 16) t[9 + a] += 1;
        } else {
            t[8] += 1;
        }
    }
    return 0;
}

/*
 * Per-class totals of the telemetry counters: out[k*32 + c] = the sum over
 * requests r with class_id[r] == k of tele[r*32 + c], for 0 <= k < K (64-bit
 * sums; requests whose class is outside [0, K) are left out).
 */
int oracle_telemetry_reduce(const uint32_t *tele, const int32_t *class_id, int32_t B,
                            int32_t K, uint64_t *out)
{
    for (int64_t i = 0; i < (int64_t)K * 32; ++i) out[i] = 0;
    for (int32_t r = 0; r < B; ++r) {
        int32_t k = class_id[r];
        if (k < 0 || k >= K) continue;
        for (int c = 0; c < 32; ++c) out[(int64_t)k * 32 + c] += tele[(int64_t)r * 32 + c];
    }
    return 0;
}

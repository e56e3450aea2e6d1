// lcd_rules.h -- per-request rules of a lookup-drafting step, as device
// functions shared by the separate step kernels and the fused decode step.
//
// Method: HyperQwen lookup-drafting article, sections "第 2 步" (fuse the lookup
// draft with the draft model's proposal: head slots need a long match, or a
// shorter one confirmed by the draft model's first tokens; tail slots take any
// match of the tail threshold), "第 3 步" (long block entered after consecutive
// nearly-full steps with a tail-filling match, kept for a few steps after the
// flag drops) and the closing paragraph (greedy verification: the longest
// block prefix equal to the target's argmax tokens is accepted).
#ifndef LCD_RULES_H
#define LCD_RULES_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lcd.h"

namespace lcd {

struct FuseArgs {
    int32_t k_max, n_head, n_block, head_full, head_agree, agree_n, tail_min;
};

struct SchedArgs {
    int32_t tail_min, entry_steps, sticky, near_full_slack;
};

// Fusion decisions of one request: head slots take the lookup draft when the
// match is long enough, or shorter but confirmed by the draft model's first
// agree_n tokens; tail slots take it in a long block with a tail-length match.
// Returns the number of draft slots verified.
__device__ inline int fuse_mode(int m, bool agree, bool is_long, const FuseArgs &a, bool &head,
                                bool &tail) {
    head = (m >= a.head_full) || (m >= a.head_agree && agree);
    tail = is_long && (m >= a.tail_min);
    return is_long ? a.n_block : a.n_head;
}

// Verify-block slot i given the draft token d and the draft model's token q
// for that slot (slots below n_head <= 7 carry the draft model's proposal).
__device__ inline int fuse_slot(int i, int d, int q, bool head, bool tail, int blk, const FuseArgs &a) {
    if (i < a.n_head) return (head && i < a.k_max) ? d : q;
    if (i < blk) return (tail && i < a.k_max) ? d : LCD_PAD;
    return LCD_PAD;
}

// True when verify slot i keeps the draft model's own token (a head slot the
// lookup draft does not replace); every other non-PAD slot is a lookup token.
__device__ inline bool fuse_slot_from_model(int i, bool head, const FuseArgs &a) {
    return i < a.n_head && !(head && i < a.k_max);
}

// Verify block of one request.  Returns the number of draft slots verified;
// from_model gets bit i set for each slot that keeps the draft model's token.
__device__ inline int fuse_row(const int (&d)[LCD_DRAFT_STRIDE], int m, const int (&q)[LCD_Q_STRIDE],
                               bool is_long, const FuseArgs &a, int (&out)[LCD_DRAFT_STRIDE],
                               uint32_t &from_model) {
    bool agree = true;
#pragma unroll
    for (int i = 0; i < LCD_Q_STRIDE; ++i)
        if (i < a.agree_n && q[i] != d[i]) agree = false;
    bool head, tail;
    const int blk = fuse_mode(m, agree, is_long, a, head, tail);
    from_model = 0;
#pragma unroll
    for (int i = 0; i < LCD_DRAFT_STRIDE; ++i) {
        out[i] = fuse_slot(i, d[i], i < LCD_Q_STRIDE ? q[i] : LCD_PAD, head, tail, blk, a);
        if (fuse_slot_from_model(i, head, a)) from_model |= 1u << i;
    }
    return blk;
}

// Greedy acceptance: the longest prefix of the block (at most blk slots)
// equal to the target's argmax tokens.
__device__ inline int accept_row(const int (&b)[LCD_DRAFT_STRIDE], int blk,
                                 const int (&t)[LCD_TARGET_STRIDE]) {
    int acc = 0;
    bool run = true;
#pragma unroll
    for (int i = 0; i < LCD_DRAFT_STRIDE; ++i) {
        run = run && (i < blk) && (b[i] == t[i]);
        acc += run ? 1 : 0;
    }
    return acc;
}

// Append the a+1 emitted tokens t[0..a] to row r, which holds have >= 0
// tokens, when they fit in its capacity; returns a, or -1 (nothing written)
// when they do not.
__device__ inline int append_row(int a, const int (&t)[LCD_TARGET_STRIDE], int32_t *__restrict__ hist,
                                 int64_t ro, int64_t have, int32_t *__restrict__ len_r, int32_t cap_r) {
    if (have + a + 1 > (int64_t)cap_r) return -1;
    int32_t *dst = hist + ro + have;
#pragma unroll
    for (int i = 0; i < LCD_TARGET_STRIDE; ++i)
        if (i <= a) dst[i] = t[i];
    *len_r = (int32_t)(have + a + 1);
    return a;
}

// Scheduler update after a step with match length m, accept a (-1 = failed
// append) and blk verified slots; returns the next step's mode.
__device__ inline int schedule_row(lcd_sched_state &st, int m, int a, int blk, const SchedArgs &s) {
    const bool flag = (m >= s.tail_min) && (a >= 0) && (a >= blk - s.near_full_slack);
    if (!st.long_mode) {
        st.streak = flag ? st.streak + 1 : 0;
        if (st.streak >= s.entry_steps) {
            st.long_mode = 1;
            st.streak = 0;
            st.down = 0;
        }
    } else if (flag) {
        st.down = 0;
    } else {
        st.down += 1;
        if (st.down > s.sticky) {
            st.long_mode = 0;
            st.down = 0;
            st.streak = 0;
        }
    }
    return st.long_mode;
}

// Telemetry increment of counter k for one step (the layout of LCD_TELE_*):
// match length m, the fusion decisions, the mode used and the next one, and
// the accepted count a (-1: failed append).
__device__ inline uint32_t telemetry_inc(int k, int m, bool head, bool tail, bool is_long,
                                         bool long_next, int a) {
    switch (k) {
    case LCD_TELE_STEPS: return 1u;
    case LCD_TELE_HITS: return m > 0 ? 1u : 0u;
    case LCD_TELE_HEAD: return head ? 1u : 0u;
    case LCD_TELE_TAIL: return tail ? 1u : 0u;
    case LCD_TELE_LONG: return is_long ? 1u : 0u;
    case LCD_TELE_ENTRIES: return (!is_long && long_next) ? 1u : 0u;
    case LCD_TELE_EXITS: return (is_long && !long_next) ? 1u : 0u;
    case LCD_TELE_EMITTED: return a >= 0 ? (uint32_t)(a + 1) : 0u;
    case LCD_TELE_FAILED: return a < 0 ? 1u : 0u;
    default: return (k >= LCD_TELE_HIST && k < LCD_TELE_HIST + 16 && a == k - LCD_TELE_HIST) ? 1u : 0u;
    }
}

inline FuseArgs fuse_args(const lcd_params *p) {
    return FuseArgs{p->k_max, p->n_head, p->n_block, p->head_full, p->head_agree, p->agree_n,
                    p->tail_min};
}

inline SchedArgs sched_args(const lcd_params *p) {
    return SchedArgs{p->tail_min, p->entry_steps, p->sticky, p->near_full_slack};
}

}  // namespace lcd

#endif  // LCD_RULES_H

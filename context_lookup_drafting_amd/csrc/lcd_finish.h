// lcd_finish.h -- the rest of one request's decode step once its lookup is
// known, done by one wave with one lane per verify slot: fusion of the verify
// block, greedy acceptance with the optional append of the emitted tokens, the
// long-block scheduler and the optional telemetry counters.  Shared by the
// scan's one-kernel decode step and the index's.
//
// Method: HyperQwen lookup-drafting article, sections "第 2 步" (verify-block
// fusion), "第 3 步" (long-block entry and sticky exit) and the closing
// paragraph (greedy verification: the longest block prefix equal to the
// target's argmax tokens is accepted, and the target's token after it is
// emitted too); the per-slot rules themselves are in lcd_rules.h.
#ifndef LCD_FINISH_H
#define LCD_FINISH_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lcd.h"
#include "lcd_rules.h"

namespace lcd {

// A store of an output word to global memory.  The scan's 16-wave kernel
// rebuilds its output pointers from kernel-argument words held in lanes, where
// the compiler cannot see that they point to global memory; a flat store would
// also count against the counter that shuffles and scalar loads wait on, so
// each later such wait would wait for the store.  kThrough: written through to
// memory (a relaxed store at device scope), so that the scan's few scattered
// output words per request are on their way while its finishing wave works,
// instead of left dirty for the kernel's end to write back (64 x 25k: 6.76 ->
// 6.48 us; non-temporal stores instead: 8.52).  The index step, whose launch
// also writes its token cache and tables, measured slower that way (+0.2 us).
template <bool kThrough, typename T>
__device__ __forceinline__ void gstore(T *p, T v) {
    if constexpr (kThrough)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *(__attribute__((address_space(1))) T *)p = v;
}

// Inputs and outputs of the rest of the decode step.  hist_w aliases the
// history: the append lies past every position a lookup of the row reads.
// len_out receives the lengths after the step; the scan's decode step takes it
// apart from the lengths its launch reads (a workgroup may read a row's length
// after another has finished that row), the index step, whose one workgroup
// per request reads and writes only its own row, may pass the same array.
struct StepIO {
    int32_t *hist_w;
    int32_t *len_out;
    const int32_t *cap;
    const int32_t *q;
    const int32_t *target;
    lcd_sched_state *state;
    int32_t *block, *block_len, *accept, *long_next;
    uint32_t *tele;                  // telemetry rows (nullable)
    FuseArgs f;
    SchedArgs s;
    int32_t append;
};

// Per-request inputs of the rest of the step, one value per lane of the
// finishing wave: lanes 0..6 the draft model's proposal, 7..22 the target
// tokens, 23..25 the scheduler state, 26 the row capacity.  Loaded early, so
// they are in flight during the lookup.
__device__ __forceinline__ int load_step_input(int r, int lane, const StepIO &io) {
    const int32_t *src = io.q + (int64_t)r * LCD_Q_STRIDE;     // lanes past 26 re-read q[0]
    if (lane < LCD_Q_STRIDE)
        src = io.q + (int64_t)r * LCD_Q_STRIDE + lane;
    else if (lane < LCD_Q_STRIDE + LCD_TARGET_STRIDE)
        src = io.target + (int64_t)r * LCD_TARGET_STRIDE + (lane - LCD_Q_STRIDE);
    else if (lane < LCD_Q_STRIDE + LCD_TARGET_STRIDE + 3)
        src = reinterpret_cast<const int32_t *>(io.state) + (int64_t)r * 3 +
              (lane - LCD_Q_STRIDE - LCD_TARGET_STRIDE);
    else if (lane == LCD_Q_STRIDE + LCD_TARGET_STRIDE + 3 && io.append)
        src = io.cap + r;
    return *src;
}

// The step after request r's lookup (match length m, -1 when the lookup gave
// no answer; row of lr tokens as stored, n = max(lr, 0), at ro), run by one
// whole wave: lane k < 15 holds dk, the draft token of verify slot k (PAD past
// k_max or without a match); sin holds the step inputs as load_step_input left
// them and tin the request's telemetry counter of the lane (unused without
// telemetry).  Returns the accepted count (-1 for a failed append).  kThrough:
// the outputs are written through (see gstore).
template <bool kThrough = false>
__device__ __forceinline__ int finish_step(int r, int m, int dk, int sin, uint32_t tin, int lane,
                                           int64_t ro, int32_t lr, int n, const StepIO &io) {
    constexpr int kSt = LCD_Q_STRIDE + LCD_TARGET_STRIDE;      // sin lane of the state
    const int qk = sin;                                       // lanes 0..6: proposal
    const int tk = __shfl(sin, LCD_Q_STRIDE + (lane < LCD_TARGET_STRIDE ? lane : 0));
    lcd_sched_state st;
    st.long_mode = __builtin_amdgcn_readlane(sin, kSt);
    st.streak = __builtin_amdgcn_readlane(sin, kSt + 1);
    st.down = __builtin_amdgcn_readlane(sin, kSt + 2);
    const int32_t capr = __builtin_amdgcn_readlane(sin, kSt + 3);
    const bool agree = __ballot(lane < io.f.agree_n && qk != dk) == 0;
    bool head, tail;
    const int blk = fuse_mode(m, agree, st.long_mode != 0, io.f, head, tail);
    const int bk = fuse_slot(lane, dk, lane < LCD_Q_STRIDE ? qk : LCD_PAD, head, tail, blk, io.f);
    if (lane < LCD_DRAFT_STRIDE) gstore<kThrough>(io.block + (int64_t)r * LCD_DRAFT_STRIDE + lane, bk);
    // greedy accept: the slots before the first mismatch within blk
    const unsigned long long miss = __ballot(lane < blk && bk != tk);
    int acc = miss ? (int)__builtin_ctzll(miss) : blk;
    if (io.append) {
        // a failed append writes nothing and leaves the length as it was
        if ((int64_t)n + acc + 1 > (int64_t)capr) acc = -1;
        else if (lane <= acc) gstore<kThrough>(io.hist_w + ro + n + lane, tk);
        if (lane == 0) gstore<kThrough>(io.len_out + r, acc >= 0 ? n + acc + 1 : lr);
    }
    const bool was_long = st.long_mode != 0;
    const int ln = schedule_row(st, m, acc, blk, io.s);
    if (lane == 0) {
        gstore<kThrough>(io.block_len + r, blk);
        gstore<kThrough>(io.accept + r, acc);
        int32_t *sw = reinterpret_cast<int32_t *>(io.state + r);
        gstore<kThrough>(sw, st.long_mode);
        gstore<kThrough>(sw + 1, st.streak);
        gstore<kThrough>(sw + 2, st.down);
        if (io.long_next) gstore<kThrough>(io.long_next + r, ln);
    }
    // telemetry: lane k owns counter k of the request's row
    if (io.tele != nullptr && lane < LCD_TELE_HIST + 16)
        gstore<kThrough>(io.tele + (int64_t)r * LCD_TELE_WORDS + lane,
               tin + telemetry_inc(lane, m, head, tail, was_long, ln != 0, acc));
    return acc;
}

}  // namespace lcd

#endif  // LCD_FINISH_H

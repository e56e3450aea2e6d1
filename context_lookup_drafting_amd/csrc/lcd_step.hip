// lcd_step.hip -- fusion, greedy acceptance and long-block scheduling for
// MI355X / gfx950.  One lane per request: each of these moves about 200 bytes
// per request, so they are bound by launch latency, not by the memory system.
//
// Method: HyperQwen lookup-drafting article, sections "第 2 步" (fuse the
// lookup draft with the draft model's proposal: head slots need a long match,
// or a shorter one confirmed by the draft model's first two tokens; tail slots
// take any match of the tail threshold), "第 3 步" (long block entered after
// two consecutive nearly-full steps with a tail-filling match, kept for a few
// steps after the flag drops) and the closing paragraph (greedy verification
// keeps the output identical: accept the longest draft prefix equal to the
// target's argmax tokens).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lcd.h"
#include "lcd_rules.h"

namespace lcd {
namespace {

constexpr int kStepThreads = 256;

__global__ void __launch_bounds__(kStepThreads)
fuse_kernel(const int32_t *__restrict__ draft, const int32_t *__restrict__ match_len,
            const int32_t *__restrict__ q, const int32_t *__restrict__ long_mode, int32_t B,
            FuseArgs a, int32_t *__restrict__ block, int32_t *__restrict__ block_len,
            uint32_t *__restrict__ model_mask) {
    const int r = blockIdx.x * kStepThreads + threadIdx.x;
    if (r >= B) return;
    int dv[LCD_DRAFT_STRIDE], qv[LCD_Q_STRIDE], out[LCD_DRAFT_STRIDE];
#pragma unroll
    for (int i = 0; i < LCD_DRAFT_STRIDE; ++i) dv[i] = draft[(int64_t)r * LCD_DRAFT_STRIDE + i];
#pragma unroll
    for (int i = 0; i < LCD_Q_STRIDE; ++i) qv[i] = q[(int64_t)r * LCD_Q_STRIDE + i];
    uint32_t from_model;
    const int blk = fuse_row(dv, match_len[r], qv, long_mode[r] != 0, a, out, from_model);
#pragma unroll
    for (int i = 0; i < LCD_DRAFT_STRIDE; ++i) block[(int64_t)r * LCD_DRAFT_STRIDE + i] = out[i];
    block_len[r] = blk;
    if (model_mask != nullptr) model_mask[r] = from_model;
}

__global__ void __launch_bounds__(kStepThreads)
accept_kernel(const int32_t *__restrict__ block, const int32_t *__restrict__ block_len,
              const int32_t *__restrict__ target, int32_t B, int32_t *__restrict__ accept,
              int32_t *__restrict__ hist, const int64_t *__restrict__ row_off,
              int32_t *__restrict__ len, const int32_t *__restrict__ cap) {
    const int r = blockIdx.x * kStepThreads + threadIdx.x;
    if (r >= B) return;
    int bv[LCD_DRAFT_STRIDE], tv[LCD_TARGET_STRIDE];
#pragma unroll
    for (int i = 0; i < LCD_DRAFT_STRIDE; ++i) bv[i] = block[(int64_t)r * LCD_DRAFT_STRIDE + i];
#pragma unroll
    for (int i = 0; i < LCD_TARGET_STRIDE; ++i) tv[i] = target[(int64_t)r * LCD_TARGET_STRIDE + i];
    int acc = accept_row(bv, block_len[r], tv);
    if (hist != nullptr) {
        const int32_t have = len[r];
        acc = append_row(acc, tv, hist, row_off[r], have > 0 ? have : 0, len + r, cap[r]);
    }
    accept[r] = acc;
}

__global__ void __launch_bounds__(kStepThreads)
schedule_kernel(lcd_sched_state *__restrict__ state, const int32_t *__restrict__ match_len,
                const int32_t *__restrict__ accept, const int32_t *__restrict__ block_len,
                int32_t B, SchedArgs a, int32_t *__restrict__ long_next) {
    const int r = blockIdx.x * kStepThreads + threadIdx.x;
    if (r >= B) return;
    lcd_sched_state st = state[r];
    const int ln = schedule_row(st, match_len[r], accept[r], block_len[r], a);
    state[r] = st;
    long_next[r] = ln;
}

// Telemetry of one step from the separate calls' outputs, one lane per request.
__global__ void __launch_bounds__(kStepThreads)
telemetry_kernel(uint32_t *__restrict__ tele, const int32_t *__restrict__ match_len,
                 const int32_t *__restrict__ draft, const int32_t *__restrict__ q,
                 const int32_t *__restrict__ long_mode, const int32_t *__restrict__ accept,
                 const int32_t *__restrict__ long_next, int32_t B, FuseArgs a) {
    const int r = blockIdx.x * kStepThreads + threadIdx.x;
    if (r >= B) return;
    int dv[LCD_DRAFT_STRIDE], qv[LCD_Q_STRIDE];
#pragma unroll
    for (int i = 0; i < LCD_DRAFT_STRIDE; ++i) dv[i] = draft[(int64_t)r * LCD_DRAFT_STRIDE + i];
#pragma unroll
    for (int i = 0; i < LCD_Q_STRIDE; ++i) qv[i] = q[(int64_t)r * LCD_Q_STRIDE + i];
    const int m = match_len[r];
    const bool is_long = long_mode[r] != 0;
    bool agree = true;
#pragma unroll
    for (int i = 0; i < LCD_Q_STRIDE; ++i)
        if (i < a.agree_n && qv[i] != dv[i]) agree = false;
    bool head, tail;
    fuse_mode(m, agree, is_long, a, head, tail);
    const bool ln = long_next[r] != 0;
    const int acc = accept[r];
    uint32_t *t = tele + (int64_t)r * LCD_TELE_WORDS;
#pragma unroll
    for (int k = 0; k < LCD_TELE_HIST + 16; ++k) t[k] += telemetry_inc(k, m, head, tail, is_long, ln, acc);
}

// Per-class totals: one lane per (class, counter), summing over requests.
__global__ void __launch_bounds__(kStepThreads)
telemetry_reduce_kernel(const uint32_t *__restrict__ tele, const int32_t *__restrict__ class_id,
                        int32_t B, int32_t K, unsigned long long *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * kStepThreads + threadIdx.x;
    if (i >= (int64_t)K * LCD_TELE_WORDS) return;
    const int k = (int)(i / LCD_TELE_WORDS), c = (int)(i % LCD_TELE_WORDS);
    unsigned long long sum = 0;
    for (int32_t r = 0; r < B; ++r)
        if (class_id[r] == k) sum += tele[(int64_t)r * LCD_TELE_WORDS + c];
    out[i] = sum;
}

inline int blocks_for(int32_t B) { return (B + kStepThreads - 1) / kStepThreads; }

}  // namespace
}  // namespace lcd

extern "C" void lcd_default_params(lcd_params *p) {
    if (!p) return;
    p->l_min = 4;
    p->l_max = 12;
    p->k_max = 15;
    p->n_head = 7;
    p->n_block = 15;
    p->head_full = 8;
    p->head_agree = 6;
    p->agree_n = 2;
    p->tail_min = 4;
    p->entry_steps = 2;
    p->sticky = 3;
    p->near_full_slack = 1;
    p->scan_wgs = 0;
    p->scan_balance = 0;
    p->merge_polls = 0;
    p->index_load = 3;
}

extern "C" int lcd_check_params(const lcd_params *p) {
    if (!p) return LCD_EINVAL;
    const bool ok = p->l_min >= 1 && p->l_min <= p->l_max && p->l_max <= LCD_MAX_SUFFIX &&
                    p->k_max >= 0 && p->k_max <= LCD_DRAFT_STRIDE &&
                    p->n_head >= 1 && p->n_head <= LCD_Q_STRIDE &&
                    p->n_block >= p->n_head && p->n_block <= LCD_DRAFT_STRIDE &&
                    p->head_full >= 1 && p->head_agree >= 1 &&
                    p->agree_n >= 0 && p->agree_n <= p->n_head && p->tail_min >= 1 &&
                    p->entry_steps >= 1 && p->sticky >= 0 && p->near_full_slack >= 0 &&
                    p->scan_wgs >= 0 && p->scan_wgs <= (1 << 20) &&
                    (p->scan_balance == 0 || p->scan_balance == 1) && p->merge_polls >= -1 &&
                    p->index_load >= 2 && p->index_load <= 16;
    return ok ? LCD_OK : LCD_EINVAL;
}

extern "C" int fuse_verify_block(const int32_t *draft, const int32_t *match_len,
                                 const int32_t *model_draft, const int32_t *long_mode, int32_t B,
                                 const lcd_params *p, int32_t *block, int32_t *block_len,
                                 uint32_t *model_mask, void *stream) {
    using namespace lcd;
    if (B < 0 || lcd_check_params(p) != LCD_OK) return LCD_EINVAL;
    if (B == 0) return LCD_OK;
    if (!draft || !match_len || !model_draft || !long_mode || !block || !block_len)
        return LCD_EINVAL;
    const FuseArgs a = fuse_args(p);
    hipLaunchKernelGGL(fuse_kernel, dim3(blocks_for(B)), dim3(kStepThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), draft, match_len, model_draft,
                       long_mode, B, a, block, block_len, model_mask);
    return hipGetLastError() == hipSuccess ? LCD_OK : LCD_EHIP;
}

extern "C" int greedy_accept(const int32_t *block, const int32_t *block_len,
                             const int32_t *target, int32_t B, int32_t *accept, int32_t *hist,
                             const int64_t *row_off, int32_t *len, const int32_t *cap,
                             void *stream) {
    using namespace lcd;
    if (B < 0) return LCD_EINVAL;
    if (B == 0) return LCD_OK;
    if (!block || !block_len || !target || !accept) return LCD_EINVAL;
    if (hist && (!row_off || !len || !cap)) return LCD_EINVAL;
    hipLaunchKernelGGL(accept_kernel, dim3(blocks_for(B)), dim3(kStepThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), block, block_len, target, B, accept,
                       hist, row_off, len, cap);
    return hipGetLastError() == hipSuccess ? LCD_OK : LCD_EHIP;
}

extern "C" int lookup_schedule_step(lcd_sched_state *state, const int32_t *match_len,
                                    const int32_t *accept, const int32_t *block_len, int32_t B,
                                    const lcd_params *p, int32_t *long_next, void *stream) {
    using namespace lcd;
    if (B < 0 || lcd_check_params(p) != LCD_OK) return LCD_EINVAL;
    if (B == 0) return LCD_OK;
    if (!state || !match_len || !accept || !block_len || !long_next) return LCD_EINVAL;
    const SchedArgs a = sched_args(p);
    hipLaunchKernelGGL(schedule_kernel, dim3(blocks_for(B)), dim3(kStepThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), state, match_len, accept, block_len,
                       B, a, long_next);
    return hipGetLastError() == hipSuccess ? LCD_OK : LCD_EHIP;
}

extern "C" int lookup_telemetry_update(uint32_t *telemetry, const int32_t *match_len,
                                       const int32_t *draft, const int32_t *model_draft,
                                       const int32_t *long_mode, const int32_t *block_len,
                                       const int32_t *accept, const int32_t *long_next, int32_t B,
                                       const lcd_params *p, void *stream) {
    using namespace lcd;
    (void)block_len;
    if (B < 0 || lcd_check_params(p) != LCD_OK) return LCD_EINVAL;
    if (B == 0) return LCD_OK;
    if (!telemetry || !match_len || !draft || !model_draft || !long_mode || !accept || !long_next)
        return LCD_EINVAL;
    hipLaunchKernelGGL(telemetry_kernel, dim3(blocks_for(B)), dim3(kStepThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), telemetry, match_len, draft,
                       model_draft, long_mode, accept, long_next, B, fuse_args(p));
    return hipGetLastError() == hipSuccess ? LCD_OK : LCD_EHIP;
}

extern "C" int lookup_telemetry_reduce(const uint32_t *telemetry, const int32_t *class_id, int32_t B,
                                       int32_t K, uint64_t *out, void *stream) {
    using namespace lcd;
    if (B < 0 || K < 0) return LCD_EINVAL;
    if (K == 0) return LCD_OK;
    if (!out || (B > 0 && (!telemetry || !class_id))) return LCD_EINVAL;
    const int64_t n = (int64_t)K * LCD_TELE_WORDS;
    if (n > (int64_t)1 << 30) return LCD_EINVAL;
    hipLaunchKernelGGL(telemetry_reduce_kernel, dim3((unsigned)((n + kStepThreads - 1) / kStepThreads)),
                       dim3(kStepThreads), 0, reinterpret_cast<hipStream_t>(stream), telemetry,
                       class_id, B, K, reinterpret_cast<unsigned long long *>(out));
    return hipGetLastError() == hipSuccess ? LCD_OK : LCD_EHIP;
}

// lcd_sample.hip -- sampled verification with point-mass lookup proposals for
// MI355X / gfx950.
//
// Method: HyperQwen lookup-drafting article, closing paragraph on losslessness
// (for sampled requests every lookup-filled slot is verified as a point mass on
// its token, a legal proposal distribution for speculative rejection sampling,
// so the output distribution is the target's).  The Polish speculative-decoding
// post gives the verification rule: the first rejected proposal ends the run.
//
// Per request the work is one short walk over the verify block (at most 15
// gathered probabilities) and one pass over a single vocabulary row: the
// residual at the rejected slot, or the target row itself when the run ended
// without a rejection.  That pass is what costs: V fp32 values per request
// (two rows when the rejected slot carries the draft model's distribution),
// read once from HBM -- a bandwidth-bound stream, not a contraction, so no
// MFMA.
//
// Layout of the work.  A row is cut into units of 1024 floats (one 16-byte
// load per lane, four times, for one wave).  Workgroup (r, c) of the B x G
// grid streams units [c*upw, (c+1)*upw) of request r's row, one unit per wave
// at a time, turns every probability into the integer weight floor(w * 2^40)
// and publishes each unit's exact 64-bit weight sum into the request's
// workspace.  The last workgroup of the request to start (arrival tickets, as
// in the lookup merge) gathers the unit sums, takes t = floor(u * S / 2^64) for
// the request's 64-bit uniform word u and total S, and narrows down to the
// token in three wave-wide steps (lane ranges, then units, then the 16 floats
// of one lane) -- integer sums are exact, so the order of summation never
// changes the token.  It then writes the accepted count, the emitted tokens and
// the append, and re-zeroes the workspace.  Published sums carry the call's
// tag (from the ticket, as in the lookup merge), so a sum published after a
// gathering gave up (accept = -1) is never taken by a later call.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lcd.h"

namespace lcd {
namespace {

using u64 = unsigned long long;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnit = 1024;                 // floats per unit: 4 x (64 lanes x 4 floats)
// A published unit sum (at most 1024 * 2^40 = 2^50) is tag << 51 | sum, tag =
// epoch + 1 in 1 .. 8191; the request's header word holds the arrival count in
// bits 0..31 and the epoch above.  Zero is "not published" for every tag.
constexpr int kTagShift = 51;
constexpr u64 kSumMask = (1ull << kTagShift) - 1;
constexpr u64 kTagLimit = (1ull << (64 - kTagShift)) - 1;   // epochs 0 .. kTagLimit - 1
constexpr int kPollMax = 1 << 20;           // bound on the gathering's polls (default)
constexpr int kBufferWord3 = 0x00020000;    // gfx9 buffer descriptor, dword 3
// The rows are streamed with the non-temporal cache policy (the nt bit): each
// is read once, and its lines would otherwise displace the launch's small
// per-request data (measured: the sampled batch 25.8 -> 24.8 us per step).
constexpr int kLoadNT = 2;

// Kinds of the distribution a request draws from.
constexpr int kPlain = 0;                   // the target row p_a itself
constexpr int kPointResidual = 1;           // p_a without the rejected token x
constexpr int kModelResidual = 2;           // max(p_a - q_a, 0)
constexpr int kKeep = 4;                    // unit sums a lane keeps in registers (U <= 256)
constexpr int kMaxUpw = 256;                // units per workgroup, at most
constexpr int kPollBatch = 8;               // unit sums a lane loads at once past kKeep

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Probabilities are read clamped into [0, 1], NaN as 0: one v_med3_f32
// against 0 and 1, which on this part sends every NaN (quiet or signalling,
// either sign), -inf and negative values (and -0) to +0, values above 1 and
// +inf to 1, and keeps subnormals.
__device__ __forceinline__ float prob01(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 1.0f); }

// floor(c * 2^40) for c in [0, 1], as A * 2^24 + B with A = floor(c * 2^16)
// and B = floor(fract(c * 2^16) * 2^24): c * 2^16 and the fraction times 2^24
// are exact in fp32, and float-to-unsigned conversion truncates.
__device__ __forceinline__ void split40(float c, uint32_t &a, uint32_t &b) {
    const float y = c * 65536.0f;
    a = (uint32_t)y;
    b = (uint32_t)(__builtin_amdgcn_fractf(y) * 16777216.0f);
}

__device__ __forceinline__ u64 fixed40(float c) {
    uint32_t a, b;
    split40(c, a, b);
    return ((u64)a << 24) + b;
}

// max(p - q, 0) of two clamped probabilities (fp32 subtraction; the median on
// the bits sends negative differences, and -0, to 0).
__device__ __forceinline__ float residual01(float pc, float qc) {
    int b = __float_as_int(pc - qc);
    b = min(max(b, 0), 0x3F800000);
    return __int_as_float(b);
}

// One DPP step on a 64-bit value: both halves move with the same lane pattern;
// lanes without a source (and rows outside the row mask) read 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ u64 dpp64(u64 v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, kCtrl, kRowMask, 0xF, true);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), kCtrl, kRowMask, 0xF, true);
    return ((u64)hi << 32) | lo;
}

// Inclusive prefix sum over the wave's lanes, on DPP: shifts by 1, 2, 4, 8
// within each row of 16 lanes, then row 0's and row 1's last lanes broadcast
// into the rows above (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows
// 2 and 3).  Exact for 64-bit integers.
__device__ __forceinline__ u64 wave_scan(u64 v) {
    v += dpp64<0x111, 0xF>(v);
    v += dpp64<0x112, 0xF>(v);
    v += dpp64<0x114, 0xF>(v);
    v += dpp64<0x118, 0xF>(v);
    v += dpp64<0x142, 0xA>(v);
    v += dpp64<0x143, 0xC>(v);
    return v;
}

__device__ __forceinline__ u64 lane_value(u64 v, int l) {
    return ((u64)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
}

// Sum over the wave's lanes, in every lane.
__device__ __forceinline__ u64 wave_sum(u64 v) { return lane_value(wave_scan(v), 63); }

struct SampleArgs {
    int32_t V;                   // vocabulary size, a multiple of 4
    int32_t U;                   // units per row, ceil(V / 1024)
    int32_t upw;                 // units per workgroup
    int32_t G;                   // workgroups per request
    int32_t polls;               // gathering polls before giving up
};

struct SampleIO {
    const int32_t *block;
    const int32_t *block_len;
    const uint32_t *model_mask;  // nullable
    const float *target_probs;   // [B, 16, V]
    const float *model_probs;    // [B, 7, V], nullable
    const double *u_accept;      // [B, 15]
    const uint64_t *u_sample;    // [B]
    int32_t *accept;
    int32_t *emitted;            // [B, 16]
    int32_t *hist;               // nullable: append
    const int64_t *row_off;
    int32_t *len;
    const int32_t *cap;
};

// The walk over the verify block, identical in every wave of every workgroup
// of the request: lane k < 15 tests slot k.  Returns a; sets the draw's kind,
// the rejected token, its clamped target probability and the lane-k token.
__device__ __forceinline__ int walk_block(int r, int lane, const SampleArgs &sa, const SampleIO &io,
                                          int &kind, int &x_rej, int &xk, float &p_rej) {
    int L = io.block_len[r];
    L = L < 0 ? 0 : (L > LCD_DRAFT_STRIDE ? LCD_DRAFT_STRIDE : L);
    xk = lane < LCD_DRAFT_STRIDE ? io.block[(int64_t)r * LCD_DRAFT_STRIDE + lane] : LCD_PAD;
    const uint32_t mm = (io.model_mask != nullptr && io.model_probs != nullptr) ? io.model_mask[r] : 0u;
    const bool valid = lane < L && xk >= 0 && xk < sa.V;
    const bool use_model = valid && lane < LCD_Q_STRIDE && ((mm >> lane) & 1u);
    const double u = lane < LCD_DRAFT_STRIDE ? io.u_accept[(int64_t)r * LCD_DRAFT_STRIDE + lane] : 0.0;
    // Both gathers in flight at once: every lane loads from an address inside
    // the request's rows (slot 0's row and token 0 where its own slot has no
    // valid token; the target rows where no draft-model rows are given) and
    // masks the value afterwards.
    const int xs = valid ? xk : 0;
    const int ks = lane < LCD_DRAFT_STRIDE ? lane : 0;
    const int qs = lane < LCD_Q_STRIDE ? lane : 0;
    const float *pp = io.target_probs + ((int64_t)r * LCD_TARGET_STRIDE + ks) * sa.V + xs;
    const float *qp = io.model_probs != nullptr
                          ? io.model_probs + ((int64_t)r * LCD_Q_STRIDE + qs) * sa.V + xs
                          : pp;
    const float pv = *pp, qv = *qp;
    const float P = valid ? prob01(pv) : 0.0f;
    const float Q = use_model ? prob01(qv) : 1.0f;
    const bool ok = valid && (u * (double)Q < (double)P);
    const u64 stop = __ballot(lane < L && !ok);
    const int a = stop ? (int)__builtin_ctzll(stop) : L;
    const bool rejected = a < L && ((__ballot(valid) >> a) & 1ull);
    kind = !rejected ? kPlain : (((__ballot(use_model) >> a) & 1ull) ? kModelResidual : kPointResidual);
    const int al = a < 63 ? a : 63;
    x_rej = __builtin_amdgcn_readlane(xk, al);
    p_rej = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(P), al));
    return a;
}

// Weight sum of unit u of the row for one wave (every lane gets it).  The
// point-mass residual is summed as the plain row, and the caller takes out the
// rejected token's weight from the unit that holds it.
__device__ __forceinline__ u64 unit_sum(__amdgpu_buffer_rsrc_t prs, __amdgpu_buffer_rsrc_t qrs,
                                        int u, int lane, bool model) {
    float4 pv[4], qv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        pv[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                               prs, (u * kUnit + 4 * (lane + 64 * k)) * 4, 0, kLoadNT));
    if (model) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            qv[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   qrs, (u * kUnit + 4 * (lane + 64 * k)) * 4, 0, kLoadNT));
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) qv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    uint32_t sa = 0, sb = 0;               // <= 16 * 2^16 and < 16 * 2^24
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float f[4] = {pv[k].x, pv[k].y, pv[k].z, pv[k].w};
        const float g[4] = {qv[k].x, qv[k].y, qv[k].z, qv[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float c = model ? residual01(prob01(f[i]), prob01(g[i])) : prob01(f[i]);
            uint32_t a, b;
            split40(c, a, b);
            sa += a;
            sb += b;
        }
    }
    return wave_sum(((u64)sa << 24) + sb);
}

__global__ void __launch_bounds__(kThreads)
rejection_accept_kernel(SampleArgs sa, SampleIO io, u64 *__restrict__ ws) {
    const int r = blockIdx.x / sa.G;
    const int c = blockIdx.x - r * sa.G;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int words = 2 + sa.U;             // counter, pad, U unit sums
    u64 *__restrict__ req = ws + (int64_t)r * words;
    u64 *__restrict__ sums = req + 2;

    // Arrival ticket, taken by thread 0 and read back (from wave 0's lane 0)
    // only after the stream; the other lanes' value is left unspecified.  Its
    // return arrives with the walk's first loads, issued after it (taken after
    // the walk instead, or by the last wave, it measured no better).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wsometimes-uninitialized"
#pragma clang diagnostic ignored "-Wuninitialized"
    unsigned long long ticket;
    if (tid == 0)
        ticket = __hip_atomic_fetch_add(req, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // the request's draw word, needed only by the last workgroup: loaded now so
    // that its round trip overlaps the walk and the stream
    const u64 u_draw = io.u_sample[r];

    int kind, x_rej, xk;
    float p_rej;
    const int a = walk_block(r, lane, sa, io, kind, x_rej, xk, p_rej);
    kind = uni(kind);
    x_rej = uni(x_rej);
    const bool model = kind == kModelResidual;
    // the rejected token's weight, taken out of its unit for a point-mass residual
    const u64 w_rej = kind == kPointResidual ? fixed40(p_rej) : 0;
    const int u_rej = kind == kPointResidual ? (x_rej >> 10) : -1;

    // The row the draw reads: target row a, and the draft model's row a for a
    // draft-model residual.  Both rows are 16-byte aligned (V % 4 == 0) and
    // the descriptors cover exactly V floats, so loads past the row read 0.
    const float *prow = io.target_probs + ((int64_t)r * LCD_TARGET_STRIDE + a) * sa.V;
    const float *qrow = model ? io.model_probs + ((int64_t)r * LCD_Q_STRIDE + a) * sa.V : prow;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(prow), 0, sa.V * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(qrow), 0, sa.V * 4, kBufferWord3);

    // ---- stream this workgroup's units -----------------------------------
    const int u0 = c * sa.upw;
    const int u1 = min(u0 + sa.upw, sa.U);
    // The unit sums wait in LDS until the workgroup's ticket -- and with it the
    // call's tag -- is in: wave 0 publishes them all after the barrier.
    __shared__ u64 s_sums[kMaxUpw];
    for (int u = u0 + wave; u < u1; u += kWaves) {
        u64 s = unit_sum(prs, qrs, u, lane, model);
        if (u == u_rej) s -= w_rej;
        if (lane == 0) s_sums[u - u0] = s;
    }
    __syncthreads();
    if (wave != 0) return;
    // lane 0 took the ticket: the arrival count and the call's epoch
    const u64 hdr = ((u64)(uint32_t)__builtin_amdgcn_readfirstlane((int)(ticket >> 32)) << 32) |
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)ticket);
#pragma clang diagnostic pop
    const u64 tagged = ((hdr >> 32) + 1) << kTagShift;   // this call's tag, in place
    for (int k = lane; k < u1 - u0; k += 64)
        __hip_atomic_store(sums + u0 + k, tagged | s_sums[k], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);

    // ---- only the last workgroup of the request to start goes on ------------
    if ((int)(uint32_t)hdr != sa.G - 1) return;

    // Every other workgroup of the request has started and publishes without
    // waiting for anything, so this gathering ends (bounded all the same).
    // Lane l owns units [l*n, l*n + n); up to kKeep of them stay in registers.
    const int n = (sa.U + 63) / 64;
    const int ua = min(lane * n, sa.U), ub = min(ua + n, sa.U);
    u64 kept[kKeep];
    u64 lsum = 0;
    bool all = false;
#pragma unroll
    for (int k = 0; k < kKeep; ++k) kept[k] = 0;
    for (int tries = 0; tries < sa.polls && !all; ++tries) {
        bool ok = true;
        lsum = 0;
        if (n <= kKeep) {
            // all of a lane's loads in flight at once
#pragma unroll
            for (int k = 0; k < kKeep; ++k)
                kept[k] = ua + k < ub ? __hip_atomic_load(sums + ua + k, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT)
                                      : tagged;
#pragma unroll
            for (int k = 0; k < kKeep; ++k) {
                ok = ok && ((kept[k] & ~kSumMask) == tagged);
                kept[k] &= kSumMask;
                lsum += kept[k];
            }
        } else {
            // more than kKeep units per lane (vocabularies past 256 units):
            // batches of kPollBatch loads in flight, not one load per round trip
            for (int u0b = ua; u0b < ub; u0b += kPollBatch) {
                u64 v[kPollBatch];
#pragma unroll
                for (int k = 0; k < kPollBatch; ++k)
                    v[k] = u0b + k < ub ? __hip_atomic_load(sums + u0b + k, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)
                                        : tagged;
#pragma unroll
                for (int k = 0; k < kPollBatch; ++k) {
                    ok = ok && ((v[k] & ~kSumMask) == tagged);
                    lsum += v[k] & kSumMask;
                }
            }
        }
        all = __ballot(!ok) == 0;
    }
    u64 incl = wave_scan(lsum);
    u64 S = lane_value(incl, 63);

    // Draws with no weight.  A draft-model residual with none falls back to the
    // target row: recompute the row's plain unit sums here (rare: it needs
    // p <= q everywhere and a rejection), overwriting the published ones.  A
    // point-mass residual with none means every weight of p_a is the rejected
    // token's.
    int draw_kind = kind;
    int z = -1;
    bool search = all;
    if (all && S == 0 && kind == kModelResidual) {
        draw_kind = kPlain;
        lsum = 0;
#pragma unroll
        for (int k = 0; k < kKeep; ++k) kept[k] = 0;
        for (int u = 0; u < sa.U; ++u) {
            const u64 s = unit_sum(prs, qrs, u, lane, false);
            if (lane == 0)
                __hip_atomic_store(sums + u, tagged | s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (u >= ua && u < ub) {
                lsum += s;
#pragma unroll
                for (int k = 0; k < kKeep; ++k)
                    if (u - ua == k) kept[k] = s;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
        incl = wave_scan(lsum);
        S = lane_value(incl, 63);
    } else if (all && S == 0 && kind == kPointResidual) {
        z = w_rej != 0 ? x_rej : -1;
        search = false;
    }
    if (S == 0) search = false;

    if (search) {
        const u64 t = __umul64hi(u_draw, S);
        // lane range holding t, then the unit, then the lane's 16 floats
        const int l0 = (int)__builtin_ctzll(__ballot(incl > t));
        const u64 before_l = lane_value(incl - lsum, l0);
        const int ub0 = min(l0 * n, sa.U);
        u64 us = 0;
        if (n <= kKeep) {
#pragma unroll
            for (int k = 0; k < kKeep; ++k) {
                const u64 v = lane_value(kept[k], l0);
                if (lane == k) us = v;
            }
        } else if (lane < n && ub0 + lane < sa.U) {
            us = __hip_atomic_load(sums + ub0 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
                 kSumMask;
        }
        if (lane >= n || ub0 + lane >= sa.U) us = 0;
        const u64 uincl = wave_scan(us) + before_l;
        const int lu = (int)__builtin_ctzll(__ballot(uincl > t));
        const int unit = ub0 + lu;
        const u64 before_u = lane_value(uincl - us, lu);
        // lane k holds floats [16k, 16k+16) of the unit
        const int base = unit * kUnit + 16 * lane;
        const bool dm = draw_kind == kModelResidual;
        // all eight loads in flight before the first is used: the draft
        // model's row is read whatever the kind (qrs is the target row itself
        // unless the request drew a draft-model residual), and used only for
        // a draft-model residual.  With the second load behind the kind's
        // test, each 16-float step waited on its own round trip.
        float4 pv4[4], qv4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            pv4[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    prs, (base + 4 * k) * 4, 0, 0));
#pragma unroll
        for (int k = 0; k < 4; ++k)
            qv4[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    qrs, (base + 4 * k) * 4, 0, 0));
        u64 w[16], ls = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 pv = pv4[k];
            const float4 qv = dm ? qv4[k] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float f[4] = {pv.x, pv.y, pv.z, pv.w};
            const float g[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float cw = dm ? residual01(prob01(f[i]), prob01(g[i])) : prob01(f[i]);
                const u64 wi = (draw_kind == kPointResidual && base + 4 * k + i == x_rej) ? 0 : fixed40(cw);
                w[4 * k + i] = wi;
                ls += wi;
            }
        }
        const u64 lincl = wave_scan(ls) + before_u;
        const int lz = (int)__builtin_ctzll(__ballot(lincl > t));
        u64 run = lincl - ls;
        int jz = -1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            run += w[i];
            if (jz < 0 && run > t) jz = base + i;
        }
        z = __builtin_amdgcn_readlane(jz, lz);
    }
    if (!all) z = -1;                       // gathering gave up: the request emits nothing

    // Re-zero the unit sums for the next call, unless the gathering gave up (a
    // late publisher may still write, with this call's tag, which no later
    // call takes); reset the count and start the next epoch.
    if (all)
        for (int u = lane; u < sa.U; u += 64)
            __hip_atomic_store(sums + u, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0) {
        const u64 e = (hdr >> 32) + 1;
        __hip_atomic_store(req, (e < kTagLimit ? e : 0) << 32, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }

    // emitted tokens: block[0..a-1], then z; the append as greedy acceptance does it
    const bool drew = z >= 0;
    const int em = !drew ? LCD_PAD : (lane < a ? xk : (lane == a ? z : LCD_PAD));
    if (lane < LCD_TARGET_STRIDE) io.emitted[(int64_t)r * LCD_TARGET_STRIDE + lane] = em;
    int acc = drew ? a : -1;
    if (drew && io.hist != nullptr) {
        const int32_t l0 = io.len[r];
        const int64_t have = l0 > 0 ? l0 : 0;
        if (have + a + 1 > (int64_t)io.cap[r]) {
            acc = -1;
        } else {
            if (lane <= a) io.hist[io.row_off[r] + have + lane] = em;
            if (lane == 0) io.len[r] = (int32_t)(have + a + 1);
        }
    }
    if (lane == 0) io.accept[r] = acc;
}

// Units per workgroup: a row cut into about 512 / B shares, so that a launch
// holds about two workgroups per CU (2 x 256), each CU streaming the same
// number of units; at least one unit per wave, a multiple of the wave count,
// at most kMaxUpw.  A CU left with one workgroup more than the others streams
// for that much longer, and many small workgroups each pay the walk and a
// slot in the merge: against about 2048 workgroups per launch, 23.1 -> 21.7 us
// at 64 requests over 248,320 ids, 14.4 -> 13.2 at 32, 39.4 -> 37.3 at 128,
// 9.8 -> 9.6 at 16; 9 shares a row at 64 requests (576 workgroups) 26.6 us.
int pick_units_per_wg(int B, int U, int wg_units) {
    if (wg_units > 0) return wg_units;
    const int64_t shares = B > 0 && B < 512 ? 512 / B : 1;
    int64_t upw = (U + shares - 1) / shares;
    upw = (upw + kWaves - 1) / kWaves * kWaves;
    if (upw > kMaxUpw) upw = kMaxUpw;
    return upw < kWaves ? kWaves : (int)upw;
}

int launch(const SampleIO &io, int32_t B, int32_t V, int32_t wg_units, int32_t merge_polls,
           void *workspace, size_t workspace_bytes, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    SampleArgs sa;
    sa.polls = merge_polls == 0 ? kPollMax : (merge_polls < 0 ? 0 : merge_polls);
    sa.V = V;
    sa.U = (V + kUnit - 1) / kUnit;
    sa.upw = pick_units_per_wg(B, sa.U, wg_units);
    sa.G = (sa.U + sa.upw - 1) / sa.upw;
    if (workspace_bytes < rejection_accept_workspace_bytes(B, V)) return LCD_EINVAL;
    const dim3 grid((unsigned)((int64_t)B * sa.G));
    u64 *ws = static_cast<u64 *>(workspace);
    if (ev0 != nullptr || ev1 != nullptr)
        hipExtLaunchKernelGGL(rejection_accept_kernel, grid, dim3(kThreads), 0u, st, ev0, ev1, 0u,
                              sa, io, ws);
    else
        hipLaunchKernelGGL(rejection_accept_kernel, grid, dim3(kThreads), 0, st, sa, io, ws);
    return hipGetLastError() == hipSuccess ? LCD_OK : LCD_EHIP;
}

int sample_entry(const int32_t *block, const int32_t *block_len, const uint32_t *model_mask,
                 const float *target_probs, const float *model_probs, int32_t V,
                 const double *u_accept, const uint64_t *u_sample, int32_t B, int32_t wg_units,
                 int32_t merge_polls, void *workspace, size_t workspace_bytes, int32_t *accept,
                 int32_t *emitted, int32_t *hist, const int64_t *row_off, int32_t *len,
                 const int32_t *cap, void *stream, void *ev0, void *ev1) {
    if (B < 0 || V < 4 || V > LCD_SAMPLE_MAX_VOCAB || (V & 3) != 0 || wg_units < 0 ||
        wg_units > kMaxUpw || merge_polls < -1)
        return LCD_EINVAL;
    if (B == 0) return LCD_OK;
    if (!block || !block_len || !target_probs || !u_accept || !u_sample || !accept || !emitted ||
        !workspace)
        return LCD_EINVAL;
    if ((reinterpret_cast<uintptr_t>(target_probs) & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(model_probs) & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(workspace) & 7) != 0)
        return LCD_EINVAL;
    if (hist && (!row_off || !len || !cap)) return LCD_EINVAL;
    if ((int64_t)B * ((V + kUnit - 1) / kUnit) > (int64_t)1 << 31) return LCD_EINVAL;
    SampleIO io{block, block_len, model_mask, target_probs, model_probs, u_accept, u_sample,
                accept, emitted, hist, row_off, len, cap};
    return launch(io, B, V, wg_units, merge_polls, workspace, workspace_bytes,
                  reinterpret_cast<hipStream_t>(stream), reinterpret_cast<hipEvent_t>(ev0),
                  reinterpret_cast<hipEvent_t>(ev1));
}

}  // namespace
}  // namespace lcd

extern "C" size_t rejection_accept_workspace_bytes(int32_t B, int32_t V) {
    if (B <= 0 || V <= 0) return 0;
    const int64_t U = (V + lcd::kUnit - 1) / lcd::kUnit;
    return (size_t)B * (size_t)(2 + U) * sizeof(unsigned long long);
}

extern "C" int rejection_accept(const int32_t *block, const int32_t *block_len,
                                const uint32_t *model_mask, const float *target_probs,
                                const float *model_probs, int32_t V, const double *u_accept,
                                const uint64_t *u_sample, int32_t B, int32_t wg_units,
                                int32_t merge_polls, void *workspace, size_t workspace_bytes,
                                int32_t *accept, int32_t *emitted, int32_t *hist,
                                const int64_t *row_off, int32_t *len, const int32_t *cap,
                                void *stream) {
    return lcd::sample_entry(block, block_len, model_mask, target_probs, model_probs, V, u_accept,
                             u_sample, B, wg_units, merge_polls, workspace, workspace_bytes, accept,
                             emitted, hist, row_off, len, cap, stream, nullptr, nullptr);
}

extern "C" int rejection_accept_timed(const int32_t *block, const int32_t *block_len,
                                      const uint32_t *model_mask, const float *target_probs,
                                      const float *model_probs, int32_t V, const double *u_accept,
                                      const uint64_t *u_sample, int32_t B, int32_t wg_units,
                                      int32_t merge_polls, void *workspace, size_t workspace_bytes,
                                      int32_t *accept, int32_t *emitted, int32_t *hist,
                                      const int64_t *row_off, int32_t *len, const int32_t *cap,
                                      void *stream, void *ev_start, void *ev_stop) {
    return lcd::sample_entry(block, block_len, model_mask, target_probs, model_probs, V, u_accept,
                             u_sample, B, wg_units, merge_polls, workspace, workspace_bytes, accept,
                             emitted, hist, row_off, len, cap, stream, ev_start, ev_stop);
}

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
// the append, and re-zeroes the workspace.

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
constexpr u64 kSumValid = 1ull << 63;       // tag of a published unit sum (sums < 2^51)
constexpr int kPollMax = 1 << 20;           // bound on the gathering's polls
constexpr int kBufferWord3 = 0x00020000;    // gfx9 buffer descriptor, dword 3

// Kinds of the distribution a request draws from.
constexpr int kPlain = 0;                   // the target row p_a itself
constexpr int kPointResidual = 1;           // p_a without the rejected token x
constexpr int kModelResidual = 2;           // max(p_a - q_a, 0)

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Probabilities are read clamped into [0, 1]; NaN reads as 0.
__device__ __forceinline__ float prob01(float x) { return x > 0.0f ? fminf(x, 1.0f) : 0.0f; }

// floor(w * 2^40) for w in [0, 1], from the float's fields: w = M * 2^(e-150)
// with the 24-bit significand M, so w * 2^40 = M * 2^(e-110).
__device__ __forceinline__ u64 fixed40(float w) {
    const uint32_t b = __float_as_uint(w);
    const int e = (int)(b >> 23);
    const u64 M = (u64)((b & 0x7FFFFFu) | 0x800000u);
    if (e >= 110) return M << (e - 110);
    if (e <= 86) return 0;                  // below 2^-40 (and zero, subnormals)
    return M >> (110 - e);
}

__device__ __forceinline__ float weight(int kind, float p, float q, int j, int x) {
    const float pc = prob01(p);
    if (kind == kModelResidual) {
        const float d = pc - prob01(q);
        return d > 0.0f ? d : 0.0f;
    }
    return (kind == kPointResidual && j == x) ? 0.0f : pc;
}

__device__ __forceinline__ u64 wave_sum(u64 v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ u64 wave_scan(u64 v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const u64 o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    return v;
}

struct SampleArgs {
    int32_t V;                   // vocabulary size, a multiple of 4
    int32_t U;                   // units per row, ceil(V / 1024)
    int32_t upw;                 // units per workgroup
    int32_t G;                   // workgroups per request
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
// the rejected token and the lane-k block token.
__device__ __forceinline__ int walk_block(int r, int lane, const SampleArgs &sa, const SampleIO &io,
                                          int &kind, int &x_rej, int &xk, float &p_rej) {
    int L = io.block_len[r];
    L = L < 0 ? 0 : (L > LCD_DRAFT_STRIDE ? LCD_DRAFT_STRIDE : L);
    xk = lane < LCD_DRAFT_STRIDE ? io.block[(int64_t)r * LCD_DRAFT_STRIDE + lane] : LCD_PAD;
    const uint32_t mm = (io.model_mask != nullptr && io.model_probs != nullptr) ? io.model_mask[r] : 0u;
    const bool valid = lane < L && xk >= 0 && xk < sa.V;
    const bool use_model = valid && lane < LCD_Q_STRIDE && ((mm >> lane) & 1u);
    float P = 0.0f, Q = 1.0f;
    double u = 0.0;
    if (valid) {
        P = prob01(io.target_probs[((int64_t)r * LCD_TARGET_STRIDE + lane) * sa.V + xk]);
        u = io.u_accept[(int64_t)r * LCD_DRAFT_STRIDE + lane];
    }
    if (use_model) Q = prob01(io.model_probs[((int64_t)r * LCD_Q_STRIDE + lane) * sa.V + xk]);
    const bool ok = valid && (u * (double)Q < (double)P);
    const u64 stop = __ballot(lane < L && !ok);
    const int a = stop ? (int)__builtin_ctzll(stop) : L;
    const bool rejected = a < L && ((__ballot(valid) >> a) & 1ull);
    kind = !rejected ? kPlain : (((__ballot(use_model) >> a) & 1ull) ? kModelResidual : kPointResidual);
    x_rej = __shfl(xk, a < 63 ? a : 63);
    p_rej = __shfl(P, a < 63 ? a : 63);
    return a;
}

__global__ void __launch_bounds__(kThreads)
rejection_accept_kernel(SampleArgs sa, SampleIO io, u64 *__restrict__ ws) {
    const int r = blockIdx.x / sa.G;
    const int c = blockIdx.x - r * sa.G;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int words = 2 + 2 * sa.U;         // counter, pad, U draw sums, U plain sums
    u64 *__restrict__ req = ws + (int64_t)r * words;
    u64 *__restrict__ sums = req + 2;

    unsigned long long ticket = 0;
    if (tid == 0)
        ticket = __hip_atomic_fetch_add(req, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    int kind, x_rej, xk;
    float p_rej;
    const int a = walk_block(r, lane, sa, io, kind, x_rej, xk, p_rej);
    kind = uni(kind);
    x_rej = uni(x_rej);

    // The row the draw reads: target row a, and the draft model's row a for a
    // draft-model residual.  Both rows are 16-byte aligned (V % 4 == 0) and
    // the descriptors cover exactly V floats, so loads past the row read 0.
    const float *prow = io.target_probs + ((int64_t)r * LCD_TARGET_STRIDE + a) * sa.V;
    const float *qrow = kind == kModelResidual
                            ? io.model_probs + ((int64_t)r * LCD_Q_STRIDE + a) * sa.V : prow;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(prow), 0, sa.V * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(qrow), 0, sa.V * 4, kBufferWord3);

    // ---- stream this workgroup's units -----------------------------------
    const int u0 = c * sa.upw;
    const int u1 = min(u0 + sa.upw, sa.U);
    for (int u = u0 + wave; u < u1; u += kWaves) {
        float4 pv[4], qv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            pv[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   prs, (u * kUnit + 4 * (lane + 64 * k)) * 4, 0, 0));
        if (kind == kModelResidual) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                qv[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       qrs, (u * kUnit + 4 * (lane + 64 * k)) * 4, 0, 0));
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) qv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        u64 s = 0, sp = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = u * kUnit + 4 * (lane + 64 * k);
            s += fixed40(weight(kind, pv[k].x, qv[k].x, j + 0, x_rej));
            s += fixed40(weight(kind, pv[k].y, qv[k].y, j + 1, x_rej));
            s += fixed40(weight(kind, pv[k].z, qv[k].z, j + 2, x_rej));
            s += fixed40(weight(kind, pv[k].w, qv[k].w, j + 3, x_rej));
            if (kind == kModelResidual)
                sp += fixed40(prob01(pv[k].x)) + fixed40(prob01(pv[k].y)) +
                      fixed40(prob01(pv[k].z)) + fixed40(prob01(pv[k].w));
        }
        s = wave_sum(s);
        if (kind == kModelResidual) sp = wave_sum(sp);
        if (lane == 0) {
            __hip_atomic_store(sums + u, kSumValid | s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (kind == kModelResidual)
                __hip_atomic_store(sums + sa.U + u, kSumValid | sp, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // ---- only the last workgroup of the request to start goes on ------------
    __shared__ int s_last;
    if (tid == 0) s_last = (int)ticket == sa.G - 1;
    __syncthreads();
    if (!s_last || wave != 0) return;

    // Every other workgroup of the request has started and publishes without
    // waiting for anything, so this gathering ends (bounded all the same).
    // Lane l owns units [l*n, l*n + n).
    const int n = (sa.U + 63) / 64;
    const int ua = min(lane * n, sa.U), ub = min(ua + n, sa.U);
    const int nsets = kind == kModelResidual ? 2 : 1;
    u64 lsum[2] = {0, 0};
    bool all = false;
    for (int tries = 0; tries < kPollMax && !all; ++tries) {
        bool ok = true;
        for (int set = 0; set < nsets; ++set) {
            u64 acc = 0;
            for (int u = ua; u < ub; ++u) {
                const u64 v = __hip_atomic_load(sums + set * sa.U + u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
                ok = ok && (v != 0);
                acc += v & ~kSumValid;
            }
            lsum[set] = acc;
        }
        all = __ballot(!ok) == 0;
    }

    // Total of the draw's weights; a draft-model residual with no mass falls
    // back to the target row (its plain sums were published alongside), a
    // point-mass residual with no mass means every weight of p_a sits on the
    // rejected token.
    int set = 0;
    int draw_kind = kind;
    u64 incl = wave_scan(lsum[0], lane);
    u64 S = __shfl(incl, 63);
    int z = -1;
    bool search = true;
    if (S == 0 && kind == kModelResidual) {
        set = 1;
        draw_kind = kPlain;
        incl = wave_scan(lsum[1], lane);
        S = __shfl(incl, 63);
    } else if (S == 0 && kind == kPointResidual) {
        z = fixed40(p_rej) != 0 ? x_rej : -1;
        search = false;
    }
    if (S == 0) search = false;

    if (search && all) {
        const u64 t = __umul64hi(io.u_sample[r], S);
        // lane range holding t, then the unit, then the lane's 16 floats
        const u64 lane_at = __ballot(incl > t);
        const int l0 = (int)__builtin_ctzll(lane_at);
        const u64 before_l = __shfl(incl - lsum[set], l0);
        const int ub0 = min(l0 * n, sa.U);
        const int uu = ub0 + lane;
        u64 us = 0;
        if (lane < n && uu < sa.U)
            us = __hip_atomic_load(sums + set * sa.U + uu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
                 ~kSumValid;
        const u64 uincl = wave_scan(us, lane) + before_l;
        const int lu = (int)__builtin_ctzll(__ballot(uincl > t));
        const int unit = ub0 + lu;
        const u64 before_u = __shfl(uincl - us, lu);
        // lane k holds floats [16k, 16k+16) of the unit
        float f[16], g[16];
        const int base = unit * kUnit + 16 * lane;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 pv = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          prs, (base + 4 * k) * 4, 0, 0));
            const float4 qv = draw_kind == kModelResidual
                                  ? __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                   qrs, (base + 4 * k) * 4, 0, 0))
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
            f[4 * k + 0] = pv.x; f[4 * k + 1] = pv.y; f[4 * k + 2] = pv.z; f[4 * k + 3] = pv.w;
            g[4 * k + 0] = qv.x; g[4 * k + 1] = qv.y; g[4 * k + 2] = qv.z; g[4 * k + 3] = qv.w;
        }
        u64 w[16], ls = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            w[i] = fixed40(weight(draw_kind, f[i], g[i], base + i, x_rej));
            ls += w[i];
        }
        const u64 lincl = wave_scan(ls, lane) + before_u;
        const int lz = (int)__builtin_ctzll(__ballot(lincl > t));
        u64 run = lincl - ls;
        int jz = -1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            run += w[i];
            if (jz < 0 && run > t) jz = base + i;
        }
        z = __shfl(jz, lz);
    }
    if (!all) z = -1;                       // gathering gave up: the request emits nothing

    // re-zero the request's workspace for the next call
    for (int u = lane; u < 2 * sa.U; u += 64)
        __hip_atomic_store(sums + u, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0) __hip_atomic_store(req, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

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

// Units per workgroup: about 2048 workgroups per launch, at least one unit per
// wave, a multiple of the wave count.
int pick_units_per_wg(int B, int U, int wg_units) {
    if (wg_units > 0) return wg_units;
    const int64_t total = (int64_t)B * U;
    int upw = (int)((total + 2047) / 2048);
    upw = (upw + kWaves - 1) / kWaves * kWaves;
    return upw < kWaves ? kWaves : upw;
}

int launch(const SampleIO &io, int32_t B, int32_t V, int32_t wg_units, void *workspace,
           size_t workspace_bytes, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    SampleArgs sa;
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
                 void *workspace, size_t workspace_bytes, int32_t *accept, int32_t *emitted,
                 int32_t *hist, const int64_t *row_off, int32_t *len, const int32_t *cap,
                 void *stream, void *ev0, void *ev1) {
    if (B < 0 || V < 4 || V > LCD_SAMPLE_MAX_VOCAB || (V & 3) != 0 || wg_units < 0 ||
        wg_units > (1 << 20))
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
    return launch(io, B, V, wg_units, workspace, workspace_bytes,
                  reinterpret_cast<hipStream_t>(stream), reinterpret_cast<hipEvent_t>(ev0),
                  reinterpret_cast<hipEvent_t>(ev1));
}

}  // namespace
}  // namespace lcd

extern "C" size_t rejection_accept_workspace_bytes(int32_t B, int32_t V) {
    if (B <= 0 || V <= 0) return 0;
    const int64_t U = (V + lcd::kUnit - 1) / lcd::kUnit;
    return (size_t)B * (size_t)(2 + 2 * U) * sizeof(unsigned long long);
}

extern "C" int rejection_accept(const int32_t *block, const int32_t *block_len,
                                const uint32_t *model_mask, const float *target_probs,
                                const float *model_probs, int32_t V, const double *u_accept,
                                const uint64_t *u_sample, int32_t B, int32_t wg_units,
                                void *workspace, size_t workspace_bytes, int32_t *accept,
                                int32_t *emitted, int32_t *hist, const int64_t *row_off,
                                int32_t *len, const int32_t *cap, void *stream) {
    return lcd::sample_entry(block, block_len, model_mask, target_probs, model_probs, V, u_accept,
                             u_sample, B, wg_units, workspace, workspace_bytes, accept, emitted,
                             hist, row_off, len, cap, stream, nullptr, nullptr);
}

extern "C" int rejection_accept_timed(const int32_t *block, const int32_t *block_len,
                                      const uint32_t *model_mask, const float *target_probs,
                                      const float *model_probs, int32_t V, const double *u_accept,
                                      const uint64_t *u_sample, int32_t B, int32_t wg_units,
                                      void *workspace, size_t workspace_bytes, int32_t *accept,
                                      int32_t *emitted, int32_t *hist, const int64_t *row_off,
                                      int32_t *len, const int32_t *cap, void *stream,
                                      void *ev_start, void *ev_stop) {
    return lcd::sample_entry(block, block_len, model_mask, target_probs, model_probs, V, u_accept,
                             u_sample, B, wg_units, workspace, workspace_bytes, accept, emitted,
                             hist, row_off, len, cap, stream, ev_start, ev_stop);
}

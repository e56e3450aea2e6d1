// lcd_lookup.hip -- batched context lookup (longest suffix, latest earlier
// occurrence, LZ-style draft copy) for MI355X / gfx950.
//
// Method: HyperQwen lookup-drafting article, section "第 1 步": each decode
// step, for every request, scan that request's own token history for the most
// recent earlier occurrence of its longest current suffix of 4..12 tokens
// (overlap with the suffix allowed) and draft the tokens that follow it; most
// candidates are rejected by a 4-token test, so extending the survivors costs
// almost nothing.  The article runs one Triton program per request on a
// consumer GPU; here the design is built around gfx950 instead:
//
//  * The whole batch is one flat token space (prefix sums of the lengths).  It
//    is cut into gridDim.x equal ranges, one per workgroup, so a ragged batch
//    is as balanced as a uniform one and a launch always fills all 256 CUs.
//    Each workgroup computes the prefix sums itself in LDS from len[] (no
//    extra launch, no host knowledge of the lengths).
//  * Within a range each wave streams contiguous 256-token tiles: lane i holds
//    tokens 4i..4i+3 of the tile from one 16-byte load, so one wave-wide load
//    moves 1 KiB, fully coalesced, 16-byte aligned.
//  * The 4-token rejection test runs on wave-wide bit masks: one v_cmp per
//    (component, suffix token) gives a 64-bit ballot, and the masks are
//    shifted by whole lanes to line up positions e, e-1, e-2, e-3.  The test
//    costs 4 compares per token and no divergence; tiles with no survivor
//    (nearly all of them) go straight to the next tile on a scalar branch.
//  * Survivor tiles extend all candidates at once with the same mask algebra
//    up to l_max tokens (lane shifts of up to 4, carried from the previous
//    tile), and pick the longest, then latest, candidate with scalar bit scans.
//  * A packed key (length << 32 | end) orders candidates; workgroups covering
//    one request merge keys with a 64-bit atomic max, and the last one to
//    arrive (counted with an acquire-release atomic) writes the result and the
//    15-token draft and re-zeroes the two workspace words it used.
//
// No MFMA: the work is integer compares on a stream; HBM bandwidth bounds it.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lcd.h"

namespace lcd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileTok = 256;   // 64 lanes x 4 tokens
constexpr int kUnroll = 8;      // tiles loaded ahead by each wave

typedef unsigned long long u64;

struct ScanArgs {
    int32_t l_min, l_max, k_max;
};

struct WsSlot {   // one per request, 16 bytes, zero between calls
    u64 key;
    unsigned int count;
    unsigned int pad;
};

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int64_t uni64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ u64 ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int tok(const int4 &t, int c) {
    return c == 0 ? t.x : (c == 1 ? t.y : (c == 2 ? t.z : t.w));
}

// Replace tokens at absolute positions < row_start by `sent`.
__device__ __forceinline__ int4 mask_before(int4 t, int64_t pos0, int64_t row_start, int sent) {
    t.x = (pos0 + 0 < row_start) ? sent : t.x;
    t.y = (pos0 + 1 < row_start) ? sent : t.y;
    t.z = (pos0 + 2 < row_start) ? sent : t.z;
    t.w = (pos0 + 3 < row_start) ? sent : t.w;
    return t;
}

// Prefilter masks of one tile for a PF-token test (PF <= 4).  Bit i of the
// result for component c stands for the candidate end at tile position 4i+c.
// in[c]  = AND over j<PF, j<=c of [token(4i+c-j) == s_j]   (same lane)
// sh[c]  = AND over j<PF, j>c  of [token(4i+c-j+4) == s_j] (taken from lane
//          i-1, i.e. this mask is shifted up by one lane before use)
template <int PF>
__device__ __forceinline__ void prefilter_masks(const int4 &t, const int *s, u64 in[4], u64 sh[4]) {
    u64 E[4][4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < PF; ++j) E[c][j] = ballot(tok(t, c) == s[j]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        u64 a = ~0ull, b = ~0ull;
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            if (j <= c) a &= E[c - j][j];
            else b &= E[c - j + 4][j];
        }
        in[c] = a;
        sh[c] = b;
    }
}

// Extend the prefilter survivors M[c] of tile t (previous tile pt) to the
// largest length L <= J for which some candidate still matches; returns L (and
// leaves in M the candidates that match at least L tokens).
template <int PF>
__device__ __forceinline__ int extend(const int4 &t, const int4 &pt, const int *s, int J, u64 M[4]) {
    int L = PF;
#pragma unroll
    for (int j = PF; j < LCD_MAX_SUFFIX; ++j) {
        if (j >= J) break;
        u64 N[4];
        u64 any = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int k = (j - c + 3) >> 2;      // lanes back: ceil((j-c)/4)
            const int cc = (c - j) & 3;          // component of position e-j
            const u64 cur = ballot(tok(t, cc) == s[j]);
            u64 term = cur;
            if (k > 0) {
                const u64 prev = ballot(tok(pt, cc) == s[j]);
                term = (cur << k) | (prev >> (64 - k));
            }
            N[c] = M[c] & term;
            any |= N[c];
        }
        if (any == 0) break;
#pragma unroll
        for (int c = 0; c < 4; ++c) M[c] = N[c];
        L = j + 1;
    }
    return L;
}

template <int PF>
__global__ void __launch_bounds__(kThreads)
lookup_scan_kernel(const int32_t *__restrict__ hist, const int64_t *__restrict__ row_off,
                   const int32_t *__restrict__ len, int32_t B, ScanArgs a,
                   WsSlot *__restrict__ ws, int32_t *__restrict__ match_len,
                   int32_t *__restrict__ match_end, int32_t *__restrict__ draft)
{
    extern __shared__ int64_t lds[];
    int64_t *s_pref = lds;            // [B+1] exclusive prefix of lengths
    int64_t *s_roff = lds + (B + 1);  // [B]   row offsets
    __shared__ u64 s_wkey[kWaves];
    __shared__ long long s_wsum[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int G = gridDim.x;
    const int g = blockIdx.x;

    // ---- prefix sums of the lengths (every workgroup, in LDS) ----------------
    for (int r = tid; r < B; r += kThreads) {
        s_roff[r] = row_off[r];
        const int32_t n = len[r];
        s_pref[r + 1] = n > 0 ? n : 0;
    }
    __syncthreads();
    {
        const int per = (B + kThreads - 1) / kThreads;
        const int lo = tid * per;
        const int hi = min(B, lo + per);
        long long local = 0;
        for (int r = lo; r < hi; ++r) local += s_pref[r + 1];
        long long incl = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const long long v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        if (lane == 63) s_wsum[wave] = incl;
        __syncthreads();
        long long run = incl - local;
        for (int w = 0; w < wave; ++w) run += s_wsum[w];
        for (int r = lo; r < hi; ++r) {
            run += s_pref[r + 1];
            s_pref[r + 1] = run;
        }
        if (tid == 0) s_pref[0] = 0;
    }
    __syncthreads();

    const int64_t N = s_pref[B];
    int64_t T = (N + G - 1) / G;
    T = ((T + kTileTok - 1) / kTileTok) * kTileTok;
    if (T == 0) T = kTileTok;
    const int64_t g_lo = (int64_t)g * T;
    const int64_t g_hi = g_lo + T;

    // ---- empty requests: written by the workgroup whose range holds them -----
    for (int r = tid; r < B; r += kThreads) {
        if (s_pref[r + 1] == s_pref[r]) {
            int64_t owner = s_pref[r] / T;
            if (owner > G - 1) owner = G - 1;
            if (owner == g) {
                match_len[r] = 0;
                match_end[r] = -1;
                for (int k = 0; k < LCD_DRAFT_STRIDE; ++k) draft[(int64_t)r * LCD_DRAFT_STRIDE + k] = LCD_PAD;
            }
        }
    }

    // first request whose tokens reach into [g_lo, g_hi)
    int rb = 0, re = B;
    while (rb < re) {
        const int mid = (rb + re) >> 1;
        if (s_pref[mid + 1] > g_lo) re = mid; else rb = mid + 1;
    }

    const int J = a.l_max;
    for (int r = uni(rb); r < B; ++r) {
        const int64_t S = uni64(s_pref[r]);
        if (S >= g_hi) break;
        const int64_t n = uni64(s_pref[r + 1]) - S;
        if (n == 0) continue;
        const int64_t ro = uni64(s_roff[r]);
        const int64_t seg_a = (g_lo > S ? g_lo : S) - S;
        const int64_t seg_b = ((g_hi < S + n) ? g_hi : S + n) - S;
        const int contrib = (int)((S + n - 1) / T - S / T + 1);

        // suffix s_j = h[n-1-j]; positions before the row are never compared
        // for a real candidate, so any filler value works there
        int s[LCD_MAX_SUFFIX];
        {
            int v = INT32_MIN;
            if (lane < LCD_MAX_SUFFIX && lane < n) v = hist[ro + n - 1 - lane];
#pragma unroll
            for (int j = 0; j < LCD_MAX_SUFFIX; ++j) s[j] = __builtin_amdgcn_readlane(v, j);
        }
        // a value equal to no suffix token stands in for tokens before the row
        int sent = s[0] + 1;
        for (int it = 0; it <= LCD_MAX_SUFFIX; ++it) {
            bool hit = false;
#pragma unroll
            for (int j = 0; j < LCD_MAX_SUFFIX; ++j) hit |= (s[j] == sent);
            if (!hit) break;
            ++sent;
        }
        sent = uni(sent);

        const int64_t cand_lo = ro + seg_a;                               // absolute
        const int64_t cand_hi = ro + (seg_b < n - 1 ? seg_b : n - 1);     // exclusive
        u64 best = 0;
        if (cand_hi > cand_lo) {
            const int64_t X0 = cand_lo & ~(int64_t)3;
            const int64_t nt = (cand_hi - X0 + kTileTok - 1) / kTileTok;
            const int64_t tpw = (nt + kWaves - 1) / kWaves;
            const int64_t k0 = tpw * wave;
            const int64_t k1 = (k0 + tpw < nt) ? k0 + tpw : nt;
            if (k0 < k1) {
                // previous-tile tokens for the first tile: lanes 60..63 hold
                // the 16 tokens just before it
                int4 pt;
                {
                    const int64_t A = X0 + kTileTok * k0;
                    const int64_t gpos = A - kTileTok + 4 * lane;
                    pt = make_int4(sent, sent, sent, sent);
                    if (lane >= 60 && gpos + 4 > ro)
                        pt = *reinterpret_cast<const int4 *>(hist + gpos);
                    pt = mask_before(pt, gpos, ro, sent);
                }
                u64 pin[4], psh[4];
                prefilter_masks<PF>(pt, s, pin, psh);

                for (int64_t kb = k0; kb < k1; kb += kUnroll) {
                    int4 buf[kUnroll];
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u) {
                        buf[u] = make_int4(sent, sent, sent, sent);
                        const int64_t gpos = X0 + kTileTok * (kb + u) + 4 * lane;
                        if (kb + u < k1 && gpos < cand_hi)
                            buf[u] = *reinterpret_cast<const int4 *>(hist + gpos);
                    }
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u) {
                        if (kb + u >= k1) break;
                        const int64_t A = X0 + kTileTok * (kb + u);
                        int4 t = buf[u];
                        if (A < ro) t = mask_before(t, A + 4 * lane, ro, sent);
                        u64 in[4], sh[4];
                        prefilter_masks<PF>(t, s, in, sh);
                        u64 P[4];
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            P[c] = in[c] & ((sh[c] << 1) | (psh[c] >> 63));
                        if (A < cand_lo || A + kTileTok > cand_hi) {
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                const int64_t x = A + 4 * lane + c;
                                P[c] &= ballot(x >= cand_lo && x < cand_hi);
                            }
                        }
                        if ((P[0] | P[1] | P[2] | P[3]) != 0) {
                            const int L = extend<PF>(t, pt, s, J, P);
                            if (L >= a.l_min) {
                                int ebest = -1;
#pragma unroll
                                for (int c = 0; c < 4; ++c) {
                                    if (P[c]) {
                                        const int e = 4 * (63 - __clzll(P[c])) + c;
                                        ebest = e > ebest ? e : ebest;
                                    }
                                }
                                const u64 key = ((u64)L << 32) | (u64)(uint32_t)(A + ebest - ro);
                                best = key > best ? key : best;
                            }
                        }
                        pt = t;
#pragma unroll
                        for (int c = 0; c < 4; ++c) psh[c] = sh[c];
                    }
                }
            }
        }

        if (lane == 0) s_wkey[wave] = best;
        __syncthreads();
        if (tid == 0) {
            u64 key = s_wkey[0];
            for (int w = 1; w < kWaves; ++w) key = s_wkey[w] > key ? s_wkey[w] : key;
            bool last = true;
            if (contrib > 1) {
                WsSlot *slot = ws + r;
                if (key) __hip_atomic_fetch_max(&slot->key, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const unsigned old = __hip_atomic_fetch_add(&slot->count, 1u, __ATOMIC_ACQ_REL,
                                                            __HIP_MEMORY_SCOPE_AGENT);
                last = (old == (unsigned)(contrib - 1));
                if (last) {
                    key = __hip_atomic_load(&slot->key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(&slot->key, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(&slot->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            if (last) {
                int32_t *d = draft + (int64_t)r * LCD_DRAFT_STRIDE;
                if (key == 0) {
                    match_len[r] = 0;
                    match_end[r] = -1;
                    for (int k = 0; k < LCD_DRAFT_STRIDE; ++k) d[k] = LCD_PAD;
                } else {
                    const int m = (int)(key >> 32);
                    const int64_t e = (int64_t)(uint32_t)key;
                    const int64_t D = n - 1 - e;
                    match_len[r] = m;
                    match_end[r] = (int32_t)e;
                    int64_t idx = 0;   // k mod D
                    for (int k = 0; k < LCD_DRAFT_STRIDE; ++k) {
                        d[k] = (k < a.k_max) ? hist[ro + n - D + idx] : LCD_PAD;
                        if (++idx == D) idx = 0;
                    }
                }
            }
        }
        __syncthreads();
    }
}

constexpr int kMaxBPerLaunch = 1024;

int pick_grid(int32_t nb, int32_t max_len, int32_t scan_wgs) {
    if (scan_wgs > 0) return scan_wgs;
    const int64_t total = (int64_t)nb * (int64_t)(max_len > 0 ? max_len : 1);
    int64_t G = (total + 4095) / 4096;
    if (G < 1) G = 1;
    if (G > 2048) G = 2048;
    return (int)G;
}

template <int PF>
hipError_t launch(const int32_t *hist, const int64_t *row_off, const int32_t *len, int32_t nb,
                  int G, ScanArgs sa, WsSlot *ws, int32_t *ml, int32_t *me, int32_t *dr,
                  hipStream_t st) {
    const size_t lds_bytes = (size_t)(2 * nb + 1) * sizeof(int64_t);
    hipLaunchKernelGGL(lookup_scan_kernel<PF>, dim3(G), dim3(kThreads), lds_bytes, st,
                       hist, row_off, len, nb, sa, ws, ml, me, dr);
    return hipGetLastError();
}

}  // namespace
}  // namespace lcd

extern "C" size_t lcd_workspace_bytes(int32_t B) {
    return B > 0 ? (size_t)B * sizeof(lcd::WsSlot) : 0;
}

extern "C" int lookup_propose(const int32_t *hist, const int64_t *row_off, const int32_t *len,
                              int32_t B, int32_t max_len, const lcd_params *p, void *workspace,
                              int32_t *match_len, int32_t *match_end, int32_t *draft, void *stream) {
    using namespace lcd;
    if (B < 0 || p == nullptr || max_len < 0) return LCD_EINVAL;
    if (lcd_check_params(p) != LCD_OK) return LCD_EINVAL;
    if (B == 0) return LCD_OK;
    if (!hist || !row_off || !len || !workspace || !match_len || !match_end || !draft)
        return LCD_EINVAL;
    if (((uintptr_t)hist & 15u) != 0 || ((uintptr_t)workspace & 15u) != 0) return LCD_EINVAL;

    ScanArgs sa{p->l_min, p->l_max, p->k_max};
    const int pf = p->l_min < 4 ? p->l_min : 4;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    WsSlot *ws = reinterpret_cast<WsSlot *>(workspace);
    for (int32_t r0 = 0; r0 < B; r0 += kMaxBPerLaunch) {
        const int32_t nb = (B - r0) < kMaxBPerLaunch ? (B - r0) : kMaxBPerLaunch;
        const int G = pick_grid(nb, max_len, p->scan_wgs);
        hipError_t err;
        switch (pf) {
        case 1: err = launch<1>(hist, row_off + r0, len + r0, nb, G, sa, ws + r0, match_len + r0,
                                match_end + r0, draft + (int64_t)r0 * LCD_DRAFT_STRIDE, st); break;
        case 2: err = launch<2>(hist, row_off + r0, len + r0, nb, G, sa, ws + r0, match_len + r0,
                                match_end + r0, draft + (int64_t)r0 * LCD_DRAFT_STRIDE, st); break;
        case 3: err = launch<3>(hist, row_off + r0, len + r0, nb, G, sa, ws + r0, match_len + r0,
                                match_end + r0, draft + (int64_t)r0 * LCD_DRAFT_STRIDE, st); break;
        default: err = launch<4>(hist, row_off + r0, len + r0, nb, G, sa, ws + r0, match_len + r0,
                                 match_end + r0, draft + (int64_t)r0 * LCD_DRAFT_STRIDE, st); break;
        }
        if (err != hipSuccess) return LCD_EHIP;
    }
    return LCD_OK;
}

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

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lcd.h"

namespace lcd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileTok = 256;   // 64 lanes x 4 tokens
#ifndef LCD_UNROLL
#define LCD_UNROLL 8
#endif
constexpr int kUnroll = LCD_UNROLL;   // tiles loaded ahead by each wave

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

// Replace the tokens of this lane's granule that lie before the row start by
// `sent`; `rel` is the row start minus the granule's first position.
__device__ __forceinline__ int4 mask_before(int4 t, int rel, int sent) {
    t.x = (0 < rel) ? sent : t.x;
    t.y = (1 < rel) ? sent : t.y;
    t.z = (2 < rel) ? sent : t.z;
    t.w = (3 < rel) ? sent : t.w;
    return t;
}

// Prefilter masks of one tile for a PF-token test (PF <= 4).  Bit i of the
// masks for component c stands for the candidate end at tile position 4i+c.
//   in[c] = [token(4i+c-j) == s_j for all j<PF, j<=c]     (same lane)
//   sh[c] = [token(4i+c-j+4) == s_j for all j<PF, j>c]    (lane i-1's
//           tokens, so this mask is shifted up one lane before use)
// Equalities are combined per lane with xor/or, then one ballot per mask
// gives a wave-uniform 64-bit mask.
template <int PF>
__device__ __forceinline__ void prefilter_masks(const int4 &t, const int (&s)[4], u64 in[4], u64 sh[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        unsigned x = 0, y = 0;
        bool has_y = false;
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            if (j <= c) {
                x |= (unsigned)(tok(t, c - j) ^ s[j]);
            } else {
                y |= (unsigned)(tok(t, c - j + 4) ^ s[j]);
                has_y = true;
            }
        }
        in[c] = ballot(x == 0);
        sh[c] = has_y ? ballot(y == 0) : ~0ull;
    }
}

// Extend the prefilter survivors M[c] of tile t (previous tile pt) one suffix
// token at a time, up to J tokens, while some candidate still matches.  Returns
// the largest length reached and leaves in M the candidates matching it.
template <int PF>
__device__ __forceinline__ int extend(const int4 &t, const int4 &pt, const int (&sj16)[LCD_MAX_SUFFIX], int J, u64 M[4]) {
    int L = PF;
    bool alive = true;
#pragma unroll
    for (int j = PF; j < LCD_MAX_SUFFIX; ++j) {
        if (alive && j < J) {
            const int sj = sj16[j];
            u64 N[4];
            u64 any = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int k = (j - c + 3) >> 2;      // lanes back: ceil((j-c)/4)
                const int cc = (c - j) & 3;          // component of position e-j
                const u64 cur = ballot(tok(t, cc) == sj);
                u64 term = cur;
                if (k > 0) {
                    const u64 prev = ballot(tok(pt, cc) == sj);
                    term = (cur << k) | (prev >> (64 - k));
                }
                N[c] = M[c] & term;
                any |= N[c];
            }
            if (any != 0) {
#pragma unroll
                for (int c = 0; c < 4; ++c) M[c] = N[c];
                L = j + 1;
            } else {
                alive = false;
            }
        }
    }
    return L;
}

__device__ __forceinline__ int4 load_granule(const int32_t *__restrict__ hist, int64_t pos) {
    return *reinterpret_cast<const int4 *>(hist + pos);
}

template <int PF>
__global__ void __launch_bounds__(kThreads)
lookup_scan_kernel(const int32_t *__restrict__ hist, const int64_t *__restrict__ row_off,
                   const int32_t *__restrict__ len, int32_t cpr, ScanArgs a,
                   WsSlot *__restrict__ ws, int32_t *__restrict__ match_len,
                   int32_t *__restrict__ match_end, int32_t *__restrict__ draft)
{
    __shared__ u64 s_wkey[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    // workgroup = (request r, chunk c); cpr chunks per request
    const int r = blockIdx.x / cpr;
    const int c0 = blockIdx.x - r * cpr;
    const int64_t ro = row_off[r];
    const int64_t n = len[r] > 0 ? len[r] : 0;

    if (n == 0) {                       // empty row: no match, chunk 0 writes it
        if (c0 == 0 && tid < LCD_DRAFT_STRIDE) {
            draft[(int64_t)r * LCD_DRAFT_STRIDE + tid] = LCD_PAD;
            if (tid == 0) {
                match_len[r] = 0;
                match_end[r] = -1;
            }
        }
        return;
    }
    // Equal chunks of whole tiles (at most 2^30 tokens, so positions inside a
    // chunk fit in 32 bits); a row with more chunks than the grid provides is
    // covered by letting each workgroup take every cpr-th chunk.
    int64_t T = (n + cpr - 1) / cpr;
    T = ((T + kTileTok - 1) / kTileTok) * kTileTok;
    if (T > (int64_t(1) << 30)) T = int64_t(1) << 30;
    const int contrib = (int)((n + T - 1) / T);
    const int J = a.l_max;

    for (int ch = c0; ch < contrib; ch += cpr) {
        const int64_t seg_a = (int64_t)ch * T;
        const int64_t seg_b = (seg_a + T < n) ? seg_a + T : n;

        // Candidate ends of this segment, as positions relative to X0 (the
        // 16-byte granule holding the first one); this wave's tiles.
        const int64_t cand_lo = ro + seg_a;
        const int64_t X0 = cand_lo & ~(int64_t)3;
        const int32_t *__restrict__ hb = hist + X0;                        // uniform base
        const int c_lo = (int)(cand_lo - X0);                              // 0..3
        const int c_hi = (int)(ro + (seg_b < n - 1 ? seg_b : n - 1) - X0); // exclusive
        const int r_lo = (ro - X0 < -(1 << 30)) ? -(1 << 30) : (int)(ro - X0);   // row start
        const int nt = c_hi > c_lo ? (c_hi + kTileTok - 1) / kTileTok : 0;
        const int tpw = (nt + kWaves - 1) / kWaves;
        const int k0 = uni(tpw * wave);
        const int k1 = uni(min(k0 + tpw, nt));
        const int g_last = (c_hi - 1) & ~3;        // last granule with a candidate
        const int g_first = r_lo & ~3;             // first granule of the row (if >= X0-16)

        // suffix s_j = h[n-1-j] through the scalar cache (filler 0 past the row)
        int s16[LCD_MAX_SUFFIX];
        if (n >= LCD_MAX_SUFFIX) {
            const int32_t *__restrict__ sp = hist + (ro + n - LCD_MAX_SUFFIX);
#pragma unroll
            for (int j = 0; j < LCD_MAX_SUFFIX; ++j) s16[j] = sp[LCD_MAX_SUFFIX - 1 - j];
        } else {
#pragma unroll
            for (int j = 0; j < LCD_MAX_SUFFIX; ++j) s16[j] = (j < n) ? hist[ro + n - 1 - j] : 0;
        }
        // Loads never leave the row: lanes whose granule lies past the last
        // candidate re-read the last candidate's granule, halo lanes whose
        // granule lies before the row re-read the row's first granule.
        auto load_tile = [&](int kt) -> int4 {
            const int off = min(kTileTok * kt + 4 * lane, g_last);
            return load_granule(hb, off);
        };
        auto load_halo = [&](int kt) -> int4 {   // 16 tokens before tile kt, lanes 60..63
            const int off = max(kTileTok * kt - kTileTok + 4 * max(lane, 60), g_first);
            return load_granule(hb, off);
        };
        // every wave issues the halo and a full batch, even past its last tile
        // (re-reading a tile it owns, or the segment's last one), so the loads
        // are unconditional and can be waited for one at a time
        const int kl = (k1 > k0) ? k1 - 1 : nt - 1;
        int4 buf[kUnroll];
        int4 halo = make_int4(0, 0, 0, 0);
        auto load_batch = [&](int kb) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) buf[u] = load_tile(min(kb + u, kl));
        };
        if (nt > 0) {                      // uniform over the workgroup
            halo = load_halo(min(k0, kl));
            load_batch(min(k0, kl));
        }

        int s4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) s4[j] = s16[j];
        // a value equal to no suffix token stands in for tokens before the row
        int sent = s16[0] + 1;
        for (int it = 0; it <= LCD_MAX_SUFFIX; ++it) {
            bool hit = false;
#pragma unroll
            for (int j = 0; j < LCD_MAX_SUFFIX; ++j) hit |= (s16[j] == sent);
            if (!hit) break;
            ++sent;
        }
        // tokens at positions before the row start become `sent`
        auto fix_tile = [&](int4 t, int kt) -> int4 {
            const int A = kTileTok * kt;
            return (A < r_lo) ? mask_before(t, r_lo - A - 4 * lane, sent) : t;
        };
        auto fix_halo = [&](int4 t, int kt) -> int4 {
            const int A = kTileTok * kt - kTileTok;
            return (A < r_lo) ? mask_before(t, r_lo - A - 4 * lane, sent) : t;
        };
        // prefilter survivors of tile kt (tokens t), given the shifted masks of
        // the tile before it; also returns this tile's shifted masks
        auto survivors = [&](const int4 &t, int kt, const u64 (&psh)[4], u64 (&P)[4], u64 (&sh)[4]) {
            u64 in[4];
            prefilter_masks<PF>(t, s4, in, sh);
#pragma unroll
            for (int c = 0; c < 4; ++c) P[c] = in[c] & ((sh[c] << 1) | (psh[c] >> 63));
            const int A = kTileTok * kt;
            if (A < c_lo || A + kTileTok > c_hi) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int x = A + 4 * lane + c;
                    P[c] &= ballot(x >= c_lo && x < c_hi);
                }
            }
        };

        u64 best = 0;
        if (k0 < k1) {
            u64 psh[4];
            {
                u64 pin[4];
                prefilter_masks<PF>(fix_halo(halo, k0), s4, pin, psh);
            }
            for (int kb = k0; kb < k1; kb += kUnroll) {
                if (kb != k0) load_batch(kb);
                // hot loop: the 4-token test only; tiles with a survivor are
                // marked and revisited below
                unsigned surv = 0;
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    if (kb + u < k1) {
                        u64 P[4], sh[4];
                        survivors(fix_tile(buf[u], kb + u), kb + u, psh, P, sh);
                        if ((P[0] | P[1] | P[2] | P[3]) != 0) surv |= 1u << u;
#pragma unroll
                        for (int c = 0; c < 4; ++c) psh[c] = sh[c];
                    }
                }
                // rare path: reload a marked tile and the 16 tokens before it
                // (both still in cache), redo its test and extend survivors
                while (surv != 0) {
                    const int kt = kb + __builtin_ctz(surv);
                    surv &= surv - 1;
                    const int4 t = fix_tile(load_tile(kt), kt);
                    const int4 pt = fix_halo(load_halo(kt), kt);
                    u64 pin[4], ppsh[4], P[4], sh[4];
                    prefilter_masks<PF>(pt, s4, pin, ppsh);
                    survivors(t, kt, ppsh, P, sh);
                    const int L = extend<PF>(t, pt, s16, J, P);
                    if (L >= a.l_min) {
                        int ebest = -1;
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            if (P[c] != 0) {
                                const int e = 4 * (63 - __clzll(P[c])) + c;
                                ebest = e > ebest ? e : ebest;
                            }
                        }
                        const int64_t e_abs = X0 + kTileTok * (int64_t)kt + ebest;
                        const u64 key = ((u64)L << 32) | (u64)(uint32_t)(e_abs - ro);
                        best = key > best ? key : best;
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
                // Merge across the workgroups covering this request.  Both words
                // are only touched by device-scope atomic read-modify-writes,
                // which the memory system performs at one coherence point per
                // address.  Waiting for this workgroup's max to return before
                // counting it means every max is performed before the final
                // count is, and the last arriver reads the key only after that.
                WsSlot *slot = ws + r;
                if (key) __hip_atomic_fetch_max(&slot->key, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_s_waitcnt(0);
                const unsigned old = __hip_atomic_fetch_add(&slot->count, 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
                last = (old == (unsigned)(contrib - 1));
                if (last) {
                    key = __hip_atomic_exchange(&slot->key, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Chunks per request.  The launch has B*cpr workgroups; by default about
// 1024 of them (4 per CU) with at least 2048 tokens per chunk.
int pick_cpr(int32_t B, int32_t max_len, int32_t scan_wgs) {
    int64_t cpr;
    if (scan_wgs > 0) {
        cpr = scan_wgs / B;
    } else {
        cpr = 1024 / B;
        const int64_t by_len = ((int64_t)max_len + 2047) / 2048;
        if (cpr > by_len) cpr = by_len;
    }
    if (cpr < 1) cpr = 1;
    const int64_t cap = (int64_t(1) << 31) / ((int64_t)B > 0 ? B : 1) - 1;
    if (cpr > cap) cpr = cap;
    return (int)cpr;
}

template <int PF>
hipError_t launch(const int32_t *hist, const int64_t *row_off, const int32_t *len, int32_t B,
                  int cpr, ScanArgs sa, WsSlot *ws, int32_t *ml, int32_t *me, int32_t *dr,
                  hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    const dim3 grid((unsigned)((int64_t)B * cpr));
    if (ev0 != nullptr || ev1 != nullptr)
        hipExtLaunchKernelGGL(lookup_scan_kernel<PF>, grid, dim3(kThreads), 0u, st, ev0, ev1, 0u,
                              hist, row_off, len, cpr, sa, ws, ml, me, dr);
    else
        hipLaunchKernelGGL(lookup_scan_kernel<PF>, grid, dim3(kThreads), 0, st,
                           hist, row_off, len, cpr, sa, ws, ml, me, dr);
    return hipGetLastError();
}

int propose(const int32_t *hist, const int64_t *row_off, const int32_t *len, int32_t B,
            int32_t max_len, const lcd_params *p, void *workspace, int32_t *match_len,
            int32_t *match_end, int32_t *draft, void *stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (B < 0 || p == nullptr || max_len < 0) return LCD_EINVAL;
    if (lcd_check_params(p) != LCD_OK) return LCD_EINVAL;
    if (B == 0) return LCD_OK;
    if (!hist || !row_off || !len || !workspace || !match_len || !match_end || !draft)
        return LCD_EINVAL;
    if (((uintptr_t)hist & 15u) != 0 || ((uintptr_t)workspace & 15u) != 0) return LCD_EINVAL;

    ScanArgs sa{p->l_min, p->l_max, p->k_max};
    const int pf = p->l_min < 4 ? p->l_min : 4;
    const int cpr = pick_cpr(B, max_len, p->scan_wgs);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    WsSlot *ws = reinterpret_cast<WsSlot *>(workspace);
    hipError_t err;
    switch (pf) {
    case 1: err = launch<1>(hist, row_off, len, B, cpr, sa, ws, match_len, match_end, draft, st, ev0, ev1); break;
    case 2: err = launch<2>(hist, row_off, len, B, cpr, sa, ws, match_len, match_end, draft, st, ev0, ev1); break;
    case 3: err = launch<3>(hist, row_off, len, B, cpr, sa, ws, match_len, match_end, draft, st, ev0, ev1); break;
    default: err = launch<4>(hist, row_off, len, B, cpr, sa, ws, match_len, match_end, draft, st, ev0, ev1); break;
    }
    return err == hipSuccess ? LCD_OK : LCD_EHIP;
}

}  // namespace
}  // namespace lcd

extern "C" size_t lcd_workspace_bytes(int32_t B) {
    return B > 0 ? (size_t)B * sizeof(lcd::WsSlot) : 0;
}

extern "C" int lookup_propose(const int32_t *hist, const int64_t *row_off, const int32_t *len,
                              int32_t B, int32_t max_len, const lcd_params *p, void *workspace,
                              int32_t *match_len, int32_t *match_end, int32_t *draft, void *stream) {
    return lcd::propose(hist, row_off, len, B, max_len, p, workspace, match_len, match_end, draft,
                        stream, nullptr, nullptr);
}

extern "C" int lookup_propose_timed(const int32_t *hist, const int64_t *row_off,
                                    const int32_t *len, int32_t B, int32_t max_len,
                                    const lcd_params *p, void *workspace, int32_t *match_len,
                                    int32_t *match_end, int32_t *draft, void *stream,
                                    void *ev_start, void *ev_stop) {
    return lcd::propose(hist, row_off, len, B, max_len, p, workspace, match_len, match_end, draft,
                        stream, reinterpret_cast<hipEvent_t>(ev_start),
                        reinterpret_cast<hipEvent_t>(ev_stop));
}

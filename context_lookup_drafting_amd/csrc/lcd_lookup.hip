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
#include "lcd_rules.h"

namespace lcd {
namespace {

#ifndef LCD_WAVES
#define LCD_WAVES 4
#endif
constexpr int kWaves = LCD_WAVES;
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

// Chunk length of a row of n > 0 tokens cut into cpr chunks: whole tiles, at
// most 2^30 tokens (positions inside a chunk then fit in 32 bits).
__device__ __forceinline__ int64_t chunk_tokens(int64_t n, int cpr) {
    int64_t T = (n + cpr - 1) / cpr;
    T = ((T + kTileTok - 1) / kTileTok) * kTileTok;
    return T > (int64_t(1) << 30) ? (int64_t(1) << 30) : T;
}

// kPartials = false: workgroups of a request merge their keys through the
// workspace (atomic max + arrival count) and the last one writes the result.
// kPartials = true: each workgroup stores its key in part[r*cpr + c] and a
// following kernel finishes the step.
template <int PF, bool kPartials>
__global__ void __launch_bounds__(kThreads)
lookup_scan_kernel(const int32_t *__restrict__ hist, const int64_t *__restrict__ row_off,
                   const int32_t *__restrict__ len, int32_t cpr, ScanArgs a,
                   WsSlot *__restrict__ ws, u64 *__restrict__ part, int32_t *__restrict__ match_len,
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
        if (!kPartials && c0 == 0 && tid < LCD_DRAFT_STRIDE) {
            draft[(int64_t)r * LCD_DRAFT_STRIDE + tid] = LCD_PAD;
            if (tid == 0) {
                match_len[r] = 0;
                match_end[r] = -1;
            }
        }
        return;
    }
    // Equal chunks of whole tiles; a row with more chunks than the grid
    // provides is covered by letting each workgroup take every cpr-th chunk.
    const int64_t T = chunk_tokens(n, cpr);
    const int contrib = (int)((n + T - 1) / T);
    if (c0 >= contrib) return;
    const int J = a.l_max;
    u64 wg_key = 0;                     // kPartials: best key over this workgroup's chunks

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
            // Quick test: a candidate end e needs h[e-jq] == s_jq for every
            // jq < PF, so a tile can hold one only if some position in it, or
            // in the previous tile's last lane, holds s_jq.  Each wave uses the
            // suffix token that is rarest in its first tile; the choice only
            // changes how many tiles get the full test, never the result.
            int jq = 0;
            {
                const int4 t = fix_tile(buf[0], k0);
                int fewest = 1 << 30;
#pragma unroll
                for (int j = 0; j < PF; ++j) {
                    const int cnt = __popcll(ballot(t.x == s4[j])) + __popcll(ballot(t.y == s4[j])) +
                                    __popcll(ballot(t.z == s4[j])) + __popcll(ballot(t.w == s4[j]));
                    if (cnt < fewest) { fewest = cnt; jq = j; }
                }
            }
            const int sq = uni(jq == 0 ? s4[0] : jq == 1 ? s4[1] : jq == 2 ? s4[2] : s4[3]);
            auto quick = [&](const int4 &t) -> u64 {
                return ballot(t.x == sq) | ballot(t.y == sq) | ballot(t.z == sq) | ballot(t.w == sq);
            };
            int4 prev = fix_halo(halo, k0);          // tile before the next one processed
            u64 carry = quick(prev) >> 63;           // a hit in its last lane
            for (int kb = k0; kb < k1; kb += kUnroll) {
                if (kb != k0) load_batch(kb);
                // hot loop: quick test on every tile; flagged tiles get the
                // full 4-token test from registers; tiles with a survivor of
                // that are marked and extended below
                unsigned surv = 0;
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    if (kb + u < k1) {
                        const int4 t = fix_tile(buf[u], kb + u);
                        const u64 q = quick(t);
                        if ((q | carry) != 0) {
                            const int4 pt = (u == 0) ? prev : fix_tile(buf[u > 0 ? u - 1 : 0], kb + u - 1);
                            u64 pin[4], psh[4], P[4], sh[4];
                            prefilter_masks<PF>(pt, s4, pin, psh);
                            survivors(t, kb + u, psh, P, sh);
                            if ((P[0] | P[1] | P[2] | P[3]) != 0) surv |= 1u << u;
                        }
                        carry = q >> 63;
                    }
                }
                prev = fix_tile(buf[kUnroll - 1], kb + kUnroll - 1);
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
            if (kPartials) {
                wg_key = key > wg_key ? key : wg_key;
            } else {
                bool last = true;
                if (contrib > 1) {
                    // Merge across the workgroups covering this request.  Both
                    // words are only touched by device-scope atomic
                    // read-modify-writes, which the memory system performs at
                    // one coherence point per address.  Waiting for this
                    // workgroup's max to return before counting it means every
                    // max is performed before the final count is, and the last
                    // arriver reads the key only after that.
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
                    const int m = (int)(key >> 32);
                    const int64_t e = key ? (int64_t)(uint32_t)key : -1;
                    int d[LCD_DRAFT_STRIDE];
                    lz_draft(hist + ro, n, m, e, a.k_max, d);
                    match_len[r] = m;
                    match_end[r] = (int32_t)e;
#pragma unroll
                    for (int k = 0; k < LCD_DRAFT_STRIDE; ++k) draft[(int64_t)r * LCD_DRAFT_STRIDE + k] = d[k];
                }
            }
        }
        __syncthreads();
    }
    if (kPartials && tid == 0) part[(int64_t)r * cpr + c0] = wg_key;
}

// Second kernel of the fused decode step: one lane per request reduces the
// chunk keys, copies the draft, fuses the verify block, accepts greedily
// (optionally appending the emitted tokens) and advances the scheduler.
struct PostArgs {
    int32_t k_max, append;
    FuseArgs f;
    SchedArgs s;
};

__global__ void __launch_bounds__(256)
decode_post_kernel(int32_t *hist, const int64_t *__restrict__ row_off, int32_t *__restrict__ len,
                   const int32_t *__restrict__ cap, int32_t B, int32_t cpr,
                   const u64 *__restrict__ part, const int32_t *__restrict__ q,
                   const int32_t *__restrict__ target, lcd_sched_state *__restrict__ state,
                   PostArgs pa, int32_t *__restrict__ match_len, int32_t *__restrict__ match_end,
                   int32_t *__restrict__ draft, int32_t *__restrict__ block,
                   int32_t *__restrict__ block_len, int32_t *__restrict__ accept,
                   int32_t *__restrict__ long_next) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= B) return;
    const int64_t ro = row_off[r];
    const int64_t n = len[r] > 0 ? len[r] : 0;
    u64 key = 0;
    if (n > 0) {
        const int64_t T = chunk_tokens(n, cpr);
        const int64_t contrib = (n + T - 1) / T;
        const int cw = (int)(contrib < cpr ? contrib : cpr);
        for (int c = 0; c < cw; ++c) {
            const u64 k = part[(int64_t)r * cpr + c];
            key = k > key ? k : key;
        }
    }
    const int m = (int)(key >> 32);
    const int64_t e = key ? (int64_t)(uint32_t)key : -1;
    int d[LCD_DRAFT_STRIDE];
    lz_draft(hist + ro, n, m, e, pa.k_max, d);
    match_len[r] = m;
    match_end[r] = (int32_t)e;
#pragma unroll
    for (int k = 0; k < LCD_DRAFT_STRIDE; ++k) draft[(int64_t)r * LCD_DRAFT_STRIDE + k] = d[k];

    int qv[LCD_Q_STRIDE], tv[LCD_TARGET_STRIDE], bv[LCD_DRAFT_STRIDE];
#pragma unroll
    for (int i = 0; i < LCD_Q_STRIDE; ++i) qv[i] = q[(int64_t)r * LCD_Q_STRIDE + i];
#pragma unroll
    for (int i = 0; i < LCD_TARGET_STRIDE; ++i) tv[i] = target[(int64_t)r * LCD_TARGET_STRIDE + i];
    lcd_sched_state st = state[r];
    const int blk = fuse_row(d, m, qv, st.long_mode != 0, pa.f, bv);
#pragma unroll
    for (int k = 0; k < LCD_DRAFT_STRIDE; ++k) block[(int64_t)r * LCD_DRAFT_STRIDE + k] = bv[k];
    block_len[r] = blk;
    int acc = accept_row(bv, blk, tv);
    if (pa.append) acc = append_row(acc, tv, hist, ro, len + r, cap[r]);
    accept[r] = acc;
    const int ln = schedule_row(st, m, acc, blk, pa.s);
    state[r] = st;
    if (long_next) long_next[r] = ln;
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

template <int PF, bool kPartials>
hipError_t launch(const int32_t *hist, const int64_t *row_off, const int32_t *len, int32_t B,
                  int cpr, ScanArgs sa, WsSlot *ws, u64 *part, int32_t *ml, int32_t *me, int32_t *dr,
                  hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    const dim3 grid((unsigned)((int64_t)B * cpr));
    if (ev0 != nullptr || ev1 != nullptr)
        hipExtLaunchKernelGGL(lookup_scan_kernel<PF, kPartials>, grid, dim3(kThreads), 0u, st, ev0, ev1,
                              0u, hist, row_off, len, cpr, sa, ws, part, ml, me, dr);
    else
        hipLaunchKernelGGL((lookup_scan_kernel<PF, kPartials>), grid, dim3(kThreads), 0, st,
                           hist, row_off, len, cpr, sa, ws, part, ml, me, dr);
    return hipGetLastError();
}

template <bool kPartials>
hipError_t launch_scan(int pf, const int32_t *hist, const int64_t *row_off, const int32_t *len,
                       int32_t B, int cpr, ScanArgs sa, WsSlot *ws, u64 *part, int32_t *ml,
                       int32_t *me, int32_t *dr, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    switch (pf) {
    case 1: return launch<1, kPartials>(hist, row_off, len, B, cpr, sa, ws, part, ml, me, dr, st, ev0, ev1);
    case 2: return launch<2, kPartials>(hist, row_off, len, B, cpr, sa, ws, part, ml, me, dr, st, ev0, ev1);
    case 3: return launch<3, kPartials>(hist, row_off, len, B, cpr, sa, ws, part, ml, me, dr, st, ev0, ev1);
    default: return launch<4, kPartials>(hist, row_off, len, B, cpr, sa, ws, part, ml, me, dr, st, ev0, ev1);
    }
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
    const hipError_t err = launch_scan<false>(pf, hist, row_off, len, B, cpr, sa, ws, nullptr,
                                              match_len, match_end, draft, st, ev0, ev1);
    return err == hipSuccess ? LCD_OK : LCD_EHIP;
}

size_t decode_workspace_bytes(int32_t B, int32_t max_len, const lcd_params *p) {
    if (B <= 0 || p == nullptr) return 0;
    return (size_t)B * (size_t)pick_cpr(B, max_len, p->scan_wgs) * sizeof(u64);
}

int decode_step(int32_t *hist, const int64_t *row_off, int32_t *len, const int32_t *cap, int32_t B,
                int32_t max_len, const int32_t *model_draft, const int32_t *target,
                lcd_sched_state *state, const lcd_params *p, void *workspace, size_t ws_bytes,
                int32_t *match_len, int32_t *match_end, int32_t *draft, int32_t *block,
                int32_t *block_len, int32_t *accept, int32_t *long_next, int32_t append,
                void *stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (B < 0 || p == nullptr || max_len < 0) return LCD_EINVAL;
    if (lcd_check_params(p) != LCD_OK) return LCD_EINVAL;
    if (B == 0) return LCD_OK;
    if (!hist || !row_off || !len || !model_draft || !target || !state || !workspace ||
        !match_len || !match_end || !draft || !block || !block_len || !accept)
        return LCD_EINVAL;
    if (append && !cap) return LCD_EINVAL;
    if (((uintptr_t)hist & 15u) != 0 || ((uintptr_t)workspace & 15u) != 0) return LCD_EINVAL;
    if (ws_bytes < decode_workspace_bytes(B, max_len, p)) return LCD_EINVAL;

    ScanArgs sa{p->l_min, p->l_max, p->k_max};
    const int pf = p->l_min < 4 ? p->l_min : 4;
    const int cpr = pick_cpr(B, max_len, p->scan_wgs);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    u64 *part = reinterpret_cast<u64 *>(workspace);
    hipError_t err = launch_scan<true>(pf, hist, row_off, len, B, cpr, sa, nullptr, part, nullptr,
                                       nullptr, nullptr, st, ev0, ev1);
    if (err != hipSuccess) return LCD_EHIP;
    PostArgs pa{p->k_max, append ? 1 : 0, fuse_args(p), sched_args(p)};
    hipLaunchKernelGGL(decode_post_kernel, dim3((B + 255) / 256), dim3(256), 0, st, hist, row_off,
                       len, cap, B, cpr, part, model_draft, target, state, pa, match_len, match_end,
                       draft, block, block_len, accept, long_next);
    return hipGetLastError() == hipSuccess ? LCD_OK : LCD_EHIP;
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

extern "C" size_t lcd_decode_step_workspace_bytes(int32_t B, int32_t max_len, const lcd_params *p) {
    return lcd::decode_workspace_bytes(B, max_len, p);
}

extern "C" int lookup_decode_step(int32_t *hist, const int64_t *row_off, int32_t *len,
                                  const int32_t *cap, int32_t B, int32_t max_len,
                                  const int32_t *model_draft, const int32_t *target,
                                  lcd_sched_state *state, const lcd_params *p, void *workspace,
                                  size_t workspace_bytes, int32_t *match_len, int32_t *match_end,
                                  int32_t *draft, int32_t *block, int32_t *block_len,
                                  int32_t *accept, int32_t *long_next, int32_t append,
                                  void *stream) {
    return lcd::decode_step(hist, row_off, len, cap, B, max_len, model_draft, target, state, p,
                            workspace, workspace_bytes, match_len, match_end, draft, block,
                            block_len, accept, long_next, append, stream, nullptr, nullptr);
}

extern "C" int lookup_decode_step_timed(int32_t *hist, const int64_t *row_off, int32_t *len,
                                        const int32_t *cap, int32_t B, int32_t max_len,
                                        const int32_t *model_draft, const int32_t *target,
                                        lcd_sched_state *state, const lcd_params *p,
                                        void *workspace, size_t workspace_bytes,
                                        int32_t *match_len, int32_t *match_end, int32_t *draft,
                                        int32_t *block, int32_t *block_len, int32_t *accept,
                                        int32_t *long_next, int32_t append, void *stream,
                                        void *ev_start, void *ev_stop) {
    return lcd::decode_step(hist, row_off, len, cap, B, max_len, model_draft, target, state, p,
                            workspace, workspace_bytes, match_len, match_end, draft, block,
                            block_len, accept, long_next, append, stream,
                            reinterpret_cast<hipEvent_t>(ev_start),
                            reinterpret_cast<hipEvent_t>(ev_stop));
}

// lcd_index.hip -- the lookup answered from an incrementally maintained n-gram
// index instead of a scan of the whole history, for MI355X / gfx950.
//
// Method: HyperQwen lookup-drafting article, section "第 1 步" (longest current
// suffix of 4..12 tokens, latest earlier occurrence, LZ-style draft); the
// forum thread's reply on the method's pitfalls (the lookup index has to be
// maintained incrementally: a full scan of a long context at every step costs
// more and more).  The answer is the same as the scan's, bit for bit.
//
// The index of request r is one open-addressed hash table of 8-byte entries
// keyed by (L, the L tokens ending at position p) for every L in
// [l_min, l_max]; the entry holds the largest such p.  A position is inserted
// only once the token after it exists (p <= n-2 for a history of n tokens), so
// the latest earlier occurrence of the current suffix's L-gram is the entry's
// position itself, and "longest, then latest" is: the largest L whose suffix
// L-gram has an entry.  Every hit is checked against the history's tokens; an
// entry shared by two different L-grams with the same fingerprint (a
// fingerprint collision, about 2^-31 per probe) can hide the answer, so such a
// request is answered by an exact scan of its history instead.
//
// Entry layout: fingerprint (high 32 bits, never 0) | position + 1 (low 32);
// 0 = empty.  Inserting is a compare-and-swap into an empty slot, or a 64-bit
// atomic max into the slot holding the same fingerprint (same high word, so
// the max is the larger position); linear probing past other fingerprints.
// A key's home slot is a multiply-shift of its low word onto the table's
// exact size (no power-of-two rounding); the plan sizes each table from the
// row's capacity and lcd_params.index_load (slots per indexed length and
// token, default 3: at most 1/3 of the slots ever taken).
//
// lookup_index_propose: one workgroup of two waves per request.  Wave 1
// inserts the positions appended since the last call (lanes over positions,
// every length's compare-and-swap in flight at once, collisions probed in
// rounds).  Wave 0 matches those positions against the suffix directly and
// queries the table for all lengths at once (lane k takes L = l_min + k),
// verifying the hits; the answer is the better of the two.  The waves do not
// wait for each other's memory traffic, so a step costs the longer of the two
// chains of dependent round trips (about five), whatever the history length.
//
// lookup_index_decode_step: the same kernel, whose wave then also does the
// rest of the decode step for its request (fusion, greedy acceptance with the
// append, scheduler, telemetry; lcd_finish.h), so a decode step through the
// index is one launch.  The step inputs are loaded when the wave starts.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lcd.h"
#include "lcd_finish.h"

namespace lcd {
namespace {

using u64 = unsigned long long;

constexpr int kBuildThreads = 256;
constexpr int kMaxL = LCD_MAX_SUFFIX;            // 16
constexpr int kMaxProbe = 1 << 20;               // bound on a probe sequence

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Rolling hash of the tokens t_p, t_{p-1}, ... (read backwards from the end
// position), then the SplitMix64 finaliser (Steele, Lea & Flood, "Fast
// Splittable Pseudorandom Number Generators", OOPSLA 2014: its two
// xor-shift-multiply rounds and constants), keyed by the length.
__device__ __forceinline__ u64 roll(u64 h, int32_t t) {
    h = (h ^ (uint32_t)t) * 0x9E3779B97F4A7C15ull;
    return h ^ (h >> 32);
}

__device__ __forceinline__ u64 finish_key(u64 h, int L) {
    u64 z = h + (u64)L * 0xD6E8FEB86659FD93ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

constexpr u64 kHashSeed = 0x243F6A8885A308D3ull;

struct IndexArgs {
    int32_t l_min, l_max, k_max;
    uint32_t fp_mask;        // fingerprint bits
};

__device__ __forceinline__ uint32_t fingerprint(u64 key, uint32_t mask) {
    return 1u + ((uint32_t)(key >> 33) & mask);
}

__device__ __forceinline__ u64 entry_of(u64 key, uint32_t mask, int32_t p) {
    return ((u64)fingerprint(key, mask) << 32) | (uint32_t)(p + 1);
}

// A key's home slot in a table of ns slots, and the slot after slot i.
__device__ __forceinline__ u64 home_slot(u64 key, uint32_t ns) { return ((u64)(uint32_t)key * ns) >> 32; }
__device__ __forceinline__ u64 next_slot(u64 i, uint32_t ns) { return i + 1 < ns ? i + 1 : 0; }

// Inserts entry `ent` (key's fingerprint | p + 1) into table T of ns slots,
// probing from slot i; returns false only if the probe bound was hit (never at
// the planned load).
__device__ bool insert_from(u64 *__restrict__ T, uint32_t ns, u64 ent, u64 i) {
    const u64 fp = ent >> 32;
    for (int probes = 0; probes < kMaxProbe; ++probes) {
        const u64 old = atomicCAS(T + i, 0ull, ent);
        if (old == 0) return true;
        if ((old >> 32) == fp) {
            atomicMax(T + i, ent);
            return true;
        }
        i = next_slot(i, ns);
    }
    return false;
}

__device__ __forceinline__ bool insert_one(u64 *__restrict__ T, uint32_t ns, u64 key, uint32_t mask,
                                           int32_t p) {
    return insert_from(T, ns, entry_of(key, mask, p), home_slot(key, ns));
}

// Exact lookup by scanning the whole history (the slow path): one wave, one
// candidate end per lane per step, the longest match (capped at l_max) and the
// latest end among equals.  Returns the packed key (L << 31 | e), 0 = none.
__device__ u64 exact_scan(const int32_t *__restrict__ h, int n, const IndexArgs &a, int lane) {
    // suffix token s_j = h[n-1-j] for j < l_max, read by every lane
    u64 best = 0;
    for (int e0 = 0; e0 <= n - 2; e0 += 64) {
        const int e = e0 + lane;
        int L = 0;
        if (e <= n - 2) {
            while (L < a.l_max && L <= e && h[e - L] == h[n - 1 - L]) ++L;
        }
        if (L >= a.l_min) {
            const u64 k = ((u64)L << 31) | (uint32_t)e;
            best = k > best ? k : best;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const u64 o = __shfl_xor(best, off);
        best = o > best ? o : best;
    }
    return best;
}

// Slots read per round trip: by an insert (kWin) and by a query (kQWin).
// Linear probing keeps a key's run of slots together, so one window of
// neighbouring slots answers what a probe sequence would ask one slot at a
// time (the tables hold at least 16 slots, so a window never wraps twice).
constexpr int kWin = 8;
constexpr int kQWin = 4;
// Each request's last tokens as the previous call left them, in the first
// kCacheWords words of the tables buffer per request (the plan puts the
// tables after them): word 0 is kCacheTag << 32 | the row length they end
// at, words 1.. hold kCacheTok tokens, the last first.  A call whose row
// length equals the cached one takes its suffix (and the tokens of the
// positions appended since) from there, in the same round trip as the row's
// length, instead of reading them from the history after it.
constexpr int kCacheWords = 32;
constexpr int kCacheTok = 48;
constexpr uint32_t kCacheTag = 0x4C434443u;
constexpr int kLanePairs = 4;          // queued entries one lane probes at once
constexpr int kQueue = 64 * kMaxL;     // (position, length) entries per 64 positions

__device__ __forceinline__ uint32_t wrap_add(uint32_t i, uint32_t k, uint32_t ns) {
    const uint32_t j = i + k;          // i < ns <= INT32_MAX and k <= 16 <= ns
    return j >= ns ? j - ns : j;
}

__device__ __forceinline__ int wave_exclusive_sum(int x, int lane) {
    int incl = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d);
        incl += lane >= d ? y : 0;
    }
    return incl - x;
}

__device__ __forceinline__ void lds_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Enters the queued entries b.. (up to kLanePairs per lane, all probed at
// once).  A round reads a window of kWin slots from each entry's next slot,
// takes the first that is empty or holds the entry's fingerprint, and
// compare-and-swaps it (empty) or atomically maxes it (same fingerprint).  A
// compare-and-swap lost to another lane of the wave goes on past that slot.
// The maxes need no answer and are issued after the round's results are read
// (a read behind one would wait for it).  Returns false if the probe bound
// was hit.
__device__ bool probe_batch(u64 *__restrict__ T, uint32_t ns, const u64 *q_ent,
                            const uint32_t *q_slot, int b, int total, int lane) {
    u64 ent[kLanePairs];
    uint32_t st[kLanePairs], at[kLanePairs];
    uint32_t act = 0;
#pragma unroll
    for (int c = 0; c < kLanePairs; ++c) {
        const int q = b + lane + 64 * c;
        ent[c] = q < total ? q_ent[q] : 0ull;
        st[c] = q < total ? q_slot[q] : 0u;
        at[c] = 0;
        act |= q < total ? 1u << c : 0u;
    }
    bool ok = true;
    for (int probed = 0; __ballot(act != 0) != 0; probed += kWin) {
        if (probed >= kMaxProbe) {
            ok = act == 0;
            break;
        }
        u64 win[kLanePairs][kWin];
#pragma unroll
        for (int c = 0; c < kLanePairs; ++c)
#pragma unroll
            for (int w = 0; w < kWin; ++w)
                win[c][w] = (act >> c) & 1u
                                ? __hip_atomic_load(T + wrap_add(st[c], w, ns), __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_WORKGROUP)
                                : 0ull;
        uint32_t cas = 0, mx = 0;
#pragma unroll
        for (int c = 0; c < kLanePairs; ++c) {
            if (!((act >> c) & 1u)) continue;
            const uint32_t fp = (uint32_t)(ent[c] >> 32);
            int hw = -1;
            bool same = false;
#pragma unroll
            for (int w = kWin - 1; w >= 0; --w) {
                const bool stop = win[c][w] == 0 || (uint32_t)(win[c][w] >> 32) == fp;
                hw = stop ? w : hw;
                same = stop ? win[c][w] != 0 : same;
            }
            if (hw < 0) {
                st[c] = wrap_add(st[c], kWin, ns);            // the whole window taken
            } else {
                at[c] = wrap_add(st[c], (uint32_t)hw, ns);
                if (same) mx |= 1u << c; else cas |= 1u << c;
            }
        }
        u64 old[kLanePairs];
#pragma unroll
        for (int c = 0; c < kLanePairs; ++c)
            old[c] = (cas >> c) & 1u ? atomicCAS(T + at[c], 0ull, ent[c]) : 0ull;
#pragma unroll
        for (int c = 0; c < kLanePairs; ++c) {
            if (!((cas >> c) & 1u)) continue;
            if (old[c] == 0) {
                act &= ~(1u << c);
            } else if ((uint32_t)(old[c] >> 32) == (uint32_t)(ent[c] >> 32)) {
                mx |= 1u << c;
            } else {
                st[c] = wrap_add(at[c], 1, ns);               // taken meanwhile: go on past it
            }
        }
#pragma unroll
        for (int c = 0; c < kLanePairs; ++c)
            if ((mx >> c) & 1u) atomicMax(T + at[c], ent[c]);
        act &= ~mx;
    }
    return ok;
}

// The inserting wave: enters the positions p_lo..p_hi (appended since the
// last call) for every indexed length.  Per 64 positions (lanes), each
// lane's (position, length) entries are queued in LDS, then probed spread
// over the lanes (probe_batch), so a position with many entries does not
// hold its lane for all of them.  Returns false if a probe bound was hit.
__device__ bool insert_positions(const int32_t *__restrict__ h, u64 *__restrict__ T, uint32_t ns,
                                 int p_lo, int p_hi, const IndexArgs &a, int lane,
                                 const int32_t (&t0)[kMaxL], u64 *q_ent, uint32_t *q_slot) {
    bool ok = true;
    for (int p0 = p_lo; p0 <= p_hi; p0 += 64) {
        const int p = p0 + lane;
        const bool ins = p <= p_hi;
        // opaque copies of the length bounds: tests against them hoisted out
        // of this loop were held (and spilled) through the whole kernel
        int lmin = a.l_min, lmax = a.l_max;
        asm volatile("" : "+s"(lmin), "+s"(lmax));
        int32_t t[kMaxL];
#pragma unroll
        for (int j = 0; j < kMaxL; ++j)
            t[j] = p0 == p_lo ? t0[j] : ((ins && j < lmax && p - j >= 0) ? h[p - j] : 0);
        uint32_t vm = 0;
#pragma unroll
        for (int j = 0; j < kMaxL; ++j) {
            const int Lj = j + 1;
            vm |= (ins && Lj >= lmin && Lj <= lmax && p - j >= 0) ? 1u << j : 0u;
        }
        const int cnt = __builtin_popcount(vm);
        const int off = wave_exclusive_sum(cnt, lane);
        const int total = __builtin_amdgcn_readlane(off + cnt, 63);
        if (p0 != p_lo) lds_wave_sync();                     // the last batch has read the queue
        u64 hs = kHashSeed;
        int k = off;
#pragma unroll
        for (int j = 0; j < kMaxL; ++j) {
            hs = roll(hs, t[j]);
            if ((vm >> j) & 1u) {
                const u64 key = finish_key(hs, j + 1);
                q_ent[k] = entry_of(key, a.fp_mask, p);
                q_slot[k] = (uint32_t)home_slot(key, ns);
                ++k;
            }
        }
        lds_wave_sync();
        for (int b = 0; b < total; b += 64 * kLanePairs)
            ok = probe_batch(T, ns, q_ent, q_slot, b, total, lane) && ok;
    }
    return __ballot(!ok) == 0;
}

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Memory scope.  Within a launch a request's table is touched only by its own
// workgroup, so the table reads of both waves are workgroup-scope loads (they
// may be served by the CU's cache): a read may miss an insert made by the
// other wave, or by another lane, earlier in the same launch, never one made
// by an earlier launch (the caches hold nothing from before the launch).  That
// is enough: a slot only ever goes from empty to a fingerprint, and then only
// to later positions; an insert that relied on a stale empty slot loses its
// compare-and-swap and goes on; and a query that stops at a stale empty slot
// misses only this launch's positions, which the direct match covers.
//
// Two waves per request (one workgroup).  Wave 1 inserts the appended
// positions and records the indexed length; wave 0 answers the lookup (the
// table query, and the direct match over the appended positions, which the
// query need not find in the table) and, with kStep, finishes the decode
// step.  Neither waits for the other's memory operations: the inserts'
// round trips run beside the query's.  Wave 0 alone reads len and
// indexed_len and hands them to wave 1 through LDS, so wave 1's write of
// indexed_len follows wave 0's read of it, and wave 0's append of the new
// length has no reader in the other wave.  A failed insert (probe bound)
// leaves this call's answer exact (the direct match covers the new
// positions) and marks the index stale for the next calls.
template <bool kStep>
__global__ void __launch_bounds__(128)
index_propose_kernel(StepIO io_arg, const int32_t *__restrict__ hist,
                     const int64_t *__restrict__ row_off, const int32_t *__restrict__ len,
                     int32_t B, IndexArgs a,
                     const int64_t *__restrict__ table_off, const int32_t *__restrict__ table_slots,
                     u64 *__restrict__ tables, int32_t *__restrict__ indexed_len,
                     int32_t *__restrict__ match_len, int32_t *__restrict__ match_end,
                     int32_t *__restrict__ draft) {
    // The step's pointers and rules are read from the kernel-argument segment
    // (io_arg is the first argument, at its start) where they are used, so
    // they are not held in scalar registers through the lookup.
    (void)io_arg;
    const StepIO *iop = (const StepIO *)__builtin_amdgcn_kernarg_segment_ptr();
    const int lane = threadIdx.x & 63;
    const bool inserter = uni(threadIdx.x >> 6) == 1;
    const int r = blockIdx.x;
    if (r >= B) return;
    // the rest of the step's inputs, in flight during the lookup
    int sin = 0;
    uint32_t tin = 0;                 // the request's telemetry row, lane k: counter k
    if (kStep && !inserter) {
        const StepIO io0 = *iop;
        sin = load_step_input(r, lane, io0);
        if (io0.tele != nullptr)
            tin = io0.tele[(int64_t)r * LCD_TELE_WORDS + (lane & (LCD_TELE_WORDS - 1))];
    }
    __shared__ int s_meta[2];
    __shared__ int s_tok[kCacheTok];
    const int64_t ro = row_off[r];
    const int32_t *__restrict__ h = hist + ro;
    u64 *__restrict__ cache = tables + (int64_t)r * kCacheWords;
    int32_t *__restrict__ ctok = reinterpret_cast<int32_t *>(cache + 1);
    // the row's last tokens, lane k < kCacheTok: h[n-1-k] (where n-1-k >= 0)
    int32_t n0 = 0, tok = 0;
    int il = 0;
    bool cached = false;
    if (!inserter) {
        const u64 head = cache[0];
        tok = lane < kCacheTok ? ctok[lane] : 0;
        n0 = len[r];
        il = indexed_len[r];
        const int nn = n0 > 0 ? n0 : 0;
        cached = (uint32_t)(head >> 32) == kCacheTag && (uint32_t)head == (uint32_t)nn;
        if (!cached) {
            const int sp = nn - 1 - (lane < kCacheTok ? lane : 0);
            tok = nn > 0 && lane < kCacheTok ? h[sp > 0 ? sp : 0] : 0;
        }
        if (lane == 0) {
            s_meta[0] = n0;
            s_meta[1] = il;
        }
        if (lane < kCacheTok) s_tok[lane] = tok;
    }
    lds_barrier();
    if (inserter) {
        n0 = s_meta[0];
        il = s_meta[1];
        tok = lane < kCacheTok ? s_tok[lane] : 0;
    }
    const int n = n0 > 0 ? n0 : 0;
    const bool stale = il < 0 || il > n;     // answered by a scan from now on
    const int p_lo = il > 0 ? il - 1 : 0;    // positions appended since the last call
    const int p_hi = n - 2;

    // tokens ending at the first 64 appended positions (lane k: p_lo + k), for
    // the inserts (wave 1) or the direct match (wave 0): h[p-j] is the token
    // (n-1-p)+j from the end, among the last tokens when p_lo >= n-33
    int32_t t[kMaxL];
    {
        const int p = p_lo + lane;
        const bool ins = !stale && p <= p_hi;
        if (p_lo >= n - (kCacheTok - kMaxL + 1)) {
#pragma unroll
            for (int j = 0; j < kMaxL; ++j) {
                const int v = __shfl(tok, (n - 1 - p + j) & 63);
                t[j] = (ins && j < a.l_max && p - j >= 0) ? v : 0;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kMaxL; ++j) t[j] = (ins && j < a.l_max && p - j >= 0) ? h[p - j] : 0;
        }
    }

    if (inserter) {
        const uint32_t ns = (uint32_t)table_slots[r];
        u64 *__restrict__ T = tables + table_off[r];
        if (stale) {
            if (lane == 0 && il > n) indexed_len[r] = -1;
            return;
        }
        __shared__ u64 q_ent[kQueue];
        __shared__ uint32_t q_slot[kQueue];
        const bool ok = insert_positions(h, T, ns, p_lo, p_hi, a, lane, t, q_ent, q_slot);
        if (lane == 0) indexed_len[r] = ok ? n : -1;
        return;
    }

    const int nL = a.l_max - a.l_min + 1;
    bool exact = stale;
    u64 key = 0;
    // The suffix s_j = h[n-1-j] is in lane j of tok; every lane reads them all.
    const int32_t sv = tok;
    if (!exact) {
        const uint32_t ns = (uint32_t)table_slots[r];
        const u64 *__restrict__ T = tables + table_off[r];
        int32_t s[kMaxL];
#pragma unroll
        for (int j = 0; j < kMaxL; ++j)
            s[j] = (j < a.l_max && n - 1 - j >= 0) ? __builtin_amdgcn_readlane(sv, j) : 0;

        // the query's key for length L = l_min + lane (ALU only)
        const int L = a.l_min + lane;
        const bool qlane = lane < nL && L <= n - 1;   // the suffix and an earlier occurrence both fit
        u64 qk = 0;
        {
            // the prefix hashes are the same in every lane; lane k keeps the
            // one of length L (a select, not a branch per length: per-length
            // lane masks kept for later uses were spilled)
            u64 hs = kHashSeed, hl = kHashSeed;
#pragma unroll
            for (int j = 0; j < kMaxL; ++j) {
                hs = roll(hs, s[j]);
                hl = j < L ? hs : hl;
            }
            qk = finish_key(hl, L);
        }
        const uint32_t qfp = fingerprint(qk, a.fp_mask);
        uint32_t qi = (uint32_t)home_slot(qk, ns);
        u64 v[kQWin];                        // a window of slots from the key's home slot
#pragma unroll
        for (int w = 0; w < kQWin; ++w)
            v[w] = qlane ? __hip_atomic_load(T + wrap_add(qi, w, ns), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_WORKGROUP)
                         : 0ull;

        // direct match of the suffix against the appended positions (from
        // their tokens), in flight with the first probe
        u64 key_new = 0;
        for (int p0 = p_lo; p0 <= p_hi; p0 += 64) {
            const int p = p0 + lane;
            const bool ins = p <= p_hi;
            int lmax = a.l_max;
            asm volatile("" : "+s"(lmax));
            if (p0 != p_lo) {
#pragma unroll
                for (int j = 0; j < kMaxL; ++j) t[j] = (ins && j < lmax && p - j >= 0) ? h[p - j] : 0;
            }
            int Lp = 0;
            bool run = ins;
#pragma unroll
            for (int j = 0; j < kMaxL; ++j) {
                run = run && j < lmax && p - j >= 0 && t[j] == s[j];
                Lp += run ? 1 : 0;
            }
            if (Lp >= a.l_min) {
                const u64 k = ((u64)Lp << 31) | (uint32_t)p;
                key_new = k > key_new ? k : key_new;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const u64 o = __shfl_xor(key_new, off);
            key_new = o > key_new ? o : key_new;
        }

        // ---- table query: lane k takes length L = l_min + k ------------------
        int e = -1;
        bool collide = false;
        if (qlane) {
            for (int probes = 0; probes < kMaxProbe; probes += kQWin) {
                if (probes > 0) {
                    qi = wrap_add(qi, kQWin, ns);
#pragma unroll
                    for (int w = 0; w < kQWin; ++w)
                        v[w] = __hip_atomic_load(T + wrap_add(qi, w, ns), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP);
                }
                // the first slot of the window that ends the probe sequence
                u64 vv = 0;
                bool found = false;
#pragma unroll
                for (int w = kQWin - 1; w >= 0; --w) {
                    const bool stop = v[w] == 0 || (uint32_t)(v[w] >> 32) == qfp;
                    vv = stop ? v[w] : vv;
                    found = found || stop;
                }
                if (!found) continue;
                if (vv == 0) break;                                  // no occurrence
                {
                    const int pe = (int)(uint32_t)vv - 1;
                    bool same = pe >= L - 1 && pe <= n - 2;
                    if (same) {
                        int Lv = L;                                  // opaque: see the hash above
                        asm volatile("" : "+v"(Lv));
                        int32_t g[kMaxL];                            // all loads in flight at once
#pragma unroll
                        for (int j = 0; j < kMaxL; ++j) g[j] = j < Lv ? h[pe - j] : 0;
#pragma unroll
                        for (int j = 0; j < kMaxL; ++j) same = same && (j >= Lv || g[j] == s[j]);
                    }
                    if (same) e = pe; else collide = true;
                    break;
                }
            }
        }
        const u64 hit = __ballot(e >= 0);
        const u64 doubt = __ballot(collide);
        u64 key_table = 0;
        if (hit != 0) {
            const int kb = 63 - __builtin_clzll(hit);
            key_table = ((u64)(a.l_min + kb) << 31) | (uint32_t)__builtin_amdgcn_readlane(e, kb);
        }
        key = key_table > key_new ? key_table : key_new;
        // a length in doubt above the answer's could hold a longer match
        if (doubt != 0) {
            const int ld = a.l_min + 63 - __builtin_clzll(doubt);
            if ((u64)ld > (key >> 31)) exact = true;
        }
    }
    if (exact) key = exact_scan(h, n, a, lane);

    // ---- match and LZ draft ------------------------------------------------
    const int m = (int)(key >> 31);
    const int e = key != 0 ? (int)(key & 0x7FFFFFFFull) : -1;
    int d = LCD_PAD;                          // lane k < 15: draft slot k
    if (lane < LCD_DRAFT_STRIDE && m > 0 && lane < a.k_max) {
        const int D = n - 1 - e;                                      // >= 1
        d = h[e + 1 + lane % D];
    }
    if (lane < LCD_DRAFT_STRIDE) draft[(int64_t)r * LCD_DRAFT_STRIDE + lane] = d;
    if (lane == 0) {
        match_len[r] = m;
        match_end[r] = e;
    }
    // the row's last tokens after this call, for the next one: with an append,
    // the emitted target tokens 0..acc then the tokens before them
    int n_next = n, tok_next = tok;
    if (kStep) {
        const int acc = finish_step(r, m, d, sin, tin, lane, ro, n0, n, *iop);
        if (iop->append && acc >= 0) {
            n_next = n + acc + 1;
            const int tk = __shfl(sin, LCD_Q_STRIDE + (lane <= acc ? acc - lane : 0));
            const int old = __shfl(tok, (lane - acc - 1) & 63);
            tok_next = lane <= acc ? tk : old;
        }
    }
    if (n_next != n || !cached) {
        if (lane < kCacheTok) ctok[lane] = tok_next;
        if (lane == 0) cache[0] = ((u64)kCacheTag << 32) | (uint32_t)n_next;
    }
}

// Build: clear the tables, then insert every position p <= n-2 of every row.
__global__ void __launch_bounds__(kBuildThreads)
index_clear_kernel(u64 *__restrict__ tables, int64_t words) {
    for (int64_t i = blockIdx.x * (int64_t)kBuildThreads + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * kBuildThreads)
        tables[i] = 0;
}

__global__ void __launch_bounds__(kBuildThreads)
clear_flags_kernel(int32_t *__restrict__ flags, int32_t n) {
    const int i = blockIdx.x * kBuildThreads + threadIdx.x;
    if (i < n) flags[i] = 0;
}

__global__ void __launch_bounds__(kBuildThreads)
index_build_kernel(const int32_t *__restrict__ hist, const int64_t *__restrict__ row_off,
                   const int32_t *__restrict__ len, int32_t B, IndexArgs a,
                   const int64_t *__restrict__ table_off, const int32_t *__restrict__ table_slots,
                   u64 *__restrict__ tables, int32_t *__restrict__ indexed_len, int32_t chunk,
                   int32_t cpr, int32_t *__restrict__ failed) {
    const int r = blockIdx.x / cpr;
    const int c = blockIdx.x - r * cpr;
    if (r >= B) return;
    const int32_t n0 = len[r];
    const int n = n0 > 0 ? n0 : 0;
    const int32_t *__restrict__ h = hist + row_off[r];
    u64 *__restrict__ T = tables + table_off[r];
    const uint32_t ns = (uint32_t)table_slots[r];
    bool ok = true;
    // positions 0..n-2, chunks of `chunk` positions per workgroup, strided by cpr
    for (int p0 = c * chunk; p0 <= n - 2; p0 += cpr * chunk) {
        for (int p = p0 + threadIdx.x; p < p0 + chunk && p <= n - 2; p += kBuildThreads) {
            u64 hs = kHashSeed;
            for (int j = 0; j < a.l_max && p - j >= 0; ++j) {
                hs = roll(hs, h[p - j]);
                const int L = j + 1;
                if (L >= a.l_min) ok = insert_one(T, ns, finish_key(hs, L), a.fp_mask, p) && ok;
            }
        }
    }
    if (!ok) atomicOr(failed + r, 1);
    if (c == 0 && threadIdx.x == 0) indexed_len[r] = n;
}

// A row whose build hit the probe bound is marked stale (answered by scans).
__global__ void index_mark_kernel(const int32_t *__restrict__ failed, int32_t B,
                                  int32_t *__restrict__ indexed_len) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r < B && failed[r] != 0) indexed_len[r] = -1;
}

IndexArgs index_args(const lcd_params *p, int32_t fp_bits) {
    IndexArgs a;
    a.l_min = p->l_min;
    a.l_max = p->l_max;
    a.k_max = p->k_max;
    const int fb = fp_bits <= 0 ? 31 : fp_bits;
    a.fp_mask = fb >= 31 ? 0x7FFFFFFFu : ((1u << fb) - 1u);
    return a;
}

// Slots of a row's table: index_load per indexed length and token of its
// capacity (at most 1/index_load of them ever taken), at least 16.
int64_t table_slots_for(int32_t cap, int nL, int load) {
    const int64_t need = (int64_t)load * nL * (int64_t)(cap > 1 ? cap : 1);
    return need > 16 ? need : 16;
}

}  // namespace
}  // namespace lcd

extern "C" int64_t lookup_index_plan(const int32_t *cap, int32_t B, const lcd_params *p,
                                     int64_t *table_off, int32_t *table_slots) {
    using namespace lcd;
    if (B < 0 || lcd_check_params(p) != LCD_OK) return LCD_EINVAL;
    if (B > 0 && (!cap || !table_off || !table_slots)) return LCD_EINVAL;
    const int nL = p->l_max - p->l_min + 1;
    int64_t off = (int64_t)B * kCacheWords;            // the requests' token caches come first
    for (int32_t r = 0; r < B; ++r) {
        if (cap[r] < 0) return LCD_EINVAL;
        const int64_t ns = table_slots_for(cap[r], nL, p->index_load);
        if (ns > INT32_MAX) return LCD_EINVAL;
        table_off[r] = off;
        table_slots[r] = (int32_t)ns;
        off += ns;
    }
    return off * 8;
}

extern "C" int lookup_index_build(const int32_t *hist, const int64_t *row_off, const int32_t *len,
                                  int32_t B, const lcd_params *p, int32_t fp_bits,
                                  const int64_t *table_off, const int32_t *table_slots,
                                  void *tables, size_t table_bytes, int32_t *indexed_len,
                                  int32_t *scratch, int32_t max_len, void *stream) {
    using namespace lcd;
    if (B < 0 || max_len < 0 || fp_bits < 0 || fp_bits > 31 || lcd_check_params(p) != LCD_OK)
        return LCD_EINVAL;
    if (B == 0) return LCD_OK;
    if (!hist || !row_off || !len || !table_off || !table_slots || !tables || !indexed_len ||
        !scratch || (reinterpret_cast<uintptr_t>(tables) & 7) != 0 || table_bytes < 8)
        return LCD_EINVAL;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const IndexArgs a = index_args(p, fp_bits);
    const int64_t words = (int64_t)(table_bytes / 8);
    const int64_t clear_blocks = (words + kBuildThreads - 1) / kBuildThreads;
    hipLaunchKernelGGL(index_clear_kernel, dim3((unsigned)(clear_blocks < 65536 ? clear_blocks : 65536)),
                       dim3(kBuildThreads), 0, st, static_cast<u64 *>(tables), words);
    // scratch: B int32 flags of rows whose build hit the probe bound
    hipLaunchKernelGGL(clear_flags_kernel, dim3((unsigned)((B + kBuildThreads - 1) / kBuildThreads)),
                       dim3(kBuildThreads), 0, st, scratch, B);
    const int32_t chunk = 4096;
    const int64_t per_row = ((int64_t)max_len + chunk - 1) / chunk;
    const int32_t cpr = (int32_t)(per_row < 1 ? 1 : (per_row > 4096 ? 4096 : per_row));
    hipLaunchKernelGGL(index_build_kernel, dim3((unsigned)((int64_t)B * cpr)), dim3(kBuildThreads),
                       0, st, hist, row_off, len, B, a, table_off, table_slots,
                       static_cast<u64 *>(tables), indexed_len, chunk, cpr, scratch);
    hipLaunchKernelGGL(index_mark_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, st,
                       scratch, B, indexed_len);
    return hipGetLastError() == hipSuccess ? LCD_OK : LCD_EHIP;
}

namespace lcd {
namespace {
template <bool kStep>
int index_launch(const int32_t *hist, const int64_t *row_off, const int32_t *len, int32_t B,
                 const lcd_params *p, int32_t fp_bits, const int64_t *table_off,
                 const int32_t *table_slots, void *tables, int32_t *indexed_len,
                 int32_t *match_len, int32_t *match_end, int32_t *draft, const StepIO &io,
                 void *stream, void *ev0, void *ev1) {
    const IndexArgs a = index_args(p, fp_bits);
    const dim3 grid((unsigned)B);
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (ev0 != nullptr || ev1 != nullptr)
        hipExtLaunchKernelGGL(index_propose_kernel<kStep>, grid, dim3(128), 0u, st,
                              reinterpret_cast<hipEvent_t>(ev0), reinterpret_cast<hipEvent_t>(ev1),
                              0u, io, hist, row_off, len, B, a, table_off, table_slots,
                              static_cast<u64 *>(tables), indexed_len, match_len, match_end, draft);
    else
        hipLaunchKernelGGL(index_propose_kernel<kStep>, grid, dim3(128), 0, st, io,
                           hist, row_off, len, B, a, table_off, table_slots,
                           static_cast<u64 *>(tables), indexed_len, match_len, match_end, draft);
    return hipGetLastError() == hipSuccess ? LCD_OK : LCD_EHIP;
}

bool index_args_ok(const void *hist, const void *row_off, const void *len, const void *table_off,
                   const void *table_slots, const void *tables, const void *indexed_len,
                   const void *match_len, const void *match_end, const void *draft) {
    return hist && row_off && len && table_off && table_slots && tables && indexed_len && match_len &&
           match_end && draft && (reinterpret_cast<uintptr_t>(tables) & 7) == 0;
}

int index_propose(const int32_t *hist, const int64_t *row_off, const int32_t *len, int32_t B,
                  const lcd_params *p, int32_t fp_bits, const int64_t *table_off,
                  const int32_t *table_slots, void *tables, int32_t *indexed_len,
                  int32_t *match_len, int32_t *match_end, int32_t *draft, void *stream,
                  void *ev0, void *ev1) {
    if (B < 0 || fp_bits < 0 || fp_bits > 31 || lcd_check_params(p) != LCD_OK) return LCD_EINVAL;
    if (B == 0) return LCD_OK;
    if (!index_args_ok(hist, row_off, len, table_off, table_slots, tables, indexed_len, match_len,
                       match_end, draft))
        return LCD_EINVAL;
    return index_launch<false>(hist, row_off, len, B, p, fp_bits, table_off, table_slots, tables,
                               indexed_len, match_len, match_end, draft, StepIO{}, stream, ev0, ev1);
}

int index_step(int32_t *hist, const int64_t *row_off, int32_t *len, const int32_t *cap, int32_t B,
               const lcd_params *p, int32_t fp_bits, const int64_t *table_off,
               const int32_t *table_slots, void *tables, int32_t *indexed_len,
               const int32_t *model_draft, const int32_t *target, lcd_sched_state *state,
               int32_t *match_len, int32_t *match_end, int32_t *draft, int32_t *block,
               int32_t *block_len, int32_t *accept, int32_t *long_next, uint32_t *tele,
               int32_t append, void *stream, void *ev0, void *ev1) {
    if (B < 0 || fp_bits < 0 || fp_bits > 31 || lcd_check_params(p) != LCD_OK) return LCD_EINVAL;
    if (B == 0) return LCD_OK;
    if (!index_args_ok(hist, row_off, len, table_off, table_slots, tables, indexed_len, match_len,
                       match_end, draft))
        return LCD_EINVAL;
    if (!model_draft || !target || !state || !block || !block_len || !accept) return LCD_EINVAL;
    if (append && !cap) return LCD_EINVAL;
    const StepIO io{hist, len, cap, model_draft, target, state, block, block_len, accept, long_next,
                    tele, fuse_args(p), sched_args(p), append ? 1 : 0};
    return index_launch<true>(hist, row_off, len, B, p, fp_bits, table_off, table_slots, tables,
                              indexed_len, match_len, match_end, draft, io, stream, ev0, ev1);
}
}  // namespace
}  // namespace lcd

extern "C" int lookup_index_propose(const int32_t *hist, const int64_t *row_off, const int32_t *len,
                                    int32_t B, const lcd_params *p, int32_t fp_bits,
                                    const int64_t *table_off, const int32_t *table_slots,
                                    void *tables, int32_t *indexed_len, int32_t *match_len,
                                    int32_t *match_end, int32_t *draft, void *stream) {
    return lcd::index_propose(hist, row_off, len, B, p, fp_bits, table_off, table_slots, tables,
                              indexed_len, match_len, match_end, draft, stream, nullptr, nullptr);
}

extern "C" int lookup_index_propose_timed(const int32_t *hist, const int64_t *row_off,
                                          const int32_t *len, int32_t B, const lcd_params *p,
                                          int32_t fp_bits, const int64_t *table_off,
                                          const int32_t *table_slots, void *tables,
                                          int32_t *indexed_len, int32_t *match_len,
                                          int32_t *match_end, int32_t *draft, void *stream,
                                          void *ev_start, void *ev_stop) {
    return lcd::index_propose(hist, row_off, len, B, p, fp_bits, table_off, table_slots, tables,
                              indexed_len, match_len, match_end, draft, stream, ev_start, ev_stop);
}

extern "C" int lookup_index_decode_step(int32_t *hist, const int64_t *row_off, int32_t *len,
                                        const int32_t *cap, int32_t B, const lcd_params *p,
                                        int32_t fp_bits, const int64_t *table_off,
                                        const int32_t *table_slots, void *tables,
                                        int32_t *indexed_len, const int32_t *model_draft,
                                        const int32_t *target, lcd_sched_state *state,
                                        int32_t *match_len, int32_t *match_end, int32_t *draft,
                                        int32_t *block, int32_t *block_len, int32_t *accept,
                                        int32_t *long_next, uint32_t *telemetry, int32_t append,
                                        void *stream) {
    return lcd::index_step(hist, row_off, len, cap, B, p, fp_bits, table_off, table_slots, tables,
                           indexed_len, model_draft, target, state, match_len, match_end, draft,
                           block, block_len, accept, long_next, telemetry, append, stream, nullptr,
                           nullptr);
}

extern "C" int lookup_index_decode_step_timed(
    int32_t *hist, const int64_t *row_off, int32_t *len, const int32_t *cap, int32_t B,
    const lcd_params *p, int32_t fp_bits, const int64_t *table_off, const int32_t *table_slots,
    void *tables, int32_t *indexed_len, const int32_t *model_draft, const int32_t *target,
    lcd_sched_state *state, int32_t *match_len, int32_t *match_end, int32_t *draft, int32_t *block,
    int32_t *block_len, int32_t *accept, int32_t *long_next, uint32_t *telemetry, int32_t append,
    void *stream, void *ev_start, void *ev_stop) {
    return lcd::index_step(hist, row_off, len, cap, B, p, fp_bits, table_off, table_slots, tables,
                           indexed_len, model_draft, target, state, match_len, match_end, draft,
                           block, block_len, accept, long_next, telemetry, append, stream, ev_start,
                           ev_stop);
}

// lcd_lookup.hip -- batched context lookup (longest suffix, latest earlier
// occurrence, LZ-style draft copy) and the one-kernel decode step, for MI355X /
// gfx950.
//
// Method: HyperQwen lookup-drafting article, section "第 1 步": each decode
// step, for every request, scan that request's own token history for the most
// recent earlier occurrence of its longest current suffix of 4..12 tokens
// (overlap with the suffix allowed) and draft the tokens that follow it; most
// candidates fail a 4-token test, so extending the survivors costs almost
// nothing.  The article runs one Triton program per request on a consumer GPU;
// the design here is built around gfx950 instead:
//
//  * The candidate ends of every request are cut into chunks of T tokens (a
//    multiple of 256; the host derives T from the longest row), one
//    workgroup per chunk, B x cpr workgroups per launch: four waves each, or
//    sixteen for batches of at most 128 long rows (one workgroup per CU from
//    32 rows of 16k+ tokens, or of 8k+ tokens and 1.2M+ in all; one per ~12k
//    tokens of the longest row for fewer rows of 6k+ tokens).
//  * Only the waves that need them read the lookup's output pointers and the
//    rest of the step's arguments, from the kernel-argument segment where
//    they are used, so they are not held (and spilled) through the scan.
//  * A decode-step scan is short, so dependent memory round trips cost as much
//    as the bytes: the row offset and length are loaded together, then the 16
//    suffix tokens (one per lane) and the wave's first batch of tiles go into
//    the vector memory queue back to back, so the suffix is waited for alone
//    and each tile as it lands.
//  * A tile is one 16-byte load per lane, 1 KiB per wave-wide load, fully
//    coalesced: lanes 4..63 hold 240 candidate ends and lanes 0..3 the 16
//    tokens before them, which the tile before also loaded.  Every test of a
//    tile then reads only its own registers, so tiles need no order: the
//    waves of a workgroup take them from a counter in LDS as they go, and
//    waves whose loads return early take over the tiles of waves whose loads
//    return late (in one launch the loads of the first round arrive over
//    about 3 us, and with fixed shares the last wave of a workgroup finished
//    that much after its first).
//  * Quick test: a tile can hold a candidate only if it holds the rarest
//    adjacent pair of suffix tokens (s_j, s_j+1): eight compares per lane and
//    one scalar branch per tile.  A wave whose pair turns out to be common
//    drops the quick test and runs the full one.
//  * Flagged tiles get the full 4-token test: each lane receives the previous
//    lane's last three tokens by one wave-wide DPP lane shift, compares the
//    four tokens ending at each of its positions, and one ballot per
//    component gives the wave-uniform survivor masks.  Survivors are extended
//    up to l_max tokens with ballot masks shifted by whole lanes.
//  * A packed key (length, end) orders candidates.  Every workgroup of a
//    request takes an arrival ticket when it starts (one atomic add, in flight
//    during its scan), and at the end publishes its best key together with the
//    15 tokens that follow that match (loaded by the wave that found it, when
//    it found it, so no load follows the scan) as tagged 8-byte words in its
//    own workspace slot.  The workgroup holding the last ticket gathers the
//    slots -- it only waits for workgroups that started before it, so the
//    wait always ends -- and thus has the winning draft without another
//    dependent load.  It finishes the
//    request with one wave (draft copy and, in the decode step, fusion,
//    acceptance, append and scheduler update) and re-zeroes the workspace.
//  * The words carry the call's tag, which the ticket returns with the arrival
//    count: the gatherer takes only words of its own call, and starts the
//    next call's tag when it resets the count.  Its wait is bounded all the
//    same; when the bound runs out the request reports match_len = -1 (no
//    answer, an error) and a slot published later carries a tag no later call
//    accepts.
//
// No MFMA: the work is integer compares on a stream; HBM bandwidth and memory
// latency bound it.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "lcd.h"
#include "lcd_finish.h"
#include "lcd_rules.h"

namespace lcd {
namespace {

// Waves per workgroup: 4 in general; 16 for batches of 32-128 rows of 16k+
// tokens (8k+ when the batch holds 1.2M+ tokens) and of 1-31 rows of 6k+
// tokens, where it measured 3-42 % faster.
constexpr int kWavesSmall = 4;
constexpr int kWavesLarge = 16;
constexpr int kNumCUs = 256;
// 4-wave workgroups of the scan resident on one CU at once, as compiled (106
// SGPRs and at most 52 VGPRs per wave: 7 waves per SIMD; lookup_scan_occupancy
// reports the runtime's figure and the GPU tests hold it to this).  A
// workgroup beyond 7 x 256 is dispatched only when an earlier one ends.
// Forcing 8 waves per SIMD with a launch bound cost more in spilled registers
// than it gained.
constexpr int kResidentSmall = 7;
constexpr int kTileTok = 256;   // chunk lengths are multiples of this
constexpr int64_t kMaxChunk = int64_t(1) << 28;   // a chunk's descriptor range stays below 2^32 bytes
#ifndef LCD_UNROLL
#define LCD_UNROLL 4
#endif
constexpr int kUnroll = LCD_UNROLL;   // tiles loaded ahead by each wave

typedef unsigned long long u64;

// Match key: end (relative to the row) in bits 0..30, length in bits 31..35;
// larger keys are longer, then later, matches.
constexpr int kLenShift = 31;
constexpr u64 kEndMask = (1ull << kLenShift) - 1;

// Workspace of one request: the header word (arrival count in bits 0..31,
// the call's epoch above), a pad word, then one slot per workgroup of 16
// words: units 0..14 hold the staged draft tokens as tag << 32 | token, unit
// 15 holds tag << 36 | key, where tag = epoch + 1 (1 .. 2^28 - 1).  A zero
// word is "not written" for every tag.
constexpr int kMaxCpr = 64;                               // workgroups per request, at most
constexpr int kSlotWords = 16;
constexpr int kReqWords = 2 + kMaxCpr * kSlotWords;
constexpr int kPollBatch = 8;                             // slot words per lane loaded at once
constexpr u64 kTagLimit = (1ull << 28) - 1;               // epochs 0 .. kTagLimit - 1
constexpr int kPollMax = 1 << 20;                         // gathering polls, at most (default)
constexpr int kBufferWord3 = 0x00020000;                  // gfx9 buffer descriptor, dword 3
constexpr int kLoadNT = 2;                                 // buffer-load cache policy: non-temporal
constexpr int kFullAfter = 4;                             // flagged tiles before a wave drops the quick test

struct ScanArgs {
    int32_t cpr;               // workgroups per request (equal chunks per row)
    int32_t T;                 // chunk length in candidate ends, a multiple of kTileTok
    int32_t l_min, l_max, k_max;
    int32_t B;                 // requests
    int32_t wgs;               // workgroups per launch (token-balanced chunks)
    int32_t waves;             // waves per workgroup (kWavesSmall or kWavesLarge)
    int32_t polls;             // gathering polls before giving up
};

// Tag of the call whose ticket returned header word h, and the header that
// starts the next call (count 0, next epoch).
__device__ __forceinline__ u64 call_tag(u64 h) { return (h >> 32) + 1; }
__device__ __forceinline__ u64 next_header(u64 h) {
    const u64 e = (h >> 32) + 1;
    return (e < kTagLimit ? e : 0) << 32;
}

// Token-balanced chunks (ragged batches): one chunk length for the whole
// batch, from the total and the longest row's candidate ends and the grid of
// wgs workgroups -- long enough that the chunks of all rows (at least one per
// row) fit the grid, and that no row has more than kMaxCpr chunks.  The device
// and the host's launch-shape query use this same rule.
__host__ __device__ inline int32_t balanced_chunk_len(int64_t total, int64_t longest, int64_t wgs,
                                                      int64_t B) {
    const int64_t room = wgs - B > 0 ? wgs - B : 1;
    int64_t t = (total + room - 1) / room;
    const int64_t t2 = (longest + 63) / 64;
    if (t < t2) t = t2;
    t = (t + 255) / 256 * 256;
    if (t < 256) t = 256;
    return (int32_t)(t < kMaxChunk ? t : kMaxChunk);
}

// (The kernel takes cpr and T as separate leading arguments.)

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ u64 ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int tok(const int4 &t, int c) {
    return c == 0 ? t.x : (c == 1 ? t.y : (c == 2 ? t.z : t.w));
}

// Tiles.  A tile is one wave-wide load of 256 consecutive tokens, 16 bytes
// per lane: lanes 0..3 repeat the last 16 tokens of the tile before it and
// lanes 4..63 hold the tile's own 240 candidate ends.  A candidate's 4-token
// test and its extension up to 16 tokens reach back at most 4 lanes, so every
// test of a tile reads only its own registers: any wave can take any tile, in
// any order, with no halo load and nothing carried from tile to tile.
constexpr int kHaloLanes = 4;
constexpr int kTileCand = (64 - kHaloLanes) * 4;          // 240 candidate ends per tile
constexpr int kHaloTok = kHaloLanes * 4;                  // 16 tokens before them
constexpr u64 kCandLanes = ~0ull << kHaloLanes;           // lanes holding candidates
constexpr u64 kPairLanes = ~0ull << (kHaloLanes - 1);     // pair positions a candidate can need
constexpr unsigned kNoTileOff = 0x80000000u;              // past every chunk's descriptor

// Lanes 0..3 and the tokens of lane 4 before the row start (`lo`: the row
// start's position within lane 4's granule) become `sent`: the head chunk's
// first tile.
__device__ __forceinline__ int4 mask_head(int4 t, int lane, int lo, int sent) {
    const int rel = lane < kHaloLanes ? 4 : (lane == kHaloLanes ? lo : 0);
    t.x = (0 < rel) ? sent : t.x;
    t.y = (1 < rel) ? sent : t.y;
    t.z = (2 < rel) ? sent : t.z;
    t.w = (3 < rel) ? sent : t.w;
    return t;
}

// Prefilter survivors of tile t (tile index kt), restricted to candidate
// ends in [c_lo, c_hi) (positions relative to the chunk's first granule):
// bit i of P[c] is set when the PF tokens ending at position 4i+c of the tile
// equal s_0..s_PF-1.  Positions before the lane's own granule are the
// previous lane's last three tokens, brought over by one wave-wide lane shift,
// so every test is a per-lane compare and one ballot per component.
constexpr int kDppWaveShr1 = 0x138;          // DPP: lane i reads lane i-1

template <int PF>
__device__ __forceinline__ void survivors(const int4 &t, const int (&s)[4], int kt, int c_lo,
                                          int c_hi, int lane, u64 (&P)[4]) {
    const int q1 = __builtin_amdgcn_update_dpp(0, t.y, kDppWaveShr1, 0xf, 0xf, true);
    const int q2 = __builtin_amdgcn_update_dpp(0, t.z, kDppWaveShr1, 0xf, 0xf, true);
    const int q3 = __builtin_amdgcn_update_dpp(0, t.w, kDppWaveShr1, 0xf, 0xf, true);
    // token at position 4i+c-j: component c-j of this lane, or component
    // c-j+4 (1..3) of the previous lane
    auto at = [&](int c, int j) -> int {
        const int k = c - j;
        return k >= 0 ? tok(t, k) : (k == -3 ? q1 : (k == -2 ? q2 : q3));
    };
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        bool ok = true;
#pragma unroll
        for (int j = 0; j < PF; ++j) ok = ok && (at(c, j) == s[j]);
        P[c] = ballot(ok) & kCandLanes;
    }
    const int A = kTileCand * kt;                  // the tile's first candidate position
    if (A < c_lo || A + kTileCand > c_hi) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int x = A + 4 * (lane - kHaloLanes) + c;
            P[c] &= ballot(x >= c_lo && x < c_hi);
        }
    }
}

// Extend the survivors M[c] of tile t, which match PF suffix tokens, one
// token at a time while some candidate still matches, up to J tokens; sv
// holds suffix token s_j in lane j.  Position e-j lies k = ceil((j-c)/4) <= 4
// lanes back, inside the tile for every candidate lane.  Returns the length
// reached and leaves in M the candidates reaching it.  Fully unrolled: a loop
// here, inside the unrolled tile loop, would make the compiler wait for every
// load in flight at its header.
template <int PF>
__device__ __forceinline__ int extend(const int4 &t, int sv, int J, u64 (&M)[4]) {
    // J is opaque here, so the compiler cannot hoist the per-length tests
    // j < J out of the tile loop: held there, they took about twenty scalar
    // registers for the whole scan and were spilled into vector lanes.
    asm volatile("" : "+s"(J));
    int L = PF;
    bool alive = true;
#pragma unroll
    for (int j = PF; j < LCD_MAX_SUFFIX; ++j) {
        if (alive && j < J) {
            const int sj = __builtin_amdgcn_readlane(sv, j);
            u64 N[4];
            u64 any = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int k = (j - c + 3) >> 2;      // lanes back: ceil((j-c)/4), 0..4
                const int cc = (c - j) & 3;          // component of position e-j
                N[c] = M[c] & (ballot(tok(t, cc) == sj) << k);
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

// Workgroup barrier ordering LDS only: the tile loads in flight are not
// waited for (a full __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Kernel modes.  kPropose: the lookup only.  kStep: the whole decode step; the
// workgroup that finishes a request also fuses the verify block, accepts
// greedily (optionally appending) and advances the scheduler.
enum { kPropose = 0, kStep = 1 };

__device__ __forceinline__ u64 readlane64(u64 v, int l) {
    return ((u64)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
}

// Running maximum within each row of 16 lanes (DPP row shifts by 1, 2, 4, 8;
// lanes with no source read 0): lane 15 ends with the maximum of lanes 0..15.
template <int kCtrl>
__device__ __forceinline__ u64 dpp_shr64(u64 v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, kCtrl, 0xf, 0xf, true);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), kCtrl, 0xf, 0xf, true);
    return ((u64)hi << 32) | lo;
}
__device__ __forceinline__ u64 row_max64(u64 v) {
    u64 o = dpp_shr64<0x111>(v);
    v = o > v ? o : v;
    o = dpp_shr64<0x112>(v);
    v = o > v ? o : v;
    o = dpp_shr64<0x114>(v);
    v = o > v ? o : v;
    o = dpp_shr64<0x118>(v);
    return o > v ? o : v;
}

// A struct of 4-byte words spread over lanes (word k in lane k), read back
// into scalar registers without a memory access.
template <typename T>
__device__ __forceinline__ T from_lanes(int v) {
    static_assert(sizeof(T) % 4 == 0 && sizeof(T) <= 256, "one word per lane");
    int w[sizeof(T) / 4];
#pragma unroll
    for (int k = 0; k < (int)(sizeof(T) / 4); ++k) w[k] = __builtin_amdgcn_readlane(v, k);
    return __builtin_bit_cast(T, w);
}

// The lookup's outputs and the rest of the step's inputs and outputs: the
// scan kernel's first argument.
struct ScanOut {
    int32_t *match_len, *match_end, *draft;
    StepIO io;
};
constexpr int kOutWords = (int)(sizeof(ScanOut) / 4);

// Result of request r (row of lr tokens as stored, n = max(lr, 0), at ro)
// given its best key, run by one whole wave.  The tokens following the
// match, h[e+1+min(k, D-1)] for k < 15 with D = n-1-e, are in lanes base+k of
// `src`.  Writes the match and draft and, in kStep mode, the rest of the step
// (sin: the per-lane step inputs) to the outputs in `so`.  `failed`: the merge
// gave up, reported as m = -1, e = -1 and an empty draft (the step then goes
// on as without a match).
template <int kMode>
__device__ __forceinline__ void finish_request(int r, u64 key, bool failed, int src, int base,
                                               int sin, uint32_t tin, int lane, int64_t ro,
                                               int32_t lr, int n, int k_max, const ScanOut &so) {
    if (failed) key = 0;
    const int m = failed ? -1 : (key ? (int)(key >> kLenShift) : 0);
    const int e = key ? (int)(key & kEndMask) : -1;
    const int D = key ? n - 1 - e : 1;
    // LZ-style copy: d[k] = h[n - D + (k mod D)], token (k mod D) of the match
    const int kk = lane < LCD_DRAFT_STRIDE ? lane : 0;
    int dk = __shfl(src, base + kk % D);
    dk = (m > 0 && lane < k_max) ? dk : LCD_PAD;
    if (lane < LCD_DRAFT_STRIDE) gstore<true>(so.draft + (int64_t)r * LCD_DRAFT_STRIDE + lane, dk);
    if (lane == 0) {
        gstore<true>(so.match_len + r, m);
        gstore<true>(so.match_end + r, e);
    }
    if (kMode == kStep) finish_step<true>(r, m, dk, sin, tin, lane, ro, lr, n, so.io);
}

constexpr int kBalPer = LCD_BALANCE_MAX_B / 64;           // lengths held per lane

// Inclusive prefix over the wave's 64 lanes by DPP: row shifts by 1, 2, 4 and
// 8 within each row of 16 lanes (lanes with no source take 0), then lane 15's
// value into row 1 and lane 47's into row 3 (row_bcast:15), and lane 31's into
// rows 2 and 3 (row_bcast:31).  kMax: running maximum instead of sum.
template <bool kMax>
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    auto op = [](uint32_t x, uint32_t y) { return kMax ? (x > y ? x : y) : x + y; };
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, true));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, true));
    return v;
}

// Token-balanced assignment of workgroup blockIdx.x: every wave reads all B
// lengths (one round trip), derives the batch's chunk length and finds its
// (request, chunk) by a prefix over the rows' chunk counts.  Returns false
// when the workgroup has no chunk.  Only the groups of 64 rows that exist are
// visited, and the cross-lane sums are DPP scans: 7 such workgroups share a
// CU, and a wave's instructions here are all in front of its first tile.
__device__ __forceinline__ bool balanced_assignment(const int32_t *__restrict__ len, int B, int lane,
                                                    int &r, int &c0, int &P, int &T) {
    const int groups = (B + 63) >> 6;
    uint32_t nc[kBalPer];
    // All of a lane's length loads in flight at once: rows past the batch
    // re-read its last row (B >= 1) and are masked afterwards.  Loads behind
    // a per-lane test were each waited for before the next was sent, one
    // round trip per 64 rows (one 262k-token row among 1,023 of 2k tokens:
    // 15.6 -> 13.0 us; 256 ragged rows 17.2 -> 16.9 us).
    int lv[kBalPer];
#pragma unroll
    for (int k = 0; k < kBalPer; ++k) {
        const int row = k * 64 + lane;
        lv[k] = len[row < B ? row : B - 1];
    }
#pragma unroll
    for (int k = 0; k < kBalPer; ++k) {
        const int row = k * 64 + lane;
        const int l = (k < groups && row < B) ? lv[k] : 0;
        nc[k] = l > 1 ? (uint32_t)(l - 1) : 0u;
    }
    // the total of candidate ends in two 32-bit halves (no carry out of either
    // for up to 1024 rows), and the longest row's
    uint32_t lo = 0, hi = 0, mx = 0;
#pragma unroll
    for (int k = 0; k < kBalPer; ++k) {
        lo += nc[k] & 0xffffu;
        hi += nc[k] >> 16;
        mx = nc[k] > mx ? nc[k] : mx;
    }
    lo = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan<false>(lo), 63);
    hi = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan<false>(hi), 63);
    mx = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan<true>(mx), 63);
    T = balanced_chunk_len(((int64_t)hi << 16) + lo, (int64_t)mx, (int64_t)gridDim.x, (int64_t)B);
    // chunks of a row: ceil(nc / T) = ceil(ceil(nc / 256) / t8), T = 256 t8,
    // from a double reciprocal: for a <= 2^23 the truncated product is the
    // quotient or, when t8 divides a, one less, which the remainder corrects
    const uint32_t t8 = (uint32_t)T >> 8;
    const double rt = 1.0 / (double)t8;
    const int w = (int)blockIdx.x;
    int base = 0;
    bool found = false;
#pragma unroll
    for (int k = 0; k < kBalPer; ++k) {
        if (found || k >= groups) continue;     // uniform
        const int row = k * 64 + lane;
        const uint32_t a = (nc[k] + 255u) >> 8;
        uint32_t q = (uint32_t)((double)a * rt);
        q += a - q * t8 >= t8 ? 1u : 0u;
        const int kr = row < B ? (nc[k] > 0 ? (int)(q + (q * t8 != a ? 1u : 0u)) : 1) : 0;
        const int incl = (int)wave_incl_scan<false>((uint32_t)kr);
        const int gsum = __builtin_amdgcn_readlane(incl, 63);
        if (w < base + gsum) {
            const int l = (int)__builtin_ctzll(ballot(base + incl > w));
            r = k * 64 + l;
            c0 = w - base - __builtin_amdgcn_readlane(incl - kr, l);
            P = __builtin_amdgcn_readlane(kr, l);
            found = true;
        }
        base += gsum;
    }
    return found;
}

template <int PF, int kMode, bool kBal, int kWaves>
__global__ void __launch_bounds__(64 * kWaves)
lookup_scan_kernel(ScanOut out_arg, const int32_t *__restrict__ hist,
                   const int64_t *__restrict__ row_off, const int32_t *__restrict__ len,
                   int32_t cpr, int32_t T, ScanArgs a,
                   u64 *__restrict__ ws)
{
    // The lookup's output pointers and the rest of the step's pointers and
    // rules are read from the kernel-argument segment (out_arg is the first
    // argument, at its start) only where they are used, by the waves that use
    // them: as ordinary arguments they were loaded by every wave at entry and
    // held in scalar registers through the scan, which spilled dozens of
    // values into vector lanes ahead of the first tile loads.
    (void)out_arg;
    const ScanOut *op = (const ScanOut *)__builtin_amdgcn_kernarg_segment_ptr();
    __shared__ u64 s_wkey[kWaves];
    __shared__ int s_wtok[kWaves * kSlotWords];
    __shared__ u64 s_units[kMaxCpr * kSlotWords];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uni(tid >> 6);   // wave-uniform
    // workgroup = (request r, chunk c0)
    int r, c0;
    if constexpr (kBal) {
        int P_b, T_b;
        if (!balanced_assignment(len, a.B, lane, r, c0, P_b, T_b)) return;
        r = uni(r);
        c0 = uni(c0);
        cpr = uni(P_b);               // this row's chunks: one workgroup each
        T = uni(T_b);
    } else {
        r = (int)(blockIdx.x / (unsigned)cpr);
        c0 = (int)blockIdx.x - r * cpr;
        // 4-wave launches: a row's chunks in an order rotated by the row, so
        // that the first chunks of short rows (their only busy workgroups)
        // are spread over the XCDs (workgroup i runs on XCD i mod 8) instead
        // of landing on the same one whenever 8 divides cpr x (row distance)
        if (kWaves == kWavesSmall) c0 = (int)(((unsigned)c0 + (unsigned)r) % (unsigned)cpr);
    }
    // the row's offset and length first: every tile load waits on them (wave
    // 0's step inputs below would otherwise go out ahead of them)
    const int64_t ro = row_off[r];
    const int32_t lr = len[r];
    int sin = 0;
    uint32_t tin = 0;                 // the request's telemetry row, lane k: counter k
    // 16-wave workgroups: word k of the first argument (the outputs and the
    // step's pointers and rules) in lane k, loaded now so that the finish
    // reads them from a register instead of waiting on one argument load
    // after another (0.1 us at 64 x 25k).  4-wave workgroups, many more per
    // launch, read them at the finish: the extra load in front of wave 0's
    // tiles cost them more (0.4 us at 256 ragged rows).
    constexpr bool kArgsInLanes = kWaves == kWavesLarge;
    int outv = 0;
    if (kArgsInLanes && wave == 0) outv = reinterpret_cast<const int *>(op)[lane < kOutWords ? lane : 0];
    auto outputs = [&]() -> ScanOut {
        if constexpr (kArgsInLanes) return from_lanes<ScanOut>(outv);
        else return *op;
    };
    if (kMode == kStep && wave == 0) {
        const StepIO io0 = op->io;
        sin = load_step_input(r, lane, io0);
        if (io0.tele != nullptr)
            tin = io0.tele[(int64_t)r * LCD_TELE_WORDS + (lane & (LCD_TELE_WORDS - 1))];
    }
    const int n = lr > 0 ? lr : 0;
    const int nc = n - 1;             // candidate ends 0..n-2
    if (nc <= 0) {                    // no earlier position: chunk 0 finishes the request
        if (c0 == 0 && wave == 0)
            finish_request<kMode>(r, 0, false, 0, 0, sin, tin, lane, ro, lr, n, a.k_max,
                                  outputs());
        return;
    }
    if ((int64_t)c0 * T >= nc) return;                  // past the row's last chunk
    const int contrib = (int)(((unsigned)nc + (unsigned)T - 1u) / (unsigned)T);
    const int P = contrib < cpr ? contrib : cpr;      // workgroups taking part
    const int J = a.l_max;
    u64 *__restrict__ req = ws + (int64_t)r * kReqWords;
    // Arrival ticket of this workgroup (the header word before its add: the
    // count of earlier arrivals and the call's epoch), taken by lane 0 and
    // read back only at the end (from lane 0): the other lanes' value is left
    // unspecified so that no register copy of the result -- which would wait
    // for it -- is needed here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wsometimes-uninitialized"
#pragma clang diagnostic ignored "-Wuninitialized"
    unsigned long long ticket;
    if (P > 1 && tid == 0)
        ticket = __hip_atomic_fetch_add(req, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // suffix token s_j = h[n-1-j] in lane j (lanes >= 16 repeat s_15, filler 0
    // past the row start); the load is the first in the vector memory queue
    int sv;
    {
        const int js = lane < LCD_MAX_SUFFIX ? lane : LCD_MAX_SUFFIX - 1;
        const int sp = n - 1 - js;
        sv = hist[ro + (sp > 0 ? sp : 0)];
    }

    u64 best = 0;                     // this wave's best key over its chunks
    // lane k < 15: h[e+1+min(k, D-1)], the tokens following the best match
    // (e its end, D = n-1-e); loaded when the match is found, so the load is
    // off the path that follows the scan
    int btok = 0;
    // Tiles of a chunk are handed out inside the workgroup: slot u of wave w
    // starts with tile w + kWaves*u, and every slot refilled after that takes
    // the next tile from this counter (taken one refill ahead), so waves
    // whose loads return early take over the tiles of waves whose loads
    // return late.  A chunk of at most kWaves*kUnroll tiles is all in the
    // first round: no counter.
    __shared__ int s_next;
    // One chunk per workgroup when every row fits in cpr chunks of T; a longer
    // row is covered by letting each workgroup take every cpr-th chunk.
    for (int ch = c0; ch < contrib; ch += cpr) {
        const unsigned seg_a = (unsigned)ch * (unsigned)T;               // < 2^31
        const unsigned seg_b = min(seg_a + (unsigned)T, (unsigned)nc);
        const bool head = (seg_a == 0);                                   // holds the row start

        // Candidate ends of this chunk, as positions relative to X0 (the
        // 16-byte granule holding the first one), and its tiles.
        const int64_t cand_lo = ro + seg_a;
        const int64_t X0 = cand_lo & ~(int64_t)3;
        const int c_lo = (int)(cand_lo - X0);                              // 0..3 (the row start if head)
        const int c_hi = c_lo + (int)(seg_b - seg_a);                      // exclusive
        const int nt = (c_hi + kTileCand - 1) / kTileCand;                 // >= 1
        const int g_last = (c_hi - 1) & ~3;        // last granule with a candidate

        // Tiles are read through a buffer descriptor from the 16 tokens
        // before the chunk's first granule to the last candidate's granule:
        // the hardware range check turns reads past it into zeros (those
        // positions are never candidates), so no load leaves the chunk.  In
        // the head chunk the 16 tokens before the row are not read: those
        // lanes of its first tile re-read the first granule and are masked.
        // (The descriptor's base may then lie before the buffer; nothing is
        // read there.)
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t *>(hist + X0 - kHaloTok), 0, (g_last + 4 + kHaloTok) * 4,
            kBufferWord3);
        // The history is read once: its tiles are loaded non-temporal (the
        // nt cache-policy bit), which keeps the streamed lines from pushing
        // the launch's small per-request data out of the caches (measured:
        // 64 x 150k 11.9 -> 11.3 us, 256 ragged rows 16.8 -> 16.4 us).
        const unsigned lane_off = 16u * (unsigned)lane;
        const unsigned head_off = head ? (unsigned)kHaloTok * 4u : 0u;
        auto load_tile = [&](int kt) -> int4 {
            unsigned off = (unsigned)(kTileCand * 4) * (unsigned)kt + lane_off;
            off = kt < nt ? off : kNoTileOff;
            off = off < head_off ? head_off : off;
            return __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, kLoadNT));
        };
        int idx[kUnroll];
        int4 buf[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            idx[u] = wave + kWaves * u;
            buf[u] = load_tile(idx[u]);
        }
        // the counter of this chunk: every wave is done with the last one's
        const bool dyn = nt > kWaves * kUnroll;
        if (dyn) {
            if (ch != c0) lds_barrier();
            if (tid == 0) s_next = 0;
            lds_barrier();
        }

        // The suffix is needed now; the empty asm keeps its lane reads here,
        // behind the tile loads, instead of hoisted ahead of them.
        asm volatile("" : "+v"(sv));
        sv = lane < n ? sv : 0;
        int s16[LCD_MAX_SUFFIX];
#pragma unroll
        for (int j = 0; j < LCD_MAX_SUFFIX; ++j) s16[j] = __builtin_amdgcn_readlane(sv, j);
        int s4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) s4[j] = s16[j];
        // a value equal to no suffix token stands in for tokens before the row:
        // one below the smallest, else one above the largest, else searched
        int smin = s16[0], smax = s16[0];
#pragma unroll
        for (int j = 1; j < LCD_MAX_SUFFIX; ++j) {
            smin = s16[j] < smin ? s16[j] : smin;
            smax = s16[j] > smax ? s16[j] : smax;
        }
        int sent = smin != INT32_MIN ? smin - 1 : smax + 1;
        if (smin == INT32_MIN && smax == INT32_MAX) {
            sent = INT32_MIN + 1;
            for (int it = 0; it <= LCD_MAX_SUFFIX; ++it) {
                bool hit = false;
#pragma unroll
                for (int j = 0; j < LCD_MAX_SUFFIX; ++j) hit |= (s16[j] == sent);
                if (!hit) break;
                ++sent;
            }
        }

        if (wave < nt) {
            // The head chunk's first tile is wave 0's first: its lanes before
            // the row start become `sent`.
            if (head && wave == 0) buf[0] = mask_head(buf[0], lane, c_lo, sent);
            // Quick test.  A candidate end e needs h[e-j] == s_j for every
            // j < PF; with PF >= 2 it needs in particular the adjacent pair
            // s_j at p = e-j and s_{j+1} at p-1, both inside e's tile.  So a
            // tile can hold a candidate only if it holds such a pair.  Each
            // wave picks the pair that is rarest in its first tile; the choice
            // only changes how many tiles get the full test, never the result.
            // Pairs, unlike single tokens, stay rare when every suffix token
            // is a common one.  (PF = 1: the single token s_0.)
            int cnt[4] = {0, 0, 0, 0};
            {
                const int4 t = buf[0];
#pragma unroll
                for (int j = 0; j < PF; ++j)
                    cnt[j] = __popcll(ballot(t.x == s4[j])) + __popcll(ballot(t.y == s4[j])) +
                             __popcll(ballot(t.z == s4[j])) + __popcll(ballot(t.w == s4[j]));
            }
            int jp = 0;
            if (PF >= 2) {
                int fewest = 1 << 30;
#pragma unroll
                for (int j = 0; j + 1 < PF; ++j) {
                    const int score = cnt[j] * cnt[j + 1] + cnt[j] + cnt[j + 1];
                    if (score < fewest) { fewest = score; jp = j; }
                }
            }
            const int sa = uni(jp == 0 ? s4[0] : jp == 1 ? s4[1] : s4[2]);                   // s_jp
            const int sb = uni(PF >= 2 ? (jp == 0 ? s4[1] : jp == 1 ? s4[2] : s4[3]) : s4[0]);  // s_jp+1
            // pair hits of tile t (bit i: a pair whose later token p lies in lane i)
            auto quick = [&](const int4 &t) -> u64 {
                if (PF < 2)
                    return (ballot(t.x == sa) | ballot(t.y == sa) | ballot(t.z == sa) | ballot(t.w == sa)) &
                           kCandLanes;
                const u64 a0 = ballot(t.x == sa), a1 = ballot(t.y == sa);
                const u64 a2 = ballot(t.z == sa), a3 = ballot(t.w == sa);
                const u64 b0 = ballot(t.x == sb), b1 = ballot(t.y == sb);
                const u64 b2 = ballot(t.z == sb), b3 = ballot(t.w == sb);
                return ((a1 & b0) | (a2 & b1) | (a3 & b2) | (a0 & (b3 << 1))) & kPairLanes;
            };
            // A wave whose pair turns out to be common stops running the quick
            // test after kFullAfter flagged tiles and gives every tile the
            // full test (which the quick test would have passed anyway).
            int nflag = 0;
            auto test_tile = [&](const int4 &t, int kt) {
                bool flagged = true;
                if (nflag < kFullAfter) flagged = quick(t) != 0;
                if (flagged) {
                    ++nflag;
                    u64 P4[4];
                    survivors<PF>(t, s4, kt, c_lo, c_hi, lane, P4);
                    if ((P4[0] | P4[1] | P4[2] | P4[3]) != 0) {
                        const int L = extend<PF>(t, sv, J, P4);
                        if (L >= a.l_min) {
                            int ebest = -1;
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                if (P4[c] != 0) {
                                    const int e = 4 * (63 - __clzll(P4[c])) + c;
                                    ebest = e > ebest ? e : ebest;
                                }
                            }
                            const int64_t e_abs = X0 + kTileCand * (int64_t)kt + ebest - kHaloTok;
                            const u64 key = ((u64)L << kLenShift) | (u64)(uint32_t)(e_abs - ro);
                            if (key > best) {
                                best = key;
                                const int D = nc - (int)(e_abs - ro);     // n-1-e >= 1
                                btok = hist[e_abs + 1 + (lane < D ? lane : D - 1)];
                            }
                        }
                    }
                }
            };
            // Each wave keeps kUnroll tiles in flight: a slot is refilled as
            // soon as its tile has been tested, with the tile taken from the
            // counter one refill earlier (a tile past the chunk points outside
            // the descriptor: zeros, no memory access).  The tiles a wave
            // takes only grow, so once slot 0 holds none, no slot does.
            auto take = [&]() -> int {
                int v = 0;
                if (lane == 0)
                    v = __hip_atomic_fetch_add(&s_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                return v;
            };
            if (dyn) {
                int pend = take();
                for (;;) {
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u) {
                        if (idx[u] < nt) test_tile(buf[u], idx[u]);
                        const int nx = uni(pend) + kWaves * kUnroll;
                        idx[u] = nx;
                        buf[u] = load_tile(nx);
                        pend = take();
                    }
                    if (idx[0] >= nt) break;
                }
            } else {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    if (idx[u] < nt) test_tile(buf[u], idx[u]);
            }
        }
        // Nothing is in flight here; saying so keeps the compiler from waiting
        // on the next chunk's loads for registers this chunk's loads used.
        __builtin_amdgcn_s_waitcnt(0);
    }

    // The workgroup's best key: each wave's key with its index in the low 4
    // bits (keys of different waves differ unless zero), reduced by wave 0
    // across lanes in one DPP row pass; the winner's staged tokens from LDS.
    if (lane == 0) s_wkey[wave] = (best << 4) | (u64)wave;
    if (lane < kSlotWords) s_wtok[wave * kSlotWords + lane] = btok;
    __syncthreads();
    if (wave != 0) return;
    const u64 kw = readlane64(row_max64(lane < kWaves ? s_wkey[lane] : 0ull), 15);
    u64 key = kw >> 4;
    int tok = s_wtok[(int)(kw & 15) * kSlotWords + (lane < kSlotWords ? lane : 0)];
    if (P > 1) {
        u64 *__restrict__ slots = req + 2;
        // lane 0 took the ticket (P > 1): the arrival count and the call's tag
        const u64 hdr = ((u64)(uint32_t)__builtin_amdgcn_readfirstlane((int)(ticket >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)ticket);
#pragma clang diagnostic pop
        const u64 tag = call_tag(hdr);
        if ((int)(uint32_t)hdr != P - 1) {          // not the last to start: publish, leave
            const u64 unit = lane < kSlotWords - 1 ? ((tag << 32) | (u64)(uint32_t)tok) : ((tag << 36) | key);
            if (lane < kSlotWords)
                __hip_atomic_store(slots + c0 * kSlotWords + lane, unit, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        // Last to start: every other workgroup taking part has started, and
        // publishes without waiting for anything, so the gathering ends.  Its
        // own key and tokens stay in registers.  Up to 4 slots (64 words)
        // are polled one word per lane and kept in registers; more go
        // through LDS.
        const int nu = P * kSlotWords;
        const bool in_regs = nu <= 64;
        const bool is_key = (lane & (kSlotWords - 1)) == kSlotWords - 1;
        u64 v0 = 0;
        bool all = false;
        for (int tries = 0; tries < a.polls && !all; ++tries) {
            bool ok = true;
            if (in_regs) {
                if (lane < nu && lane / kSlotWords != c0) {
                    v0 = __hip_atomic_load(slots + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ok = (v0 >> (is_key ? 36 : 32)) == tag;
                }
            } else {
                // the loads of a batch of up to 32 slots all in flight before
                // the first is used (a loop that consumed each word before
                // loading the next waited one round trip per 64 words)
                for (int k0 = 0; 64 * k0 < nu; k0 += kPollBatch) {
                    u64 pv[kPollBatch];
#pragma unroll
                    for (int k = 0; k < kPollBatch; ++k) {
                        const int u = lane + 64 * (k0 + k);
                        pv[k] = 0;
                        if (64 * (k0 + k) < nu && u < nu && u / kSlotWords != c0)
                            pv[k] = __hip_atomic_load(slots + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
#pragma unroll
                    for (int k = 0; k < kPollBatch; ++k) {
                        const int u = lane + 64 * (k0 + k);
                        if (64 * (k0 + k) < nu && u < nu && u / kSlotWords != c0) {
                            s_units[u] = pv[k];
                            ok = ok && ((pv[k] >> (is_key ? 36 : 32)) == tag);
                        }
                    }
                }
            }
            all = ballot(!ok) == 0;
        }
        // best key over the slots (keys of different slots differ unless
        // zero): a scalar pass over the P slot keys, which are few
        const u64 kKeyMask = (1ull << 36) - 1;
        u64 kbest = 0;
        int w = c0;
        if (in_regs) {
            for (int j = 0; j < P; ++j) {
                const u64 kj = j == c0 ? key : (readlane64(v0, j * kSlotWords + kSlotWords - 1) & kKeyMask);
                if (kj > kbest) { kbest = kj; w = j; }
            }
        } else {
            const u64 ks = lane >= P ? 0
                           : lane == c0 ? key
                                        : (s_units[lane * kSlotWords + kSlotWords - 1] & kKeyMask);
            for (int j = 0; j < P; ++j) {
                const u64 kj = readlane64(ks, j);
                if (kj > kbest) { kbest = kj; w = j; }
            }
        }
        if (kbest == 0) w = c0;
        // the winner's tokens: own (in tok), in the polled words, or in LDS
        int src = tok, base = 0;
        if (w != c0) {
            if (in_regs) {
                src = (int)(uint32_t)v0;
                base = w * kSlotWords;
            } else {
                src = (int)(uint32_t)s_units[w * kSlotWords + (lane < kSlotWords - 1 ? lane : 0)];
            }
        }
        finish_request<kMode>(r, kbest, !all, src, base, sin, tin, lane, ro, lr, n, a.k_max,
                              outputs());
        // Re-zero the slots for the next call (after the outputs: a wait for
        // these stores' acknowledgement must not sit in front of the finish),
        // unless the gathering gave up: a late publisher may still write into
        // them, and its words keep this call's tag, which no later call takes.
        if (all)
            for (int u = lane; u < nu; u += 64)
                __hip_atomic_store(slots + u, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) __hip_atomic_store(req, next_header(hdr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    finish_request<kMode>(r, key, false, tok, 0, sin, tin, lane, ro, lr, n, a.k_max,
                          outputs());
}

// Workgroups per request.  By default one workgroup per ~12k tokens of the
// batch's size bound B x max_len, at least 256 and at most 4 dispatch rounds
// (4 x 7 x 256) per launch, with chunks of at least 2048 and at most 32768
// tokens of the longest row.  Large batches take several rounds: with equal
// chunks the long rows' chunks are the critical path, so they are kept short,
// and the workgroups past a short row's end leave at once -- but not for free,
// hence the cap.  Measured (with the rotated chunk order): 256 rows of 1k-262k
// tokens 16.7 us against 19.4 us held to one round (1,792 workgroups); 256 x
// 262k 52.5 against 57.5 us; one 1M-token row among 255 of 8k, 12.8 us at the
// cap against 14.9 us at 16,384 workgroups; 200 x 150k and 256 x 53.6k even.
int pick_cpr(int32_t B, int32_t max_len, int32_t scan_wgs) {
    int64_t cpr;
    if (scan_wgs > 0) {
        cpr = scan_wgs / B;
    } else {
        int64_t wgs = (int64_t)B * max_len / 12000;
        const int64_t most_wgs = 4 * (int64_t)kResidentSmall * kNumCUs;
        wgs = wgs < 256 ? 256 : (wgs > most_wgs ? most_wgs : wgs);
        cpr = (wgs + B / 2) / B;
        const int64_t most = ((int64_t)max_len + 2047) / 2048;
        const int64_t least = ((int64_t)max_len + 32767) / 32768;
        if (cpr > most) cpr = most;
        if (cpr < least) cpr = least;
    }
    if (cpr < 1) cpr = 1;
    if (cpr > kMaxCpr) cpr = kMaxCpr;
    const int64_t cap = (int64_t(1) << 31) / ((int64_t)B > 0 ? B : 1) - 1;
    if (cpr > cap) cpr = cap;
    return (int)cpr;
}

// Chunk length: the longest row's candidate ends (max_len - 1) split over cpr
// chunks, a multiple of kTileTok, at most kMaxChunk.
int32_t chunk_len(int32_t max_len, int cpr) {
    const int64_t nc = max_len > 1 ? (int64_t)max_len - 1 : 1;
    int64_t T = (nc + cpr - 1) / cpr;
    T = (T + kTileTok - 1) / kTileTok * kTileTok;
    return (int32_t)(T < kMaxChunk ? T : kMaxChunk);
}

template <int PF, int kMode, bool kBal, int kW>
hipError_t launch_one(const int32_t *hist, const int64_t *row_off, const int32_t *len,
                      ScanArgs sa, u64 *ws, int32_t *ml, int32_t *me, int32_t *dr,
                      const StepIO &io, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    const dim3 grid((unsigned)(kBal ? (int64_t)sa.wgs : (int64_t)sa.B * sa.cpr));
    if (ev0 != nullptr || ev1 != nullptr)
        hipExtLaunchKernelGGL(lookup_scan_kernel<PF, kMode, kBal, kW>, grid, dim3(64 * kW), 0u, st,
                              ev0, ev1, 0u, ScanOut{ml, me, dr, io}, hist, row_off, len, sa.cpr, sa.T, sa, ws);
    else
        hipLaunchKernelGGL((lookup_scan_kernel<PF, kMode, kBal, kW>), grid, dim3(64 * kW), 0, st,
                           ScanOut{ml, me, dr, io}, hist, row_off, len, sa.cpr, sa.T, sa, ws);
    return hipGetLastError();
}

template <int PF, int kMode>
hipError_t launch(const int32_t *hist, const int64_t *row_off, const int32_t *len, int32_t B,
                  ScanArgs sa, u64 *ws, int32_t *ml, int32_t *me, int32_t *dr, const StepIO &io,
                  hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    (void)B;
    if (sa.wgs > 0)
        return launch_one<PF, kMode, true, kWavesSmall>(hist, row_off, len, sa, ws, ml, me, dr, io,
                                                        st, ev0, ev1);
    if (sa.waves == kWavesLarge)
        return launch_one<PF, kMode, false, kWavesLarge>(hist, row_off, len, sa, ws, ml, me, dr, io,
                                                         st, ev0, ev1);
    return launch_one<PF, kMode, false, kWavesSmall>(hist, row_off, len, sa, ws, ml, me, dr, io, st,
                                                     ev0, ev1);
}

template <int kMode>
hipError_t launch_scan(int pf, const int32_t *hist, const int64_t *row_off, const int32_t *len,
                       int32_t B, ScanArgs sa, u64 *ws, int32_t *ml, int32_t *me, int32_t *dr,
                       const StepIO &io, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    switch (pf) {
    case 1: return launch<1, kMode>(hist, row_off, len, B, sa, ws, ml, me, dr, io, st, ev0, ev1);
    case 2: return launch<2, kMode>(hist, row_off, len, B, sa, ws, ml, me, dr, io, st, ev0, ev1);
    case 3: return launch<3, kMode>(hist, row_off, len, B, sa, ws, ml, me, dr, io, st, ev0, ev1);
    default: return launch<4, kMode>(hist, row_off, len, B, sa, ws, ml, me, dr, io, st, ev0, ev1);
    }
}

// Workgroups of a token-balanced launch: scan_wgs, or 4 per request within
// [256, kResidentSmall x 256] (on 256 rows of 1k-262k tokens, 4-5 per request measured best:
// fewer, larger chunks amortise each workgroup's start and merge), at least 2
// and at most kMaxCpr per request.
int balanced_wgs(int32_t B, int32_t max_len, int32_t scan_wgs) {
    (void)max_len;
    int64_t g;
    if (scan_wgs > 0) {
        g = scan_wgs;
    } else {
        g = 4 * (int64_t)B;
        g = g < 256 ? 256 : (g > kResidentSmall * kNumCUs ? kResidentSmall * kNumCUs : g);
    }
    if (g < 2 * (int64_t)B) g = 2 * (int64_t)B;
    if (g > (int64_t)kMaxCpr * B) g = (int64_t)kMaxCpr * B;
    return (int)g;
}

ScanArgs scan_shape(int32_t B, int32_t max_len, const lcd_params *p) {
    if (p->scan_balance == 1 && B <= LCD_BALANCE_MAX_B)
        return ScanArgs{0, 0, p->l_min, p->l_max, p->k_max, B, balanced_wgs(B, max_len, p->scan_wgs),
                        kWavesSmall};
    // Batches of 32-128 rows of at least 16k tokens, or of 8k+ tokens when the
    // batch holds 1.2M+ tokens: one 16-wave workgroup per CU (at most 256
    // workgroups, equal chunks per row; a CU holds only one, so a workgroup
    // past 256 would wait for a whole one to finish).  Measured on 64 rows of
    // 25k and 150k tokens: 4 % and 7 % faster than 4-wave workgroups at their
    // best grid; on 100 x 14k and 128 x 12k, 6 % and 3 %; slower on 64 x 14k
    // and 128 x 8k.
    if (p->scan_wgs == 0 && B >= 32 && B <= 128 &&
        (max_len >= 16384 || (max_len >= 8192 && (int64_t)B * max_len >= 1200000))) {
        int cpr = kNumCUs / B;
        const int most = (max_len + 2047) / 2048;
        if (cpr > most) cpr = most;
        if (cpr < 1) cpr = 1;
        return ScanArgs{cpr, chunk_len(max_len, cpr), p->l_min, p->l_max, p->k_max, B, 0,
                        kWavesLarge};
    }
    // Smaller batches whose longest row has at least 6k tokens: 16-wave
    // workgroups too, one per ~12k tokens of the longest row, at most 256 in
    // all.  Measured on 1-31 rows of 6k-260k tokens: 6-42 % faster than 4-wave
    // workgroups, and within 10 % of the best fixed count per request on each
    // (at 4k tokens both launches are even).
    if (p->scan_wgs == 0 && B >= 1 && B < 32 && max_len >= 6000) {
        int cpr = (max_len + 6144) / 12288;
        if (cpr > kNumCUs / B) cpr = kNumCUs / B;
        if (cpr > kMaxCpr) cpr = kMaxCpr;
        if (cpr < 1) cpr = 1;
        return ScanArgs{cpr, chunk_len(max_len, cpr), p->l_min, p->l_max, p->k_max, B, 0,
                        kWavesLarge};
    }
    const int cpr = pick_cpr(B, max_len, p->scan_wgs);
    return ScanArgs{cpr, chunk_len(max_len, cpr), p->l_min, p->l_max, p->k_max, B, 0, kWavesSmall};
}

// The launch shape and the bound on the merge's wait (merge_polls: 0 = the
// default, -1 = no poll at all, a diagnostic that makes every merge give up).
ScanArgs scan_args(int32_t B, int32_t max_len, const lcd_params *p) {
    ScanArgs sa = scan_shape(B, max_len, p);
    sa.polls = p->merge_polls == 0 ? kPollMax : (p->merge_polls < 0 ? 0 : p->merge_polls);
    return sa;
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

    const int pf = p->l_min < 4 ? p->l_min : 4;
    const StepIO io{};
    const hipError_t err = launch_scan<kPropose>(pf, hist, row_off, len, B, scan_args(B, max_len, p),
                                                 reinterpret_cast<u64 *>(workspace), match_len,
                                                 match_end, draft, io,
                                                 reinterpret_cast<hipStream_t>(stream), ev0, ev1);
    return err == hipSuccess ? LCD_OK : LCD_EHIP;
}

size_t workspace_bytes(int32_t B) {
    return B > 0 ? (size_t)B * kReqWords * sizeof(u64) : 0;
}

// True when the int32 arrays [a, a+B) and [b, b+B) share an element.
bool overlaps(const int32_t *a, const int32_t *b, int32_t B) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    const uintptr_t bytes = (uintptr_t)B * sizeof(int32_t);
    return x < y + bytes && y < x + bytes;
}

int decode_step(int32_t *hist, const int64_t *row_off, const int32_t *len, int32_t *len_out,
                const int32_t *cap, int32_t B, int32_t max_len, const int32_t *model_draft,
                const int32_t *target, lcd_sched_state *state, const lcd_params *p, void *workspace,
                size_t ws_bytes, int32_t *match_len, int32_t *match_end, int32_t *draft,
                int32_t *block, int32_t *block_len, int32_t *accept, int32_t *long_next,
                uint32_t *tele, int32_t append, void *stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (B < 0 || p == nullptr || max_len < 0) return LCD_EINVAL;
    if (lcd_check_params(p) != LCD_OK) return LCD_EINVAL;
    if (B == 0) return LCD_OK;
    if (!hist || !row_off || !len || !model_draft || !target || !state || !workspace ||
        !match_len || !match_end || !draft || !block || !block_len || !accept)
        return LCD_EINVAL;
    // Appending needs the capacities and a length array apart from the one
    // the launch reads: a workgroup may read a row's length after another
    // workgroup has finished that row.
    if (append && (!cap || !len_out || overlaps(len, len_out, B))) return LCD_EINVAL;
    if (((uintptr_t)hist & 15u) != 0 || ((uintptr_t)workspace & 15u) != 0) return LCD_EINVAL;
    if (ws_bytes < workspace_bytes(B)) return LCD_EINVAL;

    const int pf = p->l_min < 4 ? p->l_min : 4;
    StepIO io{hist, len_out, cap, model_draft, target, state, block, block_len, accept, long_next,
              tele, fuse_args(p), sched_args(p), append ? 1 : 0};
    const hipError_t err = launch_scan<kStep>(pf, hist, row_off, len, B, scan_args(B, max_len, p),
                                              reinterpret_cast<u64 *>(workspace), match_len,
                                              match_end, draft, io,
                                              reinterpret_cast<hipStream_t>(stream), ev0, ev1);
    return err == hipSuccess ? LCD_OK : LCD_EHIP;
}

}  // namespace
}  // namespace lcd

extern "C" size_t lcd_workspace_bytes(int32_t B) { return lcd::workspace_bytes(B); }

extern "C" int lookup_launch_shape(int32_t B, int32_t max_len, const lcd_params *p,
                                   const int32_t *len_host, int32_t *wgs, int32_t *chunk) {
    if (B <= 0 || max_len < 0 || !wgs || !chunk || lcd_check_params(p) != LCD_OK) return LCD_EINVAL;
    const lcd::ScanArgs sa = lcd::scan_args(B, max_len, p);
    if (sa.wgs > 0) {
        if (!len_host) return LCD_EINVAL;
        int64_t tot = 0, mx = 0;
        for (int32_t r = 0; r < B; ++r) {
            const int64_t nc = len_host[r] > 1 ? (int64_t)len_host[r] - 1 : 0;
            tot += nc;
            mx = nc > mx ? nc : mx;
        }
        *wgs = sa.wgs;
        *chunk = lcd::balanced_chunk_len(tot, mx, sa.wgs, B);
    } else {
        *wgs = sa.B * sa.cpr;
        *chunk = sa.T;
    }
    return LCD_OK;
}

namespace lcd {
namespace {
// Fewest workgroups of `kW` waves per CU over the scan's instances (every
// prefilter width and mode; both chunkings for 4-wave workgroups).
template <int kW>
hipError_t min_occupancy(int *out) {
    int best = 1 << 30;
    hipError_t err = hipSuccess;
    auto take = [&](const void *fn) {
        int n = 0;
        const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 64 * kW, 0);
        if (e != hipSuccess) err = e;
        else best = n < best ? n : best;
    };
#define LCD_OCC(PF)                                                                          \
    take(reinterpret_cast<const void *>(&lookup_scan_kernel<PF, kPropose, false, kW>));     \
    take(reinterpret_cast<const void *>(&lookup_scan_kernel<PF, kStep, false, kW>));        \
    if constexpr (kW == kWavesSmall) {                                                       \
        take(reinterpret_cast<const void *>(&lookup_scan_kernel<PF, kPropose, true, kW>));  \
        take(reinterpret_cast<const void *>(&lookup_scan_kernel<PF, kStep, true, kW>));     \
    }
    LCD_OCC(1) LCD_OCC(2) LCD_OCC(3) LCD_OCC(4)
#undef LCD_OCC
    *out = best;
    return err;
}
}  // namespace
}  // namespace lcd

extern "C" int lookup_scan_occupancy(int32_t waves, int32_t *workgroups_per_cu) {
    if (!workgroups_per_cu || (waves != lcd::kWavesSmall && waves != lcd::kWavesLarge))
        return LCD_EINVAL;
    int n = 0;
    const hipError_t err = waves == lcd::kWavesSmall ? lcd::min_occupancy<lcd::kWavesSmall>(&n)
                                                     : lcd::min_occupancy<lcd::kWavesLarge>(&n);
    if (err != hipSuccess) return LCD_EHIP;
    *workgroups_per_cu = n;
    return LCD_OK;
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
    (void)max_len;
    return p != nullptr ? lcd::workspace_bytes(B) : 0;
}

extern "C" int lookup_decode_step(int32_t *hist, const int64_t *row_off, const int32_t *len,
                                  int32_t *len_out, const int32_t *cap, int32_t B, int32_t max_len,
                                  const int32_t *model_draft, const int32_t *target,
                                  lcd_sched_state *state, const lcd_params *p, void *workspace,
                                  size_t workspace_bytes, int32_t *match_len, int32_t *match_end,
                                  int32_t *draft, int32_t *block, int32_t *block_len,
                                  int32_t *accept, int32_t *long_next, uint32_t *telemetry,
                                  int32_t append, void *stream) {
    return lcd::decode_step(hist, row_off, len, len_out, cap, B, max_len, model_draft, target, state, p,
                            workspace, workspace_bytes, match_len, match_end, draft, block,
                            block_len, accept, long_next, telemetry, append, stream, nullptr,
                            nullptr);
}

extern "C" int lookup_decode_step_timed(int32_t *hist, const int64_t *row_off, const int32_t *len,
                                        int32_t *len_out, const int32_t *cap, int32_t B,
                                        int32_t max_len,
                                        const int32_t *model_draft, const int32_t *target,
                                        lcd_sched_state *state, const lcd_params *p,
                                        void *workspace, size_t workspace_bytes,
                                        int32_t *match_len, int32_t *match_end, int32_t *draft,
                                        int32_t *block, int32_t *block_len, int32_t *accept,
                                        int32_t *long_next, uint32_t *telemetry, int32_t append,
                                        void *stream, void *ev_start, void *ev_stop) {
    return lcd::decode_step(hist, row_off, len, len_out, cap, B, max_len, model_draft, target, state, p,
                            workspace, workspace_bytes, match_len, match_end, draft, block,
                            block_len, accept, long_next, telemetry, append, stream,
                            reinterpret_cast<hipEvent_t>(ev_start),
                            reinterpret_cast<hipEvent_t>(ev_stop));
}

// ---------------------------------------------------------------------------
// lookup_decode_step_noalloc: the decode step with its workspace in a static
// device array, for callers that cannot allocate.  Each GPU the library runs
// on holds its own copy of `scratch` (LCD_NOALLOC_MAX_B requests' workspace,
// 8.0 MiB) until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: its device address is taken once per
// device with hipGetSymbolAddress and only that address is passed on.
// ---------------------------------------------------------------------------
namespace lcd {
namespace {

constexpr int64_t kNoallocWords = (int64_t)LCD_NOALLOC_MAX_B * kReqWords;
static __device__ __align__(256) u64 scratch[kNoallocWords];

constexpr int kMaxDevices = 64;

__global__ void __launch_bounds__(256) zero_words_kernel(u64 *__restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0;
}

struct ScratchTable {
    std::once_flag once[kMaxDevices];
    void *ptr[kMaxDevices] = {};
    hipError_t err[kMaxDevices] = {};
};

ScratchTable &scratch_table() {
    static ScratchTable t;
    return t;
}

// The current device's copy of `scratch`, set up on the first call on that
// device: its address, then one zero fill on the caller's stream (ordered
// before this call's kernel; the array is left valid by every call after).
void *device_scratch(hipStream_t st) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    ScratchTable &t = scratch_table();
    std::call_once(t.once[dev], [&] {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e == hipSuccess) {
            hipLaunchKernelGGL(zero_words_kernel, dim3(1024), dim3(256), 0, st,
                               static_cast<u64 *>(ptr), kNoallocWords);
            e = hipGetLastError();
        }
        t.err[dev] = e;
        t.ptr[dev] = e == hipSuccess ? ptr : nullptr;
    });
    return t.ptr[dev];
}

}  // namespace
}  // namespace lcd

extern "C" int lookup_decode_step_noalloc(int32_t *hist, const int64_t *row_off, const int32_t *len,
                                          int32_t *len_out, const int32_t *cap, int32_t B,
                                          int32_t max_len, const int32_t *model_draft,
                                          const int32_t *target, lcd_sched_state *state,
                                          const lcd_params *p, int32_t *match_len,
                                          int32_t *match_end, int32_t *draft, int32_t *block,
                                          int32_t *block_len, int32_t *accept, int32_t *long_next,
                                          uint32_t *telemetry, int32_t append, void *stream) {
    if (B < 0 || B > LCD_NOALLOC_MAX_B) return LCD_EINVAL;
    if (B == 0) return lcd_check_params(p) == LCD_OK ? LCD_OK : LCD_EINVAL;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    void *ws = lcd::device_scratch(st);
    if (ws == nullptr) return LCD_EHIP;
    return lcd::decode_step(hist, row_off, len, len_out, cap, B, max_len, model_draft, target, state,
                            p, ws, (size_t)lcd::kNoallocWords * sizeof(lcd::u64), match_len,
                            match_end, draft, block, block_len, accept, long_next, telemetry,
                            append, stream, nullptr, nullptr);
}

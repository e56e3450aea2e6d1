/*
 * lcd.h -- C ABI of the context-lookup drafting hot path for AMD Instinct
 * MI355X (gfx950).
 *
 * Method source: the HyperQwen lookup-drafting article (page titled
 * "HyperQwen 上下文复述加速：lookup 草稿如何把 25k 文档复读推到 381 tok/s"),
 * sections "第 1 步" (lookup), "第 2 步" (fusion), "第 3 步" (long-block
 * scheduling) and its closing paragraph on losslessness (greedy verification).
 *
 * Every entry point handles a batch of B independent requests, runs
 * asynchronously on the caller's HIP stream and allocates nothing: all arrays
 * are DEVICE memory allocated and owned by the caller, only `p` is read on the
 * host at call time.  `stream` is a hipStream_t (NULL = the null stream).
 *
 * Token ids are opaque int32 values; LCD_PAD (-1) marks an empty draft or block
 * slot and is never produced by the lookup from a history of non-negative ids.
 *
 * Return values: LCD_OK on success; LCD_EINVAL for host-checkable misuse
 * (B < 0, a NULL array with B > 0, a misaligned pointer where alignment is
 * required, parameters out of range) -- nothing is launched; LCD_EHIP when the
 * HIP runtime reports a launch error.  B == 0 is a no-op returning LCD_OK.
 * Errors in device data cannot be seen by the host: lengths are clamped at 0,
 * an append that would overflow a row's capacity is reported per request
 * (accept = -1) without writing, and a lookup whose cross-workgroup merge gave
 * up waiting (see merge_polls) is reported per request as match_len = -1.
 */
#ifndef LCD_H
#define LCD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCD_PAD (-1)
#define LCD_DRAFT_STRIDE 15   /* int32 per row of draft[] and block[] */
#define LCD_Q_STRIDE 7        /* int32 per row of the draft-model proposal */
#define LCD_TARGET_STRIDE 16  /* int32 per row of the target argmax tokens */
#define LCD_MAX_SUFFIX 16     /* largest supported l_max */

#define LCD_OK 0
#define LCD_EINVAL (-1)
#define LCD_EHIP (-2)

/*
 * Method parameters (defaults from lcd_default_params = the article's values).
 *   l_min, l_max  suffix lengths searched, 1 <= l_min <= l_max <= 16 (4, 12)
 *   k_max         drafted tokens per lookup, 0..15 (15)
 *   n_head        draft-model proposal length = short block, 1..7 (7)
 *   n_block       draft slots of a long block, n_head..15 (15; 7 disables it)
 *   head_full     match length replacing the head outright, >= 1 (8)
 *   head_agree    shorter match length replacing the head when the draft model
 *                 agrees on its first agree_n slots, >= 1 (6)
 *   agree_n       0..n_head (2)
 *   tail_min      match length filling the tail of a long block, >= 1 (4)
 *   entry_steps   consecutive flagged steps needed to enter long mode, >= 1 (2)
 *   sticky        flag-down steps tolerated in long mode, >= 0 (3)
 *   near_full_slack  a step is "nearly full" when accept >= blk - slack, >= 0 (1)
 *   scan_wgs      launch tuning of the scan (lookup_propose, lookup_decode_step):
 *                 workgroups of 4 waves per launch; 0 = automatic (16-wave
 *                 workgroups, at most 256, for batches of 32-128 rows whose
 *                 longest row has 16k+ tokens, or 8k+ with B x max_len of
 *                 1.2M+, and of 1-31 rows whose longest row has 6k+ tokens;
 *                 4-wave workgroups otherwise, about one per 12k tokens of
 *                 B x max_len, at most 7168, except that each row gets
 *                 enough of them (up to 64) for chunks of at most 32,768
 *                 tokens of the longest row).  Results never depend on it.
 *   scan_balance  launch tuning of the scan (lookup_propose, lookup_decode_step)
 *                 for ragged batches: 1 = chunks of equal token count, sized on
 *                 the device from the rows' lengths, so long rows get more
 *                 workgroups than short ones (B <= LCD_BALANCE_MAX_B; larger
 *                 batches use equal chunks per row); 0 = every row is cut into
 *                 the same number of chunks, sized from max_len.  1 pays where
 *                 one row is far longer than very many short ones; elsewhere
 *                 the automatic launch is faster.  Results never depend on it.
 *   merge_polls   diagnostics: how often the workgroup that completes a
 *                 request's lookup polls the other workgroups' results before
 *                 it gives up (0 = the default, 2^20; -1 = not at all, which
 *                 makes every request scanned by several workgroups give up).
 *                 The wait always ends in practice -- every workgroup polled
 *                 for has started and publishes without waiting -- so the
 *                 bound is a safety net; a request whose merge gave up
 *                 reports match_len = -1 (an error, not a lookup result).
 *   index_load    incremental index (lookup_index_plan): table slots per
 *                 indexed length and token of capacity, 2..16 (3).
 */
typedef struct lcd_params {
    int32_t l_min, l_max, k_max;
    int32_t n_head, n_block;
    int32_t head_full, head_agree, agree_n, tail_min;
    int32_t entry_steps, sticky, near_full_slack;
    int32_t scan_wgs;
    int32_t scan_balance;
    int32_t merge_polls;
    int32_t index_load;
} lcd_params;

/* Largest batch the token-balanced scan (scan_balance = 1) handles. */
#define LCD_BALANCE_MAX_B 1024

/* Per-request scheduler state, caller-owned (device), start at {0,0,0}. */
typedef struct lcd_sched_state {
    int32_t long_mode, streak, down;
} lcd_sched_state;

/* Fills *p with the defaults above. */
void lcd_default_params(lcd_params *p);

/* Returns LCD_OK when *p is in range, LCD_EINVAL otherwise (host only). */
int lcd_check_params(const lcd_params *p);

/* Device workspace per request: a header word (arrival count and call epoch),
 * a pad word and one 128-byte slot for each of up to 64 workgroups scanning
 * the request. */
#define LCD_WORKSPACE_PER_REQUEST 8208

/* Bytes of device workspace lookup_propose needs for B requests
 * (B * LCD_WORKSPACE_PER_REQUEST).  The workspace must be zero-filled once
 * before its first use and is then kept valid by the calls themselves: each
 * call leaves every arrival count (bits 0..31 of a request's header word) and
 * every slot it gathered at zero, and advances the request's epoch (the
 * header's upper bits), which tags the slots' words so that a call only takes
 * words of its own.  A merge that gave up (match_len = -1) may see its slots
 * written after it returned; their tag is never taken again.  Concurrent calls
 * must not share a workspace. */
size_t lcd_workspace_bytes(int32_t B);

/*
 * lookup_propose -- article, section "第 1 步".
 *
 * For each request r, with h = hist + row_off[r] and n = max(len[r], 0):
 * among candidate ends e in [0, n-2], let ell(e) be the number of tokens,
 * capped at l_max, for which h[e-j] == h[n-1-j] for j = 0, 1, ... while
 * e-j >= 0.  The result is the candidate with the largest ell(e) >= l_min,
 * the latest such e on ties (the longest current suffix of l_min..l_max
 * tokens and its most recent earlier occurrence; the occurrence may overlap
 * the suffix).  Outputs:
 *   match_len[r] = that length m, or 0 when there is none, or -1 when the
 *     merge of the workgroups scanning the row gave up (see merge_polls; the
 *     draft is then all LCD_PAD);
 *   match_end[r] = e (an index into the row), or -1;
 *   draft[r*15 + k] = h[n - D + (k mod D)] for k < k_max with D = n-1-e
 *     (the tokens following the occurrence, copied LZ77-style, so an
 *     overlapping match repeats with period D past the end of the history),
 *     LCD_PAD for k >= k_max or when m == 0.
 *
 * hist      int32 token buffer, 16-byte aligned.  Row r occupies
 *           [row_off[r], row_off[r] + len[r]); rows may be packed (CSR) or
 *           padded.  Reads touch only the 16-byte granules that intersect a row.
 * row_off   int64[B], len int32[B] (read on the device).
 * max_len   an upper bound of len[] used only to size the launch; results are
 *           correct for any value >= 0.
 * workspace lcd_workspace_bytes(B) bytes, 16-byte aligned, see above.
 * match_len, match_end int32[B]; draft int32[B*15].
 */
int lookup_propose(const int32_t *hist, const int64_t *row_off, const int32_t *len,
                   int32_t B, int32_t max_len, const lcd_params *p, void *workspace,
                   int32_t *match_len, int32_t *match_end, int32_t *draft, void *stream);

/*
 * lookup_propose_timed -- for profiling only: the same work and launch
 * configuration as lookup_propose, launched so that the GPU itself stamps the
 * start of the first scan kernel of the call into ev_start and the end of the
 * last one into ev_stop (both hipEvent_t created by the caller, either may be
 * NULL).  The interval excludes host submission time, so it matches a kernel
 * trace of the same launch.
 */
int lookup_propose_timed(const int32_t *hist, const int64_t *row_off, const int32_t *len,
                         int32_t B, int32_t max_len, const lcd_params *p, void *workspace,
                         int32_t *match_len, int32_t *match_end, int32_t *draft, void *stream,
                         void *ev_start, void *ev_stop);

/*
 * fuse_verify_block -- article, section "第 2 步" (fusion, not overwrite).
 *
 * blk = long_mode[r] ? n_block : n_head draft slots are verified.
 * head = (m >= head_full) || (m >= head_agree && q[i] == draft[i] for all
 * i < agree_n).  Slots i < n_head: draft[i] if head and i < k_max, else q[i].
 * Slots n_head <= i < blk (tail, long blocks only): draft[i] if m >= tail_min
 * and i < k_max, else LCD_PAD.  Slots i >= blk: LCD_PAD.
 *
 * model_mask (nullable) gets bit i set for each slot i that keeps the draft
 * model's own token (i < n_head and not replaced by the lookup draft); every
 * other non-PAD slot holds a lookup token.  rejection_accept uses it to pick
 * each slot's proposal distribution.
 *
 * draft int32[B*15], match_len int32[B], model_draft (q) int32[B*7],
 * long_mode int32[B] (non-zero = long block) -> block int32[B*15],
 * block_len int32[B], model_mask uint32[B] (nullable).
 */
int fuse_verify_block(const int32_t *draft, const int32_t *match_len,
                      const int32_t *model_draft, const int32_t *long_mode, int32_t B,
                      const lcd_params *p, int32_t *block, int32_t *block_len,
                      uint32_t *model_mask, void *stream);

/*
 * greedy_accept -- article, closing paragraph (greedy verification never reads
 * the draft distribution); the first rejected slot ends the run.
 *
 * accept[r] = the largest a <= block_len[r] with block[r*15+i] ==
 * target[r*16+i] for every i < a.  The step emits target[r*16 + 0..a]
 * (a+1 tokens).  When hist is non-NULL those a+1 tokens are appended at
 * hist[row_off[r] + n], n = max(len[r], 0), and len[r] becomes n+a+1; if
 * n+a+1 > cap[r] nothing is written for that request and accept[r] = -1.
 * row_off, len and cap are only read when hist is non-NULL.
 *
 * block int32[B*15], block_len int32[B], target int32[B*16],
 * accept int32[B]; hist int32 buffer (nullable), row_off int64[B],
 * len int32[B] (in/out), cap int32[B].
 */
int greedy_accept(const int32_t *block, const int32_t *block_len, const int32_t *target,
                  int32_t B, int32_t *accept, int32_t *hist, const int64_t *row_off,
                  int32_t *len, const int32_t *cap, void *stream);

/*
 * lookup_schedule_step -- article, section "第 3 步" (long block only while a
 * copy is in progress; sticky exit).
 *
 * flag = match_len[r] >= tail_min && accept[r] >= 0 &&
 *        accept[r] >= block_len[r] - near_full_slack.
 * Short mode: streak = flag ? streak+1 : 0; at streak >= entry_steps switch to
 * long mode with streak = down = 0.  Long mode: down = flag ? 0 : down+1; at
 * down > sticky switch to short mode with streak = down = 0.  long_next[r] is
 * the mode of the next step (also written to state[r].long_mode).
 *
 * state lcd_sched_state[B] (in/out), match_len, accept, block_len int32[B],
 * long_next int32[B].
 */
int lookup_schedule_step(lcd_sched_state *state, const int32_t *match_len,
                         const int32_t *accept, const int32_t *block_len, int32_t B,
                         const lcd_params *p, int32_t *long_next, void *stream);

/*
 * lookup_decode_step -- one whole decode step: lookup_propose, then
 * fuse_verify_block under each request's current mode state[r].long_mode, then
 * greedy_accept (appending the emitted tokens when `append` is non-zero), then
 * lookup_schedule_step; every output equals what those four calls produce in
 * that order.  (Article sections "第 1 步" to "第 3 步" and the paragraph on
 * losslessness, as for the four calls.)  One kernel: the workgroups covering a
 * request merge their match keys in `workspace`, and the one whose merge
 * completes the request copies the draft, fuses, accepts, appends and
 * schedules it.  A request whose merge gave up (match_len = -1) is fused,
 * accepted and scheduled as one without a match.
 *
 * hist, row_off, cap        as for lookup_propose / greedy_accept; cap may be
 *                           NULL when append == 0 (then hist is only read)
 * len                       int32[B], the lengths the step reads; never written
 * len_out                   int32[B]; when append != 0 it receives every
 *                           request's length after the step (len[r] + a + 1,
 *                           with len[r] read as max(len[r], 0), or len[r]
 *                           unchanged when the append failed); it must not
 *                           overlap len, because a workgroup may read a row's
 *                           length after another has finished that row -- a
 *                           decode loop alternates two length arrays.  Not
 *                           touched (may be NULL) when append == 0.
 * model_draft int32[B*7], target int32[B*16]
 * state       lcd_sched_state[B], in/out; its long_mode selects this step's block
 * workspace   lcd_decode_step_workspace_bytes(B, max_len, p) bytes (as for
 *             lookup_propose), 16-byte aligned, zero-filled before its first use and
 *             left zero-filled by every completed call; workspace_bytes is its
 *             size, checked.  Concurrent calls must not share it.
 * outputs     match_len, match_end int32[B]; draft, block int32[B*15];
 *             block_len, accept int32[B]; long_next int32[B] (nullable)
 * telemetry   uint32[B * LCD_TELE_WORDS] (nullable), see lookup_telemetry_update
 * Errors: LCD_EINVAL for the misuse lookup_propose rejects, a NULL
 * model_draft, target, state, block, block_len or accept, a workspace smaller
 * than lcd_decode_step_workspace_bytes, or append != 0 with a NULL cap or
 * len_out or a len_out that overlaps len; LCD_EHIP on a launch failure.
 */
size_t lcd_decode_step_workspace_bytes(int32_t B, int32_t max_len, const lcd_params *p);

int lookup_decode_step(int32_t *hist, const int64_t *row_off, const int32_t *len, int32_t *len_out,
                       const int32_t *cap, int32_t B, int32_t max_len, const int32_t *model_draft,
                       const int32_t *target, lcd_sched_state *state, const lcd_params *p,
                       void *workspace, size_t workspace_bytes, int32_t *match_len,
                       int32_t *match_end, int32_t *draft, int32_t *block, int32_t *block_len,
                       int32_t *accept, int32_t *long_next, uint32_t *telemetry,
                       int32_t append, void *stream);

/* lookup_decode_step with GPU-stamped events around its scan kernel (see
 * lookup_propose_timed); for profiling only. */
int lookup_decode_step_timed(int32_t *hist, const int64_t *row_off, const int32_t *len,
                             int32_t *len_out, const int32_t *cap, int32_t B, int32_t max_len,
                             const int32_t *model_draft, const int32_t *target,
                             lcd_sched_state *state, const lcd_params *p, void *workspace,
                             size_t workspace_bytes, int32_t *match_len, int32_t *match_end,
                             int32_t *draft, int32_t *block, int32_t *block_len,
                             int32_t *accept, int32_t *long_next, uint32_t *telemetry,
                             int32_t append, void *stream, void *ev_start, void *ev_stop);

/*
 * lookup_decode_step_noalloc -- lookup_decode_step for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments, results and errors,
 * without the workspace.  The workspace is a static device array inside the
 * library, one per GPU (LCD_NOALLOC_MAX_B requests, 8.0 MiB, held until the
 * process ends), zero-filled by a kernel on `stream` at the first call on a
 * device and left valid by every call.  All calls on one GPU share it: calls
 * that overlap on one GPU (other streams, other threads) race, so a caller
 * orders them.  B > LCD_NOALLOC_MAX_B returns LCD_EINVAL before launching;
 * LCD_EHIP when the array's device address cannot be taken.  Calls no
 * allocating routine.
 */
#define LCD_NOALLOC_MAX_B 1024

int lookup_decode_step_noalloc(int32_t *hist, const int64_t *row_off, const int32_t *len,
                               int32_t *len_out, const int32_t *cap, int32_t B, int32_t max_len,
                               const int32_t *model_draft, const int32_t *target,
                               lcd_sched_state *state, const lcd_params *p, int32_t *match_len,
                               int32_t *match_end, int32_t *draft, int32_t *block,
                               int32_t *block_len, int32_t *accept, int32_t *long_next,
                               uint32_t *telemetry, int32_t append, void *stream);

/*
 * Acceptance telemetry -- the diagnostics the article's forum thread asks to
 * wire up first (hit rate and mean accepted length, with the distribution of
 * accepted lengths), per task class as in the Polish post's test procedure
 * ("Jak testować bez mylenia prędkości z jakością", item 5).
 *
 * telemetry is uint32[B * LCD_TELE_WORDS], device, caller-owned, zeroed by the
 * caller when a session starts.  One decode step adds to request r's row:
 *   LCD_TELE_STEPS        1
 *   LCD_TELE_HITS         1 if m > 0
 *   LCD_TELE_HEAD         1 if the head slots took the lookup draft
 *   LCD_TELE_TAIL         1 if the tail slots took the lookup draft
 *   LCD_TELE_LONG         1 if the step verified a long block
 *   LCD_TELE_ENTRIES      1 if this step was short and the next is long
 *   LCD_TELE_EXITS        1 if this step was long and the next is short
 *   LCD_TELE_EMITTED      a+1 when a >= 0 (tokens the step emits)
 *   LCD_TELE_FAILED       1 if the append failed (a = -1)
 *   LCD_TELE_HIST + i     1 if the step accepted exactly i draft slots, i < 16
 * Counters wrap modulo 2^32.  lookup_decode_step updates it when its
 * `telemetry` argument is non-NULL (nothing is read or written otherwise);
 * lookup_telemetry_update does the same from the outputs of the separate calls
 * (match_len, draft, model_draft, the mode used, block_len, accept, long_next).
 */
#define LCD_TELE_WORDS 32
#define LCD_TELE_STEPS 0
#define LCD_TELE_HITS 1
#define LCD_TELE_HEAD 2
#define LCD_TELE_TAIL 3
#define LCD_TELE_LONG 4
#define LCD_TELE_ENTRIES 5
#define LCD_TELE_EXITS 6
#define LCD_TELE_EMITTED 7
#define LCD_TELE_FAILED 8
#define LCD_TELE_HIST 9

int lookup_telemetry_update(uint32_t *telemetry, const int32_t *match_len, const int32_t *draft,
                            const int32_t *model_draft, const int32_t *long_mode,
                            const int32_t *block_len, const int32_t *accept,
                            const int32_t *long_next, int32_t B, const lcd_params *p,
                            void *stream);

/*
 * Per-class totals: out[k * LCD_TELE_WORDS + c] = sum over requests r with
 * class_id[r] == k of telemetry[r * LCD_TELE_WORDS + c], as uint64, for
 * 0 <= k < K; requests with a class outside [0, K) are left out.  out is
 * uint64[K * LCD_TELE_WORDS], device, overwritten.  One launch.
 */
int lookup_telemetry_reduce(const uint32_t *telemetry, const int32_t *class_id, int32_t B,
                            int32_t K, uint64_t *out, void *stream);

/*
 * Incremental n-gram index: the lookup of lookup_propose answered without
 * scanning the history.  Article, section "第 1 步" (the lookup itself); the
 * forum thread's reply on the method's pitfalls (the lookup index has to be
 * maintained incrementally; a full scan at every step of a long context
 * costs more and more).  Results are identical to lookup_propose's.
 *
 * `tables` begins with 256 bytes per request holding the request's last 48
 * tokens as the last call left them and the row length they end at: a cache
 * the calls keep for themselves (a call whose row length equals the cached
 * one reads its suffix from there, in the same round trip as the length;
 * lookup_index_build clears it).  After those, per request r the index is one
 * hash table of table_slots[r] 8-byte slots at
 * table_off[r] (in slots) inside `tables`, keyed by every L-gram, L in
 * [l_min, l_max], that ends at a position p <= len-2, holding the latest such
 * p; indexed_len[r] (int32, device) is the history length the table covers.
 * Tables are sized exactly: p->index_load slots per indexed length and token
 * of capacity cap[r] (at most 1/index_load of them ever taken), i.e.
 * 8 x index_load x (l_max - l_min + 1) bytes per token of capacity -- 216 at
 * the defaults, 144 with index_load = 2.  Denser tables make longer probe
 * runs; a step reads a window of neighbouring slots per round trip (8 for an
 * insert, 4 for a query), so only runs longer than a window cost another.
 * l_min and l_max must be the same at build and at every propose, and so must
 * fp_bits (fingerprint bits, 1..31, 0 = 31; fewer bits only make fingerprint
 * collisions, and with them the slow path, more frequent).
 */

/*
 * lookup_index_plan -- host only.  Fills table_off[r] and table_slots[r] (in
 * slots) for B rows of capacities cap[r] (host arrays) and returns the total
 * bytes of `tables` (256 x B bytes of token cache, then the tables), or
 * LCD_EINVAL (< 0; also for a table of 2^31 slots or more).
 */
int64_t lookup_index_plan(const int32_t *cap, int32_t B, const lcd_params *p,
                          int64_t *table_off, int32_t *table_slots);

/*
 * lookup_index_build -- clears the tables (table_bytes of them) and indexes
 * every position p <= len[r]-2 of every row; sets indexed_len[r] = max(len[r],
 * 0) (or -1 for a row whose table overflowed).  table_off / table_slots are the
 * plan's arrays, on the device; scratch is int32[B] of device memory;
 * max_len >= every len[r] (launch sizing).  Several launches on `stream`.
 */
int lookup_index_build(const int32_t *hist, const int64_t *row_off, const int32_t *len, int32_t B,
                       const lcd_params *p, int32_t fp_bits, const int64_t *table_off,
                       const int32_t *table_slots, void *tables, size_t table_bytes,
                       int32_t *indexed_len, int32_t *scratch, int32_t max_len, void *stream);

/*
 * lookup_index_propose -- the outputs of lookup_propose (match_len, match_end,
 * draft), from the index.  First indexes the positions appended since the last
 * call (indexed_len[r]-1 .. len[r]-2; histories only grow between calls), then
 * looks up every suffix length at once.  A row whose history got shorter than
 * indexed_len[r], or whose answer a fingerprint collision leaves in doubt, is
 * answered by an exact scan of its history.  A shorter history, and an insert
 * that hit the probe bound (never at the planned load; this call's answer is
 * still exact, the new positions being matched directly), mark the row stale,
 * indexed_len[r] = -1: later calls answer it by scans until it is rebuilt.
 * One launch, one workgroup of two waves per request (one inserts, one looks
 * up), no allocation.
 */
int lookup_index_propose(const int32_t *hist, const int64_t *row_off, const int32_t *len, int32_t B,
                         const lcd_params *p, int32_t fp_bits, const int64_t *table_off,
                         const int32_t *table_slots, void *tables, int32_t *indexed_len,
                         int32_t *match_len, int32_t *match_end, int32_t *draft, void *stream);

/*
 * lookup_index_propose_timed -- for profiling only: lookup_index_propose
 * launched so that the GPU stamps its kernel's start into ev_start and end into
 * ev_stop (hipEvent_t, either may be NULL).
 */
int lookup_index_propose_timed(const int32_t *hist, const int64_t *row_off, const int32_t *len,
                               int32_t B, const lcd_params *p, int32_t fp_bits,
                               const int64_t *table_off, const int32_t *table_slots, void *tables,
                               int32_t *indexed_len, int32_t *match_len, int32_t *match_end,
                               int32_t *draft, void *stream, void *ev_start, void *ev_stop);

/*
 * lookup_index_decode_step -- one whole decode step through the index:
 * lookup_index_propose, then fuse_verify_block under each request's current
 * mode state[r].long_mode, then greedy_accept (appending the emitted tokens
 * when `append` is non-zero), then lookup_schedule_step; every output equals
 * what those four calls produce in that order, and what lookup_decode_step
 * produces.  (Article sections "第 1 步" to "第 3 步" and the paragraph on
 * losslessness; the forum thread's reply on keeping the lookup index
 * incremental.)  One launch, one workgroup of two waves per request: the wave
 * that answers a request's lookup also fuses, accepts, appends and schedules
 * it.  The appended tokens are indexed by the next call, as
 * lookup_index_propose does for any growth of the histories between calls.
 *
 * hist, row_off, cap        as for lookup_decode_step; hist rows must be padded
 *                           (row_off[r] + cap[r] <= row_off[r+1]) when appending
 * len                       int32[B], updated in place when appending (len[r]
 *                           + a + 1, len[r] read as max(len[r], 0); unchanged
 *                           when the append failed): only request r's own
 *                           workgroup reads or writes len[r], so no separate
 *                           output array is needed
 * p, fp_bits, table_off, table_slots, tables, indexed_len
 *                           as for lookup_index_propose (the same index)
 * model_draft, target, state, outputs, telemetry, append
 *                           as for lookup_decode_step
 * Errors: LCD_EINVAL for the misuse lookup_index_propose rejects, a NULL
 * model_draft, target, state, block, block_len or accept, or append != 0 with a
 * NULL cap; LCD_EHIP on a launch failure.  B = 0 is a no-op.  No allocation.
 */
int lookup_index_decode_step(int32_t *hist, const int64_t *row_off, int32_t *len,
                             const int32_t *cap, int32_t B, const lcd_params *p, int32_t fp_bits,
                             const int64_t *table_off, const int32_t *table_slots, void *tables,
                             int32_t *indexed_len, const int32_t *model_draft,
                             const int32_t *target, lcd_sched_state *state, int32_t *match_len,
                             int32_t *match_end, int32_t *draft, int32_t *block,
                             int32_t *block_len, int32_t *accept, int32_t *long_next,
                             uint32_t *telemetry, int32_t append, void *stream);

/* lookup_index_decode_step with GPU-stamped events around its kernel (see
 * lookup_propose_timed); for profiling only. */
int lookup_index_decode_step_timed(int32_t *hist, const int64_t *row_off, int32_t *len,
                                   const int32_t *cap, int32_t B, const lcd_params *p,
                                   int32_t fp_bits, const int64_t *table_off,
                                   const int32_t *table_slots, void *tables, int32_t *indexed_len,
                                   const int32_t *model_draft, const int32_t *target,
                                   lcd_sched_state *state, int32_t *match_len, int32_t *match_end,
                                   int32_t *draft, int32_t *block, int32_t *block_len,
                                   int32_t *accept, int32_t *long_next, uint32_t *telemetry,
                                   int32_t append, void *stream, void *ev_start, void *ev_stop);

/*
 * lookup_scan_occupancy -- diagnostics: workgroups of the scan kernel with
 * `waves` waves (4 or 16) that one compute unit holds at once, as the runtime
 * computes it for the compiled kernels (the fewest over their instances).
 * Automatic launches assume 7 for 4-wave workgroups.  LCD_EINVAL for another
 * wave count or a NULL output, LCD_EHIP when the runtime cannot answer (no GPU).
 */
int lookup_scan_occupancy(int32_t waves, int32_t *workgroups_per_cu);

/*
 * lookup_launch_shape -- host only: the launch of the scan for B rows of at
 * most max_len tokens.  *wgs = workgroups per launch and *chunk = candidate
 * ends per chunk (a multiple of 256).  With scan_balance = 1 (and B <=
 * LCD_BALANCE_MAX_B) the chunk length depends on the rows' lengths: pass them
 * in len_host (host array of B); otherwise len_host may be NULL and every row
 * is cut into *wgs / B chunks.  For measurement (work spread per workgroup).
 * LCD_EINVAL for B <= 0, max_len < 0, bad params, or balance without lengths.
 */
int lookup_launch_shape(int32_t B, int32_t max_len, const lcd_params *p, const int32_t *len_host,
                        int32_t *wgs, int32_t *chunk);

/*
 * lcd_read_probe -- measurement only: a plain streaming read of `bytes`
 * (a multiple of 16, 16-byte aligned device buffer) by `blocks` workgroups of
 * 256 threads, each writing one int32 to out[blocks] (device), in one of the
 * variants below (loads in flight per lane; each workgroup reading one
 * contiguous share, or the workgroups interleaved over blocks of 256 x depth
 * granules), each with plain loads or, with LCD_PROBE_NT or-ed in,
 * non-temporal ones (how the scan and the sampled verification stream).  The GPU stamps the kernel's start and end into ev_start /
 * ev_stop (hipEvent_t, nullable).  The best variant and grid gives the
 * practical HBM read ceiling at a byte count on the running GPU.
 */
#define LCD_PROBE_CONTIG_4 0
#define LCD_PROBE_CONTIG_8 1
#define LCD_PROBE_INTERLEAVE_4 2
#define LCD_PROBE_INTERLEAVE_8 3
#define LCD_PROBE_INTERLEAVE_16 4
#define LCD_PROBE_NT 8
int lcd_read_probe(const void *buf, int64_t bytes, int32_t blocks, int32_t variant, int32_t *out,
                   void *stream, void *ev_start, void *ev_stop);

/*
 * lcd_empty_probe -- measurement only: a kernel of `blocks` workgroups of 256
 * threads that does nothing, with GPU-stamped events as for lcd_read_probe:
 * the floor of one launch (dispatch and completion) on the running GPU.
 */
int lcd_empty_probe(int32_t blocks, void *stream, void *ev_start, void *ev_stop);

/* Largest vocabulary rejection_accept takes (2^22). */
#define LCD_SAMPLE_MAX_VOCAB 4194304

/*
 * rejection_accept_workspace_bytes -- bytes of the rejection_accept workspace
 * for B requests over a vocabulary of V: B * 8 * (2 + ceil(V / 1024)).
 * 0 when B <= 0 or V <= 0.
 */
size_t rejection_accept_workspace_bytes(int32_t B, int32_t V);

/*
 * rejection_accept -- sampled verification with point-mass lookup proposals.
 * Article, closing paragraph on losslessness (for sampled requests each
 * lookup-filled slot is rewritten as a point mass on its token, a legal
 * proposal distribution for speculative rejection sampling, so the output
 * distribution is unchanged); the Polish speculative-decoding post, on
 * verification (the first rejected proposal ends the run).
 *
 * Per request r, slots i < L are verified, L = block_len[r] clamped to 0..15.
 * target_probs[r, i, :] is the target's distribution for the token after the
 * block's first i slots (row L is the bonus row).  Slot i's proposal
 * distribution is model_probs[r, i, :] when model_probs is non-NULL, i < 7 and
 * bit i of model_mask[r] is set (fuse_verify_block's model_mask); otherwise it
 * is the point mass on block[r, i].  Walking i = 0, 1, ...:
 *   - a token that is PAD or outside [0, V) ends the run, nothing proposed;
 *   - with P = p_i(x), Q = q_i(x) (1 for a point mass), the slot is accepted
 *     iff u_accept[r, i] * Q < P, i.e. with probability min(1, P/Q);
 *   - the first rejection ends the run, and the token is drawn from the
 *     residual max(p_i - q_i, 0) (for a point mass: p_i without x);
 *   - a run that ends without a rejection draws from p_a itself.
 * accept[r] = a, the accepted slots; emitted[r] = block[0..a-1], the drawn
 * token, then PAD.
 *
 * Arithmetic (the drawn token is an integer decided by floating point, so it
 * is fixed here): probabilities are read as fp32 clamped into [0, 1] (NaN reads
 * as 0); the acceptance test is in fp64; p - q is an fp32 subtraction, negative
 * results 0; each weight w becomes the integer floor(w * 2^40), their total S
 * is exact, t = floor(u_sample[r] * S / 2^64), and the token is the smallest j
 * whose running total of weights exceeds t.  An all-zero residual falls back to
 * p_a; an all-zero p_a draws nothing: accept[r] = -1 and emitted[r] is all PAD.
 * The result is independent of the launch shape and bit-identical to the plain
 * definition.
 *
 * With hist non-NULL the a+1 emitted tokens are appended exactly as
 * greedy_accept appends the target's tokens (n = max(len[r], 0); if
 * n+a+1 > cap[r] nothing is written and accept[r] = -1, emitted[r] still
 * holding the drawn tokens).
 *
 * block int32[B*15], block_len int32[B], model_mask uint32[B] (nullable),
 * target_probs float32[B*16*V], model_probs float32[B*7*V] (nullable), both
 * 16-byte aligned; u_accept float64[B*15]; u_sample uint64[B] (uniform 64-bit
 * words); accept int32[B]; emitted int32[B*16]; hist / row_off / len / cap as
 * for greedy_accept.  V must be a multiple of 4 in [4, LCD_SAMPLE_MAX_VOCAB]
 * (pad a vocabulary with zero-probability entries).  wg_units: vocabulary
 * units of 1024 per workgroup, 0 = automatic (launch tuning only).
 * workspace: device memory of at least rejection_accept_workspace_bytes(B, V),
 * 8-byte aligned, zero before the first call and then kept valid by the calls
 * (as lookup_propose's: arrival counts and gathered sums back at zero, a call
 * epoch per request that tags the published sums); calls that share a
 * workspace must not overlap.  merge_polls: diagnostics, as lcd_params'
 * merge_polls for the lookup (0 = default 2^20 polls, -1 = none); a request
 * whose gathering gave up reports accept = -1 and emits nothing.  wg_units is
 * at most 256.  Returns LCD_EINVAL for a bad size, alignment, pointer or too
 * small a workspace, before launching.  One launch, no allocation.
 */
int rejection_accept(const int32_t *block, const int32_t *block_len, const uint32_t *model_mask,
                     const float *target_probs, const float *model_probs, int32_t V,
                     const double *u_accept, const uint64_t *u_sample, int32_t B,
                     int32_t wg_units, int32_t merge_polls, void *workspace,
                     size_t workspace_bytes, int32_t *accept, int32_t *emitted, int32_t *hist,
                     const int64_t *row_off, int32_t *len, const int32_t *cap, void *stream);

/*
 * rejection_accept_timed -- for profiling only: rejection_accept launched so
 * that the GPU stamps the kernel's start into ev_start and its end into
 * ev_stop (hipEvent_t, either may be NULL).
 */
int rejection_accept_timed(const int32_t *block, const int32_t *block_len,
                           const uint32_t *model_mask, const float *target_probs,
                           const float *model_probs, int32_t V, const double *u_accept,
                           const uint64_t *u_sample, int32_t B, int32_t wg_units,
                           int32_t merge_polls, void *workspace, size_t workspace_bytes,
                           int32_t *accept, int32_t *emitted, int32_t *hist,
                           const int64_t *row_off, int32_t *len, const int32_t *cap, void *stream,
                           void *ev_start, void *ev_stop);

#ifdef __cplusplus
}
#endif

#endif /* LCD_H */

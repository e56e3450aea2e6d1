"""Seeded synthetic workloads for context-lookup drafting.

This module builds inputs only: int32 token histories, the "true" continuation
of each request, the draft model's 7-token proposals and the target model's
argmax vectors.  It contains none of the method's arithmetic (no suffix search,
no fusion, no acceptance, no scheduling), so both the HIP path and the CPU
oracle can be fed from it without sharing any of the method.

Shapes follow the workloads described on the pages (HyperQwen lookup-drafting
article: a 25k-token document restated verbatim, ordinary writing, 64
concurrent requests, 150k-262k contexts; the draft-vocabulary article: a full
vocabulary of about 248k ids and a 40,960-id draft vocabulary).  None of the
pages' own prompts or documents is reproduced: every token is drawn here.

Random sources
  * numpy ``Generator(PCG64(seed))`` for the histories and truth streams.
  * a counter-based SplitMix64 hash (Steele, Lea & Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014, the ``mix64`` finaliser)
    for the per-step draft-model noise, keyed by (seed, request, step, slot,
    lane), so that any divergence between two backends shows up at the first
    differing step instead of as drifting random streams.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

PAD = -1
N_DRAFT = 15          # draft slots in a long verify block
N_Q = 7               # draft-model proposal length
N_TARGET = 16         # target argmax entries per step (15 slots + bonus)

_M64 = (1 << 64) - 1
_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_C1 = np.uint64(0xBF58476D1CE4E5B9)
_C2 = np.uint64(0x94D049BB133111EB)
# floor(0.6 * 2**53): a 53-bit uniform below this value has probability 0.6.
_AGREE_060 = 5404319552844595


def _mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 step: add the golden gamma, then the variant-13 finaliser."""
    z = (np.asarray(z, dtype=np.uint64) + _GAMMA)
    z = (z ^ (z >> np.uint64(30))) * _C1
    z = (z ^ (z >> np.uint64(27))) * _C2
    return z ^ (z >> np.uint64(31))


def counter_u64(seed, r, t, i, lane) -> np.ndarray:
    """64-bit hash of the counter (seed, request, step, slot, lane)."""
    with np.errstate(over="ignore"):
        z = _mix64(np.uint64(seed & _M64))
        for v in (r, t, i, lane):
            z = _mix64(z ^ np.asarray(v, dtype=np.uint64))
    return z


def zipf_cdf(vocab: int, s: float = 1.1) -> np.ndarray:
    """CDF of the finite Zipf law over ranks 1..vocab, p_k proportional to k^-s."""
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def zipf_tokens(rng: np.random.Generator, n: int, cdf: np.ndarray) -> np.ndarray:
    """n ids drawn by inverse CDF; id = rank - 1."""
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, len(cdf) - 1).astype(np.int32)


def uniform_tokens(rng: np.random.Generator, n: int, vocab: int) -> np.ndarray:
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def draft_model_proposal(truth_window: np.ndarray, seed: int, step: int, vocab: int,
                         p_agree_bits: int = _AGREE_060) -> np.ndarray:
    """Draft-model stand-in: slot i agrees with the truth with probability 0.6.

    ``truth_window`` is [B, >=7] (the true next tokens of each request).  A
    disagreeing slot takes ``(truth + 1 + (u' mod (V-1))) mod V``, which always
    differs from the truth.
    """
    tw = np.asarray(truth_window, dtype=np.int64)[:, :N_Q]
    B = tw.shape[0]
    rid = np.arange(B, dtype=np.uint64)[:, None]
    slot = np.arange(N_Q, dtype=np.uint64)[None, :]
    u0 = counter_u64(seed, rid, np.uint64(step), slot, np.uint64(0))
    u1 = counter_u64(seed, rid, np.uint64(step), slot, np.uint64(1))
    agree = (u0 >> np.uint64(11)) < np.uint64(p_agree_bits)
    off = (u1 % np.uint64(vocab - 1)).astype(np.int64)
    other = (tw + 1 + off) % vocab
    return np.where(agree, tw, other).astype(np.int32)


@dataclasses.dataclass
class Workload:
    """A batch of requests: histories, true continuations and run settings."""

    name: str
    seed: int
    vocab: int
    hists: List[np.ndarray]               # int32 [n_r] each
    truths: List[np.ndarray]              # int32 true continuation of each request
    steps: int                            # decode steps of the run (1 = single step)
    q0: Optional[np.ndarray] = None       # fixed [B,7] proposal (single-step configs)
    target0: Optional[np.ndarray] = None  # fixed [B,16] argmax vector (single-step configs)
    note: str = ""
    classes: Optional[List[str]] = None   # per-request task class ("copy" / "ordinary")

    CLASS_NAMES = ("copy", "ordinary")

    @property
    def class_ids(self) -> np.ndarray:
        """int32 [B]: index of each request's class in CLASS_NAMES."""
        names = self.classes or ["copy"] * self.B
        return np.array([self.CLASS_NAMES.index(c) for c in names], dtype=np.int32)

    @property
    def B(self) -> int:
        return len(self.hists)

    @property
    def lens(self) -> np.ndarray:
        return np.array([len(h) for h in self.hists], dtype=np.int32)

    def step_inputs(self, pos: np.ndarray, step: int):
        """(q [B,7], target [B,16]) for a decode step at truth offsets ``pos``.

        target[r, i] = truth_r[pos_r + i]: the target model's greedy argmax for
        verify position i when every earlier slot was right.  Past the end of a
        truth stream the target repeats its last token (never reached by the
        configured step counts).
        """
        if self.q0 is not None and step == 0 and np.all(pos == 0):
            return self.q0.copy(), self.target0.copy()
        tgt = np.empty((self.B, N_TARGET), dtype=np.int32)
        for r, tr in enumerate(self.truths):
            idx = np.minimum(pos[r] + np.arange(N_TARGET), len(tr) - 1)
            tgt[r] = tr[idx]
        q = draft_model_proposal(tgt, self.seed, step, self.vocab)
        return q, tgt


def pack_rows(hists: List[np.ndarray], extra: int = 0, align: int = 4):
    """Pack histories into one int32 buffer with per-row capacity.

    Row r starts at ``row_off[r]`` (a multiple of ``align`` tokens) and has room
    for ``cap[r] = len_r + extra`` tokens (rounded up to ``align``), so a
    device-side append can grow it.  Returns (flat, row_off int64, len int32,
    cap int32).
    """
    lens = np.array([len(h) for h in hists], dtype=np.int64)
    caps = ((lens + extra + align - 1) // align) * align
    caps = np.maximum(caps, align)
    row_off = np.zeros(len(hists), dtype=np.int64)
    if len(hists) > 1:
        row_off[1:] = np.cumsum(caps)[:-1]
    total = int(caps.sum()) if len(hists) else 0
    flat = np.zeros(max(total, align), dtype=np.int32)
    for r, h in enumerate(hists):
        flat[row_off[r]:row_off[r] + len(h)] = h
    return flat, row_off, lens.astype(np.int32), caps.astype(np.int32)


def pack_csr(hists: List[np.ndarray]):
    """Tightly packed CSR layout: row_off[r+1] = row_off[r] + len_r (no alignment)."""
    lens = np.array([len(h) for h in hists], dtype=np.int64)
    row_off = np.zeros(len(hists), dtype=np.int64)
    if len(hists) > 1:
        row_off[1:] = np.cumsum(lens)[:-1]
    flat = np.concatenate(hists).astype(np.int32) if len(hists) else np.zeros(0, np.int32)
    if flat.size == 0:
        flat = np.zeros(4, dtype=np.int32)
    return flat, row_off, lens.astype(np.int32)


# ---------------------------------------------------------------------------
# The five workloads.  Config k uses seed 1000 + k unless told otherwise.
# ---------------------------------------------------------------------------

def config1(seed: int = 1001) -> Workload:
    """One request of 2,048 uniform ids (vocab 248,320) ending in a planted copy
    and a period-5 run, so that the final lookup must use an overlapping match."""
    V = 248_320
    rng = np.random.Generator(np.random.PCG64(seed))
    h = np.empty(2048, dtype=np.int32)
    h[:1648] = uniform_tokens(rng, 1648, V)
    s = int(rng.integers(0, 1201))
    h[1648:1948] = h[s:s + 300]
    while True:
        pat = uniform_tokens(rng, 5, V)
        if len(set(pat.tolist())) == 5:
            break
    h[1948:2048] = np.tile(pat, 20)
    truth = np.array([pat[i % 5] for i in range(N_TARGET + 64)], dtype=np.int32)
    q0 = uniform_tokens(rng, N_Q, V)[None, :]
    j = int(rng.integers(0, N_TARGET))
    tgt = truth[:N_TARGET].copy()
    tgt[j] = (tgt[j] + 1) % V
    return Workload("c1_single_2k", seed, V, [h], [truth], 1, q0, tgt[None, :],
                    note=f"copy source {s}, mismatch slot {j}", classes=["copy"])


def _copy_request(rng, cdf, V, doc_len, tail_len, truth_len, edit_p=0.0):
    doc = zipf_tokens(rng, doc_len, cdf)
    o = int(rng.integers(0, doc_len - tail_len - truth_len + 1))
    tail = doc[o:o + tail_len].copy()
    truth = doc[o + tail_len:o + tail_len + truth_len].copy()
    if edit_p > 0:
        for arr in (tail, truth):
            hit = rng.random(len(arr)) < edit_p
            arr[hit] = uniform_tokens(rng, int(hit.sum()), V)
    return np.concatenate([doc, tail]).astype(np.int32), truth


def config2(seed: int = 1002) -> Workload:
    """One 25,000-token request: a 24,000-token Zipf(1.1) document over 40,960
    ids followed by a 1,000-token verbatim restatement of a random offset; the
    truth continues the restatement.  200 decode steps."""
    V = 40_960
    rng = np.random.Generator(np.random.PCG64(seed))
    cdf = zipf_cdf(V)
    h, truth = _copy_request(rng, cdf, V, 24_000, 1_000, 4_112)
    return Workload("c2_b1_25k_copy", seed, V, [h], [truth], 200, classes=["copy"])


def config3(seed: int = 1003, steps: int = 256) -> Workload:
    """64 requests of 25,000 tokens: 32 copy-mode (restatement with 5% random
    edits in tail and truth) and 32 ordinary Zipf(1.1) texts with fresh Zipf
    truth.  Vocabulary 40,960.  256 decode steps."""
    V = 40_960
    rng = np.random.Generator(np.random.PCG64(seed))
    cdf = zipf_cdf(V)
    hists, truths = [], []
    tl = N_TARGET * (steps + 1)
    for r in range(64):
        if r < 32:
            h, tr = _copy_request(rng, cdf, V, 24_000, 1_000, tl, edit_p=0.05)
        else:
            h = zipf_tokens(rng, 25_000, cdf)
            tr = zipf_tokens(rng, tl, cdf)
        hists.append(h)
        truths.append(tr)
    return Workload("c3_b64_25k_mixed", seed, V, hists, truths, steps,
                    classes=["copy"] * 32 + ["ordinary"] * 32)


def _plant_periodic_runs(rng, doc, cdf, frac=0.10, p_lo=2, p_hi=8, l_lo=20, l_hi=200):
    """Overwrite about ``frac`` of ``doc`` with non-overlapping periodic runs."""
    n = len(doc)
    want = int(round(frac * n))
    lens, pers = [], []
    tot = 0
    while tot < want:
        L = int(rng.integers(l_lo, l_hi + 1))
        lens.append(L)
        pers.append(int(rng.integers(p_lo, p_hi + 1)))
        tot += L
    free = n - tot
    cuts = np.sort(rng.integers(0, free + 1, size=len(lens)))
    gaps = np.diff(np.concatenate([[0], cuts]))
    start = 0
    for k, (L, P) in enumerate(zip(lens, pers)):
        start += int(gaps[k])
        pat = zipf_tokens(rng, P, cdf)
        doc[start:start + L] = np.resize(pat, L)
        start += L
    return tot


def config4(seed: int = 1004, B: int = 64, n: int = 150_000) -> Workload:
    """64 requests of 150,000 tokens built like the single-request copy case,
    with 10% of document positions in short periodic runs (period 2-8, length
    20-200).  One lookup step."""
    V = 40_960
    rng = np.random.Generator(np.random.PCG64(seed))
    cdf = zipf_cdf(V)
    hists, truths = [], []
    doc_len = n - 1000
    for r in range(B):
        doc = zipf_tokens(rng, doc_len, cdf)
        _plant_periodic_runs(rng, doc, cdf)
        o = int(rng.integers(0, doc_len - 1000 - N_TARGET + 1))
        h = np.concatenate([doc, doc[o:o + 1000]]).astype(np.int32)
        hists.append(h)
        truths.append(doc[o + 1000:o + 1000 + N_TARGET].copy())
    w = Workload("c4_b64_150k_periodic", seed, V, hists, truths, 1, classes=["copy"] * B)
    w.target0 = np.stack(truths).astype(np.int32)
    w.q0 = draft_model_proposal(w.target0, seed, 0, V)
    return w


def config5(seed: int = 1005, B: int = 256) -> Workload:
    """256 ragged requests, lengths log-uniform in [1,024, 262,144], Zipf(1.1)
    over 248,320 ids; half of them end in a verbatim restatement tail of
    2k-20k tokens (clipped so that the copy and its 16-token continuation fit).
    One lookup step."""
    V = 248_320
    rng = np.random.Generator(np.random.PCG64(seed))
    cdf = zipf_cdf(V)
    hists, truths, classes = [], [], []
    for r in range(B):
        n = int(math.floor(math.exp(rng.uniform(math.log(1024), math.log(262_144)))))
        copy = bool(rng.random() < 0.5)
        classes.append("copy" if copy else "ordinary")
        if copy:
            tl = int(rng.integers(2000, 20_001))
            tl = min(tl, (n - N_TARGET) // 2)
            npre = n - tl
            base = zipf_tokens(rng, npre, cdf)
            o = int(rng.integers(0, npre - tl - N_TARGET + 1))
            h = np.concatenate([base, base[o:o + tl]]).astype(np.int32)
            tr = base[o + tl:o + tl + N_TARGET].copy()
        else:
            h = zipf_tokens(rng, n, cdf)
            tr = zipf_tokens(rng, N_TARGET, cdf)
        hists.append(h)
        truths.append(tr)
    w = Workload("c5_b256_ragged", seed, V, hists, truths, 1, classes=classes)
    w.target0 = np.stack(truths).astype(np.int32)
    w.q0 = draft_model_proposal(w.target0, seed, 0, V)
    return w


def make_config(k: int, seed: Optional[int] = None) -> Workload:
    fn = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}[k]
    return fn() if seed is None else fn(seed)


def prefix_batch(h: np.ndarray) -> List[np.ndarray]:
    """Every prefix h[:1], h[:2], ..., h[:n] as its own request."""
    return [h[:k].copy() for k in range(1, len(h) + 1)]


def all_strings(alphabet: int, n: int) -> np.ndarray:
    """Every string of length n over {0..alphabet-1}, as an [alphabet^n, n] array."""
    if n == 0:
        return np.zeros((1, 0), dtype=np.int32)
    idx = np.arange(alphabet ** n, dtype=np.int64)
    out = np.empty((alphabet ** n, n), dtype=np.int32)
    for j in range(n - 1, -1, -1):
        out[:, j] = idx % alphabet
        idx //= alphabet
    return out


# ---------------------------------------------------------------------------
# Sampled verification inputs
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class SampledBatch:
    """Inputs of one sampled verification step for B requests.

    block / block_len / model_mask have the fused verify block's layout (15
    slots, PAD past the verified length, bit i of the mask set for a slot that
    keeps the draft model's token).  target_probs [B,16,V] and model_probs
    [B,7,V] are float32 rows that sum to 1 up to float32 rounding; u_accept
    [B,15] holds float64 uniforms on [0,1) and u_sample [B] uniform 64-bit
    words, the random numbers the verifier consumes."""

    name: str
    seed: int
    V: int
    block: np.ndarray
    block_len: np.ndarray
    model_mask: np.ndarray
    target_probs: np.ndarray
    model_probs: Optional[np.ndarray]
    u_accept: np.ndarray
    u_sample: np.ndarray
    classes: List[str]

    @property
    def B(self) -> int:
        return len(self.block_len)


def _background_rows(rng, n_rows: int, V: int, zipf_w: np.ndarray) -> np.ndarray:
    """n_rows float32 rows: the Zipf profile zipf_w over a different
    pseudo-permutation of the vocabulary per row (token = (rank * a + b) mod V
    with a odd and coprime to V), each row summing to 1."""
    out = np.empty((n_rows, V), np.float32)
    ranks = np.arange(V, dtype=np.int64)
    for i in range(n_rows):
        while True:
            a = int(rng.integers(1, V)) | 1
            if math.gcd(a, V) == 1:
                break
        b = int(rng.integers(0, V))
        out[i, (ranks * a + b) % V] = zipf_w
    return out


def sampled_batch(seed: int = 1006, B: int = 64, V: int = 248_320, with_model: bool = True,
                  name: Optional[str] = None) -> SampledBatch:
    """Half copy-mode requests (long blocks, lookup tokens that the target
    gives most of its mass: 0.75-0.99), half ordinary (short blocks, draft-model
    tokens with target mass 0.02-0.6 and draft-model mass 0.3-0.9).  Every row
    mixes that point mass with a Zipf(1.1) background; bonus rows and PAD slots'
    rows are background only.  Vocabulary 248,320 by default (the full
    vocabulary the pages name); V must be a multiple of 4."""
    assert V % 4 == 0 and V >= 4
    rng = np.random.Generator(np.random.PCG64(seed))
    zw = np.arange(1, V + 1, dtype=np.float64) ** -1.1
    zw = (zw / zw.sum()).astype(np.float32)
    classes = ["copy" if r < (B + 1) // 2 else "ordinary" for r in range(B)]
    block = np.full((B, N_DRAFT), PAD, np.int32)
    block_len = np.zeros(B, np.int32)
    model_mask = np.zeros(B, np.uint32)
    tp = _background_rows(rng, B * N_TARGET, V, zw).reshape(B, N_TARGET, V)
    mp = _background_rows(rng, B * N_Q, V, zw).reshape(B, N_Q, V) if with_model else None
    for r in range(B):
        copy = classes[r] == "copy"
        blk = N_DRAFT if (copy and rng.random() < 0.7) else N_Q
        block_len[r] = blk
        from_model = (not copy) or rng.random() < 0.2        # head kept the draft model's tokens
        if from_model:
            model_mask[r] = (1 << N_Q) - 1
        n_tok = blk if (copy or blk == N_Q) else N_Q          # ordinary long blocks: tail PAD
        block[r, :n_tok] = rng.integers(0, V, n_tok)
        for i in range(n_tok):
            x = int(block[r, i])
            model_slot = bool((model_mask[r] >> i) & 1)
            m = rng.uniform(0.75, 0.99) if (copy and not model_slot) else rng.uniform(0.02, 0.6)
            tp[r, i] *= np.float32(1.0 - m)
            tp[r, i, x] += np.float32(m)
            if mp is not None and model_slot:
                w = rng.uniform(0.3, 0.9)
                mp[r, i] *= np.float32(1.0 - w)
                mp[r, i, x] += np.float32(w)
    u_accept = rng.random((B, N_DRAFT))
    u_sample = rng.integers(0, 2 ** 64, B, dtype=np.uint64)
    return SampledBatch(name or f"sampled_b{B}_v{V}", seed, V, block, block_len, model_mask, tp,
                        mp, u_accept, u_sample, classes)

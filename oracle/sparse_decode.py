"""CPU oracle for one sparse-attention decode step over an int8-scored KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may.  It shares no code with the HIP
library; its inputs come from the seeded generator module, which holds none
of the method's arithmetic.

Everything here is written to be checked by eye against the pages:

[HiP]  "韩国通过卸载键值缓存节约英伟达GPU内存，实现18.95倍解码加速" (news article on
       InfiniteHiP), section "实现 7.24 倍的端到端解码加速": a pruning module cuts
       the sequence into fixed-length chunks, finds in parallel an approximate
       highest-scoring token of each chunk, and passes only the K best chunks
       (K a constant) to the next module; stacked modules refine a
       block-sparse attention mask step by step.  Same section: the offload
       policy is LRU based.
[HCA]  "HCAttention: Extreme KV cache compression via heterogeneous attention
       computing for LLMs" (summary page), sections 摘要, 引言 and HCAttention:
       keys are quantised and kept on the GPU, where they drive a global
       approximate attention scoring; values live in CPU memory and are
       fetched late, for the final aggregation only.
[KVN]  "KV Cache 与长上下文推理", section "KV Cache 回顾": the decode attention
       equation softmax(q K^T / sqrt(d_k)) V over all cached tokens; section
       "KV Cache 压缩技术": the GQA table (query heads share K/V heads), INT8
       key quantisation, and StreamingLLM's sink tokens plus sliding window.

Readings where the pages leave a step open (each is also listed in the
design notes):

* representative of a chunk at stage s: the maximum token score over the
  samples x, x + r_s, x + 2 r_s, ... inside the chunk (offset 0), t < L;
* token score: S_t = Q_j . K8_t with Q_j the sum of the group's int8 query
  vectors (equivalently the sum over the group of int8 dot products);
* int8 codes: symmetric, range [-127, 127], round half to even, one absmax
  scale per (request, KV head) for keys and per (request, query head) for
  the query; the decision is taken in fp32 (the kernel's precision), which
  the tests prove equal to exact rational rounding;
* selection order: score descending, then chunk start ascending; kept
  starts are stored ascending, padded with -1;
* children of a kept chunk: its sub-chunks of the next stage's length
  that start before L;
* attended set: kept last-stage chunks, union sink [0, sigma), union window
  [L - omega, L), each token once;
* exact attention uses the bf16 query and bf16 keys (not the int8 codes)
  in fp64.

Functions with no pin are marked "parity unpinned"; at present there are
none (see tests/test_oracle_pins.py for the pin of each function).
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# bf16 values (bit patterns in uint16) -> exact floats
# --------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact: bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def f64_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 value (ties to even), returned as fp64.

    Used only to state the rounding of an fp32 result; the tolerance test
    compares against the unrounded fp64 output.
    """
    f = np.asarray(x, dtype=np.float32)            # fp64 -> fp32 (RNE)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << np.uint32(16)
    return r.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# O1-O2: key quantisation [HCA 引言, asymmetric K/V: quantised keys on GPU;
#        KVN "KV Cache 压缩技术": INT8 keys]
# --------------------------------------------------------------------------
def key_absmax(k_bits: np.ndarray, length: int) -> np.float32:
    """a = max |K| over the valid rows t < length and all channels of one
    (request, KV head).  Padding rows are excluded."""
    vals = np.abs(bf16_to_f32(k_bits[:length]))
    return np.float32(vals.max()) if vals.size else np.float32(0.0)


def quantize_symmetric(x_bits: np.ndarray, scale: np.float32) -> np.ndarray:
    """code = round_half_even(127 * x / scale) in fp32, code in [-127, 127];
    scale == 0 gives all-zero codes.

    127 * x is exact in fp32 (bf16 has an 8-bit significand), and one
    correctly rounded fp32 division followed by rint equals the exact
    rational rounding (proved in the tests against fractions.Fraction)."""
    if scale == 0:
        return np.zeros(np.shape(x_bits), dtype=np.int8)
    x = np.float32(127.0) * bf16_to_f32(x_bits)
    code = np.rint(x / np.float32(scale))
    return code.astype(np.int8)


def quantize_keys(k_bits: np.ndarray, length: int) -> Tuple[np.ndarray, np.float32]:
    """One (request, KV head): returns (int8 codes of rows < length, a)."""
    a = key_absmax(k_bits, length)
    return quantize_symmetric(k_bits[:length], a), a


def quantize_int4(x_bits: np.ndarray, scale: np.float32) -> np.ndarray:
    """4-bit code = round_half_even(7 * x / scale) in fp32, code in [-7, 7];
    scale == 0 gives all-zero codes.  7 * x is exact in fp32, so as for the
    int8 codes one correctly rounded division and rint give the exact
    rational rounding (proved in the tests)."""
    if scale == 0:
        return np.zeros(np.shape(x_bits), dtype=np.int8)
    x = np.float32(7.0) * bf16_to_f32(x_bits)
    return np.rint(x / np.float32(scale)).astype(np.int8)


def key_sketch4(k_bits: np.ndarray, length: int, stride: int) -> np.ndarray:
    """int4 codes (held as int8 values) of the rows t = 0, stride, 2 stride,
    ... < length of one (request, KV head), with the key scale a of
    quantize_keys: the rows the first pruning stage samples, scored at 4 bits
    (the notes page's INT4 cache quantisation, "KV Cache 压缩技术", applied to
    the scoring keys only)."""
    a = key_absmax(k_bits, length)
    return quantize_int4(k_bits[:length:stride], a)


# --------------------------------------------------------------------------
# O3-O5: query quantisation, group sum, token scores
# [KVN "KV Cache 压缩技术", GQA table: query heads h of one group share KV head j]
# --------------------------------------------------------------------------
def quantize_query(q_bits: np.ndarray) -> np.ndarray:
    """q_bits [Hq][d] -> int8 [Hq][d], one absmax scale per query head."""
    out = np.zeros(q_bits.shape, dtype=np.int8)
    for h in range(q_bits.shape[0]):
        amax = np.float32(np.abs(bf16_to_f32(q_bits[h])).max())
        out[h] = quantize_symmetric(q_bits[h], amax)
    return out


def group_query(q8: np.ndarray, num_kv_heads: int) -> np.ndarray:
    """Q_j = sum of q8_h over the query heads h with h // G == j (int64)."""
    Hq = q8.shape[0]
    G = Hq // num_kv_heads
    Q = np.zeros((num_kv_heads, q8.shape[1]), dtype=np.int64)
    for h in range(Hq):
        Q[h // G] += q8[h].astype(np.int64)
    return Q


def token_scores(Q_j: np.ndarray, k8_rows: np.ndarray) -> np.ndarray:
    """S_t = Q_j . K8_t (exact int64) for the given int8 key rows."""
    return k8_rows.astype(np.int64) @ Q_j.astype(np.int64)


# --------------------------------------------------------------------------
# O6-O9: stacked pruning stages [HiP "实现 7.24 倍的端到端解码加速"]
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class StageSpec:
    chunk: int
    stride: int
    keep: int


def chunk_scores(S_of_rows, starts: np.ndarray, chunk: int, stride: int, length: int) -> np.ndarray:
    """Score of each chunk = max of S_t over t = x, x+stride, ... < min(x+chunk, length)."""
    n_samp = chunk // stride
    t = starts[:, None] + stride * np.arange(n_samp, dtype=np.int64)[None, :]
    valid = t < length
    S = S_of_rows(np.where(valid, t, 0))
    S = np.where(valid, S, np.iinfo(np.int64).min)
    return S.max(axis=1)


def select_top(starts: np.ndarray, scores: np.ndarray, keep: int) -> np.ndarray:
    """The first min(keep, n) chunks in the order (score desc, start asc),
    returned sorted ascending by start."""
    order = np.lexsort((starts, -scores))            # last key is primary
    return np.sort(starts[order[:keep]])


def children(kept: np.ndarray, parent_chunk: int, chunk: int, length: int) -> np.ndarray:
    """Sub-chunks of length ``chunk`` of every kept parent chunk, start < length."""
    x = (kept[:, None] + chunk * np.arange(parent_chunk // chunk, dtype=np.int64)[None, :]).reshape(-1)
    return x[x < length]


def prune(S_of_rows, length: int, stages: Sequence[StageSpec],
          given: Sequence[np.ndarray] = (), S0_of_rows=None) -> List[np.ndarray]:
    """Runs the stages; returns the kept chunk starts P_1..P_S (ascending).

    ``S0_of_rows``, when given, scores the first stage's samples in place of
    ``S_of_rows`` (the int4 sketch of the first stage's rows).

    ``given`` holds kept sets of the first len(given) stages, reused from an
    earlier step ([HiP] same section: the modular design lets the pruning
    stages' results be cached, for faster decoding): those stages are not
    run, and the first stage that runs takes the children of the last given
    set.  Only entries in [0, length) of a given set count."""
    r = len(given)
    kept_all = [np.asarray(g, dtype=np.int64) for g in given]
    kept_all = [g[(g >= 0) & (g < length)] for g in kept_all]
    if r == 0:
        cand = np.arange(0, length, stages[0].chunk, dtype=np.int64)
    elif r < len(stages):
        cand = children(kept_all[r - 1], stages[r - 1].chunk, stages[r].chunk, length)
    for s in range(r, len(stages)):
        st = stages[s]
        score_fn = S0_of_rows if (s == 0 and S0_of_rows is not None) else S_of_rows
        sc = chunk_scores(score_fn, cand, st.chunk, st.stride, length)
        kept = select_top(cand, sc, st.keep)
        kept_all.append(kept)
        if s + 1 < len(stages):
            cand = children(kept, st.chunk, stages[s + 1].chunk, length)
    return kept_all


# --------------------------------------------------------------------------
# O10: attended set [KVN "KV Cache 压缩技术", StreamingLLM sink + window]
# --------------------------------------------------------------------------
def attended_tokens(kept_last: np.ndarray, chunk: int, length: int, sink: int, window: int) -> np.ndarray:
    mask = np.zeros(length, dtype=bool)
    for x in kept_last:
        mask[x:min(x + chunk, length)] = True
    mask[:min(sink, length)] = True
    mask[max(0, length - window):] = True
    return np.flatnonzero(mask)


# --------------------------------------------------------------------------
# O11: exact attention over the attended set
# [KVN "KV Cache 回顾", decode attention equation, restricted to T]
# --------------------------------------------------------------------------
def attend(q_f64: np.ndarray, k_f64: np.ndarray, v_f64: np.ndarray, scale: float):
    """softmax(scale * q . k_t) weighted sum of v_t over the given rows.

    Returns (output [d], probabilities [n]) in fp64."""
    z = scale * (k_f64 @ q_f64)
    m = z.max()
    e = np.exp(z - m)
    p = e / e.sum()
    return p @ v_f64, p


def dense_attention(q_f64: np.ndarray, k_f64: np.ndarray, v_f64: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q K^T * scale) V written directly, for the full-budget check."""
    logits = (q_f64[None, :] @ k_f64.T)[0] * scale
    w = np.exp(logits - logits.max())
    return (w / w.sum()) @ v_f64


# --------------------------------------------------------------------------
# Whole step
# --------------------------------------------------------------------------
@dataclass
class StepConfig:
    stages: Tuple[StageSpec, ...]
    sink: int
    window: int
    scale: float = 1.0 / np.sqrt(128.0)

    @property
    def keep_total(self) -> int:
        return sum(s.keep for s in self.stages)


@dataclass
class StepResult:
    q8: np.ndarray                 # int8 [B][Hq][d]
    Q: np.ndarray                  # int64 [B][Hkv][d]
    kept_idx: np.ndarray           # int32 [B][Hkv][sum keep]
    attended: List[List[np.ndarray]]   # [b][j] sorted token indices
    out: np.ndarray                # fp64 [B][Hq][d]
    psum: np.ndarray               # fp64 [B][Hq]  (sum of softmax weights)


def decode_step(q_bits: np.ndarray, k_bits: np.ndarray, k8: np.ndarray, v_bits: np.ndarray,
                lengths: Sequence[int], cfg: StepConfig, reuse: int = 0,
                kept_prev: Optional[np.ndarray] = None,
                sketch4: Optional[Sequence[Sequence[np.ndarray]]] = None) -> StepResult:
    """One decode step for a batch.

    q_bits [B][Hq][d] bf16 bits; k_bits, v_bits [B][Hkv][Lmax][d] bf16 bits;
    k8 [B][Hkv][Lmax][d] int8 codes (only rows t < L_b are read).  With
    reuse > 0 the first ``reuse`` stages are not run: their kept sets are
    taken from kept_prev [B][Hkv][sum keep] (an earlier step's kept_idx),
    whose rows for those stages are also returned unchanged.  With
    ``sketch4`` ([b][j] -> key_sketch4 codes of rows 0, r_1, 2 r_1, ...) the
    first stage scores S4_t = Q_j . K4_(t / r_1) instead of Q_j . K8_t."""
    if reuse:
        assert kept_prev is not None and 0 < reuse <= len(cfg.stages)
    B, Hq, d = q_bits.shape
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    q8 = np.stack([quantize_query(q_bits[b]) for b in range(B)])
    Qs = np.stack([group_query(q8[b], Hkv) for b in range(B)])
    kept_idx = np.full((B, Hkv, cfg.keep_total), -1, dtype=np.int32)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    psum = np.zeros((B, Hq), dtype=np.float64)
    attended: List[List[np.ndarray]] = []
    for b in range(B):
        L = int(lengths[b])
        row = []
        for j in range(Hkv):
            Qj = Qs[b, j]
            k8_bj = k8[b, j]
            S_of_rows = lambda t, k8_bj=k8_bj, Qj=Qj: token_scores(Qj, k8_bj[t.reshape(-1)]).reshape(t.shape)
            S0 = None
            if sketch4 is not None:
                r1 = cfg.stages[0].stride
                k4_bj = sketch4[b][j]
                # every first-stage sample is a multiple of r_1 (chunk starts are
                # multiples of the chunk, which r_1 divides)
                S0 = lambda t, k4_bj=k4_bj, Qj=Qj, r1=r1: token_scores(Qj, k4_bj[t.reshape(-1) // r1]).reshape(t.shape)
            offs = np.cumsum([0] + [st.keep for st in cfg.stages])
            given = [kept_prev[b, j, offs[s]:offs[s + 1]] for s in range(reuse)]
            kept = prune(S_of_rows, L, cfg.stages, given, S0)
            for s, (st, P) in enumerate(zip(cfg.stages, kept)):
                if s < reuse:
                    kept_idx[b, j, offs[s]:offs[s + 1]] = given[s]
                else:
                    kept_idx[b, j, offs[s]:offs[s] + len(P)] = P
            T = attended_tokens(kept[-1], cfg.stages[-1].chunk, L, cfg.sink, cfg.window)
            row.append(T)
            kf = bf16_to_f64(k_bits[b, j, T])
            vf = bf16_to_f64(v_bits[b, j, T])
            for h in range(j * G, (j + 1) * G):
                o, p = attend(bf16_to_f64(q_bits[b, h]), kf, vf, cfg.scale)
                out[b, h] = o
                psum[b, h] = p.sum()
        attended.append(row)
    return StepResult(q8, Qs, kept_idx, attended, out, psum)


# --------------------------------------------------------------------------
# O12: LRU over 8-token value blocks [HiP "实现 7.24 倍的端到端解码加速": LRU
#      based offload cache; HCA 引言: values fetched late from CPU memory]
# --------------------------------------------------------------------------
def needed_blocks(tokens: np.ndarray, block: int = 8) -> np.ndarray:
    """Ascending ids of the value blocks that hold any attended token."""
    return np.unique(np.asarray(tokens, dtype=np.int64) // block)


class LRU:
    """One KV head's block cache: ``capacity`` slots; at each step every
    needed block is touched (hit or loaded); when a block must be loaded
    into a full cache, the resident block with the smallest
    (last step used, block id) is evicted."""

    def __init__(self, capacity: int):
        self.capacity = capacity
        self.last: Dict[int, int] = {}         # resident block -> last step used
        self._heap: List[Tuple[int, int]] = []  # (last, block); stale entries skipped

    def _evict_one(self) -> int:
        while True:
            last, blk = heapq.heappop(self._heap)
            if self.last.get(blk) == last:      # still the block's current entry
                del self.last[blk]
                return blk

    def step(self, blocks: Sequence[int], t: int) -> Tuple[int, int]:
        blocks = sorted(set(int(x) for x in blocks))
        if len(blocks) > self.capacity:
            raise ValueError("needed set larger than the cache")
        hits = [x for x in blocks if x in self.last]
        misses = [x for x in blocks if x not in self.last]
        for x in hits:                          # touched blocks are the newest
            self.last[x] = t
            heapq.heappush(self._heap, (t, x))
        for x in misses:
            if len(self.last) == self.capacity:
                self._evict_one()
            self.last[x] = t
            heapq.heappush(self._heap, (t, x))
        return len(hits), len(misses)

"""Seeded synthetic inputs for one sparse decode step.

This module only draws random numbers and lays them out.  It holds none of
the method's arithmetic (no quantisation, scoring, selection or attention),
so both the CPU oracle and the HIP path may take their inputs from it.

Workloads (shapes, budgets and distributions) follow the five decode
configurations the method is measured on:

* ``tiny16k``   -- 1 KV head, 4 query heads, 16,384 tokens, 16 planted keys.
* ``llama8b_128k`` -- GQA 32/8, 131,072 tokens, keys scaled per channel by a
  log-uniform [0.25, 4] factor, 64 planted keys per KV head.
* ``ragged_b16`` -- as ``llama8b_128k`` at batch 16 with per-request lengths
  256 * U{128..512}.
* ``ctx_1m``    -- as ``llama8b_128k`` at 1,048,576 tokens, 256 planted keys.
* ``ctx_3m_hostv`` -- 3,145,728 tokens, values in pinned host memory behind
  an LRU of 65,536 tokens per KV head, 32 steps of a drifting query
  q_t = 0.9 q_{t-1} + N(0, 0.44).

Recipe (all "N(m, s)" are mean / standard deviation; every bf16 value is the
round-to-nearest-even of an fp32 draw):

* ``SeedSequence(seed).spawn(B)`` gives one child per request; each child is
  spawned into streams for length, query, channel scales, planted positions,
  planted noise, keys and values.  Keys and values are drawn per
  (KV head, 65,536-token block) from their own spawned child, so generation
  is parallel and independent of thread scheduling.
* K ~ N(0,1), times the channel scale where the workload has one; V ~ N(0,1);
  q ~ N(0,1).
* Planted keys: distinct positions uniform in [sink, L - window) (not
  aligned to any chunk), each row set to 2 * mean of the group's bf16 query
  vectors + N(0, 0.5), unscaled.
* Rows t >= L_b of a shorter request are filled with the bf16 value 64.0 in
  both K and V, so that any read of padding shows up in the results.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

HEAD_DIM = 128
GEN_BLOCK = 65536          # tokens per independently seeded generation block
PAD_BF16 = 0x4280          # bf16 bit pattern of 64.0, written into padding rows


@dataclass(frozen=True)
class Stage:
    chunk: int
    stride: int
    keep: int


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    max_context: int
    stages: Tuple[Stage, ...]
    sink: int
    window: int
    seed: int
    planted: int
    channel_scale: bool
    ragged: bool = False            # lengths 256 * U{128..512} per request
    values_on_host: bool = False
    value_cache_tokens: int = 0
    steps: int = 1                  # >1: drifting query sequence
    head_dim: int = HEAD_DIM

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def keep_total(self) -> int:
        return sum(s.keep for s in self.stages)

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


_BIG = (Stage(256, 8, 64), Stage(32, 2, 128), Stage(8, 1, 256))

WORKLOADS = {
    "tiny16k": Workload("tiny16k", 1, 4, 1, 16384,
                        (Stage(256, 8, 16), Stage(32, 2, 32), Stage(8, 1, 64)),
                        64, 512, 1000, 16, False),
    "llama8b_128k": Workload("llama8b_128k", 1, 32, 8, 131072, _BIG,
                             64, 1024, 1001, 64, True),
    "ragged_b16": Workload("ragged_b16", 16, 32, 8, 131072, _BIG,
                           64, 1024, 1002, 64, True, ragged=True),
    "ctx_1m": Workload("ctx_1m", 1, 32, 8, 1048576, _BIG,
                       64, 1024, 1003, 256, True),
    "ctx_3m_hostv": Workload("ctx_3m_hostv", 1, 32, 8, 3145728, _BIG,
                             64, 1024, 1004, 256, True, values_on_host=True,
                             value_cache_tokens=65536, steps=32),
}
WORKLOAD_ORDER = ["tiny16k", "llama8b_128k", "ragged_b16", "ctx_1m", "ctx_3m_hostv"]


# --------------------------------------------------------------------------
# bf16 helpers (bit patterns stored as uint16)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs)."""
    x = np.asarray(x, dtype=np.float32)
    u = np.ascontiguousarray(x).view(np.uint32).reshape(x.shape)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# generation
# --------------------------------------------------------------------------
@dataclass
class Inputs:
    workload: Workload
    q: np.ndarray                  # uint16 [B][Hq][d]; [steps][B][Hq][d] if steps > 1
    k: np.ndarray                  # uint16 [B][Hkv][Lmax][d]
    v: np.ndarray                  # uint16 [B][Hkv][Lmax][d]
    lengths: np.ndarray            # int32 [B]
    planted: List[List[np.ndarray]] = field(default_factory=list)   # [b][j] positions
    channel_scale: Optional[np.ndarray] = None                      # f32 [B][Hkv][d]

    @property
    def q_step0(self) -> np.ndarray:
        return self.q[0] if self.workload.steps > 1 else self.q


def _threads() -> int:
    n = os.environ.get("SD_GEN_THREADS")
    if n:
        return max(1, int(n))
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def _request_streams(w: Workload, seed: int):
    root = np.random.SeedSequence(seed)
    out = []
    for child in root.spawn(w.batch):
        ss_len, ss_q, ss_scale, ss_pos, ss_noise, ss_k, ss_v = child.spawn(7)
        out.append(dict(len=ss_len, q=ss_q, scale=ss_scale, pos=ss_pos,
                        noise=ss_noise, k=ss_k, v=ss_v))
    return out


def draw_lengths(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    seed = w.seed if seed is None else seed
    streams = _request_streams(w, seed)
    L = np.full(w.batch, w.max_context, dtype=np.int32)
    if w.ragged:
        for b, st in enumerate(streams):
            rng = np.random.Generator(np.random.PCG64(st["len"]))
            L[b] = 256 * int(rng.integers(128, 512, endpoint=True))
        assert L.max() <= w.max_context
    return L


def _fill_blocks(dst: np.ndarray, ss: np.random.SeedSequence, L: int,
                 scale: Optional[np.ndarray], pool: ThreadPoolExecutor) -> None:
    """dst: uint16 [Lmax][d] view for one (request, KV head)."""
    nblk = (L + GEN_BLOCK - 1) // GEN_BLOCK
    seeds = ss.spawn(nblk) if nblk else []

    def one(i):
        t0, t1 = i * GEN_BLOCK, min(L, (i + 1) * GEN_BLOCK)
        rng = np.random.Generator(np.random.PCG64(seeds[i]))
        x = rng.standard_normal((GEN_BLOCK, dst.shape[1]), dtype=np.float32)[: t1 - t0]
        if scale is not None:
            x *= scale[None, :]
        dst[t0:t1] = f32_to_bf16_bits(x)

    list(pool.map(one, range(nblk)))
    if L < dst.shape[0]:
        dst[L:] = PAD_BF16


def _queries(w: Workload, streams, steps: int) -> np.ndarray:
    """[B][Hq][d] bf16 bits for one step; for more, [steps][B][Hq][d] with
    q_0 ~ N(0, 1) and q_t = 0.9 q_{t-1} + 0.44 N(0, 1) (fp32, then bf16)."""
    B, Hq, d = w.batch, w.num_q_heads, w.head_dim
    q = np.empty((steps, B, Hq, d) if steps > 1 else (B, Hq, d), np.uint16)
    for b, st in enumerate(streams):
        rq = np.random.Generator(np.random.PCG64(st["q"]))
        if steps > 1:
            cur = rq.standard_normal((Hq, d), dtype=np.float32)
            q[0, b] = f32_to_bf16_bits(cur)
            for s in range(1, steps):
                cur = np.float32(0.9) * cur + np.float32(0.44) * rq.standard_normal((Hq, d), dtype=np.float32)
                q[s, b] = f32_to_bf16_bits(cur)
        else:
            q[b] = f32_to_bf16_bits(rq.standard_normal((Hq, d), dtype=np.float32))
    return q


def make_queries(w: Workload, steps: int, seed: Optional[int] = None) -> np.ndarray:
    """The drifting query sequence [steps][B][Hq][d] that make_inputs draws
    for a workload of `steps` steps (its first step is the query of the
    one-step workload), without generating the cache."""
    seed = w.seed if seed is None else seed
    return _queries(w, _request_streams(w, seed), max(2, steps))[:steps]


def make_inputs(w: Workload, seed: Optional[int] = None,
                k_out: Optional[np.ndarray] = None,
                v_out: Optional[np.ndarray] = None,
                lengths: Optional[Sequence[int]] = None) -> Inputs:
    """Generate one workload's inputs.

    ``k_out`` / ``v_out`` may be caller-provided uint16 arrays of shape
    [B][Hkv][Lmax][d] (e.g. numpy views of pinned torch tensors) that are
    filled in place.  ``lengths`` overrides the drawn lengths (tests of
    edge cases); it never changes any other draw.
    """
    seed = w.seed if seed is None else seed
    B, Hq, Hkv, d, Lmax = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_context
    G = w.group
    streams = _request_streams(w, seed)
    L = draw_lengths(w, seed) if lengths is None else np.asarray(lengths, dtype=np.int32)
    assert L.shape == (B,) and L.min() >= 1 and L.max() <= Lmax

    shape = (B, Hkv, Lmax, d)
    k = np.empty(shape, np.uint16) if k_out is None else k_out
    v = np.empty(shape, np.uint16) if v_out is None else v_out
    assert k.shape == shape and v.shape == shape and k.dtype == np.uint16 and v.dtype == np.uint16

    q = _queries(w, streams, w.steps)
    scales = np.ones((B, Hkv, d), np.float32) if w.channel_scale else None
    for b, st in enumerate(streams):
        if scales is not None:
            rs = np.random.Generator(np.random.PCG64(st["scale"]))
            scales[b] = np.exp(rs.uniform(np.log(0.25), np.log(4.0), size=(Hkv, d))).astype(np.float32)

    q0 = q[0] if w.steps > 1 else q
    planted: List[List[np.ndarray]] = []
    with ThreadPoolExecutor(_threads()) as pool:
        for b, st in enumerate(streams):
            ks, vs = st["k"].spawn(Hkv), st["v"].spawn(Hkv)
            for j in range(Hkv):
                _fill_blocks(k[b, j], ks[j], int(L[b]), None if scales is None else scales[b, j], pool)
                _fill_blocks(v[b, j], vs[j], int(L[b]), None, pool)
            # planted heavy keys
            rp = np.random.Generator(np.random.PCG64(st["pos"]))
            rn = np.random.Generator(np.random.PCG64(st["noise"]))
            row = []
            lo, hi = w.sink, int(L[b]) - w.window
            if hi - lo < w.planted:          # short request: plant anywhere
                lo, hi = 0, int(L[b])
            n_pl = min(w.planted, hi - lo)
            for j in range(Hkv):
                pos = np.sort(rp.choice(hi - lo, size=n_pl, replace=False).astype(np.int64) + lo)
                mean_q = bf16_bits_to_f32(q0[b, j * G:(j + 1) * G]).mean(axis=0, dtype=np.float32)
                noise = rn.standard_normal((n_pl, d), dtype=np.float32) * np.float32(0.5)
                k[b, j, pos] = f32_to_bf16_bits(np.float32(2.0) * mean_q[None, :] + noise)
                row.append(pos)
            planted.append(row)
    return Inputs(w, q, k, v, L, planted, scales)


def make_append_tokens(w: Workload, n: int, seed: int):
    """New key and value rows for an append of n tokens per request:
    uint16 bf16 bits [B][Hkv][n][d], i.i.d. N(0, 1) (keys times the
    workload's channel scales when it has them, drawn afresh from `seed`)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, n])))
    shape = (w.batch, w.num_kv_heads, n, w.head_dim)
    k = rng.standard_normal(shape, dtype=np.float32)
    if w.channel_scale:
        k *= np.exp(rng.uniform(np.log(0.25), np.log(4.0), size=(w.batch, w.num_kv_heads, 1, w.head_dim))
                    ).astype(np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def tiny_workload(**kw) -> Workload:
    """A small variant of ``tiny16k`` for quick tests; fields overridable."""
    return WORKLOADS["tiny16k"].replace(**kw)

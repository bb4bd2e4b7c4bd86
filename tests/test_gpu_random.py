"""Randomised GPU parity: seeded random configurations (stage count, chunk /
stride / keep per stage, group size, KV heads, batch, ragged lengths
including 1 and Lmax, sink and window, budgets above the candidate count)
through the C ABI against the oracle, under both the fused and the unfused
last stage.  Bar as everywhere: int8 codes, every stage's scores and kept
sets bit-exact; outputs within 8e-3.  Each configuration prints its seed
and shape before it runs.
"""
import numpy as np
import pytest

from sparse_attention_kv_int8_amd.inputs import Stage, tiny_workload
from tests.test_gpu_parity import fusion, run_case  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

SEEDS = list(range(24))


def random_case(seed: int):
    """A valid configuration (the library's limits: stride divides chunk,
    chunks nest, the last chunk is a multiple of 8, at most 64 samples per
    chunk) and request lengths, drawn from `seed`."""
    rng = np.random.default_rng(10_000 + seed)
    S = int(rng.integers(1, 5))
    chunks = [int(rng.choice([8, 16, 32]))]
    for _ in range(S - 1):
        chunks.insert(0, chunks[0] * int(rng.choice([2, 4, 8])))
    Lmax = int(rng.integers(1000, 20001))
    n = -(-Lmax // chunks[0])
    stages = []
    for s, c in enumerate(chunks):
        strides = [1 << e for e in range(15) if (1 << e) <= c and c % (1 << e) == 0 and c // (1 << e) <= 64]
        r = int(rng.choice(strides))
        keep = int(rng.integers(1, min(n, 300) + 3))            # sometimes more than the candidates
        stages.append(Stage(c, r, keep))
        if s + 1 < S:
            n = keep * (c // chunks[s + 1])
    G = int(rng.choice([1, 2, 4]))
    Hkv = int(rng.integers(1, 4))
    B = int(rng.integers(1, 4))
    sink = int(rng.choice([0, 1, 7, 64]))
    window = int(rng.choice([0, 5, 100, 512]))
    lengths = rng.integers(1, Lmax + 1, size=B)
    if B >= 2 and rng.random() < 0.5:
        lengths[0] = Lmax
    if B >= 3 and rng.random() < 0.5:
        lengths[2] = 1
    w = tiny_workload(name=f"random{seed}", batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, max_context=Lmax,
                      stages=tuple(stages), sink=sink, window=window, planted=4, seed=20_000 + seed)
    return w, [int(x) for x in lengths]


def test_random_cases_are_valid_configurations():
    """The generator stays inside the documented limits (checked without a
    context, so a generator mistake shows here and not as a create error)."""
    for seed in SEEDS:
        w, lengths = random_case(seed)
        st = w.stages
        assert all(s.chunk % s.stride == 0 and s.chunk // s.stride <= 64 for s in st)
        assert all(st[i].chunk % st[i + 1].chunk == 0 for i in range(len(st) - 1))
        assert st[-1].chunk % 8 == 0
        assert len(lengths) == w.batch and min(lengths) >= 1 and max(lengths) <= w.max_context
    for seed in WIDE_SEEDS:
        w, lengths = random_wide_case(seed)
        st = w.stages
        assert w.batch * w.num_kv_heads >= 32 and w.num_q_heads == 4 * w.num_kv_heads
        assert all(s.chunk % s.stride == 0 and s.chunk // s.stride <= 64 for s in st)
        assert all(st[i].chunk % st[i + 1].chunk == 0 for i in range(len(st) - 1))
        assert len(lengths) == w.batch and min(lengths) >= 1 and max(lengths) <= w.max_context


@pytest.mark.parametrize("seed", SEEDS)
def test_random_configuration(seed, fusion):
    w, lengths = random_case(seed)
    print(f"seed {seed} lengths {lengths}", flush=True)
    run_case(w, lengths=lengths, check_scores=True)


WIDE_SEEDS = list(range(6))


def random_wide_case(seed: int):
    """32 or 64 (request, KV head) pipelines at G = 4: the plan for many
    pipelines (two load batches in the later stages, the wide decode, whose
    kept-chunk splits score pairs of blocks on the matrix cores when a wave
    takes more than one pair), with random strides, budgets that put from a
    few to a few dozen blocks in a split, ragged lengths, sink and window."""
    rng = np.random.default_rng(30_000 + seed)
    BH = int(rng.choice([32, 64]))
    B = int(rng.choice([2, 4, 8]))
    Hkv = BH // B
    Lmax = int(rng.integers(3000, 9001))
    n0 = -(-Lmax // 256)
    k0 = int(rng.integers(4, n0 + 3))
    k1 = int(rng.integers(k0, 8 * k0 + 1))
    c2 = int(rng.choice([8, 16]))
    k2 = int(rng.integers(max(1, k1 // 2), k1 * (32 // c2) + 3))
    stages = (Stage(256, int(rng.choice([4, 8, 16])), k0), Stage(32, int(rng.choice([1, 2, 4])), k1),
              Stage(c2, int(rng.choice([1, 2])), k2))
    sink = int(rng.choice([0, 3, 64]))
    window = int(rng.choice([0, 37, 256]))
    lengths = rng.integers(1, Lmax + 1, size=B)
    lengths[0] = Lmax
    if B >= 4:
        lengths[-1] = int(rng.integers(1, 65))
    w = tiny_workload(name=f"random_wide{seed}", batch=B, num_q_heads=4 * Hkv, num_kv_heads=Hkv, max_context=Lmax,
                      stages=stages, sink=sink, window=window, planted=4, seed=40_000 + seed)
    return w, [int(x) for x in lengths]


@pytest.mark.parametrize("seed", WIDE_SEEDS)
def test_random_wide_configuration(seed, fusion):
    w, lengths = random_wide_case(seed)
    print(f"wide seed {seed} B={w.batch} Hkv={w.num_kv_heads} Lmax={w.max_context} "
          f"stages={[(s.chunk, s.stride, s.keep) for s in w.stages]} lengths {lengths}", flush=True)
    run_case(w, lengths=lengths, check_scores=True)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_configuration_sketch_and_dense(seed, monkeypatch):
    """The same configurations through the int4 first-stage sketch step
    (sketch codes, first-stage scores, kept sets, outputs) and the dense
    decode (every head against the oracle's dense attention).  Two-stage
    configurations run unfused there (a fused first stage reads rows the
    sketch does not hold)."""
    from tests.test_gpu_dense import DenseRun, all_pairs, check
    from tests.test_gpu_sketch4 import run_sketch_case
    w, lengths = random_case(seed)
    print(f"seed {seed} lengths {lengths} (sketch, dense)", flush=True)
    if len(w.stages) == 2:
        monkeypatch.setenv("SD_FUSE_LAST_STAGE", "0")
    g, _ = run_sketch_case(w, lengths=lengths, check_scores=True)
    d = DenseRun(g.inp)
    check(g.inp, d.run(), all_pairs(w))
    assert d.dec.sd_check() == 0

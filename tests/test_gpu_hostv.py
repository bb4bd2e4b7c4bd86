"""GPU parity of the host-resident-value path: values in pinned host memory
behind the device LRU of 8-token blocks, over a sequence of decode steps
with a drifting query.

Bar: every step's kept indices bit-exact and outputs within 8e-3 of the
oracle, and every step's cache hits and misses equal to the oracle's LRU
simulation (oracle.sparse_decode.LRU) fed with the oracle's own attended
sets.
"""
import numpy as np
import pytest

from oracle import sparse_decode as O
from sparse_attention_kv_int8_amd.inputs import WORKLOADS, make_inputs
from tests.gpu_util import GpuRun, compare_step, oracle_config, oracle_keys

pytestmark = pytest.mark.gpu


def run_sequence(w, check_every=1, reuse_at=None):
    """reuse_at(t): how many pruning stages step t reuses from step t - 1
    (default none)."""
    print(f"host-value case {w.name} L={w.max_context} cache={w.value_cache_tokens} steps={w.steps}", flush=True)
    inp = make_inputs(w)
    g = GpuRun(inp)
    g.quantize()
    k8_ref, a_ref = oracle_keys(inp)
    k8 = g.k8.cpu().numpy()
    for b in range(w.batch):
        assert np.array_equal(k8[b, :, :int(inp.lengths[b])], k8_ref[b, :, :int(inp.lengths[b])])
    cap = w.value_cache_tokens // 8
    lrus = [[O.LRU(cap) for _ in range(w.num_kv_heads)] for _ in range(w.batch)]
    cfg = oracle_config(w)
    tot_h = tot_m = 0
    ref = None
    for t in range(w.steps):
        q = inp.q[t]
        r = reuse_at(t) if reuse_at and t > 0 else 0
        if r:
            out, kept = g.step_reuse(q, r)
            ref = O.decode_step(q, inp.k, k8_ref, inp.v, inp.lengths, cfg, reuse=r, kept_prev=ref.kept_idx)
        else:
            out, kept = g.step(q)
            ref = O.decode_step(q, inp.k, k8_ref, inp.v, inp.lengths, cfg)
        hits = misses = 0
        for b in range(w.batch):
            for j in range(w.num_kv_heads):
                h, m = lrus[b][j].step(O.needed_blocks(ref.attended[b][j]), t)
                hits += h
                misses += m
        st = g.dec.sd_get_stats()
        assert (st.last_hits, st.last_misses) == (hits, misses), f"step {t}: gpu {(st.last_hits, st.last_misses)} oracle {(hits, misses)}"
        tot_h += hits
        tot_m += misses
        if t % check_every == 0 or t == w.steps - 1:
            compare_step(inp, q, k8_ref, out, kept, ref=ref)
        print(f"  step {t} (reuse {r}): hits {hits} misses {misses}", flush=True)
    st = g.dec.sd_get_stats()
    assert (st.steps, st.hits, st.misses) == (w.steps, tot_h, tot_m)
    assert st.h2d_bytes == tot_m * 8 * 128 * 2
    return tot_h, tot_m


def test_hostv_small_with_evictions():
    """128K tokens, a 2,048-block cache per KV head: the drifting query makes
    the attended blocks outgrow the cache, so evictions happen."""
    w = WORKLOADS["ctx_3m_hostv"].replace(name="hostv_small", max_context=131072, value_cache_tokens=16384,
                                          planted=64, steps=24)
    h, m = run_sequence(w)
    assert m > 2048 * 8        # more misses than slots: evictions took place
    assert h > 0


def test_hostv_with_reused_stages():
    """Host values with pruning stages reused between refreshes: every
    fourth step runs all stages, the others reuse one, two or all three."""
    w = WORKLOADS["ctx_3m_hostv"].replace(name="hostv_reuse", max_context=65536, value_cache_tokens=16384,
                                          planted=32, steps=12)
    run_sequence(w, reuse_at=lambda t: t % 4)


def test_hostv_reset_starts_cold():
    w = WORKLOADS["ctx_3m_hostv"].replace(name="hostv_reset", max_context=32768, value_cache_tokens=8192,
                                          planted=16, steps=3)
    inp = make_inputs(w)
    g = GpuRun(inp)
    g.quantize()
    g.step(inp.q[0])
    g.step(inp.q[0])
    st = g.dec.sd_get_stats()
    assert st.last_misses == 0 and st.last_hits == st.last_needed > 0
    g.dec.sd_reset_value_cache()
    g.step(inp.q[0])
    st = g.dec.sd_get_stats()
    assert st.steps == 1 and st.last_hits == 0 and st.last_misses == st.last_needed


@pytest.mark.timeout(900)
def test_hostv_full_3m_workload():
    run_sequence(WORKLOADS["ctx_3m_hostv"], check_every=4)

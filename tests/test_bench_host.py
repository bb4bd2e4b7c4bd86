"""Host logic of the benchmark, without a GPU: the algorithmic byte count
behind `value` and `roofline` (against a brute-force count over the
oracle's kept sets), the counter scaling of the traffic record, and the
one-GPU guard."""
import csv
import os
import subprocess
import sys

import numpy as np

from oracle import sparse_decode as O
from sparse_attention_kv_int8_amd.inputs import Stage, make_inputs, tiny_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def brute_bytes(w, kept, lengths):
    """Every int8 row some stage samples, counted once (128 B); K + V of
    every attended token (512 B); the query read and the output written."""
    koff = np.cumsum([0] + [s.keep for s in w.stages])
    total = 0
    for b in range(w.batch):
        L = int(lengths[b])
        for j in range(w.num_kv_heads):
            rows = set()
            cand = list(range(0, L, w.stages[0].chunk))
            for s, st in enumerate(w.stages):
                for x in cand:
                    for i in range(st.chunk // st.stride):
                        t = x + i * st.stride
                        if t < L:
                            rows.add(t)
                ks = [int(v) for v in kept[b, j, koff[s]:koff[s + 1]] if v >= 0]
                if s + 1 < len(w.stages):
                    c = w.stages[s + 1].chunk
                    cand = [x + i * c for x in ks for i in range(st.chunk // c) if x + i * c < L]
            T = set(range(min(w.sink, L))) | set(range(max(0, L - w.window), L))
            for x in ks:
                T |= set(range(x, min(x + w.stages[-1].chunk, L)))
            total += 128 * len(rows) + 512 * len(T)
    return total + 3 * 2 * w.batch * w.num_q_heads * w.head_dim


def test_algorithmic_bytes_match_brute_force():
    w = tiny_workload(name="bytes", batch=2, num_q_heads=8, num_kv_heads=2, max_context=3000,
                      stages=(Stage(256, 8, 5), Stage(32, 2, 9), Stage(8, 1, 17)), sink=13, window=100, planted=4)
    inp = make_inputs(w, lengths=[3000, 1234])
    k8 = np.zeros(inp.k.shape, np.int8)
    for b in range(w.batch):
        for j in range(w.num_kv_heads):
            k8[b, j, :inp.lengths[b]] = O.quantize_keys(inp.k[b, j], int(inp.lengths[b]))[0]
    cfg = O.StepConfig(tuple(O.StageSpec(s.chunk, s.stride, s.keep) for s in w.stages), w.sink, w.window,
                       1 / np.sqrt(128))
    ref = O.decode_step(inp.q, inp.k, k8, inp.v, inp.lengths, cfg)
    got = bench.algorithmic_bytes(w, ref.kept_idx, inp.lengths)
    assert got["total"] == brute_bytes(w, ref.kept_idx, inp.lengths)
    assert got["attended_tokens"] == sum(len(t) for row in ref.attended for t in row)


def test_traffic_record_scales_by_the_copy(tmp_path):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by copy_bytes
    over what the same counter read for the copy kernel."""
    from sparse_attention_kv_int8_amd.profiling import traffic_record
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]

    def write(path, counter, rows):
        with open(path, "w", newline="") as f:
            wr = csv.writer(f)
            wr.writerow(hdr)
            for name, v in rows:
                wr.writerow([name, counter, v])
    fetch, wrt = tmp_path / "f.csv", tmp_path / "w.csv"
    write(fetch, "FETCH_SIZE", [("neg_kernel", 512.0), ("decode_kernel", 100.0), ("decode_kernel", 300.0)])
    write(wrt, "WRITE_SIZE", [("neg_kernel", 1024.0), ("decode_kernel", 10.0)])
    r = traffic_record(str(fetch), str(wrt), "decode", "neg", 1 << 20)
    assert r["factor_fetch"] == 2.0 and r["factor_write"] == 1.0
    assert r["fetch_bytes"] == 200 * 1024 * 2 and r["write_bytes"] == 10 * 1024
    assert r["traffic_bytes"] == r["fetch_bytes"] + r["write_bytes"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr

#!/usr/bin/env python3
"""Benchmark of one sparse decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  A step is the whole per-step path: query codes,
three pruning stages with their top-K selects, the attended set, the sparse
flash decode and its log-sum-exp merge.  Inputs sit in HBM before the timed
region starts.  Successive steps rotate over several copies of the KV cache
at different addresses so that no step finds its bytes in the 256 MB
Infinity Cache or the L2 (a cold-cache measurement; the copies hold the same
data).  The int8 key quantisation runs once per cache and is reported
separately.

value  = algorithmic HBM bytes of a step / wall time per step (GB/s), where
         the algorithmic bytes are the unique int8 key rows any stage samples
         (128 B each), bf16 K and V of every attended token (512 B each), and
         the query read and output written.
roofline = the dominant kernel's algorithmic bytes per launch / its average
         launch duration, timed with HIP events on the launch stream during
         the timed region, against 8 TB/s.  `traffic` is that kernel's HBM
         bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE counters
         (scaled by a plain copy of known size; see profiles/), or null when
         no record exists or the kernel sources changed since it was taken.
cpu_baseline = the CPU oracle (numpy, one of the process's cores) on full
         steps of the same workload, repeated for about 10 s of CPU work
         (median step), with the CPU model.
us_per_step_spread = p10 / p50 / p90 of single replayed steps, each
         between HIP events (outside the timed region).
stream_ceiling = a plain streaming copy (torch.neg, 1 GiB read + 1 GiB
         written) on the same GPU: the practically reachable HBM rate, for
         context.
dense  = dense decode attention over every cached token (sd_dense_decode),
         timed the same way: us per step, its kernel's bandwidth against
         8 TB/s, and the sparse step's speedup over it.
sketch4 = the first stage scored from the int4 sketch of its rows
         (sd_decode_step_sketch4), timed the same way, with its selection
         compared to the int8 step's on the same query.
append = KV append (sd_append_kv) of one token per call on the same
         workload grown to hold more tokens: us per append, us for one
         append that raises a scale (its rows recoded), and us per token of
         a decode loop (step + append).
batched = the 16-request ragged workload (up to 128K tokens each), timed
         like the main figure: what the same kernels reach with many
         requests in flight (context; `value` stays the B = 1 figure).
per_kernel_frac = each step kernel's algorithmic bytes (a stage scored
         inside the kernel of the stage before it counts with that kernel) /
         its average duration, against 8 TB/s, and the pruning and decode
         kernels together; `target` compares the latter at 128K and 1M with
         60% of 8 TB/s.
hostv  = the 3M-token host-resident-value workload (32 steps, drifting
         query, cold cache): graph-replayed us per step with and without
         the cold first step, hit rate, the PCIe rate (missed bytes / the
         time of the decode kernel that reads them), and the same sequence
         with the gathered hipMemcpyAsync side-stream fetch for comparison.
reuse  = steps that reuse the first r pruning stages' kept sets from an
         earlier step (sd_decode_step_reuse): us per step for each r, and,
         over a drifting query sequence, how much of the fully recomputed
         last-stage kept set such a step still finds.
"""
from __future__ import annotations

import os

import argparse
import json
import math
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from sparse_attention_kv_int8_amd.inputs import WORKLOADS, make_inputs, make_queries  # noqa: E402

METRIC = "sparse decode-attention µs/step + achieved HBM GB/s at 128K and 1M ctx (GQA 32/8)"
HBM_PEAK_GBS = 8000.0
KIND_NAMES = ["stage0", "stage1", "stage2", "stage3", "value_cache", "attend", "quantize", "combine", "dense",
              "append"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- bytes ---
def algorithmic_bytes(w, kept: np.ndarray, lengths: np.ndarray) -> dict:
    """Bytes the method must move once, per kernel kind, from the step's kept
    sets: int8 rows first sampled by each stage, K+V of the attended tokens,
    the query and the output."""
    per = {f"stage{s}": 0 for s in range(len(w.stages))}
    per["attend"] = 0
    rows_total = 0
    tokens_total = 0
    koff = np.cumsum([0] + [s.keep for s in w.stages])
    for b in range(w.batch):
        L = int(lengths[b])
        for j in range(w.num_kv_heads):
            seen = np.zeros(L, dtype=bool)
            cand = np.arange(0, L, w.stages[0].chunk, dtype=np.int64)
            for s, st in enumerate(w.stages):
                t = (cand[:, None] + st.stride * np.arange(st.chunk // st.stride)[None, :]).ravel()
                t = t[t < L]
                new = np.unique(t[~seen[t]])
                seen[new] = True
                per[f"stage{s}"] += 128 * len(new)
                rows_total += len(new)
                kept_s = kept[b, j, koff[s]:koff[s + 1]]
                kept_s = kept_s[kept_s >= 0].astype(np.int64)
                if s + 1 < len(w.stages):
                    c_n = w.stages[s + 1].chunk
                    cand = (kept_s[:, None] + c_n * np.arange(st.chunk // c_n)[None, :]).ravel()
                    cand = cand[cand < L]
            T = np.zeros(L, dtype=bool)
            for x in kept_s:
                T[x:x + w.stages[-1].chunk] = True
            T[:w.sink] = True
            T[max(0, L - w.window):] = True
            n = int(T.sum())
            tokens_total += n
            per["attend"] += 512 * n
    qbytes = 2 * w.batch * w.num_q_heads * w.head_dim
    per["stage0"] += qbytes
    per["attend"] += 2 * qbytes            # query in, output out
    return dict(per_kernel=per, total=sum(per.values()), int8_rows=rows_total, attended_tokens=tokens_total)


def kernel_bytes(per: dict, avg_us: dict) -> dict:
    """Algorithmic bytes per kernel that ran: a stage scored inside the
    kernel of the stage before it (the fused plan launches no kernel of its
    own for it) counts with that kernel."""
    out = dict(per)
    n = sum(1 for k in per if k.startswith("stage"))
    for s in range(n - 1, 0, -1):
        if f"stage{s}" not in avg_us and f"stage{s - 1}" in avg_us:
            out[f"stage{s - 1}"] += out.pop(f"stage{s}")
    return out


def kernel_fracs(kb: dict, avg_us: dict) -> dict:
    """Each step kernel's algorithmic bytes / its average duration, as a
    fraction of 8 TB/s; and the pruning + decode kernels together."""
    fr = {k: round(kb[k] / (avg_us[k] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) for k in kb if k in avg_us}
    ks = [k for k in kb if k in avg_us]
    fr["prune_and_decode"] = round(sum(kb[k] for k in ks) / (sum(avg_us[k] for k in ks) * 1e-6) / 1e9 /
                                   HBM_PEAK_GBS, 4)
    return fr


# ---------------------------------------------------------------- GPU -----
class Bench:
    def __init__(self, w, copies: int):
        import torch
        from sparse_attention_kv_int8_amd import binding as B
        self.torch, self.B, self.w = torch, B, w
        t = time.perf_counter()
        inp = make_inputs(w)
        log(f"[bench] {w.name}: inputs generated in {time.perf_counter() - t:.1f}s")
        self.inp = inp
        dev = "cuda"
        to_bf16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        self.dec = B.SparseDecoder.for_workload(w)
        q = inp.q_step0
        self.q = to_bf16(np.ascontiguousarray(q))
        self.lengths = torch.from_numpy(inp.lengths.astype(np.int32)).to(dev)
        k0 = to_bf16(inp.k)
        v0 = to_bf16(inp.v)
        k80 = torch.empty(inp.k.shape, dtype=torch.int8, device=dev)
        # one-time key quantisation, timed with events
        self.dec.sd_profile_start(1 << B.SD_PROF_QUANTIZE, 4)
        self.dec.sd_quantize_keys(k0, self.lengths, k80)
        prof = self.dec.sd_profile_stop()
        self.quantize_us = prof["quantize"][0] * 1e3
        self.ks, self.vs, self.k8s = [k0], [v0], [k80]
        for _ in range(copies - 1):
            self.ks.append(k0.clone())
            self.vs.append(v0.clone())
            self.k8s.append(k80.clone())
        self.out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
        self.kept = torch.empty((w.batch, w.num_kv_heads, w.keep_total), dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        self.stream = torch.cuda.current_stream().cuda_stream
        # raw pointers so that the timed loop is one ctypes call per step
        self.args = [(self.q.data_ptr(), self.ks[i].data_ptr(), self.k8s[i].data_ptr(), self.vs[i].data_ptr(),
                      self.lengths.data_ptr(), self.out.data_ptr(), self.kept.data_ptr())
                     for i in range(copies)]

    def run(self, n: int) -> None:
        lib, h, s = self.B.lib, self.dec.handle, self.stream
        nc = len(self.args)
        for i in range(n):
            a = self.args[i % nc]
            st = lib.sd_decode_step(h, *a, s)
            if st:
                self.B.check(st, "sd_decode_step")

    def capture(self) -> None:
        """One HIP graph per KV-cache copy, each holding one decode step."""
        torch, lib, h = self.torch, self.B.lib, self.dec.handle
        self.graphs = []
        torch.cuda.synchronize()
        for a in self.args:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                st = lib.sd_decode_step(h, *a, torch.cuda.current_stream().cuda_stream)
                if st:
                    self.B.check(st, "sd_decode_step (capture)")
            self.graphs.append(g)
        torch.cuda.synchronize()

    def replay(self, n: int) -> None:
        gs = self.graphs
        for i in range(n):
            gs[i % len(gs)].replay()

    def profile(self, n: int, mask: int) -> dict:
        self.dec.sd_profile_start(mask, 8 * n + 8)
        self.run(n)
        return self.dec.sd_profile_stop()


def reuse_study(b, steps: int, seq: int = 8) -> dict:
    """Pruning stages reused from an earlier step (sd_decode_step_reuse).

    time: us per step when the first r stages are reused, r = 1..S, timed
    like the main figure (HIP graph replay over the rotating cache copies,
    kept_idx holding the last full step's kept sets).  recall: over the
    workload's drifting query sequence (q_t = 0.9 q_(t-1) + 0.44 N(0, 1)),
    steps t = 1..seq-1 reuse the first r stages of step 0; the share of the
    last stage's fully recomputed kept chunks that the reusing step also
    keeps (mean over steps, requests and KV heads; also per step), the
    largest |output difference| to the fully recomputed step, and the share
    of the planted heavy tokens (the stand-in for a needle the query looks
    for) that the attended set holds, for reused and full steps."""
    torch, lib, h, w = b.torch, b.B.lib, b.dec.handle, b.w
    S = len(w.stages)
    res = {"us_per_step": {}, "recall_last_stage": {}, "max_abs_out_diff": {}, "sequence_steps": seq}
    b.run(1)                                     # kept_idx: a full step's kept sets
    torch.cuda.synchronize()
    for r in range(1, S + 1):
        graphs = []
        for a in b.args:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                st = lib.sd_decode_step_reuse(h, *a, r, torch.cuda.current_stream().cuda_stream)
                if st:
                    b.B.check(st, "sd_decode_step_reuse (capture)")
            graphs.append(g)
        for i in range(20):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        res["us_per_step"][str(r)] = round((time.perf_counter() - t0) / steps * 1e6, 3)
        del graphs
    # quality over the drifting sequence (outside any timed region)
    qs = make_queries(w, seq)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    kept0 = torch.empty_like(b.kept)
    kept_f, kept_r = torch.empty_like(b.kept), torch.empty_like(b.kept)
    out_f, out_r = torch.empty_like(b.out), torch.empty_like(b.out)
    b.dec.sd_decode_step(to_dev(qs[0]), b.ks[0], b.k8s[0], b.vs[0], b.lengths, b.out, kept0)
    off = sum(st.keep for st in w.stages[:-1])
    c_last = w.stages[-1].chunk
    lengths = b.inp.lengths

    def planted_hit(kept_last, bb, j):
        """planted heavy tokens of (bb, j) inside the attended set"""
        L = int(lengths[bb])
        pos = np.asarray(b.inp.planted[bb][j])
        ks = kept_last[kept_last >= 0]
        inside = ((pos[:, None] >= ks[None, :]) & (pos[:, None] < ks[None, :] + c_last)).any(axis=1)
        inside |= (pos < w.sink) | (pos >= L - w.window)
        return int(inside.sum()), len(pos)

    res["recall_by_step"] = {}
    res["planted_recall"] = {}
    full_hit = full_n = 0
    for r in range(1, S + 1):
        rec_t, diff, hit, n = [], 0.0, 0, 0
        for t in range(1, seq):
            q = to_dev(qs[t])
            b.dec.sd_decode_step(q, b.ks[0], b.k8s[0], b.vs[0], b.lengths, out_f, kept_f)
            kept_r.copy_(kept0)
            b.dec.sd_decode_step_reuse(q, b.ks[0], b.k8s[0], b.vs[0], b.lengths, out_r, kept_r, r)
            torch.cuda.synchronize()
            kf, kr = kept_f.cpu().numpy()[..., off:], kept_r.cpu().numpy()[..., off:]
            rec = []
            for bb in range(w.batch):
                for j in range(w.num_kv_heads):
                    f = set(kf[bb, j][kf[bb, j] >= 0].tolist())
                    if f:
                        rec.append(len(f & set(kr[bb, j].tolist())) / len(f))
                    h1, n1 = planted_hit(kr[bb, j], bb, j)
                    hit, n = hit + h1, n + n1
                    if r == 1:
                        h0, n0 = planted_hit(kf[bb, j], bb, j)
                        full_hit, full_n = full_hit + h0, full_n + n0
            rec_t.append(round(statistics.fmean(rec), 4))
            diff = max(diff, float((out_f.float() - out_r.float()).abs().max()))
        res["recall_last_stage"][str(r)] = round(statistics.fmean(rec_t), 4)
        res["recall_by_step"][str(r)] = rec_t
        res["max_abs_out_diff"][str(r)] = round(diff, 4)
        res["planted_recall"][str(r)] = round(hit / max(1, n), 4)
    res["planted_recall"]["full"] = round(full_hit / max(1, full_n), 4)
    return res


def dense_study(b, steps: int, warmup: int, sparse_us: float) -> dict:
    """Dense decode attention over every cached token (sd_dense_decode), the
    comparison the sparse step is made to beat: timed like the main figure
    (one HIP graph per cache copy, replayed), then the same steps launched
    eagerly with the dense kernel's and its merge's dispatches carrying HIP
    events on the launch stream.  bytes = bf16 K and V of every token t < L_b
    of every (request, KV head), plus the query and the output."""
    torch, lib, h, w, B = b.torch, b.B.lib, b.dec.handle, b.w, b.B
    out = torch.empty_like(b.out)
    args = [(b.q.data_ptr(), b.ks[i].data_ptr(), b.vs[i].data_ptr(), b.lengths.data_ptr(), out.data_ptr())
            for i in range(len(b.ks))]
    graphs = []
    torch.cuda.synchronize()
    for a in args:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st = lib.sd_dense_decode(h, *a, torch.cuda.current_stream().cuda_stream)
            if st:
                B.check(st, "sd_dense_decode (capture)")
        graphs.append(g)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / steps * 1e6
    del graphs
    b.dec.sd_profile_start((1 << B.SD_PROF_DENSE) | (1 << B.SD_PROF_COMBINE), 2 * steps + 8)
    for i in range(steps):
        st = lib.sd_dense_decode(h, *args[i % len(args)], b.stream)
        if st:
            B.check(st, "sd_dense_decode")
    prof = b.dec.sd_profile_stop()
    k_us = prof["dense"][0] * 1e3 / prof["dense"][1]
    c_us = prof["combine"][0] * 1e3 / prof["combine"][1]
    nbytes = int(512 * w.num_kv_heads * int(np.sum(b.inp.lengths.astype(np.int64)))
                 + 4 * w.batch * w.num_q_heads * w.head_dim)
    return {"us_per_step": round(us, 3), "value_GBs": round(nbytes / (us * 1e-6) / 1e9, 2),
            "bytes": nbytes, "kernel_us": round(k_us, 3), "combine_us": round(c_us, 3),
            "kernel_roofline": {"bound": "hbm", "achieved": round(nbytes / (k_us * 1e-6) / 1e9, 2),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(nbytes / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
            "sparse_speedup": round(us / sparse_us, 2),
            "note": "sd_dense_decode over every token, same rotating cold copies, HIP graph replay"}


def sketch_study(b, steps: int, warmup: int, sparse_us: float) -> dict:
    """The first stage scored from the int4 sketch (sd_decode_step_sketch4),
    timed like the main figure (HIP graph replay over the rotating copies,
    each with its own sketch), with the first-stage kernel timed by HIP
    events carried by its dispatches.  Selection against the int8 step on
    the same query: the share of the int8 step's last-stage kept chunks the
    sketch step also keeps, the share of planted heavy tokens each attends,
    and the largest output difference."""
    torch, lib, h, w, B = b.torch, b.B.lib, b.dec.handle, b.w, b.B
    rows = b.dec.sd_sketch4_rows()
    sk0 = torch.empty((w.batch, w.num_kv_heads, rows, 64), dtype=torch.uint8, device="cuda")
    b.dec.sd_quantize_sketch4(b.ks[0], b.lengths, sk0)
    sks = [sk0] + [sk0.clone() for _ in range(len(b.ks) - 1)]
    out = torch.empty_like(b.out)
    kept = torch.empty_like(b.kept)
    args = [(b.q.data_ptr(), b.ks[i].data_ptr(), b.k8s[i].data_ptr(), sks[i].data_ptr(), b.vs[i].data_ptr(),
             b.lengths.data_ptr(), out.data_ptr(), kept.data_ptr()) for i in range(len(b.ks))]
    graphs = []
    torch.cuda.synchronize()
    for a in args:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st = lib.sd_decode_step_sketch4(h, *a, torch.cuda.current_stream().cuda_stream)
            if st:
                B.check(st, "sd_decode_step_sketch4 (capture)")
        graphs.append(g)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / steps * 1e6
    del graphs
    b.dec.sd_profile_start(0xFF, 8 * steps + 8)
    for i in range(steps):
        st = lib.sd_decode_step_sketch4(h, *args[i % len(args)], b.stream)
        if st:
            B.check(st, "sd_decode_step_sketch4")
    prof = b.dec.sd_profile_stop()
    kern = {k: round(v[0] * 1e3 / v[1], 3) for k, v in prof.items()}
    # selection against the int8 step (same query, same cache)
    b.run(1)
    torch.cuda.synchronize()
    k8set, o8 = b.kept.cpu().numpy(), b.out.float()
    k4set = kept.cpu().numpy()
    off = sum(st.keep for st in w.stages[:-1])
    c_last = w.stages[-1].chunk
    rec, hit4, hit8, n = [], 0, 0, 0
    for bb in range(w.batch):
        L = int(b.inp.lengths[bb])
        for j in range(w.num_kv_heads):
            f = set(k8set[bb, j, off:][k8set[bb, j, off:] >= 0].tolist())
            if f:
                rec.append(len(f & set(k4set[bb, j, off:].tolist())) / len(f))
            pos = np.asarray(b.inp.planted[bb][j])
            for ks_, name in ((k4set, 4), (k8set, 8)):
                kk = ks_[bb, j, off:]
                kk = kk[kk >= 0]
                inside = ((pos[:, None] >= kk[None, :]) & (pos[:, None] < kk[None, :] + c_last)).any(axis=1)
                inside |= (pos < w.sink) | (pos >= L - w.window)
                if name == 4:
                    hit4 += int(inside.sum())
                else:
                    hit8 += int(inside.sum())
            n += len(pos)
    first_rows = int(sum(-(-int(L) // w.stages[0].stride) for L in b.inp.lengths)) * w.num_kv_heads
    return {"us_per_step": round(us, 3), "speedup_vs_int8": round(sparse_us / us, 3), "step_kernels_us": kern,
            "stage0_bytes": 64 * first_rows,
            "stage0_roofline_frac": round(64 * first_rows / (kern["stage0"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "last_stage_overlap_with_int8": round(statistics.fmean(rec), 4),
            "planted_recall": {"sketch4": round(hit4 / max(1, n), 4), "int8": round(hit8 / max(1, n), 4)},
            "max_abs_out_diff_vs_int8": round(float((out.float() - o8).abs().max()), 4),
            "note": "first stage scored from the int4 sketch (64 B per sampled row, contiguous); later stages int8"}


def append_study(w, steps: int) -> dict:
    """KV append (sd_append_kv), one token per call, on the workload's cache
    grown to hold `steps` more tokens (fresh inputs of the same recipe):
    - append_us: the append's two kernels per call, timed with HIP events
      carried by their dispatches, when no new key raises a scale (the
      usual case);
    - grow_us: one append whose new key raises one KV head's scale, so that
      all of that head's rows are recoded;
    - loop_us_per_token: wall time per iteration of a decode loop (decode
      step, append of that token, lengths + 1 on the device), eager
      launches, one cache (warm in the Infinity Cache)."""
    import torch
    from sparse_attention_kv_int8_amd import binding as B
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    L0 = w.max_context
    wa = w.replace(max_context=L0 + 2 * steps + 64)
    inp = make_inputs(wa, lengths=[L0] * w.batch)
    dec = B.SparseDecoder.for_workload(wa)
    k, v = to_dev(inp.k), to_dev(inp.v)
    k8 = torch.empty(inp.k.shape, dtype=torch.int8, device="cuda")
    lengths = torch.from_numpy(inp.lengths.astype(np.int32)).cuda()
    dec.sd_quantize_keys(k, lengths, k8)
    q = to_dev(inp.q_step0)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    kept = torch.empty((w.batch, w.num_kv_heads, wa.keep_total), dtype=torch.int32, device="cuda")
    from sparse_attention_kv_int8_amd.inputs import make_append_tokens
    kn, vn = make_append_tokens(wa, 1, seed=2024)
    kn, vn = to_dev(kn), to_dev(vn)
    # every new key of the timed appends stays below the scales: |N(0,1)| keys
    # are far below the cache's absmax, checked after the loop
    absmax0 = torch.empty((w.batch, w.num_kv_heads), dtype=torch.float32, device="cuda")
    absmax1 = torch.empty_like(absmax0)
    dec.sd_append_kv(kn, vn, 1, lengths, k, k8, v, absmax0)
    lengths.add_(1)
    torch.cuda.synchronize()
    dec.sd_profile_start(1 << B.SD_PROF_APPEND, steps + 8)
    for _ in range(steps // 2):
        dec.sd_append_kv(kn, vn, 1, lengths, k, k8, v, absmax1)
        lengths.add_(1)
    prof = dec.sd_profile_stop()
    assert torch.equal(absmax0, absmax1), "a timed append raised a scale"
    app_us = prof["append"][0] * 1e3 / prof["append"][1]
    # decode loop: step, append, length + 1
    for _ in range(5):
        dec.sd_decode_step(q, k, k8, v, lengths, out, kept)
        dec.sd_append_kv(kn, vn, 1, lengths, k, k8, v, None)
        lengths.add_(1)
    torch.cuda.synchronize()
    n_loop = steps // 2 - 8
    t0 = time.perf_counter()
    for _ in range(n_loop):
        dec.sd_decode_step(q, k, k8, v, lengths, out, kept)
        dec.sd_append_kv(kn, vn, 1, lengths, k, k8, v, None)
        lengths.add_(1)
    torch.cuda.synchronize()
    loop_us = (time.perf_counter() - t0) / n_loop * 1e6
    # one append that raises KV head 0's scale of every request
    big = kn.clone()
    big[:, 0, 0, 0] = 4.0 * float(absmax1.max())
    dec.sd_profile_start(1 << B.SD_PROF_APPEND, 4)
    dec.sd_append_kv(big, vn, 1, lengths, k, k8, v, absmax1)
    prof = dec.sd_profile_stop()
    assert bool((absmax1[:, 0] > absmax0[:, 0]).all()), "the growth append did not raise the scale"
    grow_us = prof["append"][0] * 1e3
    assert dec.sd_check() == 0
    del k, v, k8
    torch.cuda.empty_cache()
    return {"append_us": round(app_us, 3), "grow_us": round(grow_us, 3), "loop_us_per_token": round(loop_us, 3),
            "tokens_appended": steps // 2 + n_loop + 7,
            "note": "one token per call; grow_us recodes one KV head's rows per request; the loop is eager "
                    "(decode step + append + lengths + 1) on one warm cache"}


def stream_ceiling(mib: int = 1024) -> dict:
    """A plain streaming kernel on the same GPU, for context: torch's
    elementwise negation of a bf16 tensor of `mib` MiB into another (the
    bytes read plus the bytes written), median of 5 event-timed runs after a
    warm-up."""
    import torch
    x = torch.ones(mib * (1 << 20) // 2, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    torch.neg(x, out=y)
    times = []
    for _ in range(5):
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.neg(x, out=y)
        e.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(e) * 1e-3)
    del x, y
    torch.cuda.empty_cache()
    t = statistics.median(times)
    return {"GBs": round(2 * mib * (1 << 20) / t / 1e9, 1), "kernel": "torch.neg, bf16 copy (read + write)",
            "bytes": 2 * mib * (1 << 20)}


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        for ln in r.stdout.splitlines():
            if ln.startswith("Model name:"):
                return ln.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_baseline(w, inp, kept_gpu_bytes: float, budget_s: float = 10.0) -> dict:
    """The CPU oracle on full steps of the same inputs (one core): the key
    quantisation once, then the step repeated for about `budget_s` seconds
    of CPU work; the median step gives the rate."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:          # pragma: no cover
        threadpool_limits = None
    from oracle import sparse_decode as O
    import contextlib
    ctx = threadpool_limits(1) if threadpool_limits else contextlib.nullcontext()
    with ctx:
        t = time.perf_counter()
        k8 = np.zeros(inp.k.shape, np.int8)
        for b in range(w.batch):
            L = int(inp.lengths[b])
            for j in range(w.num_kv_heads):
                k8[b, j, :L] = O.quantize_keys(inp.k[b, j], L)[0]
        tq = time.perf_counter() - t
        cfg = O.StepConfig(tuple(O.StageSpec(s.chunk, s.stride, s.keep) for s in w.stages), w.sink, w.window,
                           1.0 / math.sqrt(w.head_dim))
        # repeated full steps until about 10 s of CPU work (at least 3, at
        # most 1000 steps), then the median step
        times = []
        while len(times) < 3 or (sum(times) + tq < budget_s and len(times) < 1000):
            t = time.perf_counter()
            O.decode_step(inp.q_step0, inp.k, k8, inp.v, inp.lengths, cfg)
            times.append(time.perf_counter() - t)
    ts = statistics.median(times)
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):      # pragma: no cover
        avail = os.cpu_count() or 1
    return {"value": round(kept_gpu_bytes / ts / 1e9, 4), "unit": "GB/s", "cores": 1,
            "cores_note": f"1 of {avail} cores available to the process (BLAS and numpy threads pinned to 1)",
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"full decode steps of {w.name}, repeated for {sum(times) + tq:.1f} s of CPU work "
                      f"({len(times)} steps, median {ts * 1e3:.1f} ms/step) after the key quantisation "
                      f"({tq:.2f} s, once)",
            "s_per_step": round(ts, 4), "quantize_s": round(tq, 3), "steps": len(times)}


def measure(w, steps: int, warmup: int, copies: int, reuse: bool = True, dense: bool = True,
            sketch: bool = True) -> tuple:
    b = Bench(w, copies)
    torch = b.torch
    b.run(warmup)
    torch.cuda.synchronize()
    # calibration: all kernels timed, to pick the dominant one
    cal = b.profile(max(20, warmup), 0xFF)          # the step's kinds (not the dense comparison)
    avg_us = {k: v[0] * 1e3 / v[1] for k, v in cal.items()}
    dominant = max((k for k in avg_us if k != "quantize"), key=lambda k: avg_us[k])
    dom_kind = KIND_NAMES.index(dominant)
    # timed region: K steps replayed from HIP graphs (one graph per cache copy)
    b.capture()
    b.replay(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    b.replay(steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    us_per_step = (t1 - t0) / steps * 1e6
    # spread: the same replays one at a time between HIP events on the
    # replay stream (outside the timed region; each step's own time)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, e) in enumerate(evs):
        a.record()
        b.graphs[i % len(b.graphs)].replay()
        e.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(e) * 1e3 for a, e in evs)
    spread = {"p10": round(per[len(per) // 10], 3), "p50": round(per[len(per) // 2], 3),
              "p90": round(per[(9 * len(per)) // 10], 3)}
    # the same K steps launched eagerly, the dominant kernel's dispatches
    # carrying HIP events on the launch stream: its live average duration
    b.dec.sd_profile_start(1 << dom_kind, steps + 8)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    b.run(steps)
    torch.cuda.synchronize()
    us_eager = (time.perf_counter() - t0) / steps * 1e6
    live = b.dec.sd_profile_stop()
    dom_us = live[dominant][0] * 1e3 / live[dominant][1]
    kept = b.kept.cpu().numpy()
    ab = algorithmic_bytes(w, kept, b.inp.lengths)
    ab["per_launch"] = kernel_bytes(ab["per_kernel"], avg_us)
    reuse = reuse_study(b, steps) if reuse and w.steps == 1 else None
    dense = dense_study(b, steps, warmup, us_per_step) if dense else None
    sketch = sketch_study(b, steps, warmup, us_per_step) if sketch else None
    return b, dict(us_per_step=us_per_step, us_eager=us_eager, avg_us=avg_us, dominant=dominant, dominant_us=dom_us,
                   bytes=ab, reuse=reuse, spread=spread, dense=dense, sketch=sketch)


def measure_hostv(w, repeats: int = 3, sketch: bool = True) -> dict:
    """The host-resident-value workload: values in pinned host memory behind
    the device LRU of 8-token blocks, over the workload's sequence of steps
    with a drifting query, each run from a cold cache.

    graph: one step captured in a HIP graph and replayed over the sequence
      (the step's query copied into the captured buffer before each replay,
      outside its timed span; the LRU's clock lives on the device), each
      replay timed with HIP events: the headline figures.
    eager: the same sequence launched eagerly, with the decode kernel (the
      one that reads the missed blocks from host memory) timed by HIP events
      on its launch stream: the PCIe rate is the missed bytes / that
      kernel's time, i.e. over the time in which the host reads happen.
    copy: the same sequence with SD_VALUE_FETCH_COPY (missed blocks gathered
      by hipMemcpyAsync on a side stream after a host wait; eager: it cannot
      be captured), for comparison.
    sketch4: the eager sequence with the first stage scored from the int4
      sketch."""
    import torch
    from sparse_attention_kv_int8_amd import binding as B
    t = time.perf_counter()
    inp = make_inputs(w)
    log(f"[bench] {w.name}: inputs generated in {time.perf_counter() - t:.1f}s")
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    dec = B.SparseDecoder.for_workload(w)
    k = to_dev(inp.k)
    v = torch.empty(inp.v.shape, dtype=torch.bfloat16, pin_memory=True)
    v.view(torch.int16).numpy()[...] = inp.v.view(np.int16)
    lengths = torch.from_numpy(inp.lengths.astype(np.int32)).cuda()
    k8 = torch.empty(inp.k.shape, dtype=torch.int8, device="cuda")
    dec.sd_profile_start(1 << B.SD_PROF_QUANTIZE, 4)
    dec.sd_quantize_keys(k, lengths, k8)
    quantize_us = dec.sd_profile_stop()["quantize"][0] * 1e3
    qs = [to_dev(inp.q[t]) for t in range(w.steps)]
    qbuf = qs[0].clone()
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    kept = torch.empty((w.batch, w.num_kv_heads, w.keep_total), dtype=torch.int32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(w.steps)]

    def sequence(step_fn, label, before=None, reps=repeats, prof_mask=0):
        runs, prof = [], {}
        for rep in range(reps):
            dec.sd_reset_value_cache()
            torch.cuda.synchronize()
            if prof_mask:
                dec.sd_profile_start(prof_mask, 8 * w.steps + 8)
            steps = []
            for t in range(w.steps):
                if before:
                    before(t)
                a, b = ev[t]
                a.record()
                step_fn(t)
                b.record()
                torch.cuda.synchronize()
                st = dec.sd_get_stats()
                steps.append((a.elapsed_time(b) * 1e3, st.last_needed, st.last_hits, st.last_misses,
                              st.last_refills, st.last_copies))
            if prof_mask:
                for kname, (ms, n) in dec.sd_profile_stop().items():
                    pm, pn = prof.get(kname, (0.0, 0))
                    prof[kname] = (pm + ms, pn + n)
            runs.append(steps)
            log(f"[bench] host-value run {rep} ({label}): {sum(x[0] for x in steps) / len(steps):.1f} us/step")
        return runs, prof

    def summary(runs):
        flat = [x for r in runs for x in r]
        needed = sum(x[1] for x in flat)
        return {"us_per_step": round(statistics.fmean(x[0] for x in flat), 3),
                "us_first_step": round(statistics.fmean(r[0][0] for r in runs), 3),
                "us_per_step_after_first": round(statistics.fmean(x[0] for r in runs for x in r[1:]), 3),
                "hit_rate": round(sum(x[2] for x in flat) / max(1, needed), 4)}

    step = lambda t: dec.sd_decode_step(qs[t], k, k8, v, lengths, out, kept)
    # eager, with the decode kernel timed: the PCIe rate
    eruns, eprof = sequence(step, "eager", prof_mask=1 << B.SD_PROF_ATTEND)
    kept_np = kept.cpu().numpy()
    eflat = [x for r in eruns for x in r]
    missed = sum(x[3] + x[4] for x in eflat) * 8 * w.head_dim * 2      # misses and refills, bytes
    attend_ms = eprof["attend"][0]
    # graph replay: the headline
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dec.sd_decode_step(qbuf, k, k8, v, lengths, out, kept)
    granal = sequence(lambda t: graph.replay(), "graph", before=lambda t: qbuf.copy_(qs[t]))[0]
    del graph
    # hit/miss sequences must agree between the eager and the replayed runs
    same = [(x[1], x[2], x[3]) for x in eruns[0]] == [(x[1], x[2], x[3]) for x in granal[0]]
    # the gathered-copy variant (eager)
    dec.sd_set_value_fetch(B.SD_VALUE_FETCH_COPY)
    cruns = sequence(step, "side-stream copies", reps=1)[0]
    dec.sd_set_value_fetch(B.SD_VALUE_FETCH_MAPPED)
    copy = summary(cruns)
    copy["copies_per_step"] = round(statistics.fmean(x[5] for x in cruns[0]), 1)
    copy["note"] = ("SD_VALUE_FETCH_COPY: host waits for the block list, one hipMemcpyAsync per run of missed "
                    "blocks on a side stream, decode kernel after them; eager launches")
    sketch4 = None
    if sketch:
        sk = torch.empty((w.batch, w.num_kv_heads, dec.sd_sketch4_rows(), 64), dtype=torch.uint8, device="cuda")
        dec.sd_quantize_sketch4(k, lengths, sk)
        runs4 = sequence(lambda t: dec.sd_decode_step_sketch4(qs[t], k, k8, sk, v, lengths, out, kept), "sketch4",
                         reps=1)[0]
        sketch4 = summary(runs4)
        sketch4["note"] = "first stage scored from the int4 sketch; same sequence, cold cache, eager"
        del sk
    g = summary(granal)
    e = summary(eruns)
    ab = algorithmic_bytes(w, kept_np, inp.lengths)
    res = dict(graph=g, eager=e, copy=copy, sketch4=sketch4, replay_matches_eager=same,
               h2d_bytes_per_step=round(missed / len(eflat)),
               pcie_GBs=round(missed / (attend_ms * 1e-3) / 1e9, 2),
               attend_us_per_step=round(attend_ms * 1e3 / len(eflat), 3),
               quantize_us=quantize_us, bytes=ab, repeats=repeats,
               per_step_us=[round(x[0], 2) for x in granal[-1]],
               per_step_hit_rate=[round(x[2] / max(1, x[1]), 4) for x in granal[-1]])
    del k, v, k8, qs, dec
    torch.cuda.empty_cache()
    return res


def hostv_summary(w, r) -> dict:
    """The host-value figures as reported inside the line."""
    return {"workload": w.name, "context": w.max_context, "value_cache_tokens": w.value_cache_tokens,
            "sequence": f"{w.steps} steps, drifting query, cold cache, {r['repeats']} runs",
            "us_per_step": r["graph"]["us_per_step"], "us_first_step": r["graph"]["us_first_step"],
            "us_per_step_after_first": r["graph"]["us_per_step_after_first"],
            "launch": "HIP graph replay (one captured step; query copied in before each replay)",
            "hit_rate": r["graph"]["hit_rate"], "replay_matches_eager": r["replay_matches_eager"],
            "eager_us_per_step": r["eager"]["us_per_step"],
            "h2d_bytes_per_step": r["h2d_bytes_per_step"], "pcie_GBs": r["pcie_GBs"],
            "pcie_note": "bytes of missed and refilled blocks read from pinned host memory / the time of the "
                         "decode kernel that reads them (eager run, HIP events on its launch stream)",
            "attend_us_per_step": r["attend_us_per_step"],
            "value_GBs": round(r["bytes"]["total"] / (r["graph"]["us_per_step"] * 1e-6) / 1e9, 2),
            "side_stream_copy": r["copy"], "sketch4": r["sketch4"]}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8b_128k", choices=sorted(WORKLOADS))
    ap.add_argument("--copies", type=int, default=0, help="KV-cache copies rotated over (0 = enough to "
                    "defeat the 256 MB Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reuse", action="store_true", help="skip the stage-reuse study (profiling runs: its "
                    "warm-cache steps would mix into the per-kernel averages)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-decode comparison (sd_dense_decode)")
    ap.add_argument("--no-append", action="store_true", help="skip the KV-append study (sd_append_kv)")
    ap.add_argument("--no-sketch", action="store_true", help="skip the int4 first-stage sketch study")
    ap.add_argument("--batched", default="ragged_b16", help="batched workload reported inside the line for "
                    "context ('' = none): the same kernels with many requests in flight")
    ap.add_argument("--secondary", default="ctx_1m", help="second workload reported inside the line ('' = none)")
    ap.add_argument("--hostv", default="ctx_3m_hostv", help="host-resident-value workload reported inside the "
                    "line ('' = none)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain elementwise copy (torch.neg) of MIB MiB three times: the "
                         "reference that scales hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1"}))
        log("bench.py: one GPU only (the (request, KV head) pipelines are independent and shard across "
            "GPUs without communication, but only the one-GPU step is measured)")
        return 2
    w = WORKLOADS[args.workload]
    if w.values_on_host:
        r = measure_hostv(w)
        total = r["bytes"]["total"]
        h = hostv_summary(w, r)
        us = h["us_per_step"]
        print(json.dumps({
            "metric": METRIC + " [host-resident values]",
            "value": round(total / (us * 1e-6) / 1e9, 2),
            "unit": "GB/s", "n_gpus": 1, "steps": w.steps * r["repeats"], "warmup": 0,
            "ms_per_step": round(us / 1e3, 6), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "int8+fp32", "data": "synthetic (seeded; shapes and distributions of the workload)",
            "config": {"workload": w.name, "batch": w.batch, "context": w.max_context,
                       "gqa": f"{w.num_q_heads}/{w.num_kv_heads}", "stages": [[s.chunk, s.stride, s.keep] for s in w.stages],
                       "sink": w.sink, "window": w.window, "value_cache_tokens": w.value_cache_tokens,
                       "sequence": h["sequence"], "launch": h["launch"]},
            "tokens_per_s": round(w.batch / (us * 1e-6), 1),
            "algorithmic_bytes": total,
            "quantize_keys_us": round(r["quantize_us"], 2),
            "hostv": h,
            "per_step_us": r["per_step_us"], "per_step_hit_rate": r["per_step_hit_rate"],
        }), flush=True)
        return 0

    def auto_copies(wl):
        if args.copies:
            return args.copies
        est = 38e6 if wl.max_context <= 131072 else 160e6
        est *= wl.batch if wl.batch > 1 else 1
        return max(2, min(16, math.ceil(600e6 / est) + 1))

    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    b, r = measure(w, args.steps, args.warmup, auto_copies(w), not args.no_reuse, not args.no_dense,
                   not args.no_sketch)
    total = r["bytes"]["total"]
    dom_bytes = r["bytes"]["per_launch"][r["dominant"]]
    achieved = dom_bytes / (r["dominant_us"] * 1e-6) / 1e9
    sum_kernel_us = sum(v for k, v in r["avg_us"].items() if k != "quantize")
    from sparse_attention_kv_int8_amd.profiling import load_traffic
    tr = load_traffic(w.name, r["dominant"])
    line = {
        "metric": METRIC,
        "value": round(total / (r["us_per_step"] * 1e-6) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["us_per_step"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+fp32",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": w.name, "batch": w.batch, "context": w.max_context, "gqa": f"{w.num_q_heads}/{w.num_kv_heads}",
                   "stages": [[s.chunk, s.stride, s.keep] for s in w.stages], "sink": w.sink, "window": w.window,
                   "cache": f"cold: {len(b.args)} rotating copies", "launch": "HIP graph replay, one step per graph"},
        "us_per_step": round(r["us_per_step"], 3),
        "us_per_step_spread": r["spread"],
        "us_per_step_eager": round(r["us_eager"], 3),
        "tokens_per_s": round(w.batch / (r["us_per_step"] * 1e-6), 1),
        "algorithmic_bytes": total,
        "roofline": {"bound": "hbm", "kernel": r["dominant"], "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": tr["traffic_bytes"] if tr else None, "bytes_per_launch": dom_bytes,
                     "avg_launch_us": round(r["dominant_us"], 3)},
        "step_kernels_us": {k: round(v, 3) for k, v in r["avg_us"].items()},
        "per_kernel_frac": kernel_fracs(r["bytes"]["per_launch"], r["avg_us"]),
        "step_roofline": {"achieved": round(total / (sum_kernel_us * 1e-6) / 1e9, 2), "unit": "GB/s",
                          "frac": round(total / (sum_kernel_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                          "note": "all per-step bytes / sum of per-step kernel durations"},
        "quantize_keys_us": round(b.quantize_us, 2),
        "reuse": r["reuse"],
        "dense": r["dense"],
        "sketch4": r["sketch"],
    }
    inp, kb = b.inp, total
    del b
    b_torch = __import__("torch")
    b_torch.cuda.empty_cache()
    if not args.no_append:
        line["append"] = append_study(w, args.steps)
    if args.secondary and args.secondary != w.name:
        w2 = WORKLOADS[args.secondary]
        b2, r2 = measure(w2, max(20, args.steps // 2), args.warmup, auto_copies(w2), not args.no_reuse,
                         not args.no_dense, not args.no_sketch)
        t2 = r2["bytes"]["total"]
        line["secondary"] = {"workload": w2.name, "us_per_step": round(r2["us_per_step"], 3),
                             "value_GBs": round(t2 / (r2["us_per_step"] * 1e-6) / 1e9, 2),
                             "algorithmic_bytes": t2, "step_kernels_us": {k: round(v, 3) for k, v in r2["avg_us"].items()},
                             "dominant": r2["dominant"],
                             "dominant_frac": round(r2["bytes"]["per_launch"][r2["dominant"]] /
                                                    (r2["dominant_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                             "dominant_traffic": (load_traffic(w2.name, r2["dominant"]) or {}).get("traffic_bytes"),
                             "per_kernel_frac": kernel_fracs(r2["bytes"]["per_launch"], r2["avg_us"]),
                             "quantize_keys_us": round(b2.quantize_us, 2), "reuse": r2["reuse"],
                             "dense": r2["dense"], "sketch4": r2["sketch"]}
        del b2
        b_torch.cuda.empty_cache()
    if args.batched and args.batched != w.name:
        w3 = WORKLOADS[args.batched]
        b3, r3 = measure(w3, max(20, args.steps // 4), args.warmup, auto_copies(w3), False, False, False)
        t3 = r3["bytes"]["total"]
        line["batched"] = {"workload": w3.name, "batch": w3.batch, "us_per_step": round(r3["us_per_step"], 3),
                           "value_GBs": round(t3 / (r3["us_per_step"] * 1e-6) / 1e9, 2),
                           "frac": round(t3 / (r3["us_per_step"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                           "algorithmic_bytes": t3, "tokens_per_s": round(w3.batch / (r3["us_per_step"] * 1e-6), 1),
                           "step_kernels_us": {k: round(v, 3) for k, v in r3["avg_us"].items()},
                           "dominant": r3["dominant"],
                           "dominant_frac": round(r3["bytes"]["per_launch"][r3["dominant"]] /
                                                  (r3["dominant_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                           "per_kernel_frac": kernel_fracs(r3["bytes"]["per_launch"], r3["avg_us"]),
                           "note": "context: the same kernels with 16 requests of ragged lengths in flight"}
        del b3
        b_torch.cuda.empty_cache()
    # the pruning and decode kernels against 60% of 8 TB/s, at 128K (this
    # line) and 1M (the secondary workload) context
    if w.name == "llama8b_128k" and "secondary" in line and line["secondary"]["workload"] == "ctx_1m":
        f128 = line["per_kernel_frac"]["prune_and_decode"]
        f1m = line["secondary"]["per_kernel_frac"]["prune_and_decode"]
        line["target"] = {"bound": 0.6, "frac_128k": f128, "frac_1m": f1m, "met": f128 >= 0.6 and f1m >= 0.6,
                          "note": "algorithmic bytes of the pruning and decode kernels / the sum of their "
                                  "average durations, as a fraction of 8 TB/s"}
    if args.hostv and args.hostv != w.name:
        w4 = WORKLOADS[args.hostv]
        line["hostv"] = hostv_summary(w4, measure_hostv(w4, repeats=2, sketch=not args.no_sketch))
    if not args.copy_calibration:            # its copies would mix with the calibration copies
        line["stream_ceiling"] = stream_ceiling()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on one step ...")
        line["cpu_baseline"] = oracle_baseline(w, inp, kb)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

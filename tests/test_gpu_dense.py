"""GPU parity of the dense decode (sd_dense_decode) against the oracle's dense
attention: softmax(q K^T / sqrt(d)) V over every cached token t < L_b, in
fp64 on the CPU.  Bar: max |bf16 output - fp64| <= 8e-3 on every checked
(request, query head).  Shapes span several splits and ragged tails (lengths
that are not multiples of 8, a single token, fewer blocks than splits); the
full-size workloads run in the launch configuration the benchmark times,
with the oracle on sampled heads.
"""
import numpy as np
import pytest

from oracle import sparse_decode as O
from sparse_attention_kv_int8_amd.inputs import WORKLOADS, make_inputs, tiny_workload
from tests.gpu_util import OUT_TOL, bf16_dev_to_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import sparse_attention_kv_int8_amd.binding  # noqa: F401  (fails loudly when unbuilt)
    yield
    torch.cuda.synchronize()


def dense_oracle(inp, b, h):
    w = inp.workload
    L = int(inp.lengths[b])
    j = h // w.group
    return O.dense_attention(O.bf16_to_f64(inp.q_step0[b, h]), O.bf16_to_f64(inp.k[b, j, :L]),
                             O.bf16_to_f64(inp.v[b, j, :L]), 1.0 / np.sqrt(w.head_dim))


class DenseRun:
    def __init__(self, inp, lengths_dev=None):
        import torch
        from sparse_attention_kv_int8_amd.binding import SparseDecoder
        w = inp.workload
        self.torch, self.inp, self.w = torch, inp, w
        self.dec = SparseDecoder.for_workload(w)
        self.q = to_dev_bf16(inp.q_step0)
        self.k = to_dev_bf16(inp.k)
        self.v = to_dev_bf16(inp.v)
        lens = inp.lengths if lengths_dev is None else lengths_dev
        self.lengths = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
        self.out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")

    def run(self):
        self.out.fill_(7.0)
        self.dec.sd_dense_decode(self.q, self.k, self.v, self.lengths, self.out)
        self.torch.cuda.synchronize()
        return O.bf16_to_f64(bf16_dev_to_bits(self.out))


def check(inp, got, pairs):
    err = 0.0
    omax = 0.0
    for b, h in pairs:
        ref = dense_oracle(inp, b, h)
        e = float(np.abs(got[b, h] - ref).max())
        assert e <= OUT_TOL, f"request {b}, head {h}: max |err| = {e}"
        err, omax = max(err, e), max(omax, float(np.abs(ref).max()))
    print(f"  {len(pairs)} heads, max|err| = {err:.2e}, max|o| = {omax:.3f}", flush=True)
    return err


def all_pairs(w):
    return [(b, h) for b in range(w.batch) for h in range(w.num_q_heads)]


@pytest.mark.parametrize("hq,hkv,lengths", [
    (8, 2, [8192, 5003]),           # G = 4, a ragged tail
    (4, 2, [1, 4097]),              # G = 2, one token; one block past a power of two
    (2, 2, [9, 8191]),              # G = 1, one full block + 1 token; last block 7 tokens
    (8, 2, [8, 16]),                # fewer blocks than splits
])
def test_dense_small(hq, hkv, lengths):
    w = tiny_workload(name="dense_small", batch=len(lengths), num_q_heads=hq, num_kv_heads=hkv,
                      max_context=8192)
    print(f"case dense B={w.batch} Hq={hq} Hkv={hkv} lengths={lengths}", flush=True)
    inp = make_inputs(w, lengths=lengths)
    g = DenseRun(inp)
    got = g.run()
    check(inp, got, all_pairs(w))
    assert g.dec.sd_check() == 0


def test_dense_bad_length_flags_and_isolates():
    """A length outside [1, Lmax] gives a zero output for that request and
    raises the device flag; the other request is untouched."""
    w = tiny_workload(name="dense_bad", batch=3, num_q_heads=8, num_kv_heads=2, max_context=4096)
    inp = make_inputs(w, lengths=[4096, 100, 2000])
    print("case dense bad lengths [4096, 0, 4097]", flush=True)
    g = DenseRun(inp, lengths_dev=[4096, 0, 4097])
    got = g.run()
    assert np.all(got[1] == 0) and np.all(got[2] == 0)
    check(inp, got, [(0, h) for h in range(w.num_q_heads)])
    from sparse_attention_kv_int8_amd.binding import SD_ERR_DEVICE_FLAG
    assert g.dec.sd_check() == SD_ERR_DEVICE_FLAG
    assert g.dec.sd_check() == 0


def test_dense_rejects_host_values():
    import torch
    from sparse_attention_kv_int8_amd.binding import SD_ERR_UNSUPPORTED, SDError
    w = WORKLOADS["ctx_3m_hostv"].replace(max_context=65536, value_cache_tokens=8192, steps=1)
    from sparse_attention_kv_int8_amd.binding import SparseDecoder
    dec = SparseDecoder.for_workload(w)
    q = torch.zeros((1, 32, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 8, 64, 128), dtype=torch.bfloat16, device="cuda")
    lengths = torch.ones(1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(SDError) as e:
        dec.sd_dense_decode(q, k, k, lengths, out)
    assert e.value.status == SD_ERR_UNSUPPORTED


def test_dense_repeat_is_bit_identical_and_graph_replays_match():
    """Repeated calls give identical bits; a captured call replays to the
    eager result, with eager work and synchronisations between replays."""
    import torch
    w = WORKLOADS["llama8b_128k"].replace(max_context=32768, planted=16)
    inp = make_inputs(w)
    g = DenseRun(inp)
    a = g.run()
    b = g.run()
    assert np.array_equal(a, b)
    out_g = torch.empty_like(g.out)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        g.dec.sd_dense_decode(g.q, g.k, g.v, g.lengths, out_g)
    for rep in range(3):
        out_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(O.bf16_to_f64(bf16_dev_to_bits(out_g)), a), rep
        g.run()
    check(inp, a, [(0, h) for h in (0, 5, 17, 31)])


@pytest.mark.parametrize("name", ["llama8b_128k", "ragged_b16", "ctx_1m"])
def test_dense_full_workload(name):
    """Full-size workloads in the benchmark's launch configuration; the oracle
    checks every head at 128K, every head of three requests (the shortest,
    the longest and the first) of the ragged batch, and two KV heads' query
    groups at 1M."""
    w = WORKLOADS[name]
    print(f"case dense full {name}", flush=True)
    inp = make_inputs(w)
    g = DenseRun(inp)
    got = g.run()
    if name == "llama8b_128k":
        pairs = all_pairs(w)
    elif name == "ragged_b16":
        bs = sorted({0, int(np.argmin(inp.lengths)), int(np.argmax(inp.lengths))})
        pairs = [(b, h) for b in bs for h in range(w.num_q_heads)]
    else:
        pairs = [(0, h) for h in list(range(0, 4)) + list(range(28, 32))]
    check(inp, got, pairs)
    assert g.dec.sd_check() == 0

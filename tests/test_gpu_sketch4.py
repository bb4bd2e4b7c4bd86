"""GPU parity of the int4 first-stage sketch (sd_quantize_sketch4,
sd_decode_step_sketch4) against the oracle (key_sketch4; decode_step with
sketch4).  Bar: sketch codes, first-stage scores and every stage's kept
set bit-exact; outputs within 8e-3 of fp64.  The 4-bit codes make equal
chunk scores common, so the lower-start tie rule is exercised throughout.
"""
import numpy as np
import pytest

from oracle import sparse_decode as O
from sparse_attention_kv_int8_amd.inputs import WORKLOADS, Stage, make_inputs, tiny_workload
from tests.gpu_util import GpuRun, bf16_dev_to_bits, compare_step, oracle_config, oracle_keys, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import sparse_attention_kv_int8_amd.binding  # noqa: F401  (fails loudly when unbuilt)
    yield
    torch.cuda.synchronize()


def sketch_ref(inp):
    w = inp.workload
    r1 = w.stages[0].stride
    return [[O.key_sketch4(inp.k[b, j], int(inp.lengths[b]), r1) for j in range(w.num_kv_heads)]
            for b in range(w.batch)]


def unpack(sk: np.ndarray) -> np.ndarray:
    """uint8 [..][64] two's-complement nibbles (channel 2m low, 2m + 1 high) -> int8 codes [..][128]."""
    out = np.empty(sk.shape[:-1] + (128,), np.int8)
    out[..., 0::2] = ((sk & 15).astype(np.int8) ^ 8) - 8
    out[..., 1::2] = ((sk >> 4).astype(np.int8) ^ 8) - 8
    return out


def run_sketch_case(w, lengths=None, check_scores=True):
    import torch
    print(f"case sketch4 {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} Lmax={w.max_context} "
          f"stages={[(s.chunk, s.stride, s.keep) for s in w.stages]} hostv={w.values_on_host}", flush=True)
    inp = make_inputs(w, lengths=lengths)
    g = GpuRun(inp)
    g.quantize()
    rows = g.dec.sd_sketch4_rows()
    r1 = w.stages[0].stride
    assert rows == -(-w.max_context // r1)
    sk = torch.zeros((w.batch, w.num_kv_heads, rows, 64), dtype=torch.uint8, device="cuda")
    g.dec.sd_quantize_sketch4(g.k, g.lengths, sk)
    torch.cuda.synchronize()
    ref = sketch_ref(inp)
    got = unpack(sk.cpu().numpy())
    for b in range(w.batch):
        n = -(-int(inp.lengths[b]) // r1)
        for j in range(w.num_kv_heads):
            assert np.array_equal(got[b, j, :n], ref[b][j]), f"sketch codes differ (request {b}, head {j})"
    k8_ref, _ = oracle_keys(inp)
    q = to_dev_bf16(inp.q_step0)
    g.dec.sd_decode_step_sketch4(q, g.k, g.k8, sk, g.v, g.lengths, g.out, g.kept)
    torch.cuda.synchronize()
    out, kept = bf16_dev_to_bits(g.out), g.kept.cpu().numpy()
    res = O.decode_step(inp.q_step0, inp.k, k8_ref, inp.v, inp.lengths, oracle_config(w), sketch4=ref)
    _, err, omax = compare_step(inp, inp.q_step0, k8_ref, out, kept, ref=res)
    if check_scores:
        # first-stage chunk scores from the sketch, every chunk
        sc = g.stage_scores(0)
        st = w.stages[0]
        for b in range(w.batch):
            L = int(inp.lengths[b])
            for j in range(w.num_kv_heads):
                n = sc.shape[2]
                starts = np.arange(n, dtype=np.int64) * st.chunk
                valid = starts < L
                want = np.full(n, np.iinfo(np.int32).min, dtype=np.int64)
                S4 = lambda t, b=b, j=j: O.token_scores(res.Q[b, j], ref[b][j][t.reshape(-1) // st.stride]).reshape(t.shape)
                want[valid] = O.chunk_scores(S4, starts[valid], st.chunk, st.stride, L)
                assert np.array_equal(sc[b, j].astype(np.int64), want), f"first-stage scores differ ({b}, {j})"
    assert g.dec.sd_check() == 0
    print(f"  max|err| = {err:.2e}, max|o| = {omax:.3f}", flush=True)
    return g, res


@pytest.mark.parametrize("hq,hkv,lengths", [
    (8, 2, [16384, 9001]),
    (4, 2, [12345, 300]),
    (2, 2, [16384, 1]),
])
def test_sketch_small(hq, hkv, lengths):
    w = tiny_workload(name="sketch_small", batch=len(lengths), num_q_heads=hq, num_kv_heads=hkv)
    run_sketch_case(w, lengths=lengths)


def test_sketch_other_first_stride():
    """First stage (64, 4, 24): a denser sketch (every 4th row)."""
    w = tiny_workload(name="sketch_r4", batch=2, num_q_heads=8, num_kv_heads=2, max_context=8192,
                      stages=(Stage(64, 4, 24), Stage(16, 2, 48), Stage(8, 1, 60)))
    run_sketch_case(w, lengths=[8192, 5555])


def test_sketch_host_values():
    """Values in pinned host memory behind the value cache."""
    w = WORKLOADS["ctx_3m_hostv"].replace(max_context=65536, value_cache_tokens=8192, steps=1, planted=16)
    run_sketch_case(w)


def test_sketch_fused_two_stages_unsupported():
    import torch
    from sparse_attention_kv_int8_amd.binding import SD_ERR_UNSUPPORTED, SDError, SparseDecoder
    w = tiny_workload(name="sketch_2st", stages=(Stage(64, 2, 16), Stage(8, 1, 64)), max_context=4096)
    dec = SparseDecoder.for_workload(w)
    z = torch.zeros((1, 1, 4096, 128), dtype=torch.bfloat16, device="cuda")
    z8 = torch.zeros((1, 1, 4096, 128), dtype=torch.int8, device="cuda")
    sk = torch.zeros((1, 1, dec.sd_sketch4_rows(), 64), dtype=torch.uint8, device="cuda")
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    lengths = torch.full((1,), 4096, dtype=torch.int32, device="cuda")
    kept = torch.empty((1, 1, 80), dtype=torch.int32, device="cuda")
    import os
    if os.environ.get("SD_FUSE_LAST_STAGE", "1") == "0":
        pytest.skip("fusion switched off")
    with pytest.raises(SDError) as e:
        dec.sd_decode_step_sketch4(q, z, z8, sk, z, lengths, q, kept)
    assert e.value.status == SD_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["llama8b_128k", "ragged_b16", "ctx_1m"])
def test_sketch_full_workload(name):
    run_sketch_case(WORKLOADS[name], check_scores=name == "llama8b_128k")


def test_sketch_graph_replays_match_eager():
    """A sketch step captured into a HIP graph replays to the eager result,
    with eager steps and synchronisations between the replays; repeated
    eager steps are bit-identical."""
    import torch
    w = WORKLOADS["llama8b_128k"].replace(max_context=32768, planted=16)
    print("case sketch4 graph capture", flush=True)
    inp = make_inputs(w)
    g = GpuRun(inp)
    g.quantize()
    sk = torch.zeros((w.batch, w.num_kv_heads, g.dec.sd_sketch4_rows(), 64), dtype=torch.uint8, device="cuda")
    g.dec.sd_quantize_sketch4(g.k, g.lengths, sk)
    q = to_dev_bf16(inp.q_step0)

    def eager():
        g.dec.sd_decode_step_sketch4(q, g.k, g.k8, sk, g.v, g.lengths, g.out, g.kept)
        torch.cuda.synchronize()
        return bf16_dev_to_bits(g.out).copy(), g.kept.cpu().numpy().copy()

    out_e, kept_e = eager()
    out2, kept2 = eager()
    assert np.array_equal(out_e, out2) and np.array_equal(kept_e, kept2)
    out_g = torch.empty_like(g.out)
    kept_g = torch.empty_like(g.kept)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        g.dec.sd_decode_step_sketch4(q, g.k, g.k8, sk, g.v, g.lengths, out_g, kept_g)
    for rep in range(3):
        out_g.zero_()
        kept_g.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_dev_to_bits(out_g), out_e), rep
        assert np.array_equal(kept_g.cpu().numpy(), kept_e), rep
        eager()


def test_side_stream_matches_default_stream():
    """The sketch, the sketch step, the dense decode and the KV append
    enqueued on a non-default stream give the same bits as on the default
    stream (two contexts, one per stream, on copies of the same cache)."""
    import torch
    from sparse_attention_kv_int8_amd.inputs import make_append_tokens
    w = tiny_workload(name="streams", batch=2, num_q_heads=8, num_kv_heads=2, max_context=8192)
    print("case side stream (sketch, dense, append)", flush=True)
    inp = make_inputs(w, lengths=[8000, 3001])
    k_new, v_new = make_append_tokens(w, 5, seed=9)
    results = []
    for side in (False, True):
        s = torch.cuda.Stream() if side else None
        g = GpuRun(inp, stream=s)
        ctx = torch.cuda.stream(s) if side else torch.cuda.stream(torch.cuda.current_stream())
        with ctx:
            g.quantize()
            sk = torch.zeros((w.batch, w.num_kv_heads, g.dec.sd_sketch4_rows(), 64), dtype=torch.uint8,
                             device="cuda")
            g.dec.sd_quantize_sketch4(g.k, g.lengths, sk, stream=s)
            q = to_dev_bf16(inp.q_step0)
            g.dec.sd_decode_step_sketch4(q, g.k, g.k8, sk, g.v, g.lengths, g.out, g.kept, stream=s)
            out_dense = torch.empty_like(g.out)
            g.dec.sd_dense_decode(q, g.k, g.v, g.lengths, out_dense, stream=s)
            g.dec.sd_append_kv(to_dev_bf16(k_new), to_dev_bf16(v_new), 5, g.lengths, g.k, g.k8, g.v, g.absmax,
                               stream=s, k_sketch4=sk)
            (s or torch.cuda.current_stream()).synchronize()
        results.append([bf16_dev_to_bits(g.out), g.kept.cpu().numpy(), bf16_dev_to_bits(out_dense),
                        g.k8.cpu().numpy(), sk.cpu().numpy(), g.absmax.cpu().numpy()])
        assert g.dec.sd_check(stream=s) == 0
    for a, b in zip(*results):
        assert np.array_equal(a, b)

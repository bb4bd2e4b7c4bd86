"""The seeded input generator: determinism, shapes and the stated recipe."""
import numpy as np

from sparse_attention_kv_int8_amd.inputs import (WORKLOADS, PAD_BF16, bf16_bits_to_f32,
                                                 draw_lengths, f32_to_bf16_bits, make_inputs,
                                                 tiny_workload)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7, -2.5, 3.0 + 2 ** -9], np.float32)
    b = f32_to_bf16_bits(x)
    # 1+2^-8 is halfway between 1 and 1+2^-7 -> even (1); 1+3*2^-8 -> 1+2^-6
    assert list(bf16_bits_to_f32(b)) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, 3.0]


def test_tiny_workload_is_deterministic_and_shaped():
    w = tiny_workload(max_context=2048)
    a = make_inputs(w)
    b = make_inputs(w)
    assert a.q.shape == (1, 4, 128) and a.k.shape == (1, 1, 2048, 128)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    c = make_inputs(w, seed=5)
    assert not np.array_equal(a.k, c.k)
    pos = a.planted[0][0]
    assert len(pos) == 16 and len(set(pos.tolist())) == 16
    assert pos.min() >= w.sink and pos.max() < 2048 - w.window
    vals = bf16_bits_to_f32(a.k[0, 0]).astype(np.float64)
    assert abs(vals.mean()) < 0.05 and abs(vals.std() - 1) < 0.05


def test_ragged_lengths_and_padding():
    w = WORKLOADS["ragged_b16"]
    L = draw_lengths(w)
    assert L.shape == (16,) and np.all(L % 256 == 0) and L.min() >= 32768 and L.max() <= 131072
    small = w.replace(batch=2, max_context=4096, num_q_heads=8, num_kv_heads=2)
    inp = make_inputs(small, lengths=[1000, 4096])
    assert np.all(inp.k[0, :, 1000:] == PAD_BF16) and np.all(inp.v[0, :, 1000:] == PAD_BF16)


def test_drifting_queries():
    w = WORKLOADS["ctx_3m_hostv"].replace(max_context=1024, steps=4, planted=8)
    inp = make_inputs(w)
    assert inp.q.shape == (4, 1, 32, 128)
    q = bf16_bits_to_f32(inp.q).astype(np.float64)
    corr = np.corrcoef(q[0].ravel(), q[1].ravel())[0, 1]
    assert 0.8 < corr < 0.97

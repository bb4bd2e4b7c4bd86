"""The C ABI library: loads, exports every symbol include/sd.h declares, and
reports configuration errors before touching the GPU."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sd.h")

B = pytest.importorskip("sparse_attention_kv_int8_amd.binding")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sd_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(B.lib, n), n
    assert set(names) == set(B.EXPORTED)


def test_struct_layout_matches_header():
    # sd_config: 4 int32, int64, int32, 4 stages of 3 int32, 2 int32, float, int32, int64
    assert C.sizeof(B.sd_stage) == 12
    assert B.sd_config.max_context.offset == 16
    assert B.sd_config.stage.offset == 28
    assert B.sd_config.value_cache_tokens.offset == 96
    assert C.sizeof(B.sd_config) == 104
    assert C.sizeof(B.sd_stats) == 88


def test_status_strings():
    for s in range(6):
        assert B.lib.sd_status_string(s)
    assert b"unknown" in B.lib.sd_status_string(99)


def _cfg(**kw):
    base = dict(batch=1, num_q_heads=32, num_kv_heads=8, max_context=131072,
                stages=[(256, 8, 64), (32, 2, 128), (8, 1, 256)], sink=64, window=1024)
    base.update(kw)
    return B.make_config(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), B.SD_ERR_INVALID_ARG),
    (dict(num_q_heads=30), B.SD_ERR_INVALID_ARG),          # not a multiple of Hkv
    (dict(num_q_heads=64), B.SD_ERR_UNSUPPORTED),          # G = 8
    (dict(head_dim=64), B.SD_ERR_UNSUPPORTED),
    (dict(max_context=0), B.SD_ERR_INVALID_ARG),
    (dict(stages=[]), B.SD_ERR_INVALID_ARG),
    (dict(stages=[(256, 7, 64)]), B.SD_ERR_INVALID_ARG),    # stride does not divide chunk
    (dict(stages=[(256, 8, 64), (48, 2, 8)]), B.SD_ERR_INVALID_ARG),   # 48 does not divide 256
    (dict(stages=[(256, 8, 64), (32, 2, 128), (4, 1, 256)]), B.SD_ERR_UNSUPPORTED),  # last chunk % 8
    (dict(stages=[(256, 2, 64)]), B.SD_ERR_UNSUPPORTED),    # 128 samples per chunk
    (dict(max_context=1 << 30), B.SD_ERR_UNSUPPORTED),      # too many stage-1 chunks for LDS select
    (dict(sink=-1), B.SD_ERR_INVALID_ARG),
    (dict(values_on_host=True, value_cache_tokens=100), B.SD_ERR_INVALID_ARG),
    (dict(values_on_host=True, value_cache_tokens=1024), B.SD_ERR_INVALID_ARG),  # < one step's blocks
])
def test_bad_configs_are_rejected_without_gpu(kw, status):
    cfg = _cfg(**kw)
    h = C.c_void_p(123)
    assert B.lib.sd_create(C.byref(cfg), C.byref(h)) == status
    assert h.value is None


def test_null_arguments():
    h = C.c_void_p()
    assert B.lib.sd_create(None, C.byref(h)) == B.SD_ERR_INVALID_ARG
    assert B.lib.sd_create(C.byref(_cfg()), None) == B.SD_ERR_INVALID_ARG
    B.lib.sd_destroy(None)                                  # no-op
    assert B.lib.sd_decode_step(None, None, None, None, None, None, None, None, None) == B.SD_ERR_INVALID_ARG
    assert B.lib.sd_quantize_keys(None, None, None, None, None, None) == B.SD_ERR_INVALID_ARG
    assert B.lib.sd_check(None, None) == B.SD_ERR_INVALID_ARG
    assert B.lib.sd_stage_candidates(None, 0) == -1


def test_single_hip_runtime_in_process():
    """The binding loads torch first, so libsd.so binds to torch's HIP runtime
    instead of mapping a second one."""
    maps = open("/proc/self/maps").read()
    hip = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(hip) == 1, hip


def test_candidate_limit_is_exact():
    """n_1 + keep_1 = 15872 passes validation (on a machine without a GPU the
    create then fails in the HIP runtime, not in validation); 15873 is
    rejected as unsupported."""
    ok = _cfg(max_context=8 * 15808, stages=[(8, 8, 64)])
    over = _cfg(max_context=8 * 15809, stages=[(8, 8, 64)])
    h = C.c_void_p()
    st = B.lib.sd_create(C.byref(ok), C.byref(h))
    assert st not in (B.SD_ERR_INVALID_ARG, B.SD_ERR_UNSUPPORTED)
    if st == B.SD_OK:
        B.lib.sd_destroy(h)
    h = C.c_void_p(123)
    assert B.lib.sd_create(C.byref(over), C.byref(h)) == B.SD_ERR_UNSUPPORTED
    assert h.value is None


def test_null_arguments_of_the_other_entry_points():
    assert B.lib.sd_dense_decode(None, None, None, None, None, None, None) == B.SD_ERR_INVALID_ARG
    assert B.lib.sd_append_kv(None, None, None, 1, None, None, None, None, None, None, None) == B.SD_ERR_INVALID_ARG
    assert B.lib.sd_quantize_sketch4(None, None, None, None, None) == B.SD_ERR_INVALID_ARG
    assert B.lib.sd_decode_step_sketch4(None, None, None, None, None, None, None, None, None, None) == \
        B.SD_ERR_INVALID_ARG
    assert B.lib.sd_decode_step_reuse(None, None, None, None, None, None, None, None, 0, None) == B.SD_ERR_INVALID_ARG
    assert B.lib.sd_sketch4_rows(None) == -1

"""ctypes binding of libsd.so (the C ABI in include/sd.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind these calls.  Tensors are torch tensors used as device (or
pinned host) memory; bf16 tensors travel as their bit patterns.  Importing
this module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SD_LIBRARY", os.path.join(PKG, "libsd.so"))

SD_MAX_STAGES = 4
SD_OK, SD_ERR_INVALID_ARG, SD_ERR_UNSUPPORTED, SD_ERR_OUT_OF_MEMORY, SD_ERR_HIP, SD_ERR_DEVICE_FLAG = range(6)


class sd_stage(C.Structure):
    _fields_ = [("chunk", C.c_int32), ("stride", C.c_int32), ("keep", C.c_int32)]


class sd_config(C.Structure):
    _fields_ = [
        ("batch", C.c_int32),
        ("num_q_heads", C.c_int32),
        ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("max_context", C.c_int64),
        ("num_stages", C.c_int32),
        ("stage", sd_stage * SD_MAX_STAGES),
        ("sink", C.c_int32),
        ("window", C.c_int32),
        ("softmax_scale", C.c_float),
        ("values_on_host", C.c_int32),
        ("value_cache_tokens", C.c_int64),
    ]


SD_PROF_KINDS = 10
SD_PROF_STAGE0, SD_PROF_VALUE_CACHE, SD_PROF_ATTEND, SD_PROF_QUANTIZE = 0, 4, 5, 6
SD_PROF_COMBINE, SD_PROF_DENSE, SD_PROF_APPEND = 7, 8, 9
SD_VALUE_FETCH_MAPPED, SD_VALUE_FETCH_COPY = 0, 1
PROF_NAMES = ["stage0", "stage1", "stage2", "stage3", "value_cache", "attend", "quantize", "combine", "dense",
              "append"]


class sd_profile(C.Structure):
    _fields_ = [("ms", C.c_float * SD_PROF_KINDS), ("launches", C.c_int32 * SD_PROF_KINDS)]


class sd_stats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("steps", "blocks_needed", "hits", "misses", "h2d_bytes",
                                         "last_needed", "last_hits", "last_misses", "refills", "last_refills",
                                         "last_copies")]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_attention_kv_int8_amd.build` "
                      "(there is no fallback implementation)")
# torch provides device memory and streams and brings its own HIP runtime.
# It must be loaded first: libsd.so then binds to that already-loaded runtime
# (same SONAME) instead of loading a second HIP runtime into the process.
import torch  # noqa: E402,F401
lib = C.CDLL(LIB_PATH)

_p = C.c_void_p
_SIGS = {
    "sd_create": (C.c_int, [C.POINTER(sd_config), C.POINTER(_p)]),
    "sd_destroy": (None, [_p]),
    "sd_status_string": (C.c_char_p, [C.c_int]),
    "sd_last_error": (C.c_char_p, []),
    "sd_quantize_keys": (C.c_int, [_p, _p, _p, _p, _p, _p]),
    "sd_decode_step": (C.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "sd_decode_step_reuse": (C.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, C.c_int32, _p]),
    "sd_decode_step_noalloc": (C.c_int, [C.POINTER(sd_config), _p, _p, _p, _p, _p, _p, _p, _p]),
    "sd_dense_decode": (C.c_int, [_p, _p, _p, _p, _p, _p, _p]),
    "sd_append_kv": (C.c_int, [_p, _p, _p, C.c_int32, _p, _p, _p, _p, _p, _p, _p]),
    "sd_sketch4_rows": (C.c_int64, [_p]),
    "sd_quantize_sketch4": (C.c_int, [_p, _p, _p, _p, _p]),
    "sd_decode_step_sketch4": (C.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "sd_quantize_query": (C.c_int, [_p, _p, _p, _p, _p]),
    "sd_stage_scores": (C.c_int, [_p, C.c_int32, _p, C.c_int64, _p]),
    "sd_record_attended": (C.c_int, [_p, _p, C.c_int64]),
    "sd_set_value_fetch": (C.c_int, [_p, C.c_int32]),
    "sd_stage_candidates": (C.c_int64, [_p, C.c_int32]),
    "sd_check": (C.c_int, [_p, _p]),
    "sd_get_stats": (C.c_int, [_p, C.POINTER(sd_stats), _p]),
    "sd_reset_value_cache": (C.c_int, [_p, _p]),
    "sd_profile_start": (C.c_int, [_p, C.c_uint32, C.c_int32]),
    "sd_profile_stop": (C.c_int, [_p, C.POINTER(sd_profile)]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args
EXPORTED = tuple(_SIGS)


class SDError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        detail = lib.sd_last_error().decode(errors="replace") if status == SD_ERR_HIP else ""
        super().__init__(f"{what}: {lib.sd_status_string(status).decode()} (status {status})"
                         + (f" [{detail}]" if detail else ""))


def check(status: int, what: str) -> None:
    if status != SD_OK:
        raise SDError(status, what)


def make_config(batch: int, num_q_heads: int, num_kv_heads: int, max_context: int,
                stages: Sequence, sink: int, window: int, head_dim: int = 128,
                softmax_scale: float = 0.0, values_on_host: bool = False,
                value_cache_tokens: int = 0) -> sd_config:
    cfg = sd_config()
    cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim = batch, num_q_heads, num_kv_heads, head_dim
    cfg.max_context = max_context
    cfg.num_stages = len(stages)
    for i, s in enumerate(stages):
        c, r, k = (s.chunk, s.stride, s.keep) if hasattr(s, "chunk") else s
        cfg.stage[i] = sd_stage(c, r, k)
    cfg.sink, cfg.window = sink, window
    cfg.softmax_scale = softmax_scale
    cfg.values_on_host = 1 if values_on_host else 0
    cfg.value_cache_tokens = value_cache_tokens
    return cfg


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def decode_step_noalloc(cfg: sd_config, q, k, k_int8, v, lengths, out, kept_idx, stream=None) -> None:
    """sd_decode_step_noalloc: the step without a context, its workspace in
    the library's fixed per-GPU scratch array (no allocation)."""
    check(lib.sd_decode_step_noalloc(C.byref(cfg), _ptr(q), _ptr(k), _ptr(k_int8), _ptr(v), _ptr(lengths),
                                     _ptr(out), _ptr(kept_idx), _stream(stream)), "sd_decode_step_noalloc")


class SparseDecoder:
    """Owns one sd_ctx.  Methods mirror the C entry points one to one."""

    def __init__(self, cfg: sd_config):
        self.cfg = cfg
        h = _p()
        check(lib.sd_create(C.byref(cfg), C.byref(h)), "sd_create")
        self.handle = h

    @classmethod
    def for_workload(cls, w, **overrides) -> "SparseDecoder":
        kw = dict(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                  max_context=w.max_context, stages=w.stages, sink=w.sink, window=w.window,
                  head_dim=w.head_dim, values_on_host=w.values_on_host,
                  value_cache_tokens=w.value_cache_tokens)
        kw.update(overrides)
        return cls(make_config(**kw))

    @property
    def keep_total(self) -> int:
        return sum(self.cfg.stage[i].keep for i in range(self.cfg.num_stages))

    def close(self) -> None:
        if getattr(self, "handle", None):
            lib.sd_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # ---- entry points ----
    def sd_quantize_keys(self, k, lengths, k_int8, k_absmax=None, stream=None) -> None:
        check(lib.sd_quantize_keys(self.handle, _ptr(k), _ptr(lengths), _ptr(k_int8), _ptr(k_absmax),
                                   _stream(stream)), "sd_quantize_keys")

    def sd_decode_step(self, q, k, k_int8, v, lengths, out, kept_idx, stream=None) -> None:
        check(lib.sd_decode_step(self.handle, _ptr(q), _ptr(k), _ptr(k_int8), _ptr(v), _ptr(lengths),
                                 _ptr(out), _ptr(kept_idx), _stream(stream)), "sd_decode_step")

    def sd_decode_step_reuse(self, q, k, k_int8, v, lengths, out, kept_idx, reuse_stages: int,
                             stream=None) -> None:
        check(lib.sd_decode_step_reuse(self.handle, _ptr(q), _ptr(k), _ptr(k_int8), _ptr(v), _ptr(lengths),
                                       _ptr(out), _ptr(kept_idx), int(reuse_stages), _stream(stream)),
              "sd_decode_step_reuse")

    def sd_dense_decode(self, q, k, v, lengths, out, stream=None) -> None:
        check(lib.sd_dense_decode(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(lengths), _ptr(out),
                                  _stream(stream)), "sd_dense_decode")

    def sd_append_kv(self, k_new, v_new, n_new: int, lengths, k, k_int8, v, k_absmax=None, stream=None,
                     k_sketch4=None) -> None:
        check(lib.sd_append_kv(self.handle, _ptr(k_new), _ptr(v_new), int(n_new), _ptr(lengths), _ptr(k),
                               _ptr(k_int8), _ptr(v), _ptr(k_sketch4), _ptr(k_absmax), _stream(stream)),
              "sd_append_kv")

    def sd_sketch4_rows(self) -> int:
        return int(lib.sd_sketch4_rows(self.handle))

    def sd_quantize_sketch4(self, k, lengths, k_sketch4, stream=None) -> None:
        check(lib.sd_quantize_sketch4(self.handle, _ptr(k), _ptr(lengths), _ptr(k_sketch4), _stream(stream)),
              "sd_quantize_sketch4")

    def sd_decode_step_sketch4(self, q, k, k_int8, k_sketch4, v, lengths, out, kept_idx, stream=None) -> None:
        check(lib.sd_decode_step_sketch4(self.handle, _ptr(q), _ptr(k), _ptr(k_int8), _ptr(k_sketch4), _ptr(v),
                                         _ptr(lengths), _ptr(out), _ptr(kept_idx), _stream(stream)),
              "sd_decode_step_sketch4")

    def sd_quantize_query(self, q, q8=None, q_group=None, stream=None) -> None:
        check(lib.sd_quantize_query(self.handle, _ptr(q), _ptr(q8), _ptr(q_group), _stream(stream)),
              "sd_quantize_query")

    def sd_stage_candidates(self, stage: int) -> int:
        return int(lib.sd_stage_candidates(self.handle, stage))

    def sd_stage_scores(self, stage: int, dst, stream=None) -> None:
        check(lib.sd_stage_scores(self.handle, stage, _ptr(dst), dst.numel(), _stream(stream)),
              "sd_stage_scores")

    def sd_set_value_fetch(self, mode: int) -> None:
        check(lib.sd_set_value_fetch(self.handle, mode), "sd_set_value_fetch")

    def sd_record_attended(self, dst) -> None:
        """dst: a device uint32/int32 tensor of B * Hkv * max_blocks words, or None to stop."""
        if dst is None:
            check(lib.sd_record_attended(self.handle, None, 0), "sd_record_attended")
        else:
            check(lib.sd_record_attended(self.handle, _ptr(dst), dst.numel()), "sd_record_attended")

    def sd_check(self, stream=None) -> int:
        return int(lib.sd_check(self.handle, _stream(stream)))

    def sd_get_stats(self, stream=None) -> sd_stats:
        st = sd_stats()
        check(lib.sd_get_stats(self.handle, C.byref(st), _stream(stream)), "sd_get_stats")
        return st

    def sd_profile_start(self, kind_mask: int = (1 << SD_PROF_KINDS) - 1, max_launches: int = 4096) -> None:
        check(lib.sd_profile_start(self.handle, kind_mask, max_launches), "sd_profile_start")

    def sd_profile_stop(self) -> dict:
        pr = sd_profile()
        check(lib.sd_profile_stop(self.handle, C.byref(pr)), "sd_profile_stop")
        return {PROF_NAMES[i]: (float(pr.ms[i]), int(pr.launches[i])) for i in range(SD_PROF_KINDS)
                if pr.launches[i]}

    def sd_reset_value_cache(self, stream=None) -> None:
        check(lib.sd_reset_value_cache(self.handle, _stream(stream)), "sd_reset_value_cache")

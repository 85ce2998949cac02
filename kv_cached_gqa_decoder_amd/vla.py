"""ctypes binding of libvla.so: the C entry points of include/vla.h under the same names.

Argument marshalling only: every step of the path runs in the library's HIP
kernels. Device pointers are passed as integers or as objects with a
``data_ptr()`` method (torch tensors); streams as integers (a hipStream_t, e.g.
``torch.cuda.current_stream().cuda_stream``) or None for the null stream.
Failures raise ``VlaError`` carrying the status code and vla_last_error().
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_double, c_int32, c_int64, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvla.so")

VLA_OK, VLA_E_INVALID, VLA_E_NO_BLOCKS, VLA_E_NOTHING_TO_EVICT, VLA_E_HIP, VLA_E_STATE = \
    0, -1, -2, -3, -4, -5
VLA_E_TIMEOUT = -6
VLA_OPT_PERSISTENT_DECODE, VLA_OPT_BARRIER_SPIN_LIMIT, VLA_OPT_BARRIER_TEST_UNREACHABLE = 1, 2, 3
VLA_INFO_LAST_DECODE_PERSISTENT = 100
VLA_F32, VLA_BF16, VLA_INT4_G128 = 0, 1, 2
VLA_SWIGLU, VLA_GEGLU = 0, 1
VLA_TOKEN_DEVICE = -1   # decode input: the previous forward's greedy token, on the device
VLA_EVICT_SEMANTIC, VLA_EVICT_FIFO, VLA_EVICT_ADJACENT = 0, 1, 2
EVICT_POLICIES = {"semantic": VLA_EVICT_SEMANTIC, "fifo": VLA_EVICT_FIFO,
                  "adjacent": VLA_EVICT_ADJACENT}

# kernel classes for vla_profile_enable
K_CLASSES = {
    "gemv_qkv": 1, "gemv_o": 2, "gemv_gateup": 3, "gemv_down": 4, "gemv_head": 5,
    "attn_decode": 6, "gemm_qkv": 7, "gemm_o": 8, "gemm_gateup": 9, "gemm_down": 10,
    "attn_prefill": 11, "meankeys": 12, "score": 13, "rmsnorm": 14,
}


class VlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"vla status {status}: {msg}")
        self.status = status


class vla_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", c_int32), ("hidden", c_int32), ("n_heads", c_int32),
        ("n_kv_heads", c_int32), ("head_dim", c_int32), ("ffn", c_int32), ("vocab", c_int32),
        ("rms_eps", ctypes.c_float), ("rope_theta", c_double),
        ("wdtype", c_int32), ("act_dtype", c_int32), ("ffn_kind", c_int32),
        ("block_tokens", c_int32), ("num_blocks", c_int32), ("max_frames", c_int32),
        ("max_chunk", c_int32), ("seed", c_uint64), ("init_std", c_double),
        ("kv_only_last", c_int32), ("stream_base", ctypes.c_uint32),
    ]


class vla_state(ctypes.Structure):
    _fields_ = [("next_position", c_int64), ("next_frame_id", c_int32), ("n_frames", c_int32),
                ("resident_tokens", c_int32), ("free_blocks", c_int32),
                ("logical_blocks", c_int32)]


class vla_admission_config(ctypes.Structure):
    _fields_ = [("deadline_ms", c_double), ("safety_margin_ms", c_double), ("ema_alpha", c_double),
                ("prefill_tokens", c_int32), ("decode_tokens", c_int32)]


class vla_admission_stats(ctypes.Structure):
    _fields_ = [("cycles", c_int64), ("admitted", c_int64), ("refused", c_int64),
                ("deadline_misses", c_int64), ("worst_cycle_ms", c_double),
                ("last_overrun_ms", c_double), ("ema_prefill_ms_per_token", c_double),
                ("ema_decode_ms_per_token", c_double), ("has_sample", c_int32)]


_SIGS = {
    "vla_model_create": (c_int32, [POINTER(vla_config), POINTER(c_void_p)]),
    "vla_model_destroy": (None, [c_void_p]),
    "vla_model_create_sibling": (c_int32, [c_void_p, POINTER(c_void_p)]),
    "vla_prefill_chunk": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, POINTER(c_int32),
                                    c_void_p]),
    "vla_decode_step": (c_int32, [c_void_p, c_int32, POINTER(c_int32), c_void_p]),
    "vla_kv_score_and_evict": (c_int32, [c_void_p, c_int32, POINTER(c_int32), POINTER(c_double),
                                         c_void_p]),
    "vla_kv_score": (c_int32, [c_void_p, c_int32, POINTER(c_int32), POINTER(c_double), c_void_p]),
    "vla_kv_evict": (c_int32, [c_void_p, c_int32, c_int32, POINTER(c_int32), POINTER(c_double),
                               c_void_p]),
    "vla_kv_make_room": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, POINTER(c_int32),
                                   c_void_p]),
    "vla_logits_out": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p]),
    "vla_kv_score_noalloc": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "vla_last_error": (ctypes.c_char_p, []),
    "vla_kv_append_raw": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, POINTER(c_int32),
                                    c_void_p]),
    "vla_kv_rollback": (c_int32, [c_void_p, c_int32]),
    "vla_kv_refresh_mean_keys": (c_int32, [c_void_p, c_void_p]),
    "vla_get_state": (c_int32, [c_void_p, POINTER(vla_state)]),
    "vla_kv_block_table": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, POINTER(c_int32)]),
    "vla_kv_frames": (c_int32, [c_void_p, c_void_p, c_int32, POINTER(c_int32)]),
    "vla_kv_free_list": (c_int32, [c_void_p, c_void_p, c_int32, POINTER(c_int32)]),
    "vla_pool_free_list": (c_int32, [c_void_p, c_void_p, c_int32, POINTER(c_int32)]),
    "vla_mean_keys_out": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, POINTER(c_int32),
                                    c_void_p]),
    "vla_kv_gather": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                                POINTER(c_int32), c_void_p]),
    "vla_weight_out": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_int64, c_void_p]),
    "vla_set_option": (c_int32, [c_void_p, c_int32, c_int64]),
    "vla_probe_barrier": (c_int32, [c_int32, c_int32, c_void_p, POINTER(c_double)]),
    "vla_probe_read_bandwidth": (c_int32, [c_int64, c_int32, c_void_p, POINTER(c_double)]),
    "vla_get_option": (c_int32, [c_void_p, c_int32, POINTER(c_int64)]),
    "vla_profile_enable": (c_int32, [c_void_p, c_int32]),
    "vla_profile_read": (c_int32, [c_void_p, POINTER(c_double), POINTER(c_int32)]),
    "vla_profile_replay": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, POINTER(c_double)]),
    "vla_probe_mfma_peak": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, POINTER(c_double)]),
    "vla_expert_create": (c_int32, [c_void_p, POINTER(vla_config), c_int32, POINTER(c_void_p)]),
    "vla_expert_destroy": (None, [c_void_p]),
    "vla_expert_create_sibling": (c_int32, [c_void_p, c_void_p, POINTER(c_void_p)]),
    "vla_pipeline_create": (c_int32, [c_void_p, c_void_p, POINTER(c_void_p)]),
    "vla_pipeline_destroy": (None, [c_void_p]),
    "vla_pipeline_prefill": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, POINTER(c_int64)]),
    "vla_pipeline_act": (c_int32, [c_void_p, c_void_p, c_int32, c_double, c_void_p,
                                   POINTER(c_int64)]),
    "vla_pipeline_sync": (c_int32, [c_void_p]),
    "vla_pipeline_stats": (c_int32, [c_void_p, POINTER(c_int64), POINTER(c_int64),
                                     POINTER(c_int64)]),
    "vla_asr_create": (c_int32, [c_void_p, POINTER(c_void_p)]),
    "vla_asr_destroy": (None, [c_void_p]),
    "vla_asr_model": (c_void_p, [c_void_p]),
    "vla_asr_prefill": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                  POINTER(c_int64)]),
    "vla_asr_evict": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, POINTER(c_int64),
                                POINTER(c_double)]),
    "vla_asr_reconcile_begin": (c_int32, [c_void_p, c_void_p]),
    "vla_asr_try_swap": (c_int32, [c_void_p, c_void_p, POINTER(c_int32)]),
    "vla_asr_sync": (c_int32, [c_void_p]),
    "vla_asr_frames": (c_int32, [c_void_p, c_void_p, c_int32, POINTER(c_int32)]),
    "vla_asr_stats": (c_int32, [c_void_p, POINTER(c_int64), POINTER(c_int64), POINTER(c_int64),
                                POINTER(c_int32)]),
    "vla_expert_denoise": (c_int32, [c_void_p, c_void_p, c_int32, c_double, c_void_p]),
    "vla_pool_create": (c_int32, [c_int32, POINTER(c_void_p)]),
    "vla_pool_destroy": (None, [c_void_p]),
    "vla_pool_alloc": (c_int32, [c_void_p, c_int32, c_void_p]),
    "vla_pool_release": (c_int32, [c_void_p, c_void_p, c_int32]),
    "vla_pool_free_count": (c_int32, [c_void_p]),
    "vla_admission_create": (c_int32, [POINTER(vla_admission_config), POINTER(c_void_p)]),
    "vla_admission_destroy": (None, [c_void_p]),
    "vla_admission_cycle_begin": (c_int32, [c_void_p]),
    "vla_admission_elapsed_ms": (c_int32, [c_void_p, POINTER(c_double)]),
    "vla_admission_should_admit": (c_int32, [c_void_p, c_double, POINTER(c_int32),
                                             POINTER(c_double)]),
    "vla_admission_record": (c_int32, [c_void_p, c_double, c_int32, c_double, c_int32]),
    "vla_admission_cycle_end": (c_int32, [c_void_p, c_int32, POINTER(c_double)]),
    "vla_admission_sleep_until_deadline": (c_int32, [c_void_p]),
    "vla_admission_stats_out": (c_int32, [c_void_p, POINTER(vla_admission_stats)]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libvla.so (raises if it has not been built: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python kv_cached_gqa_decoder_amd/build.py` (hipcc, gfx950)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(st: int):
    if st != VLA_OK:
        raise VlaError(st, load().vla_last_error().decode())


# ---- the C entry points ----------------------------------------------------
def vla_model_create(cfg: vla_config) -> int:
    h = c_void_p()
    _check(load().vla_model_create(byref(cfg), byref(h)))
    return h.value


def vla_model_destroy(m: int) -> None:
    load().vla_model_destroy(m)


def vla_prefill_chunk(m: int, tokens=None, embeds=None, n: int = 0, stream=None) -> int:
    """tokens: host int32 buffer (numpy array or ctypes array) or None; embeds: device pointer."""
    fid = c_int32(-1)
    tok_ptr = None
    if tokens is not None:
        import numpy as np
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        tok_ptr = tokens.ctypes.data
        n = n or tokens.size
    _check(load().vla_prefill_chunk(m, tok_ptr, _ptr(embeds), n, byref(fid), _stream(stream)))
    return fid.value


def vla_decode_step(m: int, token: int, stream=None, want_token: bool = True):
    nxt = c_int32(-1)
    _check(load().vla_decode_step(m, int(token), byref(nxt) if want_token else None,
                                  _stream(stream)))
    return nxt.value if want_token else None


def vla_kv_score_and_evict(m: int, layer: int = 0, stream=None):
    fid, sc = c_int32(-1), c_double(0.0)
    _check(load().vla_kv_score_and_evict(m, layer, byref(fid), byref(sc), _stream(stream)))
    return fid.value, sc.value


def vla_kv_score(m: int, layer: int = 0, stream=None):
    fid, sc = c_int32(-1), c_double(0.0)
    _check(load().vla_kv_score(m, layer, byref(fid), byref(sc), _stream(stream)))
    return fid.value, sc.value


def vla_kv_evict(m: int, policy: int, layer: int = 0, stream=None):
    fid, sc = c_int32(-1), c_double(0.0)
    _check(load().vla_kv_evict(m, policy, layer, byref(fid), byref(sc), _stream(stream)))
    return fid.value, sc.value


def vla_kv_make_room(m: int, policy: int, layer: int, n_tokens: int, window: int = 0,
                     stream=None) -> int:
    n = c_int32(0)
    _check(load().vla_kv_make_room(m, policy, layer, n_tokens, window, byref(n), _stream(stream)))
    return n.value


def vla_kv_score_noalloc(mean_keys, n_frames: int, dim: int, out_index, out_score,
                         stream=None) -> None:
    """Device pointers: mean_keys fp64 [n_frames][dim], out_index int32[1], out_score fp64[1]."""
    _check(load().vla_kv_score_noalloc(_ptr(mean_keys), n_frames, dim, _ptr(out_index),
                                       _ptr(out_score), _stream(stream)))


def vla_logits_out(m: int, out, n: int, stream=None) -> None:
    _check(load().vla_logits_out(m, _ptr(out) if not hasattr(out, "ctypes") else out.ctypes.data,
                                 n, _stream(stream)))


def vla_last_error() -> str:
    return load().vla_last_error().decode()


def vla_kv_append_raw(m: int, k, v, n: int, stream=None) -> int:
    fid = c_int32(-1)
    _check(load().vla_kv_append_raw(m, _ptr(k), _ptr(v), n, byref(fid), _stream(stream)))
    return fid.value


def vla_kv_rollback(m: int, keep_frame_id: int) -> None:
    _check(load().vla_kv_rollback(m, keep_frame_id))


def vla_kv_refresh_mean_keys(m: int, stream=None) -> None:
    _check(load().vla_kv_refresh_mean_keys(m, _stream(stream)))


def vla_get_state(m: int) -> dict:
    s = vla_state()
    _check(load().vla_get_state(m, byref(s)))
    return {k: getattr(s, k) for k, _ in vla_state._fields_}


def vla_kv_block_table(m: int):
    import numpy as np
    n = c_int32(0)
    _check(load().vla_kv_block_table(m, None, None, 0, byref(n)))
    blocks = np.zeros(max(n.value, 1), dtype=np.int32)
    ntok = np.zeros(max(n.value, 1), dtype=np.int32)
    _check(load().vla_kv_block_table(m, blocks.ctypes.data, ntok.ctypes.data, n.value, byref(n)))
    return blocks[: n.value], ntok[: n.value]


def vla_kv_frames(m: int):
    import numpy as np
    n = c_int32(0)
    _check(load().vla_kv_frames(m, None, 0, byref(n)))
    ids = np.zeros(max(n.value, 1), dtype=np.int32)
    _check(load().vla_kv_frames(m, ids.ctypes.data, n.value, byref(n)))
    return ids[: n.value]


def _free_list(fn, h):
    import numpy as np
    n = c_int32(0)
    _check(fn(h, None, 0, byref(n)))
    out = np.zeros(max(n.value, 1), dtype=np.int32)
    _check(fn(h, out.ctypes.data, n.value, byref(n)))
    return [int(b) for b in out[: n.value]]


def vla_kv_free_list(m: int):
    """The free-list bottom first (the last entry is popped next)."""
    return _free_list(load().vla_kv_free_list, m)


def vla_pool_free_list(p: int):
    return _free_list(load().vla_pool_free_list, p)


def vla_mean_keys_out(m: int, layer: int, cap_frames: int, dim: int, stream=None):
    import numpy as np
    out = np.zeros((max(cap_frames, 1), dim), dtype=np.float64)
    n = c_int32(0)
    _check(load().vla_mean_keys_out(m, layer, out.ctypes.data, cap_frames, byref(n),
                                    _stream(stream)))
    return out[: min(n.value, cap_frames)]


def vla_kv_gather(m: int, layer: int, k_out, v_out, cap_tokens: int, stream=None) -> int:
    n = c_int32(0)
    _check(load().vla_kv_gather(m, layer, _ptr(k_out), _ptr(v_out), cap_tokens, byref(n),
                                _stream(stream)))
    return n.value


def vla_weight_out(m: int, kind: int, layer: int, out, nbytes: int, stream=None) -> None:
    _check(load().vla_weight_out(m, kind, layer, _ptr(out), nbytes, _stream(stream)))


def vla_set_option(m: int, key: int, value: int) -> None:
    _check(load().vla_set_option(m, key, int(value)))


def vla_probe_barrier(grid: int, nbar: int, stream=None) -> float:
    """Microseconds per device-scope barrier over `grid` resident workgroups."""
    us = c_double(0.0)
    _check(load().vla_probe_barrier(grid, nbar, _stream(stream), byref(us)))
    return us.value


def vla_probe_read_bandwidth(nbytes: int, reps: int = 5, stream=None) -> float:
    """GB/s of a streaming read of an nbytes device buffer."""
    g = c_double(0.0)
    _check(load().vla_probe_read_bandwidth(int(nbytes), reps, _stream(stream), byref(g)))
    return g.value


def vla_get_option(m: int, key: int) -> int:
    v = c_int64(0)
    _check(load().vla_get_option(m, key, byref(v)))
    return v.value


def vla_profile_enable(m: int, kernel_class: int) -> None:
    _check(load().vla_profile_enable(m, kernel_class))


def vla_profile_read(m: int):
    ms, n = c_double(0.0), c_int32(0)
    _check(load().vla_profile_read(m, byref(ms), byref(n)))
    return ms.value, n.value


def vla_profile_replay(m: int, kernel_class: int, reps: int, stream=None) -> float:
    ms = c_double(0.0)
    _check(load().vla_profile_replay(m, kernel_class, reps, _stream(stream), byref(ms)))
    return ms.value


def vla_probe_mfma_peak(out, blocks: int, iters: int, stream=None) -> float:
    """Achieved bf16 MFMA TFLOP/s of a register-only MFMA loop (out: device float[blocks])."""
    t = c_double(0.0)
    _check(load().vla_probe_mfma_peak(_ptr(out), blocks, iters, _stream(stream), byref(t)))
    return t.value


def vla_expert_create(prefix: int, cfg: vla_config, n_actions: int) -> int:
    h = c_void_p()
    _check(load().vla_expert_create(prefix, byref(cfg), n_actions, byref(h)))
    return h.value


def vla_expert_destroy(e: int) -> None:
    load().vla_expert_destroy(e)


def vla_model_create_sibling(src: int) -> int:
    h = c_void_p()
    _check(load().vla_model_create_sibling(src, byref(h)))
    return h.value


def vla_expert_create_sibling(prefix: int, src: int) -> int:
    h = c_void_p()
    _check(load().vla_expert_create_sibling(prefix, src, byref(h)))
    return h.value


def vla_pipeline_create(prefix: int, expert: int) -> int:
    h = c_void_p()
    _check(load().vla_pipeline_create(prefix, expert, byref(h)))
    return h.value


def vla_pipeline_destroy(p: int) -> None:
    load().vla_pipeline_destroy(p)


def vla_pipeline_prefill(p: int, embeds, n: int, stream=None) -> int:
    f = c_int64(-1)
    _check(load().vla_pipeline_prefill(p, _ptr(embeds), n, _stream(stream), byref(f)))
    return f.value


def vla_pipeline_act(p: int, x, n_steps: int, dt: float, stream=None) -> int:
    f = c_int64(-1)
    _check(load().vla_pipeline_act(p, _ptr(x), n_steps, dt, _stream(stream), byref(f)))
    return f.value


def vla_pipeline_sync(p: int) -> None:
    _check(load().vla_pipeline_sync(p))


def vla_asr_create(primary: int) -> int:
    h = c_void_p()
    _check(load().vla_asr_create(primary, byref(h)))
    return h.value


def vla_asr_destroy(a: int) -> None:
    load().vla_asr_destroy(a)


def vla_asr_model(a: int) -> int:
    return load().vla_asr_model(a)


def vla_asr_prefill(a: int, tokens=None, embeds=None, n: int = 0, stream=None) -> int:
    f = c_int64(-1)
    if tokens is not None:
        import numpy as np
        arr = np.ascontiguousarray(tokens, dtype=np.int32)
        n = len(arr)
        _check(load().vla_asr_prefill(a, arr.ctypes.data, None, n, _stream(stream), byref(f)))
    else:
        _check(load().vla_asr_prefill(a, None, _ptr(embeds), n, _stream(stream), byref(f)))
    return f.value


def vla_asr_evict(a: int, policy: int, layer: int = 0, stream=None):
    f, sc = c_int64(-1), c_double(0.0)
    _check(load().vla_asr_evict(a, policy, layer, _stream(stream), byref(f), byref(sc)))
    return f.value, sc.value


def vla_asr_reconcile_begin(a: int, stream=None) -> None:
    _check(load().vla_asr_reconcile_begin(a, _stream(stream)))


def vla_asr_try_swap(a: int, stream=None) -> bool:
    s = c_int32(0)
    _check(load().vla_asr_try_swap(a, _stream(stream), byref(s)))
    return bool(s.value)


def vla_asr_sync(a: int) -> None:
    _check(load().vla_asr_sync(a))


def vla_asr_frames(a: int):
    import numpy as np
    n = c_int32(0)
    _check(load().vla_asr_frames(a, None, 0, byref(n)))
    ids = np.zeros(max(n.value, 1), dtype=np.int64)
    _check(load().vla_asr_frames(a, ids.ctypes.data, n.value, byref(n)))
    return [int(i) for i in ids[:n.value]]


def vla_asr_stats(a: int) -> dict:
    r, s, f, on = c_int64(0), c_int64(0), c_int64(0), c_int32(0)
    _check(load().vla_asr_stats(a, byref(r), byref(s), byref(f), byref(on)))
    return {"reconciliations": r.value, "swaps": s.value, "frames_replayed": f.value,
            "reconciling": bool(on.value)}


def vla_pipeline_stats(p: int) -> dict:
    a, b, c = c_int64(0), c_int64(0), c_int64(0)
    _check(load().vla_pipeline_stats(p, byref(a), byref(b), byref(c)))
    return {"prefills": a.value, "acts": b.value, "acts_on_older": c.value}


def vla_expert_denoise(e: int, x, n_steps: int, dt: float, stream=None) -> None:
    _check(load().vla_expert_denoise(e, _ptr(x), n_steps, dt, _stream(stream)))


def vla_pool_create(num_blocks: int) -> int:
    h = c_void_p()
    _check(load().vla_pool_create(num_blocks, byref(h)))
    return h.value


def vla_pool_destroy(p: int) -> None:
    load().vla_pool_destroy(p)


def vla_pool_alloc(p: int, n: int):
    import numpy as np
    out = np.zeros(max(n, 1), dtype=np.int32)
    _check(load().vla_pool_alloc(p, n, out.ctypes.data))
    return [int(v) for v in out[:n]]


def vla_pool_release(p: int, blocks) -> None:
    import numpy as np
    b = np.ascontiguousarray(blocks, dtype=np.int32)
    _check(load().vla_pool_release(p, b.ctypes.data, b.size))


def vla_pool_free_count(p: int) -> int:
    return load().vla_pool_free_count(p)


def vla_admission_create(deadline_ms=33.0, safety_margin_ms=2.0, ema_alpha=0.2,
                         prefill_tokens=32, decode_tokens=8) -> int:
    cfg = vla_admission_config(deadline_ms, safety_margin_ms, ema_alpha, prefill_tokens,
                               decode_tokens)
    h = c_void_p()
    _check(load().vla_admission_create(byref(cfg), byref(h)))
    return h.value


def vla_admission_destroy(a: int) -> None:
    load().vla_admission_destroy(a)


def vla_admission_cycle_begin(a: int) -> None:
    _check(load().vla_admission_cycle_begin(a))


def vla_admission_elapsed_ms(a: int) -> float:
    v = c_double(0.0)
    _check(load().vla_admission_elapsed_ms(a, byref(v)))
    return v.value


def vla_admission_should_admit(a: int, elapsed_ms: float):
    """(admit?, estimate in ms)."""
    ok, est = c_int32(0), c_double(0.0)
    _check(load().vla_admission_should_admit(a, elapsed_ms, byref(ok), byref(est)))
    return bool(ok.value), est.value


def vla_admission_record(a: int, prefill_ms: float, prefill_tokens: int, decode_ms: float,
                         decode_tokens: int) -> None:
    _check(load().vla_admission_record(a, prefill_ms, prefill_tokens, decode_ms, decode_tokens))


def vla_admission_cycle_end(a: int, admitted: bool) -> float:
    ms = c_double(0.0)
    _check(load().vla_admission_cycle_end(a, 1 if admitted else 0, byref(ms)))
    return ms.value


def vla_admission_sleep_until_deadline(a: int) -> None:
    _check(load().vla_admission_sleep_until_deadline(a))


def vla_admission_stats_out(a: int) -> dict:
    st = vla_admission_stats()
    _check(load().vla_admission_stats_out(a, byref(st)))
    return {k: getattr(st, k) for k, _ in vla_admission_stats._fields_}


# ---- configurations of the workloads --------------------------------------
PRESETS = {
    # tiny GQA decoder, fp32: 64-token prompt then 16 greedy decodes
    "c1_tiny_f32": dict(n_layers=2, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn=688,
                        vocab=1024, rope_theta=1e4, wdtype=VLA_F32, num_blocks=8,
                        max_frames=8, max_chunk=64, seed=1235),
    # Qwen2.5-1.5B-shaped GQA decoder, bf16: 1024 cached + 256-token chunk + 16 decodes
    "c2_qwen1p5b_bf16": dict(n_layers=28, hidden=1536, n_heads=12, n_kv_heads=2, head_dim=128,
                             ffn=8960, vocab=151936, rope_theta=1e6, wdtype=VLA_BF16,
                             num_blocks=96, max_frames=16, max_chunk=256, seed=1236),
    # same shape, 128 frames of 64 tokens at a 512-block budget, 32 eviction cycles
    "c3_semantic_eviction": dict(n_layers=28, hidden=1536, n_heads=12, n_kv_heads=2,
                                 head_dim=128, ffn=8960, vocab=151936, rope_theta=1e6,
                                 wdtype=VLA_BF16, num_blocks=512, max_frames=128, max_chunk=64,
                                 seed=1237),
    # Llama-3-8B-shaped decoder, INT4 group-128 weights, bf16 activations: a 120,000-token
    # cached prefix (raw frames of up to 512 tokens), a 512-token chunk, 32 decodes
    "c5_llama3_8b_int4": dict(n_layers=32, hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128,
                              ffn=14336, vocab=128256, rope_theta=5e5, wdtype=VLA_INT4_G128,
                              act_dtype=VLA_BF16, num_blocks=7534, max_frames=256,
                              max_chunk=512, seed=1239),
    # pi0-style policy: Gemma-2B-shaped prefix (17 GeGLU layers + a K/V-only 18th, MQA,
    # head dim 256) over 2 x 256 image tokens, and the 300M action expert (18 layers,
    # hidden 1024) denoising a 63-token action chunk in 10 Euler steps
    "c4_pi0_vlm": dict(n_layers=18, hidden=2048, n_heads=8, n_kv_heads=1, head_dim=256,
                       ffn=16384, vocab=0, rope_theta=1e4, wdtype=VLA_BF16, ffn_kind=VLA_GEGLU,
                       kv_only_last=1, num_blocks=40, max_frames=4, max_chunk=512, seed=1238),
    "c4_pi0_action_expert": dict(n_layers=18, hidden=1024, n_heads=8, n_kv_heads=1,
                                 head_dim=256, ffn=4096, vocab=0, rope_theta=1e4,
                                 wdtype=VLA_BF16, ffn_kind=VLA_GEGLU, stream_base=0x8000,
                                 num_blocks=0, max_frames=0, max_chunk=63, seed=1238),
}


def make_config(**kw) -> vla_config:
    c = vla_config()
    c.n_layers = kw["n_layers"]
    c.hidden = kw["hidden"]
    c.n_heads = kw["n_heads"]
    c.n_kv_heads = kw["n_kv_heads"]
    c.head_dim = kw["head_dim"]
    c.ffn = kw["ffn"]
    c.vocab = kw["vocab"]
    c.rms_eps = kw.get("rms_eps", 1e-6)
    c.rope_theta = kw.get("rope_theta", 1e4)
    c.wdtype = kw.get("wdtype", VLA_BF16)
    c.act_dtype = kw.get("act_dtype", VLA_BF16 if c.wdtype == VLA_INT4_G128 else c.wdtype)
    c.ffn_kind = kw.get("ffn_kind", VLA_SWIGLU)
    c.block_tokens = kw.get("block_tokens", 16)
    c.num_blocks = kw["num_blocks"]
    c.max_frames = kw["max_frames"]
    c.max_chunk = kw["max_chunk"]
    c.seed = kw["seed"]
    c.init_std = kw.get("init_std", 0.02)
    c.kv_only_last = int(kw.get("kv_only_last", 0))
    c.stream_base = int(kw.get("stream_base", 0))
    return c


def preset(name: str, **overrides) -> vla_config:
    kw = dict(PRESETS[name])
    kw.update(overrides)
    return make_config(**kw)


class Model:
    """Owns one handle; methods forward to the C entry points of the same names."""

    def __init__(self, cfg: vla_config, _handle=None):
        self.cfg = cfg
        self.h = _handle if _handle is not None else vla_model_create(cfg)

    def sibling(self):
        """A second model over the same (shared) weights: vla_model_create_sibling."""
        return Model(self.cfg, _handle=vla_model_create_sibling(self.h))

    def close(self):
        if self.h:
            vla_model_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def prefill_chunk(self, tokens=None, embeds=None, n=0, stream=None):
        return vla_prefill_chunk(self.h, tokens, embeds, n, stream)

    def decode_step(self, token, stream=None, want_token=True):
        return vla_decode_step(self.h, token, stream, want_token)

    def kv_score_and_evict(self, layer=0, stream=None):
        return vla_kv_score_and_evict(self.h, layer, stream)

    def kv_score(self, layer=0, stream=None):
        return vla_kv_score(self.h, layer, stream)

    def kv_evict(self, policy, layer=0, stream=None):
        return vla_kv_evict(self.h, EVICT_POLICIES.get(policy, policy), layer, stream)

    def kv_make_room(self, policy, n_tokens, window=0, layer=0, stream=None):
        return vla_kv_make_room(self.h, EVICT_POLICIES.get(policy, policy), layer, n_tokens,
                                window, stream)

    def logits_out(self, out, stream=None):
        vla_logits_out(self.h, out, self.cfg.vocab, stream)

    def kv_append_raw(self, k, v, n, stream=None):
        return vla_kv_append_raw(self.h, k, v, n, stream)

    def kv_rollback(self, keep_frame_id):
        vla_kv_rollback(self.h, keep_frame_id)

    def kv_refresh_mean_keys(self, stream=None):
        vla_kv_refresh_mean_keys(self.h, stream)

    def state(self):
        return vla_get_state(self.h)

    def block_table(self):
        return vla_kv_block_table(self.h)

    def frames(self):
        return vla_kv_frames(self.h)

    def free_list(self):
        return vla_kv_free_list(self.h)

    def mean_keys(self, layer, stream=None):
        return vla_mean_keys_out(self.h, layer, self.cfg.max_frames,
                                 self.cfg.n_kv_heads * self.cfg.head_dim, stream)

    def kv_gather(self, layer, k_out, v_out, cap_tokens, stream=None):
        return vla_kv_gather(self.h, layer, k_out, v_out, cap_tokens, stream)

    def weight_out(self, kind, layer, out, nbytes, stream=None):
        vla_weight_out(self.h, kind, layer, out, nbytes, stream)

    def set_option(self, key, value):
        vla_set_option(self.h, key, value)

    def get_option(self, key):
        return vla_get_option(self.h, key)

    def profile_enable(self, kernel_class):
        vla_profile_enable(self.h, K_CLASSES.get(kernel_class, kernel_class)
                           if isinstance(kernel_class, str) else kernel_class)

    def profile_read(self):
        return vla_profile_read(self.h)

    def profile_replay(self, kernel_class, reps=4, stream=None):
        """Mean ms per launch of `kernel_class` replayed over all layers, back to back."""
        return vla_profile_replay(self.h, K_CLASSES.get(kernel_class, kernel_class)
                                  if isinstance(kernel_class, str) else kernel_class, reps, stream)


class Expert:
    """An action expert bound to a prefix Model; forwards to the vla_expert_* entry points."""

    def __init__(self, prefix: Model, cfg: vla_config, n_actions: int, _handle=None):
        self.prefix = prefix
        self.cfg = cfg
        self.n_actions = n_actions
        self.h = _handle if _handle is not None else vla_expert_create(prefix.h, cfg, n_actions)

    def sibling(self, prefix: Model):
        """An expert with these (shared) weights bound to `prefix`: vla_expert_create_sibling."""
        return Expert(prefix, self.cfg, self.n_actions,
                      _handle=vla_expert_create_sibling(prefix.h, self.h))

    def close(self):
        if self.h:
            vla_expert_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def denoise(self, x, n_steps=10, dt=None, stream=None):
        vla_expert_denoise(self.h, x, n_steps, 1.0 / n_steps if dt is None else dt, stream)


class Pipeline:
    """Overlapped prefix and expert streams over a (Model, Expert) pair: vla_pipeline_*."""

    def __init__(self, prefix: Model, expert: Expert):
        self.prefix = prefix
        self.expert = expert
        self.h = vla_pipeline_create(prefix.h, expert.h)

    def close(self):
        if self.h:
            vla_pipeline_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def prefill(self, embeds, n, stream=None):
        return vla_pipeline_prefill(self.h, embeds, n, stream)

    def act(self, x, n_steps=10, dt=None, stream=None):
        return vla_pipeline_act(self.h, x, n_steps, 1.0 / n_steps if dt is None else dt, stream)

    def sync(self):
        vla_pipeline_sync(self.h)

    def stats(self):
        return vla_pipeline_stats(self.h)


class Reconciler:
    """Reconciliation on a sibling state (vla_asr_*); the serving model changes on a swap."""

    def __init__(self, primary: Model):
        self.primary = primary
        self.h = vla_asr_create(primary.h)

    def close(self):
        if self.h:
            vla_asr_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def model_handle(self) -> int:
        return vla_asr_model(self.h)

    def prefill(self, tokens=None, embeds=None, n=0, stream=None):
        return vla_asr_prefill(self.h, tokens, embeds, n, stream)

    def evict(self, policy, layer=0, stream=None):
        if isinstance(policy, str):
            policy = EVICT_POLICIES[policy]
        return vla_asr_evict(self.h, policy, layer, stream)

    def begin(self, stream=None):
        vla_asr_reconcile_begin(self.h, stream)

    def try_swap(self, stream=None):
        return vla_asr_try_swap(self.h, stream)

    def sync(self):
        vla_asr_sync(self.h)

    def frames(self):
        return vla_asr_frames(self.h)

    def stats(self):
        return vla_asr_stats(self.h)

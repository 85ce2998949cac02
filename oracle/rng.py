"""Seeded weight generator of the oracle: splitmix64 feeding Box-Muller.

"Can an LLM Forget the Right Things?", §6: the untrained weights come from a
deterministic PRNG, splitmix64 feeding a Box-Muller transform, seeded so that
every run sees identical weights. The page gives no stream layout, so this
module fixes a counter-based one (each element is a pure function of
(seed, stream, index)), which lets any physical layout be generated in place:

    sm(x)        splitmix64 finaliser of x + golden-gamma (mod 2^64)
    key          sm(seed XOR sm(stream))
    u53(x)       (x >> 11) * 2^-53                      in [0, 1)
    N(i)         sqrt(-2 ln(1 - u53(sm(key + 2i)))) * cos(2 pi u53(sm(key + 2i + 1)))
    id(i)        floor(u53(sm(key + i)) * V)            uniform token ids

splitmix64 is the published generator of Steele, Lea and Flood (OOPSLA 2014,
"Fast splittable pseudorandom number generators"); Box-Muller is the classic
transform (Box and Muller, 1958). A tensor value is ``std * N(i)`` with ``i``
its row-major index in the logical (out, in) layout, rounded to nearest-even
into the storage type.

Streams: per-layer tensor ((layer + 1) << 8) | kind with kinds Wq 1, Wk 2,
Wv 3, Wo 4, Wgate 5, Wup 6, Wdown 7; the embedding E is stream 1, the output
head W_Y stream 2.

This is the oracle's own implementation; the GPU library has its own.
``_oracle_rng.so`` (plain C, built from ``oracle/csrc/oracle_rng.c``) computes
the same definition faster, and a CPU test checks it bit for bit against the
numpy code below.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

KIND_Q, KIND_K, KIND_V, KIND_O, KIND_GATE, KIND_UP, KIND_DOWN = 1, 2, 3, 4, 5, 6, 7
STREAM_EMBED = 1
STREAM_HEAD = 2


def layer_stream(layer: int, kind: int) -> int:
    """Stream id of a per-layer tensor."""
    return ((layer + 1) << 8) | kind


def splitmix64(x):
    """splitmix64 output function applied to state ``x`` (uint64, wraps mod 2^64)."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x = x + _GAMMA
        z = (x ^ (x >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> np.uint64:
    return np.uint64(splitmix64(np.uint64(seed) ^ splitmix64(np.uint64(stream))))


def u53(x):
    """Top 53 bits of a uint64 as a double in [0, 1)."""
    return (np.asarray(x, dtype=np.uint64) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal_np(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    """N(0,1) values for element indices start .. start+n-1 (fp64, numpy)."""
    key = stream_key(seed, stream)
    i = np.arange(start, start + n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        a = splitmix64(key + np.uint64(2) * i)
        b = splitmix64(key + np.uint64(2) * i + np.uint64(1))
    u1 = u53(a)
    u2 = u53(b)
    return np.sqrt(-2.0 * np.log(1.0 - u1)) * np.cos(2.0 * np.pi * u2)


def uniform_ids(seed: int, stream: int, n: int, vocab: int) -> np.ndarray:
    """Uniform token ids in [0, vocab) (int64)."""
    key = stream_key(seed, stream)
    i = np.arange(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x = splitmix64(key + i)
    return np.floor(u53(x) * vocab).astype(np.int64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bfloat16 (8 significant bits), nearest-even, kept as fp64.

    Normal range only (the generated values never reach bf16 overflow or its
    subnormals).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def round_storage(x: np.ndarray, storage: str) -> np.ndarray:
    """Round fp64 values into the storage type ('f32', 'bf16' or 'f64'), returned as fp64."""
    if storage == "f64":
        return np.asarray(x, dtype=np.float64)
    if storage == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if storage == "bf16":
        return round_bf16(x)
    raise ValueError(storage)


# --------------------------------------------------------------------------
# plain-C twin of normal_np + round_storage (same definition, OpenMP threads)
# --------------------------------------------------------------------------
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_oracle_rng.so")
_lib = None
_STORAGE_CODE = {"f64": 0, "f32": 1, "bf16": 2}


def _load_c():
    global _lib
    if _lib is None and os.path.exists(_LIB_PATH):
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_normal.argtypes = [
            ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
            ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_normal.restype = None
        _lib = lib
    return _lib


def have_c() -> bool:
    return _load_c() is not None


def normal_c(seed: int, stream: int, start: int, n: int, std: float, storage: str,
             out_f32: bool = False) -> np.ndarray:
    """std * N(i) rounded into ``storage``; returns fp64 (or fp32 when out_f32 and storage != f64)."""
    lib = _load_c()
    if lib is None:
        raise RuntimeError("oracle/_oracle_rng.so is not built (run __graft_entry__.build())")
    if out_f32 and storage == "f64":
        raise ValueError("f64 storage cannot be returned as f32")
    out = np.empty(n, dtype=np.float32 if out_f32 else np.float64)
    lib.oracle_normal(seed, stream, start, n, std, _STORAGE_CODE[storage],
                      out.ctypes.data, 1 if out_f32 else 0)
    return out


def tensor(seed: int, stream: int, shape, std: float, storage: str,
           out_f32: bool = False) -> np.ndarray:
    """A seeded weight tensor in logical row-major layout.

    Values are std * N(i) rounded into ``storage``. Uses the C twin when it is
    built, else numpy (identical definition, slower).
    """
    n = int(np.prod(shape))
    if have_c():
        return normal_c(seed, stream, 0, n, std, storage, out_f32).reshape(shape)
    v = round_storage(std * normal_np(seed, stream, 0, n), storage)
    return (v.astype(np.float32) if out_f32 else v).reshape(shape)

"""Seeded synthetic inputs shared by the GPU tests, the bench and the oracle checks.

Holds none of the decoder's arithmetic: it only draws seeded random inputs
(token ids, N(0,1) visual-token embeddings, raw key/value frames) and encodes
them in the storage type the model consumes. Every array comes back twice:
as float32 values (exact) and as the raw storage bits (uint16 for bf16, or
float32), so both sides read the very same numbers.

Draws use numpy's PCG64 seeded by a (seed, stream, call) triple.
"""
from __future__ import annotations

import numpy as np

STREAM_TOKENS = 0x10000
STREAM_EMBEDS = 0x20000
STREAM_RAW_KV = 0x30000
STREAM_CENTRES = 0x40000
STREAM_NOISE = 0x41000
STREAM_ACTION_NOISE = 0x50000


def _gen(seed: int, stream: int, call: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream), int(call)])


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def encode(x32: np.ndarray, storage: str):
    """(exact float32 values, storage array) for storage 'bf16' or 'f32'."""
    x32 = np.asarray(x32, dtype=np.float32)
    if storage == "f32":
        return x32, x32
    if storage == "bf16":
        b = bf16_bits(x32)
        return bf16_to_f32(b), b
    raise ValueError(storage)


def token_ids(seed: int, call: int, n: int, vocab: int) -> np.ndarray:
    """n uniform token ids in [0, vocab) (int32)."""
    return _gen(seed, STREAM_TOKENS, call).integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def embeddings(seed: int, call: int, n: int, hidden: int, storage: str):
    """n visual-token embeddings drawn N(0, 1) per element: (float32 values, storage array)."""
    x = _gen(seed, STREAM_EMBEDS, call).standard_normal((n, hidden), dtype=np.float32)
    return encode(x, storage)


def action_noise(seed: int, call: int, n: int, width: int) -> np.ndarray:
    """An action chunk's starting noise, N(0, 1) per element, float32 [n][width]."""
    return _gen(seed, STREAM_ACTION_NOISE, call).standard_normal((n, width), dtype=np.float32)


def raw_kv_frame(seed: int, frame: int, n_layers: int, ntok: int, n_kv_heads: int,
                 head_dim: int, storage: str):
    """A raw frame's K and V, each [L][ntok][Hkv][d], N(0, 1): ((k32, v32), (k_store, v_store))."""
    g = _gen(seed, STREAM_RAW_KV, frame)
    shape = (n_layers, ntok, n_kv_heads, head_dim)
    k = g.standard_normal(shape, dtype=np.float32)
    v = g.standard_normal(shape, dtype=np.float32)
    k32, ks = encode(k, storage)
    v32, vs = encode(v, storage)
    return (k32, v32), (ks, vs)


def clustered_frame(seed: int, frame: int, n_layers: int, ntok: int, n_kv_heads: int,
                    head_dim: int, n_clusters: int = 16, sigma: float = 0.1,
                    storage: str = "bf16"):
    """A raw frame whose layer-0 keys are a cluster centre plus N(0, sigma^2) noise per token.

    Frame f belongs to cluster f mod n_clusters; the centres are N(0, I) over
    the flattened Hkv*d key vector. Other layers' keys and all values are
    N(0, 1). Returns ((k32, v32), (k_store, v_store)), each [L][ntok][Hkv][d].
    """
    d = n_kv_heads * head_dim
    centres = _gen(seed, STREAM_CENTRES).standard_normal((n_clusters, d), dtype=np.float32)
    g = _gen(seed, STREAM_RAW_KV, frame)
    shape = (n_layers, ntok, n_kv_heads, head_dim)
    k = g.standard_normal(shape, dtype=np.float32)
    v = g.standard_normal(shape, dtype=np.float32)
    noise = _gen(seed, STREAM_NOISE, frame).standard_normal((ntok, d), dtype=np.float32)
    k[0] = (centres[frame % n_clusters][None, :] + np.float32(sigma) * noise).reshape(
        ntok, n_kv_heads, head_dim)
    k32, ks = encode(k, storage)
    v32, vs = encode(v, storage)
    return (k32, v32), (ks, vs)

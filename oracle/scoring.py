"""Redundant-frame scoring of the oracle (fp64).

"Can an LLM Forget the Right Things?", §5: the semantic policy asks which frame
is least likely to be missed; the cosine similarity is a plain dot product and
two norms, with denominator sqrt(|a|^2) * sqrt(|b|^2) and a result of 0 when
that denominator is below 1e-8; on equal similarity the first pair found wins
(strict greater-than), and the older frame of the pair is removed.

The vectors scored here are per-frame mean keys (one layer, both KV heads
concatenated), and every unordered pair of resident frames is compared:

    s_ij = cos(a_i, a_j) for i < j, computed once and used for both i and j
    m_i  = max_{j != i} s_ij
    winner = argmax_i m_i, ties to the lowest index (the oldest frame)
"""
from __future__ import annotations

import numpy as np


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    """dot(a, b) / (sqrt(|a|^2) * sqrt(|b|^2)); 0 when the denominator is < 1e-8."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    dot = float(np.dot(a, b))
    na = float(np.dot(a, a))
    nb = float(np.dot(b, b))
    den = np.sqrt(na) * np.sqrt(nb)
    if den < 1e-8:
        return 0.0
    return dot / den


def pair_matrix(vectors: np.ndarray) -> np.ndarray:
    """Symmetric matrix S with S[i, j] = cosine(v_i, v_j) for i != j and -inf on the diagonal."""
    f = vectors.shape[0]
    s = np.full((f, f), -np.inf)
    for i in range(f):
        for j in range(i + 1, f):
            s[i, j] = s[j, i] = cosine(vectors[i], vectors[j])
    return s


def pick_redundant(vectors: np.ndarray):
    """(index of the frame to evict, its max similarity, the m vector).

    vectors: [F, D] fp64 mean keys in frame-arrival order, F >= 2.
    """
    s = pair_matrix(vectors)
    m = s.max(axis=1)
    win = int(np.argmax(m))          # first occurrence = lowest index on ties
    return win, float(m[win]), m


def mean_key(keys: np.ndarray) -> np.ndarray:
    """fp64 mean over a frame's tokens of its stored keys [ntok, Hkv, d] -> [Hkv*d]."""
    return np.mean(np.asarray(keys, dtype=np.float64), axis=0).reshape(-1)


def adjacent_pair_pick(vectors: np.ndarray) -> int:
    """The page's adjacent-pair rule, for comparison: index of the older frame of the most
    similar neighbouring pair (strict greater-than keeps the first pair on ties)."""
    best, best_s = 0, -2.0
    for i in range(vectors.shape[0] - 1):
        s = cosine(vectors[i], vectors[i + 1])
        if s > best_s:
            best_s, best = s, i
    return best

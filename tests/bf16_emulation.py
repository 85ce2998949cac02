"""Test helper: the oracle's decoder with the device path's bf16 storage points.

The bf16 configurations store the projection inputs (the normalised rows fed
to the q/k/v and gate/up projections, the attention output, the gated FFN
activation), q, the KV cache and the attention probabilities fed to the P*V
product in bf16 (nearest-even), with everything else in higher precision. This copy of the oracle's forward rounds exactly
those values (each point can be switched on alone) and keeps the rest in fp64,
so it gives the error that any implementation storing those values in bf16
carries, whatever its kernels. It is not the oracle and never serves as one:
the tests use it only to state the precision budget of a model.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import decoder as D
from oracle.rng import round_bf16

POINTS = ("u_qkv", "q", "kv", "p", "o", "u_ffn", "act", "head_in")


class Bf16Session(D.Session):
    def __init__(self, cfg: D.Config, points=POINTS, weights=None):
        super().__init__(cfg, weights)
        self.points = set(points)

    def _r(self, x, point):
        return round_bf16(x) if point in self.points else x

    def _forward(self, x, positions, place):
        c = self.cfg
        n = x.shape[0]
        ang = D.rope_angles(positions, c.head_dim, c.rope_theta)
        g = c.n_heads // c.n_kv_heads
        for l in range(c.n_layers):
            t_before = self.resident_tokens() - n
            u = self._r(D.rmsnorm(x, self.w.norm(l), c.rms_eps), "u_qkv")
            q = (u @ self.w.f64("q", l).T).reshape(n, c.n_heads, c.head_dim)
            k = (u @ self.w.f64("k", l).T).reshape(n, c.n_kv_heads, c.head_dim)
            v = (u @ self.w.f64("v", l).T).reshape(n, c.n_kv_heads, c.head_dim)
            q = self._r(D.apply_rope(q, ang), "q")
            k = self._r(D.apply_rope(k, ang), "kv")
            v = self._r(v, "kv")
            place(l, k, v)
            K, V = self.gather(l)
            vis = np.ones((n, K.shape[0]), dtype=bool)
            vis[:, t_before:] = np.tril(np.ones((n, n), dtype=bool))
            o = np.empty((n, c.n_heads, c.head_dim))
            for h in range(c.n_heads):
                s = np.where(vis, (q[:, h] @ K[:, h // g].T) / math.sqrt(c.head_dim), -np.inf)
                p = self._r(np.exp(s - s.max(axis=1, keepdims=True)), "p")
                o[:, h] = (p @ V[:, h // g]) / p.sum(axis=1, keepdims=True)
            o = self._r(o, "o")
            x = x + o.reshape(n, -1) @ self.w.f64("o", l).T
            u2 = self._r(D.rmsnorm(x, self.w.norm(l), c.rms_eps), "u_ffn")
            a = (D.gelu_erf if c.ffn_kind == "geglu" else D.silu)(u2 @ self.w.f64("gate", l).T) \
                * (u2 @ self.w.f64("up", l).T)
            x = x + self._r(a, "act") @ self.w.f64("down", l).T
        return x

    def _logits(self, h_last):
        u = self._r(D.rmsnorm(h_last, self.w.norm(), self.cfg.rms_eps), "head_in")
        return self.w.f64("head") @ u

"""The oracle's pi0-style two-part policy step (fp64, numpy): TEST INFRASTRUCTURE ONLY.

"Running VLAs at Real-time Speed", §2: pi0 couples a vision-language prefix
model (VLM) with an action expert (AE) that predicts an action chunk by flow
matching; §4.1: the VLM's last layer is reduced to the K/V it hands to the
expert; §4.2: gated FFNs. What is computed here:

  prefix   the VLM (decoder.Session with GeGLU and a K/V-only last layer)
           prefills the image-token embeddings; its layer-l cache is the
           prefix K/V of expert layer l.
  velocity v(x, tau) for the action chunk x [n][H_ae]:
             h = x + temb(tau)                        (time enters additively)
             per layer l: u = RMSNorm(h); q, k, v = u W^T; RoPE at positions
             P .. P+n-1 (P = the prefix's next position); o = softmax(q K^T /
             sqrt(d)) V over K, V = [prefix layer-l K/V ; the chunk's own k, v]
             with every key visible (the chunk attends to itself in both
             directions); h += o Wo^T; h += Wdown-map of gelu(u2 Wg^T) *
             (u2 Wu^T), u2 = RMSNorm(h)
             v = RMSNorm(h)                           (no output projection)
  denoise  Euler steps x <- x + dt * v(x, tau_k), tau_k = k * dt, k = 0 ..
           steps-1, from the noise at tau = 0.

Readings (the pages give none of these): the time embedding is the sinusoidal
one with periods spaced geometrically from 0.004 to 4 over the first half of
the width (sines) and repeated for the cosines; the action tokens live in the
expert's width with no input or output projection; the expert's weights use
the per-layer weight streams offset by 0x8000 so they differ from the VLM's.
"""
from __future__ import annotations

import math

import numpy as np

from . import decoder as D

AE_STREAM_BASE = 0x8000

# Gemma-2B-shaped prefix (17 full layers + the K/V-only 18th) and the 300M-parameter
# action expert, bf16 weights, both seeded from the workload's seed
C4_VLM = D.Config("c4_pi0_vlm", 18, 2048, 8, 1, 256, 16384, 0, rope_theta=1e4,
                  wdtype="bf16", act="bf16", num_blocks=40, max_frames=4, seed=1238,
                  ffn_kind="geglu", kv_only_last=True)
C4_AE = D.Config("c4_pi0_action_expert", 18, 1024, 8, 1, 256, 4096, 0, rope_theta=1e4,
                 wdtype="bf16", act="bf16", num_blocks=0, max_frames=0, seed=1238,
                 ffn_kind="geglu", stream_base=AE_STREAM_BASE)
C4_PREFIX_TOKENS = 512      # 2 views x 256 image tokens, empty prompt
C4_ACTIONS = 63
C4_STEPS = 10


def time_embedding(tau: float, width: int) -> np.ndarray:
    """[sin(tau w_j) for j < width/2] ++ [cos(tau w_j)], w_j = 2 pi / p_j,
    p_j = 0.004 * 1000^(j / (width/2 - 1)) (fp64)."""
    half = width // 2
    frac = np.arange(half, dtype=np.float64) / (half - 1)
    period = 0.004 * (4.0 / 0.004) ** frac
    ang = tau * (2.0 * math.pi / period)
    return np.concatenate([np.sin(ang), np.cos(ang)])


class ActionExpert:
    """The expert bound to a prefix session (the VLM); reads its resident K/V."""

    def __init__(self, cfg: D.Config, prefix: D.Session, weights: D.Weights | None = None):
        if cfg.n_layers != prefix.cfg.n_layers or cfg.n_kv_heads != prefix.cfg.n_kv_heads \
                or cfg.head_dim != prefix.cfg.head_dim:
            raise ValueError("expert layers / KV heads / head dim must match the prefix")
        self.cfg = cfg
        self.prefix = prefix
        self.w = weights if weights is not None else D.Weights(cfg)

    def velocity(self, x: np.ndarray, tau: float) -> np.ndarray:
        c = self.cfg
        n = x.shape[0]
        h = np.asarray(x, dtype=np.float64) + time_embedding(tau, c.hidden)[None, :]
        pos = self.prefix.next_pos + np.arange(n)
        ang = D.rope_angles(pos, c.head_dim, c.rope_theta)
        for l in range(c.n_layers):
            u = D.rmsnorm(h, self.w.norm(l), c.rms_eps)
            q = D.apply_rope((u @ self.w.f64("q", l).T).reshape(n, c.n_heads, c.head_dim), ang)
            k = D.apply_rope((u @ self.w.f64("k", l).T).reshape(n, c.n_kv_heads, c.head_dim),
                             ang)
            v = (u @ self.w.f64("v", l).T).reshape(n, c.n_kv_heads, c.head_dim)
            Kp, Vp = self.prefix.gather(l)
            K = np.concatenate([Kp, k])
            V = np.concatenate([Vp, v])
            visible = np.ones((n, K.shape[0]), dtype=bool)
            o = D.gqa_attention(q, K, V, visible)
            h = h + o.reshape(n, -1) @ self.w.f64("o", l).T
            u2 = D.rmsnorm(h, self.w.norm(l), c.rms_eps)
            h = h + D.ffn(c, u2, self.w.f64("gate", l), self.w.f64("up", l),
                          self.w.f64("down", l))
        return D.rmsnorm(h, self.w.norm(), c.rms_eps)

    def denoise(self, x0: np.ndarray, steps: int = C4_STEPS, dt: float | None = None):
        """Euler integration from tau = 0: returns the final action chunk."""
        dt = 1.0 / steps if dt is None else dt
        x = np.asarray(x0, dtype=np.float64)
        for k in range(steps):
            x = x + dt * self.velocity(x, k * dt)
        return x


def param_count(cfg: D.Config) -> int:
    """Projection parameters of a decoder's layers (no embedding, no head)."""
    qd, kd = cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    per = (qd + 2 * kd) * cfg.hidden + cfg.hidden * qd + 3 * cfg.ffn * cfg.hidden
    return per * cfg.n_layers

"""Pins of the oracle's pi0-style policy step against things other than itself.

* exact GELU: the normal CDF's textbook values and its odd symmetry;
* the time embedding's closed forms (tau = 0, quarter periods);
* the Euler loop with a velocity that ignores x (x_0 plus the sum of dt v(tau_k));
* the expert's velocity against HF Llama (exact-GELU MLP) run bidirectionally
  over the prefix model's cache, in fp64;
* the K/V-only last layer stores exactly the K/V a full model stores;
* the expert's parameter count against the pages' "300M".
"""
import math

import numpy as np
import torch

from oracle import decoder as D
from oracle import pi0
from tests.test_oracle_decoder import _hf_model, rel

VLM_T = D.Config("vlm_t", n_layers=3, hidden=64, n_heads=4, n_kv_heads=1, head_dim=32, ffn=96,
                 vocab=0, rope_theta=1e4, wdtype="f32", act="f32", num_blocks=16, max_frames=4,
                 seed=81, init_std=0.2, ffn_kind="geglu", kv_only_last=True)
AE_T = D.Config("ae_t", n_layers=3, hidden=48, n_heads=4, n_kv_heads=1, head_dim=32, ffn=80,
                vocab=0, rope_theta=1e4, wdtype="f32", act="f32", num_blocks=0, max_frames=0,
                seed=81, init_std=0.2, ffn_kind="geglu", stream_base=pi0.AE_STREAM_BASE)


def test_gelu_textbook_values_and_symmetry():
    phi1 = 0.8413447460685429            # standard normal CDF at 1
    z = np.array([0.0, 1.0, -1.0, 8.0, -8.0])
    g = D.gelu_erf(z)
    assert g[0] == 0.0
    assert abs(g[1] - phi1) < 1e-15 and abs(g[2] + (1 - phi1)) < 1e-15
    assert abs(g[3] - 8.0) < 1e-13 and abs(g[4]) < 1e-13
    x = np.random.default_rng(0).standard_normal(100) * 3
    assert np.max(np.abs(D.gelu_erf(x) - D.gelu_erf(-x) - x)) < 1e-14


def test_time_embedding_closed_forms():
    e0 = pi0.time_embedding(0.0, 1024)
    assert np.array_equal(e0, np.concatenate([np.zeros(512), np.ones(512)]))
    # shortest period 0.004: a quarter period gives sin = 1; longest period 4
    assert abs(pi0.time_embedding(0.001, 1024)[0] - 1.0) < 1e-12
    assert abs(pi0.time_embedding(1.0, 1024)[511] - 1.0) < 1e-12
    assert abs(pi0.time_embedding(2.0, 1024)[1023] + 1.0) < 1e-12


def test_euler_with_x_independent_velocity():
    """x_10 = x_0 + sum_k 0.1 v(tau_k), tau_k = k / 10, k = 0..9 (the same additions)."""
    prefix = D.Session(VLM_T)
    ae = pi0.ActionExpert(AE_T, prefix)
    ae.velocity = lambda x, tau: np.full_like(x, tau * tau)
    x0 = np.random.default_rng(1).standard_normal((5, AE_T.hidden))
    got = ae.denoise(x0, steps=10)
    ref = x0.copy()
    for k in range(10):
        ref = ref + 0.1 * (k * 0.1) ** 2
    assert np.array_equal(got, ref)
    assert abs(np.mean(got - x0) - 0.1 * sum((k / 10) ** 2 for k in range(10))) < 1e-14


def _prefix_session():
    s = D.Session(VLM_T)
    x = np.random.default_rng(2).standard_normal((10, VLM_T.hidden))
    fid, logits = s.prefill_chunk(embeds=x)
    assert logits is None
    return s


def test_kv_only_last_layer_stores_what_a_full_model_stores():
    s = _prefix_session()
    full = D.Session(VLM_T.with_(kv_only_last=False), D.Weights(VLM_T.with_(kv_only_last=False)))
    full.prefill_chunk(embeds=np.random.default_rng(2).standard_normal((10, VLM_T.hidden)))
    for l in range(VLM_T.n_layers):
        a, b = s.gather(l), full.gather(l)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_expert_velocity_matches_hf_llama_bidirectional_over_prefix_cache():
    from transformers import DynamicCache
    prefix = _prefix_session()
    ae = pi0.ActionExpert(AE_T, prefix)
    x = np.random.default_rng(3).standard_normal((7, AE_T.hidden))
    tau = 0.3
    ours = ae.velocity(x, tau)

    m = _hf_model(AE_T, ae.w, exact_angles=True).model
    cache = DynamicCache()
    for l in range(AE_T.n_layers):
        K, V = prefix.gather(l)                      # [T, Hkv, d], post-RoPE
        cache.update(torch.from_numpy(K.transpose(1, 0, 2)[None].copy()),
                     torch.from_numpy(V.transpose(1, 0, 2)[None].copy()), l)
    T = prefix.resident_tokens()
    n = x.shape[0]
    h0 = x + pi0.time_embedding(tau, AE_T.hidden)[None, :]
    mask = torch.zeros((1, 1, n, T + n), dtype=torch.float64)     # every key visible
    with torch.no_grad():
        out = m(inputs_embeds=torch.from_numpy(h0)[None],
                position_ids=torch.arange(T, T + n)[None], past_key_values=cache,
                attention_mask=mask, use_cache=True).last_hidden_state[0].numpy()
    assert rel(ours, out) < 1e-10
    # and the chunk really attends to itself in both directions
    x2 = x.copy()
    x2[-1] += 1.0
    assert np.max(np.abs(ae.velocity(x2, tau)[0] - ours[0])) > 1e-6


def test_expert_parameter_count_is_the_pages_300m():
    n = pi0.param_count(pi0.C4_AE)
    assert n == 311_427_072
    assert abs(n - 300e6) / 300e6 < 0.05

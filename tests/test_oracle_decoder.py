"""Pins of the oracle's decoder against things other than itself.

* a textbook library model: the HF Llama forward (pre-norm RMSNorm, rotate-half
  RoPE, GQA, SwiGLU, untied head) on the very same weights, in fp64;
* torch's scaled-dot-product attention for the masked GQA attention;
* the dense, uncached causal forward (the cached session must equal it);
* invariants: chunking, paged vs contiguous storage, GQA -> MHA, RoPE norm and
  relative-position properties, identity layers, one-key / equal-key attention,
  the online (m, l, o) softmax of "Rebuilding Kshipra Around Memory", §4.
"""
import math

import numpy as np
import pytest
import torch

from oracle import decoder as D
from oracle.kvpool import NoBlocks

T1 = D.Config("t1", n_layers=2, hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, ffn=96,
              vocab=128, rope_theta=1e4, wdtype="f32", act="f32", num_blocks=16,
              max_frames=8, seed=77, init_std=0.2)


def rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / np.max(np.abs(np.asarray(b))))


def _hf_model(cfg, w, exact_angles):
    """HF Llama on the oracle's weights (hidden_act "gelu" = exact GELU for GeGLU configs;
    a config without vocabulary gets a one-row dummy embedding and head)."""
    from transformers import LlamaConfig, LlamaForCausalLM
    act = {"swiglu": "silu", "geglu": "gelu"}[cfg.ffn_kind]
    hc = LlamaConfig(vocab_size=max(cfg.vocab, 1), hidden_act=act,
                     hidden_size=cfg.hidden, intermediate_size=cfg.ffn,
                     num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_heads,
                     num_key_value_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                     rms_norm_eps=cfg.rms_eps,
                     rope_parameters={"rope_type": "default", "rope_theta": cfg.rope_theta},
                     tie_word_embeddings=False, attention_bias=False, mlp_bias=False,
                     max_position_embeddings=1 << 20)
    hc._attn_implementation = "sdpa"   # the eager path runs its softmax in fp32
    m = LlamaForCausalLM(hc).double().eval()
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    with torch.no_grad():
        if cfg.vocab:
            m.model.embed_tokens.weight.copy_(t(w.f64("embed")))
            m.lm_head.weight.copy_(t(w.f64("head")))
        m.model.norm.weight.fill_(1.0)
        for l, layer in enumerate(m.model.layers):
            a, f = layer.self_attn, layer.mlp
            a.q_proj.weight.copy_(t(w.f64("q", l)))
            a.k_proj.weight.copy_(t(w.f64("k", l)))
            a.v_proj.weight.copy_(t(w.f64("v", l)))
            a.o_proj.weight.copy_(t(w.f64("o", l)))
            f.gate_proj.weight.copy_(t(w.f64("gate", l)))
            f.up_proj.weight.copy_(t(w.f64("up", l)))
            f.down_proj.weight.copy_(t(w.f64("down", l)))
            layer.input_layernorm.weight.fill_(1.0)
            layer.post_attention_layernorm.weight.fill_(1.0)
    if exact_angles:
        # HF evaluates the RoPE angles in fp32; re-evaluate them in fp64 so the
        # rest of the model can be compared at fp64 precision.
        rot = m.model.rotary_emb
        inv = 1.0 / (cfg.rope_theta ** (torch.arange(0, cfg.head_dim, 2, dtype=torch.float64)
                                        / cfg.head_dim))

        def fwd(x, position_ids):
            fr = position_ids[:, :, None].double() * inv[None, None, :]
            emb = torch.cat((fr, fr), dim=-1)
            return emb.cos().to(x.dtype), emb.sin().to(x.dtype)
        rot.forward = fwd
        # HF's RMSNorm also evaluates in fp32; use torch's fp64 rms_norm routine instead
        norms = [m.model.norm] + [x for ly in m.model.layers
                                  for x in (ly.input_layernorm, ly.post_attention_layernorm)]
        for nm in norms:
            nm.forward = (lambda mod: lambda h: torch.nn.functional.rms_norm(
                h, (h.shape[-1],), mod.weight, eps=cfg.rms_eps))(nm)
    return m


@pytest.mark.parametrize("exact_angles,tol", [(True, 1e-10), (False, 1e-4)])
def test_dense_forward_matches_hf_llama(exact_angles, tol):
    w = D.Weights(T1)
    ids = np.random.default_rng(1).integers(0, T1.vocab, 40)
    ours = D.dense_forward(T1, w, w.f64("embed")[ids], np.arange(40))
    m = _hf_model(T1, w, exact_angles)
    with torch.no_grad():
        ref = m(torch.from_numpy(ids)[None]).logits[0].numpy()
    assert rel(ours, ref) < tol


def test_c1_shape_matches_hf_llama():
    cfg = D.C1
    w = D.Weights(cfg)
    ids = np.random.default_rng(2).integers(0, cfg.vocab, 80)
    ours = D.dense_forward(cfg, w, w.f64("embed")[ids], np.arange(80))
    m = _hf_model(cfg, w, exact_angles=True)
    with torch.no_grad():
        ref = m(torch.from_numpy(ids)[None]).logits[0].numpy()
    assert rel(ours, ref) < 1e-10


def test_geglu_dense_forward_matches_hf_llama_with_exact_gelu():
    cfg = T1.with_(name="t1g", ffn_kind="geglu", seed=78)
    w = D.Weights(cfg)
    ids = np.random.default_rng(6).integers(0, cfg.vocab, 30)
    ours = D.dense_forward(cfg, w, w.f64("embed")[ids], np.arange(30))
    m = _hf_model(cfg, w, exact_angles=True)
    with torch.no_grad():
        ref = m(torch.from_numpy(ids)[None]).logits[0].numpy()
    assert rel(ours, ref) < 1e-10


def test_cached_session_equals_dense_forward():
    w = D.Weights(T1)
    g = np.random.default_rng(3)
    s = D.Session(T1, w)
    chunks = [g.integers(0, T1.vocab, n) for n in (16, 7, 9)]
    got = []
    for c in chunks:
        got.append(s.prefill_chunk(tokens=c)[1])
    toks = [int(t) for t in g.integers(0, T1.vocab, 5)]
    for t in toks:
        got.append(s.decode_step(t)[1])
    seq = np.concatenate(chunks + [np.array(toks)])
    dense = D.dense_forward(T1, w, w.f64("embed")[seq], np.arange(seq.size))
    ends = np.cumsum([c.size for c in chunks]) - 1
    ref = [dense[e] for e in ends] + [dense[ends[-1] + 1 + i] for i in range(len(toks))]
    for a, b in zip(got, ref):
        assert rel(a, b) < 1e-11


def test_chunking_invariance():
    w = D.Weights(T1)
    x = np.random.default_rng(4).standard_normal((32, T1.hidden))
    one = D.Session(T1, w).prefill_chunk(embeds=x)[1]
    s = D.Session(T1, w)
    for a, b in ((0, 5), (5, 16), (16, 32)):
        last = s.prefill_chunk(embeds=x[a:b])[1]
    assert rel(last, one) < 1e-12


def test_paged_equals_contiguous_bit_exact():
    w = D.Weights(T1)
    g = np.random.default_rng(5)
    perm = list(g.permutation(T1.num_blocks))
    a = D.Session(T1, w, paged=False)
    b = D.Session(T1, w, paged=True, initial_free=perm)
    for n in (20, 3, 17):
        x = g.standard_normal((n, T1.hidden))
        la = a.prefill_chunk(embeds=x)[1]
        lb = b.prefill_chunk(embeds=x)[1]
        assert np.array_equal(la, lb)
    for t in (3, 9, 27, 4):
        assert np.array_equal(a.decode_step(t)[1], b.decode_step(t)[1])
    # the physical blocks really are scattered
    assert [blk for blk, _ in b.block_table()] != sorted(blk for blk, _ in b.block_table())


def test_gqa_reduces_to_mha_with_repeated_kv_heads():
    cfg = T1
    w = D.Weights(cfg)
    mha = cfg.with_(n_kv_heads=cfg.n_heads)
    wm = D.Weights(mha)
    for name in ("embed", "head"):
        wm.set(name, -1, w.f64(name))
    g = cfg.group
    for l in range(cfg.n_layers):
        for name in ("q", "o", "gate", "up", "down"):
            wm.set(name, l, w.f64(name, l))
        for name in ("k", "v"):
            heads = w.f64(name, l).reshape(cfg.n_kv_heads, cfg.head_dim, cfg.hidden)
            wm.set(name, l, np.repeat(heads, g, axis=0).reshape(-1, cfg.hidden))
    x = np.random.default_rng(6).standard_normal((24, cfg.hidden))
    a = D.Session(cfg, w).prefill_chunk(embeds=x)[1]
    b = D.Session(mha, wm).prefill_chunk(embeds=x)[1]
    assert rel(a, b) < 1e-12


def test_gqa_attention_matches_torch_sdpa():
    g = np.random.default_rng(7)
    n, T, hq, hkv, d = 9, 30, 6, 2, 16
    q = g.standard_normal((n, hq, d))
    k = g.standard_normal((T, hkv, d))
    v = g.standard_normal((T, hkv, d))
    vis = np.ones((n, T), dtype=bool)
    vis[:, T - n:] = np.tril(np.ones((n, n), dtype=bool))
    ours = D.gqa_attention(q, k, v, vis)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None].contiguous()
    tv = torch.from_numpy(v).permute(1, 0, 2)[None].contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(vis), enable_gqa=True)
    assert rel(ours, ref[0].permute(1, 0, 2).numpy()) < 1e-13


def test_one_visible_key_and_equal_keys():
    g = np.random.default_rng(8)
    q = g.standard_normal((1, 2, 8))
    k = g.standard_normal((5, 1, 8))
    v = g.standard_normal((5, 1, 8))
    vis = np.zeros((1, 5), dtype=bool)
    vis[0, 3] = True
    o = D.gqa_attention(q, k, v, vis)
    assert np.allclose(o[0, 0], v[3, 0], rtol=0, atol=1e-15)
    assert np.allclose(o[0, 1], v[3, 0], rtol=0, atol=1e-15)
    keq = np.repeat(k[:1], 5, axis=0)
    o = D.gqa_attention(q, keq, v, np.ones((1, 5), dtype=bool))
    assert np.allclose(o[0, 0], v[:, 0].mean(axis=0), atol=1e-14)


def test_online_block_softmax_equals_two_pass():
    # the (m, l, o) recurrence over KV blocks of "Rebuilding Kshipra Around Memory", §4
    g = np.random.default_rng(9)
    d, T = 16, 70
    q = g.standard_normal(d) * 3
    k = g.standard_normal((T, d))
    v = g.standard_normal((T, d))
    scale = 1 / math.sqrt(d)
    m, l_, o = -np.inf, 0.0, np.zeros(d)
    for b in range(0, T, 16):
        s = k[b:b + 16] @ q * scale
        m_new = max(m, s.max())
        p = np.exp(s - m_new)
        l_ = l_ * math.exp(m - m_new) + p.sum()
        o = o * math.exp(m - m_new) + p @ v[b:b + 16]
        m = m_new
    ours = D.gqa_attention(q[None, None], k[:, None], v[:, None], np.ones((1, T), dtype=bool))
    assert rel(ours[0, 0], o / l_) < 1e-13


def test_rope_preserves_norm_and_depends_on_relative_position():
    g = np.random.default_rng(10)
    d = 64
    qv = g.standard_normal((1, 1, d))
    kv = g.standard_normal((1, 1, d))
    for p in (0, 1, 17, 1000, 120_000):
        r = D.apply_rope(qv, D.rope_angles([p], d, 5e5))
        assert abs(np.linalg.norm(r) - np.linalg.norm(qv)) < 1e-12 * np.linalg.norm(qv)
    dots = []
    for m_, n_ in ((5, 2), (105, 102), (100_003, 100_000)):
        a = D.apply_rope(qv, D.rope_angles([m_], d, 1e4))
        b = D.apply_rope(kv, D.rope_angles([n_], d, 1e4))
        dots.append(float(np.sum(a * b)))
    assert max(dots) - min(dots) < 1e-9


def test_rope_unit_vector_rotation_and_hf_helper():
    d, theta, p = 8, 1e4, 3
    ang = D.rope_angles([p], d, theta)
    for j in range(d // 2):
        e = np.zeros((1, 1, d))
        e[0, 0, j] = 1.0
        r = D.apply_rope(e, ang)[0, 0]
        w = p * theta ** (-2.0 * j / d)
        want = np.zeros(d)
        want[j], want[j + d // 2] = math.cos(w), math.sin(w)
        assert np.allclose(r, want, atol=1e-15)
    # the HF helper (rotate_half form) on the same cos / sin tables
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    g = np.random.default_rng(11)
    x = g.standard_normal((5, 2, d))
    ang = D.rope_angles(np.arange(7, 12), d, theta)
    cos = torch.from_numpy(np.concatenate([np.cos(ang)] * 2, axis=-1))[None]
    sin = torch.from_numpy(np.concatenate([np.sin(ang)] * 2, axis=-1))[None]
    t = torch.from_numpy(x).permute(1, 0, 2)[None]
    ref, _ = apply_rotary_pos_emb(t, t, cos, sin)
    assert rel(D.apply_rope(x, ang), ref[0].permute(1, 0, 2).numpy()) < 1e-15


def test_position_shift_leaves_logits_unchanged():
    w = D.Weights(T1)
    x = np.random.default_rng(12).standard_normal((12, T1.hidden))
    a = D.dense_forward(T1, w, x, np.arange(12))
    b = D.dense_forward(T1, w, x, np.arange(12) + 5000)
    assert rel(a, b) < 1e-10


def test_rmsnorm_and_silu_match_torch():
    g = np.random.default_rng(13)
    x = g.standard_normal((7, 33)) * 5
    gw = g.standard_normal(33)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(gw), eps=1e-6)
    assert rel(D.rmsnorm(x, gw, 1e-6), ref.numpy()) < 1e-14
    z = g.standard_normal(1000) * 10
    assert rel(D.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy()) < 1e-14


def test_identity_layers_give_head_of_normed_embedding():
    w = D.Weights(T1)
    for l in range(T1.n_layers):
        w.set("o", l, np.zeros(w.shape("o")))
        w.set("down", l, np.zeros(w.shape("down")))
    ids = np.array([5, 9, 100, 3])
    _, logits = D.Session(T1, w).prefill_chunk(tokens=ids)
    x0 = w.f64("embed")[3]
    want = w.f64("head") @ (x0 / np.sqrt(np.mean(x0 ** 2) + T1.rms_eps))
    assert rel(logits, want) < 1e-14


def test_no_blocks_leaves_state_unchanged():
    cfg = T1.with_(num_blocks=4)
    s = D.Session(cfg)
    s.prefill_chunk(embeds=np.ones((40, cfg.hidden)))     # 3 blocks
    before = (list(s.pool.free), s.next_pos, s.next_frame_id, len(s.segments))
    with pytest.raises(NoBlocks):
        s.prefill_chunk(embeds=np.ones((20, cfg.hidden)))  # needs 2, 1 free
    assert before == (list(s.pool.free), s.next_pos, s.next_frame_id, len(s.segments))

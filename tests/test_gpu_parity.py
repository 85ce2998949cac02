"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Small configurations that the oracle finishes in seconds, spanning several
tiles with ragged tails: the fp32 tiny decoder (its exact workload shape), a
tiny bf16 decoder with ragged chunks, interleaved decode tails and raw-frame
eviction. Every input comes from synth.py; every expected value from oracle/.
"""
import numpy as np
import pytest
import torch

import kv_cached_gqa_decoder_amd as vla
import synth
from oracle import decoder as D
from tests.gpu_util import (KEY_BAND, check_argmax, check_logits, dev_from_storage,
                            eviction_margin, log, logits_of, metrics, oracle_config)

pytestmark = pytest.mark.gpu

TINY_BF16 = dict(n_layers=2, hidden=256, n_heads=6, n_kv_heads=2, head_dim=128, ffn=512,
                 vocab=1000, rope_theta=1e4, wdtype=vla.VLA_BF16, num_blocks=40, max_frames=8,
                 max_chunk=160, seed=99)


# INT4 group-128 projections with bf16 activations (every K a multiple of 128)
TINY_INT4 = dict(TINY_BF16, n_heads=4, wdtype=vla.VLA_INT4_G128, seed=98)


def _model(p, init_std=0.02):
    return vla.Model(vla.make_config(**p, init_std=init_std))


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("which", ["c1", "tiny_bf16", "tiny_int4"])
def test_device_weights_equal_oracle_weights(which):
    """Device-generated weights equal the oracle's bit for bit; INT4 projections are
    compared dequantised (q * s is exact in fp32, so equal values mean equal codes
    and equal fp16 scales wherever a group is not all zero)."""
    p = {"c1": vla.PRESETS["c1_tiny_f32"], "tiny_bf16": TINY_BF16, "tiny_int4": TINY_INT4}[which]
    ocfg = oracle_config(p)
    w = D.Weights(ocfg, cache_f64=False)
    m = _model(p)
    kinds = {1: "q", 2: "k", 3: "v", 4: "o", 5: "gate", 6: "up", 7: "down", 8: "embed",
             9: "head"}
    for kind, name in kinds.items():
        for layer in ([0, p["n_layers"] - 1] if kind <= 7 else [-1]):
            ref = w.f32(name, layer)
            dt = torch.float32 if which == "c1" or (which == "tiny_int4" and kind != 8) \
                else torch.bfloat16
            out = torch.empty(ref.shape, dtype=dt, device="cuda")
            m.weight_out(kind, max(layer, 0), out, out.numel() * out.element_size())
            got = out.float().cpu().numpy()
            assert np.array_equal(got, ref), f"{name} layer {layer}"
    m.close()


# ---------------------------------------------------------------------------
def _run_c1(init_std):
    p = vla.PRESETS["c1_tiny_f32"]
    ocfg = oracle_config(p, init_std=init_std)
    sess = D.Session(ocfg)
    m = _model(p, init_std)
    ids = synth.token_ids(ocfg.seed, 0, 64, ocfg.vocab)
    m.prefill_chunk(tokens=ids)
    _, ref = sess.prefill_chunk(tokens=ids)
    out = [metrics(logits_of(m), ref)]
    check_logits(logits_of(m), ref, "f32", "c1 prefill")
    tok = int(np.argmax(ref))
    for step in range(16):
        g = m.decode_step(tok)
        nxt, ref = sess.decode_step(tok)
        check_logits(logits_of(m), ref, "f32", f"c1 decode {step}")
        check_argmax(g, ref, "f32", f"c1 decode {step}")
        out.append(metrics(logits_of(m), ref))
        tok = nxt
    log("c1 worst cos %.7f worst rel %.2e" % (min(c for c, _ in out), max(r for _, r in out)))
    return m, sess


@pytest.mark.parametrize("init_std", [0.02, 0.1])
def test_c1_prefill_and_greedy_decode(init_std):
    m, sess = _run_c1(init_std)
    # stored keys / values of every layer, in logical order
    T = sess.resident_tokens()
    c = sess.cfg
    for layer in range(c.n_layers):
        k = torch.empty((T, c.n_kv_heads, c.head_dim), dtype=torch.float32, device="cuda")
        v = torch.empty_like(k)
        n = m.kv_gather(layer, k, v, T)
        K, V = sess.gather(layer)
        assert n == T
        assert metrics(k.cpu().numpy().ravel(), K.ravel())[1] < 1e-5
        assert metrics(v.cpu().numpy().ravel(), V.ravel())[1] < 1e-5
    m.close()


# ---------------------------------------------------------------------------
def test_bf16_ragged_chunks_interleaved_decodes_and_eviction():
    p = TINY_BF16
    init_std = 0.08
    ocfg = oracle_config(p, init_std=init_std)
    sess = D.Session(ocfg)
    m = _model(p, init_std)
    H = p["hidden"]
    call = 0

    def prefill_embeds(n):
        nonlocal call
        x32, xs = synth.embeddings(p["seed"], call, n, H, "bf16")
        call += 1
        fid = m.prefill_chunk(embeds=dev_from_storage(xs, "bf16"), n=n)
        ofid, ref = sess.prefill_chunk(embeds=x32)
        assert fid == ofid
        check_logits(logits_of(m), ref, "bf16", f"prefill n={n}")
        return ref

    def prefill_ids(n):
        nonlocal call
        ids = synth.token_ids(p["seed"], call, n, p["vocab"])
        call += 1
        fid = m.prefill_chunk(tokens=ids)
        ofid, ref = sess.prefill_chunk(tokens=ids)
        assert fid == ofid
        check_logits(logits_of(m), ref, "bf16", f"prefill ids n={n}")
        return ref

    def decode(ref, k):
        tok = int(np.argmax(ref))
        for i in range(k):
            g = m.decode_step(tok)
            nxt, ref = sess.decode_step(tok)
            check_logits(logits_of(m), ref, "bf16", f"decode {i}")
            check_argmax(g, ref, "bf16", f"decode {i}")
            tok = nxt
        return ref

    ref = prefill_embeds(37)       # 3 blocks, ragged
    ref = prefill_ids(100)         # several 16-row tiles, ragged
    ref = decode(ref, 3)           # a tail segment
    ref = prefill_embeds(16)       # exactly one block
    ref = prefill_embeds(1)        # a one-token frame
    ref = decode(ref, 18)          # tail spanning two blocks
    ref = prefill_embeds(61)
    blocks, ntok = m.block_table()
    assert [(int(b), int(n)) for b, n in zip(blocks, ntok)] == sess.block_table()
    # mean keys: GPU (bf16-stored keys) vs oracle (fp64 keys) are close, not exact
    for layer in (0, 1):
        mk = m.mean_keys(layer)
        omk = np.stack([v for _, v in sess.mean_keys(layer)])
        assert mk.shape == omk.shape
        assert metrics(mk.ravel(), omk.ravel())[1] < 2e-2
    # eviction: each side scores its own keys (the device's are bf16-rounded), so
    # the picks are compared only when the oracle's margin is outside the key band;
    # the oracle always evicts its own pick and never takes the device's
    gfid, _ = m.kv_score(0)
    omk = [v for _, v in sess.mean_keys(0)]
    win, gap, _ = eviction_margin(np.stack(omk))
    ofid, oscore = sess.score_and_evict(0)
    log(f"  eviction: oracle frame {ofid}, margin {gap:.3e} (band {KEY_BAND})")
    if gap < KEY_BAND:
        log("  eviction margin inside the key band: comparison stops here")
        m.close()
        return
    assert gfid == ofid, (gfid, ofid)
    fid, score = m.kv_score_and_evict(0)
    assert fid == ofid and abs(score - oscore) < KEY_BAND
    assert m.free_list() == sess.pool.free
    ref = prefill_embeds(40)       # reuses the freed blocks
    blocks, ntok = m.block_table()
    assert [(int(b), int(n)) for b, n in zip(blocks, ntok)] == sess.block_table()
    assert m.free_list() == sess.pool.free
    decode(ref, 2)
    m.close()


# ---------------------------------------------------------------------------
def test_raw_frames_mean_keys_and_eviction_bit_exact():
    """Stored keys are given, so both sides score the very same numbers: mean keys
    must be bit-identical and every eviction must pick the same frame."""
    p = dict(TINY_BF16, num_blocks=64, max_frames=12)
    ocfg = oracle_config(p)
    sess = D.Session(ocfg)
    m = _model(p)
    L, hkv, d = p["n_layers"], p["n_kv_heads"], p["head_dim"]
    for f in range(12):
        n = 64 if f % 3 else 40
        (k32, v32), (ks, vs) = synth.clustered_frame(7, f, L, n, hkv, d, n_clusters=5)
        fid = m.kv_append_raw(dev_from_storage(ks, "bf16"), dev_from_storage(vs, "bf16"), n)
        assert fid == sess.append_raw(k32, v32)
    for layer in range(L):
        mk = m.mean_keys(layer)
        omk = np.stack([v for _, v in sess.mean_keys(layer)])
        assert np.array_equal(mk, omk), layer
    for cycle in range(10):
        fid, score = m.kv_score_and_evict(0)
        ofid, oscore = sess.score_and_evict(0)
        assert fid == ofid, (cycle, fid, ofid)
        assert abs(score - oscore) < 1e-12
        blocks, ntok = m.block_table()
        assert [(int(b), int(n)) for b, n in zip(blocks, ntok)] == sess.block_table()
        assert m.free_list() == sess.pool.free
    # the scoring on layer 1 (no cluster structure) also agrees
    assert m.kv_score(1)[0] == sess.score(1)[0]
    m.close()


# ---------------------------------------------------------------------------
def test_error_paths_leave_state_unchanged():
    p = dict(TINY_BF16, num_blocks=6, max_frames=3)
    m = _model(p)
    x = torch.zeros((80, p["hidden"]), dtype=torch.bfloat16, device="cuda")
    m.prefill_chunk(embeds=x, n=80)                 # 5 blocks
    st0 = m.state()
    with pytest.raises(vla.VlaError) as e:
        m.prefill_chunk(embeds=x, n=20)             # needs 2 blocks, 1 free
    assert e.value.status == vla.VLA_E_NO_BLOCKS and m.state() == st0
    with pytest.raises(vla.VlaError) as e:
        m.kv_score_and_evict(0)
    assert e.value.status == vla.VLA_E_NOTHING_TO_EVICT and m.state() == st0
    with pytest.raises(vla.VlaError) as e:
        m.decode_step(p["vocab"])
    assert e.value.status == vla.VLA_E_INVALID and m.state() == st0
    with pytest.raises(vla.VlaError) as e:
        m.prefill_chunk(embeds=x, n=0)
    assert e.value.status == vla.VLA_E_INVALID
    for _ in range(16):
        m.decode_step(1)                            # the last free block
    st1 = m.state()
    with pytest.raises(vla.VlaError) as e:
        m.decode_step(1)
    assert e.value.status == vla.VLA_E_NO_BLOCKS and m.state() == st1
    m.close()


def test_rollback_repeats_bit_identically():
    p = TINY_BF16
    m = _model(p, 0.08)
    x32, xs = synth.embeddings(5, 0, 48, p["hidden"], "bf16")
    base = m.prefill_chunk(embeds=dev_from_storage(xs, "bf16"), n=48)
    st0 = m.state()
    runs = []
    for _ in range(2):
        _, ys = synth.embeddings(5, 1, 33, p["hidden"], "bf16")
        m.prefill_chunk(embeds=dev_from_storage(ys, "bf16"), n=33)
        toks = [m.decode_step(3)]
        for _ in range(5):
            toks.append(m.decode_step(toks[-1]))
        runs.append((logits_of(m), toks, m.state()))
        m.kv_rollback(base)
        assert m.state() == st0
    assert np.array_equal(runs[0][0], runs[1][0]) and runs[0][1] == runs[1][1]
    assert runs[0][2] == runs[1][2]
    m.close()


def test_profile_replay_leaves_results_unchanged():
    """Replaying the decode gate/up projection for timing changes no result: decodes
    after a replay give bit-identical logits and tokens to decodes without one; other
    classes and out-of-range repeat counts are refused."""
    p = TINY_BF16
    runs = []
    for replay in (False, True):
        m = _model(p, 0.08)
        _, xs = synth.embeddings(6, 0, 40, p["hidden"], "bf16")
        m.prefill_chunk(embeds=dev_from_storage(xs, "bf16"), n=40)
        toks = [m.decode_step(7)]
        if replay:
            ms = m.profile_replay("gemv_gateup", reps=3)
            assert ms > 0.0
            for bad in (("gemv_o", 3), ("gemv_gateup", 0), ("gemv_gateup", 1001)):
                with pytest.raises(vla.VlaError) as err:
                    m.profile_replay(bad[0], reps=bad[1])
                assert err.value.status == vla.VLA_E_INVALID
        for _ in range(4):
            toks.append(m.decode_step(toks[-1]))
        runs.append((logits_of(m), toks))
        m.close()
    assert np.array_equal(runs[0][0], runs[1][0]) and runs[0][1] == runs[1][1]


# ---------------------------------------------------------------------------
def test_bf16_long_context_split_attention():
    """A 1,920-token cached context (30 raw frames, 120 blocks) so that both the
    prefill and the decode attention split the keys over many workgroups and merge
    the partials; then a 200-token prefill and 6 greedy decodes."""
    p = dict(TINY_BF16, num_blocks=160, max_frames=40, max_chunk=200)
    init_std = 0.08
    ocfg = oracle_config(p, init_std=init_std)
    sess = D.Session(ocfg)
    m = _model(p, init_std)
    L, hkv, d = p["n_layers"], p["n_kv_heads"], p["head_dim"]
    for f in range(30):
        (k32, v32), (ks, vs) = synth.raw_kv_frame(11, f, L, 64, hkv, d, "bf16")
        fid = m.kv_append_raw(dev_from_storage(ks, "bf16"), dev_from_storage(vs, "bf16"), 64)
        assert fid == sess.append_raw(k32, v32)
    x32, xs = synth.embeddings(p["seed"], 0, 200, p["hidden"], "bf16")
    m.prefill_chunk(embeds=dev_from_storage(xs, "bf16"), n=200)
    _, ref = sess.prefill_chunk(embeds=x32)
    log("long ctx prefill cos %.6f rel %.2e" % metrics(logits_of(m), ref))
    check_logits(logits_of(m), ref, "bf16", "long-context prefill")
    tok = int(np.argmax(ref))
    for i in range(6):
        g = m.decode_step(tok)
        nxt, ref = sess.decode_step(tok)
        check_logits(logits_of(m), ref, "bf16", f"long-context decode {i}")
        check_argmax(g, ref, "bf16", f"long-context decode {i}")
        tok = nxt
    m.close()


def test_bf16_long_cache_prefill_shape():
    """More than 256 resident blocks (300 blocks of raw frames), then a 120-token chunk
    (360 query rows per KV head: the 64-row workgroups with many key splits) and a
    180-token chunk (540 rows: the long-cache shape, 256-row workgroups, 4-stage ring);
    each splits the keys and merges; then 3 greedy decodes."""
    p = dict(TINY_BF16, num_blocks=330, max_frames=80, max_chunk=180)
    init_std = 0.08
    ocfg = oracle_config(p, init_std=init_std)
    sess = D.Session(ocfg)
    m = _model(p, init_std)
    L, hkv, d = p["n_layers"], p["n_kv_heads"], p["head_dim"]
    for f in range(75):
        (k32, v32), (ks, vs) = synth.raw_kv_frame(12, f, L, 64, hkv, d, "bf16")
        fid = m.kv_append_raw(dev_from_storage(ks, "bf16"), dev_from_storage(vs, "bf16"), 64)
        assert fid == sess.append_raw(k32, v32)
    ref = None
    for call, n in enumerate((120, 180)):
        x32, xs = synth.embeddings(p["seed"], call, n, p["hidden"], "bf16")
        m.prefill_chunk(embeds=dev_from_storage(xs, "bf16"), n=n)
        _, ref = sess.prefill_chunk(embeds=x32)
        check_logits(logits_of(m), ref, "bf16", f"long-cache prefill {n}")
    tok = int(np.argmax(ref))
    for i in range(3):
        g = m.decode_step(tok)
        nxt, ref = sess.decode_step(tok)
        check_logits(logits_of(m), ref, "bf16", f"long-cache decode {i}")
        check_argmax(g, ref, "bf16", f"long-cache decode {i}")
        tok = nxt
    m.close()


def test_qwen_shape_one_layer_chunk_sizes():
    """One layer at the Qwen2.5-1.5B shape (hidden 1536, 12/2 heads, FFN 8960; a
    4,096-entry vocabulary): a 64-token chunk (the gated projection's 64 x 128 tiles,
    which it takes from 128 column tiles on, and the 64 x 32 split tiles of the other
    projections), a 256-token chunk (256 x 128 gated tiles of eight wavefronts, split
    q/k/v and residual projections) and 2 greedy decodes."""
    p = dict(vla.PRESETS["c2_qwen1p5b_bf16"], n_layers=1, vocab=4096, num_blocks=24,
             max_frames=4)
    init_std = 0.02
    sess = D.Session(oracle_config(p, init_std=init_std))
    m = _model(p, init_std)
    ref = None
    for call, n in enumerate((64, 256)):
        x32, xs = synth.embeddings(p["seed"], call, n, p["hidden"], "bf16")
        m.prefill_chunk(embeds=dev_from_storage(xs, "bf16"), n=n)
        _, ref = sess.prefill_chunk(embeds=x32)
        log("qwen-shape prefill %d cos %.6f rel %.2e" % ((n,) + metrics(logits_of(m), ref)))
        check_logits(logits_of(m), ref, "bf16", f"qwen-shape prefill {n}")
    tok = int(np.argmax(ref))
    for i in range(2):
        g = m.decode_step(tok)
        nxt, ref = sess.decode_step(tok)
        check_logits(logits_of(m), ref, "bf16", f"qwen-shape decode {i}")
        check_argmax(g, ref, "bf16", f"qwen-shape decode {i}")
        tok = nxt
    m.close()


def test_qwen_shape_two_layers_64_token_chunks():
    """Two layers at the Qwen2.5-1.5B shape, 64-token chunks: the gated projection
    (17,920 columns) and the down projection (K 8,960) of up to 64 rows take the
    two-stream kernel with 64-row tiles. With two layers every row's FFN output reaches
    the logits through layer 1's keys and values, so a wrong row of the 64 shows."""
    p = dict(vla.PRESETS["c2_qwen1p5b_bf16"], n_layers=2, vocab=4096, num_blocks=24,
             max_frames=4)
    init_std = 0.02
    sess = D.Session(oracle_config(p, init_std=init_std))
    m = _model(p, init_std)
    ref = None
    for call, n in enumerate((64, 37)):
        x32, xs = synth.embeddings(p["seed"], 10 + call, n, p["hidden"], "bf16")
        m.prefill_chunk(embeds=dev_from_storage(xs, "bf16"), n=n)
        _, ref = sess.prefill_chunk(embeds=x32)
        log("qwen-shape 2-layer prefill %d cos %.6f rel %.2e" % ((n,) + metrics(logits_of(m), ref)))
        check_logits(logits_of(m), ref, "bf16", f"qwen-shape 2-layer prefill {n}")
    tok = int(np.argmax(ref))
    g = m.decode_step(tok)
    _, ref = sess.decode_step(tok)
    check_logits(logits_of(m), ref, "bf16", "qwen-shape 2-layer decode")
    check_argmax(g, ref, "bf16", "qwen-shape 2-layer decode")
    m.close()


def test_device_resident_tokens_chain_like_host_tokens():
    """Greedy decoding with the token kept on the device (no host round trip, no
    synchronisation per step) gives bit-identical logits and the same cache as
    decoding with host tokens."""
    p = TINY_BF16
    x32, xs = synth.embeddings(p["seed"], 3, 50, p["hidden"], "bf16")
    a, b = _model(p, 0.08), _model(p, 0.08)
    for m in (a, b):
        m.prefill_chunk(embeds=dev_from_storage(xs, "bf16"), n=50)
    tok = int(np.argmax(logits_of(a)))
    for _ in range(20):
        tok = a.decode_step(tok)
        assert b.decode_step(vla.VLA_TOKEN_DEVICE, want_token=False) is None
    assert np.array_equal(logits_of(a), logits_of(b))
    assert a.state() == b.state()
    # the device token needs a previous forward
    c = _model(p, 0.08)
    with pytest.raises(vla.VlaError) as e:
        c.decode_step(vla.VLA_TOKEN_DEVICE)
    assert e.value.status == vla.VLA_E_STATE and c.state()["n_frames"] == 0
    for m in (a, b, c):
        m.close()


# ---------------------------------------------------------------------------
# properties of the GPU path
def test_mha_config_kv_heads_equal_heads():
    """Hkv = Hq (no grouping: one query row per KV head and token) against the oracle."""
    p = dict(TINY_BF16, n_heads=2, n_kv_heads=2, seed=91)
    ocfg = oracle_config(p, init_std=0.08)
    sess = D.Session(ocfg)
    m = _model(p, 0.08)
    x32, xs = synth.embeddings(p["seed"], 0, 70, p["hidden"], "bf16")
    m.prefill_chunk(embeds=dev_from_storage(xs, "bf16"), n=70)
    _, ref = sess.prefill_chunk(embeds=x32)
    check_logits(logits_of(m), ref, "bf16", "mha prefill")
    tok = int(np.argmax(ref))
    for i in range(5):
        g = m.decode_step(tok)
        nxt, ref = sess.decode_step(tok)
        check_logits(logits_of(m), ref, "bf16", f"mha decode {i}")
        check_argmax(g, ref, "bf16", f"mha decode {i}")
        tok = nxt
    m.close()


def test_physical_block_placement_is_invisible():
    """The same frames placed in other physical blocks (a free-list reordered by earlier
    frames, an eviction and a rollback) give bit-identical logits: every kernel reads the
    cache in logical order through the block table."""
    p = TINY_BF16
    fresh = _model(p, 0.08)
    moved = _model(p, 0.08)
    H = p["hidden"]
    # reorder moved's free-list: frames of various lengths, evict one, roll back
    junk = [synth.embeddings(77, i, n, H, "bf16")[1] for i, n in enumerate((33, 50, 17))]
    moved.prefill_chunk(embeds=dev_from_storage(junk[0], "bf16"), n=33)
    moved.prefill_chunk(embeds=dev_from_storage(junk[1], "bf16"), n=50)
    moved.prefill_chunk(embeds=dev_from_storage(junk[2], "bf16"), n=17)
    moved.kv_score_and_evict(0)
    moved.kv_rollback(-1)
    assert moved.state()["free_blocks"] == p["num_blocks"]
    chunks = [synth.embeddings(78, i, n, H, "bf16")[1] for i, n in enumerate((45, 20))]
    for m in (fresh, moved):
        for xs in chunks:
            m.prefill_chunk(embeds=dev_from_storage(xs, "bf16"), n=xs.shape[0])
    assert not np.array_equal(fresh.block_table()[0], moved.block_table()[0])
    assert np.array_equal(logits_of(fresh), logits_of(moved))
    t1 = fresh.decode_step(5)
    t2 = moved.decode_step(5)
    assert t1 == t2 and np.array_equal(logits_of(fresh), logits_of(moved))
    fresh.close()
    moved.close()


def test_chunking_changes_only_rounding():
    """One 96-token chunk, or the same tokens as 40 + 16 + 40: both match the oracle (which
    is exactly chunking-invariant) and each other within the bf16 tolerance."""
    p = dict(TINY_BF16, seed=92)
    ocfg = oracle_config(p, init_std=0.08)
    ids = synth.token_ids(p["seed"], 0, 96, p["vocab"])
    one, three = _model(p, 0.08), _model(p, 0.08)
    one.prefill_chunk(tokens=ids)
    for a, b in ((0, 40), (40, 56), (56, 96)):
        three.prefill_chunk(tokens=ids[a:b])
    _, ref = D.Session(ocfg).prefill_chunk(tokens=ids)
    check_logits(logits_of(one), ref, "bf16", "one chunk")
    check_logits(logits_of(three), ref, "bf16", "three chunks")
    check_logits(logits_of(three), logits_of(one), "bf16", "three vs one")
    one.close()
    three.close()

"""Eviction policies ("Can an LLM Forget the Right Things?", section 5) through the C ABI,
against the oracle: FIFO, the page's adjacent-pair rule and the all-pairs scoring, one
eviction at a time and through the evict-until-room loop with and without a frame window.

Raw frames carry the very same stored keys on both sides, so the mean keys are
bit-identical and every pick must agree; free-list and block table are compared after
every eviction.
"""
import numpy as np
import pytest

import kv_cached_gqa_decoder_amd as vla
import synth
from oracle import decoder as D
from tests.gpu_util import dev_from_storage, oracle_config
from tests.test_gpu_parity import TINY_BF16

pytestmark = pytest.mark.gpu


def _pair(nframes=12, num_blocks=64, max_frames=12, seed=7, clusters=5):
    p = dict(TINY_BF16, num_blocks=num_blocks, max_frames=max_frames)
    sess = D.Session(oracle_config(p))
    m = vla.Model(vla.make_config(**p))
    L, hkv, d = p["n_layers"], p["n_kv_heads"], p["head_dim"]
    for f in range(nframes):
        n = 64 if f % 3 else 40
        (k32, v32), (ks, vs) = synth.clustered_frame(seed, f, L, n, hkv, d, n_clusters=clusters)
        fid = m.kv_append_raw(dev_from_storage(ks, "bf16"), dev_from_storage(vs, "bf16"), n)
        assert fid == sess.append_raw(k32, v32)
    return p, m, sess


def _same_tables(m, sess, what):
    blocks, ntok = m.block_table()
    assert [(int(b), int(n)) for b, n in zip(blocks, ntok)] == sess.block_table(), what
    assert m.free_list() == sess.pool.free, what
    assert list(m.frames()) == [s.frame_id for s in sess.frames()], what


def test_single_evictions_by_policy():
    p, m, sess = _pair()
    seq = ["adjacent", "fifo", "semantic", "adjacent", "adjacent", "fifo", "semantic", "adjacent"]
    for i, policy in enumerate(seq):
        gfid, gscore = m.kv_evict(policy, 0)
        ofid, oscore = sess.pick(policy, 0)
        sess.evict(ofid)
        assert gfid == ofid, (i, policy, gfid, ofid)
        assert abs(gscore - oscore) <= 1e-12, (i, policy, gscore, oscore)
        _same_tables(m, sess, f"step {i} {policy}")
    # the adjacent rule's score is the all-pairs value of the same pair
    a_fid, a_score = sess.pick("adjacent", 1)
    frames = [s.frame_id for s in sess.frames()]
    j = frames.index(a_fid)
    mk = m.mean_keys(1)[: len(frames)]
    from oracle.scoring import cosine
    assert abs(cosine(mk[j], mk[j + 1]) - a_score) <= 1e-12
    m.close()


def test_make_room_loops_and_windows():
    p, m, sess = _pair(nframes=12, num_blocks=44)
    assert m.state()["free_blocks"] == sess.pool.free.__len__()
    # 64 tokens need 4 blocks: FIFO evicts the oldest frames until they are free
    n = m.kv_make_room("fifo", 64)
    assert n == len(sess.make_room("fifo", 64))
    _same_tables(m, sess, "fifo make_room")
    # a window of 6 frames: evict until fewer than 6 remain, the scoring policies
    for policy, window in (("semantic", 8), ("adjacent", 6)):
        n = m.kv_make_room(policy, 16, window=window)
        assert n == len(sess.make_room(policy, 16, window=window)), policy
        _same_tables(m, sess, f"{policy} window {window}")
    # nothing to do: no eviction
    assert m.kv_make_room("semantic", 16) == 0
    # one frame left: every policy takes it
    while len(sess.frames()) > 1:
        fid, _ = m.kv_evict("fifo")
        sess.evict(fid)
    st = m.state()
    n = m.kv_make_room("semantic", 16, window=1)
    assert n == len(sess.make_room("semantic", 16, window=1)) == 1
    _same_tables(m, sess, "last frame")
    assert m.state()["n_frames"] == 0 and st["n_frames"] == 1
    m.close()


def test_policy_errors_leave_state_unchanged():
    p, m, sess = _pair(nframes=3, num_blocks=16)
    st = m.state()
    for args, status in (((7, 16), vla.VLA_E_INVALID),                 # unknown policy
                         (("fifo", 0), vla.VLA_E_INVALID),             # n_tokens < 1
                         (("fifo", p["max_chunk"] + 1), vla.VLA_E_INVALID)):
        with pytest.raises(vla.VlaError) as e:
            m.kv_make_room(*args)
        assert e.value.status == status and m.state() == st
    with pytest.raises(vla.VlaError) as e:
        m.kv_make_room("fifo", 16, window=-1)
    assert e.value.status == vla.VLA_E_INVALID and m.state() == st
    with pytest.raises(vla.VlaError) as e:
        m.kv_evict("fifo", layer=p["n_layers"])
    assert e.value.status == vla.VLA_E_INVALID and m.state() == st
    # a frame bigger than the whole pool: refused before anything is evicted
    big = dict(TINY_BF16, num_blocks=4, max_frames=4, max_chunk=160)
    mb = vla.Model(vla.make_config(**big))
    _, (ks, vs) = synth.clustered_frame(7, 0, big["n_layers"], 40, 2, 128)
    mb.kv_append_raw(dev_from_storage(ks, "bf16"), dev_from_storage(vs, "bf16"), 40)
    stb = mb.state()
    with pytest.raises(vla.VlaError) as e:
        mb.kv_make_room("fifo", 80)
    assert e.value.status == vla.VLA_E_NO_BLOCKS and mb.state() == stb
    # no frames: nothing to evict
    mb.kv_evict("fifo")
    with pytest.raises(vla.VlaError) as e:
        mb.kv_evict("fifo")
    assert e.value.status == vla.VLA_E_NOTHING_TO_EVICT
    mb.close()
    m.close()

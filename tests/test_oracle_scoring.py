"""Pins of the oracle's redundancy scoring, LIFO pool and eviction bookkeeping."""
import json
import os

import numpy as np
import pytest
from scipy.spatial.distance import cdist

from oracle import decoder as D
from oracle import scoring as S
from oracle.kvpool import BlockPool, NoBlocks, NothingToEvict

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAGES = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))


def test_cosine_special_values_and_guard():
    g = np.random.default_rng(0)
    a = g.standard_normal(256)
    assert S.cosine(a, a) == pytest.approx(1.0, abs=1e-15)
    assert S.cosine(a, -a) == pytest.approx(-1.0, abs=1e-15)
    assert S.cosine(a, np.zeros(256)) == 0.0
    e0, e1 = np.eye(256)[0], np.eye(256)[1]
    assert S.cosine(e0, e1) == 0.0
    # below the page's 1e-8 denominator threshold the result is 0
    thr = PAGES["p1_cosine_guard"]["den_threshold"]
    tiny = np.full(4, 1e-5)        # |a| |b| = 4e-10 < 1e-8
    assert S.cosine(tiny, tiny) == 0.0
    big = np.full(4, 1e-4)         # 4e-8 >= 1e-8
    assert 4e-8 >= thr and S.cosine(big, big) == pytest.approx(1.0)


def test_cosine_matches_scipy():
    g = np.random.default_rng(1)
    x = g.standard_normal((20, 256))
    ref = 1.0 - cdist(x, x, metric="cosine")
    for i in range(20):
        for j in range(20):
            assert S.cosine(x[i], x[j]) == pytest.approx(ref[i, j], abs=1e-14)


def test_pair_matrix_symmetric_and_brute_force_winner():
    g = np.random.default_rng(2)
    for trial in range(20):
        f = int(g.integers(2, 40))
        x = g.standard_normal((f, 32))
        win, score, m = S.pick_redundant(x)
        s = S.pair_matrix(x)
        assert np.array_equal(s, s.T)
        # brute force: best unordered pair by normalised Gram matrix, older of the pair
        xn = x / np.linalg.norm(x, axis=1, keepdims=True)
        gram = xn @ xn.T
        np.fill_diagonal(gram, -np.inf)
        i, j = np.unravel_index(np.argmax(gram), gram.shape)
        assert win == min(i, j)
        assert score == pytest.approx(gram[i, j], abs=1e-13)


def test_planted_duplicate_pair_and_tie_rule():
    g = np.random.default_rng(3)
    x = g.standard_normal((10, 64))
    x[7] = x[3] * 2.5           # cos(3, 7) = 1 exactly in real arithmetic
    win, score, _ = S.pick_redundant(x)
    assert win == 3 and score == pytest.approx(1.0, abs=1e-15)
    # two identical pairs: the lowest index wins
    x[8] = x[1]
    win, _, _ = S.pick_redundant(x)
    assert win == 1


def test_adjacent_pair_rule_of_the_page():
    x = np.array([[1, 0], [0, 1], [0, 1.0001], [1, 0.1], [1, 0.1]], dtype=float)
    # pairs (1,2) and (3,4) are the most similar neighbours; (3,4) has cos 1, older = 3
    assert S.adjacent_pair_pick(x) == 3
    x[4] = [0.2, 1]
    assert S.adjacent_pair_pick(x) == 1


def test_mean_key_of_bf16_values_is_exact_in_fp64():
    # sums of bf16-valued keys are exact in fp64, so the order of summation cannot matter
    g = np.random.default_rng(4)
    from synth import encode
    k32, _ = encode(g.standard_normal((64, 2, 128)).astype(np.float32), "bf16")
    k = k32.astype(np.float64)
    a = S.mean_key(k)
    b = S.mean_key(k[::-1])
    c = np.zeros(256)
    for t in g.permutation(64):
        c += k[t].reshape(-1)
    assert np.array_equal(a, b) and np.array_equal(a, c / 64)


def test_lifo_pool_order_from_the_page():
    p = PAGES["kshipra_lifo"]
    pool = BlockPool(p["num_blocks"])
    assert pool.alloc(3) == p["first_pops"]
    pool.release([6])
    assert pool.alloc(1) == [6]        # the freed block is reused next
    with pytest.raises(NoBlocks):
        pool.alloc(10)


def _tiny_eviction_session():
    cfg = D.Config("t3", n_layers=2, hidden=32, n_heads=4, n_kv_heads=2, head_dim=8, ffn=48,
                   vocab=64, num_blocks=24, max_frames=6, seed=5, wdtype="f32", act="f32")
    return cfg, D.Session(cfg)


def test_eviction_pushes_blocks_in_logical_order_and_pops_reverse():
    cfg, s = _tiny_eviction_session()
    from synth import clustered_frame
    for f in range(6):
        (k, v), _ = clustered_frame(9, f, cfg.n_layers, 64, cfg.n_kv_heads, cfg.head_dim,
                                    n_clusters=4, storage="f32")
        s.append_raw(k, v)
    fid, _ = s.score(0)[:2]
    blocks = [seg.blocks for seg in s.frames() if seg.frame_id == fid][0]
    s.evict(fid)
    got = s.pool.alloc(len(blocks))
    assert got == list(reversed(blocks))


def test_clustered_frames_evict_a_cluster_member_and_refuse_below_two():
    cfg, s = _tiny_eviction_session()
    from synth import clustered_frame
    for f in range(6):
        (k, v), _ = clustered_frame(9, f, cfg.n_layers, 16, cfg.n_kv_heads, cfg.head_dim,
                                    n_clusters=4, storage="f32")
        s.append_raw(k, v)
    # frames 0/4 and 1/5 share clusters: the first eviction is the older of the closer pair
    fid, score = s.score_and_evict(0)
    assert fid in (0, 1) and score > 0.9
    fid2, _ = s.score_and_evict(0)
    assert fid2 in (0, 1) and fid2 != fid
    while len(s.frames()) > 1:
        s.score_and_evict(0)
    with pytest.raises(NothingToEvict):
        s.score_and_evict(0)


def test_rollback_restores_free_list_and_counters():
    cfg, s = _tiny_eviction_session()
    g = np.random.default_rng(6)
    s.prefill_chunk(embeds=g.standard_normal((20, cfg.hidden)))
    snap = (list(s.pool.free), s.next_pos, s.next_frame_id)
    ref = s.prefill_chunk(embeds=g.standard_normal((5, cfg.hidden)))[1]
    for t in (1, 2, 3):
        s.decode_step(t)
    s.rollback(0)
    assert (list(s.pool.free), s.next_pos, s.next_frame_id) == snap
    x = np.random.default_rng(6).standard_normal((20, cfg.hidden))   # same draws again
    again = s.prefill_chunk(embeds=np.random.default_rng(6).standard_normal((25, cfg.hidden))[20:])
    assert np.array_equal(again[1], ref) and x.shape == (20, cfg.hidden)

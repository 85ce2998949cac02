"""Pins of the INT4 codec and of the pages' closed-form sizes."""
import json
import os

import numpy as np

from oracle import decoder as D
from oracle import int4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAGES = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))


def _w(n=64, k=512, seed=0):
    g = np.random.default_rng(seed)
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[3, :128] = 0.0                      # an all-zero group: s = 0, q = 0
    w[5, 128:256] *= 1e-3                 # a group with a tiny scale
    return w


def test_int4_error_bound_half_step():
    w = _w()
    packed, s16, w_hat = int4.quantize_g128(w)
    s = np.repeat(s16.astype(np.float32), 128, axis=1)
    assert np.all(np.abs(w.astype(np.float64) - w_hat) <= s.astype(np.float64) / 2 + 0.0)
    assert np.all(w_hat[3, :128] == 0)


def test_int4_bits_per_weight_and_fraction_of_fp16():
    p = PAGES["kshipra_int4"]
    assert int4.bits_per_weight(4096) == p["bits_per_weight"]
    assert abs(int4.bits_per_weight(4096) / 16 - p["fraction_of_fp16_approx"]) < 0.005
    packed, s16, _ = int4.quantize_g128(_w(8, 4096))
    assert (packed.nbytes * 8 + s16.nbytes * 8) / (8 * 4096) == p["bits_per_weight"]


def test_int4_pack_roundtrip_and_idempotence():
    w = _w()
    packed, s16, w_hat = int4.quantize_g128(w)
    assert np.array_equal(int4.dequantize_g128(packed, s16), w_hat)
    p2, s2, w_hat2 = int4.quantize_g128(w_hat)
    assert np.array_equal(s2, s16) and np.array_equal(w_hat2, w_hat) and np.array_equal(p2, packed)


def test_int4_even_k_in_low_nibble():
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, 0], w[0, 1] = 7.0, -7.0          # s = 1: q0 = 7 (0x7), q1 = -7 (0x9)
    packed, s16, _ = int4.quantize_g128(w)
    assert float(s16[0, 0]) == 1.0 and packed[0, 0] == 0x97


def test_int4_scale_bug_of_the_page_is_avoided():
    # encoding with the fp32 scale and decoding with its fp16 rounding breaks the bound
    g = np.random.default_rng(7)
    w = (g.standard_normal((256, 128)) * 0.02).astype(np.float32)
    amax = np.abs(w).max(axis=1, keepdims=True)
    s32 = amax / np.float32(7.0)
    s16 = s32.astype(np.float16).astype(np.float32)
    q_bad = np.clip(np.rint(w / s32), -8, 7)
    err_bad = np.abs(w - q_bad * s16) - s16 / 2
    _, _, w_hat = int4.quantize_g128(w)
    err_ok = np.abs(w - w_hat) - np.repeat(s16, 128, axis=1) / 2
    assert err_bad.max() > 0 and err_ok.max() <= 0


def test_kv_sizes_from_the_pages():
    k = PAGES["kshipra_gqa_sizing"]
    assert D.kv_bytes_per_token(D.C5, 2) == k["kib_per_token"] * 1024
    assert D.kv_bytes_per_token(D.C5.with_(n_kv_heads=32), 2) == k["kib_per_token_mha"] * 1024
    assert D.kv_bytes_per_token(D.C5, 2) * k["tokens"] == k["mib_at_tokens"] * 2 ** 20
    assert D.kv_bytes_per_token(D.C5.with_(n_kv_heads=32), 2) * k["tokens"] == \
        k["gib_at_tokens_mha"] * 2 ** 30
    p1 = PAGES["p1_kv_cache"]
    total = p1["slots"] * D.kv_bytes_per_token(D.C2, 4)      # the page's cache is fp32
    assert total == 234_881_024 and round(total / 1e6) == p1["approx_mb"]
    assert D.kv_bytes_per_token(D.C2, 2) == 28 * 1024
    f = PAGES["p1_slots_per_frame"]
    assert f["max_tokens"] // f["slots_per_frame"] == f["max_frames"]

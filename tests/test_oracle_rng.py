"""Pins of the oracle's seeded generator (splitmix64 -> Box-Muller) and of its rounding."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_sequence():
    # state k*gamma is the state before the (k+1)-th output of the reference generator
    vals = json.load(open(os.path.join(GOLDEN, "splitmix64.json")))["seed0_outputs"]
    gamma = np.uint64(0x9E3779B97F4A7C15)
    with np.errstate(over="ignore"):
        got = [int(rng.splitmix64(np.uint64(k) * gamma)) for k in range(len(vals))]
    assert got == [int(v, 16) for v in vals]


def test_box_muller_closed_form_for_chosen_uniforms():
    # with u1 = 1 - e^-2 and u2 = 0 the transform gives sqrt(-2 ln e^-2) * cos(0) = 2
    u1, u2 = 1.0 - math.exp(-2.0), 0.0
    assert math.isclose(math.sqrt(-2.0 * math.log(1.0 - u1)) * math.cos(2 * math.pi * u2), 2.0,
                        rel_tol=1e-12)
    # and the vectorised stream uses exactly the two splitmix outputs 2i, 2i+1 of its key
    key = rng.stream_key(7, 99)
    i = 5
    with np.errstate(over="ignore"):
        a = int(rng.splitmix64(key + np.uint64(2 * i)))
        b = int(rng.splitmix64(key + np.uint64(2 * i + 1)))
    ua, ub = (a >> 11) * 2.0 ** -53, (b >> 11) * 2.0 ** -53
    ref = math.sqrt(-2.0 * math.log(1.0 - ua)) * math.cos(2 * math.pi * ub)
    assert rng.normal_np(7, 99, i, 1)[0] == pytest.approx(ref, rel=1e-14)


def test_normal_distribution_moments():
    z = rng.normal_np(1234, 3, 0, 400_000)
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2.0 / n)
    # fraction within one sigma of a standard normal: erf(1/sqrt 2) = 0.682689...
    p = math.erf(1 / math.sqrt(2))
    frac = np.mean(np.abs(z) < 1.0)
    assert abs(frac - p) < 5 * math.sqrt(p * (1 - p) / n)
    # fourth moment 3 (kurtosis of a Gaussian)
    assert abs(np.mean(z ** 4) - 3.0) < 0.05


def test_streams_are_distinct_and_counter_based():
    a = rng.normal_np(1234, rng.layer_stream(0, rng.KIND_Q), 0, 1000)
    b = rng.normal_np(1234, rng.layer_stream(0, rng.KIND_K), 0, 1000)
    assert np.corrcoef(a, b)[0, 1] < 0.15
    # element i does not depend on where the draw starts
    full = rng.normal_np(1234, 42, 0, 100)
    part = rng.normal_np(1234, 42, 37, 20)
    assert np.array_equal(full[37:57], part)


def test_uniform_ids_uniformity():
    v = 16
    ids = rng.uniform_ids(1234, 0x10000, 160_000, v)
    assert ids.min() >= 0 and ids.max() < v
    counts = np.bincount(ids, minlength=v)
    e = ids.size / v
    chi2 = float(((counts - e) ** 2 / e).sum())
    assert chi2 < 45.0      # 15 dof, p ~ 1e-4


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x32 = (g.standard_normal(200_000) * np.exp(g.uniform(-20, 20, 200_000))).astype(np.float32)
    # include exact ties: values halfway between two bf16 numbers
    # (normal range: exponent fields 0x40 .. 0xBF, both signs)
    hi = np.concatenate([np.arange(0x2000, 0x5F80, 7), np.arange(0xA000, 0xDF80, 7)]).astype(np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    x32 = np.concatenate([x32, ties])
    ours = rng.round_bf16(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_f32_storage_is_ieee_nearest():
    x = rng.normal_np(3, 4, 0, 10000)
    assert np.array_equal(rng.round_storage(x, "f32"), x.astype(np.float32).astype(np.float64))


def test_c_twin_matches_numpy(oracle_c_built):
    for storage in ("bf16", "f32"):
        a = rng.round_storage(0.02 * rng.normal_np(1236, 513, 1000, 50_000), storage)
        b = rng.normal_c(1236, 513, 1000, 50_000, 0.02, storage)
        assert np.array_equal(a, b), storage
    a = rng.normal_np(1236, 513, 0, 50_000)
    b = rng.normal_c(1236, 513, 0, 50_000, 1.0, "f64")
    assert np.max(np.abs(a - b) / np.maximum(np.abs(a), 1e-300)) < 1e-15


def test_generator_pins_computed_independently(oracle_c_built):
    """sm(0), sm(1), a stream key, the first normals and uniform ids of one stream,
    as computed from the generator's definition by a separate implementation."""
    pins = json.load(open(os.path.join(GOLDEN, "generator_pins.json")))
    for x, want in pins["sm"].items():
        assert int(rng.splitmix64(np.uint64(int(x)))) == int(want, 16), x
    k = pins["key"]
    assert int(rng.stream_key(k["seed"], k["stream"])) == int(k["value"], 16)
    nrm = pins["normal"]
    got = rng.normal_np(nrm["seed"], nrm["stream"], 0, len(nrm["first"]))
    assert got.tolist() == nrm["first"]
    # the C twin gives the same doubles (std 1, fp64 storage)
    got_c = rng.normal_c(nrm["seed"], nrm["stream"], 0, len(nrm["first"]), 1.0, "f64")
    assert np.max(np.abs(got_c - np.array(nrm["first"]))) <= 1e-15
    u = pins["uniform_ids"]
    assert rng.uniform_ids(u["seed"], u["stream"], len(u["first"]), u["vocab"]).tolist() == u["first"]

"""CPU checks of the C-ABI library: it loads, exports every declared entry point,
and its host-only LIFO pool behaves like the oracle's (no GPU calls here)."""
import os
import re
import subprocess

import numpy as np
import pytest

from oracle.kvpool import BlockPool

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "kv_cached_gqa_decoder_amd", "libvla.so")
HDR = os.path.join(ROOT, "include", "vla.h")


@pytest.fixture(scope="module")
def vla():
    if not os.path.exists(LIB):
        from kv_cached_gqa_decoder_amd import build
        build.build()
    import kv_cached_gqa_decoder_amd as k
    k.load()
    return k


def declared_symbols():
    txt = open(HDR).read()
    return sorted(set(re.findall(r"\b(vla_[a-z_0-9]+)\(", txt)))


def test_library_exports_every_declared_symbol(vla):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [s for s in declared_symbols() if s not in exported]
    assert not missing, missing
    lib = vla.load()
    for s in declared_symbols():
        assert hasattr(lib, s)
    assert len(declared_symbols()) >= 20


def test_binding_names_match_the_header(vla):
    for s in declared_symbols():
        assert hasattr(vla, s), s


def test_host_pool_matches_oracle_lifo(vla):
    g = np.random.default_rng(0)
    p = vla.vla_pool_create(32)
    ref = BlockPool(32)
    held = []
    try:
        for _ in range(300):
            if held and g.random() < 0.45:
                k = int(g.integers(1, len(held) + 1))
                idx = g.choice(len(held), size=k, replace=False)
                rel = [held[i] for i in idx]
                held = [h for i, h in enumerate(held) if i not in set(idx.tolist())]
                vla.vla_pool_release(p, rel)
                ref.release(rel)
            else:
                k = int(g.integers(0, 6))
                if k > len(ref.free):
                    with pytest.raises(vla.VlaError) as e:
                        vla.vla_pool_alloc(p, k)
                    assert e.value.status == vla.VLA_E_NO_BLOCKS
                    continue
                got = vla.vla_pool_alloc(p, k)
                assert got == ref.alloc(k)
                held += got
            assert vla.vla_pool_free_count(p) == len(ref.free)
            assert vla.vla_pool_free_list(p) == ref.free
    finally:
        vla.vla_pool_destroy(p)


def test_host_pool_rejects_double_free_and_bad_ids(vla):
    p = vla.vla_pool_create(4)
    try:
        a = vla.vla_pool_alloc(p, 2)
        assert a == [3, 2]
        for bad in ([3, 3], [7], [-1], [1]):
            with pytest.raises(vla.VlaError) as e:
                vla.vla_pool_release(p, bad)
            assert e.value.status == vla.VLA_E_INVALID
        assert vla.vla_pool_free_count(p) == 2
        vla.vla_pool_release(p, a)
        assert vla.vla_pool_alloc(p, 2) == [2, 3]
    finally:
        vla.vla_pool_destroy(p)


def test_config_presets_match_the_oracle_shapes(vla):
    from oracle import decoder as D
    from oracle import pi0
    configs = dict(D.CONFIGS, **{c.name: c for c in (pi0.C4_VLM, pi0.C4_AE)})
    for name, p in vla.PRESETS.items():
        c = configs[name]
        assert (p.get("ffn_kind", vla.VLA_SWIGLU) == vla.VLA_GEGLU) == (c.ffn_kind == "geglu")
        assert bool(p.get("kv_only_last", 0)) == c.kv_only_last
        assert p.get("stream_base", 0) == c.stream_base
        assert (p["n_layers"], p["hidden"], p["n_heads"], p["n_kv_heads"], p["head_dim"],
                p["ffn"], p["vocab"], p["num_blocks"], p["max_frames"], p["seed"]) == \
            (c.n_layers, c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, c.vocab,
             c.num_blocks, c.max_frames, c.seed)
        assert p["rope_theta"] == c.rope_theta

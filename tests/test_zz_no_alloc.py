"""The scoring entry point that allocates nothing, against the model's own scoring.

vla_kv_score_noalloc keeps its per-frame scores in a library-owned static device
array; given a model's mean-key table it must pick the same frame with the same
score as vla_kv_score on that model, call after call, also when a later call is
smaller than an earlier one.
"""
import numpy as np
import pytest
import torch

import kv_cached_gqa_decoder_amd as vla
import synth
from tests.gpu_util import dev_from_storage, log
from tests.test_gpu_parity import TINY_BF16

pytestmark = pytest.mark.gpu


def _noalloc(mk: np.ndarray):
    st = torch.cuda.current_stream()
    tab = torch.from_numpy(np.ascontiguousarray(mk, dtype=np.float64)).cuda()
    idx = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    sc = torch.full((1,), np.nan, dtype=torch.float64, device="cuda")
    vla.vla_kv_score_noalloc(tab, mk.shape[0], mk.shape[1], idx, sc, st)
    st.synchronize()
    return int(idx.item()), float(sc.item())


def test_noalloc_scoring_equals_model_scoring_call_after_call():
    p = dict(TINY_BF16, num_blocks=64, max_frames=12)
    m = vla.Model(vla.make_config(**p))
    L, hkv, d = p["n_layers"], p["n_kv_heads"], p["head_dim"]
    D = hkv * d
    for f in range(12):
        n = 64 if f % 3 else 40
        _, (ks, vs) = synth.clustered_frame(7, f, L, n, hkv, d, n_clusters=5)
        m.kv_append_raw(dev_from_storage(ks, "bf16"), dev_from_storage(vs, "bf16"), n)
    for evictions in (0, 5, 4):          # 12 frames, then 7, then 3
        for _ in range(evictions):
            m.kv_score_and_evict(0)
        frames = list(m.frames())
        for layer in (0, 1):
            fid, score = m.kv_score(layer)
            mk = m.mean_keys(layer)[: len(frames)]
            idx, sc = _noalloc(mk)
            log(f"  {len(frames)} frames, layer {layer}: frame {frames[idx]} score {sc!r}")
            assert frames[idx] == fid and sc == score
    m.close()


def test_noalloc_scoring_rejects_bad_sizes():
    tab = torch.zeros((4097, 8), dtype=torch.float64, device="cuda")
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    sc = torch.zeros(1, dtype=torch.float64, device="cuda")
    with pytest.raises(vla.VlaError) as e:
        vla.vla_kv_score_noalloc(tab, 4097, 8, idx, sc)
    assert e.value.status == vla.VLA_E_INVALID and "maximum" in str(e.value)
    with pytest.raises(vla.VlaError) as e:
        vla.vla_kv_score_noalloc(tab, 1, 8, idx, sc)
    assert e.value.status == vla.VLA_E_NOTHING_TO_EVICT
    with pytest.raises(vla.VlaError) as e:
        vla.vla_kv_score_noalloc(tab, 4, 0, idx, sc)
    assert e.value.status == vla.VLA_E_INVALID
    # a valid call after the refusals still works: two identical rows are the pair
    t = torch.zeros((3, 8), dtype=torch.float64)
    t[0, 0] = 1.0
    t[1, 1] = 1.0
    t[2, 1] = 2.0
    assert _noalloc(t.numpy()) == (1, 1.0)

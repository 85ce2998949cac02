"""Reconciliation on a second state ("CSR: Infinite-Horizon Real-Time Policies with
Massive Cached State Representations", section III-E and Appendix D), through the C ABI.

After evictions the spare (a sibling model) re-prefills the kept frames from their
logged inputs at contiguous positions, catches up on frames that arrive meanwhile,
and takes over. Once swapped, the serving state must equal, bit for bit, a fresh
model that prefilled the same frames in arrival order (same weights, same kernels,
same chunks), and must match the oracle's fresh session within the bf16 tolerance.
"""
import numpy as np
import pytest
import torch

import kv_cached_gqa_decoder_amd as vla
import synth
from oracle import decoder as D
from tests.gpu_util import check_logits, dev_from_storage, oracle_config
from tests.test_gpu_parity import TINY_BF16

pytestmark = pytest.mark.gpu

P = dict(TINY_BF16, num_blocks=48, max_frames=10, max_chunk=64)
LENS = [40, 24, 33, 17, 40, 29, 12, 21, 9]


def _logits(h, vocab):
    out = np.zeros(vocab, dtype=np.float32)
    vla.vla_logits_out(h, out, vocab)
    return out


def _swap(rec, stream):
    for _ in range(100):
        if rec.try_swap(stream):
            return True
        rec.sync()
    return False


def test_reconciled_state_equals_a_fresh_prefill_of_the_kept_frames():
    stream = torch.cuda.current_stream()
    m = vla.Model(vla.make_config(**P, init_std=0.08))
    rec = vla.Reconciler(m)
    ids = [synth.token_ids(P["seed"], i, n, P["vocab"]) for i, n in enumerate(LENS)]
    for i in range(6):
        assert rec.prefill(tokens=ids[i], stream=stream) == i
    # two evictions on the serving model, then the spare starts re-prefilling
    evicted = [rec.evict("semantic", 0, stream)[0], rec.evict("fifo", 0, stream)[0]]
    serving0 = rec.model_handle()
    rec.begin(stream)
    assert rec.stats()["reconciling"]
    # frames keep arriving and leaving while the spare warms up
    assert rec.prefill(tokens=ids[6], stream=stream) == 6
    evicted.append(rec.evict("fifo", 0, stream)[0])
    assert rec.prefill(tokens=ids[7], stream=stream) == 7
    assert rec.model_handle() == serving0          # the old state serves until the swap
    assert _swap(rec, stream)
    assert rec.model_handle() != serving0
    kept = rec.frames()
    assert kept == [i for i in range(8) if i not in evicted]
    # one more frame through the new serving state, and its logits
    assert rec.prefill(tokens=ids[8], stream=stream) == 8
    torch.cuda.synchronize()
    got = _logits(rec.model_handle(), P["vocab"])
    st = vla.vla_get_state(rec.model_handle())
    assert st["next_position"] == sum(LENS[i] for i in kept) + LENS[8]
    assert st["n_frames"] == len(kept) + 1
    # a fresh model over the same frames, in the same order
    ref = vla.Model(vla.make_config(**P, init_std=0.08))
    for i in kept + [8]:
        ref.prefill_chunk(tokens=ids[i])
    assert np.array_equal(got, _logits(ref.h, P["vocab"]))
    # and the oracle's fresh session
    sess = D.Session(oracle_config(P, "asr", init_std=0.08))
    for i in kept + [8]:
        _, lg = sess.prefill_chunk(tokens=ids[i])
    check_logits(got.astype(np.float64), lg, "bf16", "reconciled state vs oracle")
    s = rec.stats()
    assert s["swaps"] == 1 and s["reconciliations"] == 1 and not s["reconciling"]
    ref.close()
    rec.close()
    m.close()


def test_two_rounds_with_embeddings_input():
    """Frames given as device embeddings (logged on the device); two reconciliations, so
    the caller's own model serves again after the second swap."""
    stream = torch.cuda.current_stream()
    m = vla.Model(vla.make_config(**P, init_std=0.08))
    rec = vla.Reconciler(m)
    embs = []
    for i, n in enumerate(LENS[:6]):
        _, xs = synth.embeddings(P["seed"], i, n, P["hidden"], "bf16")
        embs.append(dev_from_storage(xs, "bf16"))
        rec.prefill(embeds=embs[-1], n=n, stream=stream)
    rec.evict("adjacent", 0, stream)
    rec.begin(stream)
    assert _swap(rec, stream)
    rec.evict("semantic", 0, stream)
    rec.begin(stream)
    assert _swap(rec, stream)
    assert rec.model_handle() == m.h
    torch.cuda.synchronize()
    kept = rec.frames()
    assert len(kept) == 4
    ref = vla.Model(vla.make_config(**P, init_std=0.08))
    for i in kept:
        ref.prefill_chunk(embeds=embs[i], n=LENS[i])
    assert np.array_equal(_logits(m.h, P["vocab"]), _logits(ref.h, P["vocab"]))
    ref.close()
    rec.close()
    m.close()


def test_reconciler_checks_its_state():
    stream = torch.cuda.current_stream()
    m = vla.Model(vla.make_config(**P, init_std=0.08))
    m.prefill_chunk(tokens=synth.token_ids(P["seed"], 0, 8, P["vocab"]))
    with pytest.raises(vla.VlaError) as err:
        vla.Reconciler(m)                               # inputs of resident frames unknown
    assert err.value.status == vla.VLA_E_STATE
    m.kv_rollback(-1)
    rec = vla.Reconciler(m)
    with pytest.raises(vla.VlaError) as err:
        rec.try_swap(stream)                            # nothing running
    assert err.value.status == vla.VLA_E_STATE
    rec.prefill(tokens=synth.token_ids(P["seed"], 1, 8, P["vocab"]), stream=stream)
    rec.begin(stream)
    with pytest.raises(vla.VlaError) as err:
        rec.begin(stream)                               # one at a time
    assert err.value.status == vla.VLA_E_STATE
    assert _swap(rec, stream)
    rec.close()
    m.close()

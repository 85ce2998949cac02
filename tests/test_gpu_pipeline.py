"""Models over shared weights, and the overlapped prefix / expert streams
("Running VLAs at Real-time Speed", section 6.1), through the C ABI.

A sibling model runs the same kernels on the same weights, so its results are
bit-identical to the source model's, and the weights outlive whichever model is
destroyed first. The pipeline's action runs must equal, bit for bit, a
sequential (prefix model, expert) pair that prefilled the frame the pipeline
reports it used; the frame may be the newest one or the one before it,
depending on which prefill had finished when the run was submitted. The
pipeline replays its action loop from a captured graph; the runs that reuse one
buffer check every replay, with eager copies between them.
"""
import numpy as np
import pytest
import torch

import kv_cached_gqa_decoder_amd as vla
import synth
from tests.gpu_util import dev_from_storage, logits_of
from tests.test_gpu_parity import TINY_BF16
from tests.test_gpu_pi0 import TINY_AE, TINY_VLM

pytestmark = pytest.mark.gpu

N_PREFIX, N_ACT, STEPS, DT = 40, 19, 4, 0.25


def test_sibling_model_is_bit_identical_and_outlives_its_source():
    p = dict(TINY_BF16, max_chunk=64)
    a = vla.Model(vla.make_config(**p, init_std=0.08))
    b = a.sibling()
    ids = synth.token_ids(p["seed"], 0, 37, p["vocab"])
    a.prefill_chunk(tokens=ids)
    b.prefill_chunk(tokens=ids)
    assert np.array_equal(logits_of(a), logits_of(b))
    tok = int(np.argmax(logits_of(a)))
    assert a.decode_step(tok) == b.decode_step(tok)
    ref = logits_of(a)
    assert np.array_equal(ref, logits_of(b))
    # the source goes first: the shared weights stay until the sibling is destroyed
    a.close()
    b.kv_rollback(-1)
    b.prefill_chunk(tokens=ids)
    b.decode_step(tok)
    assert np.array_equal(ref, logits_of(b))
    b.close()


def _frame(i):
    _, xs = synth.embeddings(TINY_VLM["seed"], i, N_PREFIX, TINY_VLM["hidden"], "bf16")
    return dev_from_storage(xs, "bf16")


def _noise(i):
    return synth.action_noise(TINY_VLM["seed"], i, N_ACT, TINY_AE["hidden"])


def _reference(frame_embeds, x0):
    """A fresh sequential pair: prefill the frame from scratch, denoise x0."""
    m = vla.Model(vla.make_config(**TINY_VLM, init_std=0.08))
    e = vla.Expert(m, vla.make_config(**TINY_AE, init_std=0.08), N_ACT)
    m.prefill_chunk(embeds=frame_embeds, n=N_PREFIX)
    x = torch.from_numpy(x0.copy()).cuda()
    e.denoise(x, n_steps=STEPS, dt=DT)
    torch.cuda.synchronize()
    out = x.cpu().numpy()
    e.close()
    m.close()
    return out


def test_pipeline_actions_equal_a_sequential_pair_on_the_frame_used():
    frames = [_frame(i) for i in range(5)]
    m = vla.Model(vla.make_config(**TINY_VLM, init_std=0.08))
    e = vla.Expert(m, vla.make_config(**TINY_AE, init_std=0.08), N_ACT)
    pl = vla.Pipeline(m, e)
    stream = torch.cuda.current_stream()
    runs = []            # (frame used, noise call, result)
    call = 0
    # the action runs are replayed from a captured graph while x stays the same buffer:
    # fresh buffers first (a capture each), then one buffer refilled between runs
    xbuf = torch.empty((N_ACT, TINY_AE["hidden"]), dtype=torch.float32, device="cuda")
    for f in range(5):
        assert pl.prefill(frames[f], N_PREFIX, stream) == f
        for _ in range(2 if f % 2 else 1):
            if call < 3:
                x = torch.from_numpy(_noise(call).copy()).cuda()
            else:
                x = xbuf
                x.copy_(torch.from_numpy(_noise(call)))
            used = pl.act(x, n_steps=STEPS, dt=DT, stream=stream)
            assert used in (f, f - 1)
            # x is ordered after the run on the caller's stream
            runs.append((used, call, x.cpu().numpy()))
            call += 1
    pl.sync()
    st = pl.stats()
    assert st["prefills"] == 5 and st["acts"] == len(runs)
    assert 0 <= st["acts_on_older"] <= len(runs)
    refs = {}
    for used, c, got in runs:
        if (used, c) not in refs:
            refs[(used, c)] = _reference(frames[used], _noise(c))
        assert np.array_equal(got, refs[(used, c)]), (used, c)
    pl.close()
    e.close()
    m.close()


def test_pipeline_checks_its_arguments():
    m = vla.Model(vla.make_config(**TINY_VLM, init_std=0.08))
    other = vla.Model(vla.make_config(**TINY_VLM, init_std=0.08))
    e = vla.Expert(m, vla.make_config(**TINY_AE, init_std=0.08), N_ACT)
    with pytest.raises(vla.VlaError) as err:
        vla.Pipeline(other, e)
    assert err.value.status == vla.VLA_E_INVALID
    pl = vla.Pipeline(m, e)
    x = torch.from_numpy(_noise(0).copy()).cuda()
    with pytest.raises(vla.VlaError) as err:
        pl.act(x, n_steps=STEPS, dt=DT)
    assert err.value.status == vla.VLA_E_STATE
    with pytest.raises(vla.VlaError) as err:
        pl.prefill(_frame(0), TINY_VLM["max_chunk"] + 1)
    assert err.value.status == vla.VLA_E_INVALID
    pl.close()
    e.close()
    other.close()
    m.close()

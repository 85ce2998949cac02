"""The persistent decode step (one launch for the embedding, RoPE table and every layer,
phases separated by bounded device-scope barriers) against the per-kernel decode path,
and its failure handling, forced from the host.

With at least 9 cached blocks both paths split the keys the same way, so the logits are
bit-identical. A barrier whose target the arrival counter can never reach (a test
option) makes every wait run to a small spin limit: every workgroup ends, the call
returns VLA_E_TIMEOUT, the model state is unchanged, and the next steps are correct.
"""
import numpy as np
import pytest

import kv_cached_gqa_decoder_amd as vla
import synth
from tests.gpu_util import dev_from_storage, logits_of
from tests.test_gpu_parity import TINY_BF16

pytestmark = pytest.mark.gpu


def _pair(n_ctx=150, seed=5):
    p = dict(TINY_BF16, max_chunk=160)
    x32, xs = synth.embeddings(seed, 0, n_ctx, p["hidden"], "bf16")
    a = vla.Model(vla.make_config(**p, init_std=0.08))
    b = vla.Model(vla.make_config(**p, init_std=0.08))
    assert b.get_option(vla.VLA_OPT_PERSISTENT_DECODE) == 0     # the default
    a.set_option(vla.VLA_OPT_PERSISTENT_DECODE, 1)
    for m in (a, b):
        m.prefill_chunk(embeds=dev_from_storage(xs, "bf16"), n=n_ctx)
    return a, b


def test_persistent_decode_is_bit_identical_to_per_kernel_decode():
    a, b = _pair()
    tok = int(np.argmax(logits_of(a)))
    for i in range(20):
        ta = a.decode_step(tok)
        tb = b.decode_step(tok)
        assert a.get_option(vla.VLA_INFO_LAST_DECODE_PERSISTENT) == 1
        assert b.get_option(vla.VLA_INFO_LAST_DECODE_PERSISTENT) == 0
        assert ta == tb and np.array_equal(logits_of(a), logits_of(b)), i
        tok = ta
    # chained on the device (no host round trip between the steps)
    for _ in range(6):
        a.decode_step(vla.VLA_TOKEN_DEVICE, want_token=False)
        b.decode_step(vla.VLA_TOKEN_DEVICE, want_token=False)
    assert np.array_equal(logits_of(a), logits_of(b))
    assert a.state() == b.state()
    a.close()
    b.close()


def test_barrier_timeout_is_reported_and_recovered():
    a, b = _pair()
    tok = int(np.argmax(logits_of(a)))
    st = a.state()
    a.set_option(vla.VLA_OPT_BARRIER_SPIN_LIMIT, 2000)
    a.set_option(vla.VLA_OPT_BARRIER_TEST_UNREACHABLE, 1)
    with pytest.raises(vla.VlaError) as e:
        a.decode_step(tok)
    assert e.value.status == vla.VLA_E_TIMEOUT
    assert a.state() == st                         # the step was rolled back
    a.set_option(vla.VLA_OPT_BARRIER_TEST_UNREACHABLE, 0)
    a.set_option(vla.VLA_OPT_BARRIER_SPIN_LIMIT, 1 << 20)
    for i in range(4):
        ta = a.decode_step(tok)
        tb = b.decode_step(tok)
        assert a.get_option(vla.VLA_INFO_LAST_DECODE_PERSISTENT) == 1
        assert ta == tb and np.array_equal(logits_of(a), logits_of(b)), i
        tok = ta
    # chained on the device: the timeout is reported by the next call that reads a result
    a.set_option(vla.VLA_OPT_BARRIER_SPIN_LIMIT, 2000)
    a.set_option(vla.VLA_OPT_BARRIER_TEST_UNREACHABLE, 1)
    a.decode_step(vla.VLA_TOKEN_DEVICE, want_token=False)
    with pytest.raises(vla.VlaError) as e:
        a.logits_out(np.zeros(a.cfg.vocab, dtype=np.float32))
    assert e.value.status == vla.VLA_E_TIMEOUT
    a.close()
    b.close()


def test_barrier_probe_runs_and_checks_its_arguments():
    us = vla.vla_probe_barrier(64, 50)
    assert 0.0 < us < 1e4
    for grid, nbar in ((0, 10), (1 << 20, 10), (64, 0)):
        with pytest.raises(vla.VlaError) as e:
            vla.vla_probe_barrier(grid, nbar)
        assert e.value.status == vla.VLA_E_INVALID


def test_options_are_checked():
    a, b = _pair(n_ctx=20)
    for key, val in ((vla.VLA_OPT_PERSISTENT_DECODE, 2), (vla.VLA_OPT_BARRIER_SPIN_LIMIT, -1),
                     (vla.VLA_OPT_BARRIER_TEST_UNREACHABLE, 5),
                     (vla.VLA_INFO_LAST_DECODE_PERSISTENT, 1), (12345, 0)):
        with pytest.raises(vla.VlaError) as e:
            a.set_option(key, val)
        assert e.value.status == vla.VLA_E_INVALID
    assert a.get_option(vla.VLA_OPT_PERSISTENT_DECODE) == 1
    assert b.get_option(vla.VLA_OPT_PERSISTENT_DECODE) == 0
    a.close()
    b.close()


def test_read_probe_runs_and_checks_its_arguments():
    """The streaming-read probe (the measured ceiling that the decode fractions are
    given against): a positive rate below the published 8 TB/s, and its argument
    checks (size outside 1 MiB..64 GiB or not a multiple of 16, reps outside 1..100)."""
    gbs = vla.vla_probe_read_bandwidth(64 << 20, 3)
    assert 0.0 < gbs < 8000.0
    for nbytes, reps in (((1 << 20) - 16, 1), ((1 << 20) + 8, 1), (64 << 20, 0), (64 << 20, 101)):
        with pytest.raises(vla.VlaError) as e:
            vla.vla_probe_read_bandwidth(nbytes, reps)
        assert e.value.status == vla.VLA_E_INVALID

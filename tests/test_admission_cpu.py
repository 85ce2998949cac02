"""Admission control ("Can an LLM Forget the Right Things?", section 4) through the C ABI,
against the oracle's plain version (oracle/admission.py); host-only, no GPU."""
import time

import numpy as np
import pytest

from oracle.admission import AdmissionController


@pytest.fixture(scope="module")
def vla():
    import os
    import kv_cached_gqa_decoder_amd as k
    if not os.path.exists(k.vla.LIB_PATH):
        from kv_cached_gqa_decoder_amd import build
        build.build()
    k.load()
    return k


def _pair(vla, **kw):
    return vla.vla_admission_create(**kw), AdmissionController(**kw)


def test_first_cycle_is_admitted_whatever_the_elapsed_time(vla):
    a, o = _pair(vla)
    try:
        assert vla.vla_admission_should_admit(a, 1e6)[0] is True
        assert o.should_admit(1e6)[0] is True
        assert vla.vla_admission_stats_out(a)["has_sample"] == 0
    finally:
        vla.vla_admission_destroy(a)


def test_large_measurements_force_a_refusal(vla):
    a, _ = _pair(vla, prefill_tokens=32, decode_tokens=8)
    try:
        vla.vla_admission_record(a, 1.0, 32, 0.5, 8)        # 1.0 ms + 0.5 ms: admitted
        ok, est = vla.vla_admission_should_admit(a, 0.0)
        assert ok and est == pytest.approx(1.5)
        # inject slow chunks until the estimate passes 33 - 0 - 2 = 31 ms
        n = 0
        while vla.vla_admission_should_admit(a, 0.0)[0]:
            vla.vla_admission_record(a, 400.0, 32, 80.0, 8)
            n += 1
        ok, est = vla.vla_admission_should_admit(a, 0.0)
        assert not ok and est > 31.0 and n >= 1
        # the same estimate is admitted when the budget is larger: it is the estimate,
        # not a latched state, that refuses
        b = vla.vla_admission_create(deadline_ms=1e4)
        vla.vla_admission_record(b, 400.0, 32, 80.0, 8)
        assert vla.vla_admission_should_admit(b, 0.0)[0]
        vla.vla_admission_destroy(b)
    finally:
        vla.vla_admission_destroy(a)


def test_elapsed_time_eats_the_budget(vla):
    a, _ = _pair(vla)
    try:
        vla.vla_admission_record(a, 32 * 0.5, 32, 8 * 1.0, 8)   # estimate 24 ms
        assert vla.vla_admission_should_admit(a, 7.0)[0]          # 33 - 7 - 2 = 24: admitted
        assert not vla.vla_admission_should_admit(a, 7.001)[0]
    finally:
        vla.vla_admission_destroy(a)


def test_decisions_and_averages_equal_the_oracle(vla):
    g = np.random.default_rng(5)
    a, o = _pair(vla, deadline_ms=33.0, safety_margin_ms=2.0, ema_alpha=0.2, prefill_tokens=256,
                 decode_tokens=16)
    try:
        for _ in range(500):
            if g.random() < 0.6:
                pt, dt = int(g.integers(1, 512)), int(g.integers(1, 32))
                pm, dm = float(g.exponential(0.05) * pt), float(g.exponential(0.5) * dt)
                vla.vla_admission_record(a, pm, pt, dm, dt)
                o.record(pm, pt, dm, dt)
            el = float(g.uniform(0.0, 40.0))
            got = vla.vla_admission_should_admit(a, el)
            ref = o.should_admit(el)
            assert got[0] == ref[0] and got[1] == ref[1]
        st = vla.vla_admission_stats_out(a)
        assert st["ema_prefill_ms_per_token"] == o.ema_prefill
        assert st["ema_decode_ms_per_token"] == o.ema_decode
    finally:
        vla.vla_admission_destroy(a)


def test_ema_update_closed_form(vla):
    a, _ = _pair(vla, ema_alpha=0.2, prefill_tokens=1, decode_tokens=1)
    try:
        vla.vla_admission_record(a, 10.0, 1, 20.0, 1)   # bootstrap: the sample itself
        vla.vla_admission_record(a, 0.0, 1, 0.0, 1)     # 0.8 * previous
        vla.vla_admission_record(a, 5.0, 1, 5.0, 1)     # 0.8 * 0.8 * prev + 0.2 * 5
        st = vla.vla_admission_stats_out(a)
        assert st["ema_prefill_ms_per_token"] == pytest.approx(0.64 * 10.0 + 1.0, rel=1e-15)
        assert st["ema_decode_ms_per_token"] == pytest.approx(0.64 * 20.0 + 1.0, rel=1e-15)
    finally:
        vla.vla_admission_destroy(a)


def test_host_sleep_past_the_deadline_is_a_miss(vla):
    a = vla.vla_admission_create(deadline_ms=33.0)
    try:
        vla.vla_admission_cycle_begin(a)
        time.sleep(0.002)
        ms_ok = vla.vla_admission_cycle_end(a, True)
        vla.vla_admission_cycle_begin(a)
        time.sleep(0.040)
        ms_late = vla.vla_admission_cycle_end(a, False)
        st = vla.vla_admission_stats_out(a)
        assert ms_ok < 33.0 <= 40.0 <= ms_late
        assert (st["cycles"], st["admitted"], st["refused"], st["deadline_misses"]) == (2, 1, 1, 1)
        assert st["last_overrun_ms"] == pytest.approx(ms_late - 33.0)
        assert st["worst_cycle_ms"] == ms_late
    finally:
        vla.vla_admission_destroy(a)


def test_sleep_until_deadline_lands_on_it(vla):
    a = vla.vla_admission_create(deadline_ms=20.0)
    try:
        vla.vla_admission_cycle_begin(a)
        vla.vla_admission_sleep_until_deadline(a)
        el = vla.vla_admission_elapsed_ms(a)
        assert 20.0 <= el < 25.0
        t0 = time.perf_counter()
        vla.vla_admission_sleep_until_deadline(a)      # already past: returns at once
        assert time.perf_counter() - t0 < 0.005
    finally:
        vla.vla_admission_destroy(a)


def test_bad_arguments_are_refused(vla):
    for kw in (dict(deadline_ms=0.0), dict(safety_margin_ms=-1.0), dict(ema_alpha=0.0),
               dict(ema_alpha=1.5), dict(prefill_tokens=0), dict(decode_tokens=-1)):
        with pytest.raises(vla.VlaError) as e:
            vla.vla_admission_create(**kw)
        assert e.value.status == vla.VLA_E_INVALID
    a = vla.vla_admission_create()
    try:
        for args in ((1.0, 0, 1.0, 1), (1.0, 1, 1.0, 0), (-1.0, 1, 1.0, 1), (float("nan"), 1, 1.0, 1)):
            with pytest.raises(vla.VlaError) as e:
                vla.vla_admission_record(a, *args)
            assert e.value.status == vla.VLA_E_INVALID
        assert vla.vla_admission_stats_out(a)["has_sample"] == 0
    finally:
        vla.vla_admission_destroy(a)

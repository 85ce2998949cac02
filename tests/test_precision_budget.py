"""Precision budget of the bf16 configurations (CPU).

The GeGLU, head-dim-256 GPU test model (hidden 256, 2 query heads on 1 KV head,
vocabulary 800) is run through the oracle and through a copy of it that rounds
the device path's bf16 storage points and nothing else (tests/bf16_emulation.py).
At weights N(0, 0.08^2) that exact bf16-storage model already misses the 2e-2
max relative error bound on its logits, and no single rounding point dominates,
so the bound cannot be met there by any implementation that keeps those values
in bf16; at N(0, 0.05^2), the scale the GPU test uses, it sits well inside.
"""
import numpy as np

import synth
from oracle import decoder as D
from tests.bf16_emulation import POINTS, Bf16Session


def _worst_rel(std, points, steps=20, seed=62):
    c = D.Config("geglu_d256", 3, 256, 2, 1, 256, 512, 800, rope_theta=1e4, wdtype="bf16",
                 act="bf16", num_blocks=16, max_frames=4, seed=seed, init_std=std,
                 ffn_kind="geglu")
    ref = D.Session(c)
    emu = Bf16Session(c, points, weights=ref.w)
    ids = synth.token_ids(seed, 0, 45, 800)
    _, r = ref.prefill_chunk(tokens=ids)
    _, e = emu.prefill_chunk(tokens=ids)
    worst = np.max(np.abs(e - r)) / np.max(np.abs(r))
    tok = int(np.argmax(r))
    for _ in range(steps):
        nxt, r = ref.decode_step(tok)
        _, e = emu.decode_step(tok)
        worst = max(worst, np.max(np.abs(e - r)) / np.max(np.abs(r)))
        tok = nxt
    return float(worst)


def test_emulation_with_no_rounding_is_the_oracle():
    assert _worst_rel(0.08, (), steps=2) < 1e-12


def test_geglu_d256_budget_exceeds_bound_at_0p08_and_not_at_0p05():
    at08 = _worst_rel(0.08, POINTS)
    at05 = _worst_rel(0.05, POINTS)
    assert at08 > 2e-2, at08          # exact bf16 storage cannot meet the bound here
    assert at05 < 1e-2, at05          # the GPU test's scale leaves a 2x margin
    # no single storage point accounts for the excess on its own
    singles = [_worst_rel(0.08, (p,), steps=8) for p in POINTS]
    assert max(singles) < 2e-2, singles

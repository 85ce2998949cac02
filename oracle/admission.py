"""Admission control of a real-time reasoning cycle (the oracle's plain version).

Test infrastructure: only tests/, the smoke check and the benchmark's CPU
baseline use this module.

"Can an LLM Forget the Right Things?", section 4: before any GPU work of a
cycle starts, the runtime estimates what the next reasoning chunk will cost and
refuses to start it when the estimate does not fit what is left of the cycle's
deadline after a safety margin. The estimate comes from two separate
exponential moving averages, per-token prefill time and per-token decode time,
each updated with weight alpha for the new measurement. The first cycle is
always admitted (there is no history yet). A refused cycle falls back to the
last action.

    remaining = deadline - elapsed - margin
    estimate  = ema_prefill_per_token * prefill_tokens + ema_decode_per_token * decode_tokens
    admit     = (no sample yet) or estimate <= remaining
    ema      <- (1 - alpha) * ema + alpha * measured          (each EMA on its own)

Readings fixed here (the page is silent): the first recorded measurement
initialises both EMAs (the "bootstrap sample"); averages are kept in fp64; a
cycle whose duration exceeds the deadline is a deadline miss and is counted,
with its overrun, whether or not its chunk was admitted.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass
class Stats:
    cycles: int = 0
    admitted: int = 0
    refused: int = 0
    deadline_misses: int = 0
    worst_cycle_ms: float = 0.0
    last_overrun_ms: float = 0.0


class AdmissionController:
    def __init__(self, deadline_ms=33.0, safety_margin_ms=2.0, ema_alpha=0.2, prefill_tokens=32,
                 decode_tokens=8):
        self.deadline_ms = float(deadline_ms)
        self.margin_ms = float(safety_margin_ms)
        self.alpha = float(ema_alpha)
        self.prefill_tokens = int(prefill_tokens)
        self.decode_tokens = int(decode_tokens)
        self.has_sample = False
        self.ema_prefill = 0.0
        self.ema_decode = 0.0
        self.stats = Stats()

    def estimate_ms(self) -> float:
        return self.ema_prefill * self.prefill_tokens + self.ema_decode * self.decode_tokens

    def should_admit(self, elapsed_ms: float):
        """(admit?, the estimate in ms)."""
        est = self.estimate_ms()
        if not self.has_sample:
            return True, est
        remaining = self.deadline_ms - elapsed_ms - self.margin_ms
        return est <= remaining, est

    def record(self, prefill_ms, prefill_tokens, decode_ms, decode_tokens) -> None:
        p = prefill_ms / prefill_tokens
        d = decode_ms / decode_tokens
        if not self.has_sample:
            self.ema_prefill, self.ema_decode = p, d
            self.has_sample = True
            return
        a = self.alpha
        self.ema_prefill = (1.0 - a) * self.ema_prefill + a * p
        self.ema_decode = (1.0 - a) * self.ema_decode + a * d

    def end_cycle(self, admitted: bool, cycle_ms: float) -> None:
        s = self.stats
        s.cycles += 1
        if admitted:
            s.admitted += 1
        else:
            s.refused += 1
        s.worst_cycle_ms = max(s.worst_cycle_ms, cycle_ms)
        if cycle_ms > self.deadline_ms:
            s.deadline_misses += 1
            s.last_overrun_ms = cycle_ms - self.deadline_ms

// Admission control of a real-time reasoning cycle ("Can an LLM Forget the
// Right Things?", section 4): before a cycle's GPU work starts, the cost of the
// next chunk is estimated from two exponential moving averages (per-token
// prefill and per-token decode time, each updated with weight alpha for a new
// measurement) and the chunk is refused when the estimate exceeds what is left
// of the deadline after a safety margin. The first cycle is always admitted; the
// first measurement initialises both averages. Cycle durations past the
// deadline are counted as misses. The cycle clock is the steady clock, and the
// wait for the cycle's end sleeps through all but the last millisecond and then
// spins (section 3 of the same page: sleep granularity is about a millisecond).
// Host-only; no HIP calls.
#pragma once

#include <stdint.h>

#include <chrono>
#include <thread>

namespace vla {

class Admission {
 public:
  using clock = std::chrono::steady_clock;

  Admission(double deadline_ms, double margin_ms, double alpha, int prefill_tokens,
            int decode_tokens)
      : deadline_ms_(deadline_ms),
        margin_ms_(margin_ms),
        alpha_(alpha),
        prefill_tokens_(prefill_tokens),
        decode_tokens_(decode_tokens),
        start_(clock::now()) {}

  double estimate_ms() const {
    return ema_prefill_ * (double)prefill_tokens_ + ema_decode_ * (double)decode_tokens_;
  }

  bool should_admit(double elapsed_ms, double* est_out) const {
    const double est = estimate_ms();
    if (est_out) *est_out = est;
    if (!has_sample_) return true;
    const double remaining = deadline_ms_ - elapsed_ms - margin_ms_;
    return est <= remaining;
  }

  void record(double prefill_ms, int prefill_tokens, double decode_ms, int decode_tokens) {
    const double p = prefill_ms / (double)prefill_tokens;
    const double d = decode_ms / (double)decode_tokens;
    if (!has_sample_) {
      ema_prefill_ = p;
      ema_decode_ = d;
      has_sample_ = true;
      return;
    }
    ema_prefill_ = (1.0 - alpha_) * ema_prefill_ + alpha_ * p;
    ema_decode_ = (1.0 - alpha_) * ema_decode_ + alpha_ * d;
  }

  void cycle_begin() { start_ = clock::now(); }

  double elapsed_ms() const {
    return std::chrono::duration<double, std::milli>(clock::now() - start_).count();
  }

  // close the cycle: count the outcome, and a miss when it ran past the deadline
  double cycle_end(bool admitted) {
    const double ms = elapsed_ms();
    ++cycles_;
    if (admitted)
      ++admitted_;
    else
      ++refused_;
    if (ms > worst_ms_) worst_ms_ = ms;
    if (ms > deadline_ms_) {
      ++misses_;
      last_overrun_ms_ = ms - deadline_ms_;
    }
    return ms;
  }

  // sleep until the cycle's deadline: sleep through all but the last millisecond,
  // then spin
  void sleep_until_deadline() const {
    const auto target =
        start_ + std::chrono::duration_cast<clock::duration>(
                     std::chrono::duration<double, std::milli>(deadline_ms_));
    for (;;) {
      const auto now = clock::now();
      if (now >= target) return;
      const auto left_ms =
          std::chrono::duration_cast<std::chrono::milliseconds>(target - now).count();
      if (left_ms > 1) std::this_thread::sleep_for(std::chrono::milliseconds(left_ms - 1));
    }
  }

  int64_t cycles_ = 0, admitted_ = 0, refused_ = 0, misses_ = 0;
  double worst_ms_ = 0.0, last_overrun_ms_ = 0.0;
  double ema_prefill_ = 0.0, ema_decode_ = 0.0;
  bool has_sample_ = false;

 private:
  double deadline_ms_, margin_ms_, alpha_;
  int prefill_tokens_, decode_tokens_;
  clock::time_point start_;
};

}  // namespace vla

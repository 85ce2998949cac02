"""CPU oracle for the KV-cached GQA decoder path: TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy (fp64) implementation of what the GPU
path computes. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call, link or run anything in
this package. The GPU library never imports it and shares no code with it; the
only thing both sides consume is the seeded input generator in ``synth.py``,
which holds none of the method's arithmetic.

Sources (the pages; cited by title and section):
  * "Can an LLM Forget the Right Things?" (vla-edge-backend blog and its
    translation): §5 KV manager (FIFO / semantic eviction, host cosine),
    §6 the hand-written transformer (RMSNorm, RoPE, GQA, SwiGLU, seeded PRNG).
  * "CSR: Infinite-Horizon Real-Time Policies with Massive Cached State
    Representations": §III-A, the KV-caching equations (q, k, v projections,
    scaled softmax attention, output head W_Y); Appendix A FLOP count.
  * "Rebuilding Kshipra Around Memory": §1 block-arena KV cache with a LIFO
    free-list and GQA-aware sizing; §2 INT4 groups of 128 with one fp16 scale
    used on both sides; §4 chunked prefill (online softmax over blocks read in
    place, absolute RoPE positions, causal mask within the chunk).
  * "Running VLAs at Real-time Speed": §2 (pi0 = VLM prefix + action expert
    with flow matching), §4.1 (last LLM layer reduced to its KV), §4.2 (fused
    gated FFN), §5.1 (weights-only roofline bytes).

Modules:
  rng       splitmix64 -> Box-Muller seeded generator (weights are regenerated
            here from the seed, independently of the GPU library).
  decoder   configs, weights, RMSNorm, RoPE, GQA attention, SwiGLU, the cached
            forward (prefill chunk / decode) over a paged KV store.
  kvpool    LIFO block free-list + frame registry (block tables).
  scoring   per-frame mean keys, all-pairs cosine, argmax eviction.
  int4      group-128 symmetric INT4 quantiser with one fp16 scale.
  pi0       the two-part policy step: GeGLU prefix model with a K/V-only last
            layer, the action expert attending to its cache and to itself in
            both directions, the time embedding and the Euler loop.

Every function here is "parity pinned" by a CPU test in tests/test_oracle_*.py
unless its docstring says "parity unpinned".
"""

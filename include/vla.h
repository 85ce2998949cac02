/* vla.h -- C ABI of the KV-cached GQA decoder library for MI355X (gfx950).
 *
 * One model instance ("handle") holds seeded random-init weights, a block-paged
 * KV cache with a LIFO free-list, per-frame mean keys, and scratch buffers, all
 * on the HIP device that was current when the handle was created. Every entry
 * point is plain C: plain pointers and sizes, no C++ or framework types.
 *
 * What is computed (cited by page title and section):
 *  - the pre-norm decoder layer: RMSNorm, fused q/k/v projection, RoPE at
 *    absolute positions, grouped-query attention over the cached keys,
 *    output projection, RMSNorm, gated (SwiGLU) feed-forward
 *    ("Can an LLM Forget the Right Things?", section 6; "CSR: Infinite-Horizon
 *    Real-Time Policies with Massive Cached State Representations", III-A);
 *  - chunked prefill reading KV blocks in place, causal inside the chunk, RoPE
 *    positions continuing after the cached tokens
 *    ("Rebuilding Kshipra Around Memory", section 4);
 *  - a block arena reserved once with a LIFO free-list
 *    ("Rebuilding Kshipra Around Memory", section 1);
 *  - redundant-frame scoring by cosine similarity and eviction of the most
 *    redundant frame ("Can an LLM Forget the Right Things?", section 5).
 *
 * Conventions shared by all calls
 *  - Return value: VLA_OK (0) or a negative vla_status. On failure the model
 *    state is unchanged and vla_last_error() holds a message (thread local).
 *    No C++ exception crosses this boundary.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream). Work is enqueued on it; pointers passed in must stay valid until
 *    the stream has reached the call.
 *  - Synchronisation: a call that returns a host value computed on the device
 *    (out_next_token, the frame id of an eviction, out_score) synchronises the
 *    stream before returning. Everything else is asynchronous.
 *  - Ownership: the library owns everything it allocates (weights, KV pool,
 *    tables, scratch); the caller owns every pointer it passes.
 *  - Threading: a handle must not be used from two threads at once.
 *  - Frames: a frame is the unit of eviction: one vla_prefill_chunk or one
 *    vla_kv_append_raw call. It starts on a fresh block. Decode tokens form a
 *    non-evictable tail that also starts on a fresh block.
 *  - Positions: a monotonic counter; every appended token takes the next
 *    position and positions are never reused (vla_kv_rollback excepted).
 */
#ifndef VLA_H
#define VLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct vla_model vla_model;   /* opaque, owned by the library */
typedef struct vla_pool vla_pool;     /* opaque host-only block pool */

typedef enum {
  VLA_OK = 0,
  VLA_E_INVALID = -1,          /* bad configuration, shape or argument */
  VLA_E_NO_BLOCKS = -2,        /* not enough free KV blocks (or frame slots) */
  VLA_E_NOTHING_TO_EVICT = -3, /* fewer than two evictable frames */
  VLA_E_HIP = -4,              /* a HIP runtime call failed */
  VLA_E_STATE = -5,            /* call not valid in the current state */
  VLA_E_TIMEOUT = -6           /* a bounded wait between the workgroups of a persistent
                                  kernel gave up (see vla_set_option) */
} vla_status;

typedef enum { VLA_F32 = 0, VLA_BF16 = 1, VLA_INT4_G128 = 2 } vla_dtype;
/* Gated FFN: SwiGLU silu(x Wg^T) * (x Wu^T), or GeGLU with the exact-erf GELU
 * ("Running VLAs at Real-time Speed", section 4.2: the gated pair, fused). */
typedef enum { VLA_SWIGLU = 0, VLA_GEGLU = 1 } vla_ffn_kind;

/* Model configuration. Sizes in elements. */
typedef struct {
  int32_t n_layers;     /* decoder layers L */
  int32_t hidden;       /* H, multiple of 64 */
  int32_t n_heads;      /* query heads Hq */
  int32_t n_kv_heads;   /* KV heads Hkv, divides Hq (Hq/Hkv = group size g) */
  int32_t head_dim;     /* d, even, <= 256, multiple of 16 */
  int32_t ffn;          /* F, multiple of 16 */
  int32_t vocab;        /* V; 0: no embedding table and no output head (embeddings
                           in, K/V out: a prefix model), and no logits */
  float rms_eps;        /* RMSNorm epsilon */
  double rope_theta;    /* RoPE base */
  int32_t wdtype;       /* projection weights: VLA_F32, VLA_BF16 (both = act_dtype) or
                           VLA_INT4_G128 (with act_dtype VLA_BF16; hidden, n_heads*head_dim
                           and ffn multiples of 128) */
  int32_t act_dtype;    /* activations, embedding table and KV cache: VLA_F32 or VLA_BF16 */
  int32_t ffn_kind;     /* VLA_SWIGLU or VLA_GEGLU */
  int32_t block_tokens; /* tokens per KV block: 16 */
  int32_t num_blocks;   /* KV budget in blocks (the fixed memory budget) */
  int32_t max_frames;   /* most frames resident at once (mean-key table rows) */
  int32_t max_chunk;    /* longest prefill chunk / raw append, in tokens */
  uint64_t seed;        /* weight seed */
  double init_std;      /* weights ~ N(0, init_std^2); norm weights are 1 */
  int32_t kv_only_last; /* 1: the last layer computes only its input norm and K/V
                           ("Running VLAs at Real-time Speed", section 4.1: only the
                           cache of that layer is used); needs vocab 0 */
  uint32_t stream_base; /* added to every per-layer weight stream (two models built
                           from one seed, e.g. a prefix model and its expert) */
} vla_config;

typedef struct vla_expert vla_expert;

/* Create a model: validates cfg, allocates weights, KV pool (K as
 * [L][num_blocks][Hkv][d/c][block_tokens][c] with c = 64 bytes / element size,
 * V as [L][num_blocks][Hkv][d][block_tokens], both in act_dtype), the mean-key table
 * ([L][max_frames][Hkv*d] fp64) and scratch on the current device, and fills
 * the weights from the seeded splitmix64 -> Box-Muller generator
 * ("Can an LLM Forget the Right Things?", section 6: untrained weights from a
 * seeded PRNG). Element i (row-major, logical (out, in) layout) of tensor
 * stream s is init_std * N(seed, s, i) rounded to nearest-even into wdtype.
 * Streams: embedding 1, output head 2, layer l's tensors stream_base +
 * ((l + 1) << 8 | kind), kinds q 1, k 2, v 3, o 4, gate 5, up 6, down 7.
 * VLA_INT4_G128 ("Rebuilding Kshipra Around Memory", section 2: INT4 weights
 * in groups of 128 with one fp16 scale, used both to encode and to decode):
 * every projection and the output head (the embedding table stays in
 * act_dtype) is drawn as above, rounded to fp32, and quantised per group of
 * 128 consecutive inputs of one output row: s = fp16(max|w| / 7) (fp32
 * division, nearest-even), q = clamp(nearest-even(w / s), -8, 7) (q = 0 when
 * s = 0). Device layout of an N x K tensor: codes [N][K/2] (two per byte, the
 * even input in the low nibble), then scales [K/128][N] fp16. Inside the
 * projections the weight is q * s, exact in fp32.
 * Synchronises the device. Errors: VLA_E_INVALID (bad cfg, out == NULL),
 * VLA_E_HIP (allocation or launch failure). */
vla_status vla_model_create(const vla_config* cfg, vla_model** out);

/* Free everything the handle owns (synchronises the device). NULL is a no-op.
 * Weights shared with sibling models are freed with the last model using them. */
void vla_model_destroy(vla_model* m);

/* A second model over the same weights ("Running VLAs at Real-time Speed",
 * section 6.1: a second prefix state, filled while the first one is read): the
 * source's config, its own KV pool, tables and scratch, and the source's
 * embedding, output head and projection weights, read-only and shared (kept
 * until the last model using them is destroyed, in any order). The source is
 * not modified. Synchronises the device. Errors: VLA_E_INVALID (NULL src or
 * out), VLA_E_HIP. */
vla_status vla_model_create_sibling(const vla_model* src, vla_model** out);

/* Append one frame of n tokens at the next n positions and run the whole
 * forward over it ("Rebuilding Kshipra Around Memory", section 4).
 * Exactly one of:
 *   tokens  host int32[n], ids in [0, vocab): rows of the embedding table;
 *   embeds  device pointer to [n][hidden] in act_dtype: caller embeddings
 *           (e.g. visual tokens), used as given.
 * Writes the new frame id to *out_frame_id (host, nullable; ids count up from
 * 0 in arrival order). The last row's logits are kept (vla_logits_out).
 * Errors: VLA_E_INVALID (n < 1, n > max_chunk, both/neither input, id out of
 * range), VLA_E_NO_BLOCKS (ceil(n/block_tokens) blocks not free, or
 * max_frames frames resident). */
vla_status vla_prefill_chunk(vla_model* m, const int32_t* tokens, const void* embeds,
                             int32_t n, int32_t* out_frame_id, void* stream);

/* One decode token at the next position ("CSR: Infinite-Horizon Real-Time
 * Policies with Massive Cached State Representations", III-A: with the K/V of
 * earlier tokens cached, each new token only computes its own q, k, v and
 * attends to the cache; "Can an LLM Forget the Right Things?", section 4: one
 * greedy argmax token per decode step): embedding row `token`, full forward,
 * logits kept, and the greedy next token (argmax over the vocabulary, ties to
 * the lowest id) written to *out_next_token (host, nullable; non-NULL
 * synchronises the stream). token VLA_TOKEN_DEVICE: the greedy token of the
 * previous forward (prefill or decode), read on the device; with
 * out_next_token NULL nothing synchronises, so greedy decode steps can be
 * enqueued back to back without a host round trip. Errors: VLA_E_INVALID
 * (token out of range), VLA_E_STATE (VLA_TOKEN_DEVICE before any forward),
 * VLA_E_NO_BLOCKS (the tail needs a new block and none is free). */
#define VLA_TOKEN_DEVICE (-1)
vla_status vla_decode_step(vla_model* m, int32_t token, int32_t* out_next_token, void* stream);

/* Score the resident frames on `layer` and evict the most redundant one
 * ("Can an LLM Forget the Right Things?", section 5). Each frame is represented
 * by its mean key on that layer (fp64 mean over its tokens of the stored,
 * post-RoPE keys, all KV heads concatenated: Hkv*d values). For every
 * unordered pair of frames s = dot / (sqrt(|a|^2) sqrt(|b|^2)) in fp64 (0 when
 * that denominator is below 1e-8), computed once per pair; each frame's score
 * is its largest similarity to any other frame; the frame with the highest
 * score is evicted, ties to the lowest frame id (the oldest). Its blocks are
 * pushed onto the free-list in logical order and its mean keys dropped.
 * Writes the evicted frame id and its score (both host, nullable).
 * Synchronises the stream. Errors: VLA_E_INVALID (layer out of range),
 * VLA_E_NOTHING_TO_EVICT (fewer than two frames resident). */
vla_status vla_kv_score_and_evict(vla_model* m, int32_t layer, int32_t* out_frame_id,
                                  double* out_score, void* stream);

/* Same scoring as vla_kv_score_and_evict without evicting (state unchanged). */
vla_status vla_kv_score(vla_model* m, int32_t layer, int32_t* out_frame_id, double* out_score,
                        void* stream);

/* Eviction policies ("Can an LLM Forget the Right Things?", section 5):
 *  VLA_EVICT_SEMANTIC  the all-pairs redundancy scoring of vla_kv_score_and_evict;
 *  VLA_EVICT_FIFO      the oldest resident frame (the page's FIFO baseline; score 0);
 *  VLA_EVICT_ADJACENT  the page's own semantic rule: the cosine of each frame's mean
 *                      key with the next frame's (arrival order), and the older frame
 *                      of the most similar pair (the first pair on ties); the score is
 *                      that pair's cosine, the same fp64 value the all-pairs scoring
 *                      gives the pair.
 * A sliding window of W frames is FIFO with vla_kv_make_room's window W (with frames
 * of one size the two evict the same frames, as the page notes). */
typedef enum { VLA_EVICT_SEMANTIC = 0, VLA_EVICT_FIFO = 1, VLA_EVICT_ADJACENT = 2 } vla_evict_policy;

/* Evict one frame chosen by `policy` on mean keys of `layer`; writes its frame id and
 * score (host, nullable). Synchronises the stream (FIFO: no device work). Errors:
 * VLA_E_INVALID (policy, layer), VLA_E_NOTHING_TO_EVICT (no frame; fewer than two for
 * the scoring policies). */
vla_status vla_kv_evict(vla_model* m, int32_t policy, int32_t layer, int32_t* out_frame_id,
                        double* out_score, void* stream);

/* Evict frames chosen by `policy` until a frame of n_tokens fits (its blocks and a frame
 * slot are free) and, when window > 0, fewer than `window` frames are resident (at most
 * `window` frames after the insert): the page's evict-until-room loop. With one frame
 * left every policy takes it. Writes the number of frames evicted (host, nullable).
 * Errors: VLA_E_INVALID (policy, layer, n_tokens outside 1..max_chunk, window < 0),
 * VLA_E_NO_BLOCKS (evicting every frame would not free enough blocks; nothing is
 * evicted). */
vla_status vla_kv_make_room(vla_model* m, int32_t policy, int32_t layer, int32_t n_tokens,
                            int32_t window, int32_t* out_evicted, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops, harnesses that forbid allocation): the scoring of
 * vla_kv_score on a caller-given mean-key table, with no handle and no
 * allocation. mean_keys: device fp64 [n_frames][dim], one row per frame in
 * arrival order. Writes the winning row's index (device int32) and its score
 * (device fp64); asynchronous on `stream`, nothing synchronises. The per-frame
 * scores live in a library-owned static device array of 4096 doubles per GPU,
 * alive until the process ends: at most 4096 frames. Calls that overlap on one
 * GPU share that array and race; serialise them (one stream, or events).
 * Errors: VLA_E_INVALID (null pointer, n_frames > 4096, dim < 1),
 * VLA_E_NOTHING_TO_EVICT (n_frames < 2), VLA_E_HIP (launch failure). */
vla_status vla_kv_score_noalloc(const double* mean_keys, int32_t n_frames, int32_t dim,
                                int32_t* out_index, double* out_score, void* stream);

/* Output head ("CSR: Infinite-Horizon Real-Time Policies with Massive Cached
 * State Representations", III-A: the distribution over the vocabulary comes from
 * W_Y applied to the last hidden state; here before the softmax, after the final
 * RMSNorm). Copy the last computed logits (fp32[vocab], from the last prefill row or
 * decode step) into `out` (host or device memory; n must equal vocab).
 * Synchronises the stream. Errors: VLA_E_INVALID (n != vocab, out NULL),
 * VLA_E_STATE (no forward has run yet). */
vla_status vla_logits_out(vla_model* m, float* out, int32_t n, void* stream);

/* Message of the last failure on this thread ("" if none). Owned by the library. */
const char* vla_last_error(void);

/* Append a frame whose keys and values are given: k, v are device pointers to
 * [n_layers][n][n_kv_heads][head_dim] in act_dtype, stored as given (already
 * rotated; no RoPE is applied). The frame takes the next n positions and its
 * mean keys are computed. Errors: as vla_prefill_chunk. */
vla_status vla_kv_append_raw(vla_model* m, const void* k, const void* v, int32_t n,
                             int32_t* out_frame_id, void* stream);

/* Drop every frame and decode tail created after frame keep_frame_id, newest
 * first, returning their blocks in reverse allocation order (this restores the
 * free-list exactly when nothing was evicted since), and reset the position
 * and frame-id counters to their values right after that frame. keep_frame_id
 * -1 drops every frame and tail (position 0, frame id 0 next). Host-only
 * bookkeeping; enqueues no work. Errors: VLA_E_INVALID (no such frame). */
vla_status vla_kv_rollback(vla_model* m, int32_t keep_frame_id);

/* Recompute every resident frame's mean keys on every layer from the stored
 * keys (a full refresh; reads the whole key cache once). */
vla_status vla_kv_refresh_mean_keys(vla_model* m, void* stream);

/* Host-side view of the state. */
typedef struct {
  int64_t next_position;    /* position the next token will take */
  int32_t next_frame_id;
  int32_t n_frames;         /* resident frames */
  int32_t resident_tokens;  /* frames + decode tail */
  int32_t free_blocks;
  int32_t logical_blocks;   /* entries of the logical block table */
} vla_state;
vla_status vla_get_state(const vla_model* m, vla_state* out);

/* Logical block table (creation order of frames/tails, blocks in order within
 * each): physical block ids and valid tokens per block, host arrays of `cap`
 * entries; *n_out receives the number of entries. */
vla_status vla_kv_block_table(const vla_model* m, int32_t* blocks, int32_t* ntok, int32_t cap,
                              int32_t* n_out);

/* The KV free-list as a stack, bottom first: out[n-1] is the block the next
 * allocation pops ("Rebuilding Kshipra Around Memory", section 1: LIFO reuse
 * of freed blocks). Host array of cap entries; *n_out receives the number of
 * free blocks (entries past cap are not written). Host-only; enqueues no work.
 * Errors: VLA_E_INVALID (null m or n_out). */
vla_status vla_kv_free_list(const vla_model* m, int32_t* out, int32_t cap, int32_t* n_out);

/* Resident frame ids in arrival order (host array of cap entries). */
vla_status vla_kv_frames(const vla_model* m, int32_t* frame_ids, int32_t cap, int32_t* n_out);

/* Copy layer `layer`'s mean keys of the resident frames, in arrival order, to
 * host memory out[cap_frames][n_kv_heads*head_dim] (fp64). Synchronises. */
vla_status vla_mean_keys_out(vla_model* m, int32_t layer, double* out, int32_t cap_frames,
                             int32_t* n_out, void* stream);

/* Copy the resident keys and values of `layer` in logical order to device
 * memory k_out, v_out: [cap_tokens][n_kv_heads][head_dim] in act_dtype. */
vla_status vla_kv_gather(vla_model* m, int32_t layer, void* k_out, void* v_out,
                         int32_t cap_tokens, int32_t* n_out, void* stream);

/* Copy one weight tensor in its logical (out, in) row-major layout and storage
 * type to device memory `out` of `bytes` bytes. kind: 1 q, 2 k, 3 v, 4 o,
 * 5 gate, 6 up, 7 down (per layer), 8 embedding, 9 output head (layer ignored).
 * INT4 models: kinds 1-7 and 9 are written dequantised (q * s, fp32). */
vla_status vla_weight_out(vla_model* m, int32_t kind, int32_t layer, void* out, int64_t bytes,
                          void* stream);

/* Execution options of a handle.
 *  VLA_OPT_PERSISTENT_DECODE (default 0): run a decode step's layers as one
 *    persistent launch when the model's shape has that kernel (bf16 weights, head
 *    dim 128, the Qwen2.5-1.5B projection shapes and the tiny test shapes): a fixed
 *    grid of resident workgroups walks the phases of every layer, separated by
 *    device-scope barriers ("Running VLAs at Real-time Speed", sections 3.1 and 5.2:
 *    the step as one unit, and the cost of synchronising many small products); a
 *    barrier counts the workgroups of each XCD first and writes each XCD's L2 back
 *    once, from its last arrival (a device reporting an XCD id outside 0..7 makes
 *    the step fail with VLA_E_HIP, reported like a barrier time-out).
 *    0: one launch per projection and attention. While a kernel class is profiled
 *    (vla_profile_enable) the per-kernel launches are used.
 *  VLA_OPT_BARRIER_SPIN_LIMIT (default 1048576): polls of a barrier wait before it
 *    gives up (>= 0). A workgroup that gives up sets an error flag and ends, every
 *    other one ends at its next wait, and the call that reads the step's result
 *    returns VLA_E_TIMEOUT (a decode step with out_next_token, else the next
 *    vla_logits_out or such decode step); the decode step is then to be rolled back.
 *  VLA_OPT_BARRIER_TEST_UNREACHABLE (default 0; for tests): 1 gives every barrier a
 *    target its generation never reaches, so each wait runs to its spin limit.
 *  VLA_INFO_LAST_DECODE_PERSISTENT (read only): 1 when the last decode step ran the
 *    persistent kernel.
 * Errors: VLA_E_INVALID (unknown key, value out of range, setting a read-only key). */
enum {
  VLA_OPT_PERSISTENT_DECODE = 1,
  VLA_OPT_BARRIER_SPIN_LIMIT = 2,
  VLA_OPT_BARRIER_TEST_UNREACHABLE = 3,
  VLA_INFO_LAST_DECODE_PERSISTENT = 100
};
vla_status vla_set_option(vla_model* m, int32_t key, int64_t value);
/* The latency of that barrier alone: nbar barriers over `grid` resident workgroups of
 * 256 threads (cooperative launch, one store per thread per phase), timed with stream
 * events after one untimed launch of 10 barriers; writes microseconds per barrier. Allocates and frees its own buffers;
 * synchronises the stream. Errors: VLA_E_INVALID (grid beyond what can be resident,
 * nbar outside 1..100000), VLA_E_TIMEOUT, VLA_E_HIP (an XCD id outside 0..7). */
vla_status vla_probe_barrier(int32_t grid, int32_t nbar, void* stream, double* out_us);
vla_status vla_get_option(const vla_model* m, int32_t key, int64_t* value);

/* Kernel timing with HIP events. While a kernel class is enabled, every
 * kernel that a call of that class launches carries a start/stop event pair
 * in its own dispatch on the launch stream (so the span is the kernel's
 * execution, as a kernel trace reports it). vla_profile_read synchronises and
 * returns the summed kernel time (ms) and the number of profiled calls since
 * the last enable; a call may launch several kernels, all summed (VLA_K_SCORE:
 * two; attention: the split pass plus, when the keys are split, the merge;
 * residual projections: the product plus the split reduction). VLA_K_NONE
 * disables. Errors: VLA_E_INVALID (bad class). */
enum {
  VLA_K_NONE = 0, VLA_K_GEMV_QKV = 1, VLA_K_GEMV_O = 2, VLA_K_GEMV_GATEUP = 3,
  VLA_K_GEMV_DOWN = 4, VLA_K_GEMV_HEAD = 5, VLA_K_ATTN_DECODE = 6, VLA_K_GEMM_QKV = 7,
  VLA_K_GEMM_O = 8, VLA_K_GEMM_GATEUP = 9, VLA_K_GEMM_DOWN = 10, VLA_K_ATTN_PREFILL = 11,
  VLA_K_MEANKEYS = 12, VLA_K_SCORE = 13, VLA_K_RMSNORM = 14, VLA_K_COUNT = 15
};
vla_status vla_profile_enable(vla_model* m, int32_t kernel_class);
vla_status vla_profile_read(vla_model* m, double* total_ms, int32_t* launches);

/* Kernel timing by replay, for kernels too short to carry events of their own
 * without changing their duration: launches the one-token projection of
 * `kernel_class` for every layer, `reps` times, back to back on `stream`
 * between two stream events, synchronises, and returns the mean time per
 * launch (ms) in *ms_per_launch. Only VLA_K_GEMV_GATEUP (the gated FFN
 * projection of a decode step): it reads the residual row and rewrites only
 * the FFN activation scratch, so the model's state and results are unchanged.
 * Errors: VLA_E_INVALID (other class, reps outside 1..1000, no gated layer). */
vla_status vla_profile_replay(vla_model* m, int32_t kernel_class, int32_t reps, void* stream,
                              double* ms_per_launch);

/* Matrix-core throughput probe (a measured peak beside the published one): launches
 * `blocks` workgroups of 4 wavefronts, each wavefront running iters x 4 independent
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each; the 16x16x32 form issues at about half
 * that rate on gfx950) on register operands, times it with
 * stream events and writes the achieved bf16 TFLOP/s. `out`: device float[blocks]
 * (one kept value per workgroup). Synchronises the stream. Errors: VLA_E_INVALID
 * (null pointers, blocks outside 1..65536, iters outside 1..1000000). */
vla_status vla_probe_mfma_peak(float* out, int32_t blocks, int32_t iters, void* stream,
                               double* out_tflops);

/* HBM read probe (a measured streaming ceiling beside the published 8 TB/s): reads a
 * device buffer of `bytes` (allocated, zeroed and freed by the call; a multiple of 16
 * in 1 MiB..64 GiB) `reps` times (1..100) with 16-byte loads, each workgroup reading
 * consecutive 4 KB pieces, in three grid shapes (512 workgroups x 4 pieces, 1024 x 1,
 * 1024 x 2 per iteration), each timed with stream events; writes the best GB/s.
 * Synchronises. Errors: VLA_E_INVALID, VLA_E_HIP. */
vla_status vla_probe_read_bandwidth(int64_t bytes, int32_t reps, void* stream, double* out_gbs);

/* Action expert of a pi0-style policy ("Running VLAs at Real-time Speed",
 * section 2: a vision-language prefix model plus an expert that predicts an
 * action chunk by flow matching). The expert is a decoder of its own (cfg:
 * vocab 0, all layers full, hidden <= 4096; n_layers, n_kv_heads, head_dim,
 * act_dtype and block_tokens equal to the prefix model's) whose layer l attends to the
 * prefix model's layer-l cache plus the n_actions tokens of the chunk, every
 * key visible to every chunk row (no causal mask inside the chunk). The
 * chunk's K/V live in ceil(n_actions / block_tokens) blocks popped from the
 * prefix model's free-list at creation and pushed back by destroy (destroy
 * every expert of a model before the model). Errors: VLA_E_INVALID (cfg or
 * shapes), VLA_E_NO_BLOCKS (no room in the prefix pool), VLA_E_HIP. */
vla_status vla_expert_create(vla_model* prefix, const vla_config* cfg, int32_t n_actions,
                             vla_expert** out);
/* An expert with src's config, chunk size and (shared, read-only) weights,
 * bound to `prefix` (which must satisfy vla_expert_create's conditions, e.g. a
 * sibling of src's prefix model). Errors as vla_expert_create. */
vla_status vla_expert_create_sibling(vla_model* prefix, const vla_expert* src, vla_expert** out);
void vla_expert_destroy(vla_expert* e);

/* Flow-matching Euler loop on the action chunk x (device fp32 [n_actions][hidden],
 * updated in place): for k = 0 .. n_steps-1, tau = k * dt,
 *   h = x + temb(tau)  (temb: sin(tau w_j) for j < hidden/2, then cos(tau w_j),
 *                       w_j = 2 pi / p_j, p_j = 0.004 * 1000^(j / (hidden/2 - 1)))
 *   h = the expert's layers over the chunk at positions P .. P+n_actions-1,
 *       P = the prefix model's next position (the prefix state is unchanged)
 *   x += dt * RMSNorm(h)   (the velocity: the final norm, no output projection)
 * Asynchronous on `stream`. The first call with more steps than any earlier call
 * allocates the table of the n_steps time embeddings (n_steps * hidden floats,
 * kept until destroy). Errors: VLA_E_INVALID (null x, n_steps < 1, dt <= 0). */
vla_status vla_expert_denoise(vla_expert* e, float* x, int32_t n_steps, double dt, void* stream);

/* ---- Overlapped prefix and expert streams ----------------------------------
 * "Running VLAs at Real-time Speed", section 6.1: the compute-bound prefix model
 * and the bandwidth-bound action expert run on two streams, the expert working
 * from the newest prefix K/V that is complete while the next frame's prefill
 * runs. A pipeline double-buffers the prefix state: the caller's (prefix,
 * expert) pair and a sibling pair over the same weights (created here, freed by
 * destroy). Frame t is prefilled (from scratch, positions 0..n-1) into buffer
 * t % 2 on the pipeline's prefix stream, after every action run that read that
 * buffer has finished. An action run (vla_expert_denoise on a caller chunk)
 * goes on the pipeline's expert stream and uses the newest buffer whose
 * prefill has finished, or, if none has, waits on the device for the older
 * submitted one. Both streams are created with the default priority. Calls
 * order themselves after the caller's `stream` (its inputs are ready there),
 * and the caller's stream waits for each action run, so x can be read there
 * right after vla_pipeline_act returns; embeds must stay unchanged until the
 * next vla_pipeline_sync. The caller must not use the prefix model or the
 * expert directly while the pipeline exists. One host thread at a time. */
typedef struct vla_pipeline vla_pipeline;
/* Errors: VLA_E_INVALID (NULL argument, expert not bound to prefix),
 * VLA_E_NO_BLOCKS / VLA_E_HIP (the sibling pair could not be created). */
vla_status vla_pipeline_create(vla_model* prefix, vla_expert* expert, vla_pipeline** out);
/* Synchronises both streams, then frees the sibling pair, streams and events. */
void vla_pipeline_destroy(vla_pipeline* p);
/* Prefill n rows of device embeddings ([n][hidden], act_dtype) as a new frame;
 * out_frame (nullable) receives its number (0, 1, ...). Asynchronous.
 * Errors: VLA_E_INVALID (NULL, n outside 1..max_chunk), VLA_E_HIP. */
vla_status vla_pipeline_prefill(vla_pipeline* p, const void* embeds, int32_t n, void* stream,
                                int64_t* out_frame);
/* One action run on the device fp32 chunk x (as vla_expert_denoise);
 * out_frame (nullable) receives the frame whose prefix K/V it used.
 * Errors: VLA_E_INVALID, VLA_E_STATE (no frame submitted yet), VLA_E_HIP. */
vla_status vla_pipeline_act(vla_pipeline* p, float* x, int32_t n_steps, double dt, void* stream,
                            int64_t* out_frame);
/* Wait for both streams. */
vla_status vla_pipeline_sync(vla_pipeline* p);
/* Counts: prefills, action runs, and action runs that used a frame older than
 * the newest one submitted (each pointer nullable). */
vla_status vla_pipeline_stats(const vla_pipeline* p, int64_t* prefills, int64_t* acts,
                              int64_t* acts_on_older);

/* ---- Reconciliation on a second state ---------------------------------------
 * "CSR: Infinite-Horizon Real-Time Policies with Massive Cached State
 * Representations", section III-E and Appendix D: after evictions, a second
 * resource re-prefills the kept state while the first keeps serving, catches up
 * on the chunks that arrived meanwhile, and the two swap roles. Here the second
 * resource is a sibling model (same weights, its own KV pool) on a second
 * stream of the same GPU. Every frame is prefilled through the reconciler,
 * which logs its input (host token ids are copied; device embeddings are copied
 * into a log of 2 x max_frames chunks, allocated on first use), so that the
 * spare model can recompute the kept frames' K/V from scratch at contiguous
 * positions. Frames are named by reconciler ids (0, 1, ... in arrival order),
 * which stay valid across swaps. The caller decodes and scores on
 * vla_asr_model() but prefills and evicts only through the reconciler, and
 * passes one stream to every call. The spare stream has the default priority. */
typedef struct vla_asr vla_asr;
/* primary must hold no frame yet. Errors: VLA_E_INVALID, VLA_E_STATE (primary
 * not empty), VLA_E_HIP. */
vla_status vla_asr_create(vla_model* primary, vla_asr** out);
/* Waits for the spare stream, frees the sibling model, the log and the stream.
 * The caller's model stays valid (it may be the spare at that point). */
void vla_asr_destroy(vla_asr* a);
/* The model serving now (the primary, or the sibling after an odd number of swaps). */
vla_model* vla_asr_model(const vla_asr* a);
/* vla_prefill_chunk on the serving model, logging the input; out_id (nullable)
 * receives the frame's reconciler id. Errors: as vla_prefill_chunk, and
 * VLA_E_NO_BLOCKS when the embeddings log is full. */
vla_status vla_asr_prefill(vla_asr* a, const int32_t* tokens, const void* embeds, int32_t n,
                           void* stream, int64_t* out_id);
/* vla_kv_evict on the serving model (and on the spare, if it already holds the
 * frame); out_id / out_score (nullable) receive the frame and its score. */
vla_status vla_asr_evict(vla_asr* a, int32_t policy, int32_t layer, void* stream, int64_t* out_id,
                         double* out_score);
/* Start re-prefilling every resident frame, in arrival order, into the emptied
 * spare model on the spare stream (after the work already on `stream`).
 * Errors: VLA_E_STATE (one is already running). */
vla_status vla_asr_reconcile_begin(vla_asr* a, void* stream);
/* Catch the spare up on frames prefilled since, then, if all of its work has
 * finished, swap: *swapped = 1 and the spare serves from now on (`stream` is
 * ordered after its work); else *swapped = 0 and nothing changes. Never waits
 * on the host. Errors: VLA_E_STATE (no reconciliation running). */
vla_status vla_asr_try_swap(vla_asr* a, void* stream, int32_t* swapped);
/* Wait for the spare stream. */
vla_status vla_asr_sync(vla_asr* a);
/* The resident frames' reconciler ids in arrival order (the first cap); n_out: their count. */
vla_status vla_asr_frames(const vla_asr* a, int64_t* ids, int32_t cap, int32_t* n_out);
/* Counts (each pointer nullable): reconciliations begun, swaps, frames re-prefilled
 * by the spare, and whether a reconciliation is running. */
vla_status vla_asr_stats(const vla_asr* a, int64_t* reconciliations, int64_t* swaps,
                         int64_t* frames_replayed, int32_t* reconciling);

/* Host-only LIFO block pool ("Rebuilding Kshipra Around Memory", section 1):
 * the free-list starts as [0 .. n-1] so the first pop returns n-1; released
 * blocks are pushed in the order given and popped first. The model uses the
 * same pool. No HIP calls; usable without a GPU. */
vla_status vla_pool_create(int32_t num_blocks, vla_pool** out);
void vla_pool_destroy(vla_pool* p);
/* Pop n blocks into out[n]; VLA_E_NO_BLOCKS (pool unchanged) if fewer are free. */
vla_status vla_pool_alloc(vla_pool* p, int32_t n, int32_t* out);
/* Push n blocks in the order given; VLA_E_INVALID for an id out of range or already free. */
vla_status vla_pool_release(vla_pool* p, const int32_t* blocks, int32_t n);
int32_t vla_pool_free_count(const vla_pool* p);
/* The pool's free-list bottom first (out[n-1] is popped next), as vla_kv_free_list. */
vla_status vla_pool_free_list(const vla_pool* p, int32_t* out, int32_t cap, int32_t* n_out);

/* ---- Admission control of a real-time reasoning cycle ------------------------
 * ("Can an LLM Forget the Right Things?", section 4: refuse to start a chunk
 * whose estimated cost does not fit the rest of the cycle's deadline.) Host-only;
 * no HIP calls; usable without a GPU. A handle is single-threaded.
 *   estimate = ema_prefill_per_token * prefill_tokens + ema_decode_per_token * decode_tokens
 *   admit    = no measurement recorded yet, or estimate <= deadline - elapsed - margin
 *   ema     <- (1 - alpha) * ema + alpha * measured   (prefill and decode separately;
 *              the first measurement initialises both)
 * A refused cycle is the caller's fallback (e.g. repeat the last action). A cycle
 * that ends after the deadline counts as a deadline miss. */
typedef struct vla_admission vla_admission;
typedef struct {
  double deadline_ms;       /* cycle deadline, ms (> 0; 33 in the page's runtime) */
  double safety_margin_ms;  /* kept free of estimated work, ms (>= 0; 2 on the page) */
  double ema_alpha;         /* weight of a new measurement, (0, 1] (0.2 on the page) */
  int32_t prefill_tokens;   /* tokens one admitted chunk prefills (>= 1) */
  int32_t decode_tokens;    /* decode steps one admitted chunk runs (>= 0) */
} vla_admission_config;
typedef struct {
  int64_t cycles;           /* cycles ended with vla_admission_cycle_end */
  int64_t admitted;         /* ... whose chunk was admitted */
  int64_t refused;          /* ... that fell back */
  int64_t deadline_misses;  /* ... that ended after the deadline */
  double worst_cycle_ms;    /* longest cycle */
  double last_overrun_ms;   /* overrun of the latest missed cycle (0 if none) */
  double ema_prefill_ms_per_token;
  double ema_decode_ms_per_token;
  int32_t has_sample;       /* 0 until the first vla_admission_record */
} vla_admission_stats;
/* Errors: VLA_E_INVALID (null out, sizes or rates outside the ranges above). */
vla_status vla_admission_create(const vla_admission_config* cfg, vla_admission** out);
void vla_admission_destroy(vla_admission* a);
/* Start a cycle: the cycle clock (steady clock) restarts. */
vla_status vla_admission_cycle_begin(vla_admission* a);
/* Milliseconds since the cycle began. */
vla_status vla_admission_elapsed_ms(const vla_admission* a, double* out_ms);
/* The decision for a cycle `elapsed_ms` into its budget: *out_admit 1 or 0, and
 * the current estimate (ms, nullable). */
vla_status vla_admission_should_admit(const vla_admission* a, double elapsed_ms,
                                      int32_t* out_admit, double* out_estimate_ms);
/* Feed the measured cost of a finished chunk: prefill_ms over prefill_tokens (>= 1)
 * and decode_ms over decode_tokens (>= 1). Errors: VLA_E_INVALID (token counts < 1,
 * negative or non-finite times). */
vla_status vla_admission_record(vla_admission* a, double prefill_ms, int32_t prefill_tokens,
                                double decode_ms, int32_t decode_tokens);
/* End the cycle: count it as admitted (1) or refused (0), and as a deadline miss when
 * its duration on the cycle clock exceeds the deadline; the duration goes to
 * *out_cycle_ms (nullable). */
vla_status vla_admission_cycle_end(vla_admission* a, int32_t admitted, double* out_cycle_ms);
/* Block until the cycle's deadline (cycle start + deadline): sleep through all but
 * the last millisecond, then spin (same page, section 3: sleep is only accurate to
 * about a millisecond). Returns at once when the deadline has passed. */
vla_status vla_admission_sleep_until_deadline(const vla_admission* a);
vla_status vla_admission_stats_out(const vla_admission* a, vla_admission_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* VLA_H */

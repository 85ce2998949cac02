// Host-side launch interface of the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vla {

// Kernel timing hook. While the runtime profiles a kernel class it points
// g_prof_sink at its event pool; every launch made through launch_k() then
// carries a start/stop event pair in its dispatch (hipExtLaunchKernelGGL), so
// the measured span is the kernel's own execution.
struct ProfSink;
extern thread_local ProfSink* g_prof_sink;
bool prof_take_pair(ProfSink* sink, hipEvent_t* start, hipEvent_t* stop);

template <typename... KArgs, typename... Args>
inline void launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds,
                     hipStream_t s, Args... args) {
  hipEvent_t e0, e1;
  if (g_prof_sink && prof_take_pair(g_prof_sink, &e0, &e1)) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, e0, e1, 0u, static_cast<KArgs>(args)...);
    return;
  }
  kernel<<<grid, block, lds, s>>>(static_cast<KArgs>(args)...);
}

enum Dtype { DT_F32 = 0, DT_BF16 = 1 };

// Physical weight layouts (all generated in place from the counter-based generator).
//  PLAIN   row-major [rows][cols], one stream.
//  QKV     rows = (Hq + 2 Hkv) d: q heads, then k heads, then v heads; inside each
//          head the two members (j, j + d/2) of a RoPE pair sit on adjacent rows
//          2j and 2j+1, so one output tile holds both halves of a rotation.
//  GATEUP  rows = 2F in blocks of 32: 16 gate rows f..f+15 then the 16 matching up
//          rows, so one 32-column tile holds both operands of the gated product.
enum Layout { LAYOUT_PLAIN = 0, LAYOUT_QKV = 1, LAYOUT_GATEUP = 2 };

// Paged KV pool geometry. Inside a block (l, b, h) K is split along the head
// dimension into 64-byte chunks of kc = 2^kcs elements, each stored for all bt
// keys in turn: element (l, b, h, s, i) lives at
// ((l*nb + b)*hkv + h)*bt*d + (i/kc)*bt*kc + s*kc + i%kc. A matrix-core K operand
// of 16 keys x 64 bytes is then one contiguous 1 KB run (whole 128-byte lines per
// load). V is stored transposed inside a block, element (l, b, h, s, i) at
// (((l*nb + b)*hkv + h)*d + i)*bt + s, so that a 4-key run of one head dimension
// is contiguous (the operand order of the P*V matrix-core product).
struct KvGeom {
  int L, nb, hkv, bt, d;
  int kcs;  // log2 of the K chunk's elements: 4 for fp32, 5 for bf16
  __host__ __device__ size_t kidx(int l, int b, int h, int s, int i) const {
    return ((((size_t)l * nb + b) * hkv + h) * d + (size_t)((i >> kcs) << kcs)) * bt +
           ((size_t)s << kcs) + (i & ((1 << kcs) - 1));
  }
  __host__ __device__ size_t vidx(int l, int b, int h, int s, int i) const {
    return ((((size_t)l * nb + b) * hkv + h) * d + i) * bt + s;
  }
};

// Where the rows of the current pass go: row t (0..n-1) is the token at
// absolute position pos0 + t, stored at logical chunk slot cslot0 + t of the
// blocks starting at logical block cb0.
struct FwdCtx {
  int layer = 0;
  const float2* rope = nullptr;      // [n][d/2] (cos, sin) of row t's angles (launch_rope_table)
  void* kpool = nullptr;
  void* vpool = nullptr;
  KvGeom g{};
  const int* blk_table = nullptr;    // logical block -> physical block
  int cb0 = 0;
  int cslot0 = 0;
  void* qbuf = nullptr;              // [n][Hq][d] activations
  int hq = 0;
};

enum Epi { EPI_STORE = 0, EPI_RESID = 1, EPI_QKV = 2, EPI_SWIGLU = 3, EPI_HEAD = 4,
           EPI_PARTIAL = 5 };

enum WeightFmt { WF_ACT = 0, WF_INT4 = 1 };  // weights in the activation type / INT4 g128

struct GemmArgs {
  const void* A = nullptr;  // [M][K] activations
  // bf16 only: the low part of the activations, A_lo = bf16(a - A) for the exact
  // value a whose bf16 rounding is A; when set the product is (A + A_lo) W^T, i.e.
  // the input carries about 16 significant bits (q/k/v and output projections)
  const void* A_lo = nullptr;
  const void* W = nullptr;  // [N][K] weights (physical layout); INT4: codes then scales
  int wf = WF_ACT;
  int M = 0, N = 0, K = 0;
  int epi = EPI_STORE;
  int glu = 0;              // SWIGLU epilogue: 0 silu(gate) * up, 1 gelu(gate) * up
  void* C = nullptr;        // STORE [M][N]; RESID fp32 x [M][N] (+=); SWIGLU [M][N/2]
  FwdCtx ctx;
  // bf16 RESID: split-K partials (fp32, [splits][M][N]) reduced by a second
  // kernel that adds them to x and, when norm_out is set, writes
  // norm_out = RMSNorm(x) (weights norm_g, epsilon eps) for the next projection
  float* ws = nullptr;
  size_t ws_elems = 0;
  void* norm_out = nullptr;
  void* norm_out_lo = nullptr;  // bf16: also the low part of norm_out (see A_lo)
  const float* norm_g = nullptr;
  float eps = 0.f;
  // INT4 weights: per-(128-column group, row) sums of the bf16 activations, fp32,
  // [K/128][sum_ld] (a_sum: this product's input, read instead of summing it with
  // the matrix cores; norm_sum: written with norm_out, for the next projection;
  // N % 128 == 0)
  const float* a_sum = nullptr;
  float* norm_sum = nullptr;
  int sum_ld = 0;
};

struct GemvArgs {
  const void* x = nullptr;      // [K] input row: the fp32 residual when norm_g is set,
                                // else activations in the weight type
  const float* norm_g = nullptr;  // non-null: RMSNorm the input first
  float eps = 0.f;
  const void* W = nullptr;      // [N][K]; INT4: packed codes [N][K/2] then scales [K/128][N]
  int wf = WF_ACT;
  int N = 0, K = 0;
  int epi = EPI_STORE;
  int glu = 0;                  // SWIGLU epilogue: 0 silu(gate) * up, 1 gelu(gate) * up
  void* out = nullptr;          // RESID fp32 x[N] (+=); SWIGLU act[N/2]; HEAD logits fp32[N]
  unsigned long long* argmax_part = nullptr;  // HEAD: one key per workgroup
  FwdCtx ctx;
  // RESID with part_o set: the input row is the one-token decode attention
  // output, given as its split partials (launch_attention with a fold request),
  // part_o [unit][16][hd], part_ml [unit][2][16], unit = kv head * splits + split;
  // grp query heads per KV head, K = heads * hd
  const float* part_o = nullptr;
  const float* part_ml = nullptr;
  int splits = 0, grp = 0, hd = 0;
};

// limits of the decode attention merge folded into the output projection
constexpr int kFoldMaxSplits = 16;
constexpr int kFoldMaxHeads = 16;

struct AttnArgs {
  const void* q = nullptr;   // [n][Hq][d]
  void* out = nullptr;       // [n][Hq][d]
  void* out_lo = nullptr;    // bf16, nullable: the low part of out, bf16(exact - out) (see A_lo)
  const void* kpool = nullptr;
  const void* vpool = nullptr;
  KvGeom g{};
  int layer = 0;
  const int* blk_table = nullptr;  // logical -> physical
  const int* blk_ntok = nullptr;   // valid tokens per logical block
  int nlb = 0;                     // logical blocks visible to this pass
  int last_ntok = 0;               // valid tokens of logical block nlb-1 (overrides the table)
  int cb0 = 0, cslot0 = 0;         // first token of the chunk (its own keys)
  int causal = 1;                  // 1: the chunk's own keys causal; 0: all visible
  int n = 0, hq = 0;
  int splits = 1;                  // chosen by launch_attention
  float* part_o = nullptr;         // split partials, part_rows rows of d fp32
  float* part_ml = nullptr;        // part_rows x 2 fp32 (running max, sum)
  int part_rows = 0;
  float scale = 1.f;
};

// One decode step in one launch: the embedding row and RoPE table, then every
// layer's q/k/v projection, attention, output projection, gated projection and
// down projection, each phase spread over the persistent workgroups and separated
// from the next by a device-scope barrier. The projections and the attention take
// their per-layer weights from wtab and their layer index from the loop; everything
// else is in the templates below.
struct DecodeStepArgs {
  // first phase
  int token = 0;                              // token id, or ...
  const unsigned long long* token_key = nullptr;  // ... the previous argmax key (device)
  const void* E = nullptr;
  float* x = nullptr;
  int H = 0;
  int64_t pos = 0;
  const double* inv_freq = nullptr;
  int half = 0;
  float2* rope = nullptr;
  // per-layer phases (W and the layer are set per layer)
  GemvArgs qkv, o, gu, dn;
  AttnArgs at;
  const void* const* wtab = nullptr;          // [L][4]: q/k/v, O, gate/up, down weights
  int n_layers = 0;
  int ng_qkv = 0, ng_o = 0, ng_gu = 0, ng_dn = 0;   // row groups of each projection
  int vg_qkv = 0, vg_o = 0, vg_gu = 0, vg_dn = 0;   // their virtual workgroups
  // barriers (grouped by XCD, decode_step.hip): the state words (kBarStateWords,
  // zeroed when allocated; the error flag is the first word), the launch's sequence
  // number (it uses state set seq & 1 and clears the other for the next launch) and
  // an offset added to every generation target (0; 1 << 40 makes every barrier
  // unreachable, a test of the error path). A wait gives up after spin_limit polls (or
  // when another workgroup gave up), sets the error flag and ends the workgroup.
  unsigned long long* bar = nullptr;
  int seq = 0;
  unsigned long long gen_off = 0;
  int spin_limit = 0;
};
// barrier state: 256-byte lines of 32 words; line 0 the error flag, then two sets of
// 20 lines (2 registration words, 8 XCD arrival counters, the top counter, 8 XCD
// release flags, the generation)
constexpr int kBarLineWords = 32;
constexpr int kBarSetLines = 20;
constexpr int kBarStateWords = (1 + 2 * kBarSetLines) * kBarLineWords;
// shapes with a persistent decode-step kernel (chunks per lane of the q/k/v, O and
// gated projections; rows per wavefront, chunks and K split of the down projection)
enum DecodeShape { DSHAPE_NONE = -1, DSHAPE_C3_3_3_D1_5_4 = 0, DSHAPE_C1_2_1_D2_1_1 = 1 };
// persistent workgroups of the shape's kernel (all resident at once), 0 if unknown
int decode_step_grid(int shape);
hipError_t launch_decode_step(const DecodeStepArgs& p, int shape, int grid, hipStream_t s);
// nbar barriers of that kind over `grid` resident workgroups (bar: kBarStateWords words,
// zeroed before the first launch; seq: 0, 1, ... over consecutive launches on that
// state; scratch: grid * 256 floats)
hipError_t launch_barrier_probe(unsigned long long* bar, float* scratch, int grid, int nbar,
                                int seq, int spin_limit, hipStream_t s);
int barrier_probe_max_grid();

// ---- launches (all return the launch status) ----
hipError_t launch_init_weight(void* out, int dt, int layout, int64_t rows, int64_t cols,
                              uint64_t seed, uint64_t sa, uint64_t sb, uint64_t sc, int hq,
                              int hkv, int d, double stdv, hipStream_t s);
// INT4 group-128 tensors: packed codes [rows][cols/2] then fp16 scales [cols/128][rows]
hipError_t launch_init_weight_w4(void* out, int layout, int64_t rows, int64_t cols, uint64_t seed,
                                 uint64_t sa, uint64_t sb, uint64_t sc, int hq, int hkv, int d,
                                 double stdv, hipStream_t s);
hipError_t launch_weight_logical_w4(const void* phys, float* out, int layout, int which,
                                    int64_t rows, int64_t cols, int64_t prows, int hq, int hkv,
                                    int d, hipStream_t s);
hipError_t launch_weight_logical(const void* phys, void* out, int dt, int layout, int which,
                                 int64_t rows, int64_t cols, int hq, int hkv, int d,
                                 hipStream_t s);
hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t s);
// matrix-core throughput probe: `blocks` workgroups of 4 wavefronts, each wavefront
// iters x 4 bf16 MFMAs of 32768 FLOP; out[blocks] receives one value per workgroup
hipError_t launch_mfma_peak(float* out, int blocks, int iters, hipStream_t s);
// HBM read probe over `bytes` (a multiple of 16) at p, `unroll` (1, 2, 4) consecutive 4 KB
// pieces per workgroup and iteration; out: blocks * 256 words
hipError_t launch_read_probe(const void* p, int64_t bytes, uint32_t* out, int blocks, int unroll,
                             hipStream_t s);
// (cos, sin) of pos * inv_freq[j] for rows t = 0..n-1 at positions pos0 + t: the
// angle is formed in fp64 and reduced to [-pi, pi] in fp64, then fp32 sin/cos
hipError_t launch_rope_table(int64_t pos0, int n, const double* inv_freq, int half,
                             float2* tab, hipStream_t s);
// x: the fp32 residual rows [n][H]; E and u in the activation type
hipError_t launch_to_f32(const void* in, float* out, int64_t n, int dt, hipStream_t s);
// action expert: the time-embedding rows of tau_k = k * dt (k < n_steps), and the
// boundary of two flow-matching iterations: optionally x += dt * RMSNorm(h), then,
// if temb is given, h = x + temb and u (u_lo) = RMSNorm(h) (H a multiple of 4, <= 4096)
hipError_t launch_flow_temb(float* temb, int n_steps, int H, double dt, hipStream_t s);
hipError_t launch_flow_step(float* xa, float* h, const float* temb, const float* g, void* u,
                            void* u_lo, int rows, int H, float eps, float dt, bool euler, int dtype,
                            hipStream_t s);
// one decode row: the token's embedding row (token_key non-null: the token is the
// argmax key's id) and the RoPE table of position pos, in one launch
hipError_t launch_embed_rope1(int token_scalar, const unsigned long long* token_key, const void* E,
                              void* x, int H, int dt, int64_t pos, const double* inv_freq, int half,
                              float2* tab, hipStream_t s);
hipError_t launch_embed(const int* tokens, int token_scalar, const unsigned long long* token_key,
                        int n, const void* E, void* x, int H, int dt,
                        unsigned long long* reset_cell, hipStream_t s);
// u = RMSNorm(x) rows; bf16: u_lo (nullable) receives the low part bf16(exact - u)
hipError_t launch_rmsnorm(const void* x, const float* g, void* u, void* u_lo, int rows, int H,
                          float eps,
                          int dt, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& a, int dt, hipStream_t s);
hipError_t launch_gemv(const GemvArgs& a, int dt, hipStream_t s, int* grid_out);
hipError_t launch_argmax_final(const unsigned long long* part, int nparts,
                               unsigned long long* result, hipStream_t s);
// fold_splits non-null (one-token decode): when the key splits would need the
// merge kernel and their count is within kFoldMaxSplits, the merge is left to
// the consumer and *fold_splits receives the split count (the partials are in
// a.part_o / a.part_ml); otherwise the output is written as usual and
// *fold_splits is 0.
hipError_t launch_attention(const AttnArgs& a, int dt, hipStream_t s, int* fold_splits = nullptr);
hipError_t launch_kv_scatter(const void* k, const void* v, int n, void* kpool, void* vpool,
                             KvGeom g, const int* blk_table, int cb0, int dt, hipStream_t s);
hipError_t launch_kv_gather(const void* kpool, const void* vpool, KvGeom g, int layer,
                            const int* blk_table, const int* blk_ntok, const int* tok_base,
                            int nlb, void* k_out, void* v_out, int dt, hipStream_t s);
hipError_t launch_meankeys(const void* kpool, KvGeom g, const int* blk_table,
                           const int* fr_blk0, const int* fr_nblk, const int* fr_ntok,
                           const int* fr_slot, int nframes, int layer0, int nlayers,
                           double* table, int max_frames, int dt, hipStream_t s);
hipError_t launch_score(const double* table_layer, const int* fr_slot, int nframes, int D,
                        double* m_out, double* result, hipStream_t s);
// adjacent-pair scoring: s[i] = cos(frame i, frame i + 1), then the argmax over the
// nframes - 1 pairs (ties to the first pair) into result[0] (pair index), result[1]
hipError_t launch_score_adjacent(const double* table_layer, const int* fr_slot, int nframes, int D,
                                 double* s_out, double* result, hipStream_t s);
// scoring of a dense fp64 table [nframes][D] (rows in frame order) with the
// per-frame scores in a library-owned static device array (no allocation);
// writes the winner's row index and score to device memory
constexpr int kScoreNoAllocMaxFrames = 4096;
hipError_t launch_score_noalloc(const double* table, int nframes, int D, int* out_idx,
                                double* out_score, hipStream_t s);

}  // namespace vla

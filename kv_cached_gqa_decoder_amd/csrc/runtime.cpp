// Host runtime behind the C ABI of include/vla.h: model state, frame registry,
// block tables, and the launch sequences of prefill, decode and scoring.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <memory>
#include <string>
#include <vector>

#include "../../include/vla.h"
#include "admission.hpp"
#include "block_pool.hpp"
#include "kernels.hpp"

using namespace vla;

namespace {

thread_local std::string g_err;

struct Err {
  vla_status st;
  std::string msg;
};

#define HIPCHK(expr)                                                                      \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      throw Err{VLA_E_HIP, std::string(#expr) + " failed: " + hipGetErrorString(e_)};     \
  } while (0)

[[noreturn]] void raise(vla_status st, const std::string& msg) { throw Err{st, msg}; }

constexpr int kPartRows = 131072;  // attention split partials capacity (query rows x splits)
constexpr int kGemmSplitsMax = 16; // split-K partial capacity of the prefill residual projections
constexpr int kArgmaxParts = 2048; // head GEMV workgroups at most

struct Segment {
  bool frame = true;
  int frame_id = -1;
  int64_t start_pos = 0;
  int ntok = 0;
  int slot = -1;               // mean-key table row (frames only)
  std::vector<int> blocks;
};

// pinned host staging buffer for uploads; an event guards its reuse
struct Staging {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};

}  // namespace

struct vla_pool {
  BlockPool p;
};

struct vla_admission {
  Admission a;
};

namespace vla {
// event pairs of the profiled kernel launches since the last enable
struct ProfSink {
  std::vector<hipEvent_t> ev;
  int used = 0;     // events handed out (two per kernel launch)
  int calls = 0;    // profiled calls (one call may launch several kernels)
};
thread_local ProfSink* g_prof_sink = nullptr;
bool prof_take_pair(ProfSink* s, hipEvent_t* a, hipEvent_t* b) {
  while ((int)s->ev.size() < s->used + 2) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return false;
    s->ev.push_back(e);
  }
  *a = s->ev[s->used];
  *b = s->ev[s->used + 1];
  s->used += 2;
  return true;
}
}  // namespace vla

struct vla_model;
struct vla_expert {
  vla_model* m = nullptr;        // the expert's weights and scratch (pool borrowed)
  vla_model* prefix = nullptr;   // the model whose cache it reads and writes into
  std::vector<int> reserved;     // prefix-pool blocks holding the action chunk's K/V
  int n_actions = 0;
  int* d_view = nullptr;         // block list of a pass: blk | ntok (num_blocks each)
  Staging st_view;
  float* temb = nullptr;         // time-embedding rows of one denoise call
  int temb_cap = 0;              // rows it holds
  // a denoise loop captured as a graph (replayed while these arguments stay the same)
  struct GraphKey {
    const float* x = nullptr;
    int n_steps = 0, nb = 0, last_ntok = 0, cb0 = 0;
    double dt = 0.0;
    int64_t pos = 0;
    bool operator==(const GraphKey& o) const {
      return x == o.x && n_steps == o.n_steps && nb == o.nb && last_ntok == o.last_ntok &&
             cb0 == o.cb0 && dt == o.dt && pos == o.pos;
    }
  };
  hipGraphExec_t gexec = nullptr;
  GraphKey gkey;
};

// device memory of one set of weights: shared by every model built over it (sibling
// models and experts) and freed with the last of them
struct WeightStore {
  int dev = 0;
  std::vector<void*> allocs;
  ~WeightStore() {
    (void)hipSetDevice(dev);
    for (void* p : allocs) (void)hipFree(p);
  }
};

struct vla_model {
  vla_config cfg{};
  int dev = 0;
  int dt = DT_BF16;
  int wf = WF_ACT;   // projection weights: activation type or INT4 group-128
  size_t esz = 2;
  KvGeom geom{};

  // weights (physical layouts, see kernels.hpp), in a store this model may share
  std::shared_ptr<WeightStore> wstore;
  void* embed = nullptr;
  void* head = nullptr;
  std::vector<void*> wqkv, wo, wgu, wdown;
  float* norm_ones = nullptr;   // all RMSNorm weights are 1
  double* inv_freq = nullptr;
  float2* rope_tab = nullptr;   // (cos, sin) of the current pass's rows, [max_chunk][d/2]

  // cache
  void* kpool = nullptr;
  void* vpool = nullptr;
  double* meankeys = nullptr;   // [L][max_frames][Hkv*d]

  // scratch
  void* x = nullptr;
  void* u = nullptr;
  void* u_lo = nullptr;         // bf16 weights, logits out: low part of the q/k/v input rows
  void* ao_lo = nullptr;        // ... and of the attention output rows (see GemmArgs)
  float* usum = nullptr;        // INT4 weights: per-(128-group, row) sums of u (see GemmArgs)
  int usum_ld = 0;
  void* qbuf = nullptr;
  void* ao = nullptr;
  void* act = nullptr;
  float* logits = nullptr;
  unsigned long long* amax_part = nullptr;
  unsigned long long* amax_res = nullptr;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  float* gemm_ws = nullptr;     // split-K partials of the residual projections
  size_t gemm_ws_elems = 0;
  int* d_meta = nullptr;        // blk | ntok | tokbase (nb each) | fr_slot | fr_blk0 | fr_nblk | fr_ntok
  int* d_tokens = nullptr;
  double* d_score_m = nullptr;
  double* d_score_res = nullptr;
  Staging st_meta, st_tok, st_read;

  // host state
  BlockPool pool;
  std::vector<Segment> segs;
  std::vector<int> free_slots;
  int64_t next_pos = 0;
  int next_frame_id = 0;
  bool meta_dirty = true;
  bool have_logits = false;

  // persistent decode step
  int ds_shape = DSHAPE_NONE;   // its kernel shape for this model, DSHAPE_NONE if none
  int ds_grid = 0;              // resident workgroups of that kernel (0: not queried yet)
  const void** d_wtab = nullptr;          // [L][4] weight pointers (device)
  unsigned long long* d_bar = nullptr;    // barrier state (kBarStateWords; word 0 the error flag)
  int ds_seq = 0;                         // persistent launches since the state was zeroed
  bool ds_check = false;                  // a persistent step ran since the last check
  bool last_persistent = false;
  int opt_persistent = 0;
  int opt_spin_limit = 1 << 20;
  int opt_unreachable = 0;

  // profiling
  int prof_cls = VLA_K_NONE;
  ProfSink prof;

  std::vector<void*> allocs;

  int* d_blk() const { return d_meta; }
  int* d_ntok() const { return d_meta + cfg.num_blocks; }
  int* d_tokbase() const { return d_meta + 2 * cfg.num_blocks; }
  int* d_fr_slot() const { return d_meta + 3 * cfg.num_blocks; }
  int* d_fr_blk0() const { return d_fr_slot() + cfg.max_frames; }
  int* d_fr_nblk() const { return d_fr_blk0() + cfg.max_frames; }
  int* d_fr_ntok() const { return d_fr_nblk() + cfg.max_frames; }
  size_t meta_ints() const { return 3 * (size_t)cfg.num_blocks + 4 * (size_t)cfg.max_frames; }
};

namespace {

template <typename F>
vla_status guarded(F&& f) {
  try {
    f();
    g_err.clear();
    return VLA_OK;
  } catch (const Err& e) {
    g_err = e.msg;
    return e.st;
  } catch (const std::exception& e) {
    g_err = e.what();
    return VLA_E_STATE;
  } catch (...) {
    g_err = "unknown error";
    return VLA_E_STATE;
  }
}

void* dalloc(vla_model* m, size_t bytes) {
  void* p = nullptr;
  HIPCHK(hipMalloc(&p, bytes < 256 ? 256 : bytes));
  m->allocs.push_back(p);
  return p;
}
// weight memory: in the model's weight store
void* walloc(vla_model* m, size_t bytes) {
  void* p = nullptr;
  HIPCHK(hipMalloc(&p, bytes < 256 ? 256 : bytes));
  m->wstore->allocs.push_back(p);
  return p;
}

void staging_init(Staging& s, size_t bytes) {
  HIPCHK(hipHostMalloc(&s.host, bytes, hipHostMallocDefault));
  s.cap = bytes;
  HIPCHK(hipEventCreateWithFlags(&s.ev, hipEventDisableTiming));
}
void staging_free(Staging& s) {
  if (s.ev) (void)hipEventSynchronize(s.ev);
  if (s.host) (void)hipHostFree(s.host);
  if (s.ev) (void)hipEventDestroy(s.ev);
  s = Staging{};
}
void* staging_acquire(Staging& s) {
  if (s.pending) HIPCHK(hipEventSynchronize(s.ev));
  s.pending = false;
  return s.host;
}
void staging_upload(Staging& s, void* dst, size_t bytes, hipStream_t st) {
  HIPCHK(hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, st));
  HIPCHK(hipEventRecord(s.ev, st));
  s.pending = true;
}

// ---- profiling: start/stop events carried by the profiled kernels' dispatches ----
#define LAUNCH(m, cls, st, expr)                                     \
  do {                                                               \
    const bool on_ = (m)->prof_cls == (cls) && (cls) != VLA_K_NONE; \
    if (on_) {                                                       \
      g_prof_sink = &(m)->prof;                                      \
      ++(m)->prof.calls;                                             \
    }                                                                \
    const hipError_t launch_err_ = (expr);                           \
    g_prof_sink = nullptr;                                           \
    HIPCHK(launch_err_);                                             \
  } while (0)

// ---- bookkeeping ----
int bt_of(const vla_model* m) { return m->cfg.block_tokens; }

int logical_blocks(const vla_model* m) {
  int n = 0;
  for (const auto& s : m->segs) n += (int)s.blocks.size();
  return n;
}
int resident_tokens(const vla_model* m) {
  int n = 0;
  for (const auto& s : m->segs) n += s.ntok;
  return n;
}
int n_frames(const vla_model* m) {
  int n = 0;
  for (const auto& s : m->segs) n += s.frame ? 1 : 0;
  return n;
}
// logical index of segment i's first block
int seg_blk0(const vla_model* m, size_t i) {
  int n = 0;
  for (size_t k = 0; k < i; ++k) n += (int)m->segs[k].blocks.size();
  return n;
}

// rebuild and upload the logical block table and the frame list
void sync_meta(vla_model* m, hipStream_t st) {
  if (!m->meta_dirty) return;
  const int nb = m->cfg.num_blocks, mf = m->cfg.max_frames, bt = bt_of(m);
  int* h = (int*)staging_acquire(m->st_meta);
  memset(h, 0, m->meta_ints() * sizeof(int));
  int* blk = h;
  int* ntok = h + nb;
  int* base = h + 2 * nb;
  int* fslot = h + 3 * nb;
  int* fblk0 = fslot + mf;
  int* fnblk = fblk0 + mf;
  int* fntok = fnblk + mf;
  int lb = 0, tok = 0, f = 0;
  for (const auto& s : m->segs) {
    if (s.frame) {
      fslot[f] = s.slot;
      fblk0[f] = lb;
      fnblk[f] = (int)s.blocks.size();
      fntok[f] = s.ntok;
      ++f;
    }
    for (size_t i = 0; i < s.blocks.size(); ++i) {
      blk[lb] = s.blocks[i];
      ntok[lb] = std::min(bt, s.ntok - (int)i * bt);
      base[lb] = tok;
      tok += ntok[lb];
      ++lb;
    }
  }
  staging_upload(m->st_meta, m->d_meta, m->meta_ints() * sizeof(int), st);
  m->meta_dirty = false;
}

int last_block_ntok(const vla_model* m) {
  for (auto it = m->segs.rbegin(); it != m->segs.rend(); ++it)
    if (!it->blocks.empty()) return it->ntok - ((int)it->blocks.size() - 1) * bt_of(m);
  return 0;
}

// the blocks a pass reads: logical block list (device), valid tokens per block,
// and whether the pass's own keys are causal
struct KvView {
  const int* blk = nullptr;
  const int* ntok = nullptr;
  int nlb = 0;
  int last_ntok = 0;
  int causal = 1;
};

KvView model_view(vla_model* m) {
  KvView v;
  v.blk = m->d_blk();
  v.ntok = m->d_ntok();
  v.nlb = logical_blocks(m);
  v.last_ntok = last_block_ntok(m);
  return v;
}

FwdCtx make_ctx(vla_model* m, const KvView& v, int layer, int cb0, int cslot0) {
  FwdCtx c;
  c.layer = layer;
  c.rope = m->rope_tab;
  c.kpool = m->kpool;
  c.vpool = m->vpool;
  c.g = m->geom;
  c.blk_table = v.blk;
  c.cb0 = cb0;
  c.cslot0 = cslot0;
  c.qbuf = m->qbuf;
  c.hq = m->cfg.n_heads;
  return c;
}

// one-token gated projection of layer l: the normalised residual row -> the
// FFN activations (decode, and its timing replay)
GemvArgs decode_gateup_args(vla_model* m, int l) {
  const vla_config& c = m->cfg;
  GemvArgs gu;
  gu.x = m->x;
  gu.norm_g = m->norm_ones;
  gu.eps = c.rms_eps;
  gu.W = m->wgu[l];
  gu.wf = m->wf;
  gu.N = 2 * c.ffn;
  gu.K = c.hidden;
  gu.epi = EPI_SWIGLU;
  gu.glu = c.ffn_kind == VLA_GEGLU ? 1 : 0;
  gu.out = m->act;
  return gu;
}

// the per-layer launches of one pass over n rows whose K/V go to logical slots
// (cb0, cslot0 ...); rows = prefill chunk (n >= 1, matrix path) or decode (GEMV path)
void run_layers(vla_model* m, const KvView& view, int n, int64_t pos0, int cb0, int cslot0,
                bool decode, hipStream_t st, bool rope_ready = false, bool norm_ready = false) {
  const vla_config& c = m->cfg;
  const int H = c.hidden, qd = c.n_heads * c.head_dim;
  const int nqkv = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  const int glu = c.ffn_kind == VLA_GEGLU ? 1 : 0;
  // the rows' RoPE (cos, sin), shared by every layer of this pass (a decode step
  // writes it in its embedding launch)
  if (!rope_ready) HIPCHK(launch_rope_table(pos0, n, m->inv_freq, c.head_dim / 2, m->rope_tab, st));
  AttnArgs at;
  at.q = m->qbuf;
  at.out = m->ao;
  at.kpool = m->kpool;
  at.vpool = m->vpool;
  at.g = m->geom;
  at.blk_table = view.blk;
  at.blk_ntok = view.ntok;
  at.nlb = view.nlb;
  at.last_ntok = view.last_ntok;
  at.causal = view.causal;
  at.cb0 = cb0;
  at.cslot0 = cslot0;
  at.n = n;
  at.hq = c.n_heads;
  at.part_o = m->part_o;
  at.part_ml = m->part_ml;
  at.part_rows = m->part_o ? kPartRows : 0;

  at.scale = (float)(1.0 / std::sqrt((double)c.head_dim));

  for (int l = 0; l < c.n_layers; ++l) {
    at.layer = l;
    const FwdCtx ctx = make_ctx(m, view, l, cb0, cslot0);
    // a K/V-only last layer: its input norm and q/k/v projection (K/V written), nothing more
    const bool kv_only = c.kv_only_last && l == c.n_layers - 1;
    if (decode) {
      GemvArgs g;
      g.x = m->x;
      g.norm_g = m->norm_ones;
      g.eps = c.rms_eps;
      g.W = m->wqkv[l];
      g.wf = m->wf;
      g.N = nqkv;
      g.K = H;
      g.epi = EPI_QKV;
      g.ctx = ctx;
      LAUNCH(m, VLA_K_GEMV_QKV, st, launch_gemv(g, m->dt, st, nullptr));
      if (kv_only) break;
      // bf16 output projections of up to 2048 inputs take the attention's
      // split partials directly (no merge kernel)
      const bool can_fold = m->dt == DT_BF16 && m->wf == WF_ACT && qd <= 2048;
      int fold_splits = 0;
      LAUNCH(m, VLA_K_ATTN_DECODE, st,
             launch_attention(at, m->dt, st, can_fold ? &fold_splits : nullptr));
      GemvArgs o;
      o.x = m->ao;
      o.W = m->wo[l];
      o.wf = m->wf;
      o.N = H;
      o.K = qd;
      o.epi = EPI_RESID;
      o.out = m->x;
      if (fold_splits > 0) {
        o.part_o = m->part_o;
        o.part_ml = m->part_ml;
        o.splits = fold_splits;
        o.grp = c.n_heads / c.n_kv_heads;
        o.hd = c.head_dim;
      }
      LAUNCH(m, VLA_K_GEMV_O, st, launch_gemv(o, m->dt, st, nullptr));
      LAUNCH(m, VLA_K_GEMV_GATEUP, st, launch_gemv(decode_gateup_args(m, l), m->dt, st, nullptr));
      GemvArgs dn;
      dn.x = m->act;
      dn.W = m->wdown[l];
      dn.wf = m->wf;
      dn.N = H;
      dn.K = c.ffn;
      dn.epi = EPI_RESID;
      dn.out = m->x;
      LAUNCH(m, VLA_K_GEMV_DOWN, st, launch_gemv(dn, m->dt, st, nullptr));
    } else {
      // bf16: the residual projections reduce their split-K partials into x and
      // write the next projection's normalised input u in the same pass; only
      // the first layer's input norm is a kernel of its own. fp32: plain norms.
      const bool bf16 = m->dt == DT_BF16;
      // (norm_ready: the first layer's input norm is already in u)
      if ((!bf16 || l == 0) && !(l == 0 && norm_ready))
        LAUNCH(m, VLA_K_RMSNORM, st,
               launch_rmsnorm(m->x, m->norm_ones, m->u, m->u_lo, n, H, c.rms_eps, m->dt, st));
      GemmArgs q;
      q.A = m->u;
      q.A_lo = m->u_lo;
      // INT4: the previous layer's residual reduction wrote u's group sums
      q.a_sum = l > 0 ? m->usum : nullptr;
      q.sum_ld = m->usum_ld;
      q.W = m->wqkv[l];
      q.wf = m->wf;
      q.M = n;
      q.N = nqkv;
      q.K = H;
      q.epi = EPI_QKV;
      q.ctx = ctx;
      q.ws = m->gemm_ws;
      q.ws_elems = m->gemm_ws_elems;
      LAUNCH(m, VLA_K_GEMM_QKV, st, launch_gemm(q, m->dt, st));
      if (kv_only) break;
      // the output projection's input as a bf16 pair (bf16 projection weights)
      at.out_lo = m->ao_lo;
      LAUNCH(m, VLA_K_ATTN_PREFILL, st, launch_attention(at, m->dt, st));
      GemmArgs o;
      o.A = m->ao;
      o.A_lo = m->ao_lo;
      o.W = m->wo[l];
      o.wf = m->wf;
      o.M = n;
      o.N = H;
      o.K = qd;
      o.epi = EPI_RESID;
      o.C = m->x;
      o.ws = m->gemm_ws;
      o.ws_elems = m->gemm_ws_elems;
      o.norm_out = m->u;
      o.norm_sum = m->usum;
      o.sum_ld = m->usum_ld;
      o.norm_g = m->norm_ones;
      o.eps = c.rms_eps;
      LAUNCH(m, VLA_K_GEMM_O, st, launch_gemm(o, m->dt, st));
      if (!bf16)
        LAUNCH(m, VLA_K_RMSNORM, st,
               launch_rmsnorm(m->x, m->norm_ones, m->u, nullptr, n, H, c.rms_eps, m->dt, st));
      GemmArgs gu;
      gu.A = m->u;
      gu.a_sum = m->usum;
      gu.sum_ld = m->usum_ld;
      gu.W = m->wgu[l];
      gu.wf = m->wf;
      gu.M = n;
      gu.N = 2 * c.ffn;
      gu.K = H;
      gu.epi = EPI_SWIGLU;
      gu.glu = glu;
      gu.C = m->act;
      LAUNCH(m, VLA_K_GEMM_GATEUP, st, launch_gemm(gu, m->dt, st));
      GemmArgs dn;
      dn.A = m->act;
      dn.W = m->wdown[l];
      dn.wf = m->wf;
      dn.M = n;
      dn.N = H;
      dn.K = c.ffn;
      dn.epi = EPI_RESID;
      dn.C = m->x;
      dn.ws = m->gemm_ws;
      dn.ws_elems = m->gemm_ws_elems;
      dn.norm_out = l + 1 < c.n_layers ? m->u : nullptr;
      dn.norm_out_lo = l + 1 < c.n_layers ? m->u_lo : nullptr;
      dn.norm_sum = l + 1 < c.n_layers ? m->usum : nullptr;
      dn.sum_ld = m->usum_ld;
      dn.norm_g = m->norm_ones;
      dn.eps = c.rms_eps;
      LAUNCH(m, VLA_K_GEMM_DOWN, st, launch_gemm(dn, m->dt, st));
    }
  }
}

// One decode step's embedding row, RoPE table and every layer as one persistent
// launch (decode_step.hip). Returns false, having launched nothing, when this step
// cannot take it (no kernel shape, a single cached block, no co-resident grid).
bool run_decode_persistent(vla_model* m, const KvView& view, int32_t token, int64_t pos, int cb0,
                           int cslot0, hipStream_t st) {
  const vla_config& c = m->cfg;
  if (m->ds_shape == DSHAPE_NONE || !m->opt_persistent || m->prof_cls != VLA_K_NONE ||
      view.nlb < 2)
    return false;
  if (m->ds_grid == 0) m->ds_grid = decode_step_grid(m->ds_shape);
  if (m->ds_grid < 1) return false;
  const int H = c.hidden, qd = c.n_heads * c.head_dim, hkv = c.n_kv_heads;
  const int nqkv = (c.n_heads + 2 * hkv) * c.head_dim;
  DecodeStepArgs p;
  p.token = token == VLA_TOKEN_DEVICE ? 0 : token;
  p.token_key = token == VLA_TOKEN_DEVICE ? m->amax_res : nullptr;
  p.E = m->embed;
  p.x = (float*)m->x;
  p.H = H;
  p.pos = pos;
  p.inv_freq = m->inv_freq;
  p.half = c.head_dim / 2;
  p.rope = m->rope_tab;
  const FwdCtx ctx = make_ctx(m, view, 0, cb0, cslot0);
  // q/k/v: the residual row, normalised per wavefront; RoPE + paged K/V write
  p.qkv.x = m->x;
  p.qkv.norm_g = m->norm_ones;
  p.qkv.eps = c.rms_eps;
  p.qkv.N = nqkv;
  p.qkv.K = H;
  p.qkv.epi = EPI_QKV;
  p.qkv.ctx = ctx;
  // attention: the key splits of the decode kernel, at least 2 (the output
  // projection merges them) and at most the merge's limit
  AttnArgs& at = p.at;
  at.q = m->qbuf;
  at.out = m->ao;
  at.kpool = m->kpool;
  at.vpool = m->vpool;
  at.g = m->geom;
  at.blk_table = view.blk;
  at.blk_ntok = view.ntok;
  at.nlb = view.nlb;
  at.last_ntok = view.last_ntok;
  at.causal = 1;
  at.cb0 = cb0;
  at.cslot0 = cslot0;
  at.n = 1;
  at.hq = c.n_heads;
  at.part_o = m->part_o;
  at.part_ml = m->part_ml;
  at.part_rows = kPartRows;
  at.scale = (float)(1.0 / std::sqrt((double)c.head_dim));
  // the per-kernel step's rule (launch_attention), so that both steps split alike
  int splits = std::max((view.nlb + 7) / 8, std::min(kFoldMaxSplits, (view.nlb + 3) / 4));
  splits = std::min(splits, std::max(1, 512 / hkv));
  splits = std::min(splits, kFoldMaxSplits);
  splits = std::min(splits, std::max(1, kPartRows / (hkv * 16)));
  splits = std::max(splits, 2);
  const int bps = (view.nlb + splits - 1) / splits;
  at.splits = (view.nlb + bps - 1) / bps;
  if (at.splits < 2) return false;
  // output projection: merges the splits on the way in, adds to the residual
  p.o.x = m->ao;
  p.o.N = H;
  p.o.K = qd;
  p.o.epi = EPI_RESID;
  p.o.out = m->x;
  p.o.part_o = m->part_o;
  p.o.part_ml = m->part_ml;
  p.o.splits = at.splits;
  p.o.grp = c.n_heads / hkv;
  p.o.hd = c.head_dim;
  p.gu = decode_gateup_args(m, 0);
  p.dn.x = m->act;
  p.dn.N = H;
  p.dn.K = c.ffn;
  p.dn.epi = EPI_RESID;
  p.dn.out = m->x;
  // row groups and virtual workgroups (as the separate kernels would launch them)
  const bool dks = m->ds_shape == DSHAPE_C3_3_3_D1_5_4;  // down projection K split 4 ways
  p.ng_qkv = nqkv / 2;
  p.vg_qkv = (p.ng_qkv + 3) / 4;
  p.ng_o = (H + 1) / 2;
  p.vg_o = (p.ng_o + 3) / 4;
  p.ng_gu = c.ffn;
  p.vg_gu = (p.ng_gu + 3) / 4;
  p.ng_dn = dks ? H : (H + 1) / 2;
  p.vg_dn = dks ? p.ng_dn : (p.ng_dn + 3) / 4;
  p.wtab = m->d_wtab;
  p.n_layers = c.n_layers;
  p.bar = m->d_bar;
  p.seq = m->ds_seq;
  p.gen_off = m->opt_unreachable ? (1ull << 40) : 0ull;
  p.spin_limit = m->opt_spin_limit;
  const hipError_t e = launch_decode_step(p, m->ds_shape, m->ds_grid, st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    m->ds_shape = DSHAPE_NONE;  // e.g. the grid cannot be co-resident: per-kernel path from now on
    return false;
  }
  m->ds_seq = (m->ds_seq + 1) & 1;
  m->ds_check = true;
  return true;
}

// final RMSNorm of the last row, output head, argmax
void run_head(vla_model* m, int row, hipStream_t st) {
  const vla_config& c = m->cfg;
  GemvArgs h;
  h.x = (const float*)m->x + (size_t)row * c.hidden;
  h.norm_g = m->norm_ones;
  h.eps = c.rms_eps;
  h.W = m->head;
  h.wf = m->wf;
  h.N = c.vocab;
  h.K = c.hidden;
  h.epi = EPI_HEAD;
  h.out = m->logits;
  h.argmax_part = m->amax_part;
  int grid = 0;
  LAUNCH(m, VLA_K_GEMV_HEAD, st, launch_gemv(h, m->dt, st, &grid));
  HIPCHK(launch_argmax_final(m->amax_part, grid, m->amax_res, st));
  m->have_logits = true;
}

// after a persistent decode step: reads its error flag (synchronises) and, when a
// barrier wait gave up, clears the barrier state and reports it
void check_step_error(vla_model* m, hipStream_t st) {
  if (!m->ds_check) return;
  unsigned long long* h = (unsigned long long*)staging_acquire(m->st_read) + 4;
  HIPCHK(hipMemcpyAsync(h, m->d_bar, sizeof(unsigned long long), hipMemcpyDeviceToHost, st));
  HIPCHK(hipStreamSynchronize(st));
  m->ds_check = false;
  if (*h != 0) {
    HIPCHK(hipMemsetAsync(m->d_bar, 0, kBarStateWords * sizeof(unsigned long long), st));
    HIPCHK(hipStreamSynchronize(st));
    m->ds_seq = 0;
    if (*h == 2) raise(VLA_E_HIP, "the persistent decode step found an XCD id outside 0..7");
    raise(VLA_E_TIMEOUT, "a barrier wait of the persistent decode step gave up");
  }
}

int read_argmax(vla_model* m, hipStream_t st) {
  check_step_error(m, st);
  unsigned long long* h = (unsigned long long*)staging_acquire(m->st_read);
  HIPCHK(hipMemcpyAsync(h, m->amax_res, sizeof(unsigned long long), hipMemcpyDeviceToHost, st));
  HIPCHK(hipStreamSynchronize(st));
  return (int)(0xffffffffu - (uint32_t)(*h & 0xffffffffull));
}

// chunks per lane of a whole-row one-shot GEMV over K inputs
int gemv1_cpl(int K) { return (K / 8 + 63) / 64; }

// the persistent decode-step kernel shape of a model, or DSHAPE_NONE
int decode_shape(const vla_config& c, int dt, int wf) {
  if (dt != DT_BF16 || wf != WF_ACT || c.vocab < 1 || c.kv_only_last || c.head_dim != 128)
    return DSHAPE_NONE;
  const int grp = c.n_heads / c.n_kv_heads;
  if (grp > 16 || c.n_heads > kFoldMaxHeads) return DSHAPE_NONE;
  const int nqkv = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  if (nqkv % 8 || (2 * c.ffn) % 32) return DSHAPE_NONE;
  const int cq = gemv1_cpl(c.hidden), co = gemv1_cpl(c.n_heads * c.head_dim);
  const int cg = gemv1_cpl(c.hidden), cd = gemv1_cpl(c.ffn);
  const int dks = ((c.ffn / 8 + 3) / 4 + 63) / 64;  // chunks per lane of a 4-way K split
  if (cq == 3 && co == 3 && cg == 3 && cd > 4 && dks == 5) return DSHAPE_C3_3_3_D1_5_4;
  if (cq == 1 && co == 2 && cg == 1 && cd == 1) return DSHAPE_C1_2_1_D2_1_1;
  return DSHAPE_NONE;
}

void mean_keys_for(vla_model* m, int frame_index, hipStream_t st) {
  LAUNCH(m, VLA_K_MEANKEYS, st,
         launch_meankeys(m->kpool, m->geom, m->d_blk(), m->d_fr_blk0() + frame_index,
                         m->d_fr_nblk() + frame_index, m->d_fr_ntok() + frame_index,
                         m->d_fr_slot() + frame_index, 1, 0, m->cfg.n_layers, m->meankeys,
                         m->cfg.max_frames, m->dt, st));
}

// register a new frame of n tokens (blocks, slot, positions); returns its segment index
size_t new_frame(vla_model* m, int n) {
  const int bt = bt_of(m);
  if (n < 1 || n > m->cfg.max_chunk)
    raise(VLA_E_INVALID, "chunk length " + std::to_string(n) + " outside [1, max_chunk=" +
                             std::to_string(m->cfg.max_chunk) + "]");
  if (m->free_slots.empty()) raise(VLA_E_NO_BLOCKS, "max_frames frames already resident");
  const int need = (n + bt - 1) / bt;
  Segment s;
  if (!m->pool.alloc(need, &s.blocks))
    raise(VLA_E_NO_BLOCKS, "need " + std::to_string(need) + " blocks, " +
                               std::to_string(m->pool.free_count()) + " free");
  s.frame = true;
  s.frame_id = m->next_frame_id++;
  s.start_pos = m->next_pos;
  s.ntok = n;
  s.slot = m->free_slots.back();
  m->free_slots.pop_back();
  m->next_pos += n;
  m->segs.push_back(s);
  m->meta_dirty = true;
  return m->segs.size() - 1;
}

int frame_index_of(const vla_model* m, size_t seg_index) {
  int f = 0;
  for (size_t i = 0; i < seg_index; ++i) f += m->segs[i].frame ? 1 : 0;
  return f;
}

void validate_cfg(const vla_config* c) {
  auto bad = [](const std::string& s) { raise(VLA_E_INVALID, "invalid config: " + s); };
  if (!c) bad("null");
  if (c->n_layers < 1 || c->hidden < 64 || c->n_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 2 || c->ffn < 16 || c->vocab < 0 || c->vocab == 1)
    bad("non-positive size");
  if (c->n_heads % c->n_kv_heads) bad("n_heads must be a multiple of n_kv_heads");
  if (c->head_dim % 16 || c->head_dim > 256) bad("head_dim must be a multiple of 16, <= 256");
  if (c->ffn % 16) bad("ffn must be a multiple of 16");
  if (c->hidden % 64) bad("hidden must be a multiple of 64");
  if (c->hidden > 8192) bad("hidden must be <= 8192");
  if (c->block_tokens != 16) bad("block_tokens must be 16");
  if (c->num_blocks < 1 || c->max_frames < 1 || c->max_chunk < 1) bad("budget sizes");
  if (c->act_dtype != VLA_F32 && c->act_dtype != VLA_BF16) bad("act_dtype must be VLA_F32 or VLA_BF16");
  if (c->wdtype == VLA_INT4_G128) {
    if (c->act_dtype != VLA_BF16) bad("INT4 weights need bf16 activations");
    if (c->hidden % 128 || (c->n_heads * c->head_dim) % 128 || c->ffn % 128)
      bad("INT4 weights: hidden, n_heads*head_dim and ffn must be multiples of 128");
  } else if (c->wdtype != c->act_dtype) {
    bad("wdtype must equal act_dtype (VLA_F32 or VLA_BF16) or be VLA_INT4_G128");
  }
  if (c->ffn_kind != VLA_SWIGLU && c->ffn_kind != VLA_GEGLU) bad("ffn_kind");
  if (c->kv_only_last != 0 && c->kv_only_last != 1) bad("kv_only_last must be 0 or 1");
  if (c->kv_only_last && c->vocab != 0) bad("a K/V-only last layer leaves no output for a head");
  if (c->stream_base > 0xFFFFFF) bad("stream_base");
  if (!(c->rope_theta > 1.0)) bad("rope_theta");
  const int qd = c->n_heads * c->head_dim;
  if (c->act_dtype == VLA_BF16) {
    if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
      bad("bf16 path: head_dim 64, 128 or 256");
    if (qd % 64 || c->ffn % 64) bad("bf16 path: n_heads*head_dim and ffn multiples of 64");
  } else {
    if (c->num_blocks * c->block_tokens > 2048) bad("fp32 path: at most 2048 cached tokens");
    if (qd % 8 || c->ffn % 8) bad("multiples of 8");
  }
  if ((int64_t)c->vocab * c->hidden > ((int64_t)1 << 40)) bad("vocab*hidden too large");
}

// the seeded projection, embedding and head weights (own_weights), then the norm
// weights and the RoPE inverse frequencies
void init_weights(vla_model* m, bool own_weights) {
  const vla_config& c = m->cfg;
  const int H = c.hidden, d = c.head_dim, hq = c.n_heads, hkv = c.n_kv_heads;
  const hipStream_t st = nullptr;
  const uint64_t base = c.stream_base;
  auto sid = [base](int layer, int kind) { return base + (uint64_t)(((layer + 1) << 8) | kind); };
  // a projection: in the activation type, or INT4 group-128 (codes + scales)
  auto proj = [&](void* out, int layout, int64_t rows, int64_t cols, uint64_t sa, uint64_t sb,
                  uint64_t sc) {
    if (m->wf == WF_INT4)
      HIPCHK(launch_init_weight_w4(out, layout, rows, cols, c.seed, sa, sb, sc, hq, hkv, d,
                                   c.init_std, st));
    else
      HIPCHK(launch_init_weight(out, m->dt, layout, rows, cols, c.seed, sa, sb, sc, hq, hkv, d,
                                c.init_std, st));
  };
  if (own_weights && c.vocab > 0) {
    HIPCHK(launch_init_weight(m->embed, m->dt, LAYOUT_PLAIN, c.vocab, H, c.seed, 1, 1, 1, hq, hkv,
                              d, c.init_std, st));
    proj(m->head, LAYOUT_PLAIN, c.vocab, H, 2, 2, 2);
  }
  for (int l = 0; own_weights && l < c.n_layers; ++l) {
    proj(m->wqkv[l], LAYOUT_QKV, (int64_t)(hq + 2 * hkv) * d, H, sid(l, 1), sid(l, 2), sid(l, 3));
    proj(m->wo[l], LAYOUT_PLAIN, H, (int64_t)hq * d, sid(l, 4), sid(l, 4), sid(l, 4));
    proj(m->wgu[l], LAYOUT_GATEUP, 2 * (int64_t)c.ffn, H, sid(l, 5), sid(l, 6), sid(l, 6));
    proj(m->wdown[l], LAYOUT_PLAIN, H, c.ffn, sid(l, 7), sid(l, 7), sid(l, 7));
  }
  HIPCHK(launch_fill_f32(m->norm_ones, 1.0f, H, st));
  std::vector<double> inv(d / 2);
  for (int j = 0; j < d / 2; ++j) inv[j] = std::pow(c.rope_theta, -2.0 * j / d);
  HIPCHK(hipMemcpy(m->inv_freq, inv.data(), inv.size() * sizeof(double), hipMemcpyHostToDevice));
  HIPCHK(hipDeviceSynchronize());
}

void destroy(vla_model* m) {
  if (!m) return;
  (void)hipSetDevice(m->dev);
  (void)hipDeviceSynchronize();
  for (void* p : m->allocs) (void)hipFree(p);
  staging_free(m->st_meta);
  staging_free(m->st_tok);
  staging_free(m->st_read);
  for (hipEvent_t e : m->prof.ev) (void)hipEventDestroy(e);
  delete m;
}

// allocate and initialise a model; `borrow` (non-null): the KV pool and its
// geometry belong to that model (an action expert writing into its prefix's pool);
// `share` (non-null, same config): the weights are that model's (a sibling)
void build_model(vla_model* m, const vla_config& cfg, const vla_model* borrow,
                 const vla_model* share = nullptr) {
  m->cfg = cfg;
  HIPCHK(hipGetDevice(&m->dev));
  const vla_config& c = m->cfg;
  m->dt = c.act_dtype == VLA_F32 ? DT_F32 : DT_BF16;
  m->wf = c.wdtype == VLA_INT4_G128 ? WF_INT4 : WF_ACT;
  m->esz = m->dt == DT_F32 ? 4 : 2;
  m->geom = borrow ? borrow->geom
                   : KvGeom{c.n_layers, c.num_blocks, c.n_kv_heads, c.block_tokens, c.head_dim,
                            m->esz == 4 ? 4 : 5};
  const size_t H = c.hidden, d = c.head_dim, hq = c.n_heads, hkv = c.n_kv_heads;
  const size_t e = m->esz;
  // projection bytes: activation type, or INT4 codes (half a byte) + one fp16 per 128
  auto wbytes = [&](size_t rows, size_t cols) {
    return m->wf == WF_INT4 ? rows * cols / 2 + rows * (cols / 128) * 2 : rows * cols * e;
  };
  if (share) {
    m->wstore = share->wstore;
    m->embed = share->embed;
    m->head = share->head;
    m->wqkv = share->wqkv;
    m->wo = share->wo;
    m->wgu = share->wgu;
    m->wdown = share->wdown;
  } else {
    m->wstore = std::make_shared<WeightStore>();
    m->wstore->dev = m->dev;
    m->embed = walloc(m, (size_t)c.vocab * H * e);
    m->head = walloc(m, wbytes(c.vocab, H));
    for (int l = 0; l < c.n_layers; ++l) {
      m->wqkv.push_back(walloc(m, wbytes((hq + 2 * hkv) * d, H)));
      m->wo.push_back(walloc(m, wbytes(H, hq * d)));
      m->wgu.push_back(walloc(m, wbytes(2 * (size_t)c.ffn, H)));
      m->wdown.push_back(walloc(m, wbytes(H, c.ffn)));
    }
  }
  m->norm_ones = (float*)dalloc(m, H * sizeof(float));
  m->inv_freq = (double*)dalloc(m, d / 2 * sizeof(double));
  m->rope_tab = (float2*)dalloc(m, (size_t)c.max_chunk * (d / 2) * sizeof(float2));
  if (borrow) {
    m->kpool = borrow->kpool;
    m->vpool = borrow->vpool;
  } else {
    const size_t pool_bytes = (size_t)c.n_layers * c.num_blocks * hkv * c.block_tokens * d * e;
    m->kpool = dalloc(m, pool_bytes);
    m->vpool = dalloc(m, pool_bytes);
    // stale slots of partial blocks meet zero probabilities in P*V: keep them finite
    HIPCHK(hipMemset(m->kpool, 0, pool_bytes));
    HIPCHK(hipMemset(m->vpool, 0, pool_bytes));
  }
  m->meankeys = (double*)dalloc(m, (size_t)c.n_layers * c.max_frames * hkv * d * sizeof(double));
  const size_t mc = c.max_chunk;
  m->x = dalloc(m, mc * H * sizeof(float));  // the residual stream is fp32
  m->u = dalloc(m, mc * H * e);
  // the q/k/v and output-projection inputs as bf16 pairs: for models whose output is
  // logits (the precision budget that needs them is the logits'); a prefix model (K/V
  // out) or an action expert computes those products from the rounded inputs alone
  if (m->dt == DT_BF16 && m->wf == WF_ACT && c.vocab > 0) {
    m->u_lo = dalloc(m, mc * H * e);
    m->ao_lo = dalloc(m, mc * hq * d * e);
  }
  if (m->wf == WF_INT4 && H % 128 == 0) {
    m->usum_ld = (int)((mc + 63) / 64 * 64);
    const size_t sb = (size_t)(H / 128) * m->usum_ld * sizeof(float);
    m->usum = (float*)dalloc(m, sb);
    HIPCHK(hipMemset(m->usum, 0, sb));  // padded rows stay finite
  }
  m->qbuf = dalloc(m, mc * hq * d * e);
  m->ao = dalloc(m, mc * hq * d * e);
  m->act = dalloc(m, mc * (size_t)c.ffn * e);
  m->logits = (float*)dalloc(m, (size_t)c.vocab * sizeof(float));
  m->amax_part = (unsigned long long*)dalloc(m, kArgmaxParts * sizeof(unsigned long long));
  m->amax_res = (unsigned long long*)dalloc(m, sizeof(unsigned long long));
  if (m->dt == DT_BF16) {
    m->part_o = (float*)dalloc(m, (size_t)kPartRows * d * sizeof(float));
    m->part_ml = (float*)dalloc(m, (size_t)kPartRows * 2 * sizeof(float));
    m->gemm_ws_elems = (size_t)kGemmSplitsMax * mc * std::max(H, (hq + 2 * hkv) * d);
    m->gemm_ws = (float*)dalloc(m, m->gemm_ws_elems * sizeof(float));
  }
  m->d_meta = (int*)dalloc(m, m->meta_ints() * sizeof(int));
  m->d_tokens = (int*)dalloc(m, mc * sizeof(int));
  m->d_score_m = (double*)dalloc(m, (size_t)c.max_frames * sizeof(double));
  m->d_score_res = (double*)dalloc(m, 2 * sizeof(double));
  staging_init(m->st_meta, m->meta_ints() * sizeof(int));
  staging_init(m->st_tok, mc * sizeof(int));
  staging_init(m->st_read, 64);
  m->pool.reset(c.num_blocks);
  for (int i = c.max_frames - 1; i >= 0; --i) m->free_slots.push_back(i);
  m->ds_shape = decode_shape(c, m->dt, m->wf);
  if (m->ds_shape != DSHAPE_NONE) {
    std::vector<const void*> wt;
    for (int l = 0; l < c.n_layers; ++l) {
      wt.push_back(m->wqkv[l]);
      wt.push_back(m->wo[l]);
      wt.push_back(m->wgu[l]);
      wt.push_back(m->wdown[l]);
    }
    m->d_wtab = (const void**)dalloc(m, wt.size() * sizeof(void*));
    HIPCHK(hipMemcpy(m->d_wtab, wt.data(), wt.size() * sizeof(void*), hipMemcpyHostToDevice));
    m->d_bar = (unsigned long long*)dalloc(m, kBarStateWords * sizeof(unsigned long long));
    HIPCHK(hipMemset(m->d_bar, 0, kBarStateWords * sizeof(unsigned long long)));
  }
  init_weights(m, share == nullptr);
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================
extern "C" {

const char* vla_last_error(void) { return g_err.c_str(); }

vla_status vla_model_create(const vla_config* cfg, vla_model** out) {
  vla_model* m = nullptr;
  vla_status st = guarded([&] {
    if (!out) raise(VLA_E_INVALID, "out is NULL");
    *out = nullptr;
    validate_cfg(cfg);
    m = new vla_model();
    build_model(m, *cfg, nullptr);
    *out = m;
  });
  if (st != VLA_OK && m) {
    std::string keep = g_err;
    destroy(m);
    g_err = keep;
  }
  return st;
}

vla_status vla_model_create_sibling(const vla_model* src, vla_model** out) {
  vla_model* m = nullptr;
  vla_status st = guarded([&] {
    if (!out) raise(VLA_E_INVALID, "out is NULL");
    *out = nullptr;
    if (!src) raise(VLA_E_INVALID, "null source model");
    HIPCHK(hipSetDevice(src->dev));
    m = new vla_model();
    build_model(m, src->cfg, nullptr, src);
    *out = m;
  });
  if (st != VLA_OK && m) {
    std::string keep = g_err;
    destroy(m);
    g_err = keep;
  }
  return st;
}

void vla_model_destroy(vla_model* m) { destroy(m); }

vla_status vla_prefill_chunk(vla_model* m, const int32_t* tokens, const void* embeds, int32_t n,
                             int32_t* out_frame_id, void* stream) {
  return guarded([&] {
    if (!m) raise(VLA_E_INVALID, "null model");
    if ((tokens == nullptr) == (embeds == nullptr))
      raise(VLA_E_INVALID, "exactly one of tokens / embeds must be given");
    if (n < 1 || n > m->cfg.max_chunk) raise(VLA_E_INVALID, "chunk length out of range");
    if (tokens && m->cfg.vocab == 0) raise(VLA_E_INVALID, "no vocabulary: pass embeddings");
    if (tokens)
      for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= m->cfg.vocab) raise(VLA_E_INVALID, "token id out of range");
    HIPCHK(hipSetDevice(m->dev));
    const hipStream_t st = (hipStream_t)stream;
    const size_t si = new_frame(m, n);
    const Segment seg = m->segs[si];
    try {
      sync_meta(m, st);
      if (tokens) {
        int* h = (int*)staging_acquire(m->st_tok);
        memcpy(h, tokens, (size_t)n * sizeof(int));
        staging_upload(m->st_tok, m->d_tokens, (size_t)n * sizeof(int), st);
        HIPCHK(launch_embed(m->d_tokens, 0, nullptr, n, m->embed, m->x, m->cfg.hidden, m->dt,
                            nullptr, st));
      } else {
        HIPCHK(launch_to_f32(embeds, (float*)m->x, (int64_t)n * m->cfg.hidden, m->dt, st));
      }
      run_layers(m, model_view(m), n, seg.start_pos, seg_blk0(m, si), 0, /*decode=*/false, st);
      if (m->cfg.vocab > 0) run_head(m, n - 1, st);
      mean_keys_for(m, frame_index_of(m, si), st);
    } catch (...) {
      // undo the registration (blocks back in reverse pop order)
      std::vector<int> rb(seg.blocks.rbegin(), seg.blocks.rend());
      m->pool.release(rb.data(), (int)rb.size());
      m->free_slots.push_back(seg.slot);
      m->segs.erase(m->segs.begin() + si);
      m->next_pos = seg.start_pos;
      m->next_frame_id = seg.frame_id;
      m->meta_dirty = true;
      throw;
    }
    if (out_frame_id) *out_frame_id = seg.frame_id;
  });
}

vla_status vla_decode_step(vla_model* m, int32_t token, int32_t* out_next_token, void* stream) {
  return guarded([&] {
    if (!m) raise(VLA_E_INVALID, "null model");
    if (token == VLA_TOKEN_DEVICE) {
      if (!m->have_logits || m->cfg.vocab == 0)
        raise(VLA_E_STATE, "no previous forward to take the device-resident token from");
    } else if (token < 0 || token >= m->cfg.vocab) {
      raise(VLA_E_INVALID, "token id out of range");
    }
    HIPCHK(hipSetDevice(m->dev));
    const hipStream_t st = (hipStream_t)stream;
    const int bt = bt_of(m);
    // place the token in the decode tail (a tail starts on a fresh block)
    bool new_seg = false, new_block = false;
    if (m->segs.empty() || m->segs.back().frame) {
      Segment s;
      s.frame = false;
      s.start_pos = m->next_pos;
      if (!m->pool.alloc(1, &s.blocks)) raise(VLA_E_NO_BLOCKS, "no free block for the decode tail");
      m->segs.push_back(s);
      new_seg = true;
    } else if (m->segs.back().ntok == (int)m->segs.back().blocks.size() * bt) {
      if (!m->pool.alloc(1, &m->segs.back().blocks))
        raise(VLA_E_NO_BLOCKS, "no free block for the decode tail");
      new_block = true;
    }
    Segment& tail = m->segs.back();
    const int off = tail.ntok;
    tail.ntok += 1;
    const int64_t pos = m->next_pos++;
    if (new_seg || new_block) m->meta_dirty = true;
    try {
      sync_meta(m, st);
      const int cb0 = logical_blocks(m) - 1;
      const KvView view = model_view(m);
      m->last_persistent = run_decode_persistent(m, view, token, pos, cb0, off % bt, st);
      if (!m->last_persistent) {
        // VLA_TOKEN_DEVICE: the previous forward's greedy token, read on the device;
        // the same launch writes the position's RoPE table
        HIPCHK(launch_embed_rope1(token, token == VLA_TOKEN_DEVICE ? m->amax_res : nullptr,
                                  m->embed, m->x, m->cfg.hidden, m->dt, pos, m->inv_freq,
                                  m->cfg.head_dim / 2, m->rope_tab, st));
        run_layers(m, view, 1, pos, cb0, off % bt, /*decode=*/true, st, /*rope_ready=*/true);
      }
      run_head(m, 0, st);
      if (out_next_token) *out_next_token = read_argmax(m, st);
    } catch (...) {
      tail.ntok -= 1;
      m->next_pos -= 1;
      if (new_seg) {
        m->pool.release(tail.blocks.data(), 1);
        m->segs.pop_back();
      } else if (new_block) {
        m->pool.release(&tail.blocks.back(), 1);
        tail.blocks.pop_back();
      }
      m->meta_dirty = true;
      throw;
    }
  });
}

// the resident frame (index in arrival order) that `policy` evicts next, and its
// score; synchronises the stream when the choice is made on the device
static int pick_frame(vla_model* m, int policy, int layer, hipStream_t st, double* score) {
  const int F = n_frames(m);
  if (policy == VLA_EVICT_FIFO) {
    if (F < 1) raise(VLA_E_NOTHING_TO_EVICT, "no frame resident");
    *score = 0.0;
    return 0;
  }
  if (F < 2) raise(VLA_E_NOTHING_TO_EVICT, "fewer than 2 frames resident");
  sync_meta(m, st);
  const int D = m->cfg.n_kv_heads * m->cfg.head_dim;
  const double* tab = m->meankeys + (size_t)layer * m->cfg.max_frames * D;
  if (policy == VLA_EVICT_ADJACENT)
    LAUNCH(m, VLA_K_SCORE, st, launch_score_adjacent(tab, m->d_fr_slot(), F, D, m->d_score_m,
                                                     m->d_score_res, st));
  else
    LAUNCH(m, VLA_K_SCORE, st, launch_score(tab, m->d_fr_slot(), F, D, m->d_score_m,
                                            m->d_score_res, st));
  double* h = (double*)staging_acquire(m->st_read);
  HIPCHK(hipMemcpyAsync(h, m->d_score_res, 2 * sizeof(double), hipMemcpyDeviceToHost, st));
  HIPCHK(hipStreamSynchronize(st));
  const int idx = (int)h[0];
  *score = h[1];
  // adjacent: pair i's older frame is frame i
  if (idx < 0 || idx >= F) raise(VLA_E_STATE, "scoring returned an invalid index");
  return idx;
}

// segment index of the idx-th resident frame (arrival order)
static size_t frame_seg(const vla_model* m, int idx) {
  size_t si = 0;
  for (int f = -1; si < m->segs.size(); ++si)
    if (m->segs[si].frame && ++f == idx) break;
  return si;
}

// evict the idx-th resident frame: its blocks go onto the free-list in logical order
static int evict_frame_index(vla_model* m, int idx) {
  const size_t si = frame_seg(m, idx);
  Segment s = m->segs[si];
  if (!m->pool.release(s.blocks.data(), (int)s.blocks.size()))
    raise(VLA_E_STATE, "block bookkeeping corrupted");
  m->free_slots.push_back(s.slot);
  m->segs.erase(m->segs.begin() + si);
  m->meta_dirty = true;
  return s.frame_id;
}

static void check_policy_layer(const vla_model* m, int policy, int layer) {
  if (policy != VLA_EVICT_SEMANTIC && policy != VLA_EVICT_FIFO && policy != VLA_EVICT_ADJACENT)
    raise(VLA_E_INVALID, "unknown eviction policy");
  if (layer < 0 || layer >= m->cfg.n_layers) raise(VLA_E_INVALID, "layer out of range");
}

static vla_status score_impl(vla_model* m, int32_t layer, int32_t* out_frame_id, double* out_score,
                             void* stream, bool evict) {
  return guarded([&] {
    if (!m) raise(VLA_E_INVALID, "null model");
    check_policy_layer(m, VLA_EVICT_SEMANTIC, layer);
    HIPCHK(hipSetDevice(m->dev));
    double score = 0.0;
    const int idx = pick_frame(m, VLA_EVICT_SEMANTIC, layer, (hipStream_t)stream, &score);
    const int fid = evict ? evict_frame_index(m, idx) : m->segs[frame_seg(m, idx)].frame_id;
    if (out_frame_id) *out_frame_id = fid;
    if (out_score) *out_score = score;
  });
}

vla_status vla_kv_score_and_evict(vla_model* m, int32_t layer, int32_t* out_frame_id,
                                  double* out_score, void* stream) {
  return score_impl(m, layer, out_frame_id, out_score, stream, true);
}

vla_status vla_kv_score(vla_model* m, int32_t layer, int32_t* out_frame_id, double* out_score,
                        void* stream) {
  return score_impl(m, layer, out_frame_id, out_score, stream, false);
}

vla_status vla_kv_evict(vla_model* m, int32_t policy, int32_t layer, int32_t* out_frame_id,
                        double* out_score, void* stream) {
  return guarded([&] {
    if (!m) raise(VLA_E_INVALID, "null model");
    check_policy_layer(m, policy, layer);
    HIPCHK(hipSetDevice(m->dev));
    double score = 0.0;
    const int idx = pick_frame(m, policy, layer, (hipStream_t)stream, &score);
    const int fid = evict_frame_index(m, idx);
    if (out_frame_id) *out_frame_id = fid;
    if (out_score) *out_score = score;
  });
}

vla_status vla_kv_make_room(vla_model* m, int32_t policy, int32_t layer, int32_t n_tokens,
                            int32_t window, int32_t* out_evicted, void* stream) {
  return guarded([&] {
    if (!m) raise(VLA_E_INVALID, "null model");
    check_policy_layer(m, policy, layer);
    if (n_tokens < 1 || n_tokens > m->cfg.max_chunk) raise(VLA_E_INVALID, "n_tokens out of range");
    if (window < 0) raise(VLA_E_INVALID, "window must be >= 0");
    HIPCHK(hipSetDevice(m->dev));
    const int need = (n_tokens + bt_of(m) - 1) / bt_of(m);
    int evictable = 0;
    for (const auto& sg : m->segs)
      if (sg.frame) evictable += (int)sg.blocks.size();
    if (need > m->pool.free_count() + evictable)
      raise(VLA_E_NO_BLOCKS, "need " + std::to_string(need) + " blocks; evicting every frame frees " +
                                 std::to_string(evictable) + " of them");
    int n = 0;
    for (;;) {
      const int F = n_frames(m);
      const bool room = m->pool.free_count() >= need && F < m->cfg.max_frames &&
                        (window == 0 || F < window);
      if (room) break;
      double score = 0.0;
      const int idx = F == 1 ? 0 : pick_frame(m, policy, layer, (hipStream_t)stream, &score);
      evict_frame_index(m, idx);
      ++n;
    }
    if (out_evicted) *out_evicted = n;
  });
}

vla_status vla_kv_score_noalloc(const double* mean_keys, int32_t n_frames, int32_t dim,
                                int32_t* out_index, double* out_score, void* stream) {
  return guarded([&] {
    if (!mean_keys || !out_index || !out_score) raise(VLA_E_INVALID, "null argument");
    if (n_frames < 2) raise(VLA_E_NOTHING_TO_EVICT, "fewer than 2 frames");
    if (n_frames > kScoreNoAllocMaxFrames)
      raise(VLA_E_INVALID, "n_frames " + std::to_string(n_frames) + " exceeds the maximum of " +
                               std::to_string(kScoreNoAllocMaxFrames));
    if (dim < 1) raise(VLA_E_INVALID, "dim must be >= 1");
    HIPCHK(launch_score_noalloc(mean_keys, n_frames, dim, out_index, out_score,
                                (hipStream_t)stream));
  });
}

vla_status vla_logits_out(vla_model* m, float* out, int32_t n, void* stream) {
  return guarded([&] {
    if (!m || !out) raise(VLA_E_INVALID, "null argument");
    if (n != m->cfg.vocab) raise(VLA_E_INVALID, "n must equal vocab");
    if (!m->have_logits) raise(VLA_E_STATE, "no forward has run yet");
    HIPCHK(hipSetDevice(m->dev));
    const hipStream_t st = (hipStream_t)stream;
    check_step_error(m, st);
    HIPCHK(hipMemcpyAsync(out, m->logits, (size_t)n * sizeof(float), hipMemcpyDefault, st));
    HIPCHK(hipStreamSynchronize(st));
  });
}

vla_status vla_kv_append_raw(vla_model* m, const void* k, const void* v, int32_t n,
                             int32_t* out_frame_id, void* stream) {
  return guarded([&] {
    if (!m || !k || !v) raise(VLA_E_INVALID, "null argument");
    HIPCHK(hipSetDevice(m->dev));
    const hipStream_t st = (hipStream_t)stream;
    const size_t si = new_frame(m, n);
    const Segment seg = m->segs[si];
    try {
      sync_meta(m, st);
      HIPCHK(launch_kv_scatter(k, v, n, m->kpool, m->vpool, m->geom, m->d_blk(), seg_blk0(m, si),
                               m->dt, st));
      mean_keys_for(m, frame_index_of(m, si), st);
    } catch (...) {
      std::vector<int> rb(seg.blocks.rbegin(), seg.blocks.rend());
      m->pool.release(rb.data(), (int)rb.size());
      m->free_slots.push_back(seg.slot);
      m->segs.erase(m->segs.begin() + si);
      m->next_pos = seg.start_pos;
      m->next_frame_id = seg.frame_id;
      m->meta_dirty = true;
      throw;
    }
    if (out_frame_id) *out_frame_id = seg.frame_id;
  });
}

vla_status vla_kv_rollback(vla_model* m, int32_t keep_frame_id) {
  return guarded([&] {
    if (!m) raise(VLA_E_INVALID, "null model");
    // keep_frame_id -1: drop everything (back to the empty state)
    size_t keep = m->segs.size();
    for (size_t i = 0; i < m->segs.size(); ++i)
      if (m->segs[i].frame && m->segs[i].frame_id == keep_frame_id) keep = i;
    if (keep == m->segs.size() && keep_frame_id != -1)
      raise(VLA_E_INVALID, "no such resident frame");
    const size_t n_keep = keep_frame_id == -1 ? 0 : keep + 1;
    while (m->segs.size() > n_keep) {
      Segment s = m->segs.back();
      std::vector<int> rb(s.blocks.rbegin(), s.blocks.rend());
      if (!m->pool.release(rb.data(), (int)rb.size()))
        raise(VLA_E_STATE, "block bookkeeping corrupted");
      if (s.frame) m->free_slots.push_back(s.slot);
      m->segs.pop_back();
    }
    if (n_keep == 0) {
      m->next_pos = 0;
    } else {
      const Segment& k = m->segs[keep];
      m->next_pos = k.start_pos + k.ntok;
    }
    m->next_frame_id = keep_frame_id + 1;
    m->meta_dirty = true;
  });
}

vla_status vla_kv_refresh_mean_keys(vla_model* m, void* stream) {
  return guarded([&] {
    if (!m) raise(VLA_E_INVALID, "null model");
    HIPCHK(hipSetDevice(m->dev));
    const hipStream_t st = (hipStream_t)stream;
    sync_meta(m, st);
    const int F = n_frames(m);
    LAUNCH(m, VLA_K_MEANKEYS, st,
           launch_meankeys(m->kpool, m->geom, m->d_blk(), m->d_fr_blk0(), m->d_fr_nblk(),
                           m->d_fr_ntok(), m->d_fr_slot(), F, 0, m->cfg.n_layers, m->meankeys,
                           m->cfg.max_frames, m->dt, st));
  });
}

vla_status vla_get_state(const vla_model* m, vla_state* out) {
  return guarded([&] {
    if (!m || !out) raise(VLA_E_INVALID, "null argument");
    out->next_position = m->next_pos;
    out->next_frame_id = m->next_frame_id;
    out->n_frames = n_frames(m);
    out->resident_tokens = resident_tokens(m);
    out->free_blocks = m->pool.free_count();
    out->logical_blocks = logical_blocks(m);
  });
}

vla_status vla_kv_block_table(const vla_model* m, int32_t* blocks, int32_t* ntok, int32_t cap,
                              int32_t* n_out) {
  return guarded([&] {
    if (!m || !n_out) raise(VLA_E_INVALID, "null argument");
    const int bt = m->cfg.block_tokens;
    int n = 0;
    for (const auto& s : m->segs)
      for (size_t i = 0; i < s.blocks.size(); ++i, ++n)
        if (n < cap) {
          if (blocks) blocks[n] = s.blocks[i];
          if (ntok) ntok[n] = std::min(bt, s.ntok - (int)i * bt);
        }
    *n_out = n;
  });
}

static void copy_free_list(const BlockPool& p, int32_t* out, int32_t cap, int32_t* n_out) {
  const std::vector<int>& fl = p.free_list();
  const int n = (int)fl.size();
  if (out)
    for (int i = 0; i < n && i < cap; ++i) out[i] = fl[i];
  *n_out = n;
}

vla_status vla_kv_free_list(const vla_model* m, int32_t* out, int32_t cap, int32_t* n_out) {
  return guarded([&] {
    if (!m || !n_out) raise(VLA_E_INVALID, "null argument");
    copy_free_list(m->pool, out, cap, n_out);
  });
}

vla_status vla_kv_frames(const vla_model* m, int32_t* frame_ids, int32_t cap, int32_t* n_out) {
  return guarded([&] {
    if (!m || !n_out) raise(VLA_E_INVALID, "null argument");
    int n = 0;
    for (const auto& s : m->segs)
      if (s.frame) {
        if (frame_ids && n < cap) frame_ids[n] = s.frame_id;
        ++n;
      }
    *n_out = n;
  });
}

vla_status vla_mean_keys_out(vla_model* m, int32_t layer, double* out, int32_t cap_frames,
                             int32_t* n_out, void* stream) {
  return guarded([&] {
    if (!m || !out || !n_out) raise(VLA_E_INVALID, "null argument");
    if (layer < 0 || layer >= m->cfg.n_layers) raise(VLA_E_INVALID, "layer out of range");
    HIPCHK(hipSetDevice(m->dev));
    const hipStream_t st = (hipStream_t)stream;
    const int D = m->cfg.n_kv_heads * m->cfg.head_dim;
    int f = 0;
    for (const auto& s : m->segs) {
      if (!s.frame) continue;
      if (f < cap_frames)
        HIPCHK(hipMemcpyAsync(out + (size_t)f * D,
                              m->meankeys + ((size_t)layer * m->cfg.max_frames + s.slot) * D,
                              D * sizeof(double), hipMemcpyDeviceToHost, st));
      ++f;
    }
    HIPCHK(hipStreamSynchronize(st));
    *n_out = f;
  });
}

vla_status vla_kv_gather(vla_model* m, int32_t layer, void* k_out, void* v_out,
                         int32_t cap_tokens, int32_t* n_out, void* stream) {
  return guarded([&] {
    if (!m || !k_out || !v_out || !n_out) raise(VLA_E_INVALID, "null argument");
    if (layer < 0 || layer >= m->cfg.n_layers) raise(VLA_E_INVALID, "layer out of range");
    const int T = resident_tokens(m);
    *n_out = T;
    if (T > cap_tokens) raise(VLA_E_INVALID, "cap_tokens smaller than the resident tokens");
    HIPCHK(hipSetDevice(m->dev));
    const hipStream_t st = (hipStream_t)stream;
    m->meta_dirty = true;  // the device copy of the last block's count may be stale
    sync_meta(m, st);
    HIPCHK(launch_kv_gather(m->kpool, m->vpool, m->geom, layer, m->d_blk(), m->d_ntok(),
                            m->d_tokbase(), logical_blocks(m), k_out, v_out, m->dt, st));
  });
}

vla_status vla_weight_out(vla_model* m, int32_t kind, int32_t layer, void* out, int64_t bytes,
                          void* stream) {
  return guarded([&] {
    if (!m || !out) raise(VLA_E_INVALID, "null argument");
    const vla_config& c = m->cfg;
    if (kind < 1 || kind > 9) raise(VLA_E_INVALID, "kind");
    if (kind <= 7 && (layer < 0 || layer >= c.n_layers)) raise(VLA_E_INVALID, "layer");
    if (kind >= 8 && c.vocab == 0) raise(VLA_E_INVALID, "no vocabulary");
    HIPCHK(hipSetDevice(m->dev));
    const hipStream_t st = (hipStream_t)stream;
    const int64_t H = c.hidden, d = c.head_dim, qd = (int64_t)c.n_heads * d,
                  kd = (int64_t)c.n_kv_heads * d;
    int64_t rows = 0, cols = H;
    const void* src = nullptr;
    int layout = LAYOUT_PLAIN, which = 0;
    switch (kind) {
      case 1: rows = qd; src = m->wqkv[layer]; layout = LAYOUT_QKV; which = 0; break;
      case 2: rows = kd; src = m->wqkv[layer]; layout = LAYOUT_QKV; which = 1; break;
      case 3: rows = kd; src = m->wqkv[layer]; layout = LAYOUT_QKV; which = 2; break;
      case 4: rows = H; cols = qd; src = m->wo[layer]; break;
      case 5: rows = c.ffn; src = m->wgu[layer]; layout = LAYOUT_GATEUP; which = 0; break;
      case 6: rows = c.ffn; src = m->wgu[layer]; layout = LAYOUT_GATEUP; which = 1; break;
      case 7: rows = H; cols = c.ffn; src = m->wdown[layer]; break;
      case 8: rows = c.vocab; src = m->embed; break;
      case 9: rows = c.vocab; src = m->head; break;
    }
    if (m->wf == WF_INT4 && kind != 8) {  // INT4 projection: dequantised q * s in fp32
      if (bytes < rows * cols * 4) raise(VLA_E_INVALID, "output buffer too small");
      int64_t prows = rows;  // physical rows of the whole tensor
      if (kind <= 3) prows = qd + 2 * kd;
      else if (kind == 5 || kind == 6) prows = 2 * (int64_t)c.ffn;
      HIPCHK(launch_weight_logical_w4(src, (float*)out, layout, which, rows, cols, prows, c.n_heads,
                                      c.n_kv_heads, (int)d, st));
      return;
    }
    if (bytes < rows * cols * (int64_t)m->esz) raise(VLA_E_INVALID, "output buffer too small");
    HIPCHK(launch_weight_logical(src, out, m->dt, layout, which, rows, cols, c.n_heads,
                                 c.n_kv_heads, (int)d, st));
  });
}

vla_status vla_set_option(vla_model* m, int32_t key, int64_t value) {
  return guarded([&] {
    if (!m) raise(VLA_E_INVALID, "null model");
    switch (key) {
      case VLA_OPT_PERSISTENT_DECODE:
        if (value != 0 && value != 1) raise(VLA_E_INVALID, "value must be 0 or 1");
        m->opt_persistent = (int)value;
        break;
      case VLA_OPT_BARRIER_SPIN_LIMIT:
        if (value < 0 || value > (1ll << 30)) raise(VLA_E_INVALID, "spin limit outside 0..2^30");
        m->opt_spin_limit = (int)value;
        break;
      case VLA_OPT_BARRIER_TEST_UNREACHABLE:
        if (value != 0 && value != 1) raise(VLA_E_INVALID, "value must be 0 or 1");
        m->opt_unreachable = (int)value;
        break;
      default:
        raise(VLA_E_INVALID, "unknown or read-only option");
    }
  });
}

vla_status vla_get_option(const vla_model* m, int32_t key, int64_t* value) {
  return guarded([&] {
    if (!m || !value) raise(VLA_E_INVALID, "null argument");
    switch (key) {
      case VLA_OPT_PERSISTENT_DECODE: *value = m->opt_persistent; break;
      case VLA_OPT_BARRIER_SPIN_LIMIT: *value = m->opt_spin_limit; break;
      case VLA_OPT_BARRIER_TEST_UNREACHABLE: *value = m->opt_unreachable; break;
      case VLA_INFO_LAST_DECODE_PERSISTENT: *value = m->last_persistent ? 1 : 0; break;
      default: raise(VLA_E_INVALID, "unknown option");
    }
  });
}

vla_status vla_profile_enable(vla_model* m, int32_t kernel_class) {
  return guarded([&] {
    if (!m) raise(VLA_E_INVALID, "null model");
    if (kernel_class < 0 || kernel_class >= VLA_K_COUNT) raise(VLA_E_INVALID, "kernel class");
    m->prof_cls = kernel_class;
    m->prof.used = 0;
    m->prof.calls = 0;
  });
}

vla_status vla_profile_replay(vla_model* m, int32_t kernel_class, int32_t reps, void* stream,
                              double* ms_per_launch) {
  return guarded([&] {
    if (!m) raise(VLA_E_INVALID, "null model");
    if (kernel_class != VLA_K_GEMV_GATEUP) raise(VLA_E_INVALID, "replay: gated projection only");
    if (m->cfg.n_layers < 1 || m->cfg.ffn < 1) raise(VLA_E_INVALID, "model has no gated projection");
    if (reps < 1 || reps > 1000) raise(VLA_E_INVALID, "reps out of range");
    const hipStream_t st = (hipStream_t)stream;
    // the K/V-only last layer of a prefix model has no FFN
    const int nl = m->cfg.kv_only_last ? m->cfg.n_layers - 1 : m->cfg.n_layers;
    if (nl < 1) raise(VLA_E_INVALID, "model has no gated projection");
    hipEvent_t e0, e1;
    HIPCHK(hipEventCreate(&e0));
    HIPCHK(hipEventCreate(&e1));
    HIPCHK(hipEventRecord(e0, st));
    for (int r = 0; r < reps; ++r)
      for (int l = 0; l < nl; ++l) HIPCHK(launch_gemv(decode_gateup_args(m, l), m->dt, st, nullptr));
    HIPCHK(hipEventRecord(e1, st));
    HIPCHK(hipEventSynchronize(e1));
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, e0, e1));
    HIPCHK(hipEventDestroy(e0));
    HIPCHK(hipEventDestroy(e1));
    if (ms_per_launch) *ms_per_launch = (double)ms / ((double)reps * nl);
  });
}

vla_status vla_probe_mfma_peak(float* out, int32_t blocks, int32_t iters, void* stream,
                               double* out_tflops) {
  return guarded([&] {
    if (!out || !out_tflops) raise(VLA_E_INVALID, "null argument");
    if (blocks < 1 || blocks > 65536 || iters < 1 || iters > 1000000)
      raise(VLA_E_INVALID, "blocks in 1..65536, iters in 1..1000000");
    const hipStream_t st = (hipStream_t)stream;
    HIPCHK(launch_mfma_peak(out, blocks, 1, st));  // warm-up
    hipEvent_t e0, e1;
    HIPCHK(hipEventCreate(&e0));
    HIPCHK(hipEventCreate(&e1));
    HIPCHK(hipEventRecord(e0, st));
    HIPCHK(launch_mfma_peak(out, blocks, iters, st));
    HIPCHK(hipEventRecord(e1, st));
    HIPCHK(hipEventSynchronize(e1));
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, e0, e1));
    HIPCHK(hipEventDestroy(e0));
    HIPCHK(hipEventDestroy(e1));
    const double flop = (double)blocks * 4.0 * (double)iters * 4.0 * 32768.0;
    *out_tflops = flop / ((double)ms * 1e-3) / 1e12;
  });
}

vla_status vla_probe_read_bandwidth(int64_t bytes, int32_t reps, void* stream, double* out_gbs) {
  return guarded([&] {
    if (!out_gbs) raise(VLA_E_INVALID, "null argument");
    if (bytes < (1 << 20) || bytes > ((int64_t)1 << 36) || bytes % 16 || reps < 1 || reps > 100)
      raise(VLA_E_INVALID, "bytes a multiple of 16 in 1 MiB..64 GiB, reps in 1..100");
    const hipStream_t st = (hipStream_t)stream;
    // (workgroups, consecutive 4 KB pieces per iteration): the best of three shapes
    // is the reported ceiling
    const int shapes[3][2] = {{512, 4}, {1024, 1}, {1024, 2}};
    const int max_blocks = 1024;
    void* buf = nullptr;
    uint32_t* out = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    auto cleanup = [&] {
      if (e0) (void)hipEventDestroy(e0);
      if (e1) (void)hipEventDestroy(e1);
      (void)hipFree(buf);
      (void)hipFree(out);
    };
    try {
      HIPCHK(hipMalloc(&buf, (size_t)bytes));
      HIPCHK(hipMalloc(&out, (size_t)max_blocks * 256 * sizeof(uint32_t)));
      HIPCHK(hipMemsetAsync(buf, 0, (size_t)bytes, st));
      HIPCHK(hipEventCreate(&e0));
      HIPCHK(hipEventCreate(&e1));
      double best = 0.0;
      for (const auto& sh : shapes) {
        HIPCHK(launch_read_probe(buf, bytes, out, sh[0], sh[1], st));  // warm-up
        HIPCHK(hipEventRecord(e0, st));
        for (int r = 0; r < reps; ++r) HIPCHK(launch_read_probe(buf, bytes, out, sh[0], sh[1], st));
        HIPCHK(hipEventRecord(e1, st));
        HIPCHK(hipEventSynchronize(e1));
        float ms = 0.f;
        HIPCHK(hipEventElapsedTime(&ms, e0, e1));
        best = std::max(best, (double)bytes * reps / ((double)ms * 1e-3) / 1e9);
      }
      *out_gbs = best;
    } catch (...) {
      cleanup();
      throw;
    }
    cleanup();
  });
}

vla_status vla_probe_barrier(int32_t grid, int32_t nbar, void* stream, double* out_us) {
  return guarded([&] {
    if (!out_us) raise(VLA_E_INVALID, "null argument");
    const int gmax = barrier_probe_max_grid();
    if (grid < 1 || grid > gmax || nbar < 1 || nbar > 100000)
      raise(VLA_E_INVALID, "grid outside 1.." + std::to_string(gmax) + " or nbar outside 1..100000");
    const hipStream_t st = (hipStream_t)stream;
    unsigned long long* bar = nullptr;
    float* scratch = nullptr;
    HIPCHK(hipMalloc(&bar, kBarStateWords * sizeof(unsigned long long)));
    HIPCHK(hipMalloc(&scratch, (size_t)grid * 256 * sizeof(float)));
    hipEvent_t e0 = nullptr, e1 = nullptr;
    auto cleanup = [&] {
      if (e0) (void)hipEventDestroy(e0);
      if (e1) (void)hipEventDestroy(e1);
      (void)hipFree(bar);
      (void)hipFree(scratch);
    };
    try {
      HIPCHK(hipMemsetAsync(bar, 0, kBarStateWords * sizeof(unsigned long long), st));
      HIPCHK(hipMemsetAsync(scratch, 0, (size_t)grid * 256 * sizeof(float), st));
      HIPCHK(hipEventCreate(&e0));
      HIPCHK(hipEventCreate(&e1));
      // an untimed launch first (the first cooperative launch of the kernel pays a
      // one-time cost); the timed launch then uses the other state set
      HIPCHK(launch_barrier_probe(bar, scratch, grid, 10, 0, 1 << 20, st));
      HIPCHK(hipEventRecord(e0, st));
      HIPCHK(launch_barrier_probe(bar, scratch, grid, nbar, 1, 1 << 20, st));
      HIPCHK(hipEventRecord(e1, st));
      HIPCHK(hipEventSynchronize(e1));
      float ms = 0.f;
      HIPCHK(hipEventElapsedTime(&ms, e0, e1));
      int err = 0;
      HIPCHK(hipMemcpy(&err, bar, sizeof(int), hipMemcpyDeviceToHost));
      if (err == 2) raise(VLA_E_HIP, "the barrier probe found an XCD id outside 0..7");
      if (err) raise(VLA_E_TIMEOUT, "a probe barrier gave up");
      *out_us = (double)ms * 1e3 / nbar;
    } catch (...) {
      cleanup();
      throw;
    }
    cleanup();
  });
}

vla_status vla_profile_read(vla_model* m, double* total_ms, int32_t* launches) {
  return guarded([&] {
    if (!m) raise(VLA_E_INVALID, "null model");
    double tot = 0.0;
    for (int i = 0; i + 1 < m->prof.used; i += 2) {
      HIPCHK(hipEventSynchronize(m->prof.ev[i + 1]));
      float ms = 0.f;
      HIPCHK(hipEventElapsedTime(&ms, m->prof.ev[i], m->prof.ev[i + 1]));
      tot += ms;
    }
    if (total_ms) *total_ms = tot;
    if (launches) *launches = m->prof.calls;
  });
}

// ---- action expert ("Running VLAs at Real-time Speed", section 2) ----
namespace {
// an expert bound to `prefix`; `share` (non-null): with that expert's weights
vla_status expert_create(vla_model* prefix, const vla_config* cfg, int32_t n_actions,
                         const vla_expert* share, vla_expert** out) {
  vla_expert* e = nullptr;
  vla_status st = guarded([&] {
    if (!out) raise(VLA_E_INVALID, "out is NULL");
    *out = nullptr;
    if (!prefix || !cfg) raise(VLA_E_INVALID, "null argument");
    if (n_actions < 1) raise(VLA_E_INVALID, "n_actions must be >= 1");
    const vla_config& pc = prefix->cfg;
    vla_config c = *cfg;
    if (c.vocab != 0 || c.kv_only_last)
      raise(VLA_E_INVALID, "invalid config: an expert has no vocabulary and all layers full");
    if (c.n_layers != pc.n_layers || c.n_kv_heads != pc.n_kv_heads ||
        c.head_dim != pc.head_dim || c.act_dtype != pc.act_dtype ||
        c.block_tokens != pc.block_tokens)
      raise(VLA_E_INVALID, "invalid config: layers, KV heads, head_dim, act_dtype and "
                           "block_tokens must match the prefix model");
    if (c.hidden > 4096) raise(VLA_E_INVALID, "invalid config: an expert's hidden must be <= 4096");
    c.num_blocks = pc.num_blocks;
    c.max_frames = 1;
    c.max_chunk = n_actions;
    validate_cfg(&c);
    HIPCHK(hipSetDevice(prefix->dev));
    e = new vla_expert();
    e->prefix = prefix;
    e->n_actions = n_actions;
    e->m = new vla_model();
    build_model(e->m, c, prefix, share ? share->m : nullptr);
    const int nres = (n_actions + c.block_tokens - 1) / c.block_tokens;
    if (!prefix->pool.alloc(nres, &e->reserved))
      raise(VLA_E_NO_BLOCKS, "no free blocks in the prefix pool for the action chunk's K/V");
    e->d_view = (int*)dalloc(e->m, 2 * (size_t)pc.num_blocks * sizeof(int));
    staging_init(e->st_view, 2 * (size_t)pc.num_blocks * sizeof(int));
    *out = e;
  });
  if (st != VLA_OK && e) {
    std::string keep = g_err;
    vla_expert_destroy(e);
    g_err = keep;
  }
  return st;
}
}  // namespace

vla_status vla_expert_create(vla_model* prefix, const vla_config* cfg, int32_t n_actions,
                             vla_expert** out) {
  return expert_create(prefix, cfg, n_actions, nullptr, out);
}

vla_status vla_expert_create_sibling(vla_model* prefix, const vla_expert* src, vla_expert** out) {
  if (!src) {
    g_err = "null source expert";
    if (out) *out = nullptr;
    return VLA_E_INVALID;
  }
  return expert_create(prefix, &src->m->cfg, src->n_actions, src, out);
}

void vla_expert_destroy(vla_expert* e) {
  if (!e) return;
  if (e->gexec) (void)hipGraphExecDestroy(e->gexec);
  if (e->m) destroy(e->m);
  staging_free(e->st_view);
  if (!e->reserved.empty()) {
    std::vector<int> rb(e->reserved.rbegin(), e->reserved.rend());
    e->prefix->pool.release(rb.data(), (int)rb.size());
  }
  delete e;
}

namespace {
// The Euler loop on x. graph: the launches are captured once into a graph on `st`
// (not the null stream) and replayed while the loop's arguments stay the same; the
// block list is uploaded outside the graph on every call (the kernels read it).
void expert_denoise(vla_expert* e, float* x, int32_t n_steps, double dt, hipStream_t st,
                    bool graph) {
  if (!e || !x) raise(VLA_E_INVALID, "null argument");
  if (n_steps < 1 || !(dt > 0.0) || !std::isfinite(dt))
    raise(VLA_E_INVALID, "need n_steps >= 1 and a finite dt > 0");
  vla_model* p = e->prefix;
  vla_model* m = e->m;
  HIPCHK(hipSetDevice(m->dev));
  const int bt = bt_of(p), n = e->n_actions, H = m->cfg.hidden, cap = p->cfg.num_blocks;
  // the blocks of every pass: the prefix's resident blocks in logical order, then
  // the chunk's own (its K/V are rewritten by every pass)
  int* h = (int*)staging_acquire(e->st_view);
  int nb = 0;
  for (const auto& sg : p->segs)
    for (size_t i = 0; i < sg.blocks.size(); ++i) {
      h[nb] = sg.blocks[i];
      h[cap + nb] = std::min(bt, sg.ntok - (int)i * bt);
      ++nb;
    }
  const int cb0 = nb;
  for (size_t i = 0; i < e->reserved.size(); ++i) {
    h[nb] = e->reserved[i];
    h[cap + nb] = std::min(bt, n - (int)i * bt);
    ++nb;
  }
  KvView v;
  v.blk = e->d_view;
  v.ntok = e->d_view + cap;
  v.nlb = nb;
  v.last_ntok = h[cap + nb - 1];
  v.causal = 0;
  staging_upload(e->st_view, e->d_view, 2 * (size_t)cap * sizeof(int), st);
  if (e->temb_cap < n_steps) {  // (grown on demand; the old table stays until destroy)
    if (e->gexec) {              // a captured loop may refer to the old table
      HIPCHK(hipGraphExecDestroy(e->gexec));
      e->gexec = nullptr;
    }
    e->temb = (float*)dalloc(m, (size_t)n_steps * H * sizeof(float));
    e->temb_cap = n_steps;
  }
  const float eps = m->cfg.rms_eps;
  const int64_t pos = p->next_pos;
  auto enqueue = [&] {
    HIPCHK(launch_flow_temb(e->temb, n_steps, H, dt, st));
    // iteration k: h = x + temb(tau_k), the layers, x += dt * RMSNorm(h); each boundary
    // (the Euler step of k and the input of k + 1) is one launch
    HIPCHK(launch_flow_step(x, (float*)m->x, e->temb, m->norm_ones, m->u, m->u_lo, n, H, eps,
                            (float)dt, false, m->dt, st));
    for (int k = 0; k < n_steps; ++k) {
      run_layers(m, v, n, pos, cb0, 0, /*decode=*/false, st, false, /*norm_ready=*/true);
      const float* next = k + 1 < n_steps ? e->temb + (size_t)(k + 1) * H : nullptr;
      HIPCHK(launch_flow_step(x, (float*)m->x, next, m->norm_ones, m->u, m->u_lo, n, H, eps,
                              (float)dt, true, m->dt, st));
    }
  };
  if (!graph || st == nullptr || m->prof_cls != VLA_K_NONE) {
    enqueue();
    return;
  }
  vla_expert::GraphKey key;
  key.x = x;
  key.n_steps = n_steps;
  key.nb = nb;
  key.last_ntok = v.last_ntok;
  key.cb0 = cb0;
  key.dt = dt;
  key.pos = pos;
  if (!e->gexec || !(key == e->gkey)) {
    if (e->gexec) {
      HIPCHK(hipGraphExecDestroy(e->gexec));
      e->gexec = nullptr;
    }
    hipGraph_t g = nullptr;
    HIPCHK(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal));
    try {
      enqueue();
    } catch (...) {
      hipGraph_t junk = nullptr;
      (void)hipStreamEndCapture(st, &junk);
      if (junk) (void)hipGraphDestroy(junk);
      throw;
    }
    HIPCHK(hipStreamEndCapture(st, &g));
    const hipError_t ie = hipGraphInstantiate(&e->gexec, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (ie != hipSuccess) e->gexec = nullptr;
    HIPCHK(ie);
    e->gkey = key;
  }
  HIPCHK(hipGraphLaunch(e->gexec, st));
}
}  // namespace

vla_status vla_expert_denoise(vla_expert* e, float* x, int32_t n_steps, double dt, void* stream) {
  return guarded([&] { expert_denoise(e, x, n_steps, dt, (hipStream_t)stream, false); });
}

// ---- overlapped prefix and expert streams ("Running VLAs at Real-time Speed",
// section 6.1: the bandwidth-bound expert and the compute-bound prefix model on two
// streams, the expert iterating on the newest finished prefix K/V) ----
struct vla_pipeline {
  vla_model* P[2] = {nullptr, nullptr};   // [0] the caller's prefix model, [1] its sibling
  vla_expert* E[2] = {nullptr, nullptr};  // [0] the caller's expert, [1] its sibling on P[1]
  hipStream_t sv = nullptr, sa = nullptr; // prefix stream, expert stream (default priority)
  hipEvent_t pre_done[2] = {nullptr, nullptr};  // the latest prefill into buffer b has finished
  hipEvent_t act_done[2] = {nullptr, nullptr};  // the latest action run on buffer b has finished
  hipEvent_t in_ready = nullptr;                // the caller's inputs are ready (caller's stream)
  int64_t frame[2] = {-1, -1};                  // frame held (or being written) by buffer b
  bool acted[2] = {false, false};               // act_done[b] has been recorded
  int64_t next_frame = 0;
  int64_t prefills = 0, acts = 0, acts_on_older = 0;
};

namespace {
void pipeline_free(vla_pipeline* p) {
  if (!p) return;
  if (p->sv) (void)hipStreamSynchronize(p->sv);
  if (p->sa) (void)hipStreamSynchronize(p->sa);
  if (p->E[1]) vla_expert_destroy(p->E[1]);
  if (p->P[1]) destroy(p->P[1]);
  for (int b = 0; b < 2; ++b) {
    if (p->pre_done[b]) (void)hipEventDestroy(p->pre_done[b]);
    if (p->act_done[b]) (void)hipEventDestroy(p->act_done[b]);
  }
  if (p->in_ready) (void)hipEventDestroy(p->in_ready);
  if (p->sv) (void)hipStreamDestroy(p->sv);
  if (p->sa) (void)hipStreamDestroy(p->sa);
  delete p;
}
}  // namespace

vla_status vla_pipeline_create(vla_model* prefix, vla_expert* expert, vla_pipeline** out) {
  vla_pipeline* p = nullptr;
  vla_status st = guarded([&] {
    if (!out) raise(VLA_E_INVALID, "out is NULL");
    *out = nullptr;
    if (!prefix || !expert) raise(VLA_E_INVALID, "null argument");
    if (expert->prefix != prefix) raise(VLA_E_INVALID, "the expert is not bound to this prefix model");
    HIPCHK(hipSetDevice(prefix->dev));
    p = new vla_pipeline();
    p->P[0] = prefix;
    p->E[0] = expert;
    {
      vla_model* m = nullptr;
      const vla_status ms = vla_model_create_sibling(prefix, &m);
      if (ms != VLA_OK) raise(ms, g_err);
      p->P[1] = m;
      vla_expert* e = nullptr;
      const vla_status es = vla_expert_create_sibling(m, expert, &e);
      if (es != VLA_OK) raise(es, g_err);
      p->E[1] = e;
    }
    HIPCHK(hipStreamCreateWithFlags(&p->sv, hipStreamNonBlocking));
    HIPCHK(hipStreamCreateWithFlags(&p->sa, hipStreamNonBlocking));
    for (int b = 0; b < 2; ++b) {
      HIPCHK(hipEventCreateWithFlags(&p->pre_done[b], hipEventDisableTiming));
      HIPCHK(hipEventCreateWithFlags(&p->act_done[b], hipEventDisableTiming));
    }
    HIPCHK(hipEventCreateWithFlags(&p->in_ready, hipEventDisableTiming));
    *out = p;
  });
  if (st != VLA_OK && p) {
    std::string keep = g_err;
    pipeline_free(p);
    g_err = keep;
  }
  return st;
}

void vla_pipeline_destroy(vla_pipeline* p) { pipeline_free(p); }

vla_status vla_pipeline_prefill(vla_pipeline* p, const void* embeds, int32_t n, void* stream,
                                int64_t* out_frame) {
  return guarded([&] {
    if (!p || !embeds) raise(VLA_E_INVALID, "null argument");
    if (n < 1 || n > p->P[0]->cfg.max_chunk) raise(VLA_E_INVALID, "chunk length out of range");
    HIPCHK(hipSetDevice(p->P[0]->dev));
    const int b = (int)(p->next_frame & 1);
    // the caller's embeddings are ready; no action run still reads this buffer
    HIPCHK(hipEventRecord(p->in_ready, (hipStream_t)stream));
    HIPCHK(hipStreamWaitEvent(p->sv, p->in_ready, 0));
    if (p->acted[b]) HIPCHK(hipStreamWaitEvent(p->sv, p->act_done[b], 0));
    vla_model* m = p->P[b];
    p->frame[b] = -1;  // (no frame here until this prefill is enqueued)
    vla_status s = vla_kv_rollback(m, -1);
    if (s != VLA_OK) raise(s, g_err);
    int32_t fid = -1;
    s = vla_prefill_chunk(m, nullptr, embeds, n, &fid, p->sv);
    if (s != VLA_OK) raise(s, g_err);
    HIPCHK(hipEventRecord(p->pre_done[b], p->sv));
    p->frame[b] = p->next_frame++;
    ++p->prefills;
    if (out_frame) *out_frame = p->frame[b];
  });
}

vla_status vla_pipeline_act(vla_pipeline* p, float* x, int32_t n_steps, double dt, void* stream,
                            int64_t* out_frame) {
  return guarded([&] {
    if (!p || !x) raise(VLA_E_INVALID, "null argument");
    if (p->frame[0] < 0 && p->frame[1] < 0) raise(VLA_E_STATE, "no prefix submitted yet");
    HIPCHK(hipSetDevice(p->P[0]->dev));
    // the newest buffer whose prefill has finished; if neither has, the older one,
    // waited for on the expert stream
    int order[2];
    const bool first_newer = p->frame[0] > p->frame[1];
    order[0] = first_newer ? 0 : 1;
    order[1] = 1 - order[0];
    int b = -1;
    for (int i = 0; i < 2 && b < 0; ++i) {
      const int c = order[i];
      if (p->frame[c] < 0) continue;
      const hipError_t q = hipEventQuery(p->pre_done[c]);
      if (q == hipSuccess) b = c;
      else if (q != hipErrorNotReady) HIPCHK(q);
    }
    bool wait = false;
    if (b < 0) {
      b = p->frame[order[1]] >= 0 ? order[1] : order[0];
      wait = true;
    }
    HIPCHK(hipEventRecord(p->in_ready, (hipStream_t)stream));
    HIPCHK(hipStreamWaitEvent(p->sa, p->in_ready, 0));
    if (wait) HIPCHK(hipStreamWaitEvent(p->sa, p->pre_done[b], 0));
    // the loop's ~1,600 launches from one graph: the host would otherwise spend about as
    // long enqueueing them as the device spends running them, and fall behind
    expert_denoise(p->E[b], x, n_steps, dt, p->sa, /*graph=*/true);
    HIPCHK(hipEventRecord(p->act_done[b], p->sa));
    p->acted[b] = true;
    // the caller's stream sees x after the run
    HIPCHK(hipStreamWaitEvent((hipStream_t)stream, p->act_done[b], 0));
    ++p->acts;
    if (p->frame[b] < p->next_frame - 1) ++p->acts_on_older;
    if (out_frame) *out_frame = p->frame[b];
  });
}

vla_status vla_pipeline_sync(vla_pipeline* p) {
  return guarded([&] {
    if (!p) raise(VLA_E_INVALID, "null pipeline");
    HIPCHK(hipSetDevice(p->P[0]->dev));
    HIPCHK(hipStreamSynchronize(p->sv));
    HIPCHK(hipStreamSynchronize(p->sa));
  });
}

vla_status vla_pipeline_stats(const vla_pipeline* p, int64_t* prefills, int64_t* acts,
                              int64_t* acts_on_older) {
  return guarded([&] {
    if (!p) raise(VLA_E_INVALID, "null pipeline");
    if (prefills) *prefills = p->prefills;
    if (acts) *acts = p->acts;
    if (acts_on_older) *acts_on_older = p->acts_on_older;
  });
}

// ---- reconciliation on a second state ("CSR: Infinite-Horizon Real-Time
// Policies with Massive Cached State Representations", section III-E and
// Appendix D: after an eviction, a second resource re-prefills the kept state
// while the first keeps serving, then catches up on the chunks that arrived
// meanwhile and the two swap roles). On one GPU: a sibling model over the same
// weights and a second stream. Frames are logged with their inputs so that the
// spare model can recompute their K/V at contiguous positions. ----
struct AsrFrame {
  int64_t id = -1;               // reconciler frame id (monotonic)
  int n = 0;
  std::vector<int32_t> tokens;   // host ids (tokens input), or
  int eslot = -1;                // a slot of the embeddings log (device)
  int fid[2] = {-1, -1};         // the frame's id in model 0 / model 1 (-1: not there)
  bool alive = true;             // still resident in the serving model
};

struct vla_asr {
  vla_model* M[2] = {nullptr, nullptr};  // [0] the caller's model, [1] its sibling (owned)
  int serving = 0;
  hipStream_t sr = nullptr;               // the spare model's stream (default priority)
  hipEvent_t rec_done = nullptr, in_ready = nullptr;
  std::vector<AsrFrame> log;              // frames in arrival order
  void* elog = nullptr;                   // embeddings log: n_eslots x max_chunk x hidden
  size_t eslot_bytes = 0;
  int n_eslots = 0;
  std::vector<int> free_eslots;
  bool reconciling = false;
  int64_t next_id = 0;
  int64_t reconciliations = 0, swaps = 0, replayed = 0;
};

namespace {
// drop log entries that no model needs any more (their embedding slots are free again)
void asr_compact(vla_asr* a) {
  std::vector<AsrFrame> keep;
  for (auto& f : a->log) {
    if (f.alive || f.fid[0] >= 0 || f.fid[1] >= 0) {
      keep.push_back(std::move(f));
    } else if (f.eslot >= 0) {
      a->free_eslots.push_back(f.eslot);
    }
  }
  a->log.swap(keep);
}
// prefill every live frame the spare does not hold yet, in arrival order, on the spare stream
void asr_replay(vla_asr* a) {
  const int sp = 1 - a->serving;
  vla_model* m = a->M[sp];
  for (auto& f : a->log) {
    if (!f.alive || f.fid[sp] >= 0) continue;
    const void* emb = f.eslot >= 0 ? (const char*)a->elog + (size_t)f.eslot * a->eslot_bytes : nullptr;
    int32_t fid = -1;
    const vla_status s = vla_prefill_chunk(m, emb ? nullptr : f.tokens.data(), emb, f.n, &fid, a->sr);
    if (s != VLA_OK) raise(s, g_err);
    f.fid[sp] = fid;
    ++a->replayed;
  }
}
void asr_free(vla_asr* a) {
  if (!a) return;
  if (a->sr) (void)hipStreamSynchronize(a->sr);
  if (a->M[1]) destroy(a->M[1]);
  if (a->elog) (void)hipFree(a->elog);
  if (a->rec_done) (void)hipEventDestroy(a->rec_done);
  if (a->in_ready) (void)hipEventDestroy(a->in_ready);
  if (a->sr) (void)hipStreamDestroy(a->sr);
  delete a;
}
}  // namespace

vla_status vla_asr_create(vla_model* primary, vla_asr** out) {
  vla_asr* a = nullptr;
  vla_status st = guarded([&] {
    if (!out) raise(VLA_E_INVALID, "out is NULL");
    *out = nullptr;
    if (!primary) raise(VLA_E_INVALID, "null model");
    if (!primary->segs.empty()) raise(VLA_E_STATE, "the model must be empty (no logged inputs)");
    HIPCHK(hipSetDevice(primary->dev));
    a = new vla_asr();
    a->M[0] = primary;
    vla_model* s = nullptr;
    const vla_status ms = vla_model_create_sibling(primary, &s);
    if (ms != VLA_OK) raise(ms, g_err);
    a->M[1] = s;
    HIPCHK(hipStreamCreateWithFlags(&a->sr, hipStreamNonBlocking));
    HIPCHK(hipEventCreateWithFlags(&a->rec_done, hipEventDisableTiming));
    HIPCHK(hipEventCreateWithFlags(&a->in_ready, hipEventDisableTiming));
    *out = a;
  });
  if (st != VLA_OK && a) {
    std::string keep = g_err;
    asr_free(a);
    g_err = keep;
  }
  return st;
}

void vla_asr_destroy(vla_asr* a) { asr_free(a); }

vla_model* vla_asr_model(const vla_asr* a) { return a ? a->M[a->serving] : nullptr; }

vla_status vla_asr_prefill(vla_asr* a, const int32_t* tokens, const void* embeds, int32_t n,
                           void* stream, int64_t* out_id) {
  return guarded([&] {
    if (!a) raise(VLA_E_INVALID, "null reconciler");
    vla_model* m = a->M[a->serving];
    if ((tokens == nullptr) == (embeds == nullptr))
      raise(VLA_E_INVALID, "exactly one of tokens / embeds must be given");
    if (n < 1 || n > m->cfg.max_chunk) raise(VLA_E_INVALID, "chunk length out of range");
    HIPCHK(hipSetDevice(m->dev));
    AsrFrame f;
    f.n = n;
    if (tokens) {
      f.tokens.assign(tokens, tokens + n);
    } else {
      if (!a->elog) {  // the embeddings log, on first use: 2 x max_frames chunks
        a->eslot_bytes = (size_t)m->cfg.max_chunk * m->cfg.hidden * m->esz;
        a->n_eslots = 2 * m->cfg.max_frames;
        HIPCHK(hipMalloc(&a->elog, a->eslot_bytes * a->n_eslots));
        for (int i = a->n_eslots - 1; i >= 0; --i) a->free_eslots.push_back(i);
      }
      if (a->free_eslots.empty()) raise(VLA_E_NO_BLOCKS, "the embeddings log is full");
      f.eslot = a->free_eslots.back();
      HIPCHK(hipMemcpyAsync((char*)a->elog + (size_t)f.eslot * a->eslot_bytes, embeds,
                            (size_t)n * m->cfg.hidden * m->esz, hipMemcpyDeviceToDevice,
                            (hipStream_t)stream));
    }
    int32_t fid = -1;
    const vla_status s = vla_prefill_chunk(m, f.tokens.empty() ? nullptr : f.tokens.data(),
                                           embeds, n, &fid, stream);
    if (s != VLA_OK) raise(s, g_err);
    if (f.eslot >= 0) a->free_eslots.pop_back();
    f.fid[a->serving] = fid;
    f.id = a->next_id++;
    a->log.push_back(std::move(f));
    if (out_id) *out_id = a->log.back().id;
  });
}

vla_status vla_asr_evict(vla_asr* a, int32_t policy, int32_t layer, void* stream, int64_t* out_id,
                         double* out_score) {
  return guarded([&] {
    if (!a) raise(VLA_E_INVALID, "null reconciler");
    vla_model* m = a->M[a->serving];
    int32_t fid = -1;
    const vla_status s = vla_kv_evict(m, policy, layer, &fid, out_score, stream);
    if (s != VLA_OK) raise(s, g_err);
    const int sp = 1 - a->serving;
    int64_t id = -1;
    for (auto& f : a->log)
      if (f.fid[a->serving] == fid) {
        id = f.id;
        f.alive = false;
        f.fid[a->serving] = -1;
        // a spare that already holds it rolls back to the last live frame before it, so
        // that the next catch-up recomputes the later frames at contiguous positions (its
        // work is ordered on the spare stream)
        if (a->reconciling && f.fid[sp] >= 0) {
          int keep = -1;
          for (const auto& g : a->log) {
            if (&g == &f) break;
            if (g.fid[sp] >= 0) keep = g.fid[sp];
          }
          const vla_status rs = vla_kv_rollback(a->M[sp], keep);
          if (rs != VLA_OK) raise(rs, g_err);
          bool after = false;
          for (auto& g : a->log) {
            after = after || &g == &f;
            if (after) g.fid[sp] = -1;
          }
        }
        break;
      }
    if (!a->reconciling) asr_compact(a);
    if (out_id) *out_id = id;
  });
}

vla_status vla_asr_reconcile_begin(vla_asr* a, void* stream) {
  return guarded([&] {
    if (!a) raise(VLA_E_INVALID, "null reconciler");
    if (a->reconciling) raise(VLA_E_STATE, "a reconciliation is already running");
    const int sp = 1 - a->serving;
    vla_model* m = a->M[sp];
    HIPCHK(hipSetDevice(m->dev));
    // the spare's earlier work (as the serving model) and the logged inputs are ordered
    // before its re-prefill
    HIPCHK(hipEventRecord(a->in_ready, (hipStream_t)stream));
    HIPCHK(hipStreamWaitEvent(a->sr, a->in_ready, 0));
    const vla_status s = vla_kv_rollback(m, -1);
    if (s != VLA_OK) raise(s, g_err);
    for (auto& f : a->log) f.fid[sp] = -1;
    asr_compact(a);
    a->reconciling = true;
    ++a->reconciliations;
    asr_replay(a);
    HIPCHK(hipEventRecord(a->rec_done, a->sr));
  });
}

vla_status vla_asr_try_swap(vla_asr* a, void* stream, int32_t* swapped) {
  return guarded([&] {
    if (!a) raise(VLA_E_INVALID, "null reconciler");
    if (swapped) *swapped = 0;
    if (!a->reconciling) raise(VLA_E_STATE, "no reconciliation is running");
    HIPCHK(hipSetDevice(a->M[0]->dev));
    // catch up on the frames that arrived since the last replay (their inputs are
    // ready on the caller's stream); rec_done marks the end of the spare's work so far
    const int sp = 1 - a->serving;
    bool behind = false;
    for (const auto& f : a->log) behind = behind || (f.alive && f.fid[sp] < 0);
    if (behind) {
      HIPCHK(hipEventRecord(a->in_ready, (hipStream_t)stream));
      HIPCHK(hipStreamWaitEvent(a->sr, a->in_ready, 0));
      asr_replay(a);
      HIPCHK(hipEventRecord(a->rec_done, a->sr));
    }
    const hipError_t q = hipEventQuery(a->rec_done);
    if (q == hipErrorNotReady) return;
    HIPCHK(q);
    // the spare holds every live frame at contiguous positions: it becomes the serving
    // model, and the caller's stream is ordered after its work
    HIPCHK(hipStreamWaitEvent((hipStream_t)stream, a->rec_done, 0));
    const int old = a->serving;
    a->serving = 1 - old;
    for (auto& f : a->log) f.fid[old] = -1;
    a->reconciling = false;
    ++a->swaps;
    asr_compact(a);
    if (swapped) *swapped = 1;
  });
}

vla_status vla_asr_sync(vla_asr* a) {
  return guarded([&] {
    if (!a) raise(VLA_E_INVALID, "null reconciler");
    HIPCHK(hipSetDevice(a->M[0]->dev));
    HIPCHK(hipStreamSynchronize(a->sr));
  });
}

vla_status vla_asr_frames(const vla_asr* a, int64_t* ids, int32_t cap, int32_t* n_out) {
  return guarded([&] {
    if (!a || !n_out || (!ids && cap > 0) || cap < 0) raise(VLA_E_INVALID, "bad argument");
    int n = 0;
    for (const auto& f : a->log)
      if (f.alive) {
        if (n < cap) ids[n] = f.id;
        ++n;
      }
    *n_out = n;
  });
}

vla_status vla_asr_stats(const vla_asr* a, int64_t* reconciliations, int64_t* swaps,
                         int64_t* frames_replayed, int32_t* reconciling) {
  return guarded([&] {
    if (!a) raise(VLA_E_INVALID, "null reconciler");
    if (reconciliations) *reconciliations = a->reconciliations;
    if (swaps) *swaps = a->swaps;
    if (frames_replayed) *frames_replayed = a->replayed;
    if (reconciling) *reconciling = a->reconciling ? 1 : 0;
  });
}

// ---- host-only pool ----
vla_status vla_pool_create(int32_t num_blocks, vla_pool** out) {
  return guarded([&] {
    if (!out || num_blocks < 0) raise(VLA_E_INVALID, "bad argument");
    *out = new vla_pool();
    (*out)->p.reset(num_blocks);
  });
}
void vla_pool_destroy(vla_pool* p) { delete p; }
vla_status vla_pool_alloc(vla_pool* p, int32_t n, int32_t* out) {
  return guarded([&] {
    if (!p || (!out && n > 0) || n < 0) raise(VLA_E_INVALID, "bad argument");
    std::vector<int> got;
    if (!p->p.alloc(n, &got)) raise(VLA_E_NO_BLOCKS, "not enough free blocks");
    for (int i = 0; i < n; ++i) out[i] = got[i];
  });
}
vla_status vla_pool_release(vla_pool* p, const int32_t* blocks, int32_t n) {
  return guarded([&] {
    if (!p || (!blocks && n > 0) || n < 0) raise(VLA_E_INVALID, "bad argument");
    if (!p->p.release(blocks, n)) raise(VLA_E_INVALID, "block id out of range or already free");
  });
}
int32_t vla_pool_free_count(const vla_pool* p) { return p ? p->p.free_count() : 0; }
vla_status vla_pool_free_list(const vla_pool* p, int32_t* out, int32_t cap, int32_t* n_out) {
  return guarded([&] {
    if (!p || !n_out) raise(VLA_E_INVALID, "null argument");
    copy_free_list(p->p, out, cap, n_out);
  });
}

// ---- admission control ("Can an LLM Forget the Right Things?", section 4) ----
vla_status vla_admission_create(const vla_admission_config* cfg, vla_admission** out) {
  return guarded([&] {
    if (!out || !cfg) raise(VLA_E_INVALID, "null argument");
    *out = nullptr;
    if (!(cfg->deadline_ms > 0.0) || !std::isfinite(cfg->deadline_ms))
      raise(VLA_E_INVALID, "deadline_ms must be finite and > 0");
    if (!(cfg->safety_margin_ms >= 0.0) || !std::isfinite(cfg->safety_margin_ms))
      raise(VLA_E_INVALID, "safety_margin_ms must be finite and >= 0");
    if (!(cfg->ema_alpha > 0.0 && cfg->ema_alpha <= 1.0)) raise(VLA_E_INVALID, "ema_alpha in (0, 1]");
    if (cfg->prefill_tokens < 1 || cfg->decode_tokens < 0)
      raise(VLA_E_INVALID, "prefill_tokens >= 1, decode_tokens >= 0");
    *out = new vla_admission{Admission(cfg->deadline_ms, cfg->safety_margin_ms, cfg->ema_alpha,
                                       cfg->prefill_tokens, cfg->decode_tokens)};
  });
}
void vla_admission_destroy(vla_admission* a) { delete a; }
vla_status vla_admission_cycle_begin(vla_admission* a) {
  return guarded([&] {
    if (!a) raise(VLA_E_INVALID, "null argument");
    a->a.cycle_begin();
  });
}
vla_status vla_admission_elapsed_ms(const vla_admission* a, double* out_ms) {
  return guarded([&] {
    if (!a || !out_ms) raise(VLA_E_INVALID, "null argument");
    *out_ms = a->a.elapsed_ms();
  });
}
vla_status vla_admission_should_admit(const vla_admission* a, double elapsed_ms,
                                      int32_t* out_admit, double* out_estimate_ms) {
  return guarded([&] {
    if (!a || !out_admit) raise(VLA_E_INVALID, "null argument");
    if (!std::isfinite(elapsed_ms)) raise(VLA_E_INVALID, "elapsed_ms must be finite");
    *out_admit = a->a.should_admit(elapsed_ms, out_estimate_ms) ? 1 : 0;
  });
}
vla_status vla_admission_record(vla_admission* a, double prefill_ms, int32_t prefill_tokens,
                                double decode_ms, int32_t decode_tokens) {
  return guarded([&] {
    if (!a) raise(VLA_E_INVALID, "null argument");
    if (prefill_tokens < 1 || decode_tokens < 1) raise(VLA_E_INVALID, "token counts must be >= 1");
    if (!(prefill_ms >= 0.0) || !(decode_ms >= 0.0) || !std::isfinite(prefill_ms) ||
        !std::isfinite(decode_ms))
      raise(VLA_E_INVALID, "times must be finite and >= 0");
    a->a.record(prefill_ms, prefill_tokens, decode_ms, decode_tokens);
  });
}
vla_status vla_admission_cycle_end(vla_admission* a, int32_t admitted, double* out_cycle_ms) {
  return guarded([&] {
    if (!a) raise(VLA_E_INVALID, "null argument");
    const double ms = a->a.cycle_end(admitted != 0);
    if (out_cycle_ms) *out_cycle_ms = ms;
  });
}
vla_status vla_admission_sleep_until_deadline(const vla_admission* a) {
  return guarded([&] {
    if (!a) raise(VLA_E_INVALID, "null argument");
    a->a.sleep_until_deadline();
  });
}
vla_status vla_admission_stats_out(const vla_admission* a, vla_admission_stats* out) {
  return guarded([&] {
    if (!a || !out) raise(VLA_E_INVALID, "null argument");
    const Admission& x = a->a;
    out->cycles = x.cycles_;
    out->admitted = x.admitted_;
    out->refused = x.refused_;
    out->deadline_misses = x.misses_;
    out->worst_cycle_ms = x.worst_ms_;
    out->last_overrun_ms = x.last_overrun_ms_;
    out->ema_prefill_ms_per_token = x.ema_prefill_;
    out->ema_decode_ms_per_token = x.ema_decode_;
    out->has_sample = x.has_sample_ ? 1 : 0;
  });
}

}  // extern "C"

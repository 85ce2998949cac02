// GQA attention over the block-paged KV cache (prefill and decode).
//
// softmax(q k^T / sqrt(d)) v over every visible key ("CSR ...", III-A), with
// the keys of the current chunk causal and every other resident key visible
// ("Rebuilding Kshipra Around Memory", section 4) -- or, for the action chunk
// of a pi0-style expert ("Running VLAs at Real-time Speed", section 2), every
// key of the chunk visible to every row of it -- computed as an online
// softmax (m, l, o) over KV blocks read in place from the pool (same section).
//
// bf16 path (matrix cores). Query rows are (token, q head of the group) pairs,
// so the g heads sharing a KV head consume each K/V block together and a block
// is read once per KV-head group rather than once per query head. One 16-row
// tile is one wavefront's set of query columns. Per 32-key step (two blocks):
//   S^T = K Q^T        v_mfma_f32_16x16x32_bf16, A = 16 keys x 32 dims (K rows),
//                      B = Q^T held in registers for the whole loop; the
//                      accumulator gives each lane 4 keys of one query.
//   online softmax     per query column: in-lane max/sum + 2 cross-lane steps,
//                      in base 2 (scores pre-multiplied by log2 e / sqrt(d)).
//   O^T += V^T P^T     A = V^T (the pool stores V transposed inside a block, so
//                      4 consecutive keys of one dimension are contiguous),
//                      B = P^T, which is exactly the lane's own probabilities.
// Two workgroup shapes (4 wavefronts each):
//   key split (decode, <= 16 query rows): the 4 wavefronts share one row tile
//     and take interleaved block pairs straight from memory; their partial
//     (m, l, o) are merged through LDS.
//   row tiles (prefill): each wavefront owns 16 rows; the workgroup stages each
//     block pair in LDS once (double buffered) for all 64 rows.
// The resident blocks are split over workgroups (split-K). Each workgroup
// writes its partial (m, l, o); a second kernel merges the splits in split
// order (deterministic). Merging inside the first kernel would need an
// agent-scope release/acquire per workgroup, which on this chip writes back
// and invalidates the whole L2 of the workgroup's XCD.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace vla {

constexpr int kAttnWaves = 4;
constexpr int kMaxSplitsKey = 128;  // key-split shape: 16 rows per workgroup
constexpr int kMaxSplitsRow = 32;   // row-tile shape: 64 rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bool key_visible(const AttnArgs& a, int b, int slot, int ntok, int tq) {
  if (slot >= ntok) return false;
  if (b < a.cb0 || !a.causal) return true;
  const int ck = (b - a.cb0) * a.g.bt + slot - a.cslot0;  // index inside the causal region
  return ck <= tq;
}

__device__ __forceinline__ int block_ntok(const AttnArgs& a, int b) {
  return b == a.nlb - 1 ? a.last_ntok : a.blk_ntok[b];
}

// Operands of one 32-key step held by a lane: K rows (A of S^T = K Q^T) for the
// two blocks, and V^T rows (A of O^T += V^T P^T), 8 keys per lane in the order
// {block 0 keys 4jq..4jq+3, block 1 keys 4jq..4jq+3}.
template <int D>
struct PairFrags {
  bf16x8_t k0[D / 32], k1[D / 32];
  bf16x8_t v[D / 16];
};

template <int D>
struct SoftmaxState {
  float m, l;        // running max (base 2) and sum of the query column
  f32x4_t o[D / 16]; // O^T[dim dt*16 + 4jq + e][column]
};

template <int D>
__device__ __forceinline__ void state_init(SoftmaxState<D>& st) {
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) st.o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// one online-softmax step over blocks b (and b+1 when has1) for query column (tq)
template <int D>
__device__ __forceinline__ void attn_step(const AttnArgs& a, SoftmaxState<D>& st,
                                          const bf16x8_t* qf, const PairFrags<D>& f, int b,
                                          bool has1, int tq, int jq, float sl2) {
  f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k0[ds], qf[ds], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k1[ds], qf[ds], s1, 0, 0, 0);
  }
  const int nt0 = block_ntok(a, b);
  const int nt1 = has1 ? block_ntok(a, b + 1) : 0;
  float p0[4], p1[4];
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int ks = 4 * jq + e;
    p0[e] = key_visible(a, b, ks, nt0, tq) ? s0[e] * sl2 : -INFINITY;
    p1[e] = (has1 && key_visible(a, b + 1, ks, nt1, tq)) ? s1[e] * sl2 : -INFINITY;
    mx = fmaxf(mx, fmaxf(p0[e], p1[e]));
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float m_new = fmaxf(st.m, mx);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = st.m == -INFINITY ? 0.f : exp2f(st.m - m_use);
  // probabilities rounded to bf16 once; the sum uses the rounded values
  u32x4_t pw;
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const bf16_t a0 = f32_to_bf16(exp2f(p0[2 * e] - m_use));
    const bf16_t a1 = f32_to_bf16(exp2f(p0[2 * e + 1] - m_use));
    const bf16_t b0 = f32_to_bf16(exp2f(p1[2 * e] - m_use));
    const bf16_t b1 = f32_to_bf16(exp2f(p1[2 * e + 1] - m_use));
    sum += bf16_to_f32(a0) + bf16_to_f32(a1) + bf16_to_f32(b0) + bf16_to_f32(b1);
    pw[e] = (uint32_t)a0 | ((uint32_t)a1 << 16);
    pw[2 + e] = (uint32_t)b0 | ((uint32_t)b1 << 16);
  }
  sum += __shfl_xor(sum, 16, 64);
  sum += __shfl_xor(sum, 32, 64);
  st.l = st.l * alpha + sum;
  st.m = m_new;
  const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    st.o[dt] *= alpha;
    st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.v[dt], pf, st.o[dt], 0, 0, 0);
  }
}

// operands of blocks (b, b+1) straight from the pool (key-split shape)
template <int D>
__device__ __forceinline__ void load_pair_global(const AttnArgs& a, PairFrags<D>& f, int b,
                                                 bool has1, int kvh, int cq, int jq) {
  const bf16_t* kp = (const bf16_t*)a.kpool;
  const bf16_t* vp = (const bf16_t*)a.vpool;
  const int pb0 = a.blk_table[b];
  const int pb1 = has1 ? a.blk_table[b + 1] : pb0;
  const bf16_t* k0 = kp + a.g.kidx(a.layer, pb0, kvh, cq, 0) + 8 * jq;
  const bf16_t* k1 = kp + a.g.kidx(a.layer, pb1, kvh, cq, 0) + 8 * jq;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    f.k0[ds] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(k0 + ds * 32));
    f.k1[ds] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(k1 + ds * 32));
  }
  const bf16_t* v0 = vp + a.g.vidx(a.layer, pb0, kvh, 4 * jq, 0);
  const bf16_t* v1 = vp + a.g.vidx(a.layer, pb1, kvh, 4 * jq, 0);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const size_t off = (size_t)(dt * 16 + cq) * a.g.bt;
    const u32x2_t lo = *(const u32x2_t*)(v0 + off);
    const u32x2_t hi = has1 ? *(const u32x2_t*)(v1 + off) : u32x2_t{0, 0};
    f.v[dt] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
  }
}

// LDS image of one block pair (row-tile shape). K rows: [32 keys][D + 8];
// V^T rows: [D][40], where dim i holds at 8jq + 4blk + e the key 4jq + e of block blk.
template <int D>
struct PairLds {
  static constexpr int KP = D + 8;
  static constexpr int VP = 40;
  static constexpr int KELEMS = 32 * KP;
  static constexpr int VELEMS = D * VP;
  static constexpr int ELEMS = KELEMS + VELEMS;
  static constexpr int KCH = 32 * D / 8;   // 16-byte chunks of K per pair
  static constexpr int VCH = 2 * D * 2;    // 16-byte chunks of V per pair
  static constexpr int CH = (KCH + VCH) / (kAttnWaves * 64);
};

template <int D>
__device__ __forceinline__ void stage_load(const AttnArgs& a, u32x4_t* r, int b, bool has1,
                                           int kvh) {
  using P = PairLds<D>;
  const bf16_t* kp = (const bf16_t*)a.kpool;
  const bf16_t* vp = (const bf16_t*)a.vpool;
  const int pb0 = a.blk_table[b];
  const int pb1 = has1 ? a.blk_table[b + 1] : pb0;
#pragma unroll
  for (int i = 0; i < P::CH; ++i) {
    const int c = threadIdx.x + i * kAttnWaves * 64;
    if (c < P::KCH) {
      const int blk = c / (16 * D / 8);
      const int row = (c / (D / 8)) % 16;
      const int col8 = c % (D / 8);
      r[i] = *(const u32x4_t*)(kp + a.g.kidx(a.layer, blk ? pb1 : pb0, kvh, row, col8 * 8));
    } else {
      const int cv = c - P::KCH;
      const int blk = cv / (2 * D);
      const int dim = (cv % (2 * D)) / 2;
      const int h = cv % 2;
      r[i] = (blk && !has1) ? u32x4_t{0, 0, 0, 0}
                            : *(const u32x4_t*)(vp + a.g.vidx(a.layer, blk ? pb1 : pb0, kvh,
                                                               8 * h, dim));
    }
  }
}

template <int D>
__device__ __forceinline__ void stage_store(bf16_t* lds, const u32x4_t* r) {
  using P = PairLds<D>;
  bf16_t* Ks = lds;
  bf16_t* Vs = lds + P::KELEMS;
#pragma unroll
  for (int i = 0; i < P::CH; ++i) {
    const int c = threadIdx.x + i * kAttnWaves * 64;
    if (c < P::KCH) {
      const int blk = c / (16 * D / 8);
      const int row = (c / (D / 8)) % 16;
      const int col8 = c % (D / 8);
      *(u32x4_t*)(Ks + (blk * 16 + row) * P::KP + col8 * 8) = r[i];
    } else {
      const int cv = c - P::KCH;
      const int blk = cv / (2 * D);
      const int dim = (cv % (2 * D)) / 2;
      const int h = cv % 2;
      bf16_t* row = Vs + dim * P::VP + blk * 4;
      *(u32x2_t*)(row + (2 * h) * 8) = u32x2_t{r[i][0], r[i][1]};
      *(u32x2_t*)(row + (2 * h + 1) * 8) = u32x2_t{r[i][2], r[i][3]};
    }
  }
}

template <int D>
__device__ __forceinline__ void load_pair_lds(const bf16_t* lds, PairFrags<D>& f, int cq, int jq) {
  using P = PairLds<D>;
  const bf16_t* Ks = lds;
  const bf16_t* Vs = lds + P::KELEMS;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    f.k0[ds] = *(const bf16x8_t*)(Ks + cq * P::KP + ds * 32 + 8 * jq);
    f.k1[ds] = *(const bf16x8_t*)(Ks + (16 + cq) * P::KP + ds * 32 + 8 * jq);
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    f.v[dt] = *(const bf16x8_t*)(Vs + (dt * 16 + cq) * P::VP + 8 * jq);
}

template <int D, bool KEYSPLIT>
struct AttnShape {
  static constexpr int ROWS = KEYSPLIT ? 16 : 16 * kAttnWaves;
  // LDS: key split -> per-wave partials (4 x 16 x D fp32 + m, l); row tiles -> 2 pair images
  static constexpr int LDS_BYTES =
      KEYSPLIT ? kAttnWaves * 16 * (D + 2) * 4 : 2 * PairLds<D>::ELEMS * 2;
};

// partial layout: part_o[unit][ROWS][D], part_ml[unit][2][ROWS] with
// unit = (kvh * rgroups + rg) * splits + split
template <int D, bool KEYSPLIT>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a, int rgroups) {
  using S = AttnShape<D, KEYSPLIT>;
  constexpr int ROWS = S::ROWS;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDS_BYTES];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.x, rg = blockIdx.y, kvh = blockIdx.z;
  const int splits = a.splits;
  const int grp = a.hq / a.g.hkv;
  const int R = a.n * grp;
  const int jq = lane >> 4, cq = lane & 15;
  const float sl2 = a.scale * kLog2e;

  const int wrow0 = rg * ROWS + (KEYSPLIT ? 0 : wave * 16);
  const int r = wrow0 + cq;
  const bool qvalid = r < R;
  const int tq = qvalid ? r / grp : 0;
  const int hq = kvh * grp + (qvalid ? r % grp : 0);
  bf16x8_t qf[D / 32];
  {
    const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)tq * a.hq + hq) * D;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const u32x4_t v = qvalid ? *(const u32x4_t*)(qrow + ds * 32 + 8 * jq) : u32x4_t{0, 0, 0, 0};
      qf[ds] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // blocks of this split; blocks past the workgroup's last causal key are skipped
  const int bps = (a.nlb + splits - 1) / splits;
  const int b_begin = split * bps;
  int b_end = min(a.nlb, b_begin + bps);
  if (a.causal) {
    const int rlast = min(R, rg * ROWS + ROWS) - 1;
    const int tmax = rlast / grp;
    b_end = min(b_end, a.cb0 + (tmax + a.cslot0) / a.g.bt + 1);
  }

  SoftmaxState<D> st;
  state_init(st);
  if constexpr (KEYSPLIT) {
    PairFrags<D> cur, nxt;
    int b = b_begin + 2 * wave;
    if (b < b_end) load_pair_global(a, cur, b, b + 1 < b_end, kvh, cq, jq);
    for (; b < b_end; b += 2 * kAttnWaves) {
      const int bn = b + 2 * kAttnWaves;
      if (bn < b_end) load_pair_global(a, nxt, bn, bn + 1 < b_end, kvh, cq, jq);
      attn_step(a, st, qf, cur, b, b + 1 < b_end, tq, jq, sl2);
      cur = nxt;
    }
    // merge the 4 wavefronts' states through LDS
    float* Lo = (float*)smem;                       // [wave][16][D]
    float* Lml = Lo + kAttnWaves * 16 * D;           // [wave][2][16]
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) Lo[(wave * 16 + cq) * D + dt * 16 + 4 * jq + e] = st.o[dt][e];
    if (jq == 0) {
      Lml[wave * 32 + cq] = st.m;
      Lml[wave * 32 + 16 + cq] = st.l;
    }
    __syncthreads();
    const int unit = (kvh * rgroups + rg) * splits + split;
    for (int e = threadIdx.x; e < 16 * D; e += kAttnWaves * 64) {
      const int c = e / D, dim = e % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, Lml[w * 32 + c]);
      float L = 0.f, acc = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
          const float mw_ = Lml[w * 32 + c];
          const float wt = mw_ == -INFINITY ? 0.f : exp2f(mw_ - M);
          L += wt * Lml[w * 32 + 16 + c];
          acc += wt * Lo[(w * 16 + c) * D + dim];
        }
      }
      const int rr = rg * 16 + c;
      if (splits == 1) {
        if (rr < R)
          ((bf16_t*)a.out)[((size_t)(rr / grp) * a.hq + kvh * grp + rr % grp) * D + dim] =
              f32_to_bf16(L > 0.f ? acc / L : 0.f);
      } else {
        a.part_o[((size_t)unit * 16 + c) * D + dim] = acc;
        if (dim == 0) {
          a.part_ml[(size_t)unit * 32 + c] = M;
          a.part_ml[(size_t)unit * 32 + 16 + c] = L;
        }
      }
    }
  } else {
    using P = PairLds<D>;
    bf16_t* buf = (bf16_t*)smem;
    u32x4_t rs[P::CH];
    const int npairs = b_end > b_begin ? (b_end - b_begin + 1) / 2 : 0;
    if (npairs > 0) {
      stage_load<D>(a, rs, b_begin, b_begin + 1 < b_end, kvh);
      stage_store<D>(buf, rs);
    }
    __syncthreads();
    for (int p = 0; p < npairs; ++p) {
      const int b = b_begin + 2 * p;
      const bool more = p + 1 < npairs;
      if (more) stage_load<D>(a, rs, b + 2, b + 3 < b_end, kvh);
      PairFrags<D> f;
      load_pair_lds<D>(buf + (p & 1) * P::ELEMS, f, cq, jq);
      attn_step(a, st, qf, f, b, b + 1 < b_end, tq, jq, sl2);
      if (more) stage_store<D>(buf + ((p + 1) & 1) * P::ELEMS, rs);
      __syncthreads();
    }
    const int unit = (kvh * rgroups + rg) * splits + split;
    if (splits == 1) {
      if (qvalid) {
        const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
        bf16_t* orow = (bf16_t*)a.out + ((size_t)tq * a.hq + hq) * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          u32x2_t w;
          w[0] = (uint32_t)f32_to_bf16(st.o[dt][0] * inv) |
                 ((uint32_t)f32_to_bf16(st.o[dt][1] * inv) << 16);
          w[1] = (uint32_t)f32_to_bf16(st.o[dt][2] * inv) |
                 ((uint32_t)f32_to_bf16(st.o[dt][3] * inv) << 16);
          *(u32x2_t*)(orow + dt * 16 + 4 * jq) = w;
        }
      }
    } else {
      const int c = wave * 16 + cq;  // row inside the workgroup
      float* po = a.part_o + ((size_t)unit * ROWS + c) * D;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *(f32x4_t*)(po + dt * 16 + 4 * jq) = st.o[dt];
      if (jq == 0) {
        a.part_ml[(size_t)unit * 2 * ROWS + c] = st.m;
        a.part_ml[(size_t)unit * 2 * ROWS + ROWS + c] = st.l;
      }
    }
  }
}

// Combines the splits of one (KV head, row group): with per-split running max
// m_s (base 2), sum l_s and unnormalised o_s, o = sum_s 2^(m_s - M) o_s /
// sum_s 2^(m_s - M) l_s, M = max_s m_s, taken in split order. One thread per
// output element; the splits are read 8 at a time (24 loads in flight).
template <int D, bool KEYSPLIT>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int rgroups) {
  using S = AttnShape<D, KEYSPLIT>;
  constexpr int ROWS = S::ROWS;
  constexpr int CHUNK = 8;
  const int tile = blockIdx.x;  // kvh * rgroups + rg
  const int rg = tile % rgroups, kvh = tile / rgroups;
  const int e = blockIdx.y * 256 + threadIdx.x;
  if (e >= ROWS * D) return;
  const int c = e / D, dim = e % D;
  const int grp = a.hq / a.g.hkv;
  const int rr = rg * ROWS + c;
  if (rr >= a.n * grp) return;
  const int splits = a.splits;
  const size_t unit0 = (size_t)tile * splits;
  float M = -INFINITY, L = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < splits; s0 += CHUNK) {
    float m[CHUNK], l[CHUNK], o[CHUNK];
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) {
      const size_t u = unit0 + s0 + i;
      const bool ok = s0 + i < splits;
      m[i] = ok ? a.part_ml[u * 2 * ROWS + c] : -INFINITY;
      l[i] = ok ? a.part_ml[u * 2 * ROWS + ROWS + c] : 0.f;
      o[i] = ok ? a.part_o[(u * ROWS + c) * D + dim] : 0.f;
    }
    float mc = M;
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) mc = fmaxf(mc, m[i]);
    if (mc == -INFINITY) continue;
    const float sc = M == -INFINITY ? 0.f : exp2f(M - mc);
    L *= sc;
    acc *= sc;
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) {
      const float w = m[i] == -INFINITY ? 0.f : exp2f(m[i] - mc);
      L += w * l[i];
      acc += w * o[i];
    }
    M = mc;
  }
  ((bf16_t*)a.out)[((size_t)(rr / grp) * a.hq + kvh * grp + rr % grp) * D + dim] =
      f32_to_bf16(L > 0.f ? acc / L : 0.f);
}

// ---------------------------------------------------------------------------
// fp32 path: one wavefront per (token, q head); scores for every logical key
// in LDS, then softmax and the weighted sum of V. For small fp32 caches only.
// ---------------------------------------------------------------------------
constexpr int kF32MaxKeys = 2048;

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  const int last_ntok = a.last_ntok;
  __shared__ float sc[4][kF32MaxKeys];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int unit = blockIdx.x * 4 + wave;
  if (unit >= a.n * a.hq) return;
  const int t = unit / a.hq, h = unit % a.hq;
  const int grp = a.hq / a.g.hkv;
  const int kvh = h / grp;
  const int d = a.g.d, bt = a.g.bt;
  const float* q = (const float*)a.q + ((size_t)t * a.hq + h) * d;
  const float* kp = (const float*)a.kpool;
  const float* vp = (const float*)a.vpool;
  const int nkeys = a.nlb * bt;
  float mx = -INFINITY;
  for (int i = lane; i < nkeys; i += 64) {
    const int b = i / bt, s = i % bt;
    const int nt = (b == a.nlb - 1) ? last_ntok : a.blk_ntok[b];
    float v = -INFINITY;
    if (key_visible(a, b, s, nt, t)) {
      const float* kr = kp + a.g.kidx(a.layer, a.blk_table[b], kvh, s, 0);
      float dot = 0.f;
      for (int j = 0; j < d; ++j) dot += q[j] * kr[j];
      v = dot * a.scale;
    }
    sc[wave][i] = v;
    mx = fmaxf(mx, v);
  }
  mx = wave_max(mx);
  float sum = 0.f;
  for (int i = lane; i < nkeys; i += 64) {
    const float p = sc[wave][i] == -INFINITY ? 0.f : __expf(sc[wave][i] - mx);
    sc[wave][i] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  __builtin_amdgcn_wave_barrier();
  float* orow = (float*)a.out + ((size_t)t * a.hq + h) * d;
  for (int j = lane; j < d; j += 64) {
    float acc = 0.f;
    for (int i = 0; i < nkeys; ++i) {
      const float p = sc[wave][i];
      if (p != 0.f) acc += p * vp[a.g.vidx(a.layer, a.blk_table[i / bt], kvh, i % bt, j)];
    }
    orow[j] = acc / sum;
  }
}

template <int D, bool KEYSPLIT>
static void attn_bf16_launch(const AttnArgs& a, int rgroups, hipStream_t s) {
  const dim3 grid(a.splits, rgroups, a.g.hkv);
  launch_k(attn_bf16_kernel<D, KEYSPLIT>, grid, dim3(kAttnWaves * 64), 0, s, a, rgroups);
  if (a.splits > 1) {
    constexpr int ROWS = AttnShape<D, KEYSPLIT>::ROWS;
    const dim3 mgrid(a.g.hkv * rgroups, (ROWS * D + 255) / 256);
    launch_k(attn_merge_kernel<D, KEYSPLIT>, mgrid, dim3(256), 0, s, a, rgroups);
  }
}

template <int D>
static void attn_bf16_dispatch(const AttnArgs& a, bool keysplit, int rgroups, hipStream_t s) {
  if (keysplit) attn_bf16_launch<D, true>(a, rgroups, s);
  else attn_bf16_launch<D, false>(a, rgroups, s);
}

hipError_t launch_attention(const AttnArgs& args, int dt, hipStream_t s) {
  if (args.nlb <= 0 || args.n <= 0) return hipErrorInvalidValue;
  if (dt == DT_F32) {
    if (args.nlb * args.g.bt > kF32MaxKeys) return hipErrorInvalidValue;
    launch_k(attn_f32_kernel, dim3((args.n * args.hq + 3) / 4), dim3(256), 0, s, args);
    return hipGetLastError();
  }
  AttnArgs a = args;
  // workgroup shape and split count: at least 8 blocks (4 pairs) per workgroup,
  // about 4 (decode) or 2 (prefill) workgroups per CU at most, within the
  // partial-buffer capacity
  const int R = a.n * (a.hq / a.g.hkv);
  const bool keysplit = R <= 16;
  const int rows = keysplit ? 16 : 16 * kAttnWaves;
  const int rgroups = (R + rows - 1) / rows;
  const int base = a.g.hkv * rgroups;
  int splits = (a.nlb + 7) / 8;
  splits = std::min(splits, std::max(1, (keysplit ? 1024 : 512) / base));
  splits = std::min(splits, keysplit ? kMaxSplitsKey : kMaxSplitsRow);
  splits = std::min(splits, std::max(1, a.part_rows / (base * rows)));
  splits = std::max(splits, 1);
  const int bps = (a.nlb + splits - 1) / splits;
  a.splits = (a.nlb + bps - 1) / bps;
  if (a.splits > 1 &&
      (a.part_o == nullptr || a.part_ml == nullptr || base * rows * a.splits > a.part_rows))
    return hipErrorInvalidValue;
  switch (a.g.d) {
    case 64: attn_bf16_dispatch<64>(a, keysplit, rgroups, s); break;
    case 128: attn_bf16_dispatch<128>(a, keysplit, rgroups, s); break;
    case 256: attn_bf16_dispatch<256>(a, keysplit, rgroups, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vla

// Decode attention (at most 16 query rows per workgroup) as a device function of
// the (split, row group, KV head) of a virtual workgroup, with the online-softmax
// helpers it shares with the prefill rows kernel; used by the attention kernels
// and by the persistent decode step.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace vla {

constexpr int kAttnWaves = 4;       // decode kernel
constexpr int kMaxSplitsKey = 128;  // decode: 16 rows per workgroup
constexpr int kMaxSplitsRow = 32;   // rows kernel
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bool key_visible(const AttnArgs& a, int b, int slot, int ntok, int tq) {
  if (slot >= ntok) return false;
  if (b < a.cb0 || !a.causal) return true;
  const int ck = (b - a.cb0) * a.g.bt + slot - a.cslot0;  // index inside the causal region
  return ck <= tq;
}

// Table reads with a wave-uniform index through the constant address space, so
// they become scalar loads: the tables are not written while a kernel runs, and
// vector loads would count in vmcnt and break the DMA ring's wait depths.
typedef const __attribute__((address_space(4))) int* const_int_p;
__device__ __forceinline__ int uniform_ld(const int* p, int i) {
  return ((const_int_p)(const void*)p)[i];
}
__device__ __forceinline__ int block_ntok_s(const AttnArgs& a, int b) {
  return b == a.nlb - 1 ? a.last_ntok : uniform_ld(a.blk_ntok, b);
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

// max / sum over the 4 lanes of one query column (lanes c, c+16, c+32, c+48), by
// the gfx950 row-swap permutes (no LDS traffic); every lane gets the same value
__device__ __forceinline__ float col_max4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Online-softmax update of one query column (tq) for the scores of blocks b and
// b+1 (s0, s1: keys 4jq..4jq+3 of each; has1: block b+1 exists). `masked`:
// some key of the pair may be invisible (ragged block, causal region);
// otherwise every key is visible. The running max m is in base-2 units
// (score * sl2, sl2 = log2(e) / sqrt(d) > 0, so the max of the raw scores gives
// it); p = 2^(s * sl2 - m) by one fma and the hardware exp2. Returns the bf16
// probabilities as the MFMA B operand (the running sum uses the rounded values)
// and the rescale factor of the running output.
__device__ __forceinline__ bf16x8_t softmax_pair(const AttnArgs& a, float& m, float& l,
                                                 f32x4_t s0, f32x4_t s1, int b, bool has1,
                                                 bool masked, int tq, int jq, float sl2,
                                                 float& alpha) {
  if (masked) {
    // visible: slot < ntok, and outside the causal region or at most the row's token
    // (branch-free selects; b, ntok and the region bounds are wave-uniform)
    const int nt0 = block_ntok_s(a, b);
    const int nt1 = has1 ? block_ntok_s(a, b + 1) : 0;
    const bool open0 = b < a.cb0 || !a.causal, open1 = b + 1 < a.cb0 || !a.causal;
    const int ck0 = (b - a.cb0) * a.g.bt - a.cslot0, ck1 = ck0 + a.g.bt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ks = 4 * jq + e;
      const bool v0 = (ks < nt0) & (open0 | (ck0 + ks <= tq));
      const bool v1 = (ks < nt1) & (open1 | (ck1 + ks <= tq));
      s0[e] = v0 ? s0[e] : -INFINITY;
      s1[e] = v1 ? s1[e] : -INFINITY;
    }
  }
  float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                   fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
  mx = col_max4(mx) * sl2;
  const float m_new = fmaxf(m, mx);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_use);
  u32x4_t pw;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    pw[e] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s0[2 * e], sl2, -m_use)),
                        __builtin_amdgcn_exp2f(fmaf(s0[2 * e + 1], sl2, -m_use)));
    pw[2 + e] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s1[2 * e], sl2, -m_use)),
                            __builtin_amdgcn_exp2f(fmaf(s1[2 * e + 1], sl2, -m_use)));
  }
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    sum += __uint_as_float(pw[e] << 16) + __uint_as_float(pw[e] & 0xffff0000u);
  l = l * alpha + col_sum4(sum);
  m = m_new;
  return __builtin_bit_cast(bf16x8_t, pw);
}

// one online-softmax step of the decode kernel over blocks b (and b+1 when has1)
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
  float alpha;
  const bf16x8_t pf = softmax_pair(a, st.m, st.l, s0, s1, b, has1, /*masked=*/true, tq, jq, sl2,
                                   alpha);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    st.o[dt] *= alpha;
    st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.v[dt], pf, st.o[dt], 0, 0, 0);
  }
}

// operands of blocks (b, b+1) straight from the pool (key-split shape)
template <int D>
__device__ __forceinline__ void load_pair_global(const AttnArgs& a, PairFrags<D>& f, int b,
                                                 bool has1, int kvh, int cq, int jq, int layer) {
  const bf16_t* kp = (const bf16_t*)a.kpool;
  const bf16_t* vp = (const bf16_t*)a.vpool;
  // b is wave-uniform: scalar table loads, which count in lgkmcnt, so waiting for
  // them does not wait for the previous pair's K/V loads still in flight
  const int bu = __builtin_amdgcn_readfirstlane(b);
  const int pb0 = uniform_ld(a.blk_table, bu);
  const int pb1 = has1 ? uniform_ld(a.blk_table, bu + 1) : pb0;
  // dims 32 ds + 8 jq.. of key cq: the 32-dim chunk ds of a block holds its 16 keys
  // in turn, so each load reads one contiguous 1 KB run
  const bf16_t* k0 = kp + a.g.kidx(layer, pb0, kvh, cq, 8 * jq);
  const bf16_t* k1 = kp + a.g.kidx(layer, pb1, kvh, cq, 8 * jq);
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    f.k0[ds] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(k0 + ds * 32 * 16));
    f.k1[ds] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(k1 + ds * 32 * 16));
  }
  const bf16_t* v0 = vp + a.g.vidx(layer, pb0, kvh, 4 * jq, 0);
  const bf16_t* v1 = vp + a.g.vidx(layer, pb1, kvh, 4 * jq, 0);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const size_t off = (size_t)(dt * 16 + cq) * a.g.bt;
    // without a second block pb1 = pb0: the load stays unconditional (a guarded
    // load would make every wait on earlier loads a full drain) and its keys get
    // P = 0 in the softmax, so these values add nothing
    const u32x2_t lo = *(const u32x2_t*)(v0 + off);
    const u32x2_t hi = *(const u32x2_t*)(v1 + off);
    f.v[dt] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
  }
}

// ---------------------------------------------------------------------------
// decode kernel (<= 16 query rows)
// ---------------------------------------------------------------------------
// partial layout (both kernels): part_o[unit][ROWS][D], part_ml[unit][2][ROWS] with
// unit = (kvh * rgroups + rg) * splits + split
// layer: the layer of this call (that of `a` is not read)
template <int D>
__device__ __forceinline__ void attn_decode_body(const AttnArgs& a, int rgroups, int split, int rg,
                                                 int kvh, int layer) {
  constexpr int ROWS = 16;
  // LDS: the 4 wavefronts' partial (o, m, l) for the merge
  __shared__ __attribute__((aligned(16))) float smem[kAttnWaves * 16 * (D + 2)];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int splits = a.splits;
  const int grp = a.hq / a.g.hkv;
  const int R = a.n * grp;
  const int jq = lane >> 4, cq = lane & 15;
  const float sl2 = a.scale * kLog2e;

  const int r = rg * ROWS + cq;
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
    b_end = min(b_end, a.cb0 + (rlast / grp + a.cslot0) / a.g.bt + 1);
  }

  SoftmaxState<D> st;
  state_init(st);
  PairFrags<D> cur, nxt;
  // wave-uniform block index, known as such to the compiler: the block table and
  // token counts are then read with scalar loads, which leave vmcnt to the K/V loads
  int b = __builtin_amdgcn_readfirstlane(b_begin + 2 * wave);
  if (b < b_end) load_pair_global(a, cur, b, b + 1 < b_end, kvh, cq, jq, layer);
  for (; b < b_end; b += 2 * kAttnWaves) {
    // the next pair's loads are unconditional (past the end they re-load the current
    // pair, cache-hot and unused), so the step below waits only for its own pair
    const int bn = b + 2 * kAttnWaves;
    const int bl = bn < b_end ? bn : b;
    load_pair_global(a, nxt, bl, bl + 1 < b_end, kvh, cq, jq, layer);
    attn_step(a, st, qf, cur, b, b + 1 < b_end, tq, jq, sl2);
    cur = nxt;
  }
  // merge the 4 wavefronts' states through LDS: the row weights 2^(m_w - M) and
  // the row sums first (one thread per row), then the rows' elements; rows past
  // the pass's query rows are padding and are neither merged nor stored
  float* Lo = smem;                          // [wave][16][D]
  float* Lml = Lo + kAttnWaves * 16 * D;     // [wave][2][16]
  __shared__ float wts[kAttnWaves][16], rowM[16], rowL[16];
  const int nrow = min(ROWS, R - rg * ROWS);  // real rows of this tile
  if (cq < nrow) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) Lo[(wave * 16 + cq) * D + dt * 16 + 4 * jq + e] = st.o[dt][e];
    if (jq == 0) {
      Lml[wave * 32 + cq] = st.m;
      Lml[wave * 32 + 16 + cq] = st.l;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < nrow) {
    const int c = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, Lml[w * 32 + c]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float mw_ = Lml[w * 32 + c];
      const float wt = (M == -INFINITY || mw_ == -INFINITY) ? 0.f : exp2f(mw_ - M);
      wts[w][c] = wt;
      L += wt * Lml[w * 32 + 16 + c];
    }
    rowM[c] = M;
    rowL[c] = L;
  }
  __syncthreads();
  const int unit = (kvh * rgroups + rg) * splits + split;
  for (int e = threadIdx.x; e < nrow * D; e += kAttnWaves * 64) {
    const int c = e / D, dim = e % D;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) acc += wts[w][c] * Lo[(w * 16 + c) * D + dim];
    const float L = rowL[c];
    const int rr = rg * 16 + c;
    if (splits == 1) {
      const size_t oi = ((size_t)(rr / grp) * a.hq + kvh * grp + rr % grp) * D + dim;
      const float y = L > 0.f ? acc / L : 0.f;
      const bf16_t h = f32_to_bf16(y);
      ((bf16_t*)a.out)[oi] = h;
      if (a.out_lo) ((bf16_t*)a.out_lo)[oi] = f32_to_bf16(y - bf16_to_f32(h));
    } else {
      a.part_o[((size_t)unit * 16 + c) * D + dim] = acc;
      if (dim == 0) {
        a.part_ml[(size_t)unit * 32 + c] = rowM[c];
        a.part_ml[(size_t)unit * 32 + 16 + c] = L;
      }
    }
  }
}

}  // namespace vla

// One-shot decode GEMV (one token row, bf16 weights) as a device function of a
// virtual workgroup index, shared by its own kernel and by the persistent decode
// step. See gemv1_body for what it computes.
#pragma once

#include "common.hpp"
#include "epilogue.hpp"
#include "kernels.hpp"

namespace vla {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kGemvMaxGrid = 2048;  // also the capacity of the argmax partials
constexpr int kGemv1MaxK = 2048;    // one-shot kernel: longest whole row (4 chunks per lane)

// Row group g of a wave: RW physical rows. For the gated projection the group
// is RW/2 gate rows f0 .. f0+RW/2-1 and their RW/2 up rows (LAYOUT_GATEUP puts
// 16 gate rows, then the 16 matching up rows, in each block of 32).
template <int EPI, int RW>
__device__ __forceinline__ int64_t gemv_row(int g, int r) {
  if constexpr (EPI == EPI_SWIGLU) {
    const int f = g * (RW / 2) + (r % (RW / 2));
    return (int64_t)(f / 16) * 32 + (f % 16) + (r >= RW / 2 ? 16 : 0);
  } else {
    return (int64_t)g * RW + r;
  }
}

// One-shot decode GEMV, bf16 weights. Every wavefront requests all it needs at
// once, so the kernel costs one memory round trip: first the input side (the
// row, the RMSNorm gains, or the attention partials), then the chunks of its
// rows, then the epilogue's RoPE operands. Vector loads complete in issue order,
// so staging the input waits only for the input side while the weights are in
// flight. KS = 1: a wavefront owns a group of RW rows and whole rows of CPL
// chunks per lane. The gated projection stages its normalised input once per
// workgroup in LDS; the q/k/v projection normalises per wavefront (it holds the
// whole row across its lanes). KS = 4 (residual projections with long rows):
// the workgroup owns RW rows and its 4 wavefronts split K; their sums meet in
// LDS and are added in wavefront order.
//
// Residual projection of the decode attention output (part_o set): the input
// row is merged here from the attention's split partials, o = sum_s 2^(m_s - M)
// o_s / sum_s 2^(m_s - M) l_s per query head (M = max_s m_s, splits in order),
// rounded to bf16 as the attention kernel rounds its own output, so no separate
// merge kernel runs.
// vb: the virtual workgroup; W and layer: the weights and the layer index of this
// call (those of `a` are not read)
template <int EPI, int RW, int CPL, int KS, bool FOLD>
__device__ __forceinline__ void gemv1_body(const GemvArgs& a, int ngroups, int vb, const void* Wp,
                                           int layer) {
  static_assert(KS == 1 || (KS == kGemvWaves && EPI == EPI_RESID), "K split: residual inputs only");
  static_assert(!FOLD || (EPI == EPI_RESID && KS == 1), "attention fold: whole-row residual input");
  constexpr bool kStage = EPI == EPI_SWIGLU;  // input normalised once per workgroup
  constexpr int XI = kGemv1MaxK / 4 / kGemvThreads;
  __shared__ float part[kGemvWaves][RW];
  __shared__ f32x4_t xsh[kGemv1MaxK / 4];
  __shared__ float ssq[kGemvWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = KS == 1 ? vb * kGemvWaves + wave : vb;
  const bool live = g < ngroups;  // wave-uniform
  const int K = a.K, nch = K / 8;
  const int q = KS == 1 ? nch : (nch + KS - 1) / KS;  // chunks of this wavefront's K range
  const int cbeg = KS == 1 ? 0 : wave * q;
  const int cend = min(nch, cbeg + q);
  constexpr bool fold = FOLD;

  // ---- input-side loads ----
  f32x4_t xr[XI], gr[XI];             // normalised inputs, workgroup-staged (thread's f32x4s)
  f32x4_t xw[CPL][2], gw[CPL][2];     // normalised inputs, per wavefront (lane's chunks)
  u32x4_t xb[CPL];                    // residual inputs (bf16 chunks)
  f32x4_t po[2][kFoldMaxSplits];      // folded attention: partial o of the thread's 8 elements
  float pmv[kFoldMaxSplits], plv[kFoldMaxSplits];  // ... and of their head: (m, l) per split
  if constexpr (EPI != EPI_RESID) {
    const f32x4_t* xf4 = (const f32x4_t*)a.x;
    const f32x4_t* g4 = (const f32x4_t*)a.norm_g;
    if constexpr (kStage) {
#pragma unroll
      for (int k = 0; k < XI; ++k) {
        const int i = tid + k * kGemvThreads;
        xr[k] = i < K / 4 ? xf4[i] : f32x4_t{0.f, 0.f, 0.f, 0.f};
        gr[k] = a.norm_g && i < K / 4 ? g4[i] : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    } else {
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = lane + 64 * u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          xw[u][h] = c < nch ? xf4[2 * c + h] : f32x4_t{0.f, 0.f, 0.f, 0.f};
          gw[u][h] = a.norm_g && c < nch ? g4[2 * c + h] : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  } else if constexpr (fold) {
    // elements 8t .. 8t+7 of the row (one query head, 8t / d, as 8 divides d): the
    // head's row inside its KV group's tile is head % grp, unit = kv head * splits
    // + split. Threads past the row re-load its last 8 elements (not stored);
    // splits past S are skipped (wave-uniform).
    const int S = a.splits, d = a.hd, grp = a.grp;
    const int e0 = min(8 * tid, K - 8);
    const int h = e0 >> (31 - __builtin_clz(d)), kv = h / grp, r = h - kv * grp;
    const uint32_t ustride = 16u * (uint32_t)d;  // floats between consecutive units
    const f32x4_t* pk =
        (const f32x4_t*)(a.part_o + ((uint32_t)(kv * S) * 16u + (uint32_t)r) * (uint32_t)d +
                         (uint32_t)(e0 & (d - 1)));
    const float* pmk = a.part_ml + (uint32_t)(kv * S) * 32u + (uint32_t)r;
#pragma unroll
    for (int sp = 0; sp < kFoldMaxSplits; ++sp) {
      if (sp < S) {
        po[0][sp] = pk[sp * (ustride / 4)];
        po[1][sp] = pk[sp * (ustride / 4) + 1];
        pmv[sp] = pmk[sp * 32];
        plv[sp] = pmk[sp * 32 + 16];
      }
    }
  } else {
    const bf16_t* x = (const bf16_t*)a.x;
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = cbeg + lane + 64 * u;
      xb[u] = c < cend ? *(const u32x4_t*)(x + (size_t)c * 8) : u32x4_t{0, 0, 0, 0};
    }
  }

  // ---- weights ----
  // Unconditional loads: chunks past the wavefront's range re-read its last chunk
  // (their inputs are zero, so they add nothing), and a wavefront past the last
  // group reads row N-1 (its sums are dropped). With no guarded load after them,
  // the input-side loads above can be waited for alone while these are in flight.
  const bf16_t* W = (const bf16_t*)Wp;
  u32x4_t w[CPL][RW];
  const int clast = cend > 0 ? cend - 1 : 0;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int64_t row = live ? gemv_row<EPI, RW>(g, r) : 0;
    const bf16_t* wr = W + (row < a.N ? row : (int64_t)a.N - 1) * K;
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = cbeg + lane + 64 * u;
      w[u][r] = *(const u32x4_t*)(wr + (size_t)(c < cend ? c : clast) * 8);
    }
  }
  // every load above is issued before any of them is used (the scheduler would
  // otherwise start converting the input between the weight loads and wait there)
  __builtin_amdgcn_sched_barrier(0);
  QkvPre pre;
  FwdCtx ctx = a.ctx;
  ctx.layer = layer;
  if constexpr (EPI == EPI_QKV) {
    if (live && lane < RW / 2) pre = epi_qkv_prefetch(ctx, 0, (int)gemv_row<EPI, RW>(g, 2 * lane));
  }

  // ---- the input row, as the lane's 8 values per chunk ----
  float xv[CPL][8];
  if constexpr (EPI != EPI_RESID) {
    if constexpr (kStage) {
      if (a.norm_g) {
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < XI; ++k)
#pragma unroll
          for (int e = 0; e < 4; ++e) ss += xr[k][e] * xr[k][e];
        ss = wave_sum(ss);
        if (lane == 0) ssq[wave] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int v = 0; v < kGemvWaves; ++v) tot += ssq[v];
        const float rn = rsqrtf(tot / (float)K + a.eps);
#pragma unroll
        for (int k = 0; k < XI; ++k) xr[k] = xr[k] * rn * gr[k];
      }
#pragma unroll
      for (int k = 0; k < XI; ++k) {
        const int i = tid + k * kGemvThreads;
        if (i < K / 4) xsh[i] = xr[k];
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = lane + 64 * u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4_t v = c < nch ? xsh[2 * c + h] : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[u][4 * h + e] = v[e];
        }
      }
    } else {
      float rn = 1.f;
      if (a.norm_g) {
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < CPL; ++u)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += xw[u][h][e] * xw[u][h][e];
        rn = rsqrtf(wave_sum(ss) / (float)K + a.eps);
      }
#pragma unroll
      for (int u = 0; u < CPL; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            xv[u][4 * h + e] = a.norm_g ? xw[u][h][e] * rn * gw[u][h][e] : xw[u][h][e];
    }
  } else if constexpr (fold) {
    const int S = a.splits;
    float M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < kFoldMaxSplits; ++sp)
      if (sp < S) M = fmaxf(M, pmv[sp]);
    float L = 0.f;
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < kFoldMaxSplits; ++sp) {
      if (sp < S) {
        const float wt = (M != -INFINITY && pmv[sp] != -INFINITY) ? exp2f(pmv[sp] - M) : 0.f;
        L += wt * plv[sp];
        acc0 += wt * po[0][sp];
        acc1 += wt * po[1][sp];
      }
    }
    if (8 * tid < K) {
      f32x4_t v0, v1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v0[i] = bf16_to_f32(f32_to_bf16(L > 0.f ? acc0[i] / L : 0.f));
        v1[i] = bf16_to_f32(f32_to_bf16(L > 0.f ? acc1[i] / L : 0.f));
      }
      xsh[2 * tid] = v0;
      xsh[2 * tid + 1] = v1;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = lane + 64 * u;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4_t v = c < nch ? xsh[2 * c + hh] : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) xv[u][4 * hh + e] = v[e];
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < CPL; ++u) unpack8(xb[u], xv[u]);
  }

  float acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    acc[r] = 0.f;
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      float wf[8];
      unpack8(w[u][r], wf);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[r] += wf[i] * xv[u][i];
    }
    acc[r] = wave_sum(acc[r]);
  }
  if constexpr (KS > 1) {
    if (lane == 0)
#pragma unroll
      for (int r = 0; r < RW; ++r) part[wave][r] = acc[r];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      float t = part[0][r];
#pragma unroll
      for (int v = 1; v < KS; ++v) t += part[v][r];
      acc[r] = t;
    }
  }
  if (!live) return;

  if constexpr (EPI == EPI_QKV) {
#pragma unroll
    for (int p = 0; p < RW / 2; ++p)
      if (lane == p)
        epi_qkv_store<bf16_t>(ctx, 0, (int)gemv_row<EPI, RW>(g, 2 * p), pre, acc[2 * p],
                              acc[2 * p + 1]);
  } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int64_t row = gemv_row<EPI, RW>(g, r);
      if (lane == r && row < a.N) ((float*)a.out)[row] += acc[r];
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < RW / 2; ++i)
      if (lane == i)
        St<bf16_t>::st((bf16_t*)a.out, g * (RW / 2) + i, glu_act(a.glu, acc[i], acc[RW / 2 + i]));
  }
}

}  // namespace vla

// GQA attention over the block-paged KV cache (prefill and decode).
//
// softmax(q k^T / sqrt(d)) v over every visible key ("CSR ...", III-A), with
// the keys of the current chunk causal and every other resident key visible
// ("Rebuilding Kshipra Around Memory", section 4), computed as an online
// softmax (m, l, o) over KV blocks read in place from the pool (same section).
//
// bf16 path (matrix cores). One wavefront owns (KV head, 16 query rows, key
// split). Query rows are (token, q head of the group) pairs, so the g heads
// sharing a KV head consume each K/V block together and a block is read once
// per KV-head group rather than once per query head. Per 32-key step:
//   S^T = K Q^T        v_mfma_f32_16x16x32_bf16, A = 16 keys x 32 dims (K rows,
//                      contiguous), B = Q^T held in registers for the whole loop;
//                      the accumulator gives each lane 4 keys of one query.
//   online softmax     per query column: in-lane max/sum + 2 cross-lane steps.
//   O^T += V^T P^T     A = V^T (the pool stores V transposed inside a block, so a
//                      lane reads 4 consecutive keys of one dimension), B = P^T,
//                      which is exactly the lane's own probabilities: P never
//                      leaves registers.
// With several key splits each wavefront writes (o, m, l) and a merge kernel
// combines the splits deterministically in split order.
#include "common.hpp"
#include "kernels.hpp"

namespace vla {

__device__ __forceinline__ bool key_visible(const AttnArgs& a, int b, int slot, int ntok, int tq) {
  if (slot >= ntok) return false;
  if (b < a.cb0) return true;
  const int ck = (b - a.cb0) * a.g.bt + slot - a.cslot0;  // index inside the causal region
  return ck <= tq;
}

template <int D>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a, int rtiles) {
  const int last_ntok = a.last_ntok;
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int hkv = a.g.hkv;
  if (unit >= hkv * rtiles * a.splits) return;
  const int split = unit % a.splits;
  const int rest = unit / a.splits;
  const int rt = rest % rtiles;
  const int kvh = rest / rtiles;
  const int grp = a.hq / hkv;
  const int R = a.n * grp;
  const int jq = lane >> 4;   // lane group: 4 keys / dims per lane
  const int cq = lane & 15;   // this lane's query column / key row / dim row

  // query column of this lane
  const int r = rt * 16 + cq;
  const bool qvalid = r < R;
  const int tq = qvalid ? r / grp : 0;
  const int hq = kvh * grp + (qvalid ? r % grp : 0);
  const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)tq * a.hq + hq) * D;
  bf16x8_t qf[D / 32];
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    u32x4_t v = qvalid ? *(const u32x4_t*)(qrow + ds * 32 + 8 * jq) : u32x4_t{0, 0, 0, 0};
    qf[ds] = __builtin_bit_cast(bf16x8_t, v);
  }

  const int bps = (a.nlb + a.splits - 1) / a.splits;
  const int b_begin = split * bps;
  const int b_end = min(a.nlb, b_begin + bps);

  const bf16_t* kp = (const bf16_t*)a.kpool;
  const bf16_t* vp = (const bf16_t*)a.vpool;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int b = b_begin; b < b_end; b += 2) {
    const bool has1 = b + 1 < b_end;
    const int pb0 = a.blk_table[b];
    const int pb1 = has1 ? a.blk_table[b + 1] : pb0;
    const int nt0 = (b == a.nlb - 1) ? last_ntok : a.blk_ntok[b];
    const int nt1 = has1 ? ((b + 1 == a.nlb - 1) ? last_ntok : a.blk_ntok[b + 1]) : 0;

    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const bf16_t* k0 = kp + a.g.kidx(a.layer, pb0, kvh, cq, 0);
    const bf16_t* k1 = kp + a.g.kidx(a.layer, pb1, kvh, cq, 0);
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const bf16x8_t kf0 = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(k0 + ds * 32 + 8 * jq));
      const bf16x8_t kf1 = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(k1 + ds * 32 + 8 * jq));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf0, qf[ds], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf1, qf[ds], s1, 0, 0, 0);
    }
    // lane holds S^T[key 4*jq+e][query cq] for block b (s0) and block b+1 (s1)
    float p0[4], p1[4];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ks = 4 * jq + e;
      p0[e] = key_visible(a, b, ks, nt0, tq) ? s0[e] * a.scale : -INFINITY;
      p1[e] = (has1 && key_visible(a, b + 1, ks, nt1, tq)) ? s1[e] * a.scale : -INFINITY;
      mx = fmaxf(mx, fmaxf(p0[e], p1[e]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_use);
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p0[e] = __expf(p0[e] - m_use);
      p1[e] = __expf(p1[e] - m_use);
      sum += p0[e] + p1[e];
    }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    l_run = l_run * alpha + sum;
    m_run = m_new;

    u32x4_t pw;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      pw[e] = (uint32_t)f32_to_bf16(p0[2 * e]) | ((uint32_t)f32_to_bf16(p0[2 * e + 1]) << 16);
      pw[2 + e] = (uint32_t)f32_to_bf16(p1[2 * e]) | ((uint32_t)f32_to_bf16(p1[2 * e + 1]) << 16);
    }
    const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
    const bf16_t* v0 = vp + a.g.vidx(a.layer, pb0, kvh, 4 * jq, 0);
    const bf16_t* v1 = vp + a.g.vidx(a.layer, pb1, kvh, 4 * jq, 0);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      o[dt] *= alpha;
      const int dim = dt * 16 + cq;
      const u32x2_t lo = *(const u32x2_t*)(v0 + (size_t)dim * a.g.bt);
      const u32x2_t hi = has1 ? *(const u32x2_t*)(v1 + (size_t)dim * a.g.bt) : u32x2_t{0, 0};
      const u32x4_t vv = {lo[0], lo[1], hi[0], hi[1]};
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vv), pf, o[dt],
                                                      0, 0, 0);
    }
  }
  // lane holds O^T[dim dt*16 + 4*jq + e][query cq]
  if (a.splits == 1) {
    if (qvalid) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      bf16_t* orow = (bf16_t*)a.out + ((size_t)tq * a.hq + hq) * D;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        u32x2_t w;
        w[0] = (uint32_t)f32_to_bf16(o[dt][0] * inv) | ((uint32_t)f32_to_bf16(o[dt][1] * inv) << 16);
        w[1] = (uint32_t)f32_to_bf16(o[dt][2] * inv) | ((uint32_t)f32_to_bf16(o[dt][3] * inv) << 16);
        *(u32x2_t*)(orow + dt * 16 + 4 * jq) = w;
      }
    }
  } else {
    float* po = a.part_o + ((size_t)unit * 16 + cq) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *(f32x4_t*)(po + dt * 16 + 4 * jq) = o[dt];
    if (jq == 0) {
      a.part_ml[(size_t)unit * 32 + cq] = m_run;
      a.part_ml[(size_t)unit * 32 + 16 + cq] = l_run;
    }
  }
}

// combine the splits of one (KV head, row tile): o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int rtiles) {
  const int tile = blockIdx.x;  // kvh * rtiles + rt
  const int rt = tile % rtiles, kvh = tile / rtiles;
  const int grp = a.hq / a.g.hkv;
  const int R = a.n * grp;
  for (int e = threadIdx.x; e < 16 * D; e += blockDim.x) {
    const int c = e / D, dim = e % D;
    const int r = rt * 16 + c;
    if (r >= R) continue;
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s)
      M = fmaxf(M, a.part_ml[((size_t)tile * a.splits + s) * 32 + c]);
    float L = 0.f, acc = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < a.splits; ++s) {
        const size_t u = (size_t)tile * a.splits + s;
        const float m = a.part_ml[u * 32 + c];
        if (m == -INFINITY) continue;
        const float w = __expf(m - M);
        L += w * a.part_ml[u * 32 + 16 + c];
        acc += w * a.part_o[(u * 16 + c) * D + dim];
      }
    }
    const int t = r / grp, h = kvh * grp + r % grp;
    ((bf16_t*)a.out)[((size_t)t * a.hq + h) * D + dim] = f32_to_bf16(L > 0.f ? acc / L : 0.f);
  }
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

template <int D>
static void attn_bf16_launch(const AttnArgs& a, int rtiles, hipStream_t s) {
  const int units = a.g.hkv * rtiles * a.splits;
  attn_bf16_kernel<D><<<(units + 3) / 4, 256, 0, s>>>(a, rtiles);
  if (a.splits > 1) attn_merge_kernel<D><<<a.g.hkv * rtiles, 256, 0, s>>>(a, rtiles);
}

hipError_t launch_attention(const AttnArgs& a, int dt, hipStream_t s) {
  if (a.nlb <= 0 || a.n <= 0) return hipErrorInvalidValue;
  if (dt == DT_F32) {
    if (a.nlb * a.g.bt > kF32MaxKeys) return hipErrorInvalidValue;
    attn_f32_kernel<<<(a.n * a.hq + 3) / 4, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.splits > 1 && (a.part_o == nullptr || a.part_ml == nullptr)) return hipErrorInvalidValue;
  const int rtiles = (a.n * (a.hq / a.g.hkv) + 15) / 16;
  switch (a.g.d) {
    case 64: attn_bf16_launch<64>(a, rtiles, s); break;
    case 128: attn_bf16_launch<128>(a, rtiles, s); break;
    case 256: attn_bf16_launch<256>(a, rtiles, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vla

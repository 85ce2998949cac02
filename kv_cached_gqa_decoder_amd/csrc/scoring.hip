// Redundant-frame scoring ("Can an LLM Forget the Right Things?", section 5:
// evict the frame most similar to another one, by cosine similarity; the
// cosine is a dot product over two norms, 0 below a 1e-8 denominator).
//
// mean keys   fp64 mean over a frame's tokens of its stored keys, per layer,
//             all KV heads concatenated. A sum of bf16 or fp32 values in fp64
//             is exact here, so the result does not depend on the order.
// scoring     one workgroup per frame i computes s_ij for every j != i and
//             m_i = max_j s_ij; the pair value is a pure function of the
//             unordered pair (the dot product is symmetric in its operands
//             (an fma's product is exact), the norms and the dot use one fixed
//             summation shape), so s_ij == s_ji bit for bit. A second kernel
//             takes argmax_i m_i with ties to the lowest index.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace vla {

// one lane per V consecutive dims (8 or 16 bytes) of one (frame, layer): the
// frame's tokens are added in token order (the same order for every dim and
// every run), two blocks (32 tokens) of loads in flight per step
template <typename T, int V>
struct KeyVec {
  static_assert(V * sizeof(T) == 8 || V * sizeof(T) == 16, "8- or 16-byte loads");
  using type = typename std::conditional<V * sizeof(T) == 16, u32x4_t, u32x2_t>::type;
};

template <typename T, int V>
__global__ __launch_bounds__(64) void meankeys_kernel(const T* kp, KvGeom g, const int* blk_table,
                                                      const int* fr_blk0, const int* fr_nblk,
                                                      const int* fr_ntok, const int* fr_slot,
                                                      int layer0, double* table, int max_frames) {
  using W = typename KeyVec<T, V>::type;
  const int f = blockIdx.x;
  const int layer = layer0 + blockIdx.y;
  const int D = g.hkv * g.d;
  const int i0 = (blockIdx.z * 64 + threadIdx.x) * V;  // first dim of this lane
  if (i0 >= D) return;
  const int h = i0 / g.d, dd = i0 % g.d;
  const int blk0 = fr_blk0[f], nblk = fr_nblk[f], ntok = fr_ntok[f];
  double acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.0;
  for (int k = 0; k < nblk; k += 2) {
    W w[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kk = k + j < nblk ? k + j : k;
      const int b = blk_table[blk0 + kk];
#pragma unroll
      for (int sl = 0; sl < 16; ++sl) w[j][sl] = *(const W*)(kp + g.kidx(layer, b, h, sl, dd));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (k + j >= nblk) break;
      const int nt = min(g.bt, ntok - (k + j) * g.bt);
#pragma unroll
      for (int sl = 0; sl < 16; ++sl) {
        if (sl >= nt) break;
        const T* v = (const T*)&w[j][sl];
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] += (double)St<T>::ld(v, e);
      }
    }
  }
  double* out = table + ((size_t)layer * max_frames + fr_slot[f]) * D + i0;
#pragma unroll
  for (int e = 0; e < V; ++e) out[e] = acc[e] / (double)ntok;
}

template <typename T, int V>
static void meankeys_go(const void* kpool, KvGeom g, const int* blk_table, const int* fr_blk0,
                        const int* fr_nblk, const int* fr_ntok, const int* fr_slot, int nframes,
                        int layer0, int nlayers, double* table, int max_frames, hipStream_t s) {
  const int D = g.hkv * g.d;
  dim3 grid(nframes, nlayers, (D / V + 63) / 64);
  launch_k(meankeys_kernel<T, V>, grid, dim3(64), 0, s, (const T*)kpool, g, blk_table, fr_blk0,
           fr_nblk, fr_ntok, fr_slot, layer0, table, max_frames);
}

hipError_t launch_meankeys(const void* kpool, KvGeom g, const int* blk_table, const int* fr_blk0,
                           const int* fr_nblk, const int* fr_ntok, const int* fr_slot, int nframes,
                           int layer0, int nlayers, double* table, int max_frames, int dt,
                           hipStream_t s) {
  if (nframes <= 0 || nlayers <= 0) return hipSuccess;
  const int D = g.hkv * g.d;
  if (g.bt != 16) return hipErrorInvalidValue;
  // 8-byte loads while they keep all 64 lanes busy, else 16-byte loads
  const bool narrow = D <= 64 * (dt == DT_F32 ? 2 : 4);
  if (dt == DT_F32) {
    if (g.d % 4) return hipErrorInvalidValue;
    if (narrow)
      meankeys_go<float, 2>(kpool, g, blk_table, fr_blk0, fr_nblk, fr_ntok, fr_slot, nframes,
                            layer0, nlayers, table, max_frames, s);
    else
      meankeys_go<float, 4>(kpool, g, blk_table, fr_blk0, fr_nblk, fr_ntok, fr_slot, nframes,
                            layer0, nlayers, table, max_frames, s);
  } else {
    if (g.d % 8) return hipErrorInvalidValue;
    if (narrow)
      meankeys_go<bf16_t, 4>(kpool, g, blk_table, fr_blk0, fr_nblk, fr_ntok, fr_slot, nframes,
                             layer0, nlayers, table, max_frames, s);
    else
      meankeys_go<bf16_t, 8>(kpool, g, blk_table, fr_blk0, fr_nblk, fr_ntok, fr_slot, nframes,
                             layer0, nlayers, table, max_frames, s);
  }
  return hipGetLastError();
}

// Row i of the pair matrix: s_ij = dot(lo, hi) / (|lo| |hi|) with lo = min(i, j),
// hi = max(i, j), for every j != i, and m_i = max_j s_ij. Every fp64 sum over the
// D dims has one fixed shape whatever the workgroup: lane k adds dims k, k+64,
// ... in order (fma), then a fixed xor tree across the 64 lanes. So s_ij, |a|^2
// and |b|^2 come out bit-identical in the workgroups of i and of j, and the pair
// value is the same for both rows. 16 wavefronts per row, 4 rows j in flight per
// wavefront (independent loads and reductions).
constexpr int kScoreWaves = 16;
constexpr int kScoreBatch = 4;

__global__ __launch_bounds__(kScoreWaves * 64) void score_rows_kernel(const double* tab,
                                                                      const int* fr_slot, int F,
                                                                      int D, double* m_out) {
  __shared__ double wmax[kScoreWaves];
  const int i = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const double* a = tab + (size_t)fr_slot[i] * D;
  // |row i|^2 (every wavefront computes it the same way)
  double aa = 0.0;
  for (int k = lane; k < D; k += 64) aa = fma(a[k], a[k], aa);
  aa = wave_sum_d(aa);
  double best = -INFINITY;
  for (int j0 = wave * kScoreBatch; j0 < F; j0 += kScoreWaves * kScoreBatch) {
    double ab[kScoreBatch], bb[kScoreBatch];
    const double* b[kScoreBatch];
#pragma unroll
    for (int u = 0; u < kScoreBatch; ++u) {
      ab[u] = 0.0;
      bb[u] = 0.0;
      const int j = min(j0 + u, F - 1);
      b[u] = tab + (size_t)fr_slot[j] * D;
    }
#pragma unroll 2
    for (int k = lane; k < D; k += 64) {
      const double x = a[k];
#pragma unroll
      for (int u = 0; u < kScoreBatch; ++u) {
        const double y = b[u][k];
        ab[u] = fma(x, y, ab[u]);
        bb[u] = fma(y, y, bb[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kScoreBatch; ++u) {
      ab[u] = wave_sum_d(ab[u]);
      bb[u] = wave_sum_d(bb[u]);
    }
#pragma unroll
    for (int u = 0; u < kScoreBatch; ++u) {
      const int j = j0 + u;
      if (j >= F || j == i) continue;
      // (lo, hi) order: |lo|^2 and |hi|^2 are row i's or row j's, whichever is lower
      const double nlo = i < j ? aa : bb[u];
      const double nhi = i < j ? bb[u] : aa;
      const double den = sqrt(nlo) * sqrt(nhi);
      const double sij = den < 1e-8 ? 0.0 : ab[u] / den;
      best = sij > best ? sij : best;
    }
  }
  if (lane == 0) wmax[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    double mx = wmax[0];
    for (int w = 1; w < kScoreWaves; ++w) mx = wmax[w] > mx ? wmax[w] : mx;
    m_out[i] = mx;
  }
}

// argmax over m[0..F), ties to the lowest index; result[0] = index, result[1] = value
__global__ __launch_bounds__(256) void score_argmax_kernel(const double* m, int F, double* result) {
  __shared__ double sv[256];
  __shared__ int si[256];
  double bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < F; i += 256) {
    if (m[i] > bv) { bv = m[i]; bi = i; }  // ascending i: strict > keeps the lowest
  }
  sv[threadIdx.x] = bv;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      const double v2 = sv[threadIdx.x + o];
      const int i2 = si[threadIdx.x + o];
      if (v2 > sv[threadIdx.x] || (v2 == sv[threadIdx.x] && i2 < si[threadIdx.x])) {
        sv[threadIdx.x] = v2;
        si[threadIdx.x] = i2;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    result[0] = (double)si[0];
    result[1] = sv[0];
  }
}

hipError_t launch_score(const double* table_layer, const int* fr_slot, int nframes, int D,
                        double* m_out, double* result, hipStream_t s) {
  if (nframes < 2) return hipErrorInvalidValue;
  launch_k(score_rows_kernel, dim3(nframes), dim3(kScoreWaves * 64), 0, s, table_layer, fr_slot,
           nframes, D, m_out);
  launch_k(score_argmax_kernel, dim3(1), dim3(256), 0, s, (const double*)m_out, nframes, result);
  return hipGetLastError();
}

}  // namespace vla

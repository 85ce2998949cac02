// Redundant-frame scoring ("Can an LLM Forget the Right Things?", section 5:
// evict the frame most similar to another one, by cosine similarity; the
// cosine is a dot product over two norms, 0 below a 1e-8 denominator).
//
// mean keys   fp64 mean over a frame's tokens of its stored keys, per layer,
//             all KV heads concatenated. A sum of bf16 or fp32 values in fp64
//             is exact here, so the result does not depend on the order.
// scoring     one workgroup per frame i computes s_ij for every j != i and
//             m_i = max_j s_ij; the pair value is a pure function of the
//             unordered pair (same operand order, same reduction tree for
//             (i, j) and (j, i)), so s_ij == s_ji bit for bit. A second
//             kernel takes argmax_i m_i with ties to the lowest index.
#include "common.hpp"
#include "kernels.hpp"

namespace vla {

// one lane per 8 consecutive dims of one (frame, layer): the frame's tokens are
// added in token order (the same order for every dim and every run), two
// blocks (32 tokens) of 16-byte loads in flight per step
template <typename T>
__global__ __launch_bounds__(64) void meankeys_kernel(const T* kp, KvGeom g, const int* blk_table,
                                                      const int* fr_blk0, const int* fr_nblk,
                                                      const int* fr_ntok, const int* fr_slot,
                                                      int layer0, double* table, int max_frames) {
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte load
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
    u32x4_t w[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kk = k + j < nblk ? k + j : k;
      const int b = blk_table[blk0 + kk];
#pragma unroll
      for (int sl = 0; sl < 16; ++sl)
        w[j][sl] = *(const u32x4_t*)(kp + g.kidx(layer, b, h, sl, dd));
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

hipError_t launch_meankeys(const void* kpool, KvGeom g, const int* blk_table, const int* fr_blk0,
                           const int* fr_nblk, const int* fr_ntok, const int* fr_slot, int nframes,
                           int layer0, int nlayers, double* table, int max_frames, int dt,
                           hipStream_t s) {
  if (nframes <= 0 || nlayers <= 0) return hipSuccess;
  const int D = g.hkv * g.d;
  const int V = dt == DT_F32 ? 4 : 8;
  if (g.bt != 16 || g.d % V) return hipErrorInvalidValue;
  dim3 grid(nframes, nlayers, (D / V + 63) / 64);
  if (dt == DT_F32)
    launch_k(meankeys_kernel<float>, grid, dim3(64), 0, s, (const float*)kpool, g, blk_table,
             fr_blk0, fr_nblk, fr_ntok, fr_slot, layer0, table, max_frames);
  else
    launch_k(meankeys_kernel<bf16_t>, grid, dim3(64), 0, s, (const bf16_t*)kpool, g, blk_table,
             fr_blk0, fr_nblk, fr_ntok, fr_slot, layer0, table, max_frames);
  return hipGetLastError();
}

// dot product of two fp64 rows by one wavefront: lane sums k = lane, lane+64, ...
// in order, then a fixed xor-tree across lanes
__device__ __forceinline__ double wave_dot(const double* x, const double* y, int D, int lane) {
  double s = 0.0;
  for (int k = lane; k < D; k += 64) s = fma(x[k], y[k], s);
  return wave_sum_d(s);
}

__global__ __launch_bounds__(256) void score_rows_kernel(const double* tab, const int* fr_slot,
                                                         int F, int D, double* m_out) {
  __shared__ double wmax[4];
  const int i = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double best = -INFINITY;
  for (int j = wave; j < F; j += 4) {
    if (j == i) continue;
    const int lo = min(i, j), hi = max(i, j);
    const double* a = tab + (size_t)fr_slot[lo] * D;
    const double* b = tab + (size_t)fr_slot[hi] * D;
    const double dot = wave_dot(a, b, D, lane);
    const double na = wave_dot(a, a, D, lane);
    const double nb = wave_dot(b, b, D, lane);
    const double den = sqrt(na) * sqrt(nb);
    const double sij = den < 1e-8 ? 0.0 : dot / den;
    best = sij > best ? sij : best;
  }
  if (lane == 0) wmax[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    double m = wmax[0];
    for (int w = 1; w < 4; ++w) m = wmax[w] > m ? wmax[w] : m;
    m_out[i] = m;
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
  launch_k(score_rows_kernel, dim3(nframes), dim3(256), 0, s, table_layer, fr_slot, nframes, D,
           m_out);
  launch_k(score_argmax_kernel, dim3(1), dim3(256), 0, s, (const double*)m_out, nframes, result);
  return hipGetLastError();
}

}  // namespace vla

// Redundant-frame scoring ("Can an LLM Forget the Right Things?", section 5:
// evict the frame most similar to another one, by cosine similarity; the
// cosine is a dot product over two norms, 0 below a 1e-8 denominator).
//
// mean keys   fp64 mean over a frame's tokens of its stored keys, per layer,
//             all KV heads concatenated. For bf16 keys (8 significant bits) a
//             sum of up to 2^45 values is exact in fp64 whenever the exponents
//             of the summed values span at most 45 - log2(count) binades, so it
//             does not depend on the order: the device and a plain left-to-right
//             sum agree bit for bit. For fp32 keys (24 bits) that span shrinks to
//             29 - log2(count) binades; outside it the 4-way split below and a
//             sequential sum may round differently (last-bit differences).
// scoring     one workgroup per frame i computes s_ij for every j != i and
//             m_i = max_j s_ij; the pair value is a pure function of the
//             unordered pair (the dot product is symmetric in its operands
//             (an fma's product is exact), the norms and the dot use one fixed
//             summation shape), so s_ij == s_ji bit for bit. A second kernel
//             takes argmax_i m_i with ties to the lowest index.
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace vla {

// one lane per V consecutive dims (8 or 16 bytes) of one (frame, layer); the 4
// wavefronts of a workgroup take the frame's blocks round-robin, one block (16
// token loads per lane) per step, the next step's block id requested before the
// current step's keys are added; few registers, so many workgroups are resident. fp64 sums of bf16 keys
// are exact (see above), so the 4 partial sums (added through LDS) give the same
// table whatever the split.
template <typename T, int V>
struct KeyVec {
  static_assert(V * sizeof(T) == 8 || V * sizeof(T) == 16, "8- or 16-byte loads");
  using type = typename std::conditional<V * sizeof(T) == 16, u32x4_t, u32x2_t>::type;
};

// element e of a loaded key vector (bf16 pairs or fp32 words), without going
// through memory
template <typename T, typename W>
__device__ __forceinline__ float key_elem(const W& w, int e) {
  if constexpr (sizeof(T) == 2)
    return __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
  else
    return __uint_as_float(w[e]);
}

typedef const __attribute__((address_space(4))) int* mk_const_int_p;
__device__ __forceinline__ int mk_uniform_ld(const int* p, int i) {
  return ((mk_const_int_p)(const void*)p)[i];
}

template <typename T, int V>
__global__ __launch_bounds__(256) void meankeys_kernel(const T* kp, KvGeom g, const int* blk_table,
                                                       const int* fr_blk0, const int* fr_nblk,
                                                       const int* fr_ntok, const int* fr_slot,
                                                       int layer0, double* table, int max_frames) {
  using W = typename KeyVec<T, V>::type;
  constexpr int BPS = 1;  // blocks per wavefront step: few registers, many resident wavefronts
  __shared__ double red[4][64][V];
  const int f = blockIdx.x;
  const int layer = layer0 + blockIdx.y;
  const int D = g.hkv * g.d;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int i0 = min((int)(blockIdx.z * 64 + lane) * V, D - V);  // first dim of this lane
  const int h = i0 / g.d, dd = i0 % g.d;
  const int blk0 = mk_uniform_ld(fr_blk0, f), nblk = mk_uniform_ld(fr_nblk, f);
  const int ntok = mk_uniform_ld(fr_ntok, f);
  const int mine = nblk > wave ? (nblk - 1 - wave) / 4 + 1 : 0;  // this wavefront's blocks
  double acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.0;
  // block i of this wavefront: frame block wave + 4 i (ids past `mine` re-read a valid one)
  auto ids = [&](int i0b, int (&b)[BPS]) {
#pragma unroll
    for (int j = 0; j < BPS; ++j) {
      const int i = min(i0b + j, mine - 1);
      b[j] = mk_uniform_ld(blk_table, blk0 + wave + 4 * i);
    }
  };
  int bcur[BPS], bnext[BPS];
  if (mine > 0) ids(0, bcur);
  for (int i = 0; i < mine; i += BPS) {
    W w[BPS][16];
#pragma unroll
    for (int j = 0; j < BPS; ++j) {
      if (i + j < mine) {  // wave-uniform: only this wavefront's own blocks
#pragma unroll
        for (int sl = 0; sl < 16; ++sl) w[j][sl] = *(const W*)(kp + g.kidx(layer, bcur[j], h, sl, dd));
      } else {
#pragma unroll
        for (int sl = 0; sl < 16; ++sl) w[j][sl] = W{};
      }
    }
    if (i + BPS < mine) ids(i + BPS, bnext);
    // valid tokens of each block (0 past this wavefront's blocks); predicated adds,
    // no loop exits, so the loaded vectors stay in registers
#pragma unroll
    for (int j = 0; j < BPS; ++j) {
      const int kb = wave + 4 * (i + j);
      const int nt = i + j < mine ? min(g.bt, ntok - kb * g.bt) : 0;
#pragma unroll
      for (int sl = 0; sl < 16; ++sl) {
        const bool on = sl < nt;
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] += on ? (double)key_elem<T>(w[j][sl], e) : 0.0;
      }
    }
#pragma unroll
    for (int j = 0; j < BPS; ++j) bcur[j] = bnext[j];
  }
#pragma unroll
  for (int e = 0; e < V; ++e) red[wave][lane][e] = acc[e];
  __syncthreads();
  if (wave != 0 || (int)(blockIdx.z * 64 + lane) * V >= D) return;
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = ((red[0][lane][e] + red[1][lane][e]) + red[2][lane][e]) + red[3][lane][e];
  double* out = table + ((size_t)layer * max_frames + mk_uniform_ld(fr_slot, f)) * D + i0;
#pragma unroll
  for (int e = 0; e < V; ++e) out[e] = acc[e] / (double)ntok;
}

template <typename T, int V>
static void meankeys_go(const void* kpool, KvGeom g, const int* blk_table, const int* fr_blk0,
                        const int* fr_nblk, const int* fr_ntok, const int* fr_slot, int nframes,
                        int layer0, int nlayers, double* table, int max_frames, hipStream_t s) {
  const int D = g.hkv * g.d;
  dim3 grid(nframes, nlayers, (D / V + 63) / 64);
  launch_k(meankeys_kernel<T, V>, grid, dim3(256), 0, s, (const T*)kpool, g, blk_table, fr_blk0,
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
// value is the same for both rows. 16 wavefronts per row, 8 rows j in flight per
// wavefront (independent loads and reductions; 128 frames take one batch per
// wavefront). The frame slots are read with scalar loads (the index is uniform).
constexpr int kScoreWaves = 16;
constexpr int kScoreBatch = 8;

// KD > 0: rows of at most 64 * KD dims, every load of a batch issued together (indexes
// past the row clamped to its last element and masked in the sums); KD = 0: any D
template <int KD>
__global__ __launch_bounds__(kScoreWaves * 64) void score_rows_kernel(const double* tab,
                                                                      const int* fr_slot, int F,
                                                                      int D, double* m_out) {
  __shared__ double wmax[kScoreWaves];
  const int i = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // fr_slot null: the table rows are the frames themselves, in order
  const double* a = tab + (size_t)(fr_slot ? mk_uniform_ld(fr_slot, i) : i) * D;
  // |row i|^2 (every wavefront computes it the same way)
  double aa = 0.0;
  double av[KD > 0 ? KD : 1];
  if constexpr (KD > 0) {
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      const int k = lane + 64 * kk;
      av[kk] = a[k < D ? k : D - 1];
      av[kk] = k < D ? av[kk] : 0.0;
      aa = fma(av[kk], av[kk], aa);
    }
  } else {
    for (int k = lane; k < D; k += 64) aa = fma(a[k], a[k], aa);
  }
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
      b[u] = tab + (size_t)(fr_slot ? mk_uniform_ld(fr_slot, j) : j) * D;
    }
    if constexpr (KD > 0) {
      double y[kScoreBatch][KD];
#pragma unroll
      for (int u = 0; u < kScoreBatch; ++u)
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
          const int k = lane + 64 * kk;
          y[u][kk] = b[u][k < D ? k : D - 1];
        }
#pragma unroll
      for (int u = 0; u < kScoreBatch; ++u)
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
          const double yv = lane + 64 * kk < D ? y[u][kk] : 0.0;
          ab[u] = fma(av[kk], yv, ab[u]);
          bb[u] = fma(yv, yv, bb[u]);
        }
    } else {
#pragma unroll 2
      for (int k = lane; k < D; k += 64) {
        const double x = a[k];
#pragma unroll
        for (int u = 0; u < kScoreBatch; ++u) {
          const double yv = b[u][k];
          ab[u] = fma(x, yv, ab[u]);
          bb[u] = fma(yv, yv, bb[u]);
        }
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


// rows of up to 256 dims (the Qwen shape's 2 x 128) take the fully issued batch
static void launch_score_rows(dim3 grid, hipStream_t s, const double* tab, const int* fr_slot,
                              int F, int D, double* m_out) {
  if (D <= 256)
    launch_k(score_rows_kernel<4>, grid, dim3(kScoreWaves * 64), 0, s, tab, fr_slot, F, D, m_out);
  else
    launch_k(score_rows_kernel<0>, grid, dim3(kScoreWaves * 64), 0, s, tab, fr_slot, F, D, m_out);
}

// argmax over m[0..F), ties to the lowest index: result[0] = index, result[1] =
// value (result non-null), or *out_idx = index, *out_val = value
__global__ __launch_bounds__(256) void score_argmax_kernel(const double* m, int F, double* result,
                                                           int* out_idx, double* out_val) {
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
    if (result) {
      result[0] = (double)si[0];
      result[1] = sv[0];
    } else {
      *out_idx = si[0];
      *out_val = sv[0];
    }
  }
}

// Adjacent pairs, the page's own rule ("Can an LLM Forget the Right Things?",
// section 5: compare each retained frame with the next one and evict the older frame
// of the most similar pair): s_i = cos(frame i, frame i + 1) in arrival order. The
// sums have the all-pairs kernel's fixed shape (lane k adds dims k, k+64, ... by fma,
// then the xor tree; |lo|^2 from frame i), so s_i equals that kernel's value of the
// pair bit for bit. One wavefront per pair.
__global__ __launch_bounds__(64) void score_adjacent_kernel(const double* tab, const int* fr_slot,
                                                            int D, double* s_out) {
  const int i = blockIdx.x, lane = threadIdx.x;
  const double* a = tab + (size_t)fr_slot[i] * D;
  const double* b = tab + (size_t)fr_slot[i + 1] * D;
  double ab = 0.0, aa = 0.0, bb = 0.0;
  for (int k = lane; k < D; k += 64) {
    const double x = a[k], y = b[k];
    ab = fma(x, y, ab);
    aa = fma(x, x, aa);
    bb = fma(y, y, bb);
  }
  ab = wave_sum_d(ab);
  aa = wave_sum_d(aa);
  bb = wave_sum_d(bb);
  if (lane == 0) {
    const double den = sqrt(aa) * sqrt(bb);
    s_out[i] = den < 1e-8 ? 0.0 : ab / den;
  }
}

hipError_t launch_score_adjacent(const double* table_layer, const int* fr_slot, int nframes, int D,
                                 double* s_out, double* result, hipStream_t s) {
  if (nframes < 2) return hipErrorInvalidValue;
  launch_k(score_adjacent_kernel, dim3(nframes - 1), dim3(64), 0, s, table_layer, fr_slot, D,
           s_out);
  launch_k(score_argmax_kernel, dim3(1), dim3(256), 0, s, (const double*)s_out, nframes - 1, result,
           (int*)nullptr, (double*)nullptr);
  return hipGetLastError();
}

hipError_t launch_score(const double* table_layer, const int* fr_slot, int nframes, int D,
                        double* m_out, double* result, hipStream_t s) {
  if (nframes < 2) return hipErrorInvalidValue;
  launch_score_rows(dim3(nframes), s, table_layer, fr_slot,
           nframes, D, m_out);
  launch_k(score_argmax_kernel, dim3(1), dim3(256), 0, s, (const double*)m_out, nframes, result,
           (int*)nullptr, (double*)nullptr);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scoring that allocates nothing: the per-frame scores m_i live in a
// file-scope device array (one copy per GPU, alive until the process ends)
// instead of a model's scratch. Its device address is looked up once per GPU
// with hipGetSymbolAddress and only that address is passed to the kernels (in
// host code the array's name does not denote device memory). Every frame's
// score is written before the argmax reads it, so nothing needs clearing; two
// calls in flight on one GPU share the array and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) double scratch[kScoreNoAllocMaxFrames];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
double* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t launch_score_noalloc(const double* table, int nframes, int D, int* out_idx,
                                double* out_score, hipStream_t s) {
  if (nframes < 2 || nframes > kScoreNoAllocMaxFrames || D < 1) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  double* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch_ptr[dev] = (double*)p;
    }
    ptr = g_scratch_ptr[dev];
  }
  launch_score_rows(dim3(nframes), s, table,
           (const int*)nullptr, nframes, D, ptr);
  launch_k(score_argmax_kernel, dim3(1), dim3(256), 0, s, (const double*)ptr, nframes,
           (double*)nullptr, out_idx, out_score);
  return hipGetLastError();
}

}  // namespace vla

// Decode projections (one token row): weight-streaming GEMV with fused input
// RMSNorm and fused epilogues (RoPE + paged KV write, residual add, SwiGLU,
// output head with argmax). HBM-bound: every weight byte is read once with
// 16-byte loads; the input row lives in LDS as fp32.
#include "common.hpp"
#include "epilogue.hpp"
#include "kernels.hpp"

namespace vla {

constexpr int kGemvThreads = 256;
constexpr int kGemvRows = 4;  // output rows per workgroup step

// physical rows handled by row group `grp`
template <int EPI>
__device__ __forceinline__ void gemv_rows(int grp, int64_t* rows) {
  if constexpr (EPI == EPI_SWIGLU) {
    // gate rows of f = 2grp, 2grp+1 and their up rows (LAYOUT_GATEUP)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f = 2 * grp + i;
      rows[i] = (int64_t)(f / 16) * 32 + (f % 16);
      rows[2 + i] = rows[i] + 16;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kGemvRows; ++i) rows[i] = (int64_t)grp * kGemvRows + i;
  }
}

template <typename T, int EPI>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs a, int ngroups) {
  extern __shared__ float xs[];  // the input row, fp32
  __shared__ float red[kGemvThreads / 64][kGemvRows];
  __shared__ float ys[kGemvRows];
  __shared__ float ssq[kGemvThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  const T* x = (const T*)a.x;

  float ss = 0.f;
  for (int i = tid; i < K; i += kGemvThreads) {
    const float v = St<T>::ld(x, i);
    xs[i] = v;
    ss += v * v;
  }
  if (a.norm_g) {  // RMSNorm of the input row (fp32 statistics)
    ss = wave_sum(ss);
    if (lane == 0) ssq[wave] = ss;
    __syncthreads();
    const float r = rsqrtf((ssq[0] + ssq[1] + ssq[2] + ssq[3]) / (float)K + a.eps);
    for (int i = tid; i < K; i += kGemvThreads) xs[i] = xs[i] * r * a.norm_g[i];
  }
  __syncthreads();

  constexpr int CH = 16 / sizeof(T);  // elements per 16-byte load
  const int nch = K / CH;
  const T* W = (const T*)a.W;
  unsigned long long best = 0ull;

  for (int grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    int64_t rows[kGemvRows];
    gemv_rows<EPI>(grp, rows);
    bool ok[kGemvRows];
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) ok[r] = rows[r] < a.N;
    float acc[kGemvRows];
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) acc[r] = 0.f;

    for (int c = tid; c < nch; c += kGemvThreads) {
      float xv[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) xv[i] = xs[c * CH + i];
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r) {
        if (!ok[r]) continue;
        const u32x4_t w = *(const u32x4_t*)(W + rows[r] * K + (int64_t)c * CH);
        float wf[CH];
        if constexpr (sizeof(T) == 2) {
          unpack8(w, wf);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) wf[i] = __uint_as_float(w[i]);
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) acc[r] += wf[i] * xv[i];
      }
    }
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) acc[r] = wave_sum(acc[r]);
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r) red[wave][r] = acc[r];
    }
    __syncthreads();
    if (tid < kGemvRows) ys[tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    __syncthreads();

    if constexpr (EPI == EPI_QKV) {
      if (tid < kGemvRows / 2)
        epi_qkv_pair<T>(a.ctx, 0, (int)rows[2 * tid], ys[2 * tid], ys[2 * tid + 1]);
    } else if constexpr (EPI == EPI_RESID) {
      if (tid < kGemvRows && ok[tid]) {
        T* xo = (T*)a.out;
        St<T>::st(xo, rows[tid], St<T>::ld(xo, rows[tid]) + ys[tid]);
      }
    } else if constexpr (EPI == EPI_SWIGLU) {
      if (tid < 2) St<T>::st((T*)a.out, 2 * grp + tid, silu(ys[tid]) * ys[2 + tid]);
    } else if constexpr (EPI == EPI_HEAD) {
      if (tid == 0) {
#pragma unroll
        for (int r = 0; r < kGemvRows; ++r) {
          if (!ok[r]) continue;
          ((float*)a.out)[rows[r]] = ys[r];
          const unsigned long long k = argmax_key(ys[r], (uint32_t)rows[r]);
          best = k > best ? k : best;
        }
      }
    }
    __syncthreads();
  }
  if constexpr (EPI == EPI_HEAD) {
    if (tid == 0) a.argmax_part[blockIdx.x] = best;
  }
}

template <typename T, int EPI>
static hipError_t gemv_launch(const GemvArgs& a, hipStream_t s, int* grid_out) {
  int ngroups;
  if (EPI == EPI_SWIGLU) ngroups = a.N / 4;  // N = 2F physical rows, two f per group
  else ngroups = (a.N + kGemvRows - 1) / kGemvRows;
  int grid = ngroups < 2048 ? ngroups : 2048;
  if (grid_out) *grid_out = grid;
  const size_t lds = (size_t)a.K * sizeof(float);
  launch_k(gemv_kernel<T, EPI>, dim3(grid), dim3(kGemvThreads), (uint32_t)lds, s, a, ngroups);
  return hipGetLastError();
}

template <typename T>
static hipError_t gemv_dispatch(const GemvArgs& a, hipStream_t s, int* grid_out) {
  switch (a.epi) {
    case EPI_QKV: return gemv_launch<T, EPI_QKV>(a, s, grid_out);
    case EPI_RESID: return gemv_launch<T, EPI_RESID>(a, s, grid_out);
    case EPI_SWIGLU: return gemv_launch<T, EPI_SWIGLU>(a, s, grid_out);
    case EPI_HEAD: return gemv_launch<T, EPI_HEAD>(a, s, grid_out);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(const GemvArgs& a, int dt, hipStream_t s, int* grid_out) {
  if (a.K % 8 != 0) return hipErrorInvalidValue;
  return dt == DT_F32 ? gemv_dispatch<float>(a, s, grid_out)
                      : gemv_dispatch<bf16_t>(a, s, grid_out);
}

// final argmax over the per-workgroup keys (one workgroup)
__global__ __launch_bounds__(1024) void argmax_final_kernel(const unsigned long long* part,
                                                            int nparts,
                                                            unsigned long long* result) {
  __shared__ unsigned long long sm[1024];
  unsigned long long b = 0ull;
  for (int i = threadIdx.x; i < nparts; i += blockDim.x) b = part[i] > b ? part[i] : b;
  sm[threadIdx.x] = b;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      const unsigned long long c = sm[threadIdx.x + o];
      if (c > sm[threadIdx.x]) sm[threadIdx.x] = c;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) *result = sm[0];
}

hipError_t launch_argmax_final(const unsigned long long* part, int nparts,
                               unsigned long long* result, hipStream_t s) {
  argmax_final_kernel<<<1, 1024, 0, s>>>(part, nparts, result);
  return hipGetLastError();
}

}  // namespace vla

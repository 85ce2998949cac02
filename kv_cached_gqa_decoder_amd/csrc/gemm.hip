// Prefill projections C[M][N] = A[M][K] * W[N][K]^T with fused epilogues.
//  bf16: matrix-core kernel on v_mfma_f32_16x16x32_bf16 (fp32 accumulate),
//        LDS-staged 64-deep K tiles with register prefetch of the next tile.
//  fp32: FMA kernel (the fp32 configuration never touches bf16 matrix cores).
// Epilogues: plain store, residual add (x += C), RoPE + paged K/V write on the
// fused q/k/v projection, SwiGLU on the interleaved gate/up projection
// ("Running VLAs at Real-time Speed", section 4.2: both gated projections in
// one GEMM, only the gated product written back; section 4.4: bias-free
// residual and activation fused into the GEMM epilogue).
#include "common.hpp"
#include "epilogue.hpp"
#include "kernels.hpp"

namespace vla {

// ---------------------------------------------------------------------------
// bf16 matrix-core GEMM: block tile BM x 64, 4 wavefronts in a 2 x 2 grid,
// each wavefront BM/2 rows x 32 columns = (BM/32) x 2 tiles of 16 x 16.
// ---------------------------------------------------------------------------
constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;  // LDS row pitch in bf16 elements (144 B)

template <int EPI, int BM>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int BN = 64;
  constexpr int WM = BM / 2;
  constexpr int MT = WM / 16;
  constexpr int ACH = BM * 8 / 256;  // 16-byte chunks of the A tile per thread
  constexpr int WCH = BN * 8 / 256;
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * kPitch];
  __shared__ __attribute__((aligned(16))) bf16_t Ws[BN * kPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = a.M, K = a.K;
  const bf16_t* A = (const bf16_t*)a.A;
  const bf16_t* W = (const bf16_t*)a.W;

  f32x4_t acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ra[ACH], rw[WCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3, kc = (c & 7) * 8;
      const int row = m0 + r;
      ra[i] = row < M ? *(const u32x4_t*)(A + (int64_t)row * K + k0 + kc) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3, kc = (c & 7) * 8;
      rw[i] = *(const u32x4_t*)(W + (int64_t)(n0 + r) * K + k0 + kc);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + 256 * i;
      *(u32x4_t*)(As + (c >> 3) * kPitch + (c & 7) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + 256 * i;
      *(u32x4_t*)(Ws + (c >> 3) * kPitch + (c & 7) * 8) = rw[i];
    }
  };

  const int nk = K / kBK;
  gload(0);
  for (int kt = 0; kt < nk; ++kt) {
    lstore();
    __syncthreads();
    if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kk = ks * 32 + 8 * (lane >> 4);
      bf16x8_t bf[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bf[ni] = *(const bf16x8_t*)(Ws + (wn * 32 + ni * 16 + (lane & 15)) * kPitch + kk);
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const bf16x8_t af = *(const bf16x8_t*)(As + (wm * WM + mi * 16 + (lane & 15)) * kPitch + kk);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[ni], acc[mi][ni], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // accumulator element e of tile (mi, ni): row 4*(lane/16)+e, column lane%16
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = m0 + wm * WM + mi * 16 + 4 * (lane >> 4) + e;
      if constexpr (EPI == EPI_SWIGLU) {
        // tile ni=0 holds gate rows f, ni=1 the matching up rows (LAYOUT_GATEUP)
        const int f = (n0 + wn * 32) / 2 + (lane & 15);
        if (row < M)
          St<bf16_t>::st((bf16_t*)a.C, (size_t)row * (a.N / 2) + f,
                         silu(acc[mi][0][e]) * acc[mi][1][e]);
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int col = n0 + wn * 32 + ni * 16 + (lane & 15);
          const float v = acc[mi][ni][e];
          if constexpr (EPI == EPI_QKV) {
            const float partner = __shfl_xor(v, 1, 64);
            if (row < M && (col & 1) == 0) epi_qkv_pair<bf16_t>(a.ctx, row, col, v, partner);
          } else if constexpr (EPI == EPI_RESID) {
            if (row < M) {
              bf16_t* x = (bf16_t*)a.C + (size_t)row * a.N + col;
              *x = f32_to_bf16(bf16_to_f32(*x) + v);
            }
          } else {
            if (row < M) ((bf16_t*)a.C)[(size_t)row * a.N + col] = f32_to_bf16(v);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 FMA GEMM: 64 x 64 tile, 16-deep K steps, 4 x 4 outputs per thread; the
// epilogue runs from an LDS copy of the tile so any column pairing works.
// ---------------------------------------------------------------------------
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Ws[BK][BN + 4];
  __shared__ float Cs[BM][BN + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = a.M, N = a.N, K = a.K;
  const float* A = (const float*)a.A;
  const float* W = (const float*)a.W;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int r = e / BK, k = e % BK;
      const int row = m0 + r, kk = k0 + k;
      As[k][r] = (row < M && kk < K) ? A[(int64_t)row * K + kk] : 0.f;
      const int col = n0 + r;
      Ws[k][r] = (col < N && kk < K) ? W[(int64_t)col * K + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float av[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[k][ty * 4 + i];
        wv[i] = Ws[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * wv[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) Cs[ty * 4 + i][tx * 4 + j] = acc[i][j];
  __syncthreads();

  if constexpr (EPI == EPI_SWIGLU) {
    // 64 columns = two 32-column gate|up blocks -> 32 outputs per row
    for (int e = tid; e < BM * 32; e += 256) {
      const int r = e / 32, o = e % 32;
      const int blk = o / 16, cc = o % 16;
      const int row = m0 + r;
      if (row < M && n0 + blk * 32 < N)
        ((float*)a.C)[(size_t)row * (N / 2) + (n0 + blk * 32) / 2 + cc] =
            silu(Cs[r][blk * 32 + cc]) * Cs[r][blk * 32 + 16 + cc];
    }
  } else if constexpr (EPI == EPI_QKV) {
    for (int e = tid; e < BM * 32; e += 256) {
      const int r = e / 32, cp = (e % 32) * 2;
      const int row = m0 + r, col = n0 + cp;
      if (row < M && col < N) epi_qkv_pair<float>(a.ctx, row, col, Cs[r][cp], Cs[r][cp + 1]);
    }
  } else {
    for (int e = tid; e < BM * BN; e += 256) {
      const int r = e / BN, c = e % BN;
      const int row = m0 + r, col = n0 + c;
      if (row < M && col < N) {
        float* o = (float*)a.C + (size_t)row * N + col;
        *o = (EPI == EPI_RESID) ? *o + Cs[r][c] : Cs[r][c];
      }
    }
  }
}

template <int EPI>
static hipError_t gemm_launch(const GemmArgs& a, int dt, hipStream_t s) {
  if (dt == DT_F32) {
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
    launch_k(gemm_f32_kernel<EPI>, grid, dim3(256), 0, s, a);
  } else {
    if (a.K % kBK != 0 || a.N % 64 != 0) return hipErrorInvalidValue;
    if (a.M > 64) {
      dim3 grid(a.N / 64, (a.M + 127) / 128);
      launch_k(gemm_bf16_kernel<EPI, 128>, grid, dim3(256), 0, s, a);
    } else {
      dim3 grid(a.N / 64, (a.M + 63) / 64);
      launch_k(gemm_bf16_kernel<EPI, 64>, grid, dim3(256), 0, s, a);
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, int dt, hipStream_t s) {
  switch (a.epi) {
    case EPI_STORE: return gemm_launch<EPI_STORE>(a, dt, s);
    case EPI_RESID: return gemm_launch<EPI_RESID>(a, dt, s);
    case EPI_QKV: return gemm_launch<EPI_QKV>(a, dt, s);
    case EPI_SWIGLU: return gemm_launch<EPI_SWIGLU>(a, dt, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vla

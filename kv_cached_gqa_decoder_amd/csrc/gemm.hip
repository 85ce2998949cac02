// Prefill projections C[M][N] = A[M][K] * W[N][K]^T with fused epilogues.
//  bf16: matrix-core kernel on v_mfma_f32_16x16x32_bf16 (fp32 accumulate),
//        LDS-staged 64-deep K tiles with register prefetch of the next tile.
//  fp32: FMA kernel (the fp32 configuration never touches bf16 matrix cores).
// Epilogues: plain store, residual add (x += C), RoPE + paged K/V write on the
// fused q/k/v projection, SwiGLU on the interleaved gate/up projection
// ("Running VLAs at Real-time Speed", section 4.2: both gated projections in
// one GEMM, only the gated product written back; section 4.4: bias-free
// residual and activation fused into the GEMM epilogue).
#include <algorithm>

#include "common.hpp"
#include "epilogue.hpp"
#include "kernels.hpp"

namespace vla {

// ---------------------------------------------------------------------------
// bf16 matrix-core GEMM. Block tile BM x BN (64 or 128 each), 4 wavefronts in a
// 2 x 2 grid, each wavefront (BM/2) x (BN/2) = MT x NT tiles of 16 x 16 on
// v_mfma_f32_16x16x32_bf16. 64-deep K steps staged through a double-buffered
// LDS image (register prefetch of the next step, one barrier per step).
// Tiles are ordered so that each XCD (workgroup L runs on XCD L % 8) walks a
// contiguous run of tiles with the M tiles of one weight tile adjacent: the
// weight tile is fetched from HBM once and re-read from that XCD's L2.
// Split-K (blockIdx over splits) writes fp32 partials for the residual
// projections; a reduction kernel adds them to the residual in split order.
// ---------------------------------------------------------------------------
constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;  // LDS row pitch in bf16 elements (144 B)
constexpr int kXcds = 8;

template <int BM, int BN>
struct GemmTile {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MT = WM / 16, NT = WN / 16;
  static constexpr int ACH = BM * kBK / 8 / 256;  // 16-byte chunks per thread per step
  static constexpr int WCH = BN * kBK / 8 / 256;
  static constexpr int STAGE = (BM + BN) * kPitch;
};

template <int EPI, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a, int tiles_m, int tiles,
                                                        int ksteps) {
  using G = GemmTile<BM, BN>;
  constexpr int MT = G::MT, NT = G::NT;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * G::STAGE];

  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int slot = blockIdx.x % (kXcds * per_xcd);
  const int z = blockIdx.x / (kXcds * per_xcd);
  const int t = (slot % kXcds) * per_xcd + slot / kXcds;
  if (t >= tiles) return;
  const int m0 = (t % tiles_m) * BM, n0 = (t / tiles_m) * BN;
  const int M = a.M, K = a.K;
  const int kt0 = z * ksteps;
  const int nk = min(K / kBK - kt0, ksteps);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bf16_t* A = (const bf16_t*)a.A;
  const bf16_t* W = (const bf16_t*)a.W;

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ra[G::ACH], rw[G::WCH];
  auto gload = [&](int kt) {
    const int k0 = (kt0 + kt) * kBK;
#pragma unroll
    for (int i = 0; i < G::ACH; ++i) {
      const int c = tid + 256 * i;
      const int row = m0 + (c >> 3), kc = (c & 7) * 8;
      ra[i] = row < M ? *(const u32x4_t*)(A + (int64_t)row * K + k0 + kc) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < G::WCH; ++i) {
      const int c = tid + 256 * i;
      rw[i] = *(const u32x4_t*)(W + (int64_t)(n0 + (c >> 3)) * K + k0 + (c & 7) * 8);
    }
  };
  auto lstore = [&](bf16_t* st) {
#pragma unroll
    for (int i = 0; i < G::ACH; ++i) {
      const int c = tid + 256 * i;
      *(u32x4_t*)(st + (c >> 3) * kPitch + (c & 7) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < G::WCH; ++i) {
      const int c = tid + 256 * i;
      *(u32x4_t*)(st + (BM + (c >> 3)) * kPitch + (c & 7) * 8) = rw[i];
    }
  };

  if (nk > 0) {
    gload(0);
    lstore(smem);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
    const bf16_t* As = smem + (kt & 1) * G::STAGE;
    const bf16_t* Ws = As + BM * kPitch;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kk = ks * 32 + 8 * (lane >> 4);
      bf16x8_t bf[NT];
#pragma unroll
      for (int ni = 0; ni < NT; ++ni)
        bf[ni] = *(const bf16x8_t*)(Ws + (wn * G::WN + ni * 16 + (lane & 15)) * kPitch + kk);
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const bf16x8_t af =
            *(const bf16x8_t*)(As + (wm * G::WM + mi * 16 + (lane & 15)) * kPitch + kk);
#pragma unroll
        for (int ni = 0; ni < NT; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[ni], acc[mi][ni], 0, 0, 0);
      }
    }
    if (more) lstore(smem + ((kt + 1) & 1) * G::STAGE);
    __syncthreads();
  }

  // accumulator element e of tile (mi, ni): row 4*(lane/16)+e, column lane%16
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = m0 + wm * G::WM + mi * 16 + 4 * (lane >> 4) + e;
      if constexpr (EPI == EPI_SWIGLU) {
        // tiles (ni, ni+1), ni even: gate rows f and the matching up rows (LAYOUT_GATEUP)
#pragma unroll
        for (int ni = 0; ni < NT; ni += 2) {
          const int f = (n0 + wn * G::WN + ni * 16) / 2 + (lane & 15);
          if (row < M)
            St<bf16_t>::st((bf16_t*)a.C, (size_t)row * (a.N / 2) + f,
                           silu(acc[mi][ni][e]) * acc[mi][ni + 1][e]);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) {
          const int col = n0 + wn * G::WN + ni * 16 + (lane & 15);
          const float v = acc[mi][ni][e];
          if constexpr (EPI == EPI_QKV) {
            const float partner = __shfl_xor(v, 1, 64);
            if (row < M && (col & 1) == 0) epi_qkv_pair<bf16_t>(a.ctx, row, col, v, partner);
          } else {  // EPI_PARTIAL
            if (row < M) a.ws[((size_t)z * M + row) * a.N + col] = v;
          }
        }
      }
    }
  }
}

// x[row] += sum over splits of the partials (split order), rounded to bf16;
// then, if u is given, u[row] = RMSNorm(x[row]) with fp32 statistics. One
// workgroup per row; each thread keeps up to 4 chunks of 8 columns in registers.
constexpr int kResidMaxChunks = 4;
__global__ __launch_bounds__(256) void resid_norm_kernel(const float* ws, int splits, int M, int N,
                                                         bf16_t* x, bf16_t* u, const float* g,
                                                         float eps) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int nch = N / 8;
  float v[kResidMaxChunks][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kResidMaxChunks; ++j) {
    const int c = tid + 256 * j;
    if (c >= nch) continue;
    bf16_t* xp = x + (size_t)row * N + c * 8;
    unpack8(*(const u32x4_t*)xp, v[j]);
    for (int s = 0; s < splits; ++s) {
      const float* p = ws + ((size_t)s * M + row) * N + c * 8;
      const f32x4_t p0 = *(const f32x4_t*)p, p1 = *(const f32x4_t*)(p + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[j][i] += p0[i];
        v[j][4 + i] += p1[i];
      }
    }
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16_t lo = f32_to_bf16(v[j][2 * i]), hi = f32_to_bf16(v[j][2 * i + 1]);
      o[i] = (uint32_t)lo | ((uint32_t)hi << 16);
      v[j][2 * i] = bf16_to_f32(lo);
      v[j][2 * i + 1] = bf16_to_f32(hi);
      ss += v[j][2 * i] * v[j][2 * i] + v[j][2 * i + 1] * v[j][2 * i + 1];
    }
    *(u32x4_t*)xp = o;
  }
  if (u == nullptr) return;
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float r = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)N + eps);
#pragma unroll
  for (int j = 0; j < kResidMaxChunks; ++j) {
    const int c = tid + 256 * j;
    if (c >= nch) continue;
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)f32_to_bf16(v[j][2 * i] * r * g[c * 8 + 2 * i]) |
             ((uint32_t)f32_to_bf16(v[j][2 * i + 1] * r * g[c * 8 + 2 * i + 1]) << 16);
    *(u32x4_t*)(u + (size_t)row * N + c * 8) = o;
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
static hipError_t gemm_f32_launch(const GemmArgs& a, hipStream_t s) {
  dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
  launch_k(gemm_f32_kernel<EPI>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int EPI, int BM, int BN>
static void gemm_bf16_go(const GemmArgs& a, int splits, int ksteps, hipStream_t s) {
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles = tiles_m * (a.N / BN);
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  launch_k(gemm_bf16_kernel<EPI, BM, BN>, dim3(kXcds * per_xcd * splits), dim3(256), 0, s, a,
           tiles_m, tiles, ksteps);
}

template <int EPI>
static void gemm_bf16_shape(const GemmArgs& a, int bm, int bn, int splits, int ksteps,
                            hipStream_t s) {
  if (bm == 128 && bn == 128) gemm_bf16_go<EPI, 128, 128>(a, splits, ksteps, s);
  else if (bm == 128) gemm_bf16_go<EPI, 128, 64>(a, splits, ksteps, s);
  else if (bn == 128) gemm_bf16_go<EPI, 64, 128>(a, splits, ksteps, s);
  else gemm_bf16_go<EPI, 64, 64>(a, splits, ksteps, s);
}

// Tile shape: start from 128 x 128 (64 rows for short chunks) and narrow N, then
// M, while fewer than 192 tiles would run. Residual projections also split K so
// that about 256 workgroups run, each with at least 4 K steps.
static hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.K % kBK != 0 || a.N % 64 != 0 || a.M < 1) return hipErrorInvalidValue;
  int bm = a.M > 64 ? 128 : 64;
  int bn = a.N % 128 == 0 ? 128 : 64;
  auto ntiles = [&](int m, int n) { return ((a.M + m - 1) / m) * (a.N / n); };
  if (ntiles(bm, bn) < 192 && bn == 128) bn = 64;
  if (ntiles(bm, bn) < 192 && bm == 128) bm = 64;
  const int tiles = ntiles(bm, bn);
  const int ksteps_all = a.K / kBK;
  int splits = 1;
  if (a.epi == EPI_RESID) {
    splits = std::max(1, std::min(16, (256 + tiles - 1) / tiles));
    while (splits > 1 && ksteps_all / splits < 4) --splits;
    while (splits > 1 && (size_t)splits * a.M * a.N > a.ws_elems) --splits;
    if ((size_t)a.M * a.N > a.ws_elems || a.ws == nullptr) return hipErrorInvalidValue;
    if (a.N % 8 != 0 || a.N / 8 > 256 * kResidMaxChunks) return hipErrorInvalidValue;
  }
  const int ksteps = (ksteps_all + splits - 1) / splits;
  splits = (ksteps_all + ksteps - 1) / ksteps;
  switch (a.epi) {
    case EPI_QKV: gemm_bf16_shape<EPI_QKV>(a, bm, bn, 1, ksteps, s); break;
    case EPI_SWIGLU:
      if (a.N % 64 != 0) return hipErrorInvalidValue;
      gemm_bf16_shape<EPI_SWIGLU>(a, bm, bn, 1, ksteps, s);
      break;
    case EPI_RESID:
      gemm_bf16_shape<EPI_PARTIAL>(a, bm, bn, splits, ksteps, s);
      launch_k(resid_norm_kernel, dim3(a.M), dim3(256), 0, s, (const float*)a.ws, splits, a.M,
               a.N, (bf16_t*)a.C, (bf16_t*)a.norm_out, a.norm_g, a.eps);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, int dt, hipStream_t s) {
  if (dt == DT_BF16) return gemm_bf16(a, s);
  switch (a.epi) {
    case EPI_STORE: return gemm_f32_launch<EPI_STORE>(a, s);
    case EPI_RESID: return gemm_f32_launch<EPI_RESID>(a, s);
    case EPI_QKV: return gemm_f32_launch<EPI_QKV>(a, s);
    case EPI_SWIGLU: return gemm_f32_launch<EPI_SWIGLU>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vla

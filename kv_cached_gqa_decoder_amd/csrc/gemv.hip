// Decode projections (one token row): weight-streaming GEMV with fused input
// RMSNorm and fused epilogues (RoPE + paged KV write, residual add, SwiGLU,
// output head with argmax). HBM-bound: every weight byte is read once with
// 16-byte loads, many independent loads in flight per lane.
#include <hip/hip_fp16.h>

#include "common.hpp"
#include "epilogue.hpp"
#include "gemv_body.hpp"
#include "kernels.hpp"

namespace vla {

// One workgroup = 4 wavefronts; a wavefront owns RW whole rows at a time and
// streams them with 16-byte loads, UNR chunks per lane per step (RW * UNR
// independent loads in flight per lane). The input row sits in LDS (fp32 when
// it is the normalised residual); partial sums are reduced across the wavefront
// with xor shuffles, so
// the epilogue of a row group needs no workgroup barrier.
template <typename T, int EPI, int RW>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs a, int ngroups) {
  extern __shared__ __attribute__((aligned(16))) unsigned char gsmem[];
  T* xs = (T*)gsmem;
  __shared__ float ssq[kGemvWaves];
  __shared__ unsigned long long wbest[kGemvWaves];
  constexpr int CH = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int UNR = RW >= 8 ? 2 : (RW >= 4 ? 4 : 8);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  const int nch = K / CH;

  // input row -> LDS. Every epilogue but the residual one reads the fp32 residual
  // stream, normalises it (RMSNorm, fp32 statistics) and keeps it in fp32 (these
  // projections run on the vector ALUs, so the input need not be rounded); the
  // residual projections read activations already in the weight type.
  if constexpr (EPI != EPI_RESID) {
    f32x4_t* xs4 = (f32x4_t*)gsmem;
    const f32x4_t* xf4 = (const f32x4_t*)a.x;
    float ss = 0.f;
    for (int i = tid; i < K / 4; i += kGemvThreads) {
      const f32x4_t v = xf4[i];
      xs4[i] = v;
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += v[e] * v[e];
    }
    if (a.norm_g) {
      ss = wave_sum(ss);
      if (lane == 0) ssq[wave] = ss;
      __syncthreads();
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < kGemvWaves; ++w) tot += ssq[w];
      const float rn = rsqrtf(tot / (float)K + a.eps);
      const f32x4_t* g4 = (const f32x4_t*)a.norm_g;
      for (int i = tid; i < K / 4; i += kGemvThreads) xs4[i] = xs4[i] * rn * g4[i];  // own elements
    }
  } else {
    const T* x = (const T*)a.x;
    for (int c = tid; c < nch; c += kGemvThreads)
      *(u32x4_t*)(xs + (size_t)c * CH) = *(const u32x4_t*)(x + (size_t)c * CH);
  }
  __syncthreads();

  const T* W = (const T*)a.W;
  unsigned long long best = 0ull;
  for (int g = blockIdx.x * kGemvWaves + wave; g < ngroups; g += gridDim.x * kGemvWaves) {
    const T* wr[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {  // rows past N (a partial last group) re-read row N-1
      const int64_t row = gemv_row<EPI, RW>(g, r);
      wr[r] = W + (row < a.N ? row : (int64_t)a.N - 1) * K;
    }
    float acc[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) acc[r] = 0.f;
    for (int c0 = lane; c0 < nch; c0 += 64 * UNR) {
      u32x4_t w[UNR][RW];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int c = c0 + 64 * u;
#pragma unroll
        for (int r = 0; r < RW; ++r)
          w[u][r] = c < nch ? *(const u32x4_t*)(wr[r] + (size_t)c * CH) : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int c = c0 + 64 * u;
        float xv[CH];
        if constexpr (EPI != EPI_RESID) {
          const f32x4_t* xp = (const f32x4_t*)gsmem + (size_t)c * (CH / 4);
#pragma unroll
          for (int i = 0; i < CH / 4; ++i) {
            const f32x4_t q = c < nch ? xp[i] : f32x4_t{0.f, 0.f, 0.f, 0.f};
            xv[4 * i] = q[0];
            xv[4 * i + 1] = q[1];
            xv[4 * i + 2] = q[2];
            xv[4 * i + 3] = q[3];
          }
        } else {
          const u32x4_t xr = c < nch ? *(const u32x4_t*)(xs + (size_t)c * CH) : u32x4_t{0, 0, 0, 0};
          if constexpr (sizeof(T) == 2) unpack8(xr, xv);
          else
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[i] = __uint_as_float(xr[i]);
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          float wf[CH];
          if constexpr (sizeof(T) == 2) unpack8(w[u][r], wf);
          else
#pragma unroll
            for (int i = 0; i < 4; ++i) wf[i] = __uint_as_float(w[u][r][i]);
#pragma unroll
          for (int i = 0; i < CH; ++i) acc[r] += wf[i] * xv[i];
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) acc[r] = wave_sum(acc[r]);

    if constexpr (EPI == EPI_QKV) {
#pragma unroll
      for (int p = 0; p < RW / 2; ++p)
        if (lane == p) epi_qkv_pair<T>(a.ctx, 0, (int)gemv_row<EPI, RW>(g, 2 * p), acc[2 * p],
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
        if (lane == i) St<T>::st((T*)a.out, g * (RW / 2) + i, glu_act(a.glu, acc[i], acc[RW / 2 + i]));
    } else if constexpr (EPI == EPI_HEAD) {
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const int64_t row = gemv_row<EPI, RW>(g, r);
        if (row < a.N) {
          if (lane == r) ((float*)a.out)[row] = acc[r];
          const unsigned long long k = argmax_key(acc[r], (uint32_t)row);
          best = k > best ? k : best;
        }
      }
    }
  }
  if constexpr (EPI == EPI_HEAD) {
    if (lane == 0) wbest[wave] = best;
    __syncthreads();
    if (tid == 0) {
      unsigned long long b = wbest[0];
#pragma unroll
      for (int w = 1; w < kGemvWaves; ++w) b = wbest[w] > b ? wbest[w] : b;
      a.argmax_part[blockIdx.x] = b;
    }
  }
}

template <int EPI, int RW, int CPL, int KS, bool FOLD>
__global__ __launch_bounds__(kGemvThreads) void gemv1_kernel(GemvArgs a, int ngroups) {
  gemv1_body<EPI, RW, CPL, KS, FOLD>(a, ngroups, blockIdx.x, a.W, a.ctx.layer);
}

template <int EPI, int RW, int CPL, int KS, bool FOLD = false>
static hipError_t gemv1_go(const GemvArgs& a, hipStream_t s, int* grid_out) {
  const int ngroups = (EPI == EPI_SWIGLU) ? a.N / RW : (a.N + RW - 1) / RW;
  const int grid = KS == 1 ? (ngroups + kGemvWaves - 1) / kGemvWaves : ngroups;
  if (grid_out) *grid_out = grid;
  launch_k(gemv1_kernel<EPI, RW, CPL, KS, FOLD>, dim3(grid), dim3(kGemvThreads), 0, s, a, ngroups);
  return hipGetLastError();
}

// Shapes of the one-shot kernel: whole rows of up to 4 chunks per lane (K <= 2048)
// two rows per wavefront; residual rows up to 8 chunks per lane per wavefront of
// a K split (K <= 16384), one row per workgroup. Returns false when K fits neither.
template <int EPI>
static bool gemv1_launch(const GemvArgs& a, hipStream_t s, int* grid_out, hipError_t* err) {
  const int nch = a.K / 8;
  const int cpl = (nch + 63) / 64;
  static_assert(kGemv1MaxK == 4 * 64 * 8, "whole rows of up to 4 chunks per lane");
  if constexpr (EPI == EPI_RESID) {
    if (a.part_o) {  // the decode attention's partials, merged on the way in
      const int heads = a.hd > 0 ? a.K / a.hd : 0;
      if (cpl > 4 || a.splits < 2 || a.splits > kFoldMaxSplits || a.grp < 1 || heads < 1 ||
          heads > kFoldMaxHeads || heads * a.hd != a.K || heads % a.grp != 0) {
        *err = hipErrorInvalidValue;
        return true;
      }
      switch (cpl) {
        case 1: *err = gemv1_go<EPI, 2, 1, 1, true>(a, s, grid_out); return true;
        case 2: *err = gemv1_go<EPI, 2, 2, 1, true>(a, s, grid_out); return true;
        case 3: *err = gemv1_go<EPI, 2, 3, 1, true>(a, s, grid_out); return true;
        default: *err = gemv1_go<EPI, 2, 4, 1, true>(a, s, grid_out); return true;
      }
    }
  }
  if (cpl <= 4) {
    switch (cpl) {
      case 1: *err = gemv1_go<EPI, 2, 1, 1>(a, s, grid_out); return true;
      case 2: *err = gemv1_go<EPI, 2, 2, 1>(a, s, grid_out); return true;
      case 3: *err = gemv1_go<EPI, 2, 3, 1>(a, s, grid_out); return true;
      case 4: *err = gemv1_go<EPI, 2, 4, 1>(a, s, grid_out); return true;
    }
  }
  if constexpr (EPI == EPI_RESID) {
    const int ks = ((nch + kGemvWaves - 1) / kGemvWaves + 63) / 64;
    switch (ks) {
      case 2: *err = gemv1_go<EPI, 1, 2, kGemvWaves>(a, s, grid_out); return true;
      case 3: *err = gemv1_go<EPI, 1, 3, kGemvWaves>(a, s, grid_out); return true;
      case 4: *err = gemv1_go<EPI, 1, 4, kGemvWaves>(a, s, grid_out); return true;
      case 5: *err = gemv1_go<EPI, 1, 5, kGemvWaves>(a, s, grid_out); return true;
      case 6: *err = gemv1_go<EPI, 1, 6, kGemvWaves>(a, s, grid_out); return true;
      case 7: *err = gemv1_go<EPI, 1, 7, kGemvWaves>(a, s, grid_out); return true;
      case 8: *err = gemv1_go<EPI, 1, 8, kGemvWaves>(a, s, grid_out); return true;
    }
  }
  return false;
}

template <typename T, int EPI, int RW>
static hipError_t gemv_launch_rw(const GemvArgs& a, hipStream_t s, int* grid_out) {
  // rows of the residual and head projections may end in a partial group
  const int ngroups = (EPI == EPI_SWIGLU) ? a.N / RW : (a.N + RW - 1) / RW;
  int grid = (ngroups + kGemvWaves - 1) / kGemvWaves;
  grid = grid < kGemvMaxGrid ? grid : kGemvMaxGrid;
  if (grid_out) *grid_out = grid;
  const uint32_t lds = (uint32_t)((size_t)a.K * (EPI == EPI_RESID ? sizeof(T) : sizeof(float)));
  launch_k(gemv_kernel<T, EPI, RW>, dim3(grid), dim3(kGemvThreads), lds, s, a, ngroups);
  return hipGetLastError();
}

// rows per wavefront: 8 when that still gives >= 2048 wavefronts, else 4 when
// >= 1024, else 2 (small projections spread over more of the chip)
template <typename T, int EPI>
static hipError_t gemv_launch(const GemvArgs& a, hipStream_t s, int* grid_out) {
  if constexpr (EPI == EPI_QKV) {
    if (a.N % 8) return hipErrorInvalidValue;
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (a.N % 32) return hipErrorInvalidValue;
  }
  if constexpr (sizeof(T) == 2 && EPI != EPI_HEAD) {
    hipError_t err;
    if (gemv1_launch<EPI>(a, s, grid_out, &err)) return err;
  }
  if (a.N / 8 >= 2048) return gemv_launch_rw<T, EPI, 8>(a, s, grid_out);
  if (a.N / 4 >= 1024) return gemv_launch_rw<T, EPI, 4>(a, s, grid_out);
  return gemv_launch_rw<T, EPI, 2>(a, s, grid_out);
}

// ---------------------------------------------------------------------------
// INT4 group-128 weights: a 16-byte chunk holds the 32 codes of K positions
// 32c .. 32c+31 (even k in the low nibble), inside group c / 4 whose fp16 scale
// (scales stored [K/128][N]) multiplies the chunk's partial sum in fp32.
// Unpacking: flipping each nibble's sign bit turns a code q into u = q + 8
// (0..15); two nibbles masked into a bf16 pair with the exponent of 128 are the
// values 128 + u, and v_dot2c_f32_bf16 adds two products to an fp32 sum per
// instruction. Per 32-code chunk, sum_k q_k x_k = sum_k (128 + u_k) x_k -
// 136 sum_k x_k, the second sum shared by all rows that use the chunk's inputs.
// The input is rounded to bf16 (as the matrix-core path does) and kept as bf16
// pairs in the order the nibbles come out of a 32-bit word: for its 8 codes
// k0..k7, pairs (k0, k4), (k1, k5), (k2, k6), (k3, k7).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

// the 8 inputs x0..x7 of one word's codes, as the 4 pairs of that order
__device__ __forceinline__ void w4_pairs(const float (&x)[8], uint32_t (&pr)[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) pr[p] = pack_bf16x2(x[p], x[p + 4]);
}
// (x0, x1), (x2, x3), (x4, x5), (x6, x7) as bf16 words -> the 4 pairs of that order
__device__ __forceinline__ void w4_pairs_bf16(const u32x4_t& n, uint32_t (&pr)[4]) {
  pr[0] = __builtin_amdgcn_perm(n[2], n[0], 0x05040100u);  // (x0, x4)
  pr[1] = __builtin_amdgcn_perm(n[2], n[0], 0x07060302u);  // (x1, x5)
  pr[2] = __builtin_amdgcn_perm(n[3], n[1], 0x05040100u);  // (x2, x6)
  pr[3] = __builtin_amdgcn_perm(n[3], n[1], 0x07060302u);  // (x3, x7)
}
__device__ __forceinline__ float w4_dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, a),
                                         __builtin_bit_cast(bf16x2v_t, b), acc, false);
}
// sum over one chunk (4 words of codes) of (128 + u_k) x_k
__device__ __forceinline__ float w4_chunk(const u32x4_t& w, const uint32_t (&xp)[16]) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int p = 0; p < 4; ++p) acc = w4_dot2(w4_pair_bits(w[i] >> (4 * p)), xp[4 * i + p], acc);
  return acc;
}


// Streaming INT4 GEMV: same row groups and epilogues as the 16-bit kernel. A
// wavefront walks its (row group, block of 64 * UNR chunks per row) steps; per
// step every code and scale load of the step is issued before any is used
// (chunk indexes past the row are clamped, their scale zeroed at use, so the
// loads carry no branches). The input row is read once into registers (XG groups
// of 8 per thread), the first step's loads go out right behind it, and the row
// is then staged in LDS as bf16 pairs (normalised residual, or bf16 activations)
// while those loads are in flight. ONE: exactly one row group per wavefront and
// one step per row (the whole row in flight at once, no loop).
template <int UNR, int RW>
struct W4Step {
  u32x4_t w[UNR][RW];
  uint16_t sc[UNR][RW];  // fp16 bits
};

template <int EPI, int RW, int UNR, int NW, int XG, bool ONE>
__global__ __launch_bounds__(64 * NW) void gemv_w4_kernel(GemvArgs a, int ngroups) {
  extern __shared__ __attribute__((aligned(16))) unsigned char gsmem[];
  uint32_t* xsh = (uint32_t*)gsmem;  // K/2 words: the input as bf16 pairs
  __shared__ float ssq[NW];
  __shared__ unsigned long long wbest[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, nch = K / 32, ng8 = K / 8;
  constexpr int PER = 64 * UNR;  // chunks per row per step
  const int nit = ONE ? 1 : (nch + PER - 1) / PER;
  const int stride = gridDim.x * NW;
  const uint8_t* W = (const uint8_t*)a.W;
  const uint16_t* Sc16 = (const uint16_t*)(W + (size_t)a.N * K / 2);

  // ---- the input row, one load round trip ----
  f32x4_t xr[XG][2], gr[XG][2];
  u32x4_t xb[XG];
#pragma unroll
  for (int k = 0; k < XG; ++k) {
    int gi = tid + k * 64 * NW;
    gi = gi < ng8 ? gi : ng8 - 1;
    if constexpr (EPI != EPI_RESID) {
      const f32x4_t* xf4 = (const f32x4_t*)a.x;
      xr[k][0] = xf4[2 * gi];
      xr[k][1] = xf4[2 * gi + 1];
      if (a.norm_g) {
        const f32x4_t* g4 = (const f32x4_t*)a.norm_g;
        gr[k][0] = g4[2 * gi];
        gr[k][1] = g4[2 * gi + 1];
      }
    } else {
      xb[k] = *(const u32x4_t*)((const bf16_t*)a.x + (size_t)gi * 8);
    }
  }

  // ---- load cursor: (group lg, chunk block lit) ----
  int lg = blockIdx.x * NW + wave, lit = 0;
  W4Step<UNR, RW> st;
  auto load = [&]() {
    const int gg = __builtin_amdgcn_readfirstlane(lg < ngroups ? lg : ngroups - 1);
    const uint8_t* wrow[RW];
    const uint16_t* srow[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {  // rows past N (a partial last group) re-read row N-1
      const int64_t row0 = gemv_row<EPI, RW>(gg, r);
      const int64_t row = row0 < a.N ? row0 : (int64_t)a.N - 1;
      wrow[r] = W + row * (K / 2);
      srow[r] = Sc16 + row;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      int c = lane + lit * PER + 64 * u;
      c = c < nch ? c : nch - 1;
      const uint32_t wo = (uint32_t)c * 16u, so = (uint32_t)(c / 4) * (uint32_t)a.N;
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        st.w[u][r] = *(const u32x4_t*)(wrow[r] + wo);
        st.sc[u][r] = srow[r][so];
      }
    }
    if (++lit == nit) {
      lit = 0;
      lg += stride;
    }
  };
  load();

  // ---- input -> LDS as bf16 pairs ----
  if constexpr (EPI != EPI_RESID) {
    float rn = 1.f;
    if (a.norm_g) {
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < XG; ++k)
        if (tid + k * 64 * NW < ng8)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += xr[k][h][e] * xr[k][h][e];
      ss = wave_sum(ss);
      if (lane == 0) ssq[wave] = ss;
      __syncthreads();
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += ssq[w];
      rn = rsqrtf(tot / (float)K + a.eps);
    }
#pragma unroll
    for (int k = 0; k < XG; ++k) {
      const int gi = tid + k * 64 * NW;
      if (gi < ng8) {
        f32x4_t v0 = xr[k][0], v1 = xr[k][1];
        if (a.norm_g) {
          v0 = v0 * rn * gr[k][0];
          v1 = v1 * rn * gr[k][1];
        }
        const float xv8[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        uint32_t pr[4];
        w4_pairs(xv8, pr);
        *(u32x4_t*)(xsh + 4 * gi) = u32x4_t{pr[0], pr[1], pr[2], pr[3]};
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < XG; ++k) {
      const int gi = tid + k * 64 * NW;
      if (gi < ng8) {
        uint32_t pr[4];
        w4_pairs_bf16(xb[k], pr);
        *(u32x4_t*)(xsh + 4 * gi) = u32x4_t{pr[0], pr[1], pr[2], pr[3]};
      }
    }
  }
  __syncthreads();

  // ---- compute cursor: same walk as the loads ----
  int cg = blockIdx.x * NW + wave, cit = 0;
  float acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) acc[r] = 0.f;
  unsigned long long best = 0ull;
  while (cg < ngroups) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int c0 = lane + cit * PER + 64 * u;
      const int c = c0 < nch ? c0 : nch - 1;
      uint32_t xp[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4_t v = *(const u32x4_t*)(xsh + 16 * c + 4 * i);
#pragma unroll
        for (int p = 0; p < 4; ++p) xp[4 * i + p] = v[p];
      }
      float sx = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) sx = w4_dot2(xp[j], 0x3f803f80u, sx);  // (1, 1)
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const float scv = c0 < nch ? __half2float(__builtin_bit_cast(__half, st.sc[u][r])) : 0.f;
        acc[r] += scv * (w4_chunk(st.w[u][r], xp) - 136.f * sx);
      }
    }
    const int g = cg;
    const bool last = ++cit == nit;
    if (last) {
      cit = 0;
      cg += stride;
    }
    if constexpr (!ONE) {
      if (cg < ngroups) load();
      if (!last) continue;
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) acc[r] = wave_sum(acc[r]);

    if constexpr (EPI == EPI_QKV) {
#pragma unroll
      for (int p = 0; p < RW / 2; ++p)
        if (lane == p) epi_qkv_pair<bf16_t>(a.ctx, 0, (int)gemv_row<EPI, RW>(g, 2 * p), acc[2 * p],
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
    } else if constexpr (EPI == EPI_HEAD) {
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const int64_t row = gemv_row<EPI, RW>(g, r);
        if (row < a.N) {
          if (lane == r) ((float*)a.out)[row] = acc[r];
          const unsigned long long k = argmax_key(acc[r], (uint32_t)row);
          best = k > best ? k : best;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) acc[r] = 0.f;
    if constexpr (ONE) break;
  }
  if constexpr (EPI == EPI_HEAD) {
    if (lane == 0) wbest[wave] = best;
    __syncthreads();
    if (tid == 0) {
      unsigned long long b = wbest[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) b = wbest[w] > b ? wbest[w] : b;
      a.argmax_part[blockIdx.x] = b;
    }
  }
}

template <int EPI, int RW, int UNR, bool ONE, int XG>
static hipError_t gemv_w4_go(const GemvArgs& a, int ngroups, int grid, hipStream_t s) {
  launch_k(gemv_w4_kernel<EPI, RW, UNR, kGemvWaves, XG, ONE>, dim3(grid), dim3(kGemvThreads),
           (uint32_t)(a.K * 2), s, a, ngroups);
  return hipGetLastError();
}

// RW rows per wavefront, 64 * UNR chunks per row per step; ONE: one row group per
// wavefront and the whole row in one step (needs K <= 2048 * UNR), else a grid of
// at most kGemvMaxGrid workgroups striding over the groups
template <int EPI, int RW, int UNR, bool ONE>
static hipError_t gemv_w4_launch_rw(const GemvArgs& a, hipStream_t s, int* grid_out) {
  static_assert(!(ONE && EPI == EPI_HEAD), "the output head's argmax partials need a bounded grid");
  const int ngroups = (EPI == EPI_SWIGLU) ? a.N / RW : (a.N + RW - 1) / RW;
  if (ngroups <= 0) return hipErrorInvalidValue;
  if (ONE && a.K / 32 > 64 * UNR) return hipErrorInvalidValue;
  int grid = (ngroups + kGemvWaves - 1) / kGemvWaves;
  if (!ONE) grid = grid < kGemvMaxGrid ? grid : kGemvMaxGrid;
  if (grid_out) *grid_out = grid;
  // input groups of 8 per thread: K / 8 <= XG * kGemvThreads (K <= 16384 checked by the caller)
  const int xg = (a.K / 8 + kGemvThreads - 1) / kGemvThreads;
  if (xg <= 1) return gemv_w4_go<EPI, RW, UNR, ONE, 1>(a, ngroups, grid, s);
  if (xg <= 2) return gemv_w4_go<EPI, RW, UNR, ONE, 2>(a, ngroups, grid, s);
  if (xg <= 4) return gemv_w4_go<EPI, RW, UNR, ONE, 4>(a, ngroups, grid, s);
  if (xg <= 8) return gemv_w4_go<EPI, RW, UNR, ONE, 8>(a, ngroups, grid, s);
  return hipErrorInvalidValue;
}

template <int EPI>
static hipError_t gemv_w4_launch(const GemvArgs& a, hipStream_t s, int* grid_out) {
  if (a.K % 128 != 0 || a.K > 16384) return hipErrorInvalidValue;
  if constexpr (EPI == EPI_QKV) {
    if (a.N % 8) return hipErrorInvalidValue;
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (a.N % 32) return hipErrorInvalidValue;
  }
  // q/k/v (epilogue: RoPE'd keys and values into the paged cache) and residual rows
  // up to 4096: one row group of 2 rows per wavefront with the whole row in flight
  // (Llama-3-8B shape, in the decode step: q/k/v 9.7 -> 7.1 us and O 6.7 -> 5.5 us
  // against a one-shot kernel whose 2-row wavefronts each took a whole workgroup's
  // input staging)
  if constexpr (EPI == EPI_QKV || EPI == EPI_RESID) {
    if (a.K <= 2048) return gemv_w4_launch_rw<EPI, 2, 1, true>(a, s, grid_out);
    if (a.K <= 4096) return gemv_w4_launch_rw<EPI, 2, 2, true>(a, s, grid_out);
  }
  if constexpr (EPI == EPI_QKV) {
    if (a.K <= 8192) return gemv_w4_launch_rw<EPI, 2, 4, true>(a, s, grid_out);
  }
  // streaming kernel, measured at the Llama-3-8B shape in the decode step: down
  // projection (14336 -> 4096, 2 rows per wavefront, 64 chunks per row per step)
  // 10.8 us; gated projection (4096 -> 2 x 14336, one row group of 4 rows per
  // wavefront, whole rows in flight) 15.9 us; output head (4096 -> 128256, 8 rows) 53 us
  if constexpr (EPI == EPI_RESID) return gemv_w4_launch_rw<EPI, 2, 1, false>(a, s, grid_out);
  if constexpr (EPI == EPI_SWIGLU) {
    if (a.K <= 2048) return gemv_w4_launch_rw<EPI, 4, 1, true>(a, s, grid_out);
    if (a.K <= 4096) return gemv_w4_launch_rw<EPI, 4, 2, true>(a, s, grid_out);
    return gemv_w4_launch_rw<EPI, 8, 1, false>(a, s, grid_out);
  }
  if (a.N / 8 >= 2048) return gemv_w4_launch_rw<EPI, 8, 1, false>(a, s, grid_out);
  if (a.N / 4 >= 1024) return gemv_w4_launch_rw<EPI, 4, 1, false>(a, s, grid_out);
  return gemv_w4_launch_rw<EPI, 2, 1, false>(a, s, grid_out);
}

static hipError_t gemv_w4_dispatch(const GemvArgs& a, hipStream_t s, int* grid_out) {
  switch (a.epi) {
    case EPI_QKV: return gemv_w4_launch<EPI_QKV>(a, s, grid_out);
    case EPI_RESID: return gemv_w4_launch<EPI_RESID>(a, s, grid_out);
    case EPI_SWIGLU: return gemv_w4_launch<EPI_SWIGLU>(a, s, grid_out);
    case EPI_HEAD: return gemv_w4_launch<EPI_HEAD>(a, s, grid_out);
    default: return hipErrorInvalidValue;
  }
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
  if (a.wf == WF_INT4) return dt == DT_BF16 ? gemv_w4_dispatch(a, s, grid_out) : hipErrorInvalidValue;
  // the input row lives in LDS: fp32 (residual inputs) or 16-bit, at most 64 KiB
  if (a.K % 8 != 0 || a.K > (a.epi == EPI_RESID ? 32768 : 16384)) return hipErrorInvalidValue;
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

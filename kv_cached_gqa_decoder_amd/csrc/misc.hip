// Weight generation, embedding gather, RMSNorm, raw KV scatter / gather.
#include <hip/hip_fp16.h>

#include "common.hpp"
#include "kernels.hpp"
#include "rope_body.hpp"

namespace vla {

static int grid_for(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

// ---------------------------------------------------------------------------
// Seeded generator ("Can an LLM Forget the Right Things?", section 6: weights
// from splitmix64 feeding Box-Muller). splitmix64 is the generator of Steele,
// Lea and Flood (2014); counter based here: element i of stream s under seed k
// draws the two outputs at key + 2i and key + 2i + 1 with key = sm(k ^ sm(s)).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t sm64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  uint64_t z = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ double u53(uint64_t x) { return (double)(x >> 11) * 0x1.0p-53; }

__device__ __forceinline__ double normal_at(uint64_t key, uint64_t i) {
  const double u1 = u53(sm64(key + 2 * i));
  const double u2 = u53(sm64(key + 2 * i + 1));
  return sqrt(-2.0 * log(1.0 - u1)) * cos(6.283185307179586 * u2);
}

// nearest-even rounding of a double to 8 significant bits (bfloat16), normal range
__device__ __forceinline__ double round_bf16_d(double v) {
  int e;
  const double m = frexp(v, &e);
  return ldexp(rint(m * 256.0) / 256.0, e);
}

// physical row -> (stream selector 0/1/2, logical row) for the three layouts
__device__ __forceinline__ void phys_to_logical(int layout, int64_t r, int hq, int hkv, int d,
                                                int* which, int64_t* lr) {
  if (layout == LAYOUT_QKV) {
    const int64_t head = r / d;
    const int w = (int)(r % d);
    const int j = (w >> 1) + (w & 1) * (d / 2);
    if (head < hq) { *which = 0; *lr = head * d + j; }
    else if (head < hq + hkv) { *which = 1; *lr = (head - hq) * d + j; }
    else { *which = 2; *lr = (head - hq - hkv) * d + j; }
  } else if (layout == LAYOUT_GATEUP) {
    const int64_t b = r / 32;
    const int w = (int)(r % 32);
    *which = w < 16 ? 0 : 1;
    *lr = b * 16 + (w & 15);
  } else {
    *which = 0;
    *lr = r;
  }
}

template <typename T>
__global__ void init_weight_kernel(T* out, int layout, int64_t rows, int64_t cols, uint64_t seed,
                                   uint64_t sa, uint64_t sb, uint64_t sc, int hq, int hkv, int d,
                                   double stdv) {
  const uint64_t keys[3] = {sm64(seed ^ sm64(sa)), sm64(seed ^ sm64(sb)), sm64(seed ^ sm64(sc))};
  const int64_t total = rows * cols;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = p / cols, c = p % cols;
    int which;
    int64_t lr;
    phys_to_logical(layout, r, hq, hkv, d, &which, &lr);
    const double v = stdv * normal_at(keys[which], (uint64_t)(lr * cols + c));
    if constexpr (sizeof(T) == 4) {
      out[p] = (float)v;
    } else {
      out[p] = (bf16_t)(__float_as_uint((float)round_bf16_d(v)) >> 16);
    }
  }
}

// Group-128 INT4 weights ("Rebuilding Kshipra Around Memory", section 2: 4-bit
// codes in groups of 128 along a row, two per byte, one fp16 scale per group,
// and the same fp16 scale used to encode and to decode so |w - q s| <= s / 2).
// One thread per (physical row, group): the 128 master values are drawn like
// the other weights and rounded to fp32; s = fp16(max|w| / 7) with the division
// in fp32; q = clamp(round-half-even(w / s), -8, 7) with the division in fp32 by
// s widened to fp32 (q = 0 when s = 0); even k in the low nibble.
// Storage of an N x K tensor: packed bytes [N][K/2], then scales [K/128][N]
// (group-major: the scales of one group for consecutive rows are contiguous).
__global__ void init_weight_w4_kernel(uint8_t* out, int layout, int64_t rows, int64_t cols,
                                      uint64_t seed, uint64_t sa, uint64_t sb, uint64_t sc,
                                      int hq, int hkv, int d, double stdv) {
  const uint64_t keys[3] = {sm64(seed ^ sm64(sa)), sm64(seed ^ sm64(sb)), sm64(seed ^ sm64(sc))};
  const int64_t groups = cols / 128;
  const int64_t total = rows * groups;
  __half* scales = (__half*)(out + rows * cols / 2);
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = p / groups, g = p % groups;
    int which;
    int64_t lr;
    phys_to_logical(layout, r, hq, hkv, d, &which, &lr);
    // pass 1: the group's max |w|; pass 2: regenerate and encode (no 128-value array)
    const uint64_t base = (uint64_t)(lr * cols + g * 128);
    float amax = 0.f;
    for (int k = 0; k < 128; ++k)
      amax = fmaxf(amax, fabsf((float)(stdv * normal_at(keys[which], base + k))));
    const __half s16 = __float2half_rn(__fdiv_rn(amax, 7.0f));
    const float s32 = __half2float(s16);
    scales[g * rows + r] = s16;
    uint8_t* o = out + r * (cols / 2) + g * 64;
    for (int k = 0; k < 128; k += 2) {
      int q[2] = {0, 0};
      if (s32 != 0.f) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float w = (float)(stdv * normal_at(keys[which], base + k + h));
          q[h] = (int)fminf(fmaxf(rintf(__fdiv_rn(w, s32)), -8.f), 7.f);
        }
      }
      o[k / 2] = (uint8_t)((q[0] & 0xF) | ((q[1] & 0xF) << 4));
    }
  }
}

hipError_t launch_init_weight_w4(void* out, int layout, int64_t rows, int64_t cols, uint64_t seed,
                                 uint64_t sa, uint64_t sb, uint64_t sc, int hq, int hkv, int d,
                                 double stdv, hipStream_t s) {
  if (cols % 128) return hipErrorInvalidValue;
  init_weight_w4_kernel<<<grid_for(rows * (cols / 128), 64), 64, 0, s>>>(
      (uint8_t*)out, layout, rows, cols, seed, sa, sb, sc, hq, hkv, d, stdv);
  return hipGetLastError();
}

// logical (out, in) element (lr, c) of sub-tensor `which` -> physical row
__device__ __forceinline__ int64_t logical_to_phys(int layout, int which, int64_t lr, int hq,
                                                   int hkv, int d) {
  if (layout == LAYOUT_QKV) {
    const int64_t head = lr / d + (which == 0 ? 0 : which == 1 ? hq : hq + hkv);
    const int j = (int)(lr % d);
    const int w = j < d / 2 ? 2 * j : 2 * (j - d / 2) + 1;
    return head * d + w;
  }
  if (layout == LAYOUT_GATEUP) return (lr / 16) * 32 + (lr % 16) + (which ? 16 : 0);
  return lr;
}

template <typename T>
__global__ void weight_logical_kernel(const T* phys, T* out, int layout, int which, int64_t rows,
                                      int64_t cols, int hq, int hkv, int d) {
  const int64_t total = rows * cols;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lr = p / cols, c = p % cols;
    out[p] = phys[logical_to_phys(layout, which, lr, hq, hkv, d) * cols + c];
  }
}


// INT4 tensor element (lr, c) of sub-tensor `which`, dequantised: q * s (exact in fp32)
__global__ void weight_logical_w4_kernel(const uint8_t* phys, float* out, int layout, int which,
                                         int64_t rows, int64_t cols, int64_t prows, int hq,
                                         int hkv, int d) {
  const int64_t total = rows * cols;
  const __half* scales = (const __half*)(phys + prows * cols / 2);
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lr = p / cols, c = p % cols;
    const int64_t r = logical_to_phys(layout, which, lr, hq, hkv, d);
    const uint8_t b = phys[r * (cols / 2) + c / 2];
    const int q = (int)((int8_t)((c & 1) ? (b & 0xF0) : (uint8_t)(b << 4)) >> 4);
    out[p] = (float)q * __half2float(scales[(c / 128) * prows + r]);
  }
}
hipError_t launch_weight_logical_w4(const void* phys, float* out, int layout, int which,
                                    int64_t rows, int64_t cols, int64_t prows, int hq, int hkv,
                                    int d, hipStream_t s) {
  weight_logical_w4_kernel<<<grid_for(rows * cols, 256), 256, 0, s>>>(
      (const uint8_t*)phys, out, layout, which, rows, cols, prows, hq, hkv, d);
  return hipGetLastError();
}

hipError_t launch_weight_logical(const void* phys, void* out, int dt, int layout, int which,
                                 int64_t rows, int64_t cols, int hq, int hkv, int d,
                                 hipStream_t s) {
  const int g = grid_for(rows * cols, 256);
  if (dt == DT_F32)
    weight_logical_kernel<float><<<g, 256, 0, s>>>((const float*)phys, (float*)out, layout, which,
                                                    rows, cols, hq, hkv, d);
  else
    weight_logical_kernel<bf16_t><<<g, 256, 0, s>>>((const bf16_t*)phys, (bf16_t*)out, layout,
                                                     which, rows, cols, hq, hkv, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(int64_t pos0, int n, const double* inv_freq, int half,
                                  float2* tab) {
  const int64_t total = (int64_t)n * half;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (int64_t)gridDim.x * blockDim.x)
    rope_entry(p, pos0, inv_freq, half, tab);
}
hipError_t launch_rope_table(int64_t pos0, int n, const double* inv_freq, int half, float2* tab,
                             hipStream_t s) {
  rope_table_kernel<<<grid_for((int64_t)n * half, 256), 256, 0, s>>>(pos0, n, inv_freq, half, tab);
  return hipGetLastError();
}

__global__ void fill_f32_kernel(float* p, float v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}
hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t s) {
  fill_f32_kernel<<<grid_for(n, 256), 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Matrix-core throughput probe: every wavefront runs `iters` rounds of 8
// independent v_mfma_f32_16x16x32_bf16 chains on register operands (no memory
// traffic in the loop); one value per workgroup is stored so the work is kept.
// 16384 FLOP per instruction.
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* out, int iters) {
  // four chains of v_mfma_f32_32x32x16_bf16 (32768 flops each) with distinct B operands
  // and start values, so none can be merged; the 16 x 16 x 32 form issues at about
  // half this rate on gfx950
  bf16x8_t a, b[4];
  f32x16_t acc[4];
  for (int i = 0; i < 8; ++i) a[i] = (__bf16)(0.001f * (float)((threadIdx.x + i) & 7));
  for (int j = 0; j < 4; ++j) {
    for (int i = 0; i < 8; ++i) b[j][i] = (__bf16)(0.002f * (float)((threadIdx.x * 3 + i + j) & 7));
    for (int e = 0; e < 16; ++e) acc[j][e] = (float)(j + e);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[j], acc[j], 0, 0, 0);
  }
  float t = 0.f;
  for (int j = 0; j < 4; ++j)
    for (int e = 0; e < 16; ++e) t += acc[j][e];
  if (threadIdx.x == 0) out[blockIdx.x] = t;
}
// HBM read probe: 16-byte loads over n16 chunks. Per iteration a workgroup reads U
// consecutive 4 KB pieces (256 threads x 16 bytes; chunks past the end re-read the
// last one), then moves on by the whole grid's span, so each wavefront load is one
// contiguous 1 KB and the pieces in flight lie close together (loads spread 8 MB
// apart per thread measured 4.8 TB/s against 6.3-6.5 here). The loads are folded into
// one xor per thread that is stored, so that none can be dropped.
template <int U>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4_t* p, int64_t n16,
                                                         uint32_t* out) {
  const int64_t step = (int64_t)gridDim.x * 256 * U;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * 256 * U + threadIdx.x; i < n16; i += step) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + u * 256;
      v[u] = p[j < n16 ? j : n16 - 1];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}
hipError_t launch_read_probe(const void* p, int64_t bytes, uint32_t* out, int blocks, int unroll,
                             hipStream_t s) {
  if (bytes < 16 || bytes % 16 || blocks < 1) return hipErrorInvalidValue;
  const u32x4_t* q = (const u32x4_t*)p;
  switch (unroll) {
    case 1: read_probe_kernel<1><<<blocks, 256, 0, s>>>(q, bytes / 16, out); break;
    case 2: read_probe_kernel<2><<<blocks, 256, 0, s>>>(q, bytes / 16, out); break;
    case 4: read_probe_kernel<4><<<blocks, 256, 0, s>>>(q, bytes / 16, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mfma_peak(float* out, int blocks, int iters, hipStream_t s) {
  mfma_peak_kernel<<<blocks, 256, 0, s>>>(out, iters);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// embedding rows (activation type) -> fp32 residual rows; block 0 also clears
// the argmax cell of this pass
template <typename T>
__global__ void embed_kernel(const int* tokens, int token_scalar, const unsigned long long* token_key,
                             int n, const T* E, float* x, int H, unsigned long long* reset_cell) {
  if (reset_cell && blockIdx.x == 0 && threadIdx.x == 0) *reset_cell = 0ull;
  for (int t = blockIdx.x; t < n; t += gridDim.x) {
    // token_key: an argmax key of the output head (the token id is stored as its
    // complement in the low 32 bits, so that ties go to the lowest id)
    const int64_t id = tokens      ? tokens[t]
                       : token_key ? (int64_t)(0xffffffffu - (uint32_t)(*token_key & 0xffffffffull))
                                   : token_scalar;
    for (int i = threadIdx.x; i < H; i += blockDim.x)
      x[(int64_t)t * H + i] = St<T>::ld(E, id * H + i);
  }
}
// one decode row: block 0 gathers the token's embedding row, block 1 writes the
// row's RoPE table (one launch instead of two at the start of a decode step)
template <typename T>
__global__ void embed_rope1_kernel(int token_scalar, const unsigned long long* token_key,
                                   const T* E, float* x, int H, int64_t pos, const double* inv_freq,
                                   int half, float2* tab) {
  embed_rope1_body<T>(token_scalar, token_key, E, x, H, pos, inv_freq, half, tab, blockIdx.x);
}
hipError_t launch_embed_rope1(int token_scalar, const unsigned long long* token_key, const void* E,
                              void* x, int H, int dt, int64_t pos, const double* inv_freq, int half,
                              float2* tab, hipStream_t s) {
  if (dt == DT_F32)
    embed_rope1_kernel<float><<<2, 256, 0, s>>>(token_scalar, token_key, (const float*)E, (float*)x,
                                                H, pos, inv_freq, half, tab);
  else
    embed_rope1_kernel<bf16_t><<<2, 256, 0, s>>>(token_scalar, token_key, (const bf16_t*)E,
                                                 (float*)x, H, pos, inv_freq, half, tab);
  return hipGetLastError();
}
hipError_t launch_embed(const int* tokens, int token_scalar, const unsigned long long* token_key,
                        int n, const void* E, void* x, int H, int dt,
                        unsigned long long* reset_cell, hipStream_t s) {
  const int g = n < 1024 ? n : 1024;
  if (dt == DT_F32)
    embed_kernel<float><<<g, 256, 0, s>>>(tokens, token_scalar, token_key, n, (const float*)E,
                                          (float*)x, H, reset_cell);
  else
    embed_kernel<bf16_t><<<g, 256, 0, s>>>(tokens, token_scalar, token_key, n, (const bf16_t*)E,
                                           (float*)x, H, reset_cell);
  return hipGetLastError();
}

template <typename T>
__global__ void to_f32_kernel(const T* in, float* out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = St<T>::ld(in, i);
}
hipError_t launch_to_f32(const void* in, float* out, int64_t n, int dt, hipStream_t s) {
  const int g = grid_for(n, 256);
  if (dt == DT_F32) to_f32_kernel<float><<<g, 256, 0, s>>>((const float*)in, out, n);
  else to_f32_kernel<bf16_t><<<g, 256, 0, s>>>((const bf16_t*)in, out, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm of fp32 residual rows into the activation type, one wavefront per
// row, fp32 statistics: u = x * (mean(x^2) + eps)^-1/2 * g. H is a multiple of 64.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* x, const float* g, T* u,
                                                      T* u_lo, int rows, int H, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* xr = x + (int64_t)row * H;
  T* ur = u + (int64_t)row * H;
  float ss = 0.f;
  for (int c = lane; c < H / 4; c += 64) {
    const f32x4_t v = *(const f32x4_t*)(xr + c * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) ss += v[i] * v[i];
  }
  ss = wave_sum(ss);
  const float r = rsqrtf(ss / (float)H + eps);
  for (int c = lane; c < H / 4; c += 64) {
    const f32x4_t v = *(const f32x4_t*)(xr + c * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y = v[i] * r * g[c * 4 + i];
      St<T>::st(ur, (size_t)c * 4 + i, y);
      if constexpr (sizeof(T) == 2) {
        // low part: the rounding error of the stored value, itself rounded to bf16
        if (u_lo) u_lo[(int64_t)row * H + c * 4 + i] = f32_to_bf16(y - bf16_to_f32(f32_to_bf16(y)));
      }
    }
  }
}
hipError_t launch_rmsnorm(const void* x, const float* g, void* u, void* u_lo, int rows, int H,
                          float eps, int dt, hipStream_t s) {
  const int grid = (rows + 3) / 4;
  if (dt == DT_F32)
    launch_k(rmsnorm_kernel<float>, dim3(grid), dim3(256), 0, s, (const float*)x, g, (float*)u,
             (float*)nullptr, rows, H, eps);
  else
    launch_k(rmsnorm_kernel<bf16_t>, dim3(grid), dim3(256), 0, s, (const float*)x, g, (bf16_t*)u,
             (bf16_t*)u_lo, rows, H, eps);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// action expert ("Running VLAs at Real-time Speed", section 2: flow matching on
// the action chunk). Time embedding of tau_k = k * dt, width H: sin(tau w_j) for
// j < H/2, cos(tau w_{j-H/2}) after, w_j = 2 pi / p_j, p_j = 0.004 * 1000^(j / (H/2 - 1)),
// evaluated in fp64 and stored in fp32, one row per iteration k < n_steps.
__global__ void flow_temb_kernel(float* temb, int n_steps, int H, double dt) {
  const int half = H / 2;
  const int64_t total = (int64_t)n_steps * H;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (int64_t)gridDim.x * blockDim.x) {
    const int k = (int)(p / H), j = (int)(p % H);
    const int jj = j < half ? j : j - half;
    const double period = 0.004 * pow(1000.0, (double)jj / (double)(half - 1));
    const double ang = ((double)k * dt) * (6.283185307179586 / period);
    temb[p] = (float)(j < half ? sin(ang) : cos(ang));
  }
}
hipError_t launch_flow_temb(float* temb, int n_steps, int H, double dt, hipStream_t s) {
  if (H < 4 || H % 2 || n_steps < 1) return hipErrorInvalidValue;
  launch_k(flow_temb_kernel, dim3(grid_for((int64_t)n_steps * H, 256)), dim3(256), 0, s, temb,
           n_steps, H, dt);
  return hipGetLastError();
}

// The boundary between two flow-matching iterations, one wavefront per action row
// with the whole row in registers (NC chunks of 4 per lane):
//   euler: x += dt * RMSNorm(h) (the velocity: the expert's final norm, no output
//          projection), fp32;
//   temb:  h = x + temb (the next iteration's input), then u = RMSNorm(h) in the
//          activation type (bf16: with its low part), the first layer's input.
template <typename T, int NC>
__global__ __launch_bounds__(256) void flow_step_kernel(float* xa, float* h, const float* temb,
                                                        const float* g, T* u, T* u_lo, int rows,
                                                        int H, float eps, float dt, int euler) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nq = H / 4;
  float* xr = xa + (int64_t)row * H;
  float* hr = h + (int64_t)row * H;
  f32x4_t xv[NC], hv[NC], gv[NC];
  // every load of the row first
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + 64 * i;
    if (c < nq) {
      xv[i] = *(const f32x4_t*)(xr + 4 * c);
      gv[i] = *(const f32x4_t*)(g + 4 * c);
      hv[i] = euler ? *(const f32x4_t*)(hr + 4 * c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
  if (euler) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i)
      if (lane + 64 * i < nq)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += hv[i][e] * hv[i][e];
    ss = wave_sum(ss);
    const float r = rsqrtf(ss / (float)H + eps);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) xv[i][e] += dt * (hv[i][e] * r * gv[i][e]);
        *(f32x4_t*)(xr + 4 * c) = xv[i];
      }
    }
  }
  if (temb) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nq) {
        const f32x4_t t = *(const f32x4_t*)(temb + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hv[i][e] = xv[i][e] + t[e];
          ss += hv[i][e] * hv[i][e];
        }
        *(f32x4_t*)(hr + 4 * c) = hv[i];
      }
    }
    ss = wave_sum(ss);
    const float r = rsqrtf(ss / (float)H + eps);
    T* ur = u + (int64_t)row * H;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < nq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y = hv[i][e] * r * gv[i][e];
          St<T>::st(ur, (size_t)c * 4 + e, y);
          if constexpr (sizeof(T) == 2) {
            if (u_lo)
              u_lo[(int64_t)row * H + c * 4 + e] = f32_to_bf16(y - bf16_to_f32(f32_to_bf16(y)));
          }
        }
      }
    }
  }
}
template <typename T>
static void flow_step_go(float* xa, float* h, const float* temb, const float* g, void* u,
                         void* u_lo, int rows, int H, float eps, float dt, int euler, hipStream_t s) {
  const dim3 grid((rows + 3) / 4), block(256);
  if (H <= 1024)
    launch_k(flow_step_kernel<T, 4>, grid, block, 0, s, xa, h, temb, g, (T*)u, (T*)u_lo, rows, H,
             eps, dt, euler);
  else
    launch_k(flow_step_kernel<T, 16>, grid, block, 0, s, xa, h, temb, g, (T*)u, (T*)u_lo, rows, H,
             eps, dt, euler);
}
hipError_t launch_flow_step(float* xa, float* h, const float* temb, const float* g, void* u,
                            void* u_lo, int rows, int H, float eps, float dt, bool euler, int dtype,
                            hipStream_t s) {
  if (H % 4 || H > 4096 || rows < 1 || (!euler && !temb)) return hipErrorInvalidValue;
  if (dtype == DT_F32)
    flow_step_go<float>(xa, h, temb, g, u, nullptr, rows, H, eps, dt, euler ? 1 : 0, s);
  else
    flow_step_go<bf16_t>(xa, h, temb, g, u, u_lo, rows, H, eps, dt, euler ? 1 : 0, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// raw frame append: k, v [L][n][Hkv][d] -> the paged pool at the frame's blocks
template <typename T>
__global__ void kv_scatter_kernel(const T* k, const T* v, int n, T* kp, T* vp, KvGeom g,
                                  const int* blk_table, int cb0) {
  const int64_t total = (int64_t)g.L * n * g.hkv * g.d;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(p % g.d);
    int64_t r = p / g.d;
    const int h = (int)(r % g.hkv);
    r /= g.hkv;
    const int t = (int)(r % n);
    const int l = (int)(r / n);
    const int b = blk_table[cb0 + t / g.bt];
    const int sl = t % g.bt;
    kp[g.kidx(l, b, h, sl, i)] = k[p];
    vp[g.vidx(l, b, h, sl, i)] = v[p];
  }
}
hipError_t launch_kv_scatter(const void* k, const void* v, int n, void* kpool, void* vpool,
                             KvGeom g, const int* blk_table, int cb0, int dt, hipStream_t s) {
  const int grid = grid_for((int64_t)g.L * n * g.hkv * g.d, 256);
  if (dt == DT_F32)
    kv_scatter_kernel<float><<<grid, 256, 0, s>>>((const float*)k, (const float*)v, n,
                                                  (float*)kpool, (float*)vpool, g, blk_table, cb0);
  else
    kv_scatter_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)k, (const bf16_t*)v, n,
                                                   (bf16_t*)kpool, (bf16_t*)vpool, g, blk_table,
                                                   cb0);
  return hipGetLastError();
}

// resident K/V of one layer in logical order -> [tokens][Hkv][d]
template <typename T>
__global__ void kv_gather_kernel(const T* kp, const T* vp, KvGeom g, int layer,
                                 const int* blk_table, const int* blk_ntok, const int* tok_base,
                                 T* ko, T* vo) {
  const int lb = blockIdx.x;
  const int b = blk_table[lb];
  const int nt = blk_ntok[lb];
  const int base = tok_base[lb];
  const int per = g.hkv * g.d;
  for (int e = threadIdx.x; e < nt * per; e += blockDim.x) {
    const int sl = e / per;
    const int h = (e % per) / g.d;
    const int i = e % g.d;
    const int64_t o = (int64_t)(base + sl) * per + h * g.d + i;
    ko[o] = kp[g.kidx(layer, b, h, sl, i)];
    vo[o] = vp[g.vidx(layer, b, h, sl, i)];
  }
}
hipError_t launch_kv_gather(const void* kpool, const void* vpool, KvGeom g, int layer,
                            const int* blk_table, const int* blk_ntok, const int* tok_base,
                            int nlb, void* k_out, void* v_out, int dt, hipStream_t s) {
  if (nlb <= 0) return hipSuccess;
  if (dt == DT_F32)
    kv_gather_kernel<float><<<nlb, 256, 0, s>>>((const float*)kpool, (const float*)vpool, g, layer,
                                                blk_table, blk_ntok, tok_base, (float*)k_out,
                                                (float*)v_out);
  else
    kv_gather_kernel<bf16_t><<<nlb, 256, 0, s>>>((const bf16_t*)kpool, (const bf16_t*)vpool, g,
                                                 layer, blk_table, blk_ntok, tok_base,
                                                 (bf16_t*)k_out, (bf16_t*)v_out);
  return hipGetLastError();
}

hipError_t launch_init_weight(void* out, int dt, int layout, int64_t rows, int64_t cols,
                              uint64_t seed, uint64_t sa, uint64_t sb, uint64_t sc, int hq,
                              int hkv, int d, double stdv, hipStream_t s) {
  const int g = grid_for(rows * cols, 256);
  if (dt == DT_F32)
    init_weight_kernel<float><<<g, 256, 0, s>>>((float*)out, layout, rows, cols, seed, sa, sb, sc,
                                                hq, hkv, d, stdv);
  else
    init_weight_kernel<bf16_t><<<g, 256, 0, s>>>((bf16_t*)out, layout, rows, cols, seed, sa, sb,
                                                 sc, hq, hkv, d, stdv);
  return hipGetLastError();
}

}  // namespace vla

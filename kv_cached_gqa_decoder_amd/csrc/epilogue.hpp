// Epilogues shared by the projection kernels (matrix-core GEMM, fp32 GEMM, GEMV).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace vla {

// One RoPE pair of the fused q/k/v projection for token row t.
// `col` is the even physical column of the pair (LAYOUT_QKV): logical dims
// j and j + d/2 of head col/d, with j = (col % d) / 2. q and k are rotated by
// the angle of row t's absolute position times theta^(-2j/d) ("Rebuilding
// Kshipra Around Memory", section 4: RoPE at absolute positions; rotate-half
// pairing), read from the pass's (cos, sin) table; q goes to the query buffer,
// k and v to the paged pool at the token's block and slot (the cache stores
// post-RoPE keys).
// The pair's operands that do not depend on the projection (its rotation and,
// for k/v heads, the physical block of the token), so a kernel can request them
// before its sums are ready.
struct QkvPre {
  float2 cs = {1.f, 0.f};
  int blk = 0;
};
__device__ __forceinline__ QkvPre epi_qkv_prefetch(const FwdCtx& c, int t, int col) {
  QkvPre p;
  const int d = c.g.d;
  const int head = col / d;
  const int j = (col % d) >> 1;
  if (head < c.hq + c.g.hkv) p.cs = c.rope[(size_t)t * (d / 2) + j];
  if (head >= c.hq) p.blk = c.blk_table[c.cb0 + (c.cslot0 + t) / c.g.bt];
  return p;
}
// The same factors for any head, loaded unconditionally (row t < the chunk's rows):
// a guarded load is waited for before its default value can be written to the
// same registers, so many guarded prefetches cost one round trip each.
__device__ __forceinline__ QkvPre epi_qkv_prefetch_all(const FwdCtx& c, int t, int col) {
  QkvPre p;
  const int d = c.g.d;
  p.cs = c.rope[(size_t)t * (d / 2) + ((col % d) >> 1)];
  p.blk = c.blk_table[c.cb0 + (c.cslot0 + t) / c.g.bt];
  return p;
}
template <typename T>
__device__ __forceinline__ void epi_qkv_store(const FwdCtx& c, int t, int col, const QkvPre& p,
                                              float lo, float hi) {
  const int d = c.g.d;
  const int head = col / d;
  const int j = (col % d) >> 1;
  const int hkv = c.g.hkv;
  if (head < c.hq + hkv) {
    const float rlo = lo * p.cs.x - hi * p.cs.y;
    const float rhi = hi * p.cs.x + lo * p.cs.y;
    lo = rlo;
    hi = rhi;
  }
  if (head < c.hq) {
    T* q = (T*)c.qbuf + ((size_t)t * c.hq + head) * d;
    St<T>::st(q, j, lo);
    St<T>::st(q, j + d / 2, hi);
    return;
  }
  const int s = (c.cslot0 + t) % c.g.bt;
  if (head < c.hq + hkv) {
    const int h = head - c.hq;
    T* kp = (T*)c.kpool;
    St<T>::st(kp, c.g.kidx(c.layer, p.blk, h, s, j), lo);
    St<T>::st(kp, c.g.kidx(c.layer, p.blk, h, s, j + d / 2), hi);
  } else {
    const int h = head - c.hq - hkv;
    T* vp = (T*)c.vpool;
    St<T>::st(vp, c.g.vidx(c.layer, p.blk, h, s, j), lo);
    St<T>::st(vp, c.g.vidx(c.layer, p.blk, h, s, j + d / 2), hi);
  }
}
template <typename T>
__device__ __forceinline__ void epi_qkv_pair(const FwdCtx& c, int t, int col, float lo, float hi) {
  epi_qkv_store<T>(c, t, col, epi_qkv_prefetch(c, t, col), lo, hi);
}

// order-preserving map of an fp32 value to uint32 (larger float -> larger key)
__device__ __forceinline__ uint32_t f32_order_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// argmax key: value in the high word, (0xffffffff - index) in the low word, so the
// largest key is the largest value and, among equal values, the lowest index
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx) {
  return ((unsigned long long)f32_order_key(v) << 32) | (unsigned long long)(0xffffffffu - idx);
}

}  // namespace vla

// The decode step's first phase as device functions: the token's embedding row
// and the position's RoPE table, shared by their kernels and the persistent
// decode step.
#pragma once

#include "common.hpp"

namespace vla {

// entry p = t * half + j of the table: (cos, sin) of (pos0 + t) * inv_freq[j]
__device__ __forceinline__ void rope_entry(int64_t p, int64_t pos0, const double* inv_freq,
                                           int half, float2* tab) {
  const int64_t t = p / half;
  const int j = (int)(p % half);
  const double ang = (double)(pos0 + t) * inv_freq[j];
  const double red = fma(-rint(ang * 0.15915494309189535), 6.283185307179586, ang);
  float sn, cs;
  sincosf((float)red, &sn, &cs);
  tab[p] = make_float2(cs, sn);
}
// one decode row: virtual block 0 gathers the token's embedding row, block 1 writes
// the row's RoPE table
template <typename T>
__device__ __forceinline__ void embed_rope1_body(int token_scalar,
                                                 const unsigned long long* token_key, const T* E,
                                                 float* x, int H, int64_t pos,
                                                 const double* inv_freq, int half, float2* tab,
                                                 int vb) {
  if (vb == 0) {
    const int64_t id = token_key ? (int64_t)(0xffffffffu - (uint32_t)(*token_key & 0xffffffffull))
                                 : token_scalar;
    for (int i = threadIdx.x; i < H; i += blockDim.x) x[i] = St<T>::ld(E, id * H + i);
  } else {
    for (int p = threadIdx.x; p < half; p += blockDim.x) rope_entry(p, pos, inv_freq, half, tab);
  }
}

}  // namespace vla

// One decode step in one launch ("Running VLAs at Real-time Speed", section 3.1:
// replaying the step as one unit instead of a chain of separate launches; section
// 5.2: the synchronisation between the many small products is a cost of its own).
//
// A fixed grid of workgroups, all resident (cooperative launch), walks the phases
// of the step: the token's embedding row and the position's RoPE table, then for
// every layer the q/k/v projection (RoPE + paged K/V write), the decode attention
// (key splits), the output projection (which merges the splits on the way in), the
// gated projection and the down projection. A phase is the work of the separate
// kernel it replaces, dealt out by virtual workgroup index (the same device
// functions, so the same arithmetic in the same order), and phases are separated
// by a device-scope barrier: every workgroup releases its writes (L2 write-back),
// adds one to an arrival counter with a vector atomic, polls it with vector loads
// until all workgroups have arrived, then acquires (L2 invalidate). A wait is
// bounded: after spin_limit polls, or once another workgroup has given up, the
// workgroup sets the error flag and ends, so the launch always completes.
#include <hip/hip_runtime.h>

#include "attn_decode.hpp"
#include "common.hpp"
#include "gemv_body.hpp"
#include "kernels.hpp"
#include "rope_body.hpp"

namespace vla {

__device__ __forceinline__ bool step_barrier(const DecodeStepArgs& p, unsigned long long target) {
  __shared__ int ok_s;
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(p.bar, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int ok = 1;
    for (int it = 0;
         __hip_atomic_load(p.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++it) {
      if (it >= p.spin_limit ||
          __hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (!ok) __hip_atomic_store(p.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ok_s = ok;
  }
  __syncthreads();
  return ok_s != 0;
}

template <int D, int CQ, int CO, int CG, int DRW, int DCPL, int DKS>
__global__ __launch_bounds__(kGemvThreads) void decode_step_kernel(DecodeStepArgs p) {
  const int G = gridDim.x;
  unsigned long long target = p.base;
  for (int vb = blockIdx.x; vb < 2; vb += G)
    embed_rope1_body<bf16_t>(p.token, p.token_key, (const bf16_t*)p.E, p.x, p.H, p.pos,
                             p.inv_freq, p.half, p.rope, vb);
  for (int l = 0; l < p.n_layers; ++l) {
    const void* const* w = p.wtab + 4 * l;
    target += G;
    if (!step_barrier(p, target)) return;
    for (int vb = blockIdx.x; vb < p.vg_qkv; vb += G) {
      gemv1_body<EPI_QKV, 2, CQ, 1, false>(p.qkv, p.ng_qkv, vb, w[0], l);
      __syncthreads();
    }
    target += G;
    if (!step_barrier(p, target)) return;
    for (int vb = blockIdx.x; vb < p.at.splits * p.at.g.hkv; vb += G) {
      attn_decode_body<D>(p.at, 1, vb % p.at.splits, 0, vb / p.at.splits, l);
      __syncthreads();
    }
    target += G;
    if (!step_barrier(p, target)) return;
    for (int vb = blockIdx.x; vb < p.vg_o; vb += G) {
      gemv1_body<EPI_RESID, 2, CO, 1, true>(p.o, p.ng_o, vb, w[1], l);
      __syncthreads();
    }
    target += G;
    if (!step_barrier(p, target)) return;
    for (int vb = blockIdx.x; vb < p.vg_gu; vb += G) {
      gemv1_body<EPI_SWIGLU, 2, CG, 1, false>(p.gu, p.ng_gu, vb, w[2], l);
      __syncthreads();
    }
    target += G;
    if (!step_barrier(p, target)) return;
    for (int vb = blockIdx.x; vb < p.vg_dn; vb += G) {
      gemv1_body<EPI_RESID, DRW, DCPL, DKS, false>(p.dn, p.ng_dn, vb, w[3], l);
      __syncthreads();
    }
  }
}

// Barrier latency probe: nbar barriers of the decode step's kind over `grid`
// workgroups (cooperative launch), each phase one store per thread.
__global__ __launch_bounds__(kGemvThreads) void barrier_probe_kernel(DecodeStepArgs p, int nbar,
                                                                    float* scratch) {
  unsigned long long target = p.base;
  for (int i = 0; i < nbar; ++i) {
    scratch[blockIdx.x * kGemvThreads + threadIdx.x] += 1.f;
    target += gridDim.x;
    if (!step_barrier(p, target)) return;
  }
}

hipError_t launch_barrier_probe(unsigned long long* bar, int* err, float* scratch, int grid,
                                int nbar, int spin_limit, hipStream_t s) {
  DecodeStepArgs p;
  p.bar = bar;
  p.err = err;
  p.base = 0;
  p.spin_limit = spin_limit;
  void* args[] = {&p, &nbar, &scratch};
  return hipLaunchCooperativeKernel((const void*)barrier_probe_kernel, dim3(grid),
                                    dim3(kGemvThreads), args, 0, s);
}

int barrier_probe_max_grid() {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, barrier_probe_kernel, kGemvThreads, 0) !=
      hipSuccess)
    return 0;
  return per * cus;
}

template <int D, int CQ, int CO, int CG, int DRW, int DCPL, int DKS>
static int grid_of() {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per, decode_step_kernel<D, CQ, CO, CG, DRW, DCPL, DKS>, kGemvThreads, 0) != hipSuccess)
    return 0;
  return per * cus;
}

int decode_step_grid(int shape) {
  switch (shape) {
    case DSHAPE_C3_3_3_D1_5_4: return grid_of<128, 3, 3, 3, 1, 5, 4>();
    case DSHAPE_C1_2_1_D2_1_1: return grid_of<128, 1, 2, 1, 2, 1, 1>();
    default: return 0;
  }
}

template <int D, int CQ, int CO, int CG, int DRW, int DCPL, int DKS>
static hipError_t go(const DecodeStepArgs& p, int grid, hipStream_t s) {
  DecodeStepArgs q = p;
  void* args[] = {&q};
  return hipLaunchCooperativeKernel((const void*)decode_step_kernel<D, CQ, CO, CG, DRW, DCPL, DKS>,
                                    dim3(grid), dim3(kGemvThreads), args, 0, s);
}

hipError_t launch_decode_step(const DecodeStepArgs& p, int shape, int grid, hipStream_t s) {
  if (grid < 1) return hipErrorInvalidValue;
  switch (shape) {
    case DSHAPE_C3_3_3_D1_5_4: return go<128, 3, 3, 3, 1, 5, 4>(p, grid, s);
    case DSHAPE_C1_2_1_D2_1_1: return go<128, 1, 2, 1, 2, 1, 1>(p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vla

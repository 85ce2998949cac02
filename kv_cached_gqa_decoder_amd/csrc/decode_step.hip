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
// by a device-scope barrier.
//
// The barrier groups the workgroups by XCD, each XCD having an L2 of its own: a
// workgroup waits for its own stores (vmcnt), counts in on its XCD's counter and,
// unless it is the XCD's last arrival, polls the XCD's release flag. The last
// arrival writes the XCD's L2 back (agent-scope release), counts in on the top
// counter (the last XCD there publishes the generation), polls the generation,
// invalidates the XCD's L2 (agent-scope acquire) and raises the XCD's release flag;
// the others then invalidate their own CU's L1 and L2 view (agent-scope acquire).
// One L2 write-back per XCD instead of one per workgroup: 4.4 against 8.3 us per
// barrier at 256 workgroups, 6.5 against 31 at 512. Workgroups learn their XCD from
// the hardware register and register themselves (per-XCD counts, 16 bits each, in
// two words) when the launch starts; the first barrier waits for all of them. All
// atomics and polls are vector memory operations. A wait is bounded: after
// spin_limit polls, or once another workgroup has given up, the workgroup sets the
// error flag and ends, so the launch always completes.
#include <hip/hip_runtime.h>

#include "attn_decode.hpp"
#include "common.hpp"
#include "gemv_body.hpp"
#include "kernels.hpp"
#include "rope_body.hpp"

namespace vla {

typedef unsigned long long u64;

__device__ __forceinline__ u64 bar_ld(const u64* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool bar_failed(const DecodeStepArgs& p) {
  return __hip_atomic_load((const int*)p.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}
// polls *w until it reaches target; false after spin_limit polls or once the error
// flag is set
__device__ __forceinline__ bool bar_wait(const DecodeStepArgs& p, const u64* w, u64 target) {
  for (int it = 0; bar_ld(w) < target; ++it) {
    if (it >= p.spin_limit || bar_failed(p)) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}
// this launch's state set: registration words (lines 0, 1), XCD counters (2..9), top
// counter (10), XCD release flags (11..18), generation (19)
__device__ __forceinline__ u64* bar_set(const DecodeStepArgs& p, int seq) {
  return p.bar + kBarLineWords * (1 + kBarSetLines * (seq & 1));
}
// the XCD this workgroup runs on (hardware register XCC_ID, bits 0..3; 0..7 on a
// device of 8 XCDs)
__device__ __forceinline__ int xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15;
}

// thread 0's barrier state: its XCD, the workgroups on it, the XCDs in use (0 until
// the registration has been read)
struct BarState {
  int x = 0, nx = 0, nxa = 0;
};

// launch start: workgroup 0 clears the other set for the next launch; every
// workgroup registers on its XCD
__device__ __forceinline__ void bar_start(const DecodeStepArgs& p, BarState& b) {
  if (blockIdx.x == 0 && threadIdx.x < kBarSetLines)
    bar_set(p, p.seq + 1)[threadIdx.x * kBarLineWords] = 0ull;
  if (threadIdx.x == 0) {
    b.x = xcc_id();
    if (b.x > 7) {
      // more than 8 XCDs: the groups would not match the L2s; error flag 2 (the
      // first barrier then gives up)
      __hip_atomic_store((int*)p.bar, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      b.x = 0;
    }
    __hip_atomic_fetch_add(bar_set(p, p.seq) + (b.x >> 2) * kBarLineWords,
                           1ull << (16 * (b.x & 3)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// barrier number gen (1, 2, ...) of this launch
__device__ __forceinline__ bool step_barrier(const DecodeStepArgs& p, BarState& b, u64 gen) {
  __shared__ int ok_s;
  // every thread's stores of the phase have reached L2 before the workgroup counts in
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    u64* S = bar_set(p, p.seq);
    int ok = 1;
    if (b.nx == 0) {  // first barrier: wait until every workgroup has registered
      for (int it = 0;; ++it) {
        const u64 r0 = bar_ld(S), r1 = bar_ld(S + kBarLineWords);
        int tot = 0, nxa = 0;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int c0 = (int)((r0 >> (16 * f)) & 0xffff), c1 = (int)((r1 >> (16 * f)) & 0xffff);
          tot += c0 + c1;
          nxa += (c0 > 0) + (c1 > 0);
        }
        if (tot == (int)gridDim.x) {
          b.nx = (int)(((b.x < 4 ? r0 : r1) >> (16 * (b.x & 3))) & 0xffff);
          b.nxa = nxa;
          break;
        }
        if (it >= p.spin_limit || bar_failed(p)) {
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (ok) {
      const u64 target = gen + p.gen_off;
      u64* flag = S + (11 + b.x) * kBarLineWords;
      const u64 old = __hip_atomic_fetch_add(S + (2 + b.x) * kBarLineWords, 1ull, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      if (old + 1 == gen * (u64)b.nx) {  // the XCD's last arrival
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const u64 t = __hip_atomic_fetch_add(S + 10 * kBarLineWords, 1ull, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        if (t + 1 == gen * (u64)b.nxa)
          __hip_atomic_store(S + 19 * kBarLineWords, gen, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        ok = bar_wait(p, S + 19 * kBarLineWords, target);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(flag, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        ok = bar_wait(p, flag, target);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
    }
    if (!ok && !bar_failed(p))
      __hip_atomic_store((int*)p.bar, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ok_s = ok;
  }
  __syncthreads();
  return ok_s != 0;
}

template <int D, int CQ, int CO, int CG, int DRW, int DCPL, int DKS>
__global__ __launch_bounds__(kGemvThreads) void decode_step_kernel(DecodeStepArgs p) {
  const int G = gridDim.x;
  BarState bs;
  bar_start(p, bs);
  u64 gen = 0;
  for (int vb = blockIdx.x; vb < 2; vb += G)
    embed_rope1_body<bf16_t>(p.token, p.token_key, (const bf16_t*)p.E, p.x, p.H, p.pos,
                             p.inv_freq, p.half, p.rope, vb);
  for (int l = 0; l < p.n_layers; ++l) {
    const void* const* w = p.wtab + 4 * l;
    if (!step_barrier(p, bs, ++gen)) return;
    for (int vb = blockIdx.x; vb < p.vg_qkv; vb += G) {
      gemv1_body<EPI_QKV, 2, CQ, 1, false>(p.qkv, p.ng_qkv, vb, w[0], l);
      __syncthreads();
    }
    if (!step_barrier(p, bs, ++gen)) return;
    for (int vb = blockIdx.x; vb < p.at.splits * p.at.g.hkv; vb += G) {
      attn_decode_body<D>(p.at, 1, vb % p.at.splits, 0, vb / p.at.splits, l);
      __syncthreads();
    }
    if (!step_barrier(p, bs, ++gen)) return;
    for (int vb = blockIdx.x; vb < p.vg_o; vb += G) {
      gemv1_body<EPI_RESID, 2, CO, 1, true>(p.o, p.ng_o, vb, w[1], l);
      __syncthreads();
    }
    if (!step_barrier(p, bs, ++gen)) return;
    for (int vb = blockIdx.x; vb < p.vg_gu; vb += G) {
      gemv1_body<EPI_SWIGLU, 2, CG, 1, false>(p.gu, p.ng_gu, vb, w[2], l);
      __syncthreads();
    }
    if (!step_barrier(p, bs, ++gen)) return;
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
  BarState bs;
  bar_start(p, bs);
  for (int i = 0; i < nbar; ++i) {
    scratch[blockIdx.x * kGemvThreads + threadIdx.x] += 1.f;
    if (!step_barrier(p, bs, (u64)i + 1)) return;
  }
}

hipError_t launch_barrier_probe(unsigned long long* bar, float* scratch, int grid, int nbar,
                                int seq, int spin_limit, hipStream_t s) {
  DecodeStepArgs p;
  p.bar = bar;
  p.seq = seq;
  p.gen_off = 0;
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

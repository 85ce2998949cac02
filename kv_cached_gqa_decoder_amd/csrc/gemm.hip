// Prefill projections C[M][N] = A[M][K] * W[N][K]^T with fused epilogues.
//  bf16: matrix-core kernels on v_mfma_f32_16x16x32_bf16 (fp32 accumulate),
//        operands streamed into a multi-stage LDS ring by global_load_lds
//        (direct-to-LDS DMA, no register staging); gated projections of
//        129-256 rows on a two-stream kernel (separate activation and weight
//        rings, each with its own producer wavefronts).
//  fp32: FMA kernel (the fp32 configuration never touches bf16 matrix cores).
// Epilogues: plain store, residual add (x += C), RoPE + paged K/V write on the
// fused q/k/v projection, SwiGLU on the interleaved gate/up projection
// ("Running VLAs at Real-time Speed", section 4.2: both gated projections in
// one GEMM, only the gated product written back; section 4.4: bias-free
// residual and activation fused into the GEMM epilogue).
#include <hip/hip_fp16.h>

#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "epilogue.hpp"
#include "kernels.hpp"

namespace vla {

// ---------------------------------------------------------------------------
// bf16 matrix-core GEMM. Block tile BM x BN (64 or 128 each), 4 wavefronts in a
// 2 x 2 grid, each wavefront (BM/2) x (BN/2) = MT x NT tiles of 16 x 16 on
// v_mfma_f32_16x16x32_bf16, fp32 accumulation.
//
// Operands stream straight from memory into an NS-stage LDS ring with
// global_load_lds_dwordx4 (no register staging): a stage is one 64-deep K
// step of the A tile (BM rows) and the W tile (BN rows), 128 bytes per row.
// One such load fills 1 KiB of LDS (8 rows); lane i writes the 16-byte chunk
// at position i % 8 of row i / 8, and fetches the K chunk (i % 8) ^ (row % 8)
// of that row, so the matrix-core operand reads (16 rows, one chunk column)
// fall in distinct LDS banks. NS-1 stages are in flight while one is used.
//
// Tiles are ordered so that each XCD (workgroup L runs on XCD L % 8) walks a
// contiguous run of tiles with the M tiles of one weight tile adjacent: the
// weight tile is fetched from HBM once and re-read from that XCD's L2.
// Split-K (over blockIdx) writes fp32 partials for the residual projections;
// a reduction kernel adds them to the residual in split order.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
// kernel-side epilogue id of the gated product with the GELU gate (the host
// arguments say EPI_SWIGLU with glu = 1)
constexpr int EPI_GEGLU_K = 16;
template <int EPI> constexpr bool kGated = EPI == EPI_SWIGLU || EPI == EPI_GEGLU_K;

// LO: the activations come as a bf16 pair (A, A_lo); a stage holds the BM rows of
// A, then the BM rows of A_lo, then the BN weight rows, and every weight fragment
// meets both activation fragments (two MFMAs, the high part first)
template <int BM, int BN, int BK, int NS, int WGM = 2, int WGN = 2, bool LO = false>
struct GemmTile {
  static constexpr int NW = WGM * WGN;               // wavefronts per workgroup
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int MT = WM / 16, NT = WN / 16;
  static constexpr int ROWB = BK * 2;                // bytes of one LDS row (one K step)
  static constexpr int CPR = BK / 8;                 // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;               // rows filled by one DMA load
  static constexpr int AROWS = LO ? 2 * BM : BM;     // activation rows per stage
  static constexpr int ROWS = AROWS + BN;            // LDS rows per stage
  static constexpr int STAGE = ROWS * ROWB;          // bytes
  static constexpr int LOADS = ROWS / RPI / NW;      // DMA loads per wavefront per stage
  static_assert(LOADS * RPI * NW == ROWS && WM % 16 == 0 && WN % 16 == 0, "tile shape");
  static constexpr int LDS = NS * STAGE;
  static_assert(LDS <= 160 * 1024, "LDS");
  // chunk position of K chunk kc in LDS row r: 8 consecutive rows read at one chunk
  // column land in 8 distinct 16-byte bank groups (32 or 64 banks)
  static __device__ __forceinline__ int pos(int r, int kc) {
    return BK == 64 ? (kc ^ (r & 7)) : (kc ^ ((r >> 1) & 3));
  }
};

// Epilogue of a wavefront's (MT x NT) tiles. Accumulator element e of tile
// (mi, ni) is row 4*(lane/16)+e, column lane%16 of that 16 x 16 tile.
template <int EPI, int MT, int NT, int WM, int WN>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, f32x4_t (&acc)[MT][NT], int m0,
                                              int n0, int z, int wm, int wn, int lane) {
  const int M = a.M;
  if constexpr (EPI == EPI_QKV) {
    // every pair's RoPE factors and K/V block id are requested, unconditionally,
    // before the first store (loads cannot move past the stores, so per-pair
    // load-then-store cost one memory round trip per pair)
    QkvPre pre[MT][4][NT];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) {
          const int row = m0 + wm * WM + mi * 16 + 4 * (lane >> 4) + e;
          const int col = n0 + wn * WN + ni * 16 + (lane & 15);
          pre[mi][e][ni] = epi_qkv_prefetch_all(a.ctx, row < M ? row : M - 1, col);
        }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of every store
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) {
          const int row = m0 + wm * WM + mi * 16 + 4 * (lane >> 4) + e;
          const int col = n0 + wn * WN + ni * 16 + (lane & 15);
          const float v = acc[mi][ni][e];
          // the neighbouring lane's value (DPP quad permute [1, 0, 3, 2]: no LDS round)
          const float partner =
              __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
          if (row < M && (col & 1) == 0)
            epi_qkv_store<bf16_t>(a.ctx, row, col, pre[mi][e][ni], v, partner);
        }
    return;
  }
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = m0 + wm * WM + mi * 16 + 4 * (lane >> 4) + e;
      if constexpr (kGated<EPI>) {
        // tiles (ni, ni+1), ni even: gate rows f and the matching up rows (LAYOUT_GATEUP)
#pragma unroll
        for (int ni = 0; ni < NT; ni += 2) {
          const int f = (n0 + wn * WN + ni * 16) / 2 + (lane & 15);
          const bf16_t o = bf16_rne(glu_fast<EPI == EPI_GEGLU_K>(acc[mi][ni][e], acc[mi][ni + 1][e]));
          if (row < M) ((bf16_t*)a.C)[(size_t)row * (a.N / 2) + f] = o;
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) {
          const int col = n0 + wn * WN + ni * 16 + (lane & 15);
          const float v = acc[mi][ni][e];
          if (row < M) a.ws[((size_t)z * M + row) * a.N + col] = v;  // EPI_PARTIAL
        }
      }
    }
  }
}

template <int EPI, int BM, int BN, int BK, int NS, int WGM, int WGN, bool LO>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_kernel(GemmArgs a, int tiles_m,
                                                                   int tiles, int ksteps) {
  using G = GemmTile<BM, BN, BK, NS, WGM, WGN, LO>;
  constexpr int MT = G::MT, NT = G::NT, LOADS = G::LOADS;
  static_assert(LOADS * (NS - 1) <= 63 && NS - 2 <= 6, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[G::LDS];

  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int slot = blockIdx.x % (kXcds * per_xcd);
  const int z = blockIdx.x / (kXcds * per_xcd);
  const int t = (slot % kXcds) * per_xcd + slot / kXcds;
  if (t >= tiles) return;
  const int m0 = (t % tiles_m) * BM, n0 = (t / tiles_m) * BN;
  const int M = a.M, K = a.K;
  const int kt0 = z * ksteps;
  const int nk = min(K / BK - kt0, ksteps);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  // this lane's sources for its LOADS DMA loads (rows past M re-read row M-1): load j
  // reads a uniform base (its 1 KiB piece lies wholly in the activation rows, their low
  // part or the weight rows) plus the lane's 32-bit byte offset
  const unsigned char* base[LOADS];
  uint32_t off[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int row0 = (wave * LOADS + j) * G::RPI;  // the piece's first row (uniform)
    const int row = row0 + lane / G::CPR;
    const int kc = G::pos(row, lane % G::CPR);  // pos() is an involution in kc
    if (row0 < G::AROWS) {
      const int ar = min(m0 + (row < BM ? row : row - BM), M - 1);
      base[j] = (const unsigned char*)(row0 < BM ? a.A : a.A_lo) +
                ((int64_t)m0 * K + (int64_t)kt0 * BK) * 2;
      off[j] = (uint32_t)(((ar - m0) * K + kc * 8) * 2);
    } else {
      base[j] = (const unsigned char*)a.W + ((int64_t)n0 * K + (int64_t)kt0 * BK) * 2;
      off[j] = (uint32_t)(((row - G::AROWS) * K + kc * 8) * 2);
    }
  }
  // stage kt -> ring slot kt % NS. Past the last step the DMA re-loads the last
  // step's data into the slot just freed (never read), so every step issues the
  // same loads and every wait has one constant depth
  auto issue = [&](int kt) {
    unsigned char* st = smem + (kt % NS) * G::STAGE + wave * LOADS * 1024;
    const int kd = kt < nk ? kt : nk - 1;
#pragma unroll
    for (int j = 0; j < LOADS; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(base[j] + kd * (BK * 2) + off[j]),
                                       (__attribute__((address_space(3))) void*)(st + j * 1024),
                                       16, 0, 0);
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (nk <= 0) {  // (the host never splits K into an empty piece)
    gemm_epilogue<EPI, MT, NT, G::WM, G::WN>(a, acc, m0, n0, z, wm, wn, lane);
    return;
  }
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once at most NS-2 younger stages are outstanding
    wait_vmcnt_steps<LOADS>(NS - 2);
    // every wavefront's loads of stage kt are in LDS, and every wavefront's reads of
    // stage kt-1 have returned (lgkmcnt), so that stage may be refilled. A bare
    // barrier: a fenced one would also drain the loads still in flight.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue(kt + NS - 1);
    const unsigned char* st = smem + (kt % NS) * G::STAGE;
    // all operand fragments of the step first, then each accumulator's MFMAs back to
    // back (sub-step 0 high, low, sub-step 1 ...): one update chain per accumulator
    // and step, so the compiler keeps every accumulator in place (two separate passes
    // over the accumulators made it rotate them through other registers every step)
    constexpr int KS = BK / 32;
    bf16x8_t bf[KS][NT], af[KS][MT], al[KS][LO ? MT : 1];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int kc = ks * 4 + (lane >> 4);
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) {
        const int r = G::AROWS + wn * G::WN + ni * 16 + (lane & 15);
        bf[ks][ni] = *(const bf16x8_t*)(st + r * G::ROWB + (G::pos(r, kc) << 4));
      }
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const int r = wm * G::WM + mi * 16 + (lane & 15);
        af[ks][mi] = *(const bf16x8_t*)(st + r * G::ROWB + (G::pos(r, kc) << 4));
        if constexpr (LO) {
          const int rl = BM + r;
          al[ks][mi] = *(const bf16x8_t*)(st + rl * G::ROWB + (G::pos(rl, kc) << 4));
        }
      }
    }
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][mi], bf[ks][ni], acc[mi][ni], 0, 0, 0);
          if constexpr (LO)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[ks][mi], bf[ks][ni], acc[mi][ni], 0, 0, 0);
        }
  }

  gemm_epilogue<EPI, MT, NT, G::WM, G::WN>(a, acc, m0, n0, z, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// Two-stream GEMM for BMT-row M tiles (128 or 256) with a wide N: the gated
// projection of a 129- to 256-token prefill, and the long-K residual projection
// (down) of one, split along K. The activation tile (re-read by every column group)
// and the weight tile (streamed from HBM once) travel in two LDS rings of
// different depths, each filled by its own two producer wavefronts with
// global_load_lds DMA. Vector-memory counters retire in issue order per
// wavefront, so a ring's producers wait only for their own stream: the weight
// ring keeps NSW-1 32-deep steps in flight (the HBM latency needs about 100 KB per
// CU) while the activation ring stays shorter. Four consumer wavefronts (BMT/4 rows
// each, every column of the group) read both operands from LDS; one barrier per
// K step hands both stages over. Columns are dealt out in units of 32 (one
// interleaved gate/up block), each workgroup taking a contiguous run of floor or
// ceil of units/groups, so a launch covers every column in about one round of
// workgroups. Unsplit launches put the M tiles of one column group on one XCD
// (they share the weight tile through its L2); split launches put the column
// groups of one (K piece, M tile) on one XCD (they share the activation piece).
// ---------------------------------------------------------------------------
template <int NTM, int NSA, int NSW, bool LO = false, int BMT = 256, int KB = 64>
struct Ws2Tile {
  // a stage holds KB bytes (KB / 2 bf16 of K) of each row: BMT activation rows (LO: then
  // the BMT rows of their low part) and NTM * 16 weight rows
  static constexpr int CPR = KB / 16;                // 16-byte chunks per row
  static constexpr int RPI = 1024 / KB;              // rows one DMA load fills
  static constexpr int KSTEP = KB / 2;               // K per stage
  static constexpr int AROWS = (LO ? 2 : 1) * BMT;
  static constexpr int ASTAGE = AROWS * KB;
  static constexpr int WROWS = NTM * 16;
  static constexpr int WSTAGE = WROWS * KB;
  static constexpr int ALOADS = ASTAGE / 1024 / 2;   // DMA loads per activation producer
  static constexpr int WLOADS = WSTAGE / 1024 / 2;   // DMA loads per weight producer
  static constexpr int LDS = NSA * ASTAGE + NSW * WSTAGE;
  static_assert((KB == 64 || KB == 128) && WSTAGE % 2048 == 0 && ALOADS * (NSA - 2) <= 63 &&
                    WLOADS * (NSW - 2) <= 63 && LDS <= 160 * 1024,
                "ring shape");
  static_assert(NTM % 2 == 0 && NTM >= 2 && NTM <= 12 && (BMT == 64 || BMT == 128 || BMT == 256),
                "tile counts");
  // chunk position of K chunk kc in LDS row r: 16 rows read at one chunk column fall in
  // distinct 16-byte bank groups (an involution in kc)
  static __device__ __forceinline__ int pos(int r, int kc) {
    return kc ^ ((r >> 1) & (CPR - 1));
  }
};

// wait until at most N of this wavefront's vector-memory operations are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | 0x70 | 0xF00 | ((N >> 4) << 14));
}

// producer wavefront of one ring: rows [row0, row0 + LOADS * RPI) of each stage; a
// DMA load fills 1 KiB = RPI rows of KB bytes, lane i writing chunk position i % CPR
// of row i / CPR with the K chunk that position holds. Load j reads base[j] (uniform,
// the K piece's first column) + off[j] (the lane's byte offset) + KB bytes per K
// step: the address is one scalar base and one 32-bit vector offset, and the LDS
// destination is uniform, so a load needs no per-lane address arithmetic and no
// register it shares with the next load
template <int LOADS, int NS, int STAGE, int KB>
__device__ __forceinline__ void ws2_produce(unsigned char* ring,
                                            const unsigned char* const (&base)[LOADS],
                                            const uint32_t (&off)[LOADS], int lds_off, int nk) {
  auto issue = [&](int kt) {
    unsigned char* st = ring + (kt % NS) * STAGE + lds_off;
    const int kd = kt < nk ? kt : nk - 1;  // past the end: the last step again (never read)
#pragma unroll
    for (int j = 0; j < LOADS; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(base[j] + kd * KB + off[j]),
                                       (__attribute__((address_space(3))) void*)(st + j * 1024),
                                       16, 0, 0);
  };
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0) issue(s0);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt_le<LOADS * (NS - 2)>();  // stage kt of this ring has landed
    asm volatile("s_barrier" ::: "memory");
    issue(kt + NS - 1);                 // into the slot of stage kt-1, read before this barrier
  }
  __builtin_amdgcn_s_waitcnt(0);        // no DMA outstanding at exit
}

// consumer wavefront c of CW: rows (BMT/CW)c .. of the M tile, NTC 16-column tiles;
// the gated product, or (EPI_PARTIAL) this K piece's fp32 partial [z][M][N]
template <int EPI, int NTC, int NTM, int NSA, int NSW, int CW, bool LO, int BMT, int KB>
__device__ __forceinline__ void ws2_consume(const GemmArgs& a, const unsigned char* smem, int nk,
                                            int n0, int m0, int c, int lane, int z) {
  static_assert(kGated<EPI> || EPI == EPI_PARTIAL, "gated products or split-K partials");
  using T = Ws2Tile<NTM, NSA, NSW, LO, BMT, KB>;
  constexpr int RPW = BMT / CW, MT = RPW / 16;  // rows and 16-row tiles per consumer
  f32x4_t acc[MT][NTC];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTC; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int kt = 0; kt < nk; ++kt) {
    asm volatile("s_barrier" ::: "memory");  // both stages of step kt are in LDS
    const unsigned char* sa = smem + (kt % NSA) * T::ASTAGE;
    const unsigned char* sw = smem + NSA * T::ASTAGE + (kt % NSW) * T::WSTAGE;
#pragma unroll
    for (int sub = 0; sub < KB / 64; ++sub) {  // 32-wide K slices of the stage
      const int kc = sub * 4 + (lane >> 4);
      bf16x8_t bf[NTC];
#pragma unroll
      for (int ni = 0; ni < NTC; ++ni) {
        const int r = ni * 16 + (lane & 15);
        bf[ni] = *(const bf16x8_t*)(sw + r * KB + (T::pos(r, kc) << 4));
      }
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const int r = RPW * c + 16 * mi + (lane & 15);
        const bf16x8_t af = *(const bf16x8_t*)(sa + r * KB + (T::pos(r, kc) << 4));
#pragma unroll
        for (int ni = 0; ni < NTC; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[ni], acc[mi][ni], 0, 0, 0);
        if constexpr (LO) {
          const int rl = BMT + r;
          const bf16x8_t al = *(const bf16x8_t*)(sa + rl * KB + (T::pos(rl, kc) << 4));
#pragma unroll
          for (int ni = 0; ni < NTC; ++ni)
            acc[mi][ni] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bf[ni], acc[mi][ni], 0, 0, 0);
        }
      }
    }
    // this step's LDS reads are complete before the barrier that lets them be refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  // accumulator element e of tile (mi, ni) is row 4*(lane/16)+e, column lane%16
  const int M = a.M;
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = m0 + RPW * c + 16 * mi + 4 * (lane >> 4) + e;
#pragma unroll
      for (int ni = 0; ni < NTC; ++ni) {
        const float v = acc[mi][ni][e];
        if constexpr (EPI == EPI_PARTIAL) {
          if (row < M) a.ws[((size_t)z * M + row) * a.N + n0 + ni * 16 + (lane & 15)] = v;
        } else if ((ni & 1) == 0) {
          // tiles (ni, ni+1), ni even: 16 gate columns, then the 16 matching up columns
          const bf16_t o =
              bf16_rne(glu_fast<EPI == EPI_GEGLU_K>(v, acc[mi][ni + 1 < NTC ? ni + 1 : ni][e]));
          if (row < M) ((bf16_t*)a.C)[(size_t)row * (a.N / 2) + (n0 + ni * 16) / 2 + (lane & 15)] = o;
        }
      }
    }
  }
}

template <int EPI, int NTM, int NSA, int NSW, int CW, bool LO, int BMT, int KB>
__global__ __launch_bounds__(64 * (CW + 4)) void gemm_ws2_kernel(GemmArgs a, int units, int groups,
                                                                 int tiles_m, int splits,
                                                                 int ksteps) {
  using T = Ws2Tile<NTM, NSA, NSW, LO, BMT, KB>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[T::LDS];
  const int g8 = (groups + 7) & ~7;
  int mt, g, z;
  if (splits == 1) {
    // workgroup -> (M tile mt, column group g); the M tiles of one group sit 8
    // workgroups apart, i.e. on one XCD
    const int r = blockIdx.x;
    mt = (r % (8 * tiles_m)) / 8;
    g = (r / (8 * tiles_m)) * 8 + r % 8;
    z = 0;
  } else {
    // workgroup -> (unit u = (K piece, M tile), column group g); unit u lives on
    // XCD u % 8 with all of its column groups
    const int xcd = blockIdx.x % 8, q = blockIdx.x / 8;
    const int u = (q / groups) * 8 + xcd;
    g = q % groups;
    if (u >= splits * tiles_m) return;
    z = u / tiles_m;
    mt = u % tiles_m;
  }
  if (g >= groups) return;  // the whole workgroup
  const int u0 = (int)((int64_t)g * units / groups), u1 = (int)((int64_t)(g + 1) * units / groups);
  const int n0 = u0 * 32, nc = (u1 - u0) * 32;
  const int M = a.M, K = a.K, m0 = mt * BMT;
  const int kt0 = z * ksteps;
  const int nk = min(K / T::KSTEP - kt0, ksteps);  // (the host never makes an empty piece)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= CW + 2) {  // weight producers: rows of the group (past its columns: a row inside it)
    const int p = wave - CW - 2;
    const unsigned char* base[T::WLOADS];
    uint32_t off[T::WLOADS];
#pragma unroll
    for (int j = 0; j < T::WLOADS; ++j) {
      const int row = (p * T::WLOADS + j) * T::RPI + lane / T::CPR;
      base[j] = (const unsigned char*)a.W + ((int64_t)n0 * K + (int64_t)kt0 * T::KSTEP) * 2;
      off[j] = (uint32_t)(((row % nc) * K + T::pos(row, lane % T::CPR) * 8) * 2);
    }
    ws2_produce<T::WLOADS, NSW, T::WSTAGE, KB>(smem + NSA * T::ASTAGE, base, off,
                                               p * T::WLOADS * 1024, nk);
    return;
  }
  if (wave >= CW) {  // activation producers: the M tile's rows (past M: row M-1), LO: then
                     // the same rows of the low part (a whole 16-row piece lies on one side)
    const int p = wave - CW;
    const unsigned char* base[T::ALOADS];
    uint32_t off[T::ALOADS];
#pragma unroll
    for (int j = 0; j < T::ALOADS; ++j) {
      const int row = (p * T::ALOADS + j) * T::RPI + lane / T::CPR;
      base[j] = (const unsigned char*)((p * T::ALOADS + j) * T::RPI < BMT ? a.A : a.A_lo) +
                ((int64_t)m0 * K + (int64_t)kt0 * T::KSTEP) * 2;
      off[j] = (uint32_t)(((min(m0 + row % BMT, M - 1) - m0) * K +
                           T::pos(row, lane % T::CPR) * 8) * 2);
    }
    ws2_produce<T::ALOADS, NSA, T::ASTAGE, KB>(smem, base, off, p * T::ALOADS * 1024, nk);
    return;
  }
  constexpr int N2 = NTM > 2 ? NTM - 2 : NTM, N4 = NTM > 4 ? NTM - 4 : N2;
  auto consume = [&](auto ntc) {
    constexpr int NTC = decltype(ntc)::value;
    ws2_consume<EPI, NTC, NTM, NSA, NSW, CW, LO, BMT, KB>(a, smem, nk, n0, m0, wave, lane, z);
  };
  switch (nc / 16) {
    case NTM: consume(std::integral_constant<int, NTM>{}); break;
    case N2: consume(std::integral_constant<int, N2>{}); break;
    default: consume(std::integral_constant<int, N4>{}); break;
  }
}

// about `target` workgroups over (K pieces x M tiles x column groups); a group holds
// NTM-4 .. NTM 16-column tiles (the consumer's shapes); false if no group count fits
template <int EPI, int NTM, int NSA, int NSW, bool LO, int BMT = 256, int CW = 4, int KB = 64>
static bool gemm_ws2_go(const GemmArgs& a, int target, int splits, hipStream_t s,
                        int* used_splits = nullptr) {
  const int units = a.N / 32;
  const int tiles_m = (a.M + BMT - 1) / BMT;
  if (a.K % (KB / 2) != 0) return false;
  const int steps = a.K / (KB / 2);
  const int ksteps = (steps + splits - 1) / splits;
  splits = (steps + ksteps - 1) / ksteps;
  const int gmin = (units + NTM / 2 - 1) / (NTM / 2);             // at most NTM tiles
  const int gmax = NTM > 4 ? units / ((NTM - 4) / 2) : units;     // at least NTM-4 tiles
  if (gmin > gmax) return false;
  const int groups = std::min(gmax, std::max(gmin, target / (tiles_m * splits)));
  const int grid = splits == 1 ? tiles_m * ((groups + 7) & ~7)
                               : 8 * ((splits * tiles_m + 7) / 8) * groups;
  if (used_splits) *used_splits = splits;
  launch_k(gemm_ws2_kernel<EPI, NTM, NSA, NSW, CW, LO, BMT, KB>, dim3(grid), dim3(64 * (CW + 4)), 0,
           s, a, units, groups, tiles_m, splits, ksteps);
  return true;
}

// x[row] += sum over splits of the partials (split order), x the fp32 residual;
// then, if u is given, u[row] = RMSNorm(x[row]) in bf16 with fp32 statistics.
// One workgroup per row; each thread keeps up to 4 chunks of 8 columns in registers.
constexpr int kResidMaxChunks = 4;
constexpr int kResidMaxSplits = 8;        // K pieces of the one-stream split projections
constexpr int kResidNormMaxSplits = 16;   // partials the reduction takes
__global__ __launch_bounds__(256) void resid_norm_kernel(const float* ws, int splits, int M, int N,
                                                         float* x, bf16_t* u, bf16_t* u_lo,
                                                         const float* g, float eps, float* usum,
                                                         int sum_ld) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int nch = N / 8;
  float v[kResidMaxChunks][8];
  f32x4_t gv[kResidMaxChunks][2];  // the chunk's RMSNorm gains, requested with its partials
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kResidMaxChunks; ++j) {
    const int c = tid + 256 * j;
    if (c >= nch) continue;
    float* xp = x + (size_t)row * N + c * 8;
    if (u != nullptr) {
      gv[j][0] = *(const f32x4_t*)(g + c * 8);
      gv[j][1] = *(const f32x4_t*)(g + c * 8 + 4);
    }
    const f32x4_t x0 = *(const f32x4_t*)xp, x1 = *(const f32x4_t*)(xp + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[j][i] = x0[i];
      v[j][4 + i] = x1[i];
    }
    // every split's partial of this chunk is requested before the sum (split order)
    f32x4_t p0[kResidNormMaxSplits], p1[kResidNormMaxSplits];
#pragma unroll
    for (int s = 0; s < kResidNormMaxSplits; ++s)
      if (s < splits) {
        const float* p = ws + ((size_t)s * M + row) * N + c * 8;
        p0[s] = *(const f32x4_t*)p;
        p1[s] = *(const f32x4_t*)(p + 4);
      }
#pragma unroll
    for (int s = 0; s < kResidNormMaxSplits; ++s)
      if (s < splits) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[j][i] += p0[s][i];
          v[j][4 + i] += p1[s][i];
        }
      }
    *(f32x4_t*)xp = f32x4_t{v[j][0], v[j][1], v[j][2], v[j][3]};
    *(f32x4_t*)(xp + 4) = f32x4_t{v[j][4], v[j][5], v[j][6], v[j][7]};
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += v[j][i] * v[j][i];
  }
  if (u == nullptr) return;
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float r = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)N + eps);
  float gs[kResidMaxChunks];  // each chunk's sum of its 8 rounded values, in order
#pragma unroll
  for (int j = 0; j < kResidMaxChunks; ++j) {
    const int c = tid + 256 * j;
    gs[j] = 0.f;
    if (c >= nch) continue;
    u32x4_t o, ol;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y0 = v[j][2 * i] * r * gv[j][i >> 1][2 * (i & 1)];
      const float y1 = v[j][2 * i + 1] * r * gv[j][i >> 1][2 * (i & 1) + 1];
      const bf16_t h0 = f32_to_bf16(y0), h1 = f32_to_bf16(y1);
      gs[j] += bf16_to_f32(h0);
      gs[j] += bf16_to_f32(h1);
      o[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      // the low part: each value's rounding error, itself rounded to bf16
      ol[i] = (uint32_t)f32_to_bf16(y0 - bf16_to_f32(h0)) |
              ((uint32_t)f32_to_bf16(y1 - bf16_to_f32(h1)) << 16);
    }
    *(u32x4_t*)(u + (size_t)row * N + c * 8) = o;
    if (u_lo) *(u32x4_t*)(u_lo + (size_t)row * N + c * 8) = ol;
  }
  if (usum == nullptr) return;
  // the sums of the rounded values per 128-column group (16 chunks on 16 consecutive
  // lanes: each chunk's 8 values in order, then a fixed tree over the lanes)
#pragma unroll
  for (int j = 0; j < kResidMaxChunks; ++j) {
    const int c = tid + 256 * j;
    // rotations by 8, 4, 2, 1 inside the 16-lane row pair the lanes as an xor tree would
    float t = gs[j];
    t += row_ror<8>(t);
    t += row_ror<4>(t);
    t += row_ror<2>(t);
    t += row_ror<1>(t);
    if (c < nch && (c & 15) == 0) usum[(size_t)(c >> 4) * sum_ld + row] = t;
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
            glu_act(a.glu, Cs[r][blk * 32 + cc], Cs[r][blk * 32 + 16 + cc]);
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

// ---------------------------------------------------------------------------
// INT4 group-128 weights ("Rebuilding Kshipra Around Memory", section 2), the
// prefill projections: C = sum over groups g of s[g][n] * (A_g q_g^T) (scales
// stored [K/128][N]). Each K step is one group of 128; its 64 column scales ride
// in the same DMA ring as the operands. The A tile (BM rows of 256 bytes, 16-byte chunk kc
// of row r at position kc ^ (r % 16)) and the packed W tile (BN rows of 64 bytes
// of codes, chunk kc at kc ^ ((r / 2) % 4)) stream into an NS-stage LDS ring by
// DMA; once per step the workgroup widens the W codes to bf16 (exact: integers
// in [-8, 7]) into a padded LDS tile; the matrix cores accumulate the group's
// products into a temporary, and s (fp16, widened) scales it into the fp32 sum,
// so no product q * s is ever rounded to bf16.
// ---------------------------------------------------------------------------
template <int BM, int BN, int NS, int WGM, int WGN>
struct GemmW4Tile {
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int MT = WM / 16, NT = WN / 16;
  static_assert(WGM * WGN == 4 && MT >= 1 && NT >= 1, "four wavefronts");
  // a stage: A tile, W codes, one 1 KiB slot whose first BN * 2 bytes are the group's
  // scales for the tile's columns (the scale DMA fills the whole slot), and one 1 KiB
  // slot whose first BM * 4 bytes are the group's activation sums of the tile's rows
  static constexpr int ASTAGE = BM * 256, WSTAGE = BN * 64, STAGE = ASTAGE + WSTAGE + 2048;
  static constexpr int ALOADS = BM / 4 / 4, WLOADS = BN / 16 / 4;  // DMA loads per wavefront
  static constexpr int LOADS = ALOADS + WLOADS;  // wavefront 0 adds the scale load
  // one scale DMA (16 bytes per lane) covers the tile's BN columns: lane % (BN / 8)
  // picks a 16-byte piece, repeated across the 1 KiB slot
  static_assert(BN % 64 == 0 && BN <= 512 && BM == 64,
                "one scale DMA covers the tile's columns, one 4-byte sum DMA its rows");
  static constexpr int LDS = NS * STAGE;
};

// The codes are unpacked in registers: each lane reads the 8 codes of its B
// fragment as one 32-bit word and unpacks them as in the decode GEMV: u = q + 8
// (sign bit flipped), a pair of nibbles masked into a bf16 pair with the exponent
// of 128 is (128 + u_k, 128 + u_k+4), so the fragment holds the pairs (k0, k4),
// (k1, k5), (k2, k6), (k3, k7); the A fragment is permuted to the same order (the
// product over a K slice does not depend on the order of k). Per group,
// P = sum_k a (128 + u) and S = sum_k a give sum_k a q = P - 136 S, scaled by the
// column's fp16 scale in fp32. S is one more MFMA against ones per 16-row tile and
// 32-wide K slice (a third of the matrix-core work at 64 x 128 tiles, repeated by
// every wavefront along N), or, with SUMS, read from the per-(group, row) sums that
// the kernel producing the activations wrote (a_sum).
template <int EPI, int BM, int BN, int NS, int WGM, int WGN, bool SUMS>
__global__ __launch_bounds__(256) void gemm_w4_kernel(GemmArgs a, int tiles_m, int tiles,
                                                      int ksteps) {
  using G = GemmW4Tile<BM, BN, NS, WGM, WGN>;
  constexpr int MT = G::MT, NT = G::NT, LOADS = G::LOADS;
  static_assert(LOADS * (NS - 1) <= 63 && NS - 2 <= 6 && G::WLOADS >= 1, "shape");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[G::LDS];

  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int slot = blockIdx.x % (kXcds * per_xcd);
  const int z = blockIdx.x / (kXcds * per_xcd);
  const int t = (slot % kXcds) * per_xcd + slot / kXcds;
  if (t >= tiles) return;
  const int m0 = (t % tiles_m) * BM, n0 = (t / tiles_m) * BN;
  const int M = a.M, K = a.K, ngk = K / 128;
  const int kt0 = z * ksteps;
  const int nk = min(ngk - kt0, ksteps);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const uint8_t* Wq = (const uint8_t*)a.W;
  const __half* Sc = (const __half*)(Wq + (size_t)a.N * K / 2);  // [K/128][N]

  // DMA sources: A rows (4 per load, 16 chunks of 16 bytes each), W code rows (16 per load)
  const unsigned char* srcA[G::ALOADS];
  const unsigned char* srcW[G::WLOADS];
#pragma unroll
  for (int j = 0; j < G::ALOADS; ++j) {
    const int row = (wave * G::ALOADS + j) * 4 + (lane >> 4);
    const int kc = (lane & 15) ^ (row & 15);
    srcA[j] = (const unsigned char*)((const bf16_t*)a.A + (int64_t)min(m0 + row, M - 1) * K +
                                     (int64_t)kt0 * 128) + kc * 16;
  }
#pragma unroll
  for (int j = 0; j < G::WLOADS; ++j) {
    const int row = (wave * G::WLOADS + j) * 16 + (lane >> 2);
    const int kc = (lane & 3) ^ ((row >> 1) & 3);
    srcW[j] = Wq + (int64_t)(n0 + row) * (K / 2) + (int64_t)kt0 * 64 + kc * 16;
  }
  // stage kt goes to ring slot kt % NS. Past the last stage the DMA re-loads that
  // stage's data into the slot just freed (no later step reads it): every step
  // then issues the same loads, so every wait below has one constant depth.
  // scale source: group (kt0 + kd), columns n0 .. n0+BN-1 (lane % (BN/8) picks a 16-byte piece)
  const unsigned char* srcS =
      (const unsigned char*)(Sc + (size_t)kt0 * a.N + n0) + (lane % (BN / 8)) * 16;
  auto issue = [&](int kt) {
    unsigned char* st = smem + (kt % NS) * G::STAGE;
    const int kd = kt < nk ? kt : nk - 1;
#pragma unroll
    for (int j = 0; j < G::ALOADS; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void*)(srcA[j] + (size_t)kd * 256),
          (__attribute__((address_space(3))) void*)(st + (wave * G::ALOADS + j) * 1024), 16, 0,
          0);
#pragma unroll
    for (int j = 0; j < G::WLOADS; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void*)(srcW[j] + (size_t)kd * 64),
          (__attribute__((address_space(3))) void*)(st + G::ASTAGE + (wave * G::WLOADS + j) * 1024),
          16, 0, 0);
    if (wave == 0)
      __builtin_amdgcn_global_load_lds(
          (const void*)(srcS + (size_t)kd * a.N * 2),
          (__attribute__((address_space(3))) void*)(st + G::ASTAGE + G::WSTAGE), 16, 0, 0);
    // SUMS: the group's activation sums of the tile's BM rows, 4 bytes per lane, into
    // the sum slot (rows past M read the padded table, never stored)
    if (SUMS && wave == 1)
      __builtin_amdgcn_global_load_lds(
          (const void*)(a.a_sum + (size_t)(kt0 + kd) * a.sum_ld + m0 + lane),
          (__attribute__((address_space(3))) void*)(st + G::ASTAGE + G::WSTAGE + 1024), 4, 0, 0);
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (nk <= 0) {
    gemm_epilogue<EPI, MT, NT, G::WM, G::WN>(a, acc, m0, n0, z, wm, wn, lane);
    return;
  }
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0) issue(s0);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt landed: at most NS-2 younger stages in flight (wavefront 0, which also
    // loads the scales, waits for a little more than it must)
    wait_vmcnt_steps<LOADS>(NS - 2);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // this step's group scales for the lane's output columns (from the stage)
    const unsigned char* st = smem + (kt % NS) * G::STAGE;
    float sc[NT];
#pragma unroll
    for (int ni = 0; ni < NT; ++ni)
      sc[ni] = __half2float(
          *(const __half*)(st + G::ASTAGE + G::WSTAGE + (wn * G::WN + ni * 16 + (lane & 15)) * 2));
    f32x4_t tmp[MT][NT], tsum[MT];
    if constexpr (SUMS) {
      // the group's activation sums of the accumulator rows 4 (lane / 16) .. +3 of each
      // 16-row tile (from the stage)
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
        tsum[mi] = *(const f32x4_t*)(st + G::ASTAGE + G::WSTAGE + 1024 +
                                     (wm * G::WM + mi * 16 + 4 * (lane >> 4)) * 4);
    }
    issue(kt + NS - 1);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if constexpr (!SUMS) tsum[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NT; ++j) tmp[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const bf16x8_t ones = __builtin_bit_cast(
        bf16x8_t, u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // B: the 8 codes of K positions ks*32 + 8*(lane/16) .. +7 of column lane%16
      bf16x8_t bf[NT];
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) {
        const int r = wn * G::WN + ni * 16 + (lane & 15);
        const uint32_t v = *(const uint32_t*)(st + G::ASTAGE + r * 64 + ((ks ^ ((r >> 1) & 3)) << 4) +
                                              4 * (lane >> 4));
        bf[ni] = __builtin_bit_cast(bf16x8_t, u32x4_t{w4_pair_bits(v), w4_pair_bits(v >> 4),
                                                      w4_pair_bits(v >> 8), w4_pair_bits(v >> 12)});
      }
      const int kc = ks * 4 + (lane >> 4);
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const int r = wm * G::WM + mi * 16 + (lane & 15);
        const u32x4_t n = *(const u32x4_t*)(st + r * 256 + ((kc ^ (r & 15)) << 4));
        // (x0, x1), (x2, x3), (x4, x5), (x6, x7) -> (x0, x4), (x1, x5), (x2, x6), (x3, x7)
        const bf16x8_t af = __builtin_bit_cast(
            bf16x8_t, u32x4_t{__builtin_amdgcn_perm(n[2], n[0], 0x05040100u),
                              __builtin_amdgcn_perm(n[2], n[0], 0x07060302u),
                              __builtin_amdgcn_perm(n[3], n[1], 0x05040100u),
                              __builtin_amdgcn_perm(n[3], n[1], 0x07060302u)});
#pragma unroll
        for (int ni = 0; ni < NT; ++ni)
          tmp[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[ni], tmp[mi][ni], 0, 0, 0);
        if constexpr (!SUMS)
          tsum[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, ones, tsum[mi], 0, 0, 0);
      }
    }
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) acc[mi][ni] += sc[ni] * (tmp[mi][ni] - 136.f * tsum[mi]);
  }
  gemm_epilogue<EPI, MT, NT, G::WM, G::WN>(a, acc, m0, n0, z, wm, wn, lane);
}

template <int EPI, int BM, int BN, int NS, int WGM, int WGN>
static void gemm_w4_go(const GemmArgs& a, int splits, int ksteps, hipStream_t s) {
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles = tiles_m * (a.N / BN);
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  if (a.a_sum)
    launch_k(gemm_w4_kernel<EPI, BM, BN, NS, WGM, WGN, true>, dim3(kXcds * per_xcd * splits),
             dim3(256), 0, s, a, tiles_m, tiles, ksteps);
  else
    launch_k(gemm_w4_kernel<EPI, BM, BN, NS, WGM, WGN, false>, dim3(kXcds * per_xcd * splits),
             dim3(256), 0, s, a, tiles_m, tiles, ksteps);
}

// q/k/v split-K reduction: sums the partials of each RoPE pair (split order) and
// applies the same epilogue as the unsplit kernel (rotation, query buffer, paged
// K/V). One thread per pair (grid: pair blocks x rows); the rotation, the block id
// and every split's partial are requested together before the sum.
constexpr int kQkvReduceMaxSplits = kResidMaxSplits;
// S splits as a template argument: every load is unconditional, so the sum waits
// for its own loads only (a runtime split count made each load a guarded one)
template <int S>
__global__ __launch_bounds__(256) void qkv_reduce_kernel(GemmArgs a) {
  const int row = blockIdx.y;
  const int cp = blockIdx.x * 256 + threadIdx.x;
  if (cp >= a.N / 2) return;
  const QkvPre pre = epi_qkv_prefetch_all(a.ctx, row, 2 * cp);
  float2 v[S];
#pragma unroll
  for (int s = 0; s < S; ++s) v[s] = *(const float2*)(a.ws + ((size_t)s * a.M + row) * a.N + 2 * cp);
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    lo += v[s].x;
    hi += v[s].y;
  }
  epi_qkv_store<bf16_t>(a.ctx, row, 2 * cp, pre, lo, hi);
}

static hipError_t launch_qkv_reduce(const GemmArgs& a, int splits, hipStream_t s) {
  static_assert(kQkvReduceMaxSplits == 8, "one instantiation per split count");
  const dim3 grid((a.N / 2 + 255) / 256, a.M), block(256);
  switch (splits) {
    case 1: launch_k(qkv_reduce_kernel<1>, grid, block, 0, s, a); break;
    case 2: launch_k(qkv_reduce_kernel<2>, grid, block, 0, s, a); break;
    case 3: launch_k(qkv_reduce_kernel<3>, grid, block, 0, s, a); break;
    case 4: launch_k(qkv_reduce_kernel<4>, grid, block, 0, s, a); break;
    case 5: launch_k(qkv_reduce_kernel<5>, grid, block, 0, s, a); break;
    case 6: launch_k(qkv_reduce_kernel<6>, grid, block, 0, s, a); break;
    case 7: launch_k(qkv_reduce_kernel<7>, grid, block, 0, s, a); break;
    case 8: launch_k(qkv_reduce_kernel<8>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int EPI, int BM, int BN, int BK, int NS, int WGM = 2, int WGN = 2, bool LO = false>
static void gemm_bf16_go(const GemmArgs& a, int splits, int ksteps, hipStream_t s) {
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles = tiles_m * (a.N / BN);
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  launch_k(gemm_bf16_kernel<EPI, BM, BN, BK, NS, WGM, WGN, LO>, dim3(kXcds * per_xcd * splits),
           dim3(64 * WGM * WGN), 0, s, a, tiles_m, tiles, ksteps);
}

// INT4 projections: 64 x 128 tiles, four wavefronts along N (64 x 32 wavefront
// tiles). Every INT4 projection has N divisible by 128 (each K is a multiple of
// 128 and N is one of those sizes or twice one). Measured at the Llama-3-8B shape
// with 512 rows (cold weights): gate/up 240 us against 309 us for 64 x 64 tiles
// whose codes were widened to bf16 in LDS (the activation tile is re-read once
// per column tile, so wider tiles cut the dominant traffic), down 117 us against
// 143 us, O 37 us against 46 us. Residual projections split the groups when
// fewer than about 384 workgroups would run (at least 4 groups per split) and
// reduce like the 16-bit path.
template <int EPI>
static void gemm_w4_pick(const GemmArgs& a, int splits, int ksteps, hipStream_t s) {
  gemm_w4_go<EPI, 64, 128, 3, 1, 4>(a, splits, ksteps, s);
}
static hipError_t gemm_w4(const GemmArgs& a, hipStream_t s) {
  if (a.K % 128 != 0 || a.N % 128 != 0) return hipErrorInvalidValue;
  // the sum table's rows: every 64-row tile whole (the DMA reads rows past M)
  if (a.a_sum && (a.sum_ld % 4 != 0 || a.sum_ld < (a.M + 63) / 64 * 64))
    return hipErrorInvalidValue;
  const int ngk = a.K / 128;
  if (a.epi == EPI_SWIGLU) {
    if (a.glu) gemm_w4_pick<EPI_GEGLU_K>(a, 1, ngk, s);
    else gemm_w4_pick<EPI_SWIGLU>(a, 1, ngk, s);
    return hipGetLastError();
  }
  if (a.epi == EPI_QKV) {
    gemm_w4_pick<EPI_QKV>(a, 1, ngk, s);
    return hipGetLastError();
  }
  if (a.epi != EPI_RESID) return hipErrorInvalidValue;
  if (a.ws == nullptr || (size_t)a.M * a.N > a.ws_elems) return hipErrorInvalidValue;
  if (a.N % 8 != 0 || a.N / 8 > 256 * kResidMaxChunks) return hipErrorInvalidValue;
  const int tiles = ((a.M + 63) / 64) * (a.N / 128);
  int splits = std::max(1, std::min(kResidMaxSplits, (384 + tiles - 1) / tiles));
  while (splits > 1 && ngk / splits < 4) --splits;
  while (splits > 1 && (size_t)splits * a.M * a.N > a.ws_elems) --splits;
  const int ksteps = (ngk + splits - 1) / splits;
  splits = (ngk + ksteps - 1) / ksteps;
  gemm_w4_pick<EPI_PARTIAL>(a, splits, ksteps, s);
  launch_k(resid_norm_kernel, dim3(a.M), dim3(256), 0, s, (const float*)a.ws, splits, a.M, a.N,
           (float*)a.C, (bf16_t*)a.norm_out, (bf16_t*)a.norm_out_lo, a.norm_g, a.eps,
           a.norm_sum, a.sum_ld);
  return hipGetLastError();
}

// Tile shapes, measured with the weights cold in HBM (rotated over more than the
// last-level cache between launches):
//  gated projection (SwiGLU or GeGLU epilogue): at most 64 rows -> 64 x 128 tiles
//    when that makes at least 128 workgroups (64 x 17920 x 1536: 17.7 us against
//    20.3 us for 64 x 64), else 64 x 32 tiles with 4 wavefronts along M (63 x 8192 x
//    1024: 6.2 us against 10.1 us for 64 x 128); up to 128 rows -> 128 x 64 in a
//    3-stage ring; 129 to 256 rows -> the two-stream kernel (separate activation and
//    weight rings): one 256-row M tile with groups of up to 96 columns (256 x 17920 x
//    1536: 0.7 us per layer faster than two 128-row tiles), with the activations' low
//    part two 128-row M tiles with groups of up to 160 columns (36 us against 44 us for
//    one 256-row tile, whose doubled activation re-reads were 7x the weight bytes); more
//    rows -> 256 x 128 with 8
//    wavefronts (4 x 2 grid of 64 x 64 wavefront tiles), 32-deep steps (256 x 17920 x
//    1536: 34 us against 37 us for 128 x 64 and 39 us for 64 x 64), or 256 x 256 (64 x
//    128 wavefront tiles) when that still makes about 192 workgroups: the activation
//    tile is re-read once per column tile (512 x 32768 x 2048: 81 us against 98 us for
//    256 x 128 and 118 us for 128 x 128), in two stages of 64 K (128-byte rows: 77.7 us
//    against 80.9 us for three of 32 K; 256 x 128 or 128 x 256 in three stages of 64 K:
//    85.6, 87.8 us); with a low part three stages of 32 K;
//  residual and q/k/v projections: 64 x 64 tiles, 64-deep steps, 3-stage ring; K is
//    split into pieces of about 36 steps and into enough splits for about 192
//    workgroups (at least 4 steps per split, at most 8 splits): 256 x 2048 x 1536
//    q/k/v 12.0 us and 256 x 1536 x 1536 O 11.1 us with 2 splits, 256 x 1536 x 8960
//    down 21.4 us with 4 (times include the reduction kernel); 129 to 256 rows with
//    K >= 4096 (down): the two-stream kernel split into up to 16 K pieces with
//    128-column groups (256 x 1536 x 8960: 18.1 us against 23.8 us for 64 x 64 tiles in
//    4 pieces, without the reduction). From 512 rows with at
//    least 128 K steps: 256 x 64 tiles with 8 wavefronts and K in pieces of 64 steps
//    (512 x 2048 x 16384: 57 us against 75 us for 64 x 64). At most 64 rows: 64 x 32
//    tiles with 4 wavefronts along M, splits for about 384 workgroups (63 x 1024 x
//    2048: 7.9 us against 8.3 us; 63 x 1024 x 4096: 8.9 against 9.5).
// Split projections reduce their fp32 partials in split order in a second kernel:
// the residual add (+ next RMSNorm), or RoPE + K/V write for q/k/v.
// LO: the activations carry a low part (A_lo); the same shapes, with one ring stage
// less where the doubled activation rows would not fit the LDS
// the two-stream gated projection: one 256-row M tile with up to 96-column groups and
// eight consumer wavefronts of 32 rows (two per SIMD: 29.2 us against 29.5 us with four
// of 64 rows), stages of 64 K (128-byte rows: every DMA request a whole cache line, 29.7
// -> 24.9 us against stages of 32 K) in 3-stage activation and 4-stage weight rings; or
// with the activations' low part (twice the activation rows) two 128-row M tiles with up
// to 160-column groups
template <int EPI, bool LO>
static bool ws2_gated(const GemmArgs& a, hipStream_t s) {
  if constexpr (LO)
    return gemm_ws2_go<EPI, 10, 4, 8, true, 128>(a, 256, 1, s);
  else
    return gemm_ws2_go<EPI, 6, 3, 4, false, 256, 8, 128>(a, 256, 1, s);
}

template <int EPI, bool LO>
static void gated_go(const GemmArgs& a, hipStream_t s) {
  // up to 64 rows, at least 128 column tiles of 128 (the Qwen-shaped gated projection of
  // a 64-token chunk): the two-stream kernel with 64-row tiles keeps more weight stages
  // in flight than the one-stream 64 x 128 tiles (64-token prefill 2.25 -> 2.18 ms); at
  // 64 tiles (the action expert) it is slower (expert iteration 0.89 -> 0.92 ms)
  if (!LO && a.M <= 64 && a.N % 128 == 0 && a.N / 128 >= 128 &&
      gemm_ws2_go<EPI, 6, 3, 4, false, 64, 4, 128>(a, 256, 1, s))
    return;
  if (a.M <= 64 && a.N % 128 == 0 && a.N / 128 >= 128)
    gemm_bf16_go<EPI, 64, 128, 64, 4, 2, 2, LO>(a, 1, a.K / 64, s);
  else if (a.M <= 64)
    gemm_bf16_go<EPI, 64, 32, 64, 4, 4, 1, LO>(a, 1, a.K / 64, s);
  else if (a.M > 128 && a.M <= 256 && a.N % 32 == 0 && ws2_gated<EPI, LO>(a, s))
    return;
  else if (!LO && a.M > 128 && a.N % 256 == 0 && ((a.M + 255) / 256) * (a.N / 256) >= 192)
    gemm_bf16_go<EPI, 256, 256, 64, 2, 4, 2, false>(a, 1, a.K / 64, s);
  else if (a.M > 128 && a.N % 256 == 0 && ((a.M + 255) / 256) * (a.N / 256) >= 192)
    gemm_bf16_go<EPI, 256, 256, 32, 3, 4, 2, LO>(a, 1, a.K / 32, s);
  else if (a.M > 128 && a.N % 128 == 0)
    gemm_bf16_go<EPI, 256, 128, 32, LO ? 3 : 4, 4, 2, LO>(a, 1, a.K / 32, s);
  else
    gemm_bf16_go<EPI, 128, 64, 64, 3, 2, 2, LO>(a, 1, a.K / 64, s);
}

// the q/k/v projection: RoPE + K/V write in the epilogue, or split-K partials and
// the q/k/v reduction
template <bool LO>
static hipError_t qkv_go(const GemmArgs& a, bool tall, bool skinny, int splits, int ksteps,
                         int ksteps_all, hipStream_t s) {
  if (splits == 1) {
    if (skinny) gemm_bf16_go<EPI_QKV, 64, 32, 64, 3, 4, 1, LO>(a, 1, ksteps_all, s);
    else gemm_bf16_go<EPI_QKV, 64, 64, 64, 3, 2, 2, LO>(a, 1, ksteps_all, s);
  } else {
    if (tall && !LO) gemm_bf16_go<EPI_PARTIAL, 256, 64, 64, 3, 4, 2>(a, splits, ksteps, s);
    else if (skinny) gemm_bf16_go<EPI_PARTIAL, 64, 32, 64, 3, 4, 1, LO>(a, splits, ksteps, s);
    else gemm_bf16_go<EPI_PARTIAL, 64, 64, 64, 3, 2, 2, LO>(a, splits, ksteps, s);
    if (hipError_t e = launch_qkv_reduce(a, splits, s); e != hipSuccess) return e;
  }
  return hipGetLastError();
}

static hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.K % 64 != 0 || a.N % 64 != 0 || a.M < 1) return hipErrorInvalidValue;
  if (a.wf == WF_INT4) return gemm_w4(a, s);
  const bool lo = a.A_lo != nullptr;
  if (a.epi == EPI_SWIGLU) {
    if (a.glu) {
      if (lo) gated_go<EPI_GEGLU_K, true>(a, s);
      else gated_go<EPI_GEGLU_K, false>(a, s);
    } else {
      if (lo) gated_go<EPI_SWIGLU, true>(a, s);
      else gated_go<EPI_SWIGLU, false>(a, s);
    }
    return hipGetLastError();
  }
  if (a.epi != EPI_QKV && a.epi != EPI_RESID) return hipErrorInvalidValue;
  const int ksteps_all = a.K / 64;
  // 256 x 64 tiles, 8 wavefronts (with a low part the doubled rows would not fit the LDS)
  const bool tall = a.M >= 512 && ksteps_all >= 128 && !lo;
  const bool skinny = !tall && a.M <= 64;               // 64 x 32 tiles, 4 wavefronts along M
  const int tiles = tall ? ((a.M + 255) / 256) * (a.N / 64)
                         : skinny ? a.N / 32 : ((a.M + 63) / 64) * (a.N / 64);
  const int target = skinny ? 384 : 192;
  int splits = tall ? (ksteps_all + 63) / 64
                    : std::max((target + tiles - 1) / tiles, (ksteps_all + 35) / 36);
  splits = std::max(1, std::min(kResidMaxSplits, splits));
  while (splits > 1 && ksteps_all / splits < 4) --splits;
  while (splits > 1 && (size_t)splits * a.M * a.N > a.ws_elems) --splits;
  if (a.ws == nullptr || (size_t)a.M * a.N > a.ws_elems) splits = 1;
  const int ksteps = (ksteps_all + splits - 1) / splits;
  splits = (ksteps_all + ksteps - 1) / ksteps;
  if (a.epi == EPI_QKV)
    return lo ? qkv_go<true>(a, tall, skinny, splits, ksteps, ksteps_all, s)
              : qkv_go<false>(a, tall, skinny, splits, ksteps, ksteps_all, s);
  // residual projection: always through the partial buffer and the reduction kernel
  if (a.ws == nullptr || (size_t)a.M * a.N > a.ws_elems) return hipErrorInvalidValue;
  if (a.N % 8 != 0 || a.N / 8 > 256 * kResidMaxChunks) return hipErrorInvalidValue;
  // 129 to 256 rows with a long K (the down projection): the two-stream kernel with
  // 128-column groups, K in up to 16 pieces, stages of 64 K (128-byte rows: 18.6 ->
  // 16.5 us against stages of 32 K)
  if (a.M > 128 && a.M <= 256 && ksteps_all >= 64 && a.N % 128 == 0 && !lo) {
    const int steps = a.K / 32;
    int sp = kResidNormMaxSplits;
    while (sp > 1 && (size_t)sp * a.M * a.N > a.ws_elems) --sp;
    const int ks = (steps + sp - 1) / sp;
    sp = (steps + ks - 1) / ks;
    if (gemm_ws2_go<EPI_PARTIAL, 8, 3, 3, false, 256, 4, 128>(a, 192, sp, s, &sp)) {
      launch_k(resid_norm_kernel, dim3(a.M), dim3(256), 0, s, (const float*)a.ws, sp, a.M, a.N,
               (float*)a.C, (bf16_t*)a.norm_out, (bf16_t*)a.norm_out_lo, a.norm_g, a.eps,
           a.norm_sum, a.sum_ld);
      return hipGetLastError();
    }
  }
  // up to 64 rows with K of 8192 or more (the Qwen-shaped down projection of a 64-token
  // chunk): the two-stream kernel with 64-row tiles, K in pieces of at least 4 stages
  // (64-token prefill 2.18 -> 2.12 ms); shorter K (the action expert's projections)
  // stays on the one-stream split tiles, which were faster there
  if (!lo && a.M <= 64 && ksteps_all >= 128 && a.N % 128 == 0) {
    int sp = std::min(kResidNormMaxSplits, (a.K / 64) / 4);
    while (sp > 1 && (size_t)sp * a.M * a.N > a.ws_elems) --sp;
    if (gemm_ws2_go<EPI_PARTIAL, 8, 3, 4, false, 64, 4, 128>(a, 256, sp, s, &sp)) {
      launch_k(resid_norm_kernel, dim3(a.M), dim3(256), 0, s, (const float*)a.ws, sp, a.M, a.N,
               (float*)a.C, (bf16_t*)a.norm_out, (bf16_t*)a.norm_out_lo, a.norm_g, a.eps,
               a.norm_sum, a.sum_ld);
      return hipGetLastError();
    }
  }
  if (tall) gemm_bf16_go<EPI_PARTIAL, 256, 64, 64, 3, 4, 2>(a, splits, ksteps, s);
  else if (skinny && lo) gemm_bf16_go<EPI_PARTIAL, 64, 32, 64, 3, 4, 1, true>(a, splits, ksteps, s);
  else if (skinny) gemm_bf16_go<EPI_PARTIAL, 64, 32, 64, 3, 4, 1>(a, splits, ksteps, s);
  else if (lo) gemm_bf16_go<EPI_PARTIAL, 64, 64, 64, 3, 2, 2, true>(a, splits, ksteps, s);
  else gemm_bf16_go<EPI_PARTIAL, 64, 64, 64, 3>(a, splits, ksteps, s);
  launch_k(resid_norm_kernel, dim3(a.M), dim3(256), 0, s, (const float*)a.ws, splits, a.M, a.N,
           (float*)a.C, (bf16_t*)a.norm_out, (bf16_t*)a.norm_out_lo, a.norm_g, a.eps,
           a.norm_sum, a.sum_ld);
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

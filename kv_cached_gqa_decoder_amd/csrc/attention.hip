// GQA attention over the block-paged KV cache (prefill and decode).
//
// softmax(q k^T / sqrt(d)) v over every visible key ("CSR ...", III-A), with
// the keys of the current chunk causal and every other resident key visible
// ("Rebuilding Kshipra Around Memory", section 4) -- or, for the action chunk
// of a pi0-style expert ("Running VLAs at Real-time Speed", section 2), every
// key of the chunk visible to every row of it -- computed as an online
// softmax (m, l, o) over KV blocks read in place from the pool (same section).
//
// bf16 path (matrix cores). Query rows are (token, q head of the group) pairs,
// so the g heads sharing a KV head consume each K/V block together and a block
// is read once per KV-head group rather than once per query head. A 16-row
// tile is a set of MFMA query columns. Per 32-key step (two blocks):
//   S^T = K Q^T        v_mfma_f32_16x16x32_bf16, A = 16 keys x 32 dims (K rows),
//                      B = Q^T held in registers for the whole loop; the
//                      accumulator gives each lane 4 keys of one query.
//   online softmax     per query column, in base 2 (scores times log2 e / sqrt(d)).
//   O^T += V^T P^T     A = V^T (the pool stores V transposed inside a block, so
//                      consecutive keys of one dimension are contiguous),
//                      B = P^T, which is exactly the lane's own probabilities.
// Two kernels:
//   decode (<= 16 query rows): 4 wavefronts share one row tile and take
//     interleaved block pairs straight from memory (one pair prefetched); their
//     partial (m, l, o) are merged through LDS.
//   rows (prefill): 4 wavefronts of 2 row tiles (8 of 1 at d = 256), so a
//     workgroup covers 128 rows; every block pair goes through a 3-4 stage
//     LDS ring filled by direct-to-LDS DMA and is read by all rows of the
//     workgroup. Its softmax keeps a lazy reference max and per-lane row sums,
//     and its ring layout lets every operand read be one 16-byte load (see the
//     layout and softmax comments below). Workgroups are numbered so that all
//     row tiles of one (KV head, key split) run on one XCD and stream the same
//     blocks through its L2.
// The resident blocks are split over workgroups (split-K). Each workgroup
// writes its partial (m, l, o); a second kernel merges the splits in split
// order (deterministic) -- or, for one-token decode with few splits, the output
// projection merges them as it reads its input. Merging inside the first
// kernel would need an agent-scope release/acquire per workgroup, which on
// this chip writes back and invalidates the whole L2 of the workgroup's XCD.
#include <algorithm>

#include "attn_decode.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace vla {

// ---------------------------------------------------------------------------
// rows kernel (prefill)
// ---------------------------------------------------------------------------
// Two shapes. Long caches: 128 rows per workgroup, each block pair read once per
// 128 rows: at d <= 128 4 wavefronts of 2 row tiles in a 3-stage ring (48 KB), three
// workgroups per CU whose per-pair barriers need not line up (a 512-token chunk over
// 120,000 keys: 29.8 ms of attention against 30.8 ms with a 4-stage ring and two
// per CU, and 32.3 ms for one workgroup of 8 wavefronts x 2 tiles), at d = 256 8
// wavefronts of one tile. Short caches (few pairs per workgroup): 4 wavefronts of
// one tile, 64 rows, for more workgroups.
template <int D, bool SHORT>
struct RowCfg {
  static constexpr int WAVES = SHORT || D <= 128 ? 4 : 8;
  static constexpr int QT = SHORT || D > 128 ? 1 : 2;  // 16-row tiles per wavefront
  static constexpr int ROWS = WAVES * QT * 16;       // rows per workgroup
  static constexpr int NS = 3;                       // ring stages (block pairs)
  static constexpr int BLK = 16 * D * 2;             // one block of K (or V) of one KV head
  static constexpr int STAGE = 4 * BLK;              // K0 K1 V0 V1
  static constexpr int LDS = NS * STAGE;
  static constexpr int CPR = D / 8;                  // 16-byte chunks per K row
  static constexpr int LOADS = STAGE / 1024 / WAVES; // 1 KB DMA instructions per wavefront per stage
  static_assert(LOADS >= 1 && STAGE % (1024 * WAVES) == 0, "stage split");
};

// Ring layout of one block pair (K0 K1 V0 V1, one BLK each), chosen so that every
// LDS read of the loop is one 16-byte load at a fixed offset and every 16 lanes
// that read together cover 16 distinct 16-byte bank slots.
//
// K, chunk-major: the 16-byte chunk c (dims 8c..8c+7) of key r of block w sits
// at slot c*16 + krow_slot(w, r) (bits 2 and 3 of r swapped, bit 3 flipped for
// block 1). The S MFMA of half h (0, 1) takes as A-row i the key
// 8*((i>>2)&1) + 4h + (i&3) of block i>>3; its slot is then i ^ 8h, and the
// accumulator leaves lane (cq, jq) the scores of keys 8*(jq&1) + 4h + e of
// block jq>>1: over both halves, 8 consecutive keys of one block.
__device__ __forceinline__ int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}
// V^T, row-major as in the pool (dimension vr: 16 keys = two 16-byte halves);
// the halves of a row trade places when bit 2 xor bit 3 of the row is set.
__device__ __forceinline__ int vhalf_swz(int vr) { return ((vr >> 2) ^ (vr >> 3)) & 1; }

// Reference maximum of the rows kernel. The base-2 running max m of a query
// column moves only when a score exceeds it by more than kRefSlack, so most
// steps skip the column max and the rescale; the probabilities 2^(s*sl2 - m)
// then stay below 2^kRefSlack (exact in fp32 and bf16 range). m starts at a
// finite floor so that no step needs a test for infinities: a column with no
// visible key yet keeps m at the floor, a floor-to-score move rescales by
// exp2(-huge) = 0, and fully masked lanes give 2^-inf = 0.
constexpr float kRefSlack = 8.f;
constexpr float kRefFloor = -1e30f;

__device__ __forceinline__ float max8(const f32x4_t& x, const f32x4_t& y) {
  // fmaximum: no NaN can occur here (finite scores, -inf for masked keys), and it
  // maps to v_maximum3_f32 without operand canonicalisation
  const float a = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]), x[2]);
  const float b = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[3], y[0]), y[1]);
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b),
                                       __builtin_elementwise_maximum(y[2], y[3]));
}

// sum of the two bf16 values of a packed pair added to acc (v_dot2c_f32_bf16)
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
}

// Online softmax of one block pair for a wavefront's QT row tiles. s0/s1: the
// raw scores of halves 0 and 1 (lane (cq, jq): keys 8*(jq&1) + 4h + e of block
// b + (jq>>1)). Leaves the bf16 probabilities as the P^T MFMA operands; l holds
// per-lane partial sums (the 4 lanes of a column are added at the end).
template <int D, int QT>
__device__ __forceinline__ void rows_softmax(const AttnArgs& a, f32x4_t (&s0)[QT],
                                             f32x4_t (&s1)[QT], float (&m)[QT],
                                             float (&thr)[QT], float (&l)[QT],
                                             f32x4_t (&o)[QT][D / 16], bf16x8_t (&pf)[QT],
                                             const int (&tq)[QT], int b, bool has1, bool masked,
                                             int jq, float sl2, float isl2) {
  if (masked) {
    // visible: slot < ntok, and outside the causal region or at most the row's token
    const int w = jq >> 1;
    const int nt0 = block_ntok_s(a, b);
    const int nt1 = has1 ? block_ntok_s(a, b + 1) : 0;
    const int nt = w ? nt1 : nt0;
    const bool open = b + w < a.cb0 || !a.causal;
    const int k0 = 8 * (jq & 1);
    const int ck = (b + w - a.cb0) * a.g.bt - a.cslot0 + k0;  // causal index of key k0
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool v0 = (k0 + e < nt) & (open | (ck + e <= tq[qt]));
        const bool v1 = (k0 + 4 + e < nt) & (open | (ck + 4 + e <= tq[qt]));
        s0[qt][e] = v0 ? s0[qt][e] : -INFINITY;
        s1[qt][e] = v1 ? s1[qt][e] : -INFINITY;
      }
  }
  float mx[QT];
  bool need = false;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mx[qt] = max8(s0[qt], s1[qt]);
    need = need || mx[qt] > thr[qt];
  }
  if (__any(need)) {  // wave-uniform: move every column's reference to its max
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float m_new = fmaxf(m[qt], col_max4(mx[qt]) * sl2);
      const float alpha = __builtin_amdgcn_exp2f(m[qt] - m_new);
      m[qt] = m_new;
      thr[qt] = (m_new + kRefSlack) * isl2;
      l[qt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[qt][dt] *= alpha;
    }
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float nm = -m[qt];
    u32x4_t pw;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      pw[e] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s0[qt][2 * e], sl2, nm)),
                          __builtin_amdgcn_exp2f(fmaf(s0[qt][2 * e + 1], sl2, nm)));
      pw[2 + e] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s1[qt][2 * e], sl2, nm)),
                              __builtin_amdgcn_exp2f(fmaf(s1[qt][2 * e + 1], sl2, nm)));
    }
    // the running sum adds the rounded probabilities the P*V product uses
#pragma unroll
    for (int e = 0; e < 4; ++e) l[qt] = add_bf16x2(pw[e], l[qt]);
    pf[qt] = __builtin_bit_cast(bf16x8_t, pw);
  }
}

// one block pair for a wavefront's QT row tiles: S^T = K Q^T for every tile (each
// K fragment read once from LDS), the softmax of every tile, then O^T += V^T P^T
// (each V fragment read once). koff / voff: the lane's K slot of half 0 and V^T
// slot of dt = 0 inside a stage (byte offsets). masked: some key of the pair may
// be invisible; only the masking itself is conditional, so both cases share one
// instruction stream.
template <int D, int QT>
__device__ __forceinline__ void rows_step(const AttnArgs& a, const unsigned char* st,
                                          const bf16x8_t (&qf)[QT][D / 32], const int (&tq)[QT],
                                          float (&m)[QT], float (&thr)[QT], float (&l)[QT],
                                          f32x4_t (&o)[QT][D / 16], int b, bool has1,
                                          bool masked, int koff, int voff, int jq, float sl2,
                                          float isl2) {
  f32x4_t s0[QT], s1[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    s0[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    s1[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const unsigned char* k0p = st + koff;
  const unsigned char* k1p = st + (koff ^ (8 * 16));  // half 1: slot i ^ 8
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    // chunk 4*ds + jq: 4 chunks of 16 slots further per ds
    const bf16x8_t k0 = *(const bf16x8_t*)(k0p + ds * 1024);
    const bf16x8_t k1 = *(const bf16x8_t*)(k1p + ds * 1024);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      s0[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[qt][ds], s0[qt], 0, 0, 0);
      s1[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[qt][ds], s1[qt], 0, 0, 0);
    }
  }
  bf16x8_t pf[QT];
  rows_softmax<D, QT>(a, s0, s1, m, thr, l, o, pf, tq, b, has1, masked, jq, sl2, isl2);
  const unsigned char* vp = st + voff;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    // V^T row dt*16 + cq: keys 8*(jq&1)..+7 of block jq>>1, the order of P^T
    const bf16x8_t vf = *(const bf16x8_t*)(vp + dt * 512);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
      o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qt], o[qt][dt], 0, 0, 0);
  }
}

template <int D, bool SHORT>
__global__ __launch_bounds__((RowCfg<D, SHORT>::WAVES * 64)) void attn_rows_kernel(AttnArgs a, int rgroups,
                                                                    int units) {
  using C = RowCfg<D, SHORT>;
  constexpr int QT = C::QT, NS = C::NS, ROWS = C::ROWS;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS];

  // XCD-aware numbering: workgroup i runs on XCD i % 8; unit u = (kvh, split)
  // lives on XCD u % 8 with all of its row tiles
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int u = (slot / rgroups) * 8 + xcd;
  const int rg = slot % rgroups;
  if (u >= units) return;
  const int splits = a.splits;
  const int kvh = u / splits, split = u % splits;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int jq = lane >> 4, cq = lane & 15;
  const int grp = a.hq / a.g.hkv;
  const int R = a.n * grp;
  const float sl2 = a.scale * kLog2e, isl2 = 1.f / sl2;

  // this wavefront's query tiles: rows rg*ROWS + wave*QT*16 + qt*16 + cq
  bf16x8_t qf[QT][D / 32];
  int tq[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = rg * ROWS + (wave * QT + qt) * 16 + cq;
    const bool ok = r < R;
    tq[qt] = ok ? r / grp : 0;
    const int h = kvh * grp + (ok ? r % grp : 0);
    const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)tq[qt] * a.hq + h) * D;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const u32x4_t v = ok ? *(const u32x4_t*)(qrow + ds * 32 + 8 * jq) : u32x4_t{0, 0, 0, 0};
      qf[qt][ds] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // blocks of this split; past the workgroup's last causal key nothing is visible
  const int bps = (a.nlb + splits - 1) / splits;
  const int b_begin = split * bps;
  int b_end = min(a.nlb, b_begin + bps);
  if (a.causal) {
    const int rlast = min(R, rg * ROWS + ROWS) - 1;
    b_end = min(b_end, a.cb0 + (rlast / grp + a.cslot0) / a.g.bt + 1);
  }
  const int np = b_end > b_begin ? (b_end - b_begin + 1) / 2 : 0;

  float m[QT], thr[QT], l[QT];
  f32x4_t o[QT][D / 16];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = kRefFloor;
    thr[qt] = (kRefFloor + kRefSlack) * isl2;
    l[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[qt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  if (np > 0) {
    const unsigned char* kp = (const unsigned char*)a.kpool;
    const unsigned char* vp = (const unsigned char*)a.vpool;
    // DMA: each wavefront moves LOADS 1 KB pieces of a stage; lane `lane` of a
    // piece fills slot part*64 + lane of its block, so its source offset inside
    // the block is fixed for the whole loop (the block base is wave-uniform)
    uint32_t doff[C::LOADS];
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      const int q = wave * C::LOADS + j;
      const int which = q / (C::BLK / 1024), part = q % (C::BLK / 1024);
      const int ls = part * 64 + lane;  // 16-byte slot inside the block
      if (which < 2) {
        // 16-byte piece ls>>4 of key r: 64-byte chunk (ls>>4)/4 holds the block's 16
        // keys in turn, so one 1 KB piece of the stage is one contiguous chunk
        const int r = swap23((ls & 15) ^ (which << 3));
        doff[j] = (ls >> 6) * 1024 + r * 64 + ((ls >> 4) & 3) * 16;
      } else {
        const int vr = ls >> 1;
        doff[j] = vr * 32 + (((ls & 1) ^ vhalf_swz(vr)) << 4);
      }
    }
    // the lane's read slots: K of half 0 (block cq>>3, chunk jq, slot cq), and
    // V^T of dt = 0 (block jq>>1, row cq)
    const int koff = (cq >> 3) * C::BLK + (jq * 16 + cq) * 16;
    const int voff = (2 + (jq >> 1)) * C::BLK + (2 * cq + ((jq & 1) ^ vhalf_swz(cq))) * 16;
    // block bases: one layer's K (V) blocks of this KV head lie bstride bytes apart
    const unsigned char* kb = kp + a.g.kidx(a.layer, 0, kvh, 0, 0) * 2;
    const unsigned char* vb = vp + a.g.vidx(a.layer, 0, kvh, 0, 0) * 2;
    const uint32_t bstride = (uint32_t)a.g.hkv * a.g.bt * D * 2;
    // physical blocks of pair p; past the last pair the DMA re-loads it (every
    // step then issues the same loads and every wait has one depth)
    auto ids = [&](int p, int& pb0, int& pb1) {
      const int pd = p < np ? p : np - 1;
      const int b = b_begin + 2 * pd;
      pb0 = uniform_ld(a.blk_table, b);
      pb1 = uniform_ld(a.blk_table, b + 1 < b_end ? b + 1 : b);
    };
    // pair p (< np) has a key that may be invisible: a missing or partial block,
    // or a block in the causal region
    // (both table entries read unconditionally, from indices inside the table, so
    // that no branch waits on a load)
    auto pair_masked = [&](int p) {
      const int b = b_begin + 2 * p;
      const int b1 = min(b + 1, a.nlb - 1);
      const int t0 = uniform_ld(a.blk_ntok, b), t1 = uniform_ld(a.blk_ntok, b1);
      const int n0 = b == a.nlb - 1 ? a.last_ntok : t0;
      const int n1 = b1 == a.nlb - 1 ? a.last_ntok : t1;
      bool mk = (b + 1 >= b_end) | (n0 != a.g.bt) | (n1 != a.g.bt);
      if (a.causal) mk = mk | (b + 1 >= a.cb0);
      return mk;
    };
    // stage p -> ring slot p % NS
    auto issue = [&](int p, int pb0, int pb1) {
      unsigned char* st = smem + (p % NS) * C::STAGE;
#pragma unroll
      for (int j = 0; j < C::LOADS; ++j) {
        const int q = wave * C::LOADS + j;            // 1 KB piece of the stage
        const int which = q / (C::BLK / 1024);        // 0 K0, 1 K1, 2 V0, 3 V1
        const int part = q % (C::BLK / 1024);
        const uint32_t pb = (which & 1) ? pb1 : pb0;
        const unsigned char* base = (which < 2 ? kb : vb) + (size_t)pb * bstride;
        __builtin_amdgcn_global_load_lds(
            (const void*)(base + doff[j]),
            (__attribute__((address_space(3))) void*)(st + which * C::BLK + part * 1024), 16, 0,
            0);
      }
    };
    int pb0, pb1;
#pragma unroll
    for (int p0 = 0; p0 < NS - 1; ++p0) {
      ids(p0, pb0, pb1);
      issue(p0, pb0, pb1);
    }
    // the scalars a step needs (the blocks its DMA fetches, whether it masks) are
    // requested one step ahead, so their latency is hidden behind a whole step
    ids(NS - 1, pb0, pb1);
    bool mk_next = pair_masked(0);

    for (int p = 0; p < np; ++p) {
      wait_vmcnt_steps<C::LOADS>(NS - 2);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      issue(p + NS - 1, pb0, pb1);
      const unsigned char* st = smem + (p % NS) * C::STAGE;
      const int b = b_begin + 2 * p;
      const bool has1 = b + 1 < b_end;
      const bool masked = mk_next;

      rows_step<D, QT>(a, st, qf, tq, m, thr, l, o, b, has1, masked, koff, voff, jq, sl2, isl2);
      // after this step's LDS reads, so that their waits do not include these loads
      __builtin_amdgcn_sched_barrier(0);
      ids(p + NS, pb0, pb1);
      mk_next = pair_masked(min(p + 1, np - 1));
    }
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) l[qt] = col_sum4(l[qt]);

  // results: the output rows directly, or this split's partial (m, l, o)
  const int tile = kvh * rgroups + rg;
  const size_t unit = (size_t)tile * splits + split;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int c = (wave * QT + qt) * 16 + cq;  // row inside the workgroup
    const int r = rg * ROWS + c;
    if (splits == 1) {
      if (r < R) {
        const float inv = l[qt] > 0.f ? 1.f / l[qt] : 0.f;
        const size_t ro = ((size_t)(r / grp) * a.hq + kvh * grp + r % grp) * D;
        bf16_t* orow = (bf16_t*)a.out + ro;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          u32x2_t w;
          w[0] = pack_bf16x2(o[qt][dt][0] * inv, o[qt][dt][1] * inv);
          w[1] = pack_bf16x2(o[qt][dt][2] * inv, o[qt][dt][3] * inv);
          *(u32x2_t*)(orow + dt * 16 + 4 * jq) = w;
          if (a.out_lo) {
            u32x2_t wl;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const float y0 = o[qt][dt][2 * h] * inv, y1 = o[qt][dt][2 * h + 1] * inv;
              wl[h] = pack_bf16x2(y0 - bf16_to_f32((bf16_t)(w[h] & 0xffffu)),
                                  y1 - bf16_to_f32((bf16_t)(w[h] >> 16)));
            }
            *(u32x2_t*)((bf16_t*)a.out_lo + ro + dt * 16 + 4 * jq) = wl;
          }
        }
      }
    } else {
      float* po = a.part_o + (unit * ROWS + c) * D;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *(f32x4_t*)(po + dt * 16 + 4 * jq) = o[qt][dt];
      if (jq == 0) {
        a.part_ml[unit * 2 * ROWS + c] = m[qt];
        a.part_ml[unit * 2 * ROWS + ROWS + c] = l[qt];
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnArgs a, int rgroups) {
  attn_decode_body<D>(a, rgroups, blockIdx.x, blockIdx.y, blockIdx.z, a.layer);
}

// Combines the splits of query rows of one (KV head, row group) tile: with
// per-split running max m_s (base 2), sum l_s and unnormalised o_s,
// o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, M = max_s m_s. D/64 dims per
// lane; splits go in chunks (32 splits, 16 at d = 256 where a split carries 4
// values per lane) whose loads are all issued together (one memory round trip
// per chunk), with a running max across chunks (the sums are rescaled when it
// rises). WAVES = 1: one wavefront per row, no LDS, no barrier. WAVES = 4 (many
// splits, few rows: long-context decode): the 4 wavefronts of a workgroup take
// consecutive quarters of one row's splits and are combined through LDS in
// wavefront order. Splits are added in order, so the result is deterministic.
constexpr int kMaxSplits = 128;

template <int D, int ROWS, int WAVES>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int rgroups) {
  constexpr int V = D / 64;  // dims per lane
  constexpr int kMergeChunk = V >= 4 ? 16 : 32;
  static_assert(V >= 1 && D % 64 == 0 && ROWS % 4 == 0 && (WAVES == 1 || WAVES == 4), "shape");
  __shared__ float comb[WAVES == 4 ? 4 : 1][64][V + 2];
  const int tile = blockIdx.x;  // kvh * rgroups + rg
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = WAVES == 1 ? (int)blockIdx.y * 4 + wave : (int)blockIdx.y;  // row inside the tile
  const int rg = tile % rgroups, kvh = tile / rgroups;
  const int grp = a.hq / a.g.hkv;
  const int rr = rg * ROWS + c;
  if (rr >= a.n * grp) return;  // uniform over the row's wavefronts (all of a workgroup at WAVES 4)
  const int splits = a.splits;
  const int per = (splits + WAVES - 1) / WAVES;
  const int sb = WAVES == 1 ? 0 : min(splits, wave * per);
  const int se = WAVES == 1 ? splits : min(splits, sb + per);
  const size_t u0 = (size_t)tile * splits;

  float M = -INFINITY, L = 0.f;
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
  for (int s0 = sb; s0 < se; s0 += kMergeChunk) {
    float mv[kMergeChunk], lv[kMergeChunk], ov[kMergeChunk][V];
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) {
      const int sp = s0 + j;
      mv[j] = -INFINITY;
      lv[j] = 0.f;
#pragma unroll
      for (int v = 0; v < V; ++v) ov[j][v] = 0.f;
      if (sp < se) {  // wave-uniform
        const size_t u = u0 + sp;
        mv[j] = a.part_ml[u * 2 * ROWS + c];
        lv[j] = a.part_ml[u * 2 * ROWS + ROWS + c];
        const float* po = a.part_o + (u * ROWS + c) * D + lane * V;
        if constexpr (V == 4) {
          const f32x4_t q = *(const f32x4_t*)po;
#pragma unroll
          for (int v = 0; v < 4; ++v) ov[j][v] = q[v];
        } else if constexpr (V == 2) {
          const float2 q = *(const float2*)po;
          ov[j][0] = q.x;
          ov[j][1] = q.y;
        } else {
          ov[j][0] = po[0];
        }
      }
    }
    float Mc = M;
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) Mc = fmaxf(Mc, mv[j]);
    if (Mc != -INFINITY) {
      const float sc = M == -INFINITY ? 0.f : exp2f(M - Mc);  // earlier chunks to the new max
      L *= sc;
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] *= sc;
#pragma unroll
      for (int j = 0; j < kMergeChunk; ++j) {
        const float w = mv[j] == -INFINITY ? 0.f : exp2f(mv[j] - Mc);
        L += w * lv[j];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] += w * ov[j][v];
      }
      M = Mc;
    }
  }
  if constexpr (WAVES == 4) {
    comb[wave][lane][0] = M;
    comb[wave][lane][1] = L;
#pragma unroll
    for (int v = 0; v < V; ++v) comb[wave][lane][2 + v] = acc[v];
    __syncthreads();
    if (wave != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mt = fmaxf(Mt, comb[w][lane][0]);
    L = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = 0.f;
    if (Mt != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = comb[w][lane][0];
        const float sc = mw == -INFINITY ? 0.f : exp2f(mw - Mt);
        L += sc * comb[w][lane][1];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] += sc * comb[w][lane][2 + v];
      }
    }
    M = Mt;
  }
  const size_t ro = ((size_t)(rr / grp) * a.hq + kvh * grp + rr % grp) * D + lane * V;
  bf16_t* orow = (bf16_t*)a.out + ro;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const float y = M != -INFINITY && L > 0.f ? acc[v] / L : 0.f;
    const bf16_t h = f32_to_bf16(y);
    orow[v] = h;
    if (a.out_lo) ((bf16_t*)a.out_lo)[ro + v] = f32_to_bf16(y - bf16_to_f32(h));
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one wavefront per (token, q head); scores for every logical key
// in LDS, then softmax and the weighted sum of V. For small fp32 caches only.
// ---------------------------------------------------------------------------
constexpr int kF32MaxKeys = 2048;

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  const int last_ntok = a.last_ntok;
  __shared__ float sc[4][kF32MaxKeys];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int unit = blockIdx.x * 4 + wave;
  if (unit >= a.n * a.hq) return;
  const int t = unit / a.hq, h = unit % a.hq;
  const int grp = a.hq / a.g.hkv;
  const int kvh = h / grp;
  const int d = a.g.d, bt = a.g.bt;
  const float* q = (const float*)a.q + ((size_t)t * a.hq + h) * d;
  const float* kp = (const float*)a.kpool;
  const float* vp = (const float*)a.vpool;
  const int nkeys = a.nlb * bt;
  float mx = -INFINITY;
  for (int i = lane; i < nkeys; i += 64) {
    const int b = i / bt, s = i % bt;
    const int nt = (b == a.nlb - 1) ? last_ntok : a.blk_ntok[b];
    float v = -INFINITY;
    if (key_visible(a, b, s, nt, t)) {
      const int pb = a.blk_table[b];
      float dot = 0.f;
      for (int j = 0; j < d; ++j) dot += q[j] * kp[a.g.kidx(a.layer, pb, kvh, s, j)];
      v = dot * a.scale;
    }
    sc[wave][i] = v;
    mx = fmaxf(mx, v);
  }
  mx = wave_max(mx);
  float sum = 0.f;
  for (int i = lane; i < nkeys; i += 64) {
    const float p = sc[wave][i] == -INFINITY ? 0.f : __expf(sc[wave][i] - mx);
    sc[wave][i] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  __builtin_amdgcn_wave_barrier();
  float* orow = (float*)a.out + ((size_t)t * a.hq + h) * d;
  for (int j = lane; j < d; j += 64) {
    float acc = 0.f;
    for (int i = 0; i < nkeys; ++i) {
      const float p = sc[wave][i];
      if (p != 0.f) acc += p * vp[a.g.vidx(a.layer, a.blk_table[i / bt], kvh, i % bt, j)];
    }
    orow[j] = acc / sum;
  }
}

template <int D, int ROWS>
static void attn_merge_go(const AttnArgs& a, int rgroups, hipStream_t s) {
  if (a.splits <= 1) return;
  // more than 32 splits (long-context decode): 4 wavefronts per row
  if (a.splits > 32)
    launch_k(attn_merge_kernel<D, ROWS, 4>, dim3(a.g.hkv * rgroups, ROWS), dim3(256), 0, s, a,
             rgroups);
  else
    launch_k(attn_merge_kernel<D, ROWS, 1>, dim3(a.g.hkv * rgroups, ROWS / 4), dim3(256), 0, s, a,
             rgroups);
}

template <int D, bool SHORT>
static void attn_rows_go(const AttnArgs& a, int rgroups, hipStream_t s) {
  using C = RowCfg<D, SHORT>;
  const int units = a.g.hkv * a.splits;
  const int grid = (units + 7) / 8 * rgroups * 8;
  launch_k(attn_rows_kernel<D, SHORT>, dim3(grid), dim3(C::WAVES * 64), 0, s, a, rgroups, units);
  attn_merge_go<D, C::ROWS>(a, rgroups, s);
}

// shape: 0 decode, 1 rows (short cache), 2 rows (long cache)
template <int D>
static void attn_bf16_go(const AttnArgs& a, int shape, int rgroups, hipStream_t s, bool fold) {
  if (shape == 0) {
    launch_k(attn_decode_kernel<D>, dim3(a.splits, rgroups, a.g.hkv), dim3(kAttnWaves * 64), 0, s,
             a, rgroups);
    if (!fold) attn_merge_go<D, 16>(a, rgroups, s);
  } else if (shape == 1) {
    attn_rows_go<D, true>(a, rgroups, s);
  } else {
    attn_rows_go<D, false>(a, rgroups, s);
  }
}

template <int D>
static int rows_per_group(int shape) {
  return shape == 0 ? 16 : shape == 1 ? RowCfg<D, true>::ROWS : RowCfg<D, false>::ROWS;
}

hipError_t launch_attention(const AttnArgs& args, int dt, hipStream_t s, int* fold_splits) {
  if (fold_splits) *fold_splits = 0;
  if (args.nlb <= 0 || args.n <= 0) return hipErrorInvalidValue;
  if (dt == DT_F32) {
    if (args.nlb * args.g.bt > kF32MaxKeys) return hipErrorInvalidValue;
    launch_k(attn_f32_kernel, dim3((args.n * args.hq + 3) / 4), dim3(256), 0, s, args);
    return hipGetLastError();
  }
  AttnArgs a = args;
  const int d = a.g.d;
  if (d != 64 && d != 128 && d != 256) return hipErrorInvalidValue;
  if (a.g.bt != 16) return hipErrorInvalidValue;
  const int R = a.n * (a.hq / a.g.hkv);
  const bool keysplit = R <= 16;
  // short caches (<= 256 blocks), and few query rows (<= 512 per KV head) at any cache
  // length, take the 64-row workgroups: a 64-token chunk over 8,128 cached keys (384
  // rows per KV head) makes the whole prefill 3.6% faster than with the 256-row tiles;
  // for a 512-token chunk over 120,000 keys (2,048 rows) the attention would take 1.7x
  // as long
  const int shape = keysplit ? 0 : (a.nlb <= 256 || R <= 512) ? 1 : 2;
  const int rows = d == 64 ? rows_per_group<64>(shape)
                           : d == 128 ? rows_per_group<128>(shape) : rows_per_group<256>(shape);
  const int rgroups = (R + rows - 1) / rows;
  const int base = a.g.hkv * rgroups;
  // split count: at least 8 blocks (4 pairs) per split; about one resident round
  // of workgroups (decode: 2 per CU, 512 in all; rows: 1 per CU, 256 in all), so
  // that workgroups run long and few partials are merged; within the
  // partial-buffer capacity
  int splits = (a.nlb + 7) / 8;
  // one-token decode over a short cache: splits of 4 blocks while the output projection
  // can still merge them as it reads its input (1,300 keys: 16 splits, decode step 1.080
  // -> 1.067 ms)
  if (keysplit && a.n == 1)
    splits = std::max(splits, std::min(kFoldMaxSplits, (a.nlb + 3) / 4));
  // (rows kernel: 12 wavefronts per CU, 3 long-cache workgroups of 4, or 8: 2 short-cache
  // workgroups, 1 long-cache workgroup of 8 at d = 256)
  const int resident = shape == 2 ? (d > 128 ? 256 : 768) : 512;
  // few row tiles over a short cache: splits of 4 blocks for more workgroups (the
  // 63-token action chunk over 575 keys: 9 splits instead of 5, expert iteration
  // 0.916 -> 0.892 ms; 2-block splits 0.908)
  if (shape == 1 && base * splits < 128) splits = std::max(splits, (a.nlb + 3) / 4);
  splits = std::min(splits, std::max(1, resident / base));
  splits = std::min(splits, keysplit ? kMaxSplitsKey : kMaxSplitsRow);
  static_assert(kMaxSplitsKey <= kMaxSplits && kMaxSplitsRow <= kMaxSplits, "merge capacity");
  splits = std::min(splits, std::max(1, a.part_rows / (base * rows)));
  splits = std::max(splits, 1);
  const int bps = (a.nlb + splits - 1) / splits;
  a.splits = (a.nlb + bps - 1) / bps;
  if (a.splits > 1 &&
      (a.part_o == nullptr || a.part_ml == nullptr || (size_t)base * rows * a.splits > (size_t)a.part_rows))
    return hipErrorInvalidValue;
  // one-token decode with few splits: the consumer merges the partials
  const bool fold = fold_splits && shape == 0 && a.n == 1 && a.splits > 1 &&
                    a.splits <= kFoldMaxSplits && a.hq <= kFoldMaxHeads;
  if (fold) *fold_splits = a.splits;
  switch (d) {
    case 64: attn_bf16_go<64>(a, shape, rgroups, s, fold); break;
    case 128: attn_bf16_go<128>(a, shape, rgroups, s, fold); break;
    default: attn_bf16_go<256>(a, shape, rgroups, s, fold); break;
  }
  return hipGetLastError();
}

}  // namespace vla

// Flash-style attention backward, bf16 I/O, fp32 statistics and accumulation.
//
// The method is the backward of the xtrain evolution page's fused kernel
// (infrastructure-phase table, row T14): the scores are recomputed from Q, K
// and the saved log-sum-exp, and the per-row scalar D = sum(dO * O)
// simplifies the softmax Jacobian to dS = P * (dP - D).  Grouped KV heads
// follow row T15: each KV head's dK/dV is the sum over its G query heads,
// done here in registers in ascending group order, with no atomics, so the
// result is bitwise reproducible.
//
// Kernels, on one stream:
//  1. preprocess: Dlt[row] = sum_d dO[row,d] * O[row,d]            (HBM bound)
//     The bf16 dQ kernel forms the same values itself (bit for bit) and
//     stores them, so the bf16 backward runs dQ first and then dK/dV, with
//     no preprocess launch.
//  2. dK/dV: one workgroup per 128 keys of one KV head, 8 waves: four
//     32-key slices, each served by a pair of waves with split roles so that
//     each wave fits in half a SIMD's registers and two waves share a SIMD:
//       P-wave : S = Q K^T, P = 2^(S*scale*log2e - LSE*log2e)  -> P to LDS,
//                dV^T += dO^T P
//       dS-wave: dP = dO V^T, dS = P (dP - Dlt) with P from LDS,
//                dK^T += Q^T dS
//     (lane = key column; K or V of the slice stays in registers as the MFMA
//     B operand).  The dS-wave runs one query tile behind the P-wave, so the
//     VALU work of one wave meets MFMA work of the other on their shared SIMD;
//     Q/dO tiles arrive two steps ahead in three LDS buffers.  The walk
//     covers every query tile of every query head of the group, in ascending
//     head order, summing in registers.  Shapes with few KV tiles (short cross-attention KV) split
//     the query range into fixed chunks that write fp32 partials, summed
//     afterwards in chunk order by a reduction kernel.
//  3. dQ: each wave owns 32 query rows, keeps their Q and dO in registers
//     and walks the 64-key K/V tiles of its head:
//        S^T = K Q^T, dP^T = V dO^T        (lane = query column)
//        dQ^T += K^T dS^T
//     One workgroup of 4 waves per 128 query rows of one head; two
//     workgroups share a CU.
// Q/dO and K/V tiles are staged in LDS once each, in a layout (SwzTile)
// whose row reads and transposed reads are both free of bank conflicts;
// every transposed MFMA operand (dO^T, Q^T, K^T) is read from that copy with
// ds_read_b64_tr_b16.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace mattn {

// Split count for the dK/dV walk.  One dK/dV workgroup fills a CU (its
// LDS), and MI355X has 256 CUs, so the grid runs in rounds of 256
// workgroups; a chunk of n_qt / ns query tiles is a workgroup's walk.  The
// split minimises rounds x walk length, plus a charge of about a third of a
// step per split for the partials' reduction, with at most 512 workgroups
// (which bounds the partials to 64 MiB at D = 128) and at least 8 query
// tiles per chunk.  Depends only on the sizes.
int bwd_nsplit(int B, int Hkv, int Sq, int Skv) {
  if (B <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0) return 1;
  constexpr long long kSlots = 256, kMaxWgs = 2 * kSlots;
  const long long n_kt = (Skv + BWD_BN - 1) / BWD_BN;
  const long long wgs = (long long)B * Hkv * n_kt;
  if (wgs >= kMaxWgs) return 1;
  const long long n_qt = (Sq + BWD_BMQ - 1) / BWD_BMQ;
  const long long cap = n_qt / 8;  // keep at least 8 query tiles per chunk
  auto cost = [&](long long ns) {   // in tenths of a step
    const long long rounds = (wgs * ns + kSlots - 1) / kSlots;
    return 10 * rounds * ((n_qt + ns - 1) / ns) + 3 * ns;
  };
  long long best = 1;
  for (long long ns = 2; ns <= cap && wgs * ns <= kMaxWgs; ++ns)
    if (cost(ns) < cost(best)) best = ns;
  return (int)best;
}

namespace {

constexpr int THREADS = 256;

// ----------------------------------------------------------------------------
// 1. preprocess
//
// Dlt of one row in bf16: two half-rows, each the fp32 fma chain below over
// the columns 16s + 8h .. 16s + 8h + 7 (s ascending) that one lane of the dQ
// kernel holds, then the two halves added.  The dQ kernel forms Dlt with the
// same steps (it already holds dO in that layout), so both give the same
// bits and either may feed the dK/dV kernel.
__device__ __forceinline__ float dlt_half_row_step(bf16x8 dout, bf16x8 o, float acc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)dout[e], (float)o[e], acc);
  return acc;
}

template <int D>
__global__ __launch_bounds__(THREADS)
void bwd_pre_bf16_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                         float* __restrict__ dlt, long long rows) {
  // Two adjacent lanes per row, one per half.
  const long long row = ((long long)blockIdx.x * THREADS + threadIdx.x) >> 1;
  const int h = threadIdx.x & 1;
  float acc = 0.f;
  if (row < rows) {
    const bf16* po = O + row * D + 8 * h;
    const bf16* pd = dO + row * D + 8 * h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      acc = dlt_half_row_step(*reinterpret_cast<const bf16x8*>(pd + 16 * s),
                              *reinterpret_cast<const bf16x8*>(po + 16 * s), acc);
  }
  const float tot = acc + __shfl_xor(acc, 1);
  if (h == 0 && row < rows) dlt[row] = tot;
}

template <typename T, int D>
__global__ __launch_bounds__(THREADS)
void bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO, float* __restrict__ dlt,
                    long long rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  constexpr int RPB = THREADS / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float s = 0.f;
  if (row < rows) {
    const T* po = O + row * D + c * 8;
    const T* pd = dO + row * D + c * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)pd[e] * (float)po[e];
  }
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (c == 0 && row < rows) dlt[row] = s;
}

// ----------------------------------------------------------------------------
// 2. dK/dV
constexpr int DKDV_THREADS = 512;  // 4 key slices x 2 roles

// Direct global -> LDS copy of one query tile for the dK/dV walk: BWD_BMQ rows
// of Q and of dO in the SwzTile layout (swizzle applied on the global side,
// as in DqKvCopy), then the tile's BWD_BMQ log-sum-exp and Dlt values.  Rows
// past Sq load as zeros: their P is then finite and their dO, dP, Dlt and dS
// are zero, so they add nothing.
// A query tile's LSE and Dlt values (64 each, 4 bytes per lane): wave 0
// copies the LSE values, wave 1 the Dlt values (w0 is wave-uniform, and each
// branch names its destination, so the copies keep their LDS alias scope).
__device__ __forceinline__ void dkdv_copy_stats(const Buf& lse, const Buf& dlt, char* buf, int w0,
                                                int lane, int lse_off, int dlt_off) {
  if (w0 == 0) ld4_to_lds(lse, lane * 4, buf + lse_off);
  else if (w0 == 64) ld4_to_lds(dlt, lane * 4, buf + dlt_off);
}

template <int D>
struct DkdvCopy {
  static constexpr int P = SwzTile<D>::P;
  static constexpr int SLOTS_PER_ROW = P / 8;
  static constexpr int TILE_SLOTS = BWD_BMQ * SLOTS_PER_ROW;  // per tensor
  static constexpr int ROUNDS = 2 * TILE_SLOTS / DKDV_THREADS;
  static constexpr int TILE_ELEMS = TILE_SLOTS * 8;             // bf16 per tensor
  static constexpr int LSE_OFF = 2 * TILE_SLOTS * 16;           // bytes
  static constexpr int DLT_OFF = LSE_OFF + BWD_BMQ * 4;
  static constexpr int BUF_BYTES = DLT_OFF + BWD_BMQ * 4;
  static_assert(2 * TILE_SLOTS % DKDV_THREADS == 0 && TILE_SLOTS % 64 == 0, "whole rounds");
  static_assert(BWD_BMQ == 64, "one 4-byte copy per lane for LSE and Dlt");
  uint32_t off[ROUNDS];
  int w0;  // first slot of this wave in round 0 (scalar)
  __device__ __forceinline__ void init(int tid) {
    w0 = __builtin_amdgcn_readfirstlane(tid & ~63);
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int q = r * DKDV_THREADS + tid;
      const int qq = q % TILE_SLOTS;
      const int row = qq / SLOTS_PER_ROW, pos = qq - row * SLOTS_PER_ROW;
      const int ch = pos ^ ((row >> 2) & 3);
      off[r] = pos < D / 8 ? (uint32_t)(row * D + ch * 8) * 2 : 0x80000000u;
    }
  }
  // Descriptors start at the tile's first row and end at Sq.
  __device__ __forceinline__ void load(const Buf& q, const Buf& dout, const Buf& lse,
                                       const Buf& dlt, char* buf, int lane) const {
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int q0 = r * DKDV_THREADS + w0;
      ld16_to_lds(q0 < TILE_SLOTS ? q : dout, off[r], buf + q0 * 16);
    }
    dkdv_copy_stats(lse, dlt, buf, w0, lane, LSE_OFF, DLT_OFF);
  }
};

// D = 128: the Q and dO tiles in the GrpTile128 layout, two groups of four
// rows per wave and tile (no padding written), then the same LSE and Dlt
// copies.
template <>
struct DkdvCopy<128> {
  static constexpr int TILE_ELEMS = GrpTile128::bytes(BWD_BMQ) / 2;  // bf16 per tensor
  static constexpr int LSE_OFF = 2 * TILE_ELEMS * 2;                 // bytes
  static constexpr int DLT_OFF = LSE_OFF + BWD_BMQ * 4;
  static constexpr int BUF_BYTES = DLT_OFF + BWD_BMQ * 4;
  static_assert(BWD_BMQ == 64, "one 4-byte copy per lane for LSE and Dlt");
  GrpCopy<BWD_BMQ, DKDV_THREADS / 64> g;
  int w0;
  __device__ __forceinline__ void init(int tid) {
    w0 = __builtin_amdgcn_readfirstlane(tid & ~63);
    g.init(w0 >> 6, tid & 63);
  }
  __device__ __forceinline__ void load(const Buf& q, const Buf& dout, const Buf& lse,
                                       const Buf& dlt, char* buf, int lane) const {
    g.load(q, buf);
    g.load(dout, buf + TILE_ELEMS * 2);
    dkdv_copy_stats(lse, dlt, buf, w0, lane, LSE_OFF, DLT_OFF);
  }
};

// One workgroup per 128 keys of one KV head (or per chunk of the query range
// for short KV), 8 waves: four 32-key slices, each served by a P-wave and a
// dS-wave on the same SIMD.  The walk goes over every query tile of every
// query head of the group; tile it arrives by direct copies two steps ahead
// into buffer it % 3 (each buffer its own LDS object, so reads never wait for
// copies in flight to the others).  One barrier per step:
//   P-wave : S = Q K^T, P = 2^(S*scale*log2e - LSE*log2e) -> P (fp16) to LDS
//            | barrier |  dV^T += dO^T P
//   dS-wave: dK^T += Q(it-1)^T dS(it-1), dP = dO V^T
//            | barrier |  dS = P (dP - Dlt)
// The P hand-off is double-buffered by step parity, so a P-wave may run into
// the next step while its dS-wave still reads the previous P.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(DKDV_THREADS)
void bwd_dkdv_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, const bf16* __restrict__ dO,
                     const float* __restrict__ LSE, const float* __restrict__ DLT,
                     bf16* __restrict__ dK, bf16* __restrict__ dV, float* __restrict__ part,
                     int Hq, int G, int Sq, int Skv, float scale, float c, int n_kt,
                     int nsplit, int q_chunk) {
  constexpr int BMQ = BWD_BMQ;            // query rows per step (two 32-row sub-blocks)
  constexpr int NSUB = BMQ / 32;
  using SW = std::conditional_t<D == 128, GrpTile128, SwzTile<D>>;
  using Copy = DkdvCopy<D>;
  __shared__ __attribute__((aligned(16))) char QT0[Copy::BUF_BYTES];
  __shared__ __attribute__((aligned(16))) char QT1[Copy::BUF_BYTES];
  __shared__ __attribute__((aligned(16))) char QT2[Copy::BUF_BYTES];
  // P handed from each P-wave to its dS-wave, by step parity, as fp16:
  // [parity][slice][sub-block][half][lane][8 fp16] (16 bytes per lane, so
  // a wave's 16-byte accesses cover all banks once).  fp16 rather than bf16:
  // the same bytes with three more mantissa bits, and the dS-wave multiplies
  // it in without widening it first (v_fma_mix_f32).
  constexpr int PEX_PAR = 4 * NSUB * 64 * 16;
  __shared__ __attribute__((aligned(16))) bf16 Pex[2 * PEX_PAR];
  auto QTbuf = [&](auto b) __attribute__((always_inline)) -> char* {
    constexpr int i = decltype(b)::value % 3;
    if constexpr (i == 0) return QT0; else if constexpr (i == 1) return QT1; else return QT2;
  };
  auto Qs = [](char* buf) __attribute__((always_inline)) { return reinterpret_cast<const bf16*>(buf); };
  auto dOs = [](char* buf) __attribute__((always_inline)) {
    return reinterpret_cast<const bf16*>(buf) + Copy::TILE_ELEMS;
  };
  auto lse_s = [](char* buf) __attribute__((always_inline)) {
    return reinterpret_cast<const float*>(buf + Copy::LSE_OFF);
  };
  auto dlt_s = [](char* buf) __attribute__((always_inline)) {
    return reinterpret_cast<const float*>(buf + Copy::DLT_OFF);
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int slice = wave & 3;
  const bool pwave = wave < 4;
  const int Hkv = Hq / G;

  // XCD-aware order: consecutive workgroup ids go round-robin to the 8 XCDs,
  // so remap them so each XCD keeps a fixed set of KV heads, whose key tiles
  // then read the same Q/dO tiles through one L2.  Causal walks shrink with
  // the key tile (key tile kt sees the queries from kt*128 on), so there each
  // XCD takes its heads' key tiles in ascending order, longest walks first;
  // otherwise each XCD walks a contiguous run of (KV head, key tile, chunk).
  const int nblk = gridDim.x;
  const int nbkv = nblk / (n_kt * nsplit);
  int split, kt, bkv;
  if (CAUSAL && nsplit == 1 && (nbkv & 7) == 0) {
    const int per = nbkv >> 3, j = blockIdx.x >> 3;
    split = 0;
    kt = j / per;
    bkv = (blockIdx.x & 7) * per + j % per;
  } else {
    const int L = ((nblk & 7) == 0) ? (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    split = L % nsplit;
    const int rest = L / nsplit;
    kt = rest % n_kt;
    bkv = rest / n_kt;
  }
  const int b = bkv / Hkv, kvh = bkv % Hkv;
  const int k0 = kt * BWD_BN;
  const int kw0 = k0 + slice * 32;
  const int key = kw0 + l32;
  const int diag = Skv - Sq;

  // Query range of this chunk (q_chunk is a multiple of BMQ).
  const int qs = split * q_chunk;
  const int qe = min(Sq, qs + q_chunk);
  int q_lo = qs;
  if (CAUSAL) {
    const int first = k0 - diag;  // first query that can see key k0
    if (first > q_lo) q_lo = (first / BMQ) * BMQ;
  }
  const int nq = qe > q_lo ? (qe - q_lo + BMQ - 1) / BMQ : 0;
  const int n_it = G * nq;  // steps: query tiles of every head of the group, heads ascending
  auto qt0_of = [&](int it) __attribute__((always_inline)) { return q_lo + (it % nq) * BMQ; };

  Copy cp;
  cp.init(tid);
  auto issue = [&](int it, char* dst) __attribute__((always_inline)) {
    const int h = kvh * G + it / nq;
    const int qt0 = qt0_of(it);
    const size_t row0 = (size_t)(b * Hq + h) * Sq + qt0;
    const uint32_t rows = (uint32_t)(Sq - qt0);
    cp.load(Buf(Q + row0 * D, rows * D * 2), Buf(dO + row0 * D, rows * D * 2),
            Buf(LSE + row0, rows * 4), Buf(DLT + row0, rows * 4), dst, lane);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;

  // The P-wave keeps K of its slice, the dS-wave keeps V, as MFMA B operands.
  const size_t kv_off = (size_t)bkv * Skv * D;
  const Buf kvbuf(pwave ? K + kv_off : V + kv_off, (uint32_t)Skv * D * 2);
  bf16x8 kvf[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    kvf[st] = as_bf16x8(kvbuf.ld16((uint32_t)(key * D + 16 * st + 8 * g) * 2));
  if (n_it > 0) issue(0, QTbuf(B0{}));
  if (n_it > 1) issue(1, QTbuf(B1{}));
  // Everything issued so far has landed before the walk starts, so that no
  // wait for these loads ends up inside the loop, where it would also wait
  // for the copies of later tiles.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  f32x16 acc[D / 32];  // dV^T (P-wave) or dK^T (dS-wave)
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = zero_f32x16();

  SW sw;
  sw.init(lane);
  // This lane's first 16 bytes of the P hand-off, sub-block 0, parity 0.
  int pex_lane = (slice * NSUB * 2 * 64 + lane) * 8;
  asm volatile("" : "+v"(pex_lane));
  // S = Q K^T (P-wave) or dP = dO V^T (dS-wave) for one tile: lane = key
  // column, registers = query rows; both sub-blocks as independent chains.
  auto score_tile = [&](const bf16* tile, f32x16 (&sc)[NSUB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < NSUB; ++qb) sc[qb] = zero_f32x16();
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
#pragma unroll
      for (int qb = 0; qb < NSUB; ++qb)
        sc[qb] = mfma32(sw.row(tile, qb * 32, st), kvf[st], sc[qb]);
    // Operand reads run four MFMAs ahead.
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NSUB * D / 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  // P = 2^(S*c - LSE*log2e), masked above the causal diagonal; P rounded to
  // bf16 stays in registers for dV, and P rounded to fp16 (nearest even; P
  // lies in [0, 1]) goes to the dS-wave through LDS.
  bf16x8 pb[NSUB][2];
  u32x4 ph[NSUB][2];  // the same P as fp16 pairs, for the dS-wave
  float pr_keep[4];
  auto exp_tile = [&](auto masked, const float* lse, bf16* pex, int qt0,
                      const f32x16 (&sc)[NSUB]) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(masked)::value;
#pragma unroll
    for (int qb = 0; qb < NSUB; ++qb) {
      // Register i holds query row qt0 + 32qb + 4g + (i/4)*8 + i%4; the key
      // is above the diagonal for that row iff y exceeds the constant part.
      const int y = key - diag - qt0 - qb * 32 - 4 * g;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const f32x4 Lv = *reinterpret_cast<const f32x4*>(&lse[qb * 32 + 8 * blk + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * blk + j;
          float pr = fast_exp2(__builtin_fmaf(sc[qb][i], c, -Lv[j] * MATTN_LOG2E));
          if (MASK && y > 8 * blk + j) pr = 0.f;
          pr_keep[j] = pr;
          pb[qb][i >> 3][i & 7] = (bf16)pr;
        }
        ph[qb][blk >> 1][(blk & 1) * 2] = pack_f16x2(pr_keep[0], pr_keep[1]);
        ph[qb][blk >> 1][(blk & 1) * 2 + 1] = pack_f16x2(pr_keep[2], pr_keep[3]);
      }
      *reinterpret_cast<u32x4*>(pex + (2 * qb) * 64 * 8) = ph[qb][0];
      *reinterpret_cast<u32x4*>(pex + (2 * qb + 1) * 64 * 8) = ph[qb][1];
    }
  };
  // dV^T += dO^T P.
  auto dv_tile = [&](const bf16* dos) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < NSUB; ++qb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 a[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) a[db] = sw.trans(dos, qb * 32 + 16 * t, db);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = mfma32(a[db], pb[qb][t], acc[db]);
      }
    // Transposed operand reads (two per fragment) run eight fragments ahead
    // (measured 5% faster than the compiler's own schedule).
#pragma unroll
    for (int i = 0; i < 16; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NSUB * D / 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };
  // dS = P (dP - Dlt) from the fp16 P, rounded to bf16 as the B operand of
  // dK^T += Q^T dS.
  auto ds_tile = [&](const float* dlt, const bf16* pex, const f32x16 (&dp)[NSUB],
                     bf16x8 (&dsb)[NSUB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < NSUB; ++qb) {
      const f16x8 p0 = *reinterpret_cast<const f16x8*>(pex + (2 * qb) * 64 * 8);
      const f16x8 p1 = *reinterpret_cast<const f16x8*>(pex + (2 * qb + 1) * 64 * 8);
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const f32x4 Dl = *reinterpret_cast<const f32x4*>(&dlt[qb * 32 + 8 * blk + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * blk + j;
          // fp16 P times an fp32 difference: one mixed-precision FMA
          // (v_fma_mix_f32), with no separate widening of P.
          const _Float16 ph16 = i < 8 ? p0[i] : p1[i - 8];
          dsb[qb][i >> 3][i & 7] = (bf16)__builtin_fmaf((float)ph16, dp[qb][i] - Dl[j], 0.f);
        }
      }
    }
  };
  auto dk_tile = [&](const bf16* qs_, const bf16x8 (&dsb)[NSUB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < NSUB; ++qb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 a[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) a[db] = sw.trans(qs_, qb * 32 + 16 * t, db);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = mfma32(a[db], dsb[qb][t], acc[db]);
      }
#pragma unroll
    for (int i = 0; i < 16; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NSUB * D / 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // Step it, tile it in buffer it % 3 (a compile-time constant of each
  // unrolled step), tile it-1 in buffer (it+2) % 3.  The barrier publishes
  // P(it) (the fence of __syncthreads waits for the LDS writes) and, since
  // every wave has first waited for its own copies (vmcnt(0): the fence does
  // not cover direct copies), tile it+1; it also ends every read of tile
  // it-1, whose buffer then takes tile it+2.
  f32x16 sc[NSUB];       // S(it) on the P-wave, dP(it) on the dS-wave
  bf16x8 dsb[NSUB][2];   // dS(it-1), dS-wave only
  auto step = [&](auto bsel, int it) __attribute__((always_inline)) {
    constexpr int bi = decltype(bsel)::value;
    char* cur = QTbuf(bsel);
    char* prev = QTbuf(std::integral_constant<int, bi + 2>{});
    bf16* pex = Pex + (it & 1) * PEX_PAR + pex_lane;
    if (pwave) {
      score_tile(Qs(cur), sc);
      const int qt0 = qt0_of(it);
      if (CAUSAL && (kw0 + 31 > qt0 + diag))
        exp_tile(std::true_type{}, lse_s(cur), pex, qt0, sc);
      else
        exp_tile(std::false_type{}, lse_s(cur), pex, qt0, sc);
    } else {
      if (it > 0) dk_tile(Qs(prev), dsb);
      score_tile(dOs(cur), sc);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
    // Tile it+2's copies: the P-waves issue theirs after the dV MFMAs, the
    // dS-waves before their dS arithmetic, so that the copies do not all
    // start at the barrier beside the operand reads of both roles.
    if (pwave) {
      dv_tile(dOs(cur));
      if (it + 2 < n_it) issue(it + 2, prev);
    } else {
      if (it + 2 < n_it) issue(it + 2, prev);
      ds_tile(dlt_s(cur), pex, sc, dsb);
    }
  };

  if (n_it > 0) __syncthreads();  // tiles 0 and 1 landed everywhere (waited for above)
  int it = 0;
  for (; it + 3 <= n_it; it += 3) {
    step(B0{}, it);
    step(B1{}, it + 1);
    step(B2{}, it + 2);
  }
  if (it < n_it) step(B0{}, it);
  if (it + 1 < n_it) step(B1{}, it + 1);
  // The dS-wave's last dK uses the last tile, still in place.
  if (!pwave && n_it > 0) {
    switch ((n_it - 1) % 3) {
      case 0: dk_tile(Qs(QTbuf(B0{})), dsb); break;
      case 1: dk_tile(Qs(QTbuf(B1{})), dsb); break;
      default: dk_tile(Qs(QTbuf(B2{})), dsb); break;
    }
  }

  const float mul = pwave ? 1.f : scale;  // dK = scale * Q^T dS
  if (nsplit == 1) {
    // dV (P-waves) and dK (dS-waves) rows through LDS (store_rows_bf16),
    // staged in two query-tile buffers once every wave is past the walk.
    static_assert(4 * stage_rows_bytes<D>() <= Copy::BUF_BYTES, "staging fits a buffer");
    __syncthreads();
    char* stg = (pwave ? QT0 : QT1) + slice * stage_rows_bytes<D>();
    store_rows_bf16<D>(acc, mul, stg, (pwave ? dV : dK) + kv_off + (size_t)kw0 * D, Skv - kw0, lane);
  } else {
    if (key >= Skv) return;
    // fp32 partials, unscaled: [dK, dV][nsplit][B*Hkv][n_kt*BWD_BN][D]
    const size_t rows_all = (size_t)(gridDim.x / nsplit / n_kt) * n_kt * BWD_BN;
    const size_t half = (size_t)nsplit * rows_all * D;
    const size_t ro = (pwave ? half : 0) +
                      ((size_t)split * rows_all + (size_t)bkv * n_kt * BWD_BN + key) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = db * 32 + r * 8 + g * 4;
        *reinterpret_cast<f32x4*>(part + ro + d) =
            f32x4{acc[db][4 * r], acc[db][4 * r + 1], acc[db][4 * r + 2], acc[db][4 * r + 3]};
      }
  }
}

// Sum of the split partials in fixed chunk order, scaled (dK) and rounded.
__global__ __launch_bounds__(THREADS)
void bwd_reduce_kernel(const float* __restrict__ part, bf16* __restrict__ dK,
                       bf16* __restrict__ dV, int nsplit, int BKV, int Skv, int n_kt, int D,
                       float scale) {
  const long long total4 = (long long)BKV * Skv * D / 4;
  const long long i4 = (long long)blockIdx.x * THREADS + threadIdx.x;
  if (i4 >= total4) return;
  const long long e = i4 * 4;
  const long long row = e / D;  // bkv*Skv + key
  const int d = (int)(e % D);
  const long long bkv = row / Skv, key = row % Skv;
  const size_t rows_all = (size_t)BKV * n_kt * BWD_BN;
  const size_t half = (size_t)nsplit * rows_all * D;
  const size_t src = ((size_t)bkv * n_kt * BWD_BN + key) * D + d;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    sk += *reinterpret_cast<const f32x4*>(part + (size_t)s * rows_all * D + src);
    sv += *reinterpret_cast<const f32x4*>(part + half + (size_t)s * rows_all * D + src);
  }
  uint2 wk, wv;
  wk.x = pack_bf16x2(sk[0] * scale, sk[1] * scale);
  wk.y = pack_bf16x2(sk[2] * scale, sk[3] * scale);
  wv.x = pack_bf16x2(sv[0], sv[1]);
  wv.y = pack_bf16x2(sv[2], sv[3]);
  *reinterpret_cast<uint2*>(dK + e) = wk;
  *reinterpret_cast<uint2*>(dV + e) = wv;
}

// ----------------------------------------------------------------------------
// 3. dQ
constexpr int DQ_WAVES = 4;                // one 32-row query slice per wave
constexpr int DQ_BM = 32 * DQ_WAVES;       // query rows per workgroup
constexpr int DQ_BN = 64;                  // keys per tile
constexpr int DQ_THREADS = 64 * DQ_WAVES;

// Direct global -> LDS copy of one K tile and one V tile (DQ_BN rows each)
// into one buffer laid out as [K tile | V tile], both in the SwzTile layout.
// The swizzle only permutes 16-byte chunks within a row, so it is applied on
// the global side: LDS slot (row, position) receives global chunk
// position ^ ((row >> 2) & 3), and every wave writes 64 consecutive slots.
// The two tiles together are a whole number of rounds of the workgroup's
// threads, so every wave issues the same number of copies per buffer.
template <int D>
struct DqKvCopy {
  static constexpr int P = SwzTile<D>::P;
  static constexpr int SLOTS_PER_ROW = P / 8;
  static constexpr int TILE_SLOTS = DQ_BN * SLOTS_PER_ROW;  // per tensor
  static constexpr int ROUNDS = 2 * TILE_SLOTS / DQ_THREADS;
  static constexpr int BUF_ELEMS = 2 * TILE_SLOTS * 8;
  static_assert(2 * TILE_SLOTS % DQ_THREADS == 0 && TILE_SLOTS % 64 == 0, "whole rounds");
  // Per-round byte offsets within a tile are below 2^15, so two share a
  // register (a register each would not fit beside the kernel's other state);
  // 0xffff marks a pad slot and lies past every tile's descriptor, so it
  // loads zeros.
  static_assert(DQ_BN * D * 2 < 0xffff, "16-bit offsets");
  uint32_t off2[(ROUNDS + 1) / 2];
  int w0;  // first slot of this wave in round 0 (scalar)
  __device__ __forceinline__ void init(int tid) {
    w0 = __builtin_amdgcn_readfirstlane(tid & ~63);
#pragma unroll
    for (int r = 0; r < (ROUNDS + 1) / 2; ++r) off2[r] = 0xffffffffu;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int q = r * DQ_THREADS + tid;
      const int qq = q % TILE_SLOTS;  // slot within its tensor's tile
      const int row = qq / SLOTS_PER_ROW, pos = qq - row * SLOTS_PER_ROW;
      const int ch = pos ^ ((row >> 2) & 3);
      const uint32_t o = pos < D / 8 ? (uint32_t)(row * D + ch * 8) * 2 : 0xffffu;
      off2[r / 2] = (r & 1) ? ((off2[r / 2] & 0xffffu) | (o << 16)) : ((off2[r / 2] & 0xffff0000u) | o);
    }
  }
  // The descriptors cover exactly the tile's rows (fewer at the end of the
  // keys); rows past them, and pad slots, load zeros.
  __device__ __forceinline__ void load(const Buf& k, const Buf& v, bf16* buf) const {
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int q0 = r * DQ_THREADS + w0;
      const uint32_t o = (r & 1) ? (off2[r / 2] >> 16) : (off2[r / 2] & 0xffffu);
      ld16_to_lds(q0 < TILE_SLOTS ? k : v, o, buf + q0 * 8);
    }
  }
};

// Tile layout and copy of the dQ kernel's [K | V] buffers: D = 128 uses the
// GrpTile128 layout (each wave copies four groups of four rows per tensor,
// no padding written); D = 64 the padded SwzTile layout.
template <int D>
struct DqLayout {
  using SW = SwzTile<D>;
  using Copy = DqKvCopy<D>;
  static constexpr int VOFF = Copy::TILE_SLOTS * 8;  // V tile's offset in a buffer (elements)
  static constexpr int BUF_ELEMS = Copy::BUF_ELEMS;
  static_assert(SW::P * DQ_BN == VOFF, "V tile follows the K tile");
};
template <>
struct DqLayout<128> {
  using SW = GrpTile128;
  static constexpr int VOFF = GrpTile128::bytes(DQ_BN) / 2;
  static constexpr int BUF_ELEMS = 2 * VOFF;
  struct Copy {
    GrpCopy<DQ_BN, DQ_WAVES> g;
    __device__ __forceinline__ void init(int tid) {
      g.init(__builtin_amdgcn_readfirstlane(tid >> 6), tid & 63);
    }
    __device__ __forceinline__ void load(const Buf& k, const Buf& v, bf16* buf) const {
      g.load(k, buf);
      g.load(v, buf + VOFF);
    }
  };
};

// dQ_i = scale * sum_j dS_ij K_j for a block of DQ_BM query rows.  Each wave
// keeps its 32 rows of Q and dO in registers and walks every 64-key tile in
// two 32-key halves.  K/V tiles arrive by direct copies into two LDS
// buffers, one tile ahead, with one barrier per tile.  Each buffer is its own
// LDS object, so reads of the current tile never wait for the copies in
// flight to the other.  Two workgroups share a CU: the two waves on a SIMD
// then belong to different workgroups and drift out of phase, so the VALU
// work of one (dS) overlaps the MFMA work of the other.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(DQ_THREADS, 2)
void bwd_dq_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                   const bf16* __restrict__ V, const bf16* __restrict__ O,
                   const bf16* __restrict__ dO, const float* __restrict__ LSE,
                   float* __restrict__ DLT, bf16* __restrict__ dQ, int Hq, int G, int Sq,
                   int Skv, float scale, float c, int n_qt) {
  using SW = typename DqLayout<D>::SW;
  using Copy = typename DqLayout<D>::Copy;
  constexpr int VOFF = DqLayout<D>::VOFF;  // V tile's offset in a buffer (elements)
  __shared__ __attribute__((aligned(16))) bf16 KV0[DqLayout<D>::BUF_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 KV1[DqLayout<D>::BUF_ELEMS];
  auto KVbuf = [&](auto b) __attribute__((always_inline)) -> bf16* {
    if constexpr (decltype(b)::value == 0) return KV0; else return KV1;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int slice = wave;  // 32 query rows
  int bh, qt;
  tile_of_block(blockIdx.x, gridDim.x / n_qt, n_qt, CAUSAL, bh, qt);
  const int h = bh % Hq, b = bh / Hq;
  const int Hkv = Hq / G;
  const size_t kv_off = ((size_t)(b * Hkv + h / G) * Skv) * D;
  const int q0 = qt * DQ_BM;
  const int qw0 = q0 + slice * 32;
  const int qrow = qw0 + l32;
  const int diag = Skv - Sq;
  SW sw;
  sw.init(lane);

  int kv_end = Skv;
  if (CAUSAL) kv_end = min(Skv, q0 + DQ_BM + diag);
  const int n_kt = (kv_end + DQ_BN - 1) / DQ_BN;

  Copy cp;
  cp.init(tid);
  const bf16* Kh = K + kv_off;
  const bf16* Vh = V + kv_off;
  auto issue = [&](int kt, bf16* dst) __attribute__((always_inline)) {
    const int j0 = kt * DQ_BN;
    const uint32_t nb = (uint32_t)min(DQ_BN, Skv - j0) * D * 2;
    cp.load(Buf(Kh + (size_t)j0 * D, nb), Buf(Vh + (size_t)j0 * D, nb), dst);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  if (n_kt > 0) issue(0, KV0);

  const Buf qbuf(Q + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
  const Buf dobuf(dO + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
  bf16x8 qf[D / 16], dof[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = as_bf16x8(qbuf.ld16((uint32_t)(qrow * D + 16 * s + 8 * g) * 2));
    dof[s] = as_bf16x8(dobuf.ld16((uint32_t)(qrow * D + 16 * s + 8 * g) * 2));
  }
  // A padded query row gets LSE = +inf, so its P (and dS) is exactly 0.
  const float lse2 = qrow < Sq ? LSE[(size_t)bh * Sq + qrow] * MATTN_LOG2E : MATTN_INF;
  // Dlt = sum_d dO * O of this lane's row: this lane's half of the row (the
  // columns its dO fragments hold), then its partner lane's half.  The
  // arithmetic is dlt_half_row's, so the value is bitwise the preprocess
  // kernel's.  It is also stored for the dK/dV kernel, which runs after this
  // one.  Rows past Sq load zeros and get 0.
  const Buf obuf(O + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
  float dhalf = 0.f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    dhalf = dlt_half_row_step(dof[s], as_bf16x8(obuf.ld16((uint32_t)(qrow * D + 16 * s + 8 * g) * 2)), dhalf);
  const float dl = dhalf + __shfl_xor(dhalf, 32);
  if (g == 0 && qrow < Sq) DLT[(size_t)bh * Sq + qrow] = dl;
  // dP^T - Dlt straight from the matrix unit: each dP^T accumulator starts
  // from one MFMA of a ones operand (k = 0..2 on the g = 0 lanes, zero
  // elsewhere) with this lane's -Dlt as three bf16 terms that sum to it
  // exactly (each the top bits of what the previous ones leave).
  bf16x8 ones_a, ndl_b;
  {
    const u32x4 o = g == 0 ? u32x4{0x3f803f80u, 0x3f80u, 0u, 0u} : u32x4{0u, 0u, 0u, 0u};
    const float x = -dl;
    const uint32_t hi = __builtin_bit_cast(uint32_t, x) & 0xffff0000u;
    const float r1 = x - __builtin_bit_cast(float, hi);
    const uint32_t mid = __builtin_bit_cast(uint32_t, r1) & 0xffff0000u;
    const float r2 = r1 - __builtin_bit_cast(float, mid);
    const u32x4 t = {(hi >> 16) | mid, __builtin_bit_cast(uint32_t, r2) >> 16, 0u, 0u};
    ones_a = __builtin_bit_cast(bf16x8, o);
    ndl_b = __builtin_bit_cast(bf16x8, t);
  }

  f32x16 adq[D / 32];  // dQ^T of this wave's 32 rows
#pragma unroll
  for (int db = 0; db < D / 32; ++db) adq[db] = zero_f32x16();

  // Tile kt sits in buffer kt & 1.  At its top this thread's copies of tile
  // kt have landed; the barrier makes that true for everyone and ends every
  // read of tile kt-1, whose buffer then takes tile kt+1.
  auto tile = [&](auto bsel, auto tail, int kt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    barrier_keep_copies();
    if (kt + 1 < n_kt) issue(kt + 1, KVbuf(std::integral_constant<int, decltype(bsel)::value ^ 1>{}));
    const bf16* Ks = KVbuf(bsel);
    const bf16* Vs = Ks + VOFF;
    const int j0 = kt * DQ_BN;
    auto step = [&](auto masked, int kb0) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(masked)::value;
      f32x16 s = zero_f32x16(), dp = mfma32(ones_a, ndl_b, zero_f32x16());
#pragma unroll
      for (int st0 = 0; st0 < D / 16; st0 += 4) {
        bf16x8 ak[4], av[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ak[u] = sw.row(Ks, kb0, st0 + u);
          av[u] = sw.row(Vs, kb0, st0 + u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          s = mfma32(ak[u], qf[st0 + u], s);
          dp = mfma32(av[u], dof[st0 + u], dp);
        }
      }
      bf16x8 dsb[2];
      // Key j0 + kb0 + crow(i, g) is visible iff crow(i, 0) <= lim.
      int lim = 0;
      if (MASK) {
        int last = Skv - 1;
        if (CAUSAL) last = min(last, qrow + diag);
        lim = last - j0 - kb0 - 4 * g;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(__builtin_fmaf(s[i], c, -lse2));
        if (MASK && crow(i, 0) > lim) p = 0.f;
        dsb[i >> 3][i & 7] = (bf16)(p * dp[i]);
      }
      // dQ^T += K^T dS^T over this wave's 32 keys.
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 a[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) a[db] = sw.trans(Ks, kb0 + 16 * t, db);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) adq[db] = mfma32(a[db], dsb[t], adq[db]);
      }
    };
#pragma unroll
    for (int kb0 = 0; kb0 < DQ_BN; kb0 += 32) {
      // Only tiles that reach past Skv (the last one at most) test for it, and
      // only outside the main loop, so the loop body holds at most the causal
      // variant.
      if constexpr (decltype(tail)::value) {
        if (j0 + kb0 >= Skv) break;  // no key of this half exists
        step(std::true_type{}, kb0);
      } else {
        // Near the diagonal a half can lie wholly past this wave's last
        // query (its dS is all zero): that wave skips it, which leaves its
        // SIMD to the other workgroup's wave.
        if (CAUSAL && (j0 + kb0 > qw0 + 31 + diag)) {
        } else if (CAUSAL && (j0 + kb0 + 31 > qw0 + diag)) {
          step(std::true_type{}, kb0);
        } else {
          step(std::false_type{}, kb0);
        }
      }
      // One half at a time: interleaving the halves needs more registers
      // than two waves per SIMD have.
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Tiles wholly below Skv run in the loop, two per trip so that each
  // buffer is named at compile time; the rest (at most two, starting on an
  // even tile) also check for keys past Skv.
  const int n_full = Skv % DQ_BN == 0 ? n_kt : min(n_kt, Skv / DQ_BN);
  int kt = 0;
  for (; kt + 2 <= n_full; kt += 2) {
    tile(B0{}, std::false_type{}, kt);
    tile(B1{}, std::false_type{}, kt + 1);
  }
  if (kt < n_kt) tile(B0{}, std::true_type{}, kt);
  if (kt + 1 < n_kt) tile(B1{}, std::true_type{}, kt + 1);

  // dQ rows through LDS (store_rows_bf16), staged in the buffer the last
  // tile did not use: every wave finished reading it before that tile's
  // barrier, and no copy goes to it afterwards.
  static_assert(DQ_WAVES * stage_rows_bytes<D>() <= DqLayout<D>::BUF_ELEMS * 2, "staging fits a buffer");
  {
    bf16* st = (n_kt & 1) ? KV1 : KV0;
    char* stg = reinterpret_cast<char*>(st) + slice * stage_rows_bytes<D>();
    store_rows_bf16<D>(adq, scale, stg, dQ + ((size_t)bh * Sq + qw0) * D, Sq - qw0, lane);
  }
}

template <int D>
hipError_t launch_pre_bf16(const Problem& p, const void* o, const void* dout, float* dlt,
                           hipStream_t stream) {
  const long long rows = (long long)p.B * p.Hq * p.Sq;
  const unsigned blocks = (unsigned)((2 * rows + THREADS - 1) / THREADS);
  hipLaunchKernelGGL((bwd_pre_bf16_kernel<D>), dim3(blocks), dim3(THREADS), 0, stream,
                     (const bf16*)o, (const bf16*)dout, dlt, rows);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_pre_t(const Problem& p, const void* o, const void* dout, float* dlt,
                        hipStream_t stream) {
  const long long rows = (long long)p.B * p.Hq * p.Sq;
  const int tpr = p.D / 8;
  const long long rpb = THREADS / tpr;
  const unsigned blocks = (unsigned)((rows + rpb - 1) / rpb);
  if (p.D == 64)
    hipLaunchKernelGGL((bwd_pre_kernel<T, 64>), dim3(blocks), dim3(THREADS), 0, stream,
                       (const T*)o, (const T*)dout, dlt, rows);
  else
    hipLaunchKernelGGL((bwd_pre_kernel<T, 128>), dim3(blocks), dim3(THREADS), 0, stream,
                       (const T*)o, (const T*)dout, dlt, rows);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv_t(const Problem& p, const void* q, const void* k, const void* v,
                         const float* lse, const float* dlt, const void* dout, void* dk, void* dv,
                         float* part, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  const float c = p.scale * MATTN_LOG2E;
  const int n_kt = (p.Skv + BWD_BN - 1) / BWD_BN;
  const int nsplit = bwd_nsplit(p.B, p.Hkv, p.Sq, p.Skv);
  const int n_qt = (p.Sq + BWD_BMQ - 1) / BWD_BMQ;
  const int q_chunk = ((n_qt + nsplit - 1) / nsplit) * BWD_BMQ;
  const long long blocks = (long long)p.B * p.Hkv * n_kt * nsplit;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(DKDV_THREADS), 0,
                     stream, (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout,
                     lse, dlt, (bf16*)dk, (bf16*)dv, part, p.Hq, G, p.Sq, p.Skv, p.scale, c,
                     n_kt, nsplit, q_chunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  const long long total4 = (long long)p.B * p.Hkv * p.Skv * D / 4;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((total4 + THREADS - 1) / THREADS)),
                     dim3(THREADS), 0, stream, (const float*)part, (bf16*)dk, (bf16*)dv, nsplit,
                     p.B * p.Hkv, p.Skv, n_kt, D, p.scale);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq_t(const Problem& p, const void* q, const void* k, const void* v,
                       const void* o, const float* lse, float* dlt, const void* dout, void* dq,
                       hipStream_t stream) {
  const int n_qt = (p.Sq + DQ_BM - 1) / DQ_BM;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)((long long)p.B * p.Hq * n_qt)),
                     dim3(DQ_THREADS), 0, stream, (const bf16*)q, (const bf16*)k, (const bf16*)v,
                     (const bf16*)o, (const bf16*)dout, lse, dlt, (bf16*)dq, p.Hq, p.Hq / p.Hkv,
                     p.Sq, p.Skv, p.scale, p.scale * MATTN_LOG2E, n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_preprocess(const Problem& p, bool bf16_io, const void* o, const void* dout,
                                 float* dlt, hipStream_t stream) {
  if (bf16_io)
    return p.D == 64 ? launch_pre_bf16<64>(p, o, dout, dlt, stream)
                     : launch_pre_bf16<128>(p, o, dout, dlt, stream);
  return launch_pre_t<float>(p, o, dout, dlt, stream);
}

hipError_t launch_dkdv_bf16(const Problem& p, const void* q, const void* k, const void* v,
                            const float* lse, const float* dlt, const void* dout, void* dk,
                            void* dv, float* part, hipStream_t stream) {
  if (p.D == 64)
    return p.causal ? launch_dkdv_t<64, true>(p, q, k, v, lse, dlt, dout, dk, dv, part, stream)
                    : launch_dkdv_t<64, false>(p, q, k, v, lse, dlt, dout, dk, dv, part, stream);
  return p.causal ? launch_dkdv_t<128, true>(p, q, k, v, lse, dlt, dout, dk, dv, part, stream)
                  : launch_dkdv_t<128, false>(p, q, k, v, lse, dlt, dout, dk, dv, part, stream);
}

hipError_t launch_dq_bf16(const Problem& p, const void* q, const void* k, const void* v,
                          const void* o, const float* lse, float* dlt, const void* dout, void* dq,
                          hipStream_t stream) {
  if (p.D == 64)
    return p.causal ? launch_dq_t<64, true>(p, q, k, v, o, lse, dlt, dout, dq, stream)
                    : launch_dq_t<64, false>(p, q, k, v, o, lse, dlt, dout, dq, stream);
  return p.causal ? launch_dq_t<128, true>(p, q, k, v, o, lse, dlt, dout, dq, stream)
                  : launch_dq_t<128, false>(p, q, k, v, o, lse, dlt, dout, dq, stream);
}

}  // namespace mattn

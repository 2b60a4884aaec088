// Fused attention forward and backward with float32 operands throughout, on
// the fp32 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Same method as the bf16 kernels (xtrain evolution page, infrastructure-
// phase table, rows T14 and T15: online softmax over K/V tiles, recompute-
// based backward with D = sum(dO * O), group-summed dK/dV without atomics),
// but no operand is ever rounded below fp32: Q, K, V, dO, P and dS enter the
// matrix instructions as fp32, and every accumulator is fp32.
//
// MFMA layout (lane l, l32 = l % 32, g = l / 32), one 32x32 block:
//   A (32 x 2): lane holds row l32, k = g;   B (2 x 32): lane holds column
//   l32, k = g;   C (32 x 32): register i holds row crow(i, g), column l32.
// A contraction over the head dimension is a sum, so its order is free:
// k-step 4j + e with lane group g carries column d = 8j + 4g + e, which lets
// each lane load four k-steps of a row operand as one 16-byte read.  A C
// tile feeds the next product as its B operand straight from registers:
// register t is k-step t, carrying row crow(t, g) of the tile (keys in the
// forward and dQ, query rows in dK/dV); the other operand is then read from
// LDS one 4-byte column element per lane, at rows crow(t, g).
//
// Kernels:
//  * forward: each wave owns 32 query rows (Q^T resident as the B operand of
//    S^T = K Q^T, lane = query), walks 32-key K/V tiles copied into
//    double-buffered LDS, and accumulates O^T += V^T P^T with the online
//    softmax statistics per lane;
//  * dQ: the same walk with dO^T resident as well: S^T, dP^T = V dO^T,
//    dS^T = P^T (dP^T - D), dQ^T += K^T dS^T;
//  * dK/dV: each wave owns 32 keys (K^T and V^T resident, lane = key) and
//    walks 32-row Q/dO tiles of every query head of its group in ascending
//    order: S = Q K^T, P, dV^T += dO^T P, dP = dO V^T, dS = P (dP - D),
//    dK^T += Q^T dS; the group sum stays in registers, no atomics.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace mattn {
namespace {

constexpr int FT = 32;  // keys (forward, dQ) or query rows (dK/dV) per LDS tile

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// LDS row pitches in floats.  ROW: tiles read as 16-byte row operands (the
// sixteen lanes of a pass read rows r..r+15 at one column, 16 bytes apart in
// the bank space).  COL: tiles read only as 4-byte column operands (the two
// half-waves read rows four apart, which then fall in disjoint bank halves).
// A tile read both ways (K in dQ, Q and dO in dK/dV) uses ROW; its column
// reads then meet 2-way conflicts on a quarter of the banks.
template <int D>
struct F32Pitch {
  static constexpr int ROW = D + 4;
  static constexpr int COL = D + 8;
};

// A 32-row fp32 tile with row pitch P floats, filled by direct global -> LDS
// copies (DirectTile counts in 2-byte units: a row of D floats is 2D of them).
template <int D, int P, int NT>
struct F32Tile {
  using DT = DirectTile<2 * D, FT, 2 * P, NT>;
  static constexpr int FLOATS = DT::LDS_ELEMS / 2;
  DT dt;
  __device__ __forceinline__ void init(int tid) { dt.init(tid); }
  // src: a descriptor from the tile's first row to its last valid row, so
  // rows past it (and the pitch padding) are written as zeros.
  __device__ __forceinline__ void load(const Buf& src, float* lds, int tid) const {
    dt.load(src, reinterpret_cast<bf16*>(lds), tid);
  }
};

// LDS row of register t of a C tile for lane group g, less the lane-group
// part 4g (carried by the per-lane base): 8(t/4) + t%4.
__device__ __forceinline__ constexpr int trow(int t) { return (t >> 2) * 8 + (t & 3); }

// Row operand fragments of one 32-row block held in registers: for a row
// owned by the lane, fragment j holds columns 8j + 4g .. 8j + 4g + 3.
template <int D>
__device__ __forceinline__ void load_frags(const Buf& b, uint32_t row_byte_off, int g,
                                           f32x4 (&f)[D / 8]) {
#pragma unroll
  for (int j = 0; j < D / 8; ++j)
    f[j] = __builtin_bit_cast(f32x4, b.ld16(row_byte_off + (uint32_t)(8 * j + 4 * g) * 4));
}

// C = A B over the head dimension, A from a ROW-pitch LDS tile (rows of the
// lane's l32, base `off` = l32 * ROW + 4g), B the resident fragments.
template <int D>
__device__ __forceinline__ void rows_times_frags(const float* tile, int off, const f32x4 (&f)[D / 8],
                                                 f32x16& c) {
  c = zero_f32x16();
#pragma unroll
  for (int j = 0; j < D / 8; ++j) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(tile + off + 8 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = mfma_f32(a[e], f[j][e], c);
  }
}

// acc[db] (rows = columns 32db .. 32db+31 of the tile, k = the tile's 32
// rows) += tile^T x, x the B operand held as a C tile (register t = k-step
// t).  `cbase` = 4g * pitch + l32.
template <int D, int PITCH>
__device__ __forceinline__ void cols_times_c(const float* tile, int cbase, const f32x16& x,
                                             f32x16 (&acc)[D / 32]) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int t = 0; t < 16; ++t)
      acc[db] = mfma_f32(tile[cbase + trow(t) * PITCH + 32 * db], x[t], acc[db]);
}

// A wave's 32 output rows held as C tiles (lane = row, register i of block
// db = column 32db + crow(i, g)), times mul; rows at or past rows_valid are
// not written.  Each store writes 16 bytes of one row.
template <int D>
__device__ __forceinline__ void store_rows_f32(const f32x16 (&acc)[D / 32], float mul, float* out,
                                               int row, int rows_valid, int g) {
  if (row >= rows_valid) return;
  float* p = out + (size_t)row * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<f32x4*>(p + 32 * db + 8 * m + 4 * g) =
          f32x4{acc[db][4 * m] * mul, acc[db][4 * m + 1] * mul, acc[db][4 * m + 2] * mul,
                acc[db][4 * m + 3] * mul};
}

using Even = std::integral_constant<int, 0>;
using Odd = std::integral_constant<int, 1>;

// ----------------------------------------------------------------------------
// Forward.  WAVES waves, 32 query rows each, of one head.  Softmax in the log2
// domain: t = s * scale * log2(e), p = 2^(t - m); the reference max m moves
// only when a tile's max exceeds it by more than RESCALE_SLACK.
template <int D, bool CAUSAL, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES)
void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                    const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                    int Hq, int G, int Sq, int Skv, float c, int n_qt) {
  constexpr int NT = 64 * WAVES, BM = 32 * WAVES;
  constexpr int PK = F32Pitch<D>::ROW, PV = F32Pitch<D>::COL;
  using KT = F32Tile<D, PK, NT>;
  using VT = F32Tile<D, PV, NT>;
  __shared__ __attribute__((aligned(16))) float Ks0[KT::FLOATS];
  __shared__ __attribute__((aligned(16))) float Ks1[KT::FLOATS];
  __shared__ __attribute__((aligned(16))) float Vs0[VT::FLOATS];
  __shared__ __attribute__((aligned(16))) float Vs1[VT::FLOATS];
  auto Ks = [&](auto par) -> float* {
    if constexpr (decltype(par)::value == 0) return Ks0; else return Ks1;
  };
  auto Vs = [&](auto par) -> float* {
    if constexpr (decltype(par)::value == 0) return Vs0; else return Vs1;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  int bh, qt;
  tile_of_block(blockIdx.x, gridDim.x / n_qt, n_qt, CAUSAL, bh, qt);
  const int b = bh / Hq, h = bh - b * Hq;
  const size_t kv_off = (size_t)(b * (Hq / G) + h / G) * Skv * D;
  const int q0 = qt * BM;
  const int qw = q0 + wave * 32;  // this wave's first query
  const int qrow = qw + l32;      // this lane's query
  const int diag = Skv - Sq;      // key j visible to query i iff j <= i + diag
  int kv_end = Skv;
  if (CAUSAL) kv_end = min(Skv, q0 + BM + diag);
  const int n_kt = (kv_end + FT - 1) / FT;

  KT kt_ld;
  VT vt_ld;
  kt_ld.init(tid);
  vt_ld.init(tid);
  auto issue = [&](int t, float* kd, float* vd) {
    const int j0 = t * FT;
    const uint32_t rows = (uint32_t)min(Skv - j0, FT);
    kt_ld.load(Buf(K + kv_off + (size_t)j0 * D, rows * D * 4), kd, tid);
    vt_ld.load(Buf(V + kv_off + (size_t)j0 * D, rows * D * 4), vd, tid);
  };
  issue(0, Ks0, Vs0);

  // Q^T fragments (B operand of S^T = K Q^T).
  f32x4 qf[D / 8];
  {
    const uint32_t rows = (uint32_t)min(Sq - q0, BM);
    load_frags<D>(Buf(Q + ((size_t)bh * Sq + q0) * D, rows * D * 4),
                  (uint32_t)((wave * 32 + l32) * D) * 4, g, qf);
  }
  int koff = l32 * PK + 4 * g;  // row operand base
  int voff = 4 * g * PV + l32;  // column operand base
  asm volatile("" : "+v"(koff), "+v"(voff));

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = zero_f32x16();
  constexpr float RESCALE_SLACK = 8.0f;
  float m = -MATTN_INF, l = 0.f;

  auto step = [&](auto par, int t) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's copies of tile t landed
    __syncthreads();                     // everyone's, and tile t-1 is done everywhere
    if (t + 1 < n_kt) {
      const std::integral_constant<int, decltype(par)::value ^ 1> other;
      issue(t + 1, Ks(other), Vs(other));
    }
    f32x16 s;
    rows_times_frags<D>(Ks(par), koff, qf, s);
    const int j0 = t * FT;
    const bool masked = (j0 + FT > Skv) || (CAUSAL && j0 + FT - 1 > qw + diag);
    float mx = -MATTN_INF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float tv = s[i] * c;
      if (masked) {
        const int key = j0 + crow(i, g);
        const bool ok = key < Skv && (!CAUSAL || key <= qrow + diag);
        tv = ok ? tv : -MATTN_INF;
      }
      s[i] = tv;
      mx = fmaxf(mx, tv);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (wave_any(mx > m + RESCALE_SLACK)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = (m_new == -MATTN_INF) ? 1.f : fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
    const float m_use = (m == -MATTN_INF) ? 0.f : m;
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(s[i] - m_use);
      rs[i & 3] += p;
      s[i] = p;
    }
    l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    cols_times_c<D, PV>(Vs(par), voff, s, acc);  // O^T += V^T P^T
  };
  int t = 0;
  for (; t + 2 <= n_kt; t += 2) {
    step(Even{}, t);
    step(Odd{}, t + 1);
  }
  if (t < n_kt) step(Even{}, t);

  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  store_rows_f32<D>(acc, inv, O + (size_t)bh * Sq * D, qrow, Sq, g);
  if (g == 0 && qrow < Sq)
    LSE[(size_t)bh * Sq + qrow] = lt > 0.f ? (m + log2f(lt)) * MATTN_LN2 : -MATTN_INF;
}

// ----------------------------------------------------------------------------
// dQ.  WAVES waves, 32 query rows each; Q^T and dO^T resident.
template <int D, bool CAUSAL, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 4 / WAVES)
void dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                   const float* __restrict__ V, const float* __restrict__ dO,
                   const float* __restrict__ LSE, const float* __restrict__ DLT,
                   float* __restrict__ dQ, int Hq, int G, int Sq, int Skv, float scale, float c,
                   int n_qt) {
  constexpr int NT = 64 * WAVES, BM = 32 * WAVES;
  constexpr int P = F32Pitch<D>::ROW;
  using TT = F32Tile<D, P, NT>;
  __shared__ __attribute__((aligned(16))) float Ks0[TT::FLOATS];
  __shared__ __attribute__((aligned(16))) float Ks1[TT::FLOATS];
  __shared__ __attribute__((aligned(16))) float Vs0[TT::FLOATS];
  __shared__ __attribute__((aligned(16))) float Vs1[TT::FLOATS];
  auto Ks = [&](auto par) -> float* {
    if constexpr (decltype(par)::value == 0) return Ks0; else return Ks1;
  };
  auto Vs = [&](auto par) -> float* {
    if constexpr (decltype(par)::value == 0) return Vs0; else return Vs1;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  int bh, qt;
  tile_of_block(blockIdx.x, gridDim.x / n_qt, n_qt, CAUSAL, bh, qt);
  const int b = bh / Hq, h = bh - b * Hq;
  const size_t kv_off = (size_t)(b * (Hq / G) + h / G) * Skv * D;
  const int q0 = qt * BM;
  const int qw = q0 + wave * 32;
  const int qrow = qw + l32;
  const int diag = Skv - Sq;
  int kv_end = Skv;
  if (CAUSAL) kv_end = min(Skv, q0 + BM + diag);
  const int n_kt = (kv_end + FT - 1) / FT;

  TT ld;
  ld.init(tid);
  auto issue = [&](int t, float* kd, float* vd) {
    const int j0 = t * FT;
    const uint32_t rows = (uint32_t)min(Skv - j0, FT);
    ld.load(Buf(K + kv_off + (size_t)j0 * D, rows * D * 4), kd, tid);
    ld.load(Buf(V + kv_off + (size_t)j0 * D, rows * D * 4), vd, tid);
  };
  issue(0, Ks0, Vs0);

  f32x4 qf[D / 8], dof[D / 8];
  {
    const uint32_t rows = (uint32_t)min(Sq - q0, BM);
    const size_t base = ((size_t)bh * Sq + q0) * D;
    const uint32_t roff = (uint32_t)((wave * 32 + l32) * D) * 4;
    load_frags<D>(Buf(Q + base, rows * D * 4), roff, g, qf);
    load_frags<D>(Buf(dO + base, rows * D * 4), roff, g, dof);
  }
  // Rows past Sq: LSE = +inf makes their P zero.
  const float lse2 = qrow < Sq ? LSE[(size_t)bh * Sq + qrow] * MATTN_LOG2E : MATTN_INF;
  const float dl = qrow < Sq ? DLT[(size_t)bh * Sq + qrow] : 0.f;
  int roff = l32 * P + 4 * g;
  int coff = 4 * g * P + l32;
  asm volatile("" : "+v"(roff), "+v"(coff));

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = zero_f32x16();

  auto step = [&](auto par, int t) {
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (t + 1 < n_kt) {
      const std::integral_constant<int, decltype(par)::value ^ 1> other;
      issue(t + 1, Ks(other), Vs(other));
    }
    f32x16 s, dp;
    rows_times_frags<D>(Ks(par), roff, qf, s);   // S^T = K Q^T
    rows_times_frags<D>(Vs(par), roff, dof, dp);  // dP^T = V dO^T
    const int j0 = t * FT;
    const bool masked = (j0 + FT > Skv) || (CAUSAL && j0 + FT - 1 > qw + diag);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = fast_exp2(s[i] * c - lse2);
      if (masked) {
        const int key = j0 + crow(i, g);
        if (!(key < Skv && (!CAUSAL || key <= qrow + diag))) p = 0.f;
      }
      s[i] = p * (dp[i] - dl);  // dS^T
    }
    cols_times_c<D, P>(Ks(par), coff, s, acc);  // dQ^T += K^T dS^T
  };
  int t = 0;
  for (; t + 2 <= n_kt; t += 2) {
    step(Even{}, t);
    step(Odd{}, t + 1);
  }
  if (t < n_kt) step(Even{}, t);
  store_rows_f32<D>(acc, scale, dQ + (size_t)bh * Sq * D, qrow, Sq, g);
}

// ----------------------------------------------------------------------------
// dK/dV.  WAVES waves, 32 keys each, of one KV head; K^T and V^T resident.
// The walk takes the 32-row query tiles of every query head of the group, in
// ascending head order, from the first tile that can see the workgroup's
// first key.  Rows past Sq load as zeros (Q, dO, LSE, D): their P is finite
// and their dO and dS are zero, so they add nothing.
template <int D, bool CAUSAL, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 4 / WAVES)
void dkdv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                     const float* __restrict__ V, const float* __restrict__ dO,
                     const float* __restrict__ LSE, const float* __restrict__ DLT,
                     float* __restrict__ dK, float* __restrict__ dV, int Hq, int G, int Sq,
                     int Skv, float scale, float c, int n_kt) {
  constexpr int NT = 64 * WAVES, BN = 32 * WAVES;
  constexpr int P = F32Pitch<D>::ROW;
  using TT = F32Tile<D, P, NT>;
  __shared__ __attribute__((aligned(16))) float Qs0[TT::FLOATS];
  __shared__ __attribute__((aligned(16))) float Qs1[TT::FLOATS];
  __shared__ __attribute__((aligned(16))) float dOs0[TT::FLOATS];
  __shared__ __attribute__((aligned(16))) float dOs1[TT::FLOATS];
  // LSE and D of a tile's rows: one 4-byte copy per lane of a wave (64 slots).
  __shared__ __attribute__((aligned(16))) float Ls0[64];
  __shared__ __attribute__((aligned(16))) float Ls1[64];
  __shared__ __attribute__((aligned(16))) float Ds0[64];
  __shared__ __attribute__((aligned(16))) float Ds1[64];
  auto Qs = [&](auto par) -> float* {
    if constexpr (decltype(par)::value == 0) return Qs0; else return Qs1;
  };
  auto dOs = [&](auto par) -> float* {
    if constexpr (decltype(par)::value == 0) return dOs0; else return dOs1;
  };
  auto Ls = [&](auto par) -> float* {
    if constexpr (decltype(par)::value == 0) return Ls0; else return Ls1;
  };
  auto Ds = [&](auto par) -> float* {
    if constexpr (decltype(par)::value == 0) return Ds0; else return Ds1;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int Hkv = Hq / G;
  // Longest causal walks (first key tiles) first; tile_of_block puts the
  // highest tile index first, so count key tiles from the end.
  int bkv, ktr;
  tile_of_block(blockIdx.x, gridDim.x / n_kt, n_kt, CAUSAL, bkv, ktr);
  const int kt = CAUSAL ? n_kt - 1 - ktr : ktr;
  const int b = bkv / Hkv, kvh = bkv - b * Hkv;
  const int k0 = kt * BN;
  const int key = k0 + wave * 32 + l32;  // this lane's key
  const int diag = Skv - Sq;
  int q_lo = 0;
  if (CAUSAL && k0 - diag > 0) q_lo = ((k0 - diag) / FT) * FT;
  const int nq = Sq > q_lo ? (Sq - q_lo + FT - 1) / FT : 0;
  const int n_it = G * nq;

  TT ld;
  ld.init(tid);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int it, float* qd, float* dod, float* ld_, float* dd) {
    const int h = kvh * G + it / nq;
    const int qt0 = q_lo + (it % nq) * FT;
    const size_t row0 = (size_t)(b * Hq + h) * Sq + qt0;
    const uint32_t rows = (uint32_t)min(Sq - qt0, FT);
    ld.load(Buf(Q + row0 * D, rows * D * 4), qd, tid);
    ld.load(Buf(dO + row0 * D, rows * D * 4), dod, tid);
    if (wv == 0) ld4_to_lds(Buf(LSE + row0, rows * 4), lane * 4, ld_);
    if (wv == (WAVES > 1 ? 1 : 0)) ld4_to_lds(Buf(DLT + row0, rows * 4), lane * 4, dd);
  };
  if (n_it > 0) issue(0, Qs0, dOs0, Ls0, Ds0);

  f32x4 kf[D / 8], vf[D / 8];
  {
    const uint32_t rows = (uint32_t)max(0, min(Skv - k0, BN));
    const size_t base = ((size_t)bkv * Skv + k0) * D;
    const uint32_t roff = (uint32_t)((wave * 32 + l32) * D) * 4;
    load_frags<D>(Buf(K + base, rows * D * 4), roff, g, kf);
    load_frags<D>(Buf(V + base, rows * D * 4), roff, g, vf);
  }
  int roff = l32 * P + 4 * g;
  int coff = 4 * g * P + l32;
  asm volatile("" : "+v"(roff), "+v"(coff));

  f32x16 adk[D / 32], adv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) adk[db] = adv[db] = zero_f32x16();

  auto step = [&](auto par, int it) {
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (it + 1 < n_it) {
      const std::integral_constant<int, decltype(par)::value ^ 1> o;
      issue(it + 1, Qs(o), dOs(o), Ls(o), Ds(o));
    }
    const int qt0 = q_lo + (it % nq) * FT;
    f32x16 s;
    rows_times_frags<D>(Qs(par), roff, kf, s);  // S = Q K^T (rows = queries, lane = key)
    // Register i holds query row qt0 + crow(i, g) = qt0 + 8(i/4) + 4g + i%4.
    const bool masked = CAUSAL && (k0 + wave * 32 + 31 > qt0 + diag);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const f32x4 lv = *reinterpret_cast<const f32x4*>(Ls(par) + 8 * mb + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * mb + e;
        float p = fast_exp2(s[i] * c - lv[e] * MATTN_LOG2E);
        if (masked && key > qt0 + crow(i, g) + diag) p = 0.f;
        s[i] = p;
      }
    }
    cols_times_c<D, P>(dOs(par), coff, s, adv);  // dV^T += dO^T P
    f32x16 dp;
    rows_times_frags<D>(dOs(par), roff, vf, dp);  // dP = dO V^T
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const f32x4 dv4 = *reinterpret_cast<const f32x4*>(Ds(par) + 8 * mb + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * mb + e;
        s[i] = s[i] * (dp[i] - dv4[e]);  // dS
      }
    }
    cols_times_c<D, P>(Qs(par), coff, s, adk);  // dK^T += Q^T dS
  };
  int it = 0;
  for (; it + 2 <= n_it; it += 2) {
    step(Even{}, it);
    step(Odd{}, it + 1);
  }
  if (it < n_it) step(Even{}, it);

  const size_t out = (size_t)bkv * Skv * D;
  store_rows_f32<D>(adk, scale, dK + out, key, Skv, g);
  store_rows_f32<D>(adv, 1.f, dV + out, key, Skv, g);
}

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Waves per workgroup: four (128 rows or keys) whenever that still gives
// every CU a workgroup, otherwise fewer so that small problems spread over
// more CUs.  The K/V (or Q/dO) tiles take the same LDS whatever the number
// of waves, so LDS, not registers, limits how many workgroups share a CU,
// and the four-wave shape keeps the most waves per CU.
int f32_waves(long long units) {
  if ((units + 127) / 128 >= 256) return 4;
  if ((units + 63) / 64 >= 256) return 2;
  return 1;
}

template <int D, bool CAUSAL, int W>
hipError_t fwd_f32_w(const Problem& p, const float* q, const float* k, const float* v, float* o,
                     float* lse, hipStream_t stream) {
  const int n_qt = (p.Sq + 32 * W - 1) / (32 * W);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, W>), dim3((unsigned)((long long)p.B * p.Hq * n_qt)),
                     dim3(64 * W), 0, stream, q, k, v, o, lse, p.Hq, p.Hq / p.Hkv, p.Sq, p.Skv,
                     p.scale * MATTN_LOG2E, n_qt);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t fwd_f32_t(const Problem& p, const float* q, const float* k, const float* v, float* o,
                     float* lse, hipStream_t stream) {
  switch (f32_waves((long long)p.B * p.Hq * (((long long)p.Sq + 31) / 32 * 32))) {
    case 4: return fwd_f32_w<D, CAUSAL, 4>(p, q, k, v, o, lse, stream);
    case 2: return fwd_f32_w<D, CAUSAL, 2>(p, q, k, v, o, lse, stream);
    default: return fwd_f32_w<D, CAUSAL, 1>(p, q, k, v, o, lse, stream);
  }
}

template <int D, bool CAUSAL, int W>
hipError_t dq_f32_w(const Problem& p, const float* q, const float* k, const float* v,
                    const float* lse, const float* dlt, const float* dout, float* dq,
                    hipStream_t stream) {
  const int n_qt = (p.Sq + 32 * W - 1) / (32 * W);
  hipLaunchKernelGGL((dq_f32_kernel<D, CAUSAL, W>), dim3((unsigned)((long long)p.B * p.Hq * n_qt)),
                     dim3(64 * W), 0, stream, q, k, v, dout, lse, dlt, dq, p.Hq, p.Hq / p.Hkv,
                     p.Sq, p.Skv, p.scale, p.scale * MATTN_LOG2E, n_qt);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dq_f32_t(const Problem& p, const float* q, const float* k, const float* v,
                    const float* lse, const float* dlt, const float* dout, float* dq,
                    hipStream_t stream) {
  switch (f32_waves((long long)p.B * p.Hq * (((long long)p.Sq + 31) / 32 * 32))) {
    case 4: return dq_f32_w<D, CAUSAL, 4>(p, q, k, v, lse, dlt, dout, dq, stream);
    case 2: return dq_f32_w<D, CAUSAL, 2>(p, q, k, v, lse, dlt, dout, dq, stream);
    default: return dq_f32_w<D, CAUSAL, 1>(p, q, k, v, lse, dlt, dout, dq, stream);
  }
}

template <int D, bool CAUSAL, int W>
hipError_t dkdv_f32_w(const Problem& p, const float* q, const float* k, const float* v,
                      const float* lse, const float* dlt, const float* dout, float* dk, float* dv,
                      hipStream_t stream) {
  const int n_kt = (p.Skv + 32 * W - 1) / (32 * W);
  hipLaunchKernelGGL((dkdv_f32_kernel<D, CAUSAL, W>),
                     dim3((unsigned)((long long)p.B * p.Hkv * n_kt)), dim3(64 * W), 0, stream, q,
                     k, v, dout, lse, dlt, dk, dv, p.Hq, p.Hq / p.Hkv, p.Sq, p.Skv, p.scale,
                     p.scale * MATTN_LOG2E, n_kt);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dkdv_f32_t(const Problem& p, const float* q, const float* k, const float* v,
                      const float* lse, const float* dlt, const float* dout, float* dk, float* dv,
                      hipStream_t stream) {
  switch (f32_waves((long long)p.B * p.Hkv * (((long long)p.Skv + 31) / 32 * 32))) {
    case 4: return dkdv_f32_w<D, CAUSAL, 4>(p, q, k, v, lse, dlt, dout, dk, dv, stream);
    case 2: return dkdv_f32_w<D, CAUSAL, 2>(p, q, k, v, lse, dlt, dout, dk, dv, stream);
    default: return dkdv_f32_w<D, CAUSAL, 1>(p, q, k, v, lse, dlt, dout, dk, dv, stream);
  }
}

}  // namespace

hipError_t launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v,
                          float* o, float* lse, hipStream_t stream) {
  if (p.D == 64) return p.causal ? fwd_f32_t<64, true>(p, q, k, v, o, lse, stream)
                                 : fwd_f32_t<64, false>(p, q, k, v, o, lse, stream);
  return p.causal ? fwd_f32_t<128, true>(p, q, k, v, o, lse, stream)
                  : fwd_f32_t<128, false>(p, q, k, v, o, lse, stream);
}

hipError_t launch_dkdv_f32(const Problem& p, const float* q, const float* k, const float* v,
                           const float* lse, const float* dlt, const float* dout, float* dk,
                           float* dv, hipStream_t stream) {
  if (p.D == 64)
    return p.causal ? dkdv_f32_t<64, true>(p, q, k, v, lse, dlt, dout, dk, dv, stream)
                    : dkdv_f32_t<64, false>(p, q, k, v, lse, dlt, dout, dk, dv, stream);
  return p.causal ? dkdv_f32_t<128, true>(p, q, k, v, lse, dlt, dout, dk, dv, stream)
                  : dkdv_f32_t<128, false>(p, q, k, v, lse, dlt, dout, dk, dv, stream);
}

hipError_t launch_dq_f32(const Problem& p, const float* q, const float* k, const float* v,
                         const float* lse, const float* dlt, const float* dout, float* dq,
                         hipStream_t stream) {
  if (p.D == 64)
    return p.causal ? dq_f32_t<64, true>(p, q, k, v, lse, dlt, dout, dq, stream)
                    : dq_f32_t<64, false>(p, q, k, v, lse, dlt, dout, dq, stream);
  return p.causal ? dq_f32_t<128, true>(p, q, k, v, lse, dlt, dout, dq, stream)
                  : dq_f32_t<128, false>(p, q, k, v, lse, dlt, dout, dq, stream);
}

hipError_t launch_zero_words(void* p, size_t n_words, hipStream_t stream) {
  if (n_words == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((n_words + 255) / 256)), dim3(256), 0,
                     stream, (uint32_t*)p, n_words);
  return hipGetLastError();
}

}  // namespace mattn

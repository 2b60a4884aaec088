// Fused attention forward, bf16 I/O, fp32 softmax statistics and accumulation.
//
// The method is the fused flash-attention forward of the xtrain evolution
// page (infrastructure-phase table, row T14): one kernel, an online softmax
// walking K/V in tiles, the score matrix never materialised.  Grouped KV
// heads follow row T15 (query head h reads KV head h / G), here by index
// arithmetic with no repeated K/V.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one head,
// or 8 waves = 256 rows of one head or 128 rows of each of two query heads
// that read the same KV head):
//  * each wave owns 32 query rows and keeps them as the B operand of
//    S^T = K Q^T in registers for the whole kernel (lane = query column);
//  * K/V tiles of 64 keys are copied straight from global memory into
//    double-buffered LDS (buffer_load ... lds), one barrier per tile, for
//    head dim 128 in the grouped layout of grp_layout.hpp (each copy
//    instruction writes four whole rows, no padding); K rows
//    are the A operand of S^T, and the A operand of O^T = V^T P^T is read
//    transposed straight from the V tile with ds_read_b64_tr_b16, in the key
//    order that P^T carries out of the S^T accumulator;
//  * S^T lands with one query per lane, so the running row max and row sum
//    are per-lane scalars: 32 in-lane values plus one exchange with lane^32;
//  * P is rounded to bf16 and fed to the PV MFMA straight from registers;
//  * O^T accumulates in fp32 registers, one query per lane, so the online
//    rescale is one multiply by a per-lane factor;
//  * the walk is software-pipelined one tile deep: while the MFMAs of
//    S(t+1) run, the same wave computes the exponentials of tile t, and the
//    row max of S(t+1) is taken under the MFMAs of O += P(t) V(t), so the
//    softmax arithmetic issues between matrix instructions instead of
//    after them.
// Softmax runs in the log2 domain: t = s * scale * log2(e), p = 2^(t - m).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace mattn {

namespace {

// WAVES waves per workgroup, each owning QB blocks of 32 query rows of one of
// the workgroup's HPW query heads (HPW > 1 only for heads that share a KV
// head, so that every wave reads the same K/V tiles).  The code is written
// for any QB, but QB = 1: two blocks per wave (one wave per SIMD with up to
// 512 registers, each K/V fragment feeding two MFMAs) made the register
// allocator spill heavily.  Four waves run two workgroups per CU; eight run
// one, which halves the K/V bytes copied into each CU's LDS per query row.
template <int D, int WAVES_, int HPW_>
struct FwdTile {
  static constexpr int QB = 1;
  static constexpr int BN = 64;       // keys per tile
  static constexpr int KB = BN / 32;  // 32-key blocks per tile
  static constexpr int WAVES = WAVES_;
  static constexpr int HPW = HPW_;    // query heads per workgroup
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WPH = WAVES / HPW;        // waves per query head
  static constexpr int BM = 32 * QB * WPH;       // query rows per workgroup
  static_assert(WAVES % HPW == 0, "waves per head");
  // D = 128: K and V tiles in the GrpTile128 layout (copies write no
  // padding); D = 64: padded row-major tiles.
  static constexpr bool GRP = D == 128;
  static constexpr int KP = RowPitch<D>::value;  // K tile: read as row operands
  static constexpr int VP = TrPitch<D>::value;   // V tile: read transposed
  using KTile = DirectTile<D, BN, KP, THREADS>;
  using VTile = DirectTile<D, BN, VP, THREADS>;
  static constexpr int K_ELEMS = GRP ? GrpTile128::bytes(BN) / 2 : KTile::LDS_ELEMS;
  static constexpr int V_ELEMS = GRP ? GrpTile128::bytes(BN) / 2 : VTile::LDS_ELEMS;
};

template <int D, bool CAUSAL, int WAVES, int HPW>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? 2 : 1)
void fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, bf16* __restrict__ O,
                     float* __restrict__ LSE, int Hq, int G, int Sq, int Skv,
                     float c /* scale*log2(e) */, int n_qt) {
  using T = FwdTile<D, WAVES, HPW>;
  constexpr int QB = T::QB, KB = T::KB, FWD_BN = T::BN;
  // Double-buffered K and V tiles, filled straight from global memory.  Each
  // buffer is its own LDS object: the compiler tracks copies in flight per
  // object, so reading one buffer does not wait for copies into another.
  __shared__ __attribute__((aligned(16))) bf16 Ks0[T::K_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 Ks1[T::K_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 Vs0[T::V_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 Vs1[T::V_ELEMS];
  auto Ks = [&](auto parity) -> bf16* {
    if constexpr (decltype(parity)::value == 0) return Ks0; else return Ks1;
  };
  auto Vs = [&](auto parity) -> bf16* {
    if constexpr (decltype(parity)::value == 0) return Vs0; else return Vs1;
  };
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  // Workgroup -> (batch, group of HPW query heads, query tile); this wave's
  // head within the group, and its rows within the tile.
  int bg, qt;
  tile_of_block(blockIdx.x, gridDim.x / n_qt, n_qt, CAUSAL, bg, qt);
  const int hg = Hq / HPW;  // head groups per batch entry
  const int b = bg / hg;
  const int h0 = (bg - b * hg) * HPW;  // first head of the group
  // Wave-uniform; readfirstlane keeps the Q descriptor in scalar registers.
  const int h = __builtin_amdgcn_readfirstlane(h0 + wave / T::WPH);
  const int bh = b * Hq + h;
  const int Hkv = Hq / G;
  const size_t kv_off = ((size_t)(b * Hkv + h0 / G) * Skv) * D;
  const bf16* Kh = K + kv_off;
  const bf16* Vh = V + kv_off;
  const Buf qbuf(Q + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);

  const int q0 = qt * T::BM;
  const int qw0 = q0 + (wave % T::WPH) * 32 * QB;  // first query of this wave
  const int diag = Skv - Sq;               // key j visible to query i iff j <= i + diag
  auto qrow_of = [&](int qb) { return qw0 + 32 * qb + l32; };  // this lane's queries

  // Q fragments, B operands of S^T = K Q^T: lane holds q[qrow][16s + 8g .. +7].
  // The kernel works with a positive multiplier: a negative scale negates Q
  // (exact in bf16) and a zero scale zeroes it (every visible score is then
  // 0, whatever the multiplier).
  bf16x8 qf[QB][D / 16];

  int kv_end = Skv;
  if (CAUSAL) kv_end = min(Skv, q0 + T::BM + diag);
  const int n_kt = (kv_end + FWD_BN - 1) / FWD_BN;

  typename T::KTile kt_ld;
  typename T::VTile vt_ld;
  GrpCopy<FWD_BN, WAVES> gcp;  // D = 128: one copy pattern serves K and V
  if constexpr (T::GRP) {
    gcp.init(__builtin_amdgcn_readfirstlane(wave), lane);
  } else {
    kt_ld.init(tid);
    vt_ld.init(tid);
  }
  // Tile t's descriptors start at its first row and end at Skv, so rows past
  // the end (and pad slots) read as zeros.
  // Tile t goes to buffer t & 1; callers pass that parity as a compile-time
  // constant, so that every LDS address names its buffer statically and the
  // compiler can see that reads of one buffer do not depend on copies still
  // in flight to the other.
  auto issue_k = [&](int t, bf16* dst) {
    const int j0 = t * FWD_BN;
    const Buf src(Kh + (size_t)j0 * D, (uint32_t)(Skv - j0) * D * 2);
    if constexpr (T::GRP) gcp.load(src, dst); else kt_ld.load(src, dst, tid);
  };
  auto issue_v = [&](int t, bf16* dst) {
    const int j0 = t * FWD_BN;
    const Buf src(Vh + (size_t)j0 * D, (uint32_t)(Skv - j0) * D * 2);
    if constexpr (T::GRP) gcp.load(src, dst); else vt_ld.load(src, dst, tid);
  };
  GrpTile128 gt;  // D = 128 operand reads
  if constexpr (T::GRP) gt.init(lane);
  // Whether some key of tile t is invisible to some query of this wave.
  auto tile_masked = [&](int t) {
    const int j0 = t * FWD_BN;
    return (j0 + FWD_BN > Skv) || (CAUSAL && (j0 + FWD_BN - 1 > qw0 + diag));
  };

  f32x16 acc[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[qb][db] = zero_f32x16();
  // Per query block: reference max m of t = s*c for this lane's query
  // (shared by lane and lane^32) and this lane's partial row sum relative to
  // it.  The reference only moves when a tile's max exceeds it by more than
  // RESCALE_SLACK (log2 units), so most tiles skip the O rescale;
  // p <= 2^RESCALE_SLACK stays well inside fp32/bf16 range and O / l is
  // unchanged.
  constexpr float RESCALE_SLACK = 8.0f;
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m[qb] = -MATTN_INF; l[qb] = 0.f; }
  bf16x8 pb[QB][KB][2];  // P^T of the current tile, B operands of O^T += V^T P^T

  // S^T = K Q^T for one 64-key tile: per query block, two 32-key blocks
  // (lane = query column, registers = keys); each K fragment feeds QB MFMAs.
  auto s_tile = [&](const bf16* Kb, f32x16 (&sc)[QB][KB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sc[qb][kb] = zero_f32x16();
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        bf16x8 a;
        if constexpr (T::GRP) a = gt.row(Kb, kb * 32, st);
        else a = ld_row_operand(Kb, T::KP, kb * 32, 16 * st, lane);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sc[qb][kb] = mfma32(a, qf[qb][st], sc[qb][kb]);
      }
  };
  // Row max of a tile's raw scores; the masked form first overwrites
  // invisible keys (past Skv, or above the causal diagonal) with -inf.
  auto max_plain = [&](const f32x16 (&sc)[KB]) {
    float mx = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
    return mx;
  };
  auto max_masked = [&](f32x16 (&sc)[KB], int t, int qrow) {
    // Key t*BN + 32 kb + crow(i, g) is visible iff it is at most the last
    // visible key, i.e. iff crow(i, 0) <= lim - 32 kb: one compare with a
    // constant per element.
    int last = Skv - 1;
    if (CAUSAL) last = min(last, qrow + diag);
    const int lim = last - t * FWD_BN - 4 * g;
    float mx = -MATTN_INF;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = crow(i, 0) <= lim - 32 * kb;
        sc[kb][i] = ok ? sc[kb][i] : -MATTN_INF;
        mx = fmaxf(mx, sc[kb][i]);
      }
    return mx;
  };
  // Move block qb's reference if the tile's max (lane and lane^32 together)
  // passed it by more than the slack; O and l are rescaled to the new one.
  auto update_ref = [&](int qb, float mx) {
    float mt = mx * c;
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    if (wave_any(mt > m[qb] + RESCALE_SLACK)) {
      const float m_new = fmaxf(m[qb], mt);
      const float alpha = (m_new == -MATTN_INF) ? 1.f : fast_exp2(m[qb] - m_new);
      m[qb] = m_new;
      l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[qb][db][i] *= alpha;
    }
  };
  // P = 2^(t - m) for one 32-key block, rounded to bf16 for the PV product;
  // the row sum stays fp32, in four partial sums so that the adds do not
  // form one long dependent chain.
  auto exp_block = [&](const f32x16& sc, int qb, int kb, float (&rs)[4]) {
    const float m_use = (m[qb] == -MATTN_INF) ? 0.f : m[qb];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(__builtin_fmaf(sc[i], c, -m_use));
      rs[i & 3] += p;
      pb[qb][kb][i >> 3][i & 7] = (bf16)p;
    }
  };
  // O^T += V^T P^T; each V^T fragment feeds QB MFMAs.
  TransReader vtr;
  if constexpr (!T::GRP) vtr.init(T::VP, lane);
  auto pv_tile = [&](const bf16* Vb) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 a[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          if constexpr (T::GRP) a[db] = gt.trans(Vb, kb * 32 + 16 * t, db);
          else a[db] = vtr(Vb, T::VP, kb * 32 + 16 * t, db * 32);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma32(a[db], pb[qb][kb][t], acc[qb][db]);
      }
  };

  // Software pipeline over key tiles.  Step t holds S(t) in registers and
  // runs, interleaved instruction by instruction:
  //   phase 1: the MFMAs of S(t+1)  with  the exponentials of tile t;
  //   phase 2: the MFMAs of O += P(t) V(t)  with  the row max of S(t+1);
  // then moves the reference max for tile t+1.  K runs one tile ahead of V:
  // step t reads K(t+1) and V(t) and loads K(t+2) and V(t+1) behind them,
  // one barrier per step.
  constexpr int NMF = QB * KB * (D / 16);  // MFMAs per phase
  auto step = [&](auto p0, int t, f32x16 (&cur)[QB][KB], f32x16 (&nxt)[QB][KB]) {
    // p0 = t & 1, p1 = the other buffer
    const std::integral_constant<int, decltype(p0)::value ^ 1> p1;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's copies landed
    __syncthreads();                     // everyone's, and step t-1 is done everywhere
    if (t + 2 < n_kt) issue_k(t + 2, Ks(p0));
    issue_v(t + 1, Vs(p1));
    float rs[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) rs[qb][i] = 0.f;
    // Phase 1: the MFMAs of S(t+1) with the 112 VALU instructions per query
    // block that turn S(t) into P(t): five after each MFMA, the rest after
    // the last (measured 1-3% faster than spreading them evenly), with the
    // K operand reads eight MFMAs ahead.
    s_tile(Ks(p1), nxt);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) exp_block(cur[qb][kb], qb, kb, rs[qb]);
#pragma unroll
    for (int i = 0; i < 8; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Pin the row sums here: left alone, the compiler sinks the adds past the
    // branch below and keeps every p live in fp32 until then.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      asm volatile("" : "+v"(rs[qb][0]), "+v"(rs[qb][1]), "+v"(rs[qb][2]), "+v"(rs[qb][3]));
      l[qb] += (rs[qb][0] + rs[qb][1]) + (rs[qb][2] + rs[qb][3]);
    }
    // Phase 2: the MFMAs of O += P(t) V(t) with the row max of S(t+1).  Each
    // V^T fragment is two transposed reads; they run four fragments ahead of
    // the MFMA that uses them (two fragments ahead measured 3-6% slower).
    float mx[QB];
    if (tile_masked(t + 1)) {
      pv_tile(Vs(p0));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mx[qb] = max_masked(nxt[qb], t + 1, qrow_of(qb));
#pragma unroll
      for (int i = 0; i < 8; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int i = 0; i < NMF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    } else {
      pv_tile(Vs(p0));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mx[qb] = max_plain(nxt[qb]);
#pragma unroll
      for (int i = 0; i < 8; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int i = 0; i < NMF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) update_ref(qb, mx[qb]);
  };
  auto last_step = [&](auto p0, f32x16 (&cur)[QB][KB]) {
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) exp_block(cur[qb][kb], qb, kb, rs);
      l[qb] += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    }
    pv_tile(Vs(p0));
  };

  f32x16 sa[QB][KB], sb[QB][KB];
  issue_k(0, Ks(Even{}));
  if (n_kt > 1) issue_k(1, Ks(Odd{}));
  issue_v(0, Vs(Even{}));
  // Q after the first copies: the tile copies then do not queue behind the
  // Q loads (each of which touches 32 rows).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[qb][s] = as_bf16x8(qbuf.ld16((uint32_t)(qrow_of(qb) * D + 16 * s + 8 * g) * 2));
  if (!(c > 0.f)) {
    const uint32_t flip = c < 0.f ? 0x80008000u : 0u, keep = c < 0.f ? ~0u : 0u;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        uint4 u = __builtin_bit_cast(uint4, qf[qb][s]);
        u.x = (u.x & keep) ^ flip; u.y = (u.y & keep) ^ flip;
        u.z = (u.z & keep) ^ flip; u.w = (u.w & keep) ^ flip;
        qf[qb][s] = as_bf16x8(u);
      }
    c = c < 0.f ? -c : 1.f;
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  s_tile(Ks(Even{}), sa);
  {
    const bool mk = tile_masked(0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      update_ref(qb, mk ? max_masked(sa[qb], 0, qrow_of(qb)) : max_plain(sa[qb]));
  }
  // Two steps per trip so that S(t) and S(t+1) swap registers without copies.
  // t stays even, so the parity of each call is known.
  int t = 0;
  for (; t + 2 < n_kt; t += 2) {
    step(Even{}, t, sa, sb);
    step(Odd{}, t + 1, sb, sa);
  }
  if (t + 2 == n_kt) {
    step(Even{}, t, sa, sb);
    last_step(Odd{}, sb);
  } else {
    last_step(Even{}, sa);
  }

  // O rows through LDS (store_rows_bf16), staged two waves per tile buffer
  // once every wave is past the last tile's reads (four buffers serve eight
  // waves).
  static_assert(QB == 1, "one 32-row block per wave");
  static_assert(2 * stage_rows_bytes<D>() <= 2 * (T::K_ELEMS < T::V_ELEMS ? T::K_ELEMS : T::V_ELEMS),
                "two waves' staging fits a tile buffer");
  __syncthreads();
  {
    const int sw = wave >> 1;
    bf16* sbuf = sw == 0 ? Ks0 : sw == 1 ? Ks1 : sw == 2 ? Vs0 : Vs1;
    char* stg = reinterpret_cast<char*>(sbuf) + (wave & 1) * stage_rows_bytes<D>();
    const float lt = l[0] + __shfl_xor(l[0], 32);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    store_rows_bf16<D>(acc[0], inv, stg, O + ((size_t)bh * Sq + qw0) * D, Sq - qw0, lane);
    const int qrow = qrow_of(0);
    if (g == 0 && qrow < Sq)
      LSE[(size_t)bh * Sq + qrow] = lt > 0.f ? (m[0] + log2f(lt)) * MATTN_LN2 : -MATTN_INF;
  }
}

}  // namespace

template <int D, bool CAUSAL, int WAVES, int HPW>
static hipError_t launch_fwd(const Problem& p, const void* q, const void* k, const void* v,
                             void* o, float* lse, hipStream_t stream) {
  using T = FwdTile<D, WAVES, HPW>;
  const int n_qt = (p.Sq + T::BM - 1) / T::BM;
  const long long blocks = (long long)p.B * (p.Hq / HPW) * n_qt;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, WAVES, HPW>), dim3((unsigned)blocks),
                     dim3(T::THREADS), 0, stream, (const bf16*)q, (const bf16*)k, (const bf16*)v,
                     (bf16*)o, lse, p.Hq, p.Hq / p.Hkv, p.Sq, p.Skv, p.scale * MATTN_LOG2E, n_qt);
  return hipGetLastError();
}

// Workgroup shape.  Eight waves (one workgroup per CU) copy half the K/V bytes
// per query row into LDS, which pays once a workgroup walks many key tiles;
// with grouped heads they take two query heads of one KV head (128 rows
// each, so causal masking wastes no more than with four waves), or, causal
// with groups of four or more, four heads of 64 rows each (less masked work
// on the diagonal and twice as many, shorter, causal workgroups to balance
// the CUs); otherwise 256 rows of one head (causal rows then walk up to 224
// fully masked keys, so that shape is kept for non-causal attention).  Short
// key ranges and small grids keep four waves and two workgroups per CU.
template <int D, bool CAUSAL>
static hipError_t launch_fwd_shape(const Problem& p, const void* q, const void* k, const void* v,
                                   void* o, float* lse, hipStream_t stream) {
  if constexpr (D == 128) {
    const int G = p.Hq / p.Hkv;
    const bool long_kv = p.Skv >= 2048;
    if constexpr (CAUSAL)
      if (long_kv && G % 4 == 0 && (long long)p.B * (p.Hq / 4) * ((p.Sq + 63) / 64) >= 512)
        return launch_fwd<D, CAUSAL, 8, 4>(p, q, k, v, o, lse, stream);
    if (long_kv && G % 2 == 0 && (long long)p.B * (p.Hq / 2) * ((p.Sq + 127) / 128) >= 512)
      return launch_fwd<D, CAUSAL, 8, 2>(p, q, k, v, o, lse, stream);
    if constexpr (!CAUSAL)
      if (long_kv && (long long)p.B * p.Hq * ((p.Sq + 255) / 256) >= 512)
        return launch_fwd<D, CAUSAL, 8, 1>(p, q, k, v, o, lse, stream);
  }
  return launch_fwd<D, CAUSAL, 4, 1>(p, q, k, v, o, lse, stream);
}

hipError_t launch_fwd_bf16(const Problem& p, const void* q, const void* k, const void* v,
                           void* o, float* lse, hipStream_t stream) {
  if (p.D == 64) return p.causal ? launch_fwd_shape<64, true>(p, q, k, v, o, lse, stream)
                                 : launch_fwd_shape<64, false>(p, q, k, v, o, lse, stream);
  return p.causal ? launch_fwd_shape<128, true>(p, q, k, v, o, lse, stream)
                  : launch_fwd_shape<128, false>(p, q, k, v, o, lse, stream);
}

}  // namespace mattn

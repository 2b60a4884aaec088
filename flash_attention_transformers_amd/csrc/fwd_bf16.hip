// Fused attention forward, bf16 I/O, fp32 softmax statistics and accumulation.
//
// The method is the fused flash-attention forward of the xtrain evolution
// page (infrastructure-phase table, row T14): one kernel, an online softmax
// walking K/V in tiles, the score matrix never materialised.  Grouped KV
// heads follow row T15 (query head h reads KV head h / G), here by index
// arithmetic with no repeated K/V.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one head):
//  * each wave owns 32 query rows and keeps them as the B operand of
//    S^T = K Q^T in registers for the whole kernel (lane = query column);
//  * K/V tiles of 64 keys are copied straight from global memory into
//    double-buffered LDS (buffer_load ... lds), one tile ahead, one barrier
//    per tile; K rows are the A operand of S^T, and the A operand of
//    O^T = V^T P^T is read transposed straight from the V tile with
//    ds_read_b64_tr_b16, in the key order that P^T carries out of the S^T
//    accumulator;
//  * S^T lands with one query per lane, so the running row max and row sum
//    are per-lane scalars: 32 in-lane values plus one exchange with lane^32;
//  * P is rounded to bf16 and fed to the PV MFMA straight from registers;
//  * O^T accumulates in fp32 registers, one query per lane, so the online
//    rescale is one multiply by a per-lane factor.
// Softmax runs in the log2 domain: t = s * scale * log2(e), p = 2^(t - m).
#include "common.hpp"
#include "kernels.hpp"

namespace mattn {

namespace {

constexpr int FWD_BM = 128;
constexpr int FWD_BN = 64;
constexpr int FWD_THREADS = 256;

template <int D>
struct FwdTile {
  static constexpr int KP = RowPitch<D>::value;  // K tile: read as row operands
  static constexpr int VP = TrPitch<D>::value;   // V tile: read transposed
  using KTile = DirectTile<D, FWD_BN, KP, FWD_THREADS>;
  using VTile = DirectTile<D, FWD_BN, VP, FWD_THREADS>;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(FWD_THREADS, 2)
void fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, bf16* __restrict__ O,
                     float* __restrict__ LSE, int Hq, int G, int Sq, int Skv,
                     float c /* scale*log2(e) */, int n_qt) {
  using T = FwdTile<D>;
  // Double-buffered K and V tiles, filled straight from global memory.
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][FWD_BN * T::KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][FWD_BN * T::VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  int bh, qt;
  tile_of_block(blockIdx.x, gridDim.x / n_qt, n_qt, CAUSAL, bh, qt);
  const int h = bh % Hq, b = bh / Hq;
  const int Hkv = Hq / G;
  const size_t kv_off = ((size_t)(b * Hkv + h / G) * Skv) * D;
  const bf16* Kh = K + kv_off;
  const bf16* Vh = V + kv_off;
  const Buf qbuf(Q + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);

  const int q0 = qt * FWD_BM;
  const int qw0 = q0 + wave * 32;          // first query of this wave
  const int qrow = qw0 + l32;              // this lane's query
  const int diag = Skv - Sq;               // key j visible to query i iff j <= i + diag

  // Q fragment, B operand of S^T = K Q^T: lane holds q[qrow][16s + 8g .. +7].
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = as_bf16x8(qbuf.ld16((uint32_t)(qrow * D + 16 * s + 8 * g) * 2));

  int kv_end = Skv;
  if (CAUSAL) kv_end = min(Skv, q0 + FWD_BM + diag);
  const int n_kt = (kv_end + FWD_BN - 1) / FWD_BN;

  typename T::KTile kt_ld;
  typename T::VTile vt_ld;
  kt_ld.init(tid);
  vt_ld.init(tid);
  // Tile j0: descriptors start at row j0 and end at Skv, so rows past the
  // end (and pad slots) read as zeros.
  auto issue_tile = [&](int j0, int buf) {
    const uint32_t nb = (uint32_t)(Skv - j0) * D * 2;
    kt_ld.load(Buf(Kh + (size_t)j0 * D, nb), Ks[buf], tid);
    vt_ld.load(Buf(Vh + (size_t)j0 * D, nb), Vs[buf], tid);
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = zero_f32x16();
  // Reference max of t = s*c for this lane's query (shared by lane and
  // lane^32) and this lane's partial row sum relative to it.  The reference
  // only moves when a tile's max exceeds it by more than RESCALE_SLACK (log2
  // units), so most tiles skip the O rescale; p <= 2^RESCALE_SLACK stays well
  // inside fp32/bf16 range and O / l is unchanged.
  constexpr float RESCALE_SLACK = 8.0f;
  float m = -MATTN_INF, l = 0.f;

  if (n_kt > 0) issue_tile(0, 0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int j0 = kt * FWD_BN, buf = kt & 1;
    // This thread's copies of tile kt are done; after the barrier every
    // thread's are, and every wave has finished reading tile kt-1, so the
    // other buffer can be refilled.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); lgkm and exp counters untouched
    __syncthreads();
    if (kt + 1 < n_kt) issue_tile(j0 + FWD_BN, buf ^ 1);
    const bf16* Kb = Ks[buf];
    const bf16* Vb = Vs[buf];

    // S^T for two 32-key blocks: lane = query column, regs = keys.
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sc[kb] = zero_f32x16();
    {
      // All K fragments of the tile, issued ahead of the MFMAs that use them
      // (eight reads in flight before the first MFMA, then one per MFMA).
      bf16x8 a[D / 16][2];
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) a[st][kb] = ld_row_operand(Kb, T::KP, kb * 32, 16 * st, lane);
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sc[kb] = mfma32(a[st][kb], qf[st], sc[kb]);
      constexpr int NREAD = D / 16 * 2, AHEAD = 8;
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int i = 0; i < NREAD - AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }

    const bool fast = !((j0 + FWD_BN > Skv) || (CAUSAL && (j0 + FWD_BN - 1 > qw0 + diag))) && c > 0.f;
    bf16x8 pb[2][2];
    f32x16 tm[2];  // masked path: t = s*c, -inf where masked
    float mt;
    if (fast) {
      float mx = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
      mt = mx * c;
    } else {
      // Convert to t = s*c in place; masked keys become -inf.
      float mx = -MATTN_INF;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j0 + kb * 32 + crow(i, g);
          const bool ok = key < Skv && (!CAUSAL || key <= qrow + diag);
          const float t = ok ? sc[kb][i] * c : -MATTN_INF;
          tm[kb][i] = t;
          mx = fmaxf(mx, t);
        }
      mt = mx;
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    if (wave_any(mt > m + RESCALE_SLACK)) {
      const float m_new = fmaxf(m, mt);
      const float alpha = (m_new == -MATTN_INF) ? 1.f : fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
    const float m_use = (m == -MATTN_INF) ? 0.f : m;
    float rs = 0.f;
    if (fast) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(sc[kb][i], c, -m_use));
          rs += p;
          pb[kb][i >> 3][i & 7] = (bf16)p;
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(tm[kb][i] - m_use);
          rs += p;
          pb[kb][i >> 3][i & 7] = (bf16)p;
        }
    }
    l += rs;

    // O^T += V^T P^T.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 a[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          a[db] = ld_trans_operand(Vb, T::VP, kb * 32 + 16 * t, db * 32, lane);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = mfma32(a[db], pb[kb][t], acc[db]);
      }
  }

  const float lt = l + __shfl_xor(l, 32);
  if (qrow < Sq) {
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    bf16* orow = O + ((size_t)bh * Sq + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = db * 32 + r * 8 + g * 4;
        uint2 w;
        w.x = pack_bf16x2(acc[db][4 * r + 0] * inv, acc[db][4 * r + 1] * inv);
        w.y = pack_bf16x2(acc[db][4 * r + 2] * inv, acc[db][4 * r + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
    if (g == 0)
      LSE[(size_t)bh * Sq + qrow] = lt > 0.f ? (m + log2f(lt)) * MATTN_LN2 : -MATTN_INF;
  }
}

}  // namespace

template <int D, bool CAUSAL>
static hipError_t launch_fwd(const Problem& p, const void* q, const void* k, const void* v,
                             void* o, float* lse, hipStream_t stream) {
  const int n_qt = (p.Sq + FWD_BM - 1) / FWD_BM;
  const long long blocks = (long long)p.B * p.Hq * n_qt;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(FWD_THREADS), 0,
                     stream, (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, p.Hq,
                     p.Hq / p.Hkv, p.Sq, p.Skv, p.scale * MATTN_LOG2E, n_qt);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const Problem& p, const void* q, const void* k, const void* v,
                           void* o, float* lse, hipStream_t stream) {
  if (p.D == 64) return p.causal ? launch_fwd<64, true>(p, q, k, v, o, lse, stream)
                                 : launch_fwd<64, false>(p, q, k, v, o, lse, stream);
  return p.causal ? launch_fwd<128, true>(p, q, k, v, o, lse, stream)
                  : launch_fwd<128, false>(p, q, k, v, o, lse, stream);
}

}  // namespace mattn

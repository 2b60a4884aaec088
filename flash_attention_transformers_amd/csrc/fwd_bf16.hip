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
//  * K/V tiles of 64 keys are staged row-major through LDS (16-byte buffer
//    loads, prefetched into registers one tile ahead); K rows are the A
//    operand of S^T, and the A operand of O^T = V^T P^T is read transposed
//    straight from the V tile with ds_read_b64_tr_b16, in the key order that
//    P^T carries out of the S^T accumulator;
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
  static constexpr int P = TilePitch<D>::value;                  // LDS row pitch (bf16)
  static constexpr int CHUNKS = FWD_BN * D / 8 / FWD_THREADS;    // 16-byte chunks per thread per tensor
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(FWD_THREADS, 2)
void fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, bf16* __restrict__ O,
                     float* __restrict__ LSE, int Hq, int G, int Sq, int Skv,
                     float c /* scale*log2(e) */, int n_qt) {
  using T = FwdTile<D>;
  __shared__ __attribute__((aligned(16))) bf16 Ks[FWD_BN * T::P];
  __shared__ __attribute__((aligned(16))) bf16 Vs[FWD_BN * T::P];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  int bh, qt;
  tile_of_block(blockIdx.x, gridDim.x / n_qt, n_qt, CAUSAL, bh, qt);
  const int h = bh % Hq, b = bh / Hq;
  const int Hkv = Hq / G;
  const size_t kv_off = ((size_t)(b * Hkv + h / G) * Skv) * D;
  const Buf qbuf(Q + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
  const Buf kbuf(K + kv_off, (uint32_t)Skv * D * 2);
  const Buf vbuf(V + kv_off, (uint32_t)Skv * D * 2);

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

  // Register staging of one K/V tile (rows past Skv load as zeros).
  uint4 kreg[T::CHUNKS], vreg[T::CHUNKS];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int r = 0; r < T::CHUNKS; ++r) {
      const int ch = tid + FWD_THREADS * r;
      const uint32_t off = (uint32_t)((j0 + ch / (D / 8)) * D + (ch % (D / 8)) * 8) * 2;
      kreg[r] = kbuf.ld16(off);
      vreg[r] = vbuf.ld16(off);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < T::CHUNKS; ++r) {
      const int ch = tid + FWD_THREADS * r;
      const int o = (ch / (D / 8)) * T::P + (ch % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(&Ks[o]) = kreg[r];
      *reinterpret_cast<uint4*>(&Vs[o]) = vreg[r];
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = zero_f32x16();
  // Reference max of t = s*c for this query (shared by lane and lane^32) and
  // this lane's partial row sum relative to it.  The reference only moves
  // when a tile's max exceeds it by more than RESCALE_SLACK (log2 units), so
  // most tiles skip the O rescale; p <= 2^RESCALE_SLACK stays well inside
  // fp32/bf16 range and O / l is unchanged.
  constexpr float RESCALE_SLACK = 8.0f;
  float m = -MATTN_INF;
  float l = 0.f;

  if (n_kt > 0) load_tile(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int j0 = kt * FWD_BN;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(j0 + FWD_BN);

    // S^T for two 32-key blocks: lane = query column, regs = keys.
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sc[kb] = zero_f32x16();
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sc[kb] = mfma32(ld_row_operand(Ks, T::P, kb * 32, 16 * st, lane), qf[st], sc[kb]);
      }

    const bool fast = !((j0 + FWD_BN > Skv) || (CAUSAL && (j0 + FWD_BN - 1 > qw0 + diag))) && c > 0.f;
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
          sc[kb][i] = t;
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
          sc[kb][i] = p;
          rs += p;
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(sc[kb][i] - m_use);
          sc[kb][i] = p;
          rs += p;
        }
    }
    l += rs;

    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[kb][t][e] = (bf16)sc[kb][8 * t + e];

    // O^T += V^T P^T.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          acc[db] = mfma32(ld_trans_operand(Vs, T::P, kb * 32 + 16 * t, db * 32, lane),
                           pb[kb][t], acc[db]);
        }
  }

  l += __shfl_xor(l, 32);
  if (qrow < Sq) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
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
      LSE[(size_t)bh * Sq + qrow] = l > 0.f ? (m + log2f(l)) * MATTN_LN2 : -MATTN_INF;
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

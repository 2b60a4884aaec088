// Attention forward over a paged KV cache (decode and chunked prefill), bf16
// I/O with fp32 softmax statistics and accumulation.
//
// The cache holds pages of `page_size` tokens, laid out [page][Hkv][token][D];
// a sequence's keys are the first seqlens_k[b] tokens of the pages listed in
// its block-table row.  The kernel reads the pages straight through the table
// (no gathered copy) and attends only to the effective length: the LingBot
// report's FA2/FA3 comparison had to exclude the padded region recorded
// beyond cu_seqlens, and its per-call length supplement shows the allocated
// length overstating the work by about 41%.  Causal masking is aligned
// bottom-right against that length, so one decoded token is the last row of
// causal attention (xtrain evolution page, decode engine milestone M2a).
//
// Work decomposition: one workgroup (4 waves) per (sequence, KV head, chunk
// of 128 packed query rows, key split).  The G query heads that share a KV
// head are packed row-wise (row r = g*Sq + i), so a decode step with G = 4 and
// Sq = 1 fills 4 rows of one wave and reads each K/V page once for all four
// heads.  Each wave computes S^T = K Q^T for its 32 rows on MFMA (lane = row),
// keeps the running max and sum per lane, and accumulates O^T = V^T P^T, the
// same register layout as the dense forward.  K/V tiles of 64 tokens go from
// global memory straight into double-buffered LDS.
//
// Long caches are split along the keys: each split writes a normalised fp32
// partial O and its log-sum-exp, and a second kernel merges the splits in a
// fixed order (LSE = ln sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE} O_s), so
// the result is deterministic.  With one split the kernel writes O and LSE
// directly.
#include "common.hpp"
#include "kernels.hpp"

namespace mattn {

namespace {

constexpr int KC_BN = 64;        // tokens per K/V tile
constexpr int KC_THREADS = 256;  // 4 waves x 32 packed query rows

template <int D>
struct KcTile {
  static constexpr int KP = RowPitch<D>::value;
  static constexpr int VP = TrPitch<D>::value;
  using KTile = DirectTile<D, KC_BN, KP, KC_THREADS>;
  using VTile = DirectTile<D, KC_BN, VP, KC_THREADS>;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(KC_THREADS, 2)
void kvcache_fwd_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ Kc,
                        const bf16* __restrict__ Vc, const int* __restrict__ block_table,
                        const int* __restrict__ seqlens_k, bf16* __restrict__ O,
                        float* __restrict__ LSE, float* __restrict__ Opart,
                        float* __restrict__ Lpart, int B, int Hq, int Hkv, int Sq,
                        int num_pages, int page_size, int pages_per_seq, int n_qc, int nsplit,
                        int tiles_per_split, float c /* scale*log2(e) */) {
  using T = KcTile<D>;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][KC_BN * T::KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][KC_BN * T::VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  int x = blockIdx.x;
  const int split = x % nsplit;
  x /= nsplit;
  const int qc = x % n_qc;
  x /= n_qc;
  const int kvh = x % Hkv;
  const int b = x / Hkv;
  const int G = Hq / Hkv;

  // Effective length, clamped to what the table can address.
  const int cap = pages_per_seq * page_size;
  int L = seqlens_k[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);

  // This lane's packed query row.
  const int R = G * Sq;
  const int r = qc * 128 + wave * 32 + l32;
  const bool valid = r < R;
  const int gq = valid ? r / Sq : 0;
  const int qi = valid ? r - gq * Sq : 0;
  const int h = kvh * G + gq;
  // Last key this row may see (-1: none).
  int lim = valid ? L - 1 : -1;
  if (CAUSAL && valid) lim = min(lim, qi + L - Sq);
  int lim_min = lim;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lim_min = min(lim_min, __shfl_xor(lim_min, o));
  const bool wave_live = wave_any(valid && lim >= 0);

  // Q fragment (B operand of S^T = K Q^T); rows past R read as zeros.
  const Buf qbuf(Q + (size_t)b * Hq * Sq * D, (uint32_t)Hq * Sq * D * 2);
  const uint32_t qoff = valid ? (uint32_t)((h * Sq + qi) * D) * 2 : 0x80000000u;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qf[s] = as_bf16x8(qbuf.ld16(qoff + (16 * s + 8 * g) * 2));
  // Positive multiplier: a negative scale negates Q, a zero scale zeroes it
  // (both exact in bf16).
  if (!(c > 0.f)) {
    const uint32_t flip = c < 0.f ? 0x80008000u : 0u, keep = c < 0.f ? ~0u : 0u;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      uint4 u = __builtin_bit_cast(uint4, qf[s]);
      u.x = (u.x & keep) ^ flip; u.y = (u.y & keep) ^ flip;
      u.z = (u.z & keep) ^ flip; u.w = (u.w & keep) ^ flip;
      qf[s] = as_bf16x8(u);
    }
    c = c < 0.f ? -c : 1.f;
  }

  // Key tiles of this split.
  const int n_t = (L + KC_BN - 1) / KC_BN;
  const int t0 = split * tiles_per_split;
  const int t1 = min(n_t, t0 + tiles_per_split);

  typename T::KTile kt_ld;
  typename T::VTile vt_ld;
  kt_ld.init(tid);
  vt_ld.init(tid);
  // Tile t lives in page block_table[b][t*64 / page_size] at token offset
  // (t*64) % page_size.  The descriptor covers only the tile's tokens below
  // L, so tokens past the sequence (and pad slots) load as zeros; a page id
  // outside [0, num_pages) gets an empty descriptor and loads zeros too.
  auto issue = [&](int t, int buf) {
    const int tok = t * KC_BN;
    const int pid = block_table[(size_t)b * pages_per_seq + tok / page_size];
    const int rows = min(KC_BN, L - tok);
    const bool ok = pid >= 0 && pid < num_pages;
    const size_t base = (((size_t)(ok ? pid : 0) * Hkv + kvh) * page_size + tok % page_size) * D;
    const uint32_t nb = ok ? (uint32_t)rows * D * 2 : 0u;
    kt_ld.load(Buf(Kc + base, nb), Ks[buf], tid);
    vt_ld.load(Buf(Vc + base, nb), Vs[buf], tid);
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = zero_f32x16();
  constexpr float RESCALE_SLACK = 8.0f;
  float m = -MATTN_INF, l = 0.f;

  if (t0 < t1) issue(t0, 0);
  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's copies landed
    __syncthreads();                     // everyone's, and the previous tile is done
    if (t + 1 < t1) issue(t + 1, buf ^ 1);
    if (!wave_live) continue;
    const bf16* Kb = Ks[buf];
    const bf16* Vb = Vs[buf];

    f32x16 sc[2];
    sc[0] = zero_f32x16();
    sc[1] = zero_f32x16();
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sc[kb] = mfma32(ld_row_operand(Kb, T::KP, kb * 32, 16 * st, lane), qf[st], sc[kb]);

    float mx;
    if (t * KC_BN + KC_BN - 1 > lim_min) {
      // Register i of block kb holds key t*64 + kb*32 + 4g + (i/4)*8 + i%4.
      const int y = lim - t * KC_BN - 4 * g;
      mx = -MATTN_INF;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (kb * 32 + (i >> 2) * 8 + (i & 3) > y) sc[kb][i] = -MATTN_INF;
          mx = fmaxf(mx, sc[kb][i]);
        }
    } else {
      mx = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
    }
    float mt = mx * c;
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
    bf16x8 pb[2][2];
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(__builtin_fmaf(sc[kb][i], c, -m_use));
        rs[i & 3] += p;
        pb[kb][i >> 3][i & 7] = (bf16)p;
      }
    l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        bf16x8 a[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          a[db] = ld_trans_operand(Vb, T::VP, kb * 32 + 16 * tt, db * 32, lane);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = mfma32(a[db], pb[kb][tt], acc[db]);
      }
  }

  if (!valid) return;
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const float lse = lt > 0.f ? (m + log2f(lt)) * MATTN_LN2 : -MATTN_INF;
  const size_t row = ((size_t)b * Hq + h) * Sq + qi;
  if (nsplit == 1) {
    bf16* orow = O + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = db * 32 + rr * 8 + g * 4;
        uint2 w;
        w.x = pack_bf16x2(acc[db][4 * rr + 0] * inv, acc[db][4 * rr + 1] * inv);
        w.y = pack_bf16x2(acc[db][4 * rr + 2] * inv, acc[db][4 * rr + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
    if (g == 0) LSE[row] = lse;
  } else {
    // Partials: [split][row][D] fp32 (normalised) and [split][row].
    const size_t rows_all = (size_t)B * Hq * Sq;
    float* prow = Opart + ((size_t)split * rows_all + row) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = db * 32 + rr * 8 + g * 4;
        *reinterpret_cast<f32x4*>(prow + d) =
            f32x4{acc[db][4 * rr] * inv, acc[db][4 * rr + 1] * inv, acc[db][4 * rr + 2] * inv,
                  acc[db][4 * rr + 3] * inv};
      }
    if (g == 0) Lpart[(size_t)split * rows_all + row] = lse;
  }
}

// One wave per output row: merge the splits in ascending order.
constexpr int KC_MERGE_THREADS = 256;

template <int D>
__global__ __launch_bounds__(KC_MERGE_THREADS)
void kvcache_merge_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart,
                          bf16* __restrict__ O, float* __restrict__ LSE, long long rows_all,
                          int nsplit) {
  constexpr int PER = D / 64;  // elements per lane
  const long long row = (long long)blockIdx.x * (KC_MERGE_THREADS / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows_all) return;
  float mx = -MATTN_INF;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, Lpart[(size_t)s * rows_all + row]);
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  float lse = -MATTN_INF;
  if (mx != -MATTN_INF) {
    float sum = 0.f;
    for (int s = 0; s < nsplit; ++s) sum += __expf(Lpart[(size_t)s * rows_all + row] - mx);
    lse = mx + __logf(sum);
    for (int s = 0; s < nsplit; ++s) {
      const float w = __expf(Lpart[(size_t)s * rows_all + row] - lse);
      const float* p = Opart + ((size_t)s * rows_all + row) * D + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] += w * p[e];
    }
  }
  bf16* orow = O + row * D + lane * PER;
  if (PER == 2) {
    *reinterpret_cast<uint32_t*>(orow) = pack_bf16x2(o[0], o[PER - 1]);
  } else {
    orow[0] = (bf16)o[0];
  }
  if (lane == 0) LSE[row] = lse;
}

template <int D, bool CAUSAL>
hipError_t launch_kc(const KvCacheProblem& p, const void* q, const void* kc, const void* vc,
                     const int* block_table, const int* seqlens_k, void* o, float* lse,
                     float* opart, float* lpart, hipStream_t stream) {
  const int n_qc = (p.Hq / p.Hkv * p.Sq + 127) / 128;
  const int ns = kvcache_nsplit(p);
  const int max_tiles = (p.pages_per_seq * p.page_size + KC_BN - 1) / KC_BN;
  const int tps = ns > 0 ? (max_tiles + ns - 1) / ns : 0;
  const long long blocks = (long long)p.B * p.Hkv * n_qc * ns;
  hipLaunchKernelGGL((kvcache_fwd_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(KC_THREADS), 0,
                     stream, (const bf16*)q, (const bf16*)kc, (const bf16*)vc, block_table,
                     seqlens_k, (bf16*)o, lse, opart, lpart, p.B, p.Hq, p.Hkv, p.Sq, p.num_pages,
                     p.page_size, p.pages_per_seq, n_qc, ns, tps, p.scale * MATTN_LOG2E);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  const long long rows_all = (long long)p.B * p.Hq * p.Sq;
  const long long mblocks = (rows_all + KC_MERGE_THREADS / 64 - 1) / (KC_MERGE_THREADS / 64);
  hipLaunchKernelGGL((kvcache_merge_kernel<D>), dim3((unsigned)mblocks), dim3(KC_MERGE_THREADS), 0,
                     stream, (const float*)opart, (const float*)lpart, (bf16*)o, lse, rows_all, ns);
  return hipGetLastError();
}

}  // namespace

int kvcache_nsplit(const KvCacheProblem& p) {
  if (p.B <= 0 || p.Hkv <= 0 || p.Sq <= 0) return 1;
  const long long max_tiles = ((long long)p.pages_per_seq * p.page_size + KC_BN - 1) / KC_BN;
  if (max_tiles <= 1) return 1;
  const long long n_qc = ((long long)(p.Hq / p.Hkv) * p.Sq + 127) / 128;
  const long long wgs = (long long)p.B * p.Hkv * n_qc;
  const long long target = 512;  // two workgroups per CU
  long long ns = (target + wgs - 1) / wgs;
  const long long cap = (max_tiles + 3) / 4;  // keep at least four tiles per split
  if (ns > cap) ns = cap;
  if (ns > 64) ns = 64;
  return ns < 1 ? 1 : (int)ns;
}

size_t kvcache_workspace_bytes(const KvCacheProblem& p) {
  const int ns = kvcache_nsplit(p);
  if (ns <= 1) return 0;
  const size_t rows = (size_t)p.B * p.Hq * p.Sq;
  const size_t o_bytes = ((size_t)ns * rows * p.D * 4 + 255) / 256 * 256;
  return o_bytes + ((size_t)ns * rows * 4 + 255) / 256 * 256;
}

hipError_t launch_kvcache_bf16(const KvCacheProblem& p, const void* q, const void* kc,
                               const void* vc, const int* block_table, const int* seqlens_k,
                               void* o, float* lse, void* workspace, hipStream_t stream) {
  float* opart = nullptr;
  float* lpart = nullptr;
  if (kvcache_nsplit(p) > 1) {
    const size_t rows = (size_t)p.B * p.Hq * p.Sq;
    const size_t o_bytes = ((size_t)kvcache_nsplit(p) * rows * p.D * 4 + 255) / 256 * 256;
    opart = static_cast<float*>(workspace);
    lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  }
  if (p.D == 64)
    return p.causal ? launch_kc<64, true>(p, q, kc, vc, block_table, seqlens_k, o, lse, opart, lpart, stream)
                    : launch_kc<64, false>(p, q, kc, vc, block_table, seqlens_k, o, lse, opart, lpart, stream);
  return p.causal ? launch_kc<128, true>(p, q, kc, vc, block_table, seqlens_k, o, lse, opart, lpart, stream)
                  : launch_kc<128, false>(p, q, kc, vc, block_table, seqlens_k, o, lse, opart, lpart, stream);
}

}  // namespace mattn

// Fused attention forward and backward with float32 operands throughout.
//
// Same method as the bf16 kernels (xtrain evolution page, infrastructure-
// phase table, rows T14 and T15: online softmax over K/V tiles, recompute-
// based backward with D = sum(dO * O), group-summed dK/dV without atomics),
// but no operand is ever rounded below fp32.  These are plain vector-ALU
// kernels, one wave per query row (forward, dQ) or per key row (dK/dV); the
// float32 path serves small problems where launch latency dominates.
//
// Lane roles: a wave walks tiles of 64 keys (or 64 queries); lane j computes
// the full dot product of its own key (query) against the wave's row, the
// softmax statistics are wave reductions, and each lane owns the output
// columns d = lane + 64*x.
#include "common.hpp"
#include "kernels.hpp"

namespace mattn {
namespace {

constexpr int F_THREADS = 256;
constexpr int F_ROWS = 4;   // rows per workgroup (one per wave)
constexpr int F_TILE = 64;  // keys (or queries) per LDS tile

template <int D>
__device__ __forceinline__ void load_rows_f32(float (*dst)[D + 1], const float* src, int row0,
                                              int nvalid, int tid) {
  for (int e = tid; e < F_TILE * D; e += F_THREADS) {
    const int r = e / D, d = e % D;
    dst[r][d] = (row0 + r < nvalid) ? src[(size_t)(row0 + r) * D + d] : 0.f;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(F_THREADS)
void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                    const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                    int Hq, int G, int Sq, int Skv, float c, int n_rt) {
  __shared__ float Ks[F_TILE][D + 1];
  __shared__ float Vs[F_TILE][D + 1];
  __shared__ float qs[F_ROWS][D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x / n_rt;
  const int r0 = (blockIdx.x % n_rt) * F_ROWS;
  const int row = r0 + wave;
  const int h = bh % Hq, b = bh / Hq, Hkv = Hq / G;
  const size_t kv_off = ((size_t)(b * Hkv + h / G) * Skv) * D;
  const int diag = Skv - Sq;
  for (int d = lane; d < D; d += 64)
    qs[wave][d] = row < Sq ? Q[((size_t)bh * Sq + row) * D + d] : 0.f;
  int kv_end = Skv;
  if (CAUSAL) kv_end = min(Skv, r0 + F_ROWS + diag);

  float o[D / 64];
#pragma unroll
  for (int x = 0; x < D / 64; ++x) o[x] = 0.f;
  float m = -MATTN_INF, l = 0.f;
  for (int j0 = 0; j0 < kv_end; j0 += F_TILE) {
    __syncthreads();
    load_rows_f32<D>(Ks, K + kv_off, j0, Skv, tid);
    load_rows_f32<D>(Vs, V + kv_off, j0, Skv, tid);
    __syncthreads();
    const int key = j0 + lane;
    float s = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) s += qs[wave][d] * Ks[lane][d];
    const bool ok = key < Skv && (!CAUSAL || key <= row + diag);
    const float t = ok ? s * c : -MATTN_INF;
    const float m_new = fmaxf(m, wave_max(t));
    const float m_use = m_new == -MATTN_INF ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    const float p = fast_exp2(t - m_use);
    l = l * alpha + wave_sum(p);
    m = m_new;
#pragma unroll
    for (int x = 0; x < D / 64; ++x) o[x] *= alpha;
    for (int j = 0; j < F_TILE; ++j) {
      const float pj = __shfl(p, j);
#pragma unroll
      for (int x = 0; x < D / 64; ++x) o[x] += pj * Vs[j][lane + 64 * x];
    }
  }
  if (row < Sq) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int x = 0; x < D / 64; ++x) O[((size_t)bh * Sq + row) * D + lane + 64 * x] = o[x] * inv;
    if (lane == 0) LSE[(size_t)bh * Sq + row] = l > 0.f ? (m + log2f(l)) * MATTN_LN2 : -MATTN_INF;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(F_THREADS)
void dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                   const float* __restrict__ V, const float* __restrict__ dO,
                   const float* __restrict__ LSE, const float* __restrict__ DLT,
                   float* __restrict__ dQ, int Hq, int G, int Sq, int Skv, float scale, float c,
                   int n_rt) {
  __shared__ float Ks[F_TILE][D + 1];
  __shared__ float Vs[F_TILE][D + 1];
  __shared__ float qs[F_ROWS][D];
  __shared__ float ds_[F_ROWS][D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x / n_rt;
  const int r0 = (blockIdx.x % n_rt) * F_ROWS;
  const int row = r0 + wave;
  const int h = bh % Hq, b = bh / Hq, Hkv = Hq / G;
  const size_t kv_off = ((size_t)(b * Hkv + h / G) * Skv) * D;
  const int diag = Skv - Sq;
  const size_t ro = (size_t)bh * Sq + row;
  for (int d = lane; d < D; d += 64) {
    qs[wave][d] = row < Sq ? Q[ro * D + d] : 0.f;
    ds_[wave][d] = row < Sq ? dO[ro * D + d] : 0.f;
  }
  const float lse2 = row < Sq ? LSE[ro] * MATTN_LOG2E : MATTN_INF;
  const float dl = row < Sq ? DLT[ro] : 0.f;
  int kv_end = Skv;
  if (CAUSAL) kv_end = min(Skv, r0 + F_ROWS + diag);
  float acc[D / 64];
#pragma unroll
  for (int x = 0; x < D / 64; ++x) acc[x] = 0.f;
  for (int j0 = 0; j0 < kv_end; j0 += F_TILE) {
    __syncthreads();
    load_rows_f32<D>(Ks, K + kv_off, j0, Skv, tid);
    load_rows_f32<D>(Vs, V + kv_off, j0, Skv, tid);
    __syncthreads();
    const int key = j0 + lane;
    float s = 0.f, dp = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) {
      s += qs[wave][d] * Ks[lane][d];
      dp += ds_[wave][d] * Vs[lane][d];
    }
    const bool ok = row < Sq && key < Skv && (!CAUSAL || key <= row + diag);
    const float p = ok ? fast_exp2(s * c - lse2) : 0.f;
    const float dsv = p * (dp - dl);
    for (int j = 0; j < F_TILE; ++j) {
      const float dj = __shfl(dsv, j);
#pragma unroll
      for (int x = 0; x < D / 64; ++x) acc[x] += dj * Ks[j][lane + 64 * x];
    }
  }
  if (row < Sq) {
#pragma unroll
    for (int x = 0; x < D / 64; ++x) dQ[ro * D + lane + 64 * x] = acc[x] * scale;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(F_THREADS)
void dkdv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                     const float* __restrict__ V, const float* __restrict__ dO,
                     const float* __restrict__ LSE, const float* __restrict__ DLT,
                     float* __restrict__ dK, float* __restrict__ dV, int Hq, int G, int Sq,
                     int Skv, float scale, float c, int n_kt) {
  __shared__ float Qs[F_TILE][D + 1];
  __shared__ float dOs[F_TILE][D + 1];
  __shared__ float ks[F_ROWS][D];
  __shared__ float vs[F_ROWS][D];
  __shared__ float lse_s[F_TILE], dlt_s[F_TILE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bkv = blockIdx.x / n_kt;
  const int k0 = (blockIdx.x % n_kt) * F_ROWS;
  const int key = k0 + wave;
  const int Hkv = Hq / G, b = bkv / Hkv, kvh = bkv % Hkv;
  const size_t ko = (size_t)bkv * Skv + key;
  const int diag = Skv - Sq;
  for (int d = lane; d < D; d += 64) {
    ks[wave][d] = key < Skv ? K[ko * D + d] : 0.f;
    vs[wave][d] = key < Skv ? V[ko * D + d] : 0.f;
  }
  int q_lo = 0;
  if (CAUSAL && k0 - diag > 0) q_lo = k0 - diag;
  float ak[D / 64], av[D / 64];
#pragma unroll
  for (int x = 0; x < D / 64; ++x) ak[x] = av[x] = 0.f;
  for (int r = 0; r < G; ++r) {  // ascending group member
    const int h = kvh * G + r;
    const size_t qbase = (size_t)(b * Hq + h) * Sq;
    for (int i0 = q_lo; i0 < Sq; i0 += F_TILE) {
      __syncthreads();
      load_rows_f32<D>(Qs, Q + qbase * D, i0, Sq, tid);
      load_rows_f32<D>(dOs, dO + qbase * D, i0, Sq, tid);
      if (tid < F_TILE) {
        const int qq = i0 + tid;
        lse_s[tid] = qq < Sq ? LSE[qbase + qq] * MATTN_LOG2E : MATTN_INF;
        dlt_s[tid] = qq < Sq ? DLT[qbase + qq] : 0.f;
      }
      __syncthreads();
      const int qi = i0 + lane;
      float s = 0.f, dp = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) {
        s += Qs[lane][d] * ks[wave][d];
        dp += dOs[lane][d] * vs[wave][d];
      }
      const bool ok = qi < Sq && key < Skv && (!CAUSAL || key <= qi + diag);
      const float p = ok ? fast_exp2(s * c - lse_s[lane]) : 0.f;
      const float dsv = p * (dp - dlt_s[lane]);
      for (int i = 0; i < F_TILE; ++i) {
        const float pi = __shfl(p, i), di = __shfl(dsv, i);
#pragma unroll
        for (int x = 0; x < D / 64; ++x) {
          av[x] += pi * dOs[i][lane + 64 * x];
          ak[x] += di * Qs[i][lane + 64 * x];
        }
      }
    }
  }
  if (key < Skv) {
#pragma unroll
    for (int x = 0; x < D / 64; ++x) {
      dK[ko * D + lane + 64 * x] = ak[x] * scale;
      dV[ko * D + lane + 64 * x] = av[x];
    }
  }
}

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <int D, bool CAUSAL>
hipError_t fwd_f32_t(const Problem& p, const float* q, const float* k, const float* v, float* o,
                     float* lse, hipStream_t stream) {
  const int n_rt = (p.Sq + F_ROWS - 1) / F_ROWS;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)((long long)p.B * p.Hq * n_rt)),
                     dim3(F_THREADS), 0, stream, q, k, v, o, lse, p.Hq, p.Hq / p.Hkv, p.Sq, p.Skv,
                     p.scale * MATTN_LOG2E, n_rt);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dkdv_f32_t(const Problem& p, const float* q, const float* k, const float* v,
                      const float* lse, const float* dlt, const float* dout, float* dk, float* dv,
                      hipStream_t stream) {
  const int n_kt = (p.Skv + F_ROWS - 1) / F_ROWS;
  hipLaunchKernelGGL((dkdv_f32_kernel<D, CAUSAL>), dim3((unsigned)((long long)p.B * p.Hkv * n_kt)),
                     dim3(F_THREADS), 0, stream, q, k, v, dout, lse, dlt, dk, dv, p.Hq,
                     p.Hq / p.Hkv, p.Sq, p.Skv, p.scale, p.scale * MATTN_LOG2E, n_kt);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dq_f32_t(const Problem& p, const float* q, const float* k, const float* v,
                    const float* lse, const float* dlt, const float* dout, float* dq,
                    hipStream_t stream) {
  const int n_rt = (p.Sq + F_ROWS - 1) / F_ROWS;
  hipLaunchKernelGGL((dq_f32_kernel<D, CAUSAL>), dim3((unsigned)((long long)p.B * p.Hq * n_rt)),
                     dim3(F_THREADS), 0, stream, q, k, v, dout, lse, dlt, dq, p.Hq, p.Hq / p.Hkv,
                     p.Sq, p.Skv, p.scale, p.scale * MATTN_LOG2E, n_rt);
  return hipGetLastError();
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

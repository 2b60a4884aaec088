// C-ABI entry points of libmattn: argument validation and kernel dispatch.
// Every check happens before anything is enqueued; on error nothing runs and
// no output is touched.
#include <math.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "mattn.h"
#include "kernels.hpp"

namespace {

constexpr long long kMaxElems = 1LL << 31;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Sizes {
  long long q_elems, kv_elems, rows;
};

// Size, flag and scale validation shared by forward and backward.
mattn_status check_args(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                        mattn_dtype dtype, Sizes* out) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Sq < 0 || Skv < 0 || D < 0) return MATTN_ERR_INVALID_ARG;
  if (Hkv == 0 || Hq % Hkv != 0) return MATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return MATTN_ERR_INVALID_ARG;
  if (!isfinite(scale)) return MATTN_ERR_INVALID_ARG;
  if (dtype != MATTN_BF16 && dtype != MATTN_F32) return MATTN_ERR_INVALID_ARG;
  const long long rows = (long long)B * Hq * Sq;
  const long long kv_rows = (long long)B * Hkv * Skv;
  if (rows > 0 && Skv == 0) return MATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return MATTN_ERR_UNSUPPORTED;
  if (rows * D >= kMaxElems || kv_rows * D >= kMaxElems) return MATTN_ERR_UNSUPPORTED;
  if (causal && Sq > Skv) return MATTN_ERR_UNSUPPORTED;
  out->q_elems = rows * D;
  out->kv_elems = kv_rows * D;
  out->rows = rows;
  return MATTN_OK;
}

// Every pointer in the list must be non-null and 16-byte aligned.
bool ptrs_ok(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return false;
  return true;
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t dlt_bytes(int B, int Hq, int Sq) { return round256((size_t)B * Hq * Sq * sizeof(float)); }

size_t part_bytes(int B, int Hkv, int Sq, int Skv, int D) {
  const int ns = mattn::bwd_nsplit(B, Hkv, Sq, Skv);
  if (ns <= 1) return 0;
  const size_t n_kt = (size_t)(Skv + mattn::BWD_BN - 1) / mattn::BWD_BN;
  return round256(2 * (size_t)ns * B * Hkv * n_kt * mattn::BWD_BN * D * sizeof(float));
}

// Backward workspace for mattn_bwd_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not a device address; its address on a device comes
// from hipGetSymbolAddress, looked up once per device with that device
// current, and only that address is ever passed to a kernel.
constexpr size_t kScratchBytes = (size_t)MATTN_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// The device the stream's work runs on (the current device for the null stream).
hipError_t stream_device(hipStream_t stream, int* dev) {
  return stream ? hipStreamGetDevice(stream, dev) : hipGetDevice(dev);
}

// Device address of `scratch` on device `dev`.
hipError_t scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

mattn_status mattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                       mattn_dtype dtype, hipStream_t stream) {
  Sizes sz;
  mattn_status st = check_args(B, Hq, Hkv, Sq, Skv, D, causal, scale, dtype, &sz);
  if (st != MATTN_OK) return st;
  if (sz.rows == 0) return MATTN_OK;
  if (!ptrs_ok({q, k, v, o, lse})) return MATTN_ERR_INVALID_ARG;
  const mattn::Problem p{B, Hq, Hkv, Sq, Skv, D, causal, scale};
  hipError_t e = dtype == MATTN_BF16
                     ? mattn::launch_fwd_bf16(p, q, k, v, o, lse, stream)
                     : mattn::launch_fwd_f32(p, (const float*)q, (const float*)k,
                                             (const float*)v, (float*)o, lse, stream);
  return e == hipSuccess ? MATTN_OK : MATTN_ERR_LAUNCH;
}

size_t mattn_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Skv, int D) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0 || Hq % Hkv != 0) return 0;
  if (D != 64 && D != 128) return 0;
  return dlt_bytes(B, Hq, Sq) + part_bytes(B, Hkv, Sq, Skv, D);
}

mattn_status mattn_bwd_stages(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                              float scale, mattn_dtype dtype, void* workspace,
                              size_t workspace_bytes, unsigned stages, hipStream_t stream) {
  const unsigned all = MATTN_BWD_PREPROCESS | MATTN_BWD_DKDV | MATTN_BWD_DQ;
  if (stages == 0 || (stages & ~all) != 0) return MATTN_ERR_INVALID_ARG;
  Sizes sz;
  mattn_status st = check_args(B, Hq, Hkv, Sq, Skv, D, causal, scale, dtype, &sz);
  if (st != MATTN_OK) return st;
  if (sz.kv_elems > 0 && !ptrs_ok({dk, dv})) return MATTN_ERR_INVALID_ARG;
  if (sz.rows > 0) {
    if (!ptrs_ok({q, k, v, o, lse, dout, dq, workspace})) return MATTN_ERR_INVALID_ARG;
    if (workspace_bytes < mattn_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D))
      return MATTN_ERR_INVALID_ARG;
  }
  if (sz.rows == 0) {
    // No query rows: every key receives a zero gradient.
    if (!(stages & MATTN_BWD_DKDV)) return MATTN_OK;
    const size_t words = (size_t)sz.kv_elems * (dtype == MATTN_BF16 ? 2 : 4) / 4;
    if (mattn::launch_zero_words(dk, words, stream) != hipSuccess) return MATTN_ERR_LAUNCH;
    if (mattn::launch_zero_words(dv, words, stream) != hipSuccess) return MATTN_ERR_LAUNCH;
    return MATTN_OK;
  }
  const mattn::Problem p{B, Hq, Hkv, Sq, Skv, D, causal, scale};
  float* dlt = (float*)workspace;
  float* part = (float*)((char*)workspace + dlt_bytes(B, Hq, Sq));
  const bool bf = dtype == MATTN_BF16;
  // Selected stages run in the order preprocess, dQ, dK/dV.  The bf16 dQ
  // kernel forms the per-row D itself and stores it, bitwise equal to the
  // preprocess result; the fp32 dQ and both dK/dV kernels read it.
  if (stages & MATTN_BWD_PREPROCESS) {
    if (mattn::launch_bwd_preprocess(p, bf, o, dout, dlt, stream) != hipSuccess)
      return MATTN_ERR_LAUNCH;
  }
  if (stages & MATTN_BWD_DQ) {
    const hipError_t e =
        bf ? mattn::launch_dq_bf16(p, q, k, v, o, lse, dlt, dout, dq, stream)
           : mattn::launch_dq_f32(p, (const float*)q, (const float*)k, (const float*)v, lse, dlt,
                                  (const float*)dout, (float*)dq, stream);
    if (e != hipSuccess) return MATTN_ERR_LAUNCH;
  }
  if (stages & MATTN_BWD_DKDV) {
    const hipError_t e =
        bf ? mattn::launch_dkdv_bf16(p, q, k, v, lse, dlt, dout, dk, dv, part, stream)
           : mattn::launch_dkdv_f32(p, (const float*)q, (const float*)k, (const float*)v, lse,
                                    dlt, (const float*)dout, (float*)dk, (float*)dv, stream);
    if (e != hipSuccess) return MATTN_ERR_LAUNCH;
  }
  return MATTN_OK;
}

mattn_status mattn_bwd(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                       int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                       mattn_dtype dtype, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  // bf16: the dQ kernel forms D itself, so no separate preprocess pass.
  const unsigned stages = dtype == MATTN_BF16 ? (MATTN_BWD_DQ | MATTN_BWD_DKDV)
                                              : (MATTN_BWD_PREPROCESS | MATTN_BWD_DQ | MATTN_BWD_DKDV);
  return mattn_bwd_stages(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, causal,
                          scale, dtype, workspace, workspace_bytes, stages, stream);
}

mattn_status mattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                               float scale, mattn_dtype dtype, hipStream_t stream) {
  Sizes sz;
  mattn_status st = check_args(B, Hq, Hkv, Sq, Skv, D, causal, scale, dtype, &sz);
  if (st != MATTN_OK) return st;
  if (sz.kv_elems > 0 && !ptrs_ok({dk, dv})) return MATTN_ERR_INVALID_ARG;
  void* ws = nullptr;
  if (sz.rows > 0) {
    if (!ptrs_ok({q, k, v, o, lse, dout, dq})) return MATTN_ERR_INVALID_ARG;
    if (mattn_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D) > kScratchBytes) return MATTN_ERR_SCRATCH;
    int dev = 0;
    if (stream_device(stream, &dev) != hipSuccess || scratch_on(dev, &ws) != hipSuccess)
      return MATTN_ERR_LAUNCH;
  }
  // The workspace contents on entry do not matter to the backward (every
  // value it reads there was written earlier in the same call), so the
  // scratch needs no clearing between calls.
  return mattn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, causal, scale,
                   dtype, ws, kScratchBytes, stream);
}

size_t mattn_fwd_kvcache_workspace_size(int B, int Hq, int Hkv, int Sq, int D, int page_size,
                                        int pages_per_seq) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || page_size <= 0 || pages_per_seq <= 0 ||
      Hq % Hkv != 0)
    return 0;
  mattn::KvCacheProblem p{B, Hq, Hkv, Sq, D, 0, 1.f, 1, page_size, pages_per_seq};
  return mattn::kvcache_workspace_bytes(p);
}

mattn_status mattn_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                               const int* block_table, const int* seqlens_k, void* o, float* lse,
                               int B, int Hq, int Hkv, int Sq, int D, int num_pages,
                               int page_size, int pages_per_seq, int causal, float scale,
                               mattn_dtype dtype, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Sq < 0 || D < 0 || num_pages < 0 || page_size <= 0 ||
      pages_per_seq < 0)
    return MATTN_ERR_INVALID_ARG;
  if (Hkv == 0 || Hq % Hkv != 0) return MATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return MATTN_ERR_INVALID_ARG;
  if (!isfinite(scale)) return MATTN_ERR_INVALID_ARG;
  if (dtype != MATTN_BF16 && dtype != MATTN_F32) return MATTN_ERR_INVALID_ARG;
  if (dtype != MATTN_BF16) return MATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return MATTN_ERR_UNSUPPORTED;
  if (page_size % 64 != 0) return MATTN_ERR_UNSUPPORTED;
  const long long rows = (long long)B * Hq * Sq;
  if (rows * D >= kMaxElems) return MATTN_ERR_UNSUPPORTED;
  if ((long long)pages_per_seq * page_size >= kMaxElems) return MATTN_ERR_UNSUPPORTED;
  if (rows == 0) return MATTN_OK;
  if (!ptrs_ok({q, o, lse})) return MATTN_ERR_INVALID_ARG;
  if (k_cache == nullptr || v_cache == nullptr || block_table == nullptr || seqlens_k == nullptr ||
      !aligned16(k_cache) || !aligned16(v_cache) || ((uintptr_t)block_table & 3u) ||
      ((uintptr_t)seqlens_k & 3u))
    return MATTN_ERR_INVALID_ARG;
  mattn::KvCacheProblem p{B, Hq, Hkv, Sq, D, causal, scale, num_pages, page_size, pages_per_seq};
  const size_t need = mattn::kvcache_workspace_bytes(p);
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need))
    return MATTN_ERR_INVALID_ARG;
  if (mattn::launch_kvcache_bf16(p, q, k_cache, v_cache, block_table, seqlens_k, o, lse,
                                 workspace, stream) != hipSuccess)
    return MATTN_ERR_LAUNCH;
  return MATTN_OK;
}

const char* mattn_strerror(mattn_status s) {
  switch (s) {
    case MATTN_OK: return "success";
    case MATTN_ERR_INVALID_ARG: return "invalid argument";
    case MATTN_ERR_UNSUPPORTED: return "unsupported problem (head dim, size or causal Sq > Skv)";
    case MATTN_ERR_LAUNCH: return "HIP kernel launch failed";
    case MATTN_ERR_SCRATCH:
      return "problem needs more backward workspace than the static scratch buffer holds "
             "(MATTN_SCRATCH_BYTES); call mattn_bwd with a workspace";
  }
  return "unknown status";
}

int mattn_version(void) { return 100; }

}  // extern "C"

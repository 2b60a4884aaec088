// Internal launcher interface between the C-ABI layer (api.hip) and the
// kernel translation units.  Arguments are validated before these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace mattn {

struct Problem {
  int B, Hq, Hkv, Sq, Skv, D, causal;
  float scale;
};

// Backward split of the query range for shapes with few KV tiles (see
// bwd_bf16.hip).  Depends only on the sizes.
int bwd_nsplit(int B, int Hkv, int Sq, int Skv);
constexpr int BWD_BN = 128;  // keys per dK/dV workgroup
constexpr int BWD_BMQ = 64;  // query rows per dK/dV inner step

hipError_t launch_fwd_bf16(const Problem& p, const void* q, const void* k, const void* v,
                           void* o, float* lse, hipStream_t stream);

// D = rowsum(dO * O) into dlt [B*Hq*Sq] fp32.
hipError_t launch_bwd_preprocess(const Problem& p, bool bf16_io, const void* o,
                                 const void* dout, float* dlt, hipStream_t stream);

// dK/dV (+ split reduction) for bf16; `part` is fp32 scratch of
// 2 * nsplit * B*Hkv*ceil(Skv/BWD_BN)*BWD_BN*D floats when nsplit > 1.
hipError_t launch_dkdv_bf16(const Problem& p, const void* q, const void* k, const void* v,
                            const float* lse, const float* dlt, const void* dout, void* dk,
                            void* dv, float* part, hipStream_t stream);
// dQ for bf16; also forms D = rowsum(dO * O) itself (bitwise the preprocess
// kernel's value) and stores it into dlt for the dK/dV kernel.
hipError_t launch_dq_bf16(const Problem& p, const void* q, const void* k, const void* v,
                          const void* o, const float* lse, float* dlt, const void* dout, void* dq,
                          hipStream_t stream);

hipError_t launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v,
                          float* o, float* lse, hipStream_t stream);
hipError_t launch_dkdv_f32(const Problem& p, const float* q, const float* k, const float* v,
                           const float* lse, const float* dlt, const float* dout, float* dk,
                           float* dv, hipStream_t stream);
hipError_t launch_dq_f32(const Problem& p, const float* q, const float* k, const float* v,
                         const float* lse, const float* dlt, const float* dout, float* dq,
                         hipStream_t stream);

// Forward over a paged KV cache (kvcache_bf16.hip).
struct KvCacheProblem {
  int B, Hq, Hkv, Sq, D, causal;
  float scale;
  int num_pages, page_size, pages_per_seq;
};
// Number of key splits; depends only on the sizes.
int kvcache_nsplit(const KvCacheProblem& p);
// Workspace for the split partials (0 when there is one split).
size_t kvcache_workspace_bytes(const KvCacheProblem& p);
hipError_t launch_kvcache_bf16(const KvCacheProblem& p, const void* q, const void* kc,
                               const void* vc, const int* block_table, const int* seqlens_k,
                               void* o, float* lse, void* workspace, hipStream_t stream);

// Zero-fill of n 4-byte words (used for dk/dv when there are no query rows).
hipError_t launch_zero_words(void* p, size_t n_words, hipStream_t stream);

}  // namespace mattn

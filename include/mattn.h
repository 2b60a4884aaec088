/*
 * libmattn — fused scaled-dot-product attention with online softmax for
 * AMD Instinct MI355X (gfx950), forward and flash-style backward.
 *
 * The operation is the one the xtrain evolution page describes in its
 * infrastructure-phase table, row T14: a single fused forward kernel with an
 * online softmax that walks K/V in tiles and never materialises the
 * Sq x Skv score matrix, and a backward that recomputes the scores and uses
 * the per-row scalar D = sum(dO * O) to simplify the softmax Jacobian before
 * forming dQ, dK and dV.  Grouped KV heads follow row T15 of that table:
 * query head h reads KV head floor(h / G), G = Hq / Hkv, and each KV head's
 * gradient is the deterministic sum over its G query heads (no atomics).
 *
 * Math, for every batch b, query head h, kv = h / G, query row i, key j:
 *   S_ij = scale * sum_d q[b,h,i,d] * k[b,kv,j,d]     (-inf where masked)
 *   P_ij = softmax_j(S_ij);   o[b,h,i,:] = sum_j P_ij v[b,kv,j,:]
 *   lse[b,h,i] = ln sum_j exp(S_ij)                  (natural log)
 * Causal masking is aligned bottom-right: key j is visible to query i iff
 * j <= i + (Skv - Sq).
 *
 * Layout: every tensor is dense, row-major, contiguous BHSD:
 *   q, o, dout, dq : [B, Hq,  Sq,  D]
 *   k, v, dk, dv   : [B, Hkv, Skv, D]
 *   lse            : [B, Hq,  Sq]     float32
 * Element type: MATTN_BF16 (bfloat16 I/O, float32 softmax statistics and
 * accumulation, outputs rounded to nearest even) or MATTN_F32 (float32
 * throughout; no operand is rounded below float32).
 *
 * Ownership: every pointer is a device pointer owned by the caller.  The
 * library allocates nothing, never synchronises the device and is safe to
 * call from several host threads.  Its only global state is the static
 * scratch array of mattn_bwd_noalloc (below) and that array's per-device
 * address, looked up once.  Work is enqueued on
 * `stream` (0 = the null stream) and runs asynchronously; buffers must stay
 * alive until the stream reaches that point.  Outputs must not alias inputs
 * and are fully overwritten (never accumulated into).
 *
 * Errors: all argument checks are synchronous and happen before anything is
 * enqueued; on any error nothing is launched and no output is written.
 *   MATTN_ERR_INVALID_ARG  a null or misaligned pointer that the call needs (all
 *                          of them when B*Hq*Sq > 0; with no query rows the
 *                          backward needs only dk and dv), a size < 0,
 *                          Hkv == 0 or Hq % Hkv != 0, Skv == 0 with Sq > 0,
 *                          causal not 0/1, a non-finite scale (pointers must be
 *                          16-byte aligned), an unknown dtype, or (backward) a
 *                          workspace smaller than mattn_bwd_workspace_size().
 *   MATTN_ERR_UNSUPPORTED  D not 64 or 128, a tensor with 2^31 or more
 *                          elements, or causal with Sq > Skv (which would
 *                          leave query rows with no visible key).
 *   MATTN_ERR_LAUNCH       the HIP runtime reported an error after a launch.
 *   MATTN_ERR_SCRATCH      (mattn_bwd_noalloc only) the problem needs more
 *                          workspace than the library's static scratch holds.
 * B*Hq*Sq == 0 with otherwise valid sizes returns MATTN_OK: the forward does
 * nothing and the backward writes zeros to dk and dv.
 */
#ifndef MATTN_H
#define MATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MATTN_OK = 0,
  MATTN_ERR_INVALID_ARG = 1,
  MATTN_ERR_UNSUPPORTED = 2,
  MATTN_ERR_LAUNCH = 3,
  MATTN_ERR_SCRATCH = 4
} mattn_status;

typedef enum { MATTN_BF16 = 0, MATTN_F32 = 1 } mattn_dtype;

/* Forward: o = softmax(scale * q k^T, masked) v and its log-sum-exp.
 * q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D] in `dtype`; writes o [B,Hq,Sq,D] in
 * `dtype` and lse [B,Hq,Sq] float32.  One kernel launch. */
mattn_status mattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                       float scale, mattn_dtype dtype, hipStream_t stream);

/* Bytes of device workspace mattn_bwd needs for these sizes: the per-row
 * D = sum(dO * O) statistic (B*Hq*Sq float32) plus, for shapes with few KV
 * tiles, float32 partial dK/dV over fixed chunks of the query range.  Rounded
 * up to 256 bytes; depends only on the arguments.  Returns 0 for invalid or
 * empty sizes. */
size_t mattn_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Skv, int D);

/* Backward of mattn_fwd for the loss gradient dout = dL/do.
 * Inputs: q, k, v, the forward's o and lse, dout.  Writes dq [B,Hq,Sq,D] and
 * dk, dv [B,Hkv,Skv,D] in `dtype` (overwritten).  `workspace` is caller-owned
 * device memory of at least mattn_bwd_workspace_size() bytes; its contents on
 * entry do not matter.  Enqueues, on `stream` and with no host
 * synchronisation, for bf16: the dQ kernel, which also forms the per-row
 * statistic D = sum(dO * O) and stores it in the workspace, then the dK/dV
 * kernel (plus a fixed-order reduction of partials when the query range is
 * split), which reads D; for fp32: the D preprocess, then the dQ kernel,
 * then the dK/dV kernel.  Results are bitwise reproducible run to run. */
mattn_status mattn_bwd(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                       float scale, mattn_dtype dtype, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* mattn_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, allocation-free serving
 * loops, harnesses that forbid hipMalloc.  Same arguments (minus the
 * workspace), checks, kernels and results as mattn_bwd (the same bits).  The
 * workspace is a static device array of MATTN_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; its device address is
 * looked up once per device on the first call there.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 * A problem whose mattn_bwd_workspace_size() exceeds MATTN_SCRATCH_BYTES
 * returns MATTN_ERR_SCRATCH before anything is enqueued.  Every call on one
 * GPU shares that GPU's array: calls whose work may overlap on one GPU
 * (different streams, or different host threads without ordering) race and
 * give wrong results; calls on one stream are ordered and safe.  The stream
 * must belong to the device whose array is used (the stream's device). */
#define MATTN_SCRATCH_BYTES (128u << 20)
mattn_status mattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                               float scale, mattn_dtype dtype, hipStream_t stream);

/* The stages mattn_bwd enqueues, selectable for callers that schedule or
 * time them separately.  Same arguments, checks and workspace as mattn_bwd;
 * `stages` is a non-zero OR of the flags below, and the selected stages run
 * in the order listed.  Each reads what an earlier one wrote into
 * `workspace` or the outputs, so separate calls follow the same order.
 *   MATTN_BWD_PREPROCESS  D = sum(dO * O) per query row into the workspace
 *   MATTN_BWD_DQ          dQ; for bf16 it also forms D itself and stores it
 *                         (bitwise the preprocess value), so a bf16 caller
 *                         may skip the preprocess; fp32 reads the stored D
 *   MATTN_BWD_DKDV        dK, dV (reads the stored D)
 * mattn_bwd enqueues DQ then DKDV for bf16, and all three for fp32; a caller
 * that enqueues all three for bf16 gets the same bits. */
enum { MATTN_BWD_PREPROCESS = 1, MATTN_BWD_DKDV = 2, MATTN_BWD_DQ = 4 };
mattn_status mattn_bwd_stages(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                              float scale, mattn_dtype dtype, void* workspace,
                              size_t workspace_bytes, unsigned stages, hipStream_t stream);

/* Forward attention over a paged KV cache: decode (Sq = 1..16 new tokens per
 * sequence) and chunked prefill against cached keys.
 *
 * Defining passages: the LingBot report (same-card FA2/FA3 counter section
 * and the per-call effective-length supplement) on attending to the
 * effective K/V length recorded in cu_seqlens rather than the allocated
 * buffer, and the xtrain evolution page (decode engine, milestone M2a) on one
 * decoded token being the last row of causal attention.
 *
 * Layout (all row-major):
 *   q, o         [B, Hq, Sq, D]                     bf16
 *   lse          [B, Hq, Sq]                        float32, natural log
 *   k_cache,
 *   v_cache      [num_pages, Hkv, page_size, D]     bf16
 *   block_table  [B, pages_per_seq]                 int32, page ids in token order
 *   seqlens_k    [B]                                int32, effective key count
 * Sequence b attends to the first seqlens_k[b] tokens of its pages (values are
 * clamped to [0, pages_per_seq*page_size]); with causal = 1, query i sees key
 * j iff j <= i + seqlens_k[b] - Sq (bottom-right).  Rows that see no key get
 * o = 0 and lse = -inf.  Tokens past a sequence's length and pages it does
 * not list are never read; a page id outside [0, num_pages) reads as zeros
 * (no fault; that sequence's result is then meaningless).
 *
 * Sizes: bf16 only (MATTN_F32 returns MATTN_ERR_UNSUPPORTED); D in {64, 128};
 * page_size a positive multiple of 64; Hq a multiple of Hkv.
 * Workspace: caller-owned device memory of at least
 * mattn_fwd_kvcache_workspace_size() bytes (0 is allowed when that is 0)
 * holding the float32 partials of long caches split along the keys; the
 * splits are merged in a fixed order, so results are bitwise reproducible.
 * Every pointer is device memory owned by the caller; q, k_cache, v_cache, o,
 * lse and workspace must be 16-byte aligned, the int32 arrays 4-byte
 * aligned.  Errors are reported before anything is enqueued: null or
 * misaligned pointers, negative sizes, Hq % Hkv != 0, causal not 0/1, a
 * non-finite scale or too small a workspace give MATTN_ERR_INVALID_ARG;
 * unsupported dtype, D or page size, or element counts of 2^31 or more give
 * MATTN_ERR_UNSUPPORTED.  B*Hq*Sq == 0 is a no-op.  Enqueues one kernel, plus
 * a merge kernel when the keys are split, on `stream`. */
size_t mattn_fwd_kvcache_workspace_size(int B, int Hq, int Hkv, int Sq, int D, int page_size,
                                        int pages_per_seq);
mattn_status mattn_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                               const int* block_table, const int* seqlens_k, void* o, float* lse,
                               int B, int Hq, int Hkv, int Sq, int D, int num_pages,
                               int page_size, int pages_per_seq, int causal, float scale,
                               mattn_dtype dtype, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* mattn_strerror(mattn_status s);

/* Library version as major*10000 + minor*100 + patch. */
int mattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MATTN_H */

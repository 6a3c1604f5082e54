/*
 * fa.h - C ABI of the exact-attention library for AMD MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention the way the
 * 'FlashAttention' pages describe it: Q, K and V are cut into tiles that live
 * on chip, the score tile S = scale * Q K^T is formed block by block, a running
 * row maximum and row sum fold each block into the output (online softmax,
 * josueisai.com section on the softmax trick; 'log-sum-exp' rescaling on the
 * kerneldigest.dev glossary entry), and only O plus one log-sum-exp per row
 * reach memory. The backward pass keeps no score or probability matrix: it
 * recomputes them from Q, K, V and the saved log-sum-exp (josueisai.com
 * section on recomputing instead of remembering).
 *
 * Conventions shared by every entry point:
 *  - Tensors are [B, H, rows, d] with d innermost. fa_fwd and fa_bwd take them
 *    dense and contiguous with N rows each; fa_fwd_ex and fa_bwd_ex take Nq
 *    query rows (Q, O, dO, dQ) and Nk key rows (K, V, dK, dV) and, per
 *    tensor, three element strides {batch, head, row} (NULL = contiguous).
 *    Q, K, V, O, dO, dQ, dK and dV all have the element type `dtype`; LSE is
 *    always contiguous float32 [B, H, Nq] and holds the natural-log
 *    log-sum-exp of the scaled scores of each query row.
 *  - Every tensor pointer is a DEVICE pointer (memory of the current HIP
 *    device). Base pointers must be 16-byte aligned. The caller allocates and
 *    owns every buffer; the library allocates, frees and retains nothing
 *    (fa_bwd_noalloc's fixed per-GPU scratch aside, see there).
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    asynchronously; outputs are valid once the stream reaches that point and
 *    inputs must stay unchanged until then.
 *  - Masks. Query i is aligned with key i + Nk - Nq (the queries are the last
 *    Nq positions of the key sequence, as when new tokens attend over a cache
 *    of earlier keys). The _ex calls take a band: key j is visible to query i
 *    iff  i + Nk - Nq - window_left <= j <= i + Nk - Nq + window_right,  a
 *    bound of -1 being absent. causal = 1 in fa_fwd / fa_bwd is the band
 *    (-1, 0): key j is masked for query i whenever j > i. A sliding window of
 *    w earlier keys is (w, 0) (local attention, which josueisai.com's
 *    'FlashAttention' page, section on what you gain and what not, pairs with
 *    the method for very long sequences). Tiles wholly outside the band are
 *    skipped. A query row that sees no key gets O = 0, LSE = -inf and dQ = 0.
 *  - A problem with no query row (B, H or Nq equal to 0) is empty: nothing is
 *    enqueued and FA_OK is returned. With Nk = 0 every row sees no key.
 *  - Errors are returned as fa_status; no exception crosses the ABI. A
 *    request the kernels do not cover returns FA_ERR_UNSUPPORTED; there is
 *    never a silent fallback to a different implementation. After an error,
 *    fa_last_error_detail() (thread-local) explains it.
 *  - The functions are thread-safe and keep no state between calls, except
 *    fa_bwd_noalloc, whose calls share one scratch array per GPU.
 */
#ifndef EXACT_ATTENTION_FA_H
#define EXACT_ATTENTION_FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad flag ... */
  FA_ERR_UNSUPPORTED = 2,      /* valid request outside what is built */
  FA_ERR_HIP = 3               /* HIP runtime or launch failure */
} fa_status;

typedef enum fa_dtype {
  FA_BF16 = 0, /* bfloat16 storage, float32 accumulation */
  FA_FP32 = 1, /* float32 storage and arithmetic (no reduced-precision modes) */
  FA_FP16 = 2  /* IEEE half storage, float32 accumulation (foqum.io's FAQ on
                  FlashAttention names FP16 and BF16 as the formats it runs in) */
} fa_dtype;

/* Library version, major * 10000 + minor * 100 + patch. */
int fa_version(void);

/* Static, human-readable name of a status code. */
const char* fa_status_string(int status);

/* Detail message of the last failing call on this thread ("" if none). */
const char* fa_last_error_detail(void);

/*
 * Forward pass: O = softmax(scale * Q K^T [+ causal mask]) V and
 * LSE_i = ln sum_j exp(scale * q_i . k_j) over the unmasked keys j.
 * (josueisai.com 'FlashAttention': three-step definition in the section on the
 * matrix that should never be stored; tiling and the running max / running sum
 * in the section on the softmax trick.)
 *
 *  Q, K, V  in   [B, H, N, d] of `dtype`
 *  O        out  [B, H, N, d] of `dtype` (rounded to nearest even from fp32)
 *  LSE      out  [B, H, N] float32
 *  scale    any finite float (1/sqrt(d) in the usual use)
 *  d        32, 64, 96, 128 or 256 (fp32: at most 128)
 *  dtype    FA_BF16, FA_FP16 or FA_FP32
 * O and LSE must not overlap any input.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void* stream);

/*
 * Bytes of device workspace fa_bwd needs for this problem: two float32 per
 * query row (the row dot product D_i = sum_k dO_ik O_ik and LSE_i in base 2),
 * with each head's rows padded to a multiple of 64: B*H*ceil(N/64)*64*8.
 * Returns 0 for an empty problem or for arguments fa_bwd would reject.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype);

/*
 * Backward pass: the gradients of sum(O * dO) with respect to Q, K and V,
 * where O = fa_fwd(Q, K, V). Scores and probabilities are recomputed from Q,
 * K and the saved LSE (josueisai.com 'FlashAttention', section on recomputing
 * instead of remembering); with P = exp(scale S - LSE):
 *   dV = P^T dO;  dP = dO V^T;  D_i = sum_k dO_ik O_ik;
 *   dS = P * (dP - D);  dQ = scale dS K;  dK = scale dS^T Q.
 * LSE is an input only (it is not differentiated).
 *
 *  Q, K, V, O, dO  in   [B, H, N, d] of `dtype`; O and LSE as fa_fwd wrote them
 *  LSE             in   [B, H, N] float32
 *  dQ, dK, dV      out  [B, H, N, d] of `dtype`
 *  workspace       device scratch of at least fa_bwd_workspace_bytes() bytes,
 *                  16-byte aligned, owned by the caller
 *  d               32, 64, 96, 128 or 256;  dtype FA_BF16 or FA_FP16
 *                  (FA_FP32 -> UNSUPPORTED)
 * Outputs and the workspace must not overlap any input or each other.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O,
           const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Size of the device scratch that fa_bwd_noalloc uses in place of a
 * workspace: 16 MiB per GPU, i.e. B*H*ceil(N/64)*64 <= 2097152 padded query
 * rows (for example 64 heads of N = 32768, or 32 heads of N = 65536).
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * fa_bwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, definition and results as fa_bwd (bit for bit), minus the
 * workspace: the per-row statistics go to a scratch array of
 * FA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on, from
 * its load until the process ends. The call allocates and frees nothing
 * (no hipMalloc, no library routine that allocates). The caller still owns
 * every input and output.
 *
 * The scratch is shared by every call on one GPU and keeps the last call's
 * contents (the backward overwrites every entry it reads, so no clearing is
 * needed). Calls that overlap in time on one GPU (different streams or host
 * threads without ordering between them) race on it and give undefined
 * results; order them on one stream or use fa_bwd with separate workspaces.
 *
 * Errors: as fa_bwd; a problem with B*H*ceil(N/64)*64*8 bytes of statistics
 * above FA_NOALLOC_SCRATCH_BYTES returns FA_ERR_UNSUPPORTED before any HIP
 * call.
 */
int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                   const void* dO, const float* LSE, void* dQ, void* dK,
                   void* dV, int B, int H, int N, int d, float scale,
                   int causal, int dtype, void* stream);

/*
 * fa_fwd for general shapes, layouts and masks: Nq queries over Nk keys, a
 * band mask (window_left, window_right; -1 = no bound; (-1, -1) = no mask,
 * (-1, 0) = causal, (w, 0) = sliding window), and strided operands. Same
 * definition as fa_fwd otherwise (josueisai.com 'FlashAttention', sections on
 * the matrix that should never be stored and on the softmax trick).
 *
 *  Q, O     [B, H, Nq, d];  K, V  [B, H, Nk, d];  LSE out, contiguous [B, H, Nq]
 *  *_strides  NULL for contiguous, else 3 int64 element strides {batch, head,
 *             row}; d is contiguous (stride 1). Strides must be >= 0, the row
 *             stride >= d, every stride a multiple of 16 bytes (8 elements in
 *             16-bit types, 4 in fp32), and one head's rows must span < 2 GiB;
 *             otherwise FA_ERR_UNSUPPORTED. O's layout must give every element
 *             its own address (FA_ERR_INVALID_ARGUMENT otherwise). Inputs may
 *             share memory (e.g. one packed QKV tensor, or a batch or head
 *             stride of 0 to broadcast K and V).
 *  bias     NULL, or a float32 additive bias on the scaled scores:
 *           S = scale * Q K^T + bias, with bias[b, h, i, j] at
 *           bias + b*s0 + h*s1 + i*s2 + j for bias_strides {s0, s1, s2}
 *           (NULL = contiguous [B, H, Nq, Nk]); strides >= 0 (0 broadcasts,
 *           e.g. {0, 0, 0} for one key-padding row shared by all), multiples
 *           of 4 floats, the row stride s2 below 2^31 floats
 *           (FA_ERR_UNSUPPORTED otherwise), base 16-byte aligned. Entries must be finite or -inf
 *           (-inf removes that key for that query: an arbitrary mask). It is
 *           applied before the band mask and is an input only. 16-bit dtypes
 *           only (FA_FP32 with a bias -> FA_ERR_UNSUPPORTED).
 *  window_left, window_right  -1 or >= 0 (FA_ERR_INVALID_ARGUMENT otherwise)
 * The address range of O (lowest to highest element) and LSE must not overlap
 * any input's.
 */
int fa_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* LSE,
              int B, int H, int Nq, int Nk, int d,
              const long long* q_strides, const long long* k_strides,
              const long long* v_strides, const long long* o_strides,
              const float* bias, const long long* bias_strides,
              float scale, int window_left, int window_right, int dtype,
              void* stream);

/*
 * Bytes of workspace fa_bwd_ex needs: B*H*ceil(Nq/64)*64*8 (two float32 per
 * query row); 0 for an empty problem or arguments fa_bwd_ex would reject.
 */
size_t fa_bwd_ex_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dtype);

/*
 * fa_bwd for general shapes, layouts and masks, with the conventions of
 * fa_fwd_ex. O and LSE are what fa_fwd_ex wrote for the same Q, K, V, band and
 * scale. Key rows that no query sees get dK = dV = 0; query rows that see no
 * key get dQ = 0.
 *
 *  Q, O, dO, dQ  [B, H, Nq, d];  K, V, dK, dV  [B, H, Nk, d]
 *  strides       as fa_fwd_ex, one set per tensor; dQ, dK, dV must each give
 *                every element its own address
 *  bias          the bias fa_fwd_ex was given (or NULL); it is not
 *                differentiated
 *  dtype         FA_BF16 or FA_FP16 (FA_FP32 -> UNSUPPORTED)
 * The address ranges of dQ, dK, dV and the workspace must not overlap any
 * input's (the bias included), LSE's or each other's (separate gradient
 * buffers).
 */
int fa_bwd_ex(const void* Q, const void* K, const void* V, const void* O,
              const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
              int B, int H, int Nq, int Nk, int d,
              const long long* q_strides, const long long* k_strides,
              const long long* v_strides, const long long* o_strides,
              const long long* do_strides, const long long* dq_strides,
              const long long* dk_strides, const long long* dv_strides,
              const float* bias, const long long* bias_strides,
              float scale, int window_left, int window_right, int dtype,
              void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* EXACT_ATTENTION_FA_H */

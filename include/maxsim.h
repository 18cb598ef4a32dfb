/*
 * maxsim.h -- C ABI of the MI355X (gfx950) fused late-interaction MaxSim
 * library, libmaxsim.so.
 *
 * The operation is MaxSim from "Flash-MaxSim: IO-Aware Fused Kernels for
 * Late-Interaction Scoring" (arXiv 2605.29517), Section 1, Eq. (1):
 *
 *     score(Q, D) = sum_i max_j <Q_i, D_j>
 *
 * computed for every (query, document) pair of Nq queries and B documents
 * (the all-pairs regime of Section 3.1) without materialising the
 * [Nq, B, Lq, Ld] similarity tensor, plus the training backward of
 * Section 4.2 and the INT8 and padding-free variants of Section 4.3.
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or synchronises; each call only enqueues work on
 *     `stream` (a hipStream_t passed as void*, NULL = the null stream) and
 *     returns.  Outputs are fully overwritten.
 *   - Tensors are dense, row-major, contiguous.  The embedding width d must be
 *     128 (MAXSIM_ERR_UNSUPPORTED otherwise).  Q, D and D_packed must be
 *     16-byte aligned, every other buffer 4-byte aligned (MAXSIM_ERR_ALIGN).
 *   - Arguments are validated on the host before any HIP call, so every
 *     MAXSIM_ERR_* other than MAXSIM_ERR_HIP is returned without touching the
 *     device.  MAXSIM_ERR_HIP reports a failed launch (hipGetLastError).
 *   - Device-side data are not validated; instead every kernel clamps what it
 *     reads so that no access leaves the buffers described by the sizes:
 *     a document length outside [0, Ld] (padded) is clamped to that range, a
 *     cu_seqlens range outside [0, T) is clamped to it, and an argmax entry
 *     at or past the document's length given to the backward is clamped to
 *     its last token (the gradients are then unspecified, but no access
 *     leaves the buffers).
 *   - In the backward a negative argmax entry -- what the forward writes for
 *     a document with no valid token -- selects no row: the source is in no
 *     CSR bucket and adds nothing to dQ or dD.
 *   - Query-token count Lq is limited to 1 <= Lq <= 1024.
 *   - A document with no valid token scores -inf and every argmax entry of
 *     it is -1 (the running maximum starts at -inf, Section 4.1).
 *   - Argmax indices are local to the document ([0, length)).  The INT8
 *     path returns exactly the first token attaining the maximum.  The
 *     fp16/bf16 paths return a token whose fp32 similarity is within 16 ulp
 *     of the row maximum (for 32x32 MFMA blocks candidates are ranked by the
 *     similarity with its low 4 mantissa bits replaced by the token's slot,
 *     which orders values closer than that by slot, and for negative values
 *     in the reverse slot order); the score itself always uses the exact
 *     fp32 maximum.
 */
#ifndef MAXSIM_H
#define MAXSIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MAXSIM_OK = 0,
    MAXSIM_ERR_NULL = 1,        /* a required pointer is NULL */
    MAXSIM_ERR_SHAPE = 2,       /* a size is negative / zero where not allowed, or overflows */
    MAXSIM_ERR_UNSUPPORTED = 3, /* d != 128, Lq > 1024, unknown dtype, shape beyond a kernel limit */
    MAXSIM_ERR_ALIGN = 4,       /* a pointer is not aligned as required */
    MAXSIM_ERR_WORKSPACE = 5,   /* workspace smaller than maxsim_bwd_workspace_bytes() */
    MAXSIM_ERR_HIP = 6,         /* the HIP runtime rejected a launch */
    MAXSIM_ERR_SCRATCH = 7      /* maxsim_bwd_noalloc: the shape needs more than its fixed scratch */
} maxsim_status;

typedef enum { MAXSIM_F16 = 0, MAXSIM_BF16 = 1 } maxsim_dtype;

/*
 * Fused forward, padded documents (Section 4.1, Algorithm 2; masking of
 * invalid positions to -inf before the row maximum, "Online-Max Recurrence").
 *   Q       [Nq, Lq, d]  fp16 or bf16 (dtype)
 *   D       [B, Ld, d]   same dtype; document b is D[b, :d_lens[b], :]
 *   d_lens  [B] int32 valid lengths, or NULL for "all Ld tokens valid"
 *   scores  [Nq, B] fp32 out: score of query q against document b
 *   argmax  [Nq, B, Lq] int32 out, or NULL to skip it: for each query token
 *           the document token attaining its maximum (Section 4.2, the
 *           saved argmax of "Runtime Inverse-Grid Construction")
 * Arithmetic: products of fp16/bf16 inputs accumulated in fp32 (MFMA), fp32
 * running maximum, fp32 sum over query tokens (Section 4.1 "Numerical
 * Fidelity").  Requires Nq >= 0, B >= 0, 1 <= Lq <= 1024, Ld >= 1.
 */
int maxsim_fwd(const void* Q, const void* D, const int32_t* d_lens, int32_t Nq, int32_t Lq,
               int32_t B, int32_t Ld, int32_t d, int32_t dtype, float* scores, int32_t* argmax,
               void* stream);

/*
 * Fused forward, padding-free documents (Section 4.3 "Padding-Free
 * Variable-Length"): only the real tokens are read and scored.
 *   D_packed    [T, d] the documents' tokens back to back
 *   cu_seqlens  [B+1] int32, cu_seqlens[0] = 0, non-decreasing; document b is
 *               rows [cu_seqlens[b], cu_seqlens[b+1]) of D_packed
 *   max_Ld      an upper bound of the document lengths (>= 1)
 * Other arguments and outputs as maxsim_fwd; argmax is local to the document.
 */
int maxsim_fwd_varlen(const void* Q, const void* D_packed, const int32_t* cu_seqlens, int32_t Nq,
                      int32_t Lq, int32_t B, int64_t T, int32_t max_Ld, int32_t d, int32_t dtype,
                      float* scores, int32_t* argmax, void* stream);

/*
 * INT8 x INT8 forward over padding-free documents (Section 4.3 "INT8xINT8
 * Quantization": per-token symmetric scales, dequantisation fused into the
 * kernel).  The page leaves the arithmetic open; this library computes,
 * exactly and bit-reproducibly:
 *     dot_ij = sum_k Q[q,i,k] * D[j,k]                 (int32, exact)
 *     s_ij   = fl32((float)dot_ij * d_scale[j])
 *     m_i    = max_j s_ij           argmax_i = first j attaining m_i
 *     v_i    = fl32(m_i * q_scale[q,i])
 *     score  = fp32 sum of v_i in ascending i, no fused multiply-add
 *   Q [Nq, Lq, d] int8, q_scale [Nq, Lq] fp32 (> 0)
 *   D_packed [T, d] int8, d_scale [T] fp32 in [2^-125, 2^100], cu_seqlens as above.
 * The d_scale range is what the kernel's exact arithmetic needs (it forms
 * fl32(dot_ij * d_scale[j]) / 2 for negative dot_ij and doubles the maximum
 * back); the quantiser's scales (max|x| / 127, or 1) lie far inside it.
 */
int maxsim_fwd_i8(const int8_t* Q, const float* q_scale, const int8_t* D_packed,
                  const float* d_scale, const int32_t* cu_seqlens, int32_t Nq, int32_t Lq,
                  int32_t B, int64_t T, int32_t max_Ld, int32_t d, float* scores, int32_t* argmax,
                  void* stream);

/* Bytes of device workspace maxsim_bwd needs for these sizes (0 on bad sizes). */
size_t maxsim_bwd_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq, int32_t Ld);

/*
 * Backward, padded documents (Section 4.2, Algorithm 3).
 *   Q [Nq, Lq, d], D [B, Ld, d] (dtype), argmax [Nq, B, Lq] int32 from the
 *   forward, grad_scores [Nq, B] fp32 = dL/dscore.
 * Step 1, inverse-grid CSR ("Runtime Inverse-Grid Construction"): with the
 *   source id s = (q*B + b)*Lq + i and destination dst(s) = b*Ld + argmax[s]
 *   (no destination when argmax[s] < 0: a document of d_lens 0),
 *     row_ptr [B*Ld + 1] out: exclusive prefix sum of the per-row counts
 *                             (row_ptr[B*Ld] = number of sources with a row),
 *     col_idx [Nq*B*Lq]  out (capacity): the sources of row r in ascending s
 *                             at col_idx[row_ptr[r] .. row_ptr[r+1]); entries
 *                             past row_ptr[B*Ld] are unspecified.
 *   Both are deterministic (bit-identical on every call).
 * Step 2, destination-owned dD ("Destination-Owned Reduction", Eq. (dd)):
 *     dD [B, Ld, d] fp32 out, dD[b,t] = sum over the sources s of row b*Ld+t
 *     of grad_scores[q(s), b] * Q[q(s), i(s)]; rows with no source are 0.
 *     Each row is written once by its owner, no atomics.
 * Step 3, gathered dQ (Eq. (dq)):
 *     dQ [Nq, Lq, d] fp32 out, dQ[q,i] = sum_b grad_scores[q,b] * D[b, argmax[q,b,i]].
 *     With few query rows the documents are split into chunks whose partial
 *     sums are added in ascending chunk order (still bit-reproducible).
 * workspace: device scratch of at least maxsim_bwd_workspace_bytes() bytes,
 * 16-byte aligned; its contents on entry do not matter.
 * Requires Nq, B >= 1, 1 <= Lq <= 1024, 1 <= Ld <= 4096, Nq*B*Lq < 2^31,
 * B*Ld < 2^31.
 */
int maxsim_bwd(const void* Q, const void* D, int32_t dtype, const int32_t* argmax,
               const float* grad_scores, int32_t Nq, int32_t Lq, int32_t B, int32_t Ld, int32_t d,
               float* dQ, float* dD, int32_t* row_ptr, int32_t* col_idx, void* workspace,
               size_t workspace_bytes, void* stream);

/*
 * Allocation-free variant of maxsim_bwd, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc): the same kernels and results as maxsim_bwd, with
 * the workspace taken from a device array the library holds, of
 * maxsim_bwd_noalloc_scratch_bytes() bytes (64 MiB) on every GPU it runs on,
 * for the life of the process.  The caller passes inputs and outputs as for
 * maxsim_bwd.  The call allocates nothing (no hipMalloc, no library routine
 * that allocates); its first call on a device looks up that device's copy
 * of the array (hipGetSymbolAddress) with the device current.
 *   Returns MAXSIM_ERR_SCRATCH, before any HIP call, when
 *   maxsim_bwd_workspace_bytes() of the shape exceeds the array; other
 *   arguments and errors as maxsim_bwd.
 * Every call on one device shares that device's array: calls that overlap
 * on one device (different streams or threads) race and give unspecified
 * results.  Calls ordered on one stream are safe; each call writes every
 * scratch word it reads.
 */
size_t maxsim_bwd_noalloc_scratch_bytes(void);
int maxsim_bwd_noalloc(const void* Q, const void* D, int32_t dtype, const int32_t* argmax,
                       const float* grad_scores, int32_t Nq, int32_t Lq, int32_t B, int32_t Ld, int32_t d,
                       float* dQ, float* dD, int32_t* row_ptr, int32_t* col_idx, void* stream);

/* Bytes of device workspace maxsim_bwd_varlen needs (0 on bad sizes). */
size_t maxsim_bwd_varlen_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq, int32_t max_Ld);

/*
 * Backward over padding-free documents (Section 4.2, Algorithm 3, with the
 * packed layout of Section 4.3 "Padding-Free Variable-Length").
 *   Q [Nq, Lq, d] and D_packed [T, d] (dtype), cu_seqlens [B+1] as for
 *   maxsim_fwd_varlen (cu_seqlens[B] = T, every length <= max_Ld), argmax
 *   [Nq, B, Lq] int32 from maxsim_fwd_varlen (local to the document),
 *   grad_scores [Nq, B] fp32.
 * A source s = (q*B + b)*Lq + i selects the packed row cu_seqlens[b] +
 * argmax[s]; an empty document has no rows and its sources select nothing
 * (their argmax and grad_scores entries are ignored).
 *   row_ptr [T + 1] out: exclusive prefix of the per-row counts, so that
 *           row_ptr[T] = Nq*Lq * (number of non-empty documents);
 *   col_idx [Nq*B*Lq] out (capacity): the first row_ptr[T] entries hold the
 *           sources of row r in ascending s at col_idx[row_ptr[r] ..
 *           row_ptr[r+1]); the rest is left unspecified;
 *   dD [T, d] fp32 out (Eq. (dd)), rows with no source are 0;
 *   dQ [Nq, Lq, d] fp32 out (Eq. (dq)), summed over the non-empty documents.
 * T = 0 is allowed (D_packed and dD may then be NULL; dQ is all zero).
 * workspace: device scratch of maxsim_bwd_varlen_workspace_bytes() bytes,
 * 256-byte aligned; its contents on entry do not matter.  Requires Nq, B >= 1,
 * 1 <= Lq <= 1024, 1 <= max_Ld <= 4096, Nq*B*Lq < 2^31, T < 2^31.  A
 * malformed cu_seqlens gives unspecified gradients but no access outside
 * the buffers.
 */
int maxsim_bwd_varlen(const void* Q, const void* D_packed, const int32_t* cu_seqlens, int32_t dtype,
                      const int32_t* argmax, const float* grad_scores, int32_t Nq, int32_t Lq, int32_t B,
                      int64_t T, int32_t max_Ld, int32_t d, float* dQ, float* dD, int32_t* row_ptr,
                      int32_t* col_idx, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace maxsim_bwd_scatter needs (0 on bad sizes). */
size_t maxsim_bwd_scatter_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq);

/*
 * Backward with dD by atomic scatter: the low-contention alternative the
 * pages pair with the destination-owned reduction (Section 4.2,
 * "Destination-Owned Reduction", the dispatch remark at its end).  dD is
 * cleared and every source adds grad_scores[q,b] * Q[q,i] into its row with
 * fp32 atomic adds; dQ is gathered exactly as in maxsim_bwd.  No CSR map is
 * built and no workspace is needed.  The order of the adds into one row is
 * not fixed, so dD may differ between runs in the last bits (maxsim_bwd is
 * bit-reproducible); rows no source selects are exactly 0.
 *   cu_seqlens NULL: padded, D and dD are [B, Ld, d] and T is ignored;
 *   otherwise packed as for maxsim_bwd_varlen, D_packed and dD are [T, d]
 *   and Ld is the longest document.
 * workspace: device scratch of maxsim_bwd_scatter_workspace_bytes() bytes,
 * 256-byte aligned (partial dQ sums when the documents are split in chunks).
 * Other arguments and requirements as maxsim_bwd / maxsim_bwd_varlen.
 */
int maxsim_bwd_scatter(const void* Q, const void* D, const int32_t* cu_seqlens, int32_t dtype,
                       const int32_t* argmax, const float* grad_scores, int32_t Nq, int32_t Lq, int32_t B,
                       int32_t Ld, int64_t T, int32_t d, float* dQ, float* dD, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * The dispatch rule between the two dD reductions: 1 when the atomic scatter
 * (maxsim_bwd_scatter) is expected to be faster than the CSR path for Nq
 * queries of Lq tokens against B documents of `rows` rows in total (B*Ld
 * padded, T packed), else 0.  The rule compares the mean number of sources
 * per destination row, Nq*Lq*B / rows, with a threshold measured on MI355X.
 * Returns 0 for non-positive sizes.  Host-only; launches nothing.
 */
int maxsim_bwd_prefer_scatter(int32_t Nq, int32_t Lq, int32_t B, int64_t rows);

/* Bytes of device staging maxsim_fwd_host_stream needs (0 on bad sizes). */
size_t maxsim_fwd_host_stream_staging_bytes(int32_t Nq, int32_t Lq, int32_t Ld, int32_t block_docs,
                                            int32_t with_argmax);

/*
 * Out-of-core forward (Section 5 "Out-of-Core Corpus Scaling", Table 4): the
 * corpus stays in host memory and is streamed to the GPU in blocks of
 * block_docs documents; each block is scored by the fused forward while the
 * next one is copied, so device memory holds two blocks, not the corpus.
 *   Q [Nq, Lq, d] device (dtype).
 *   D_host: the corpus in host memory, padded [B, Ld, d] (cu_seqlens_host
 *     NULL; d_lens device [B] or NULL as for maxsim_fwd) or packed [T, d]
 *     with cu_seqlens_host (host [B+1], read during this call; cu[0] = 0,
 *     every length <= Ld) and cu_seqlens (the same on the device).  Ld is the
 *     padded row stride, or the longest packed document (D_host may be NULL
 *     for a packed corpus without rows).  Pinned memory
 *     (hipHostMalloc) is needed for full copy speed; any host memory works.
 *   scores [Nq, B] fp32 out (device), argmax [Nq, B, Lq] int32 out or NULL.
 *   staging: device memory of maxsim_fwd_host_stream_staging_bytes() bytes,
 *     256-byte aligned: two document blocks, the block's scores, cu_seqlens
 *     and argmax.
 * The call enqueues all work and returns: the copies run on a stream the
 * library creates once per device, the forward on `stream`, which is ordered
 * after the last block.  D_host and staging must stay valid until `stream`
 * has finished.  Calls on one device are serialised while they enqueue.  Not
 * for HIP graph capture.  Results equal maxsim_fwd / maxsim_fwd_varlen on the
 * same documents.  Requires block_docs >= 1; other arguments as maxsim_fwd.
 */
int maxsim_fwd_host_stream(const void* Q, const void* D_host, const int32_t* cu_seqlens_host,
                           const int32_t* cu_seqlens, const int32_t* d_lens, int32_t Nq, int32_t Lq, int32_t B,
                           int32_t Ld, int32_t d, int32_t dtype, int32_t block_docs, void* staging,
                           size_t staging_bytes, float* scores, int32_t* argmax, void* stream);

/* Bytes of device workspace maxsim_chamfer_fwd needs (0 on bad sizes). */
size_t maxsim_chamfer_fwd_workspace_bytes(int32_t Bt, int32_t N, int32_t M);

/*
 * Chamfer forward (Section 4.2 "Generalization to Chamfer Distance"): the
 * same hard selection with the minimum of squared Euclidean distances in
 * place of the maximum of inner products, between point clouds
 * P [Bt, N, 3] and Q [Bt, M, 3] (fp32, device; item b of P is compared with
 * item b of Q only).  No [N, M] matrix is formed.
 *   dist_p [Bt, N] fp32 out: min over j of |P[b,i] - Q[b,j]|^2 (fp32,
 *     (dx*dx + dy*dy) + dz*dz with fused multiply-adds);
 *   idx_p [Bt, N] int32 out: the first j attaining it (-1 when M = 0, with
 *     dist +inf);
 *   dist_q, idx_q [Bt, M]: the same from Q to P.
 * The page's loss is mean(dist_p) + mean(dist_q) per item.
 * workspace: maxsim_chamfer_fwd_workspace_bytes() bytes, 256-byte aligned.
 * Requires Bt, N, M >= 0, Bt*N and Bt*M < 2^31.
 */
int maxsim_chamfer_fwd(const float* P, const float* Q, int32_t Bt, int32_t N, int32_t M, float* dist_p,
                       int32_t* idx_p, float* dist_q, int32_t* idx_q, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Bytes of device workspace maxsim_chamfer_bwd needs (0 on bad sizes). */
size_t maxsim_chamfer_bwd_workspace_bytes(int32_t Bt, int32_t N, int32_t M);

/*
 * Chamfer backward through the saved selections (Section 4.2: the same
 * inverse-grid CSR and destination-owned rows as the MaxSim backward).
 * With grad_p [Bt, N] = dL/d dist_p and grad_q [Bt, M] = dL/d dist_q:
 *   dP[b,i] = 2 grad_p[b,i] (P[b,i] - Q[b,idx_p[b,i]])
 *           + sum over j with idx_q[b,j] = i of 2 grad_q[b,j] (P[b,i] - Q[b,j])
 *   dQ[b,j] likewise with the roles of the clouds swapped (fp32 out).
 * CSR maps (deterministic, sources in ascending order):
 *   row_ptr_p [Bt*N + 1], col_idx_p [Bt*M]: for P point r = b*N + i, the Q
 *     points (global index b*M + j) that select it;
 *   row_ptr_q [Bt*M + 1], col_idx_q [Bt*N]: the same for the Q points.
 *   Entries past row_ptr[last] (sources with idx -1) are unspecified.
 * Selections of -1 add nothing.  workspace: maxsim_chamfer_bwd_workspace_bytes()
 * bytes, 256-byte aligned.  Requirements as maxsim_chamfer_fwd, and also
 * Bt*(N+M) < 2^31 (both directions' selections are sorted together with
 * int32 offsets); MAXSIM_ERR_SHAPE otherwise.
 */
int maxsim_chamfer_bwd(const float* P, const float* Q, const int32_t* idx_p, const int32_t* idx_q,
                       const float* grad_p, const float* grad_q, int32_t Bt, int32_t N, int32_t M, float* dP,
                       float* dQ, int32_t* row_ptr_p, int32_t* col_idx_p, int32_t* row_ptr_q, int32_t* col_idx_q,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Scores of an explicit list of (query, document) pairs over a packed corpus
 * (Eq. (1) for each listed pair only).  This is the rescoring pass of the
 * two-stage INT8 -> fp16 scan the pages list in the forward kernel family
 * (Section 4.1 "Kernel Family"), where each query has its own candidates.
 *   Q [Nq, Lq, d] and D_packed [T, d] (dtype), cu_seqlens [B+1] as for
 *   maxsim_fwd_varlen; pair p is query pair_q[p] against document pair_b[p]
 *   (device int32 arrays of P entries, 0 <= pair_q < Nq, 0 <= pair_b < B;
 *   entries out of range are clamped into range).
 *   scores [P] fp32 out; argmax [P, Lq] int32 out or NULL (exact first index
 *   on ties; -1 and -inf for an empty document).
 * Requires d = 128, 1 <= Lq <= 1024, P >= 0 (P = 0 does nothing).
 */
int maxsim_fwd_pairs(const void* Q, const void* D_packed, const int32_t* cu_seqlens, int32_t dtype,
                     const int32_t* pair_q, const int32_t* pair_b, int32_t P, int32_t Nq, int32_t Lq,
                     int32_t B, int64_t T, int32_t d, float* scores, int32_t* argmax, void* stream);

/*
 * Top-K of every query's row of scores [Nq, B] fp32 (the selection of the
 * two-stage scan, Section 4.1 "Kernel Family"): top_idx [Nq, K] and
 * top_score [Nq, K] out, best first; equal scores are ordered by ascending
 * id, where the id of entry (q, j) is ids[q*B + j] when ids (device int32
 * [Nq, B], values >= 0) is given, else j.  top_idx holds the ids.
 * -0.0 and +0.0 are equal scores (reported as +0.0).
 * Requires 1 <= K <= min(B, 1024).  NaN scores are not supported.
 */
int maxsim_topk(const float* scores, const int32_t* ids, int32_t Nq, int32_t B, int32_t K, int32_t* top_idx,
                float* top_score, void* stream);

/* Bytes of device workspace maxsim_two_stage_topk needs (0 on bad sizes). */
size_t maxsim_two_stage_workspace_bytes(int32_t Nq, int32_t B, int32_t K1);

/*
 * The two-stage scan (Section 4.1 "Kernel Family"): INT8 x INT8 scores of
 * every (query, document) pair (maxsim_fwd_i8), each query's K1 best
 * documents (maxsim_topk), their fp16/bf16 scores from Q16 / D16, the same
 * rows unquantised (maxsim_fwd_pairs), and the K2 best of those.
 *   cand [Nq, K1], cand_score8 [Nq, K1] out: the candidates and INT8 scores;
 *   top_idx [Nq, K2], top_score [Nq, K2] out: the final documents and
 *   fp16/bf16 scores, best first, equal scores by ascending document index.
 * workspace: device scratch of maxsim_two_stage_workspace_bytes() bytes,
 * 256-byte aligned.  Requires 1 <= K2 <= K1 <= min(B, 1024); the other
 * arguments as for maxsim_fwd_i8 and maxsim_fwd_pairs.
 */
int maxsim_two_stage_topk(const int8_t* Q8, const float* q_scale, const int8_t* D8, const float* d_scale,
                          const void* Q16, const void* D16, const int32_t* cu_seqlens, int32_t dtype16,
                          int32_t Nq, int32_t Lq, int32_t B, int64_t T, int32_t max_Ld, int32_t d,
                          int32_t K1, int32_t K2, int32_t* cand, float* cand_score8, int32_t* top_idx,
                          float* top_score, void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* maxsim_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MAXSIM_H */

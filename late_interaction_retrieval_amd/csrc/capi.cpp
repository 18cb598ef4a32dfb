// capi.cpp -- the C ABI declared in include/maxsim.h: host-side argument
// validation (no HIP call before it passes), then the kernel launchers.
#include "maxsim.h"

#include <hip/hip_runtime_api.h>

#include "internal.h"

namespace {

using maxsim::kDim;
using maxsim::kMaxLq;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_common(int32_t Nq, int32_t Lq, int32_t B, int32_t d) {
    if (Nq < 0 || B < 0 || Lq < 1) return MAXSIM_ERR_SHAPE;
    if (d != kDim || Lq > kMaxLq) return MAXSIM_ERR_UNSUPPORTED;
    // every output index (q*B + b)*Lq + i must fit in int64 comfortably and the
    // grid in 32 bits; sizes beyond 2^40 outputs are rejected outright
    if ((int64_t)Nq * B > (int64_t)1 << 40) return MAXSIM_ERR_SHAPE;
    return MAXSIM_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_HIP; }

}  // namespace

extern "C" {

int maxsim_fwd(const void* Q, const void* D, const int32_t* d_lens, int32_t Nq, int32_t Lq,
               int32_t B, int32_t Ld, int32_t d, int32_t dtype, float* scores, int32_t* argmax,
               void* stream) {
    int st = check_common(Nq, Lq, B, d);
    if (st != MAXSIM_OK) return st;
    if (Ld < 1) return MAXSIM_ERR_SHAPE;
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_UNSUPPORTED;
    if (Nq == 0 || B == 0) return MAXSIM_OK;
    if (!Q || !D || !scores) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(scores, 4) || !aligned(argmax, 4) ||
        !aligned(d_lens, 4))
        return MAXSIM_ERR_ALIGN;
    maxsim::FwdArgs a{};
    a.Q = Q;
    a.D = D;
    a.d_lens = d_lens;
    a.Nq = Nq;
    a.Lq = Lq;
    a.B = B;
    a.Ld = Ld;
    a.T = (int64_t)B * Ld;
    a.scores = scores;
    a.argmax = argmax;
    a.elem = dtype == MAXSIM_BF16 ? maxsim::kBF16 : maxsim::kF16;
    a.varlen = false;
    return hip_status(maxsim::launch_fwd(a, static_cast<hipStream_t>(stream)));
}

int maxsim_fwd_varlen(const void* Q, const void* D_packed, const int32_t* cu_seqlens, int32_t Nq,
                      int32_t Lq, int32_t B, int64_t T, int32_t max_Ld, int32_t d, int32_t dtype,
                      float* scores, int32_t* argmax, void* stream) {
    int st = check_common(Nq, Lq, B, d);
    if (st != MAXSIM_OK) return st;
    if (T < 0 || max_Ld < 1) return MAXSIM_ERR_SHAPE;
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_UNSUPPORTED;
    if (Nq == 0 || B == 0) return MAXSIM_OK;
    if (!Q || !cu_seqlens || !scores || (T > 0 && !D_packed)) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D_packed, 16) || !aligned(cu_seqlens, 4) ||
        !aligned(scores, 4) || !aligned(argmax, 4))
        return MAXSIM_ERR_ALIGN;
    maxsim::FwdArgs a{};
    a.Q = Q;
    a.D = D_packed;
    a.cu = cu_seqlens;
    a.Nq = Nq;
    a.Lq = Lq;
    a.B = B;
    a.Ld = max_Ld;
    a.T = T;
    a.scores = scores;
    a.argmax = argmax;
    a.elem = dtype == MAXSIM_BF16 ? maxsim::kBF16 : maxsim::kF16;
    a.varlen = true;
    return hip_status(maxsim::launch_fwd(a, static_cast<hipStream_t>(stream)));
}

int maxsim_fwd_i8(const int8_t* Q, const float* q_scale, const int8_t* D_packed,
                  const float* d_scale, const int32_t* cu_seqlens, int32_t Nq, int32_t Lq,
                  int32_t B, int64_t T, int32_t max_Ld, int32_t d, float* scores, int32_t* argmax,
                  void* stream) {
    int st = check_common(Nq, Lq, B, d);
    if (st != MAXSIM_OK) return st;
    if (T < 0 || max_Ld < 1) return MAXSIM_ERR_SHAPE;
    if (Nq == 0 || B == 0) return MAXSIM_OK;
    if (!Q || !q_scale || !cu_seqlens || !scores || (T > 0 && (!D_packed || !d_scale)))
        return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D_packed, 16) || !aligned(q_scale, 4) ||
        !aligned(d_scale, 4) || !aligned(cu_seqlens, 4) || !aligned(scores, 4) ||
        !aligned(argmax, 4))
        return MAXSIM_ERR_ALIGN;
    maxsim::FwdArgs a{};
    a.Q = Q;
    a.D = D_packed;
    a.cu = cu_seqlens;
    a.q_scale = q_scale;
    a.d_scale = d_scale;
    a.Nq = Nq;
    a.Lq = Lq;
    a.B = B;
    a.Ld = max_Ld;
    a.T = T;
    a.scores = scores;
    a.argmax = argmax;
    a.elem = maxsim::kI8;
    a.varlen = true;
    return hip_status(maxsim::launch_fwd(a, static_cast<hipStream_t>(stream)));
}

size_t maxsim_bwd_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq, int32_t Ld) {
    if (Nq < 1 || B < 1 || Lq < 1 || Ld < 1) return 0;
    return maxsim::bwd_workspace_bytes(Nq, B, Lq, Ld);
}

}  // extern "C"

namespace {
// The padded backward's arguments other than its workspace.
int check_bwd(const void* Q, const void* D, int32_t dtype, const int32_t* argmax, const float* grad_scores,
              int32_t Nq, int32_t Lq, int32_t B, int32_t Ld, int32_t d, const float* dQ, const float* dD,
              const int32_t* row_ptr, const int32_t* col_idx) {
    if (Nq < 1 || B < 1 || Lq < 1 || Ld < 1) return MAXSIM_ERR_SHAPE;
    if ((int64_t)Nq * B * Lq >= ((int64_t)1 << 31)) return MAXSIM_ERR_SHAPE;
    if ((int64_t)B * Ld >= ((int64_t)1 << 31)) return MAXSIM_ERR_SHAPE;
    if (d != kDim || Lq > kMaxLq || Ld > maxsim::kMaxLdBwd) return MAXSIM_ERR_UNSUPPORTED;
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_UNSUPPORTED;
    if (!Q || !D || !argmax || !grad_scores || !dQ || !dD || !row_ptr || !col_idx) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(dQ, 16) || !aligned(dD, 16) ||
        !aligned(argmax, 4) || !aligned(grad_scores, 4) || !aligned(row_ptr, 4) || !aligned(col_idx, 4))
        return MAXSIM_ERR_ALIGN;
    return MAXSIM_OK;
}

int launch_bwd_padded(const void* Q, const void* D, int32_t dtype, const int32_t* argmax, const float* grad_scores,
                      int32_t Nq, int32_t Lq, int32_t B, int32_t Ld, float* dQ, float* dD, int32_t* row_ptr,
                      int32_t* col_idx, void* workspace, void* stream) {
    maxsim::BwdArgs a{};
    a.Q = Q;
    a.D = D;
    a.argmax = argmax;
    a.g = grad_scores;
    a.Nq = Nq;
    a.Lq = Lq;
    a.B = B;
    a.Ld = Ld;
    a.elem = dtype == MAXSIM_BF16 ? maxsim::kBF16 : maxsim::kF16;
    a.dQ = dQ;
    a.dD = dD;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.workspace = workspace;
    return hip_status(maxsim::launch_bwd(a, static_cast<hipStream_t>(stream)));
}
}  // namespace

extern "C" {

int maxsim_bwd(const void* Q, const void* D, int32_t dtype, const int32_t* argmax,
               const float* grad_scores, int32_t Nq, int32_t Lq, int32_t B, int32_t Ld, int32_t d,
               float* dQ, float* dD, int32_t* row_ptr, int32_t* col_idx, void* workspace,
               size_t workspace_bytes, void* stream) {
    const int st = check_bwd(Q, D, dtype, argmax, grad_scores, Nq, Lq, B, Ld, d, dQ, dD, row_ptr, col_idx);
    if (st != MAXSIM_OK) return st;
    if (!workspace) return MAXSIM_ERR_NULL;
    if (!aligned(workspace, 16)) return MAXSIM_ERR_ALIGN;
    if (workspace_bytes < maxsim::bwd_workspace_bytes(Nq, B, Lq, Ld)) return MAXSIM_ERR_WORKSPACE;
    return launch_bwd_padded(Q, D, dtype, argmax, grad_scores, Nq, Lq, B, Ld, dQ, dD, row_ptr, col_idx, workspace,
                             stream);
}

size_t maxsim_bwd_noalloc_scratch_bytes(void) { return maxsim::kScratchBytes; }

int maxsim_bwd_noalloc(const void* Q, const void* D, int32_t dtype, const int32_t* argmax,
                       const float* grad_scores, int32_t Nq, int32_t Lq, int32_t B, int32_t Ld, int32_t d,
                       float* dQ, float* dD, int32_t* row_ptr, int32_t* col_idx, void* stream) {
    const int st = check_bwd(Q, D, dtype, argmax, grad_scores, Nq, Lq, B, Ld, d, dQ, dD, row_ptr, col_idx);
    if (st != MAXSIM_OK) return st;
    if (maxsim::bwd_workspace_bytes(Nq, B, Lq, Ld) > maxsim::kScratchBytes) return MAXSIM_ERR_SCRATCH;
    void* scratch = nullptr;
    if (maxsim::scratch_address(&scratch) != hipSuccess) return MAXSIM_ERR_HIP;
    return launch_bwd_padded(Q, D, dtype, argmax, grad_scores, Nq, Lq, B, Ld, dQ, dD, row_ptr, col_idx, scratch,
                             stream);
}

size_t maxsim_bwd_varlen_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq, int32_t max_Ld) {
    if (Nq < 1 || B < 1 || Lq < 1 || max_Ld < 1) return 0;
    return maxsim::bwd_varlen_workspace_bytes(Nq, B, Lq, max_Ld);
}

int maxsim_bwd_varlen(const void* Q, const void* D_packed, const int32_t* cu_seqlens, int32_t dtype,
                      const int32_t* argmax, const float* grad_scores, int32_t Nq, int32_t Lq, int32_t B,
                      int64_t T, int32_t max_Ld, int32_t d, float* dQ, float* dD, int32_t* row_ptr,
                      int32_t* col_idx, void* workspace, size_t workspace_bytes, void* stream) {
    if (Nq < 1 || B < 1 || Lq < 1 || max_Ld < 1 || T < 0) return MAXSIM_ERR_SHAPE;
    if ((int64_t)Nq * B * Lq >= ((int64_t)1 << 31)) return MAXSIM_ERR_SHAPE;
    if (T >= ((int64_t)1 << 31)) return MAXSIM_ERR_SHAPE;
    if (d != kDim || Lq > kMaxLq || max_Ld > maxsim::kMaxLdBwd) return MAXSIM_ERR_UNSUPPORTED;
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_UNSUPPORTED;
    if (!Q || !cu_seqlens || !argmax || !grad_scores || !dQ || !row_ptr || !col_idx || !workspace ||
        (T > 0 && (!D_packed || !dD)))
        return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D_packed, 16) || !aligned(dQ, 16) || !aligned(dD, 16) ||
        !aligned(cu_seqlens, 4) || !aligned(argmax, 4) || !aligned(grad_scores, 4) ||
        !aligned(row_ptr, 4) || !aligned(col_idx, 4) || !aligned(workspace, 256))
        return MAXSIM_ERR_ALIGN;
    if (workspace_bytes < maxsim::bwd_varlen_workspace_bytes(Nq, B, Lq, max_Ld)) return MAXSIM_ERR_WORKSPACE;
    maxsim::BwdArgs a{};
    a.Q = Q;
    a.D = D_packed;
    a.argmax = argmax;
    a.g = grad_scores;
    a.Nq = Nq;
    a.Lq = Lq;
    a.B = B;
    a.Ld = max_Ld;
    a.elem = dtype == MAXSIM_BF16 ? maxsim::kBF16 : maxsim::kF16;
    a.dQ = dQ;
    a.dD = dD;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.workspace = workspace;
    a.cu_seqlens = cu_seqlens;
    a.T = T;
    return hip_status(maxsim::launch_bwd(a, static_cast<hipStream_t>(stream)));
}

size_t maxsim_bwd_scatter_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq) {
    return maxsim::bwd_scatter_workspace_bytes(Nq, B, Lq);
}

int maxsim_bwd_scatter(const void* Q, const void* D, const int32_t* cu_seqlens, int32_t dtype,
                       const int32_t* argmax, const float* grad_scores, int32_t Nq, int32_t Lq, int32_t B,
                       int32_t Ld, int64_t T, int32_t d, float* dQ, float* dD, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (Nq < 1 || B < 1 || Lq < 1 || Ld < 1) return MAXSIM_ERR_SHAPE;
    if ((int64_t)Nq * B * Lq >= ((int64_t)1 << 31)) return MAXSIM_ERR_SHAPE;
    const int64_t rows = cu_seqlens ? T : (int64_t)B * Ld;
    if (rows < 0 || rows >= ((int64_t)1 << 31)) return MAXSIM_ERR_SHAPE;
    if (d != kDim || Lq > kMaxLq || Ld > maxsim::kMaxLdBwd) return MAXSIM_ERR_UNSUPPORTED;
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_UNSUPPORTED;
    if (!Q || !argmax || !grad_scores || !dQ || !workspace || (rows > 0 && (!D || !dD))) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(dQ, 16) || !aligned(dD, 16) ||
        !aligned(cu_seqlens, 4) || !aligned(argmax, 4) || !aligned(grad_scores, 4) || !aligned(workspace, 256))
        return MAXSIM_ERR_ALIGN;
    if (workspace_bytes < maxsim::bwd_scatter_workspace_bytes(Nq, B, Lq)) return MAXSIM_ERR_WORKSPACE;
    maxsim::BwdArgs a{};
    a.Q = Q;
    a.D = D;
    a.argmax = argmax;
    a.g = grad_scores;
    a.Nq = Nq;
    a.Lq = Lq;
    a.B = B;
    a.Ld = Ld;
    a.elem = dtype == MAXSIM_BF16 ? maxsim::kBF16 : maxsim::kF16;
    a.dQ = dQ;
    a.dD = dD;
    a.cu_seqlens = cu_seqlens;
    a.T = cu_seqlens ? T : 0;
    a.workspace = workspace;
    return hip_status(maxsim::launch_bwd_scatter(a, static_cast<hipStream_t>(stream)));
}

int maxsim_bwd_prefer_scatter(int32_t Nq, int32_t Lq, int32_t B, int64_t rows) {
    if (Nq < 1 || Lq < 1 || B < 1 || rows < 1) return 0;
    // mean number of sources (query tokens) per destination row
    const double per_row = (double)Nq * Lq * B / (double)rows;
    return per_row < maxsim::kScatterMaxSourcesPerRow ? 1 : 0;
}

size_t maxsim_fwd_host_stream_staging_bytes(int32_t Nq, int32_t Lq, int32_t Ld, int32_t block_docs,
                                            int32_t with_argmax) {
    if (Lq > kMaxLq) return 0;
    return maxsim::host_stream_staging_bytes(Nq, Lq, Ld, block_docs, with_argmax != 0);
}

int maxsim_fwd_host_stream(const void* Q, const void* D_host, const int32_t* cu_seqlens_host,
                           const int32_t* cu_seqlens, const int32_t* d_lens, int32_t Nq, int32_t Lq, int32_t B,
                           int32_t Ld, int32_t d, int32_t dtype, int32_t block_docs, void* staging,
                           size_t staging_bytes, float* scores, int32_t* argmax, void* stream) {
    int st = check_common(Nq, Lq, B, d);
    if (st != MAXSIM_OK) return st;
    if (Ld < 1 || block_docs < 1) return MAXSIM_ERR_SHAPE;
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_UNSUPPORTED;
    if (Nq == 0 || B == 0) return MAXSIM_OK;
    const bool packed = cu_seqlens_host != nullptr;
    if (!Q || !scores || !staging || (packed && !cu_seqlens)) return MAXSIM_ERR_NULL;
    if (!D_host && (!packed || cu_seqlens_host[B] != 0)) return MAXSIM_ERR_NULL;  // only an empty corpus has none
    if (packed && d_lens) return MAXSIM_ERR_SHAPE;  // lengths come from cu_seqlens
    if (!aligned(Q, 16) || !aligned(D_host, 16) || !aligned(scores, 4) || !aligned(argmax, 4) ||
        !aligned(d_lens, 4) || !aligned(cu_seqlens, 4) || !aligned(cu_seqlens_host, 4) || !aligned(staging, 256))
        return MAXSIM_ERR_ALIGN;
    if (staging_bytes < maxsim::host_stream_staging_bytes(Nq, Lq, Ld, block_docs, argmax != nullptr))
        return MAXSIM_ERR_WORKSPACE;
    if (packed) {  // the host offsets are read here: every block must fit its buffer
        if (cu_seqlens_host[0] != 0) return MAXSIM_ERR_SHAPE;
        for (int32_t b = 0; b < B; ++b) {
            const int64_t len = (int64_t)cu_seqlens_host[b + 1] - cu_seqlens_host[b];
            if (len < 0 || len > Ld) return MAXSIM_ERR_SHAPE;
        }
    }
    maxsim::HostStreamArgs a{};
    a.Q = Q;
    a.D_host = D_host;
    a.cu_host = cu_seqlens_host;
    a.cu_dev = cu_seqlens;
    a.d_lens = d_lens;
    a.Nq = Nq;
    a.Lq = Lq;
    a.B = B;
    a.Ld = Ld;
    a.block_docs = block_docs;
    a.elem = dtype == MAXSIM_BF16 ? maxsim::kBF16 : maxsim::kF16;
    a.staging = staging;
    a.scores = scores;
    a.argmax = argmax;
    return hip_status(maxsim::launch_fwd_host_stream(a, static_cast<hipStream_t>(stream)));
}

namespace {
int check_chamfer(int32_t Bt, int32_t N, int32_t M) {
    if (Bt < 0 || N < 0 || M < 0) return MAXSIM_ERR_SHAPE;
    if ((int64_t)Bt * N >= ((int64_t)1 << 31) || (int64_t)Bt * M >= ((int64_t)1 << 31)) return MAXSIM_ERR_SHAPE;
    return MAXSIM_OK;
}
// The backward sorts both directions' selections together: Bt*(N+M) elements
// with int32 offsets.
int check_chamfer_bwd(int32_t Bt, int32_t N, int32_t M) {
    const int st = check_chamfer(Bt, N, M);
    if (st != MAXSIM_OK) return st;
    if ((int64_t)Bt * ((int64_t)N + M) >= ((int64_t)1 << 31)) return MAXSIM_ERR_SHAPE;
    return MAXSIM_OK;
}
}  // namespace

size_t maxsim_chamfer_fwd_workspace_bytes(int32_t Bt, int32_t N, int32_t M) {
    if (check_chamfer(Bt, N, M) != MAXSIM_OK) return 0;
    return maxsim::chamfer_fwd_workspace_bytes(Bt, N, M);
}

int maxsim_chamfer_fwd(const float* P, const float* Q, int32_t Bt, int32_t N, int32_t M, float* dist_p,
                       int32_t* idx_p, float* dist_q, int32_t* idx_q, void* workspace, size_t workspace_bytes,
                       void* stream) {
    int st = check_chamfer(Bt, N, M);
    if (st != MAXSIM_OK) return st;
    if (Bt == 0 || (N == 0 && M == 0)) return MAXSIM_OK;
    if (!workspace || (N > 0 && (!P || !dist_p || !idx_p)) || (M > 0 && (!Q || !dist_q || !idx_q)))
        return MAXSIM_ERR_NULL;
    if (!aligned(P, 4) || !aligned(Q, 4) || !aligned(dist_p, 4) || !aligned(idx_p, 4) || !aligned(dist_q, 4) ||
        !aligned(idx_q, 4) || !aligned(workspace, 256))
        return MAXSIM_ERR_ALIGN;
    if (workspace_bytes < maxsim::chamfer_fwd_workspace_bytes(Bt, N, M)) return MAXSIM_ERR_WORKSPACE;
    maxsim::ChamferArgs a{};
    a.P = P;
    a.Q = Q;
    a.Bt = Bt;
    a.N = N;
    a.M = M;
    a.dist_p = dist_p;
    a.idx_p = idx_p;
    a.dist_q = dist_q;
    a.idx_q = idx_q;
    a.workspace = workspace;
    return hip_status(maxsim::launch_chamfer_fwd(a, static_cast<hipStream_t>(stream)));
}

size_t maxsim_chamfer_bwd_workspace_bytes(int32_t Bt, int32_t N, int32_t M) {
    if (check_chamfer_bwd(Bt, N, M) != MAXSIM_OK) return 0;
    return maxsim::chamfer_bwd_workspace_bytes(Bt, N, M);
}

int maxsim_chamfer_bwd(const float* P, const float* Q, const int32_t* idx_p, const int32_t* idx_q,
                       const float* grad_p, const float* grad_q, int32_t Bt, int32_t N, int32_t M, float* dP,
                       float* dQ, int32_t* row_ptr_p, int32_t* col_idx_p, int32_t* row_ptr_q, int32_t* col_idx_q,
                       void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_chamfer_bwd(Bt, N, M);
    if (st != MAXSIM_OK) return st;
    if (Bt == 0) return MAXSIM_OK;
    if (!workspace || !row_ptr_p || !row_ptr_q) return MAXSIM_ERR_NULL;
    if (N > 0 && (!P || !idx_p || !grad_p || !dP || !col_idx_q)) return MAXSIM_ERR_NULL;
    if (M > 0 && (!Q || !idx_q || !grad_q || !dQ || !col_idx_p)) return MAXSIM_ERR_NULL;
    if (!aligned(P, 4) || !aligned(Q, 4) || !aligned(idx_p, 4) || !aligned(idx_q, 4) || !aligned(grad_p, 4) ||
        !aligned(grad_q, 4) || !aligned(dP, 4) || !aligned(dQ, 4) || !aligned(row_ptr_p, 4) ||
        !aligned(col_idx_p, 4) || !aligned(row_ptr_q, 4) || !aligned(col_idx_q, 4) || !aligned(workspace, 256))
        return MAXSIM_ERR_ALIGN;
    if (workspace_bytes < maxsim::chamfer_bwd_workspace_bytes(Bt, N, M)) return MAXSIM_ERR_WORKSPACE;
    maxsim::ChamferArgs a{};
    a.P = P;
    a.Q = Q;
    a.Bt = Bt;
    a.N = N;
    a.M = M;
    a.idx_p = const_cast<int32_t*>(idx_p);
    a.idx_q = const_cast<int32_t*>(idx_q);
    a.grad_p = grad_p;
    a.grad_q = grad_q;
    a.dP = dP;
    a.dQ = dQ;
    a.row_ptr_p = row_ptr_p;
    a.col_idx_p = col_idx_p;
    a.row_ptr_q = row_ptr_q;
    a.col_idx_q = col_idx_q;
    a.workspace = workspace;
    return hip_status(maxsim::launch_chamfer_bwd(a, static_cast<hipStream_t>(stream)));
}

int maxsim_fwd_pairs(const void* Q, const void* D_packed, const int32_t* cu_seqlens, int32_t dtype,
                     const int32_t* pair_q, const int32_t* pair_b, int32_t P, int32_t Nq, int32_t Lq,
                     int32_t B, int64_t T, int32_t d, float* scores, int32_t* argmax, void* stream) {
    if (P < 0 || Nq < 1 || B < 1 || Lq < 1 || T < 0) return MAXSIM_ERR_SHAPE;
    if (d != kDim || Lq > kMaxLq) return MAXSIM_ERR_UNSUPPORTED;
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_UNSUPPORTED;
    if (P == 0) return MAXSIM_OK;
    if (!Q || !cu_seqlens || !pair_q || !pair_b || !scores || (T > 0 && !D_packed)) return MAXSIM_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(D_packed, 16) || !aligned(cu_seqlens, 4) || !aligned(pair_q, 4) ||
        !aligned(pair_b, 4) || !aligned(scores, 4) || !aligned(argmax, 4))
        return MAXSIM_ERR_ALIGN;
    maxsim::FwdArgs a{};
    a.Q = Q;
    a.D = D_packed;
    a.cu = cu_seqlens;
    a.Nq = Nq;
    a.Lq = Lq;
    a.B = B;
    a.T = T;
    a.scores = scores;
    a.argmax = argmax;
    a.elem = dtype == MAXSIM_BF16 ? maxsim::kBF16 : maxsim::kF16;
    a.varlen = true;
    return hip_status(maxsim::launch_fwd_pairs(a, pair_q, pair_b, P, static_cast<hipStream_t>(stream)));
}

int maxsim_topk(const float* scores, const int32_t* ids, int32_t Nq, int32_t B, int32_t K, int32_t* top_idx,
                float* top_score, void* stream) {
    if (Nq < 0 || B < 1 || K < 1 || K > B) return MAXSIM_ERR_SHAPE;
    if (K > maxsim::kMaxTopK) return MAXSIM_ERR_UNSUPPORTED;
    if (Nq == 0) return MAXSIM_OK;
    if (!scores || !top_idx || !top_score) return MAXSIM_ERR_NULL;
    if (!aligned(scores, 4) || !aligned(ids, 4) || !aligned(top_idx, 4) || !aligned(top_score, 4))
        return MAXSIM_ERR_ALIGN;
    return hip_status(maxsim::launch_topk(scores, ids, Nq, B, K, top_idx, top_score, static_cast<hipStream_t>(stream)));
}

size_t maxsim_two_stage_workspace_bytes(int32_t Nq, int32_t B, int32_t K1) {
    if (Nq < 1 || B < 1 || K1 < 1) return 0;
    const size_t s8 = ((size_t)Nq * B * sizeof(float) + 255) / 256 * 256;
    const size_t pq = ((size_t)Nq * K1 * sizeof(int32_t) + 255) / 256 * 256;
    const size_t s16 = (size_t)Nq * K1 * sizeof(float);
    return s8 + pq + s16;
}

int maxsim_two_stage_topk(const int8_t* Q8, const float* q_scale, const int8_t* D8, const float* d_scale,
                          const void* Q16, const void* D16, const int32_t* cu_seqlens, int32_t dtype16,
                          int32_t Nq, int32_t Lq, int32_t B, int64_t T, int32_t max_Ld, int32_t d,
                          int32_t K1, int32_t K2, int32_t* cand, float* cand_score8, int32_t* top_idx,
                          float* top_score, void* workspace, size_t workspace_bytes, void* stream) {
    if (Nq < 1 || B < 1 || K1 < 1 || K1 > B || K2 < 1 || K2 > K1) return MAXSIM_ERR_SHAPE;
    if ((int64_t)Nq * K1 >= ((int64_t)1 << 31)) return MAXSIM_ERR_SHAPE;
    if (K1 > maxsim::kMaxTopK) return MAXSIM_ERR_UNSUPPORTED;
    if (!workspace || !cand || !cand_score8 || !top_idx || !top_score) return MAXSIM_ERR_NULL;
    if (!aligned(workspace, 256) || !aligned(cand, 4) || !aligned(cand_score8, 4) || !aligned(top_idx, 4) ||
        !aligned(top_score, 4))
        return MAXSIM_ERR_ALIGN;
    if (workspace_bytes < maxsim_two_stage_workspace_bytes(Nq, B, K1)) return MAXSIM_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    float* s8 = reinterpret_cast<float*>(ws);
    int32_t* pq = reinterpret_cast<int32_t*>(ws + ((size_t)Nq * B * sizeof(float) + 255) / 256 * 256);
    float* s16 = reinterpret_cast<float*>(reinterpret_cast<char*>(pq) +
                                          ((size_t)Nq * K1 * sizeof(int32_t) + 255) / 256 * 256);
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    // 1. INT8 scores of every pair
    int st = maxsim_fwd_i8(Q8, q_scale, D8, d_scale, cu_seqlens, Nq, Lq, B, T, max_Ld, d, s8, nullptr, stream);
    if (st != MAXSIM_OK) return st;
    // 2. each query's K1 best documents
    st = maxsim_topk(s8, nullptr, Nq, B, K1, cand, cand_score8, stream);
    if (st != MAXSIM_OK) return st;
    // 3. fp16 / bf16 scores of the candidates
    if (maxsim::launch_fill_pair_q(pq, (int64_t)Nq * K1, K1, hs) != hipSuccess) return MAXSIM_ERR_HIP;
    st = maxsim_fwd_pairs(Q16, D16, cu_seqlens, dtype16, pq, cand, Nq * K1, Nq, Lq, B, T, d, s16, nullptr, stream);
    if (st != MAXSIM_OK) return st;
    // 4. their K2 best, ties by document index
    return maxsim_topk(s16, cand, Nq, K1, K2, top_idx, top_score, stream);
}

const char* maxsim_status_string(int status) {
    switch (status) {
        case MAXSIM_OK: return "MAXSIM_OK";
        case MAXSIM_ERR_NULL: return "MAXSIM_ERR_NULL: a required pointer is NULL";
        case MAXSIM_ERR_SHAPE: return "MAXSIM_ERR_SHAPE: invalid or overflowing size";
        case MAXSIM_ERR_UNSUPPORTED: return "MAXSIM_ERR_UNSUPPORTED: d, Lq, Ld or dtype outside what the kernels support";
        case MAXSIM_ERR_ALIGN: return "MAXSIM_ERR_ALIGN: misaligned pointer";
        case MAXSIM_ERR_WORKSPACE: return "MAXSIM_ERR_WORKSPACE: workspace too small";
        case MAXSIM_ERR_HIP: return "MAXSIM_ERR_HIP: kernel launch failed";
        case MAXSIM_ERR_SCRATCH:
            return "MAXSIM_ERR_SCRATCH: the shape needs more scratch than the allocation-free entry point holds";
        default: return "unknown maxsim status";
    }
}

}  // extern "C"

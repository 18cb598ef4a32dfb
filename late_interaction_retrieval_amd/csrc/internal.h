// internal.h -- host-side interface between the C ABI (capi.cpp) and the
// kernel launchers (fwd.hip, bwd.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace maxsim {

enum ElemType { kF16 = 0, kBF16 = 1, kI8 = 2 };

constexpr int kDim = 128;        // embedding width every kernel is built for
constexpr int kMaxLq = 1024;     // query tokens one workgroup keeps on chip
constexpr int kMaxLdBwd = 4096;  // longest document the backward supports (CSR fill LDS)
// Below this mean number of sources per dD row the atomic scatter is faster
// than building the CSR map (measured on MI355X).
constexpr double kScatterMaxSourcesPerRow = 0.5;

struct FwdArgs {
    const void* Q;            // [Nq, Lq, 128]
    const void* D;            // padded [B, Ld, 128] or packed [T, 128]
    const int32_t* d_lens;    // padded: [B] or nullptr
    const int32_t* cu;        // packed: [B+1]
    const float* q_scale;     // int8: [Nq, Lq]
    const float* d_scale;     // int8: [T]
    int64_t T;                // packed: rows of D
    int32_t Nq, Lq, B, Ld;    // Ld: padded row stride per document
    float* scores;            // [Nq, B]
    int32_t* argmax;          // [Nq, B, Lq] or nullptr
    int elem;                 // ElemType
    bool varlen;
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// scores of the listed (query, document) pairs over a packed corpus (a.varlen)
hipError_t launch_fwd_pairs(const FwdArgs& a, const int32_t* pair_q, const int32_t* pair_b, int32_t P,
                            hipStream_t stream);

constexpr int kMaxTopK = 1024;  // K of one top-K selection (LDS sort)
hipError_t launch_topk(const float* scores, const int32_t* ids, int Nq, int B, int K, int32_t* idx, float* val,
                       hipStream_t stream);
hipError_t launch_fill_pair_q(int32_t* pair_q, int64_t n, int K1, hipStream_t stream);

// Out-of-core forward: the corpus is in host memory (pinned for full speed)
// and is streamed through two device buffers in blocks of block_docs documents.
struct HostStreamArgs {
    const void* Q;               // device [Nq, Lq, 128]
    const void* D_host;          // host: padded [B, Ld, 128] or packed [T, 128]
    const int32_t* cu_host;      // packed: host [B+1] (nullptr: padded)
    const int32_t* cu_dev;       // packed: the same on the device
    const int32_t* d_lens;       // padded: device [B] or nullptr
    int32_t Nq, Lq, B, Ld;       // Ld: padded row stride, or the longest packed document
    int32_t block_docs;
    int elem;
    void* staging;               // host_stream_staging_bytes() bytes of device memory
    float* scores;               // device [Nq, B]
    int32_t* argmax;             // device [Nq, B, Lq] or nullptr
};
size_t host_stream_staging_bytes(int32_t Nq, int32_t Lq, int32_t Ld, int32_t block_docs, bool with_argmax);
hipError_t launch_fwd_host_stream(const HostStreamArgs& a, hipStream_t stream);

// Chamfer distance between batched point clouds P [Bt, N, 3] and Q [Bt, M, 3] (fp32).
struct ChamferArgs {
    const float* P;
    const float* Q;
    int32_t Bt, N, M;
    float* dist_p;       // [Bt, N]  squared distance to the nearest point of Q
    int32_t* idx_p;      // [Bt, N]  its index
    float* dist_q;       // [Bt, M]
    int32_t* idx_q;      // [Bt, M]
    const float* grad_p; // [Bt, N]  backward: upstream gradient of dist_p
    const float* grad_q; // [Bt, M]
    float* dP;           // [Bt, N, 3]
    float* dQ;           // [Bt, M, 3]
    int32_t* row_ptr_p;  // [Bt*N + 1]  the Q points selecting each P point
    int32_t* col_idx_p;  // [Bt*M]
    int32_t* row_ptr_q;  // [Bt*M + 1]  the P points selecting each Q point
    int32_t* col_idx_q;  // [Bt*N]
    void* workspace;
};
size_t chamfer_fwd_workspace_bytes(int32_t Bt, int32_t N, int32_t M);
hipError_t launch_chamfer_fwd(const ChamferArgs& a, hipStream_t stream);
size_t chamfer_bwd_workspace_bytes(int32_t Bt, int32_t N, int32_t M);
hipError_t launch_chamfer_bwd(const ChamferArgs& a, hipStream_t stream);

struct BwdArgs {
    const void* Q;            // [Nq, Lq, 128]
    const void* D;            // [B, Ld, 128]
    const int32_t* argmax;    // [Nq, B, Lq]
    const float* g;           // [Nq, B]
    int32_t Nq, Lq, B, Ld;
    int elem;                 // kF16 / kBF16
    float* dQ;                // [Nq, Lq, 128]
    float* dD;                // [B, Ld, 128]
    int32_t* row_ptr;         // [B*Ld + 1]
    int32_t* col_idx;         // [Nq*B*Lq]
    void* workspace;
    // packed corpus (nullptr: padded): D is [T, 128], dD is [T, 128], row_ptr
    // is [T + 1] and Ld is the longest document
    const int32_t* cu_seqlens = nullptr;  // [B + 1]
    int64_t T = 0;
};

// The allocation-free backward's scratch: a device array of kScratchBytes per
// device (noalloc.hip).  scratch_address gives the current device's copy.
constexpr size_t kScratchBytes = (size_t)64 << 20;
hipError_t scratch_address(void** out);

// Queries per CSR group (one wave each) for a document length; 0 if unsupported.
int bwd_group(int32_t Nq, int32_t Lq, int32_t Ld);
size_t bwd_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq, int32_t Ld);
size_t bwd_varlen_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq, int32_t max_Ld);
size_t bwd_scatter_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
// dD by atomic scatter (no CSR, no workspace), dQ gathered as in launch_bwd
hipError_t launch_bwd_scatter(const BwdArgs& a, hipStream_t stream);

}  // namespace maxsim

// topk.hip -- per-query top-K selection over a row of scores, and the small
// helpers of the two-stage INT8 -> fp16 scan (Flash-MaxSim, Section 4.1
// "Kernel Family": an INT8 pass ranks the corpus, the candidates are scored
// again in fp16 and ranked again).
//
// Order: larger score first; equal scores by ascending id (the document
// index, or the id array the caller passes).  Every (score, id) pair maps to
// a distinct 64-bit key (monotone image of the score in the high word, the
// complement of the id in the low word), so "the K largest keys" is exactly
// that order.  One workgroup per query: an MSB-first radix select over 8-bit
// digits finds the K-th largest key (usually after the four score digits:
// it stops once the remaining count equals the keys left under the prefix),
// the K keys at or above it are compacted into LDS and bitonic-sorted.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace maxsim {
namespace {

constexpr int kTopkThreads = 1024;

// Monotone image of a float: larger value -> larger code.  -0.0 and +0.0 are
// equal scores, so both map to the code of +0.0 (and come back as +0.0).
__device__ __forceinline__ uint32_t ord32(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unord32(uint32_t o) {
    const uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return __uint_as_float(u);
}

__device__ __forceinline__ unsigned long long topk_key(const float* row, const int32_t* ids, int j) {
    const uint32_t id = ids ? (uint32_t)ids[j] : (uint32_t)j;
    return ((unsigned long long)ord32(row[j]) << 32) | (unsigned long long)(0xffffffffu - id);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* scores, const int32_t* ids, int B, int K,
                                                            int32_t* out_idx, float* out_val) {
    __shared__ unsigned hist[256];
    __shared__ unsigned long long sel[kMaxTopK];
    __shared__ unsigned long long s_prefix;
    __shared__ int s_krem, s_done, s_nsel;
    const int q = blockIdx.x;
    const int tid = threadIdx.x;
    const float* row = scores + (int64_t)q * B;
    const int32_t* idr = ids ? ids + (int64_t)q * B : nullptr;
    unsigned long long prefix = 0ull, mask = 0ull;
    int krem = K;
    for (int shift = 56; shift >= 0; shift -= 8) {
        for (int e = tid; e < 256; e += kTopkThreads) hist[e] = 0u;
        __syncthreads();
        for (int j0 = 0; j0 < B; j0 += kTopkThreads) {  // uniform
            const int j = j0 + tid;
            bool in = false;
            unsigned d = 0u;
            if (j < B) {
                const unsigned long long key = topk_key(row, idr, j);
                in = (key & mask) == prefix;
                d = (unsigned)(key >> shift) & 255u;
            }
            // the leading digits of similar scores coincide: when every key of
            // the wave falls in one bin, one atomic adds the wave's count
            const unsigned long long inb = __ballot(in);
            if (inb != 0ull) {
                const int first = __ffsll((long long)inb) - 1;
                const unsigned d0 = (unsigned)__shfl((int)d, first);
                if (__ballot(in && d != d0) == 0ull) {
                    if ((tid & 63) == first) atomicAdd(&hist[d0], (unsigned)__popcll(inb));
                } else if (in) {
                    atomicAdd(&hist[d], 1u);
                }
            }
        }
        __syncthreads();
        if (tid < 64) {
            // the digit holding the krem-th largest key under the prefix, by
            // one wave: lane l sums bins 255-4l .. 252-4l, a scan over the
            // lanes gives the count above each lane's bins, and the lane where
            // the count reaches krem walks its four bins
            unsigned c[4], local = 0u;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                c[k] = hist[255 - 4 * tid - k];
                local += c[k];
            }
            unsigned incl = local;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const unsigned t = (unsigned)__shfl_up((int)incl, off);
                if (tid >= off) incl += t;
            }
            const unsigned above = incl - local;  // keys in bins above this lane's
            if (above < (unsigned)krem && incl >= (unsigned)krem) {  // exactly one lane
                unsigned cum = above;
                int digit = 255 - 4 * tid - 3;
                unsigned hd = c[3];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if (cum + c[k] >= (unsigned)krem) {
                        digit = 255 - 4 * tid - k;
                        hd = c[k];
                        break;
                    }
                    cum += c[k];
                }
                s_krem = krem - (int)cum;
                s_prefix = prefix | ((unsigned long long)digit << shift);
                s_done = hd == (unsigned)(krem - (int)cum);  // every key under the new prefix is taken
            }
        }
        __syncthreads();
        prefix = s_prefix;
        mask |= 255ull << shift;
        krem = s_krem;
        const bool done = s_done != 0;
        __syncthreads();
        if (done) break;
    }
    // exactly K keys are >= prefix (lower digits of prefix are 0)
    if (tid == 0) s_nsel = 0;
    __syncthreads();
    for (int j = tid; j < B; j += kTopkThreads) {
        const unsigned long long key = topk_key(row, idr, j);
        if (key >= prefix) {
            const int pos = atomicAdd(&s_nsel, 1);
            if (pos < kMaxTopK) sel[pos] = key;
        }
    }
    int P2 = 1;
    while (P2 < K) P2 <<= 1;
    __syncthreads();
    for (int e = K + tid; e < P2; e += kTopkThreads) sel[e] = 0ull;  // below every real key
    __syncthreads();
    // bitonic sort, descending
    for (int k = 2; k <= P2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < P2; i += kTopkThreads) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const unsigned long long a = sel[i], b = sel[ixj];
                    const bool desc = (i & k) == 0;
                    if (desc ? (a < b) : (a > b)) {
                        sel[i] = b;
                        sel[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int k = tid; k < K; k += kTopkThreads) {
        const unsigned long long key = sel[k];
        out_val[(int64_t)q * K + k] = unord32((uint32_t)(key >> 32));
        out_idx[(int64_t)q * K + k] = (int32_t)(0xffffffffu - (uint32_t)key);
    }
}

// pair_q[r] = r / K1 (the query of each candidate slot)
__global__ __launch_bounds__(256) void fill_pair_q(int32_t* pair_q, int64_t n, int K1) {
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (r < n) pair_q[r] = (int32_t)(r / K1);
}

}  // namespace

hipError_t launch_topk(const float* scores, const int32_t* ids, int Nq, int B, int K, int32_t* idx, float* val,
                       hipStream_t stream) {
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)Nq), dim3(kTopkThreads), 0, stream, scores, ids, B, K, idx, val);
    return hipGetLastError();
}

hipError_t launch_fill_pair_q(int32_t* pair_q, int64_t n, int K1, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_pair_q, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, pair_q, n, K1);
    return hipGetLastError();
}

}  // namespace maxsim

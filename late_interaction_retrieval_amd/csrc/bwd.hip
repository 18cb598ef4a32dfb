// bwd.hip -- MaxSim backward for gfx950 (MI355X): inverse-grid CSR build,
// destination-owned dD and gathered dQ (Flash-MaxSim Section 4.2, Eqs. (dq),
// (dd), "Runtime Inverse-Grid Construction", "Destination-Owned Reduction",
// Algorithm 3).
//
// Sources are the query tokens s = (q*B + b)*Lq + i; source s selects the
// destination row dst(s) = b*Ld + argmax[s].  The CSR lists, for every row,
// its sources in ascending s (a stable argsort of dst).  Every document's
// sources occupy the fixed range [b*Nq*Lq, (b+1)*Nq*Lq) of col_idx, so each
// document's part of the map is built independently:
//   1. csr_count : per (document, group of G queries) a histogram over the
//                  document's Ld rows (LDS atomics; counts are order-free).
//   2. csr_scan  : per document, prefix over the query groups and over the
//                  rows -> row_ptr and each group's first slot per row.
//   3. csr_fill  : per (document, query group), one wave per query.  Within a
//                  query the sources are ranked in ascending i, 64 at a time:
//                  every lane ORs its bit into a per-row 64-bit mask in LDS,
//                  reads the mask back and takes popcount(mask & lanes below)
//                  as its rank.  OR is commutative, so the result is
//                  deterministic, and the per-query prefix over the group
//                  makes the whole fill stable.
//   4. dd_owner  : one 16-lane group owns one dD row, walks its sources and
//                  writes the row once (no atomics).
//   5. dq_gather : one 16-lane group owns one dQ row and loops over the B
//                  documents (Algorithm 3 step 3).
// argmax entries outside [0, Ld) break the forward's contract; they are
// clamped into range so that no access leaves the buffers.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace maxsim {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct BwdParams {
    const char* Q;
    const char* D;
    const int32_t* A;
    const float* g;
    int Nq, Lq, B, Ld;
    int G, NG;  // queries per group (waves per workgroup), number of groups
    float* dQ;
    float* dD;
    int32_t* row_ptr;
    int32_t* col_idx;
    int32_t* ws;  // [B][NG][Ld]
    // floor(n / (B*Lq)) for 0 <= n < 2^31 as (n * magic) >> (32 + shift)
    unsigned long long magic;
    int shift;
};

__device__ __forceinline__ int clamp_tok(int t, int Ld) { return t < 0 ? 0 : (t >= Ld ? Ld - 1 : t); }

__global__ __launch_bounds__(1024) void csr_count(BwdParams p) {
    extern __shared__ int hist[];  // [Ld]
    const int qg = blockIdx.x % p.NG;
    const int b = blockIdx.x / p.NG;
    const int nt = blockDim.x;
    for (int t = threadIdx.x; t < p.Ld; t += nt) hist[t] = 0;
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = qg * p.G + wave;
    if (q < p.Nq) {
        const int32_t* a = p.A + ((int64_t)q * p.B + b) * p.Lq;
        for (int i = lane; i < p.Lq; i += 64) atomicAdd(&hist[clamp_tok(a[i], p.Ld)], 1);
    }
    __syncthreads();
    int32_t* out = p.ws + ((int64_t)b * p.NG + qg) * p.Ld;
    for (int t = threadIdx.x; t < p.Ld; t += nt) out[t] = hist[t];
}

// One workgroup of 1024 threads per document.
__global__ __launch_bounds__(1024) void csr_scan(BwdParams p) {
    __shared__ int wsum[16];
    __shared__ int carry_s;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t doc_base = (int64_t)b * p.Nq * p.Lq;
    int32_t* ws = p.ws + (int64_t)b * p.NG * p.Ld;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int t0 = 0; t0 < p.Ld; t0 += 1024) {
        const int t = t0 + tid;
        int tot = 0;
        if (t < p.Ld) {
            for (int qg = 0; qg < p.NG; ++qg) {
                const int c = ws[(int64_t)qg * p.Ld + t];
                ws[(int64_t)qg * p.Ld + t] = tot;
                tot += c;
            }
        }
        // inclusive scan of tot over the 1024 threads
        int x = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        int wpre = 0;
        for (int w = 0; w < wave; ++w) wpre += wsum[w];
        const int carry = carry_s;
        const int excl = carry + wpre + x - tot;
        if (t < p.Ld) {
            const int rp = (int)(doc_base + excl);
            p.row_ptr[(int64_t)b * p.Ld + t] = rp;
            for (int qg = 0; qg < p.NG; ++qg) ws[(int64_t)qg * p.Ld + t] += rp;
        }
        __syncthreads();
        if (tid == 1023) carry_s = carry + wpre + x;
        __syncthreads();
    }
    if (b == p.B - 1 && tid == 0) p.row_ptr[(int64_t)p.B * p.Ld] = (int)((int64_t)p.B * p.Nq * p.Lq);
}

// One wave per query of the group.  Dynamic LDS: G*Ld int (next slot per
// (query, row)) followed by G*Ld*2 uint (64-bit lane masks per (query, row)).
__global__ __launch_bounds__(1024) void csr_fill(BwdParams p) {
    extern __shared__ int lds[];
    const int qg = blockIdx.x % p.NG;
    const int b = blockIdx.x / p.NG;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int Ld = p.Ld;
    int* slot = lds;                                            // [G][Ld]
    unsigned* mask = reinterpret_cast<unsigned*>(lds + p.G * Ld);  // [G][Ld][2]
    for (int e = tid; e < p.G * Ld; e += nt) {
        slot[e] = 0;
        mask[2 * e] = 0u;
        mask[2 * e + 1] = 0u;
    }
    __syncthreads();
    const int q = qg * p.G + wave;
    const int32_t* a = p.A + ((int64_t)q * p.B + b) * p.Lq;
    if (q < p.Nq) {
        for (int i = lane; i < p.Lq; i += 64) atomicAdd(&slot[wave * Ld + clamp_tok(a[i], Ld)], 1);
    }
    __syncthreads();
    // per row: exclusive prefix over the group's queries + the group's first slot
    const int32_t* first = p.ws + ((int64_t)b * p.NG + qg) * Ld;
    for (int t = tid; t < Ld; t += nt) {
        int run = first[t];
        for (int w = 0; w < p.G; ++w) {
            const int c = slot[w * Ld + t];
            slot[w * Ld + t] = run;
            run += c;
        }
    }
    __syncthreads();
    if (q < p.Nq) {
        int* myslot = slot + wave * Ld;
        unsigned* mymask = mask + 2 * wave * Ld;
        const unsigned long long below = (1ull << lane) - 1ull;
        const int64_t s0 = ((int64_t)q * p.B + b) * p.Lq;
        for (int i0 = 0; i0 < p.Lq; i0 += 64) {
            const int i = i0 + lane;
            const bool active = i < p.Lq;
            const int t = active ? clamp_tok(a[i], Ld) : 0;
            if (active) atomicOr(&mymask[2 * t + (lane >> 5)], 1u << (lane & 31));
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the ORs have landed
            __builtin_amdgcn_wave_barrier();
            unsigned long long mk = 0;
            int base = 0;
            if (active) {
                mk = (unsigned long long)mymask[2 * t] | ((unsigned long long)mymask[2 * t + 1] << 32);
                base = myslot[t];
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            if (active) {
                const int rank = __popcll(mk & below);
                p.col_idx[base + rank] = (int)(s0 + i);
                if (rank == 0) {  // the lowest lane of the row advances it and clears the mask
                    myslot[t] = base + __popcll(mk);
                    mymask[2 * t] = 0u;
                    mymask[2 * t + 1] = 0u;
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

template <int ELEM>
__device__ __forceinline__ void load8(const char* row, float* v) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(row);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const unsigned w = raw[h];
        if constexpr (ELEM == kBF16) {
            v[2 * h] = __uint_as_float(w << 16);
            v[2 * h + 1] = __uint_as_float(w & 0xffff0000u);
        } else {
            v[2 * h] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
            v[2 * h + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
        }
    }
}

// 16 lanes per dD row, 16 rows per 256-thread workgroup.
template <int ELEM>
__global__ __launch_bounds__(256) void dd_owner(BwdParams p) {
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int l16 = threadIdx.x & 15;
    const int64_t nrows = (int64_t)p.B * p.Ld;
    if (row >= nrows) return;
    const int b = (int)(row / p.Ld);
    const int kb = p.row_ptr[row], ke = p.row_ptr[row + 1];
    const int BLq = p.B * p.Lq;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int k = kb; k < ke; ++k) {
        const int s = p.col_idx[k];
        int q = (int)(((unsigned long long)(unsigned)s * p.magic) >> (32 + p.shift));
        int i = s - q * BLq - b * p.Lq;
        q = q < 0 ? 0 : (q >= p.Nq ? p.Nq - 1 : q);  // a consistent map never clamps
        i = i < 0 ? 0 : (i >= p.Lq ? p.Lq - 1 : i);
        const float gq = p.g[(int64_t)q * p.B + b];
        float v[8];
        load8<ELEM>(p.Q + ((int64_t)q * p.Lq + i) * 256 + l16 * 16, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(gq, v[e], acc[e]);
    }
    f32x4* out = reinterpret_cast<f32x4*>(p.dD + row * 128 + l16 * 8);
    out[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    out[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// 16 lanes per dQ row, 16 rows per 256-thread workgroup.
template <int ELEM>
__global__ __launch_bounds__(256) void dq_gather(BwdParams p) {
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // q*Lq + i
    const int l16 = threadIdx.x & 15;
    if (row >= (int64_t)p.Nq * p.Lq) return;
    const int q = (int)(row / p.Lq);
    const int i = (int)(row - (int64_t)q * p.Lq);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const int32_t* a = p.A + (int64_t)q * p.B * p.Lq + i;
    const float* gq = p.g + (int64_t)q * p.B;
    int b = 0;
    for (; b + 4 <= p.B; b += 4) {
        float v[4][8];
        float gg[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = clamp_tok(a[(int64_t)(b + u) * p.Lq], p.Ld);
            gg[u] = gq[b + u];
            load8<ELEM>(p.D + ((int64_t)(b + u) * p.Ld + t) * 256 + l16 * 16, v[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(gg[u], v[u][e], acc[e]);
    }
    for (; b < p.B; ++b) {
        const int t = clamp_tok(a[(int64_t)b * p.Lq], p.Ld);
        float v[8];
        load8<ELEM>(p.D + ((int64_t)b * p.Ld + t) * 256 + l16 * 16, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(gq[b], v[e], acc[e]);
    }
    f32x4* out = reinterpret_cast<f32x4*>(p.dQ + row * 128 + l16 * 8);
    out[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    out[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

template <int ELEM>
hipError_t launch_bwd_elem(const BwdParams& p, hipStream_t stream) {
    const int nthr = 64 * p.G;
    const unsigned groups = (unsigned)((int64_t)p.B * p.NG);
    hipLaunchKernelGGL(csr_count, dim3(groups), dim3(nthr), p.Ld * sizeof(int), stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(csr_scan, dim3(p.B), dim3(1024), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(csr_fill, dim3(groups), dim3(nthr), (size_t)p.G * p.Ld * 12, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t drows = (int64_t)p.B * p.Ld;
    hipLaunchKernelGGL((dd_owner<ELEM>), dim3((unsigned)((drows + 15) / 16)), dim3(256), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t qrows = (int64_t)p.Nq * p.Lq;
    hipLaunchKernelGGL((dq_gather<ELEM>), dim3((unsigned)((qrows + 15) / 16)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

int bwd_group(int32_t Ld) {
    if (Ld < 1 || Ld > kMaxLdBwd) return 0;
    int G = 16;
    while (G > 1 && (int64_t)G * Ld > kMaxLdBwd) G >>= 1;
    return G;
}

size_t bwd_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq, int32_t Ld) {
    (void)Lq;
    const int G = bwd_group(Ld);
    if (G == 0 || Nq < 1 || B < 1) return 0;
    const int64_t NG = (Nq + G - 1) / G;
    return (size_t)(B * NG * Ld * (int64_t)sizeof(int32_t));
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
    BwdParams p;
    p.Q = static_cast<const char*>(a.Q);
    p.D = static_cast<const char*>(a.D);
    p.A = a.argmax;
    p.g = a.g;
    p.Nq = a.Nq;
    p.Lq = a.Lq;
    p.B = a.B;
    p.Ld = a.Ld;
    p.G = bwd_group(a.Ld);
    p.NG = (a.Nq + p.G - 1) / p.G;
    p.dQ = a.dQ;
    p.dD = a.dD;
    p.row_ptr = a.row_ptr;
    p.col_idx = a.col_idx;
    p.ws = static_cast<int32_t*>(a.workspace);
    // magic division by B*Lq: shift = ceil(log2 d), magic = ceil(2^(32+shift) / d)
    const unsigned long long d = (unsigned long long)a.B * a.Lq;
    int shift = 0;
    while ((1ull << shift) < d) ++shift;
    const unsigned __int128 num = (unsigned __int128)1 << (32 + shift);
    p.magic = (unsigned long long)((num + d - 1) / d);
    p.shift = shift;
    return a.elem == kBF16 ? launch_bwd_elem<kBF16>(p, stream) : launch_bwd_elem<kF16>(p, stream);
}

}  // namespace maxsim

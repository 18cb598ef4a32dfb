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
//                  one ballot per bit of the row index gives every lane the
//                  mask of lanes holding its row, and popcount(mask & lanes
//                  below) is its rank.  The per-query prefix over the group
//                  makes the whole fill stable and deterministic.
//   4. dd_owner  : a 16-lane group owns dD rows, walks their sources and
//                  writes each row once (no atomics).
//   5. dq_gather : a 16-lane group owns dQ rows and loops over the B
//                  documents (Algorithm 3 step 3).
// argmax entries outside [0, Ld) break the forward's contract; they are
// clamped into range so that no access leaves the buffers.
#include <hip/hip_runtime.h>

#include <algorithm>

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
    // floor(n / Lq) likewise
    unsigned long long magic_lq;
    int shift_lq;
    // packed corpus: cu_seqlens [B+1] (nullptr: padded documents of Ld rows),
    // T rows, and each document's first CSR slot [B+1] (workspace)
    const int32_t* cu;
    int64_t T;
    int32_t* docbase;
    // dQ over document chunks: with dq_split > 1 chunk c (blockIdx.y) sums
    // documents [c*dq_docs, (c+1)*dq_docs) into dq_part[c] ([Nq*Lq, 128]),
    // and dq_reduce adds the chunks in ascending order
    int dq_split, dq_docs;
    float* dq_part;
    // dD rows with more than kHeavy sources: dd_owner appends them to this
    // list (count first) and dd_heavy reduces each with a whole workgroup
    int32_t* heavy;
    int64_t max_heavy;
};

__device__ __forceinline__ int clamp_tok(int t, int Ld) { return t < 0 ? 0 : (t >= Ld ? Ld - 1 : t); }

// First row and number of rows of document b.  Packed documents longer than
// Ld (the stated maximum) are cut to Ld so every LDS index stays in range.
__device__ __forceinline__ void doc_rows(const BwdParams& p, int b, int64_t& start, int& len) {
    if (p.cu) {
        int64_t s0 = p.cu[b], s1 = p.cu[b + 1];
        s0 = s0 < 0 ? 0 : (s0 > p.T ? p.T : s0);
        s1 = s1 < s0 ? s0 : (s1 > p.T ? p.T : s1);
        start = s0;
        len = (int)(s1 - s0 < p.Ld ? s1 - s0 : p.Ld);
    } else {
        start = (int64_t)b * p.Ld;
        len = p.Ld;
    }
}

// First col_idx slot of document b: its sources follow those of the earlier
// non-empty documents.
__device__ __forceinline__ int doc_base(const BwdParams& p, int b) {
    return p.docbase ? p.docbase[b] : b * p.Nq * p.Lq;
}

// Packed corpus: docbase[b] = Nq*Lq * (number of non-empty documents before b),
// b = 0 .. B.  One workgroup of 1024 threads scans the documents in order.
__global__ __launch_bounds__(1024) void csr_docbase(BwdParams p) {
    __shared__ int wsum[16];
    __shared__ int carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    const int per = p.Nq * p.Lq;
    for (int b0 = 0; b0 <= p.B; b0 += 1024) {
        const int b = b0 + tid;
        int flag = 0;
        if (b < p.B) {
            int64_t st;
            int len;
            doc_rows(p, b, st, len);
            flag = len > 0;
        }
        int x = flag;
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
        if (b <= p.B) p.docbase[b] = (carry + wpre + x - flag) * per;
        __syncthreads();
        if (tid == 1023) carry_s = carry + wpre + x;
        __syncthreads();
    }
}

// Workgroup k of the count and fill grids runs on XCD k % 8; all of document
// b's query groups go to XCD b % 8 (the XCD csr_scan's workgroup b runs on),
// so its counts and its part of col_idx are written through one L2, where the
// short scattered writes of the fill combine into whole lines.  The grid has
// 8 * ceil(B / 8) * NG workgroups; those past the last document do nothing.
__device__ __forceinline__ bool doc_group(const BwdParams& p, int& b, int& qg) {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int d = j / p.NG;
    qg = j - d * p.NG;
    b = d * 8 + x;
    return b < p.B;
}

__global__ __launch_bounds__(1024) void csr_count(BwdParams p) {
    extern __shared__ int hist[];  // [Ld]
    int b, qg;
    if (!doc_group(p, b, qg)) return;  // uniform
    const int nt = blockDim.x;
    for (int t = threadIdx.x; t < p.Ld; t += nt) hist[t] = 0;
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = qg * p.G + wave;
    int64_t st;
    int len;
    doc_rows(p, b, st, len);
    if (q < p.Nq && len > 0) {  // an empty document has no rows and no sources
        const int32_t* a = p.A + ((int64_t)q * p.B + b) * p.Lq;
        for (int i = lane; i < p.Lq; i += 64) atomicAdd(&hist[clamp_tok(a[i], len)], 1);
    }
    __syncthreads();
    int32_t* out = p.ws + ((int64_t)b * p.NG + qg) * p.Ld;
    for (int t = threadIdx.x; t < p.Ld; t += nt) out[t] = hist[t];
}

// One workgroup of 1024 threads per document.  The per-group counts of a row
// are read 16 at a time (independent loads), summed, and after the scan over
// the rows read again to write each group's first slot.
__global__ __launch_bounds__(1024) void csr_scan(BwdParams p) {
    __shared__ int wsum[16];
    __shared__ int carry_s;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int base = doc_base(p, b);
    int64_t rstart;
    int len;
    doc_rows(p, b, rstart, len);
    int32_t* ws = p.ws + (int64_t)b * p.NG * p.Ld;
    if (b == 0 && tid == 0) p.heavy[0] = 0;  // dd_owner appends heavy rows after this kernel
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int t0 = 0; t0 < len; t0 += 1024) {
        const int t = t0 + tid;
        int tot = 0;
        if (t < len) {
            for (int g0 = 0; g0 < p.NG; g0 += 16) {
                int c[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) c[j] = g0 + j < p.NG ? ws[(int64_t)(g0 + j) * p.Ld + t] : 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) tot += c[j];
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
        if (t < len) {
            int run = base + excl;
            p.row_ptr[rstart + t] = run;
            for (int g0 = 0; g0 < p.NG; g0 += 16) {
                int c[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) c[j] = g0 + j < p.NG ? ws[(int64_t)(g0 + j) * p.Ld + t] : 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (g0 + j < p.NG) ws[(int64_t)(g0 + j) * p.Ld + t] = run;
                    run += c[j];
                }
            }
        }
        __syncthreads();
        if (tid == 1023) carry_s = carry + wpre + x;
        __syncthreads();
    }
    if (b == p.B - 1 && tid == 0) {  // one past the last row: the number of sources that select a row
        const int64_t nrows = p.cu ? p.T : (int64_t)p.B * p.Ld;
        p.row_ptr[nrows] = p.docbase ? p.docbase[p.B] : p.B * p.Nq * p.Lq;
    }
}

// One wave per query of the group.  Dynamic LDS: G*Ld int (next slot per
// (query, row)).
// A wave reads its query's Lq argmax entries once, into registers (at most
// kMaxLq / 64 per lane), and uses them for both the count and the fill.
constexpr int kFillIt = kMaxLq / 64;

__global__ __launch_bounds__(1024) void csr_fill(BwdParams p) {
    extern __shared__ int lds[];
    int b, qg;
    if (!doc_group(p, b, qg)) return;  // uniform
    const int tid = threadIdx.x, nt = blockDim.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int Ld = p.Ld;
    int* slot = lds;  // [G][Ld]
    const int q = qg * p.G + wave;
    int64_t rstart;
    int len;
    doc_rows(p, b, rstart, len);
    if (len == 0) return;  // uniform: an empty document has no sources
    const int32_t* a = p.A + ((int64_t)q * p.B + b) * p.Lq;
    int tk[kFillIt];  // -1: no source in this lane for step k
#pragma unroll
    for (int k = 0; k < kFillIt; ++k) {
        const int i = k * 64 + lane;
        tk[k] = (q < p.Nq && i < p.Lq) ? clamp_tok(a[i], len) : -1;
    }
    for (int e = tid; e < p.G * Ld; e += nt) slot[e] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kFillIt; ++k)
        if (tk[k] >= 0) atomicAdd(&slot[wave * Ld + tk[k]], 1);
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
        const unsigned long long below = (1ull << lane) - 1ull;
        const int64_t s0 = ((int64_t)q * p.B + b) * p.Lq;
        const int nbits = Ld > 1 ? 32 - __clz(Ld - 1) : 0;  // bits of a row index
#pragma unroll
        for (int k = 0; k < kFillIt; ++k) {
            if (k * 64 >= p.Lq) break;  // uniform
            const int t = tk[k];
            const bool active = t >= 0;
            // the lanes of this step holding the same row: one ballot per bit
            unsigned long long mk = __ballot(active);
            for (int bit = 0; bit < nbits; ++bit) {  // uniform
                const bool one = (t >> bit) & 1;
                const unsigned long long v = __ballot(one);
                mk &= one ? v : ~v;
            }
            if (active) {
                // the wave's LDS operations run in order: every lane of the row
                // reads the slot before its lowest lane advances it
                const int base = myslot[t];
                const int rank = __popcll(mk & below);
                p.col_idx[base + rank] = (int)(s0 + k * 64 + lane);
                if (rank == 0) myslot[t] = base + __popcll(mk);
            }
        }
    }
}

template <int ELEM>
__device__ __forceinline__ void cvt8(const u32x4 raw, float* v) {
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

// The two gradient kernels are gather-bound: every dD row pulls ~Nq*Lq/Ld
// query rows and every dQ row pulls one document row per document.  Both are
// persistent (kGatherBlocks workgroups, all resident) and every 16-lane
// group owns up to kRowsPerGroup output rows, which it advances together
// through the reduction index -- documents b for dQ, query windows for dD --
// in the same order as every other group.  The workgroups of one XCD so
// work on the same few documents (or queries) at a time and the rows they
// gather stay in that XCD's L2.  Each row still sums its terms one by one in
// ascending source order, so runs are bit-identical.
constexpr int kGatherThreads = 512;
constexpr int kGatherGroups = kGatherThreads / 16;  // 16-lane groups per workgroup
constexpr int kGatherBlocks = 512;                  // 2 per CU on 256 CUs
constexpr int kRowsPerGroup = 4;
constexpr int kQueryWindow = 16;  // queries per dD step
constexpr int kDdBatch = 12;      // dD sources gathered per round (loads in flight)
// A dD row with more sources than this is left to dd_heavy: one 16-lane group
// walking thousands of sources would hold up the whole grid.
constexpr int kHeavy = 512;

__device__ __forceinline__ void fma8(float* acc, float g, const float* v) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(g, v[e], acc[e]);
}

__device__ __forceinline__ void store8(float* dst, const float* acc) {
    f32x4* out = reinterpret_cast<f32x4*>(dst);
    out[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    out[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// rows of group gid: gid + k * ngroups, k < rows_per_group (consecutive
// groups hold consecutive rows, so index loads of a wave share cache lines).
// Per query window the index loads of all the group's rows are issued
// together, then each row's gathers.
//
// Packed corpus (VARLEN): the rows are the T packed rows and a source's
// document comes from the source itself (s / Lq = q*B + b).  Rows that no
// document covers hold no meaningful row_ptr entry under a malformed
// cu_seqlens; their ranges are clamped into col_idx so that no access leaves
// the buffers.
template <int ELEM, bool VARLEN>
__global__ __launch_bounds__(kGatherThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void dd_owner(BwdParams p, int rows_per_group) {
    const int l16 = threadIdx.x & 15;
    const int64_t ngroups = (int64_t)gridDim.x * kGatherGroups;
    const int64_t gid = (int64_t)blockIdx.x * kGatherGroups + (threadIdx.x >> 4);
    const int64_t nrows = VARLEN ? p.T : (int64_t)p.B * p.Ld;
    const int BLq = p.B * p.Lq;
    const int nsrc = p.Nq * BLq;  // col_idx capacity
    const int gshift = threadIdx.x & 48;  // this group's first lane in the wave
    // Packed corpus: a row's source count is about Nq*Lq over its document's
    // length, so rows of short documents carry several times the sources of
    // long ones, and rows dealt out by index left the groups holding short
    // documents' rows running about twice as long as the mean.  There each
    // group takes the contiguous rows whose first source lies in its share
    // gid*S/G .. (gid+1)*S/G of the S sources (a 16-lane search over row_ptr,
    // which is non-decreasing), and walks them kRowsPerGroup at a time.
    // Every row still belongs to exactly one group and sums its sources in the
    // same order, so the result is unchanged.
    int64_t rb = 0, rend = 1;
    if constexpr (VARLEN) {
        int64_t S = p.row_ptr[nrows];
        S = S < 0 ? 0 : (S > nsrc ? nsrc : S);
        auto lower_bound16 = [&](int64_t x) -> int64_t {  // first row with row_ptr[row] >= x, in [0, nrows]
            int64_t lo = 0, hi = nrows;
            while (lo < hi) {  // uniform per 16-lane group
                const int64_t step = (hi - lo) / 16 + 1;  // (hi - lo) / step < 16
                const int64_t i = lo + (int64_t)l16 * step;
                const bool below = i <= hi && p.row_ptr[i] < x;
                const int c = __popcll((__ballot(below) >> gshift) & 0xffffull);
                if (c == 0) {
                    hi = lo;
                } else {
                    const int64_t up = lo + (int64_t)c * step;
                    hi = up < hi ? up : hi;
                    lo = lo + (int64_t)(c - 1) * step + 1;
                    lo = lo < hi ? lo : hi;
                }
            }
            return lo;
        };
        rb = gid == 0 ? 0 : lower_bound16(gid * S / ngroups);
        rend = gid + 1 >= ngroups ? nrows : lower_bound16((gid + 1) * S / ngroups);
        rend = rend < rb ? rb : rend;
    }
    for (; rb < rend; rb += VARLEN ? kRowsPerGroup : 1) {  // uniform per 16-lane group
    // rows of this pass: packed, rb + k (< rend); padded, gid + k * ngroups
    auto row_of = [&](int k) -> int64_t { return VARLEN ? rb + k : gid + k * ngroups; };
    auto row_ok = [&](int k, int64_t row) { return VARLEN ? row < rend : (k < rows_per_group && row < nrows); };
    int cur[kRowsPerGroup], end[kRowsPerGroup], bdoc[kRowsPerGroup];
    bool heavy[kRowsPerGroup];
    float acc[kRowsPerGroup][8];
#pragma unroll
    for (int k = 0; k < kRowsPerGroup; ++k) {
        const int64_t row = row_of(k);
        const bool ok = row_ok(k, row);
        cur[k] = ok ? p.row_ptr[row] : 0;
        end[k] = ok ? p.row_ptr[row + 1] : 0;
        if constexpr (VARLEN) {
            cur[k] = cur[k] < 0 ? 0 : (cur[k] > nsrc ? nsrc : cur[k]);
            end[k] = end[k] < cur[k] ? cur[k] : (end[k] > nsrc ? nsrc : end[k]);
            bdoc[k] = 0;
        } else {
            bdoc[k] = ok ? (int)(row / p.Ld) : 0;
        }
        heavy[k] = end[k] - cur[k] > kHeavy;  // uniform per group
        if (heavy[k]) {
            if (l16 == 0) {
                const int slot = atomicAdd(&p.heavy[0], 1);
                if (slot < p.max_heavy) p.heavy[1 + slot] = (int)row;  // bounded by the workspace
            }
            cur[k] = end[k];  // this group skips the row
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
    }
    for (int q0 = 0; q0 < p.Nq; q0 += kQueryWindow) {
        const int qend = q0 + kQueryWindow;
        bool more = true;
        while (more) {  // uniform per 16-lane group; a second round only when a row has > kDdBatch sources here
            int src[kRowsPerGroup];
#pragma unroll
            for (int k = 0; k < kRowsPerGroup; ++k) {
                const int navail = min(kDdBatch, end[k] - cur[k]);
                src[k] = l16 < navail ? p.col_idx[cur[k] + l16] : -1;
            }
            more = false;
#pragma unroll
            for (int k = 0; k < kRowsPerGroup; ++k) {
                int qi = 0;
                float gv = 0.f;
                bool in = false;
                if (src[k] >= 0) {
                    int q = (int)(((unsigned long long)(unsigned)src[k] * p.magic) >> (32 + p.shift));
                    int b = bdoc[k];
                    if constexpr (VARLEN) {
                        const int qb = (int)(((unsigned long long)(unsigned)src[k] * p.magic_lq) >> (32 + p.shift_lq));
                        b = qb - q * p.B;
                        b = b < 0 ? 0 : (b >= p.B ? p.B - 1 : b);
                    }
                    int i = src[k] - q * BLq - b * p.Lq;
                    q = q < 0 ? 0 : (q >= p.Nq ? p.Nq - 1 : q);  // a consistent map never clamps
                    i = i < 0 ? 0 : (i >= p.Lq ? p.Lq - 1 : i);
                    in = q < qend;
                    gv = p.g[(int64_t)q * p.B + b];
                    qi = q * p.Lq + i;
                }
                // sources are in ascending q: the ones in this window are a prefix
                const int n = __popcll((__ballot(in) >> gshift) & 0xffffull);
                if (n == 0) continue;
                u32x4 raw[kDdBatch];
#pragma unroll
                for (int j = 0; j < kDdBatch; ++j) {
                    const int qj = __shfl(qi, j, 16);
                    if (j < n) raw[j] = *reinterpret_cast<const u32x4*>(p.Q + (int64_t)qj * 256 + l16 * 16);
                }
#pragma unroll
                for (int j = 0; j < kDdBatch; ++j) {
                    const float gj = __shfl(gv, j, 16);
                    if (j < n) {
                        float v[8];
                        cvt8<ELEM>(raw[j], v);
                        fma8(acc[k], gj, v);
                    }
                }
                cur[k] += n;
                if (n == kDdBatch) more = true;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kRowsPerGroup; ++k) {
        const int64_t row = row_of(k);
        if (row_ok(k, row) && !heavy[k]) store8(p.dD + row * 128 + l16 * 8, acc[k]);
    }
    }
}

// The heavy rows, one workgroup at a time each: the row's sources are cut
// into kGatherGroups contiguous chunks, every 16-lane group sums its chunk in
// ascending order (16 loads in flight), and the chunk sums are added in
// group order.  The split is fixed by the row's length, so runs are
// bit-identical.  The source's document comes from the source (s / Lq).
template <int ELEM>
__global__ __launch_bounds__(kGatherThreads) void dd_heavy(BwdParams p) {
    __shared__ float part[kGatherGroups][128];
    const int l16 = threadIdx.x & 15, grp = threadIdx.x >> 4;
    const int BLq = p.B * p.Lq;
    const int nsrc = p.Nq * BLq;
    const int count = (int)(p.heavy[0] < p.max_heavy ? p.heavy[0] : p.max_heavy);
    for (int h = blockIdx.x; h < count; h += gridDim.x) {  // uniform
        const int64_t row = p.heavy[1 + h];
        int beg = p.row_ptr[row], end = p.row_ptr[row + 1];
        beg = beg < 0 ? 0 : (beg > nsrc ? nsrc : beg);
        end = end < beg ? beg : (end > nsrc ? nsrc : end);
        const int len = end - beg;
        const int c0 = beg + (int)((int64_t)len * grp / kGatherGroups);
        const int c1 = beg + (int)((int64_t)len * (grp + 1) / kGatherGroups);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        for (int e0 = c0; e0 < c1; e0 += 16) {  // uniform per group
            const int n = min(16, c1 - e0);
            int qi = 0;
            float gv = 0.f;
            if (l16 < n) {
                const int src = p.col_idx[e0 + l16];
                int q = (int)(((unsigned long long)(unsigned)src * p.magic) >> (32 + p.shift));
                const int qb = (int)(((unsigned long long)(unsigned)src * p.magic_lq) >> (32 + p.shift_lq));
                int b = qb - q * p.B;
                b = b < 0 ? 0 : (b >= p.B ? p.B - 1 : b);
                int i = src - q * BLq - b * p.Lq;
                q = q < 0 ? 0 : (q >= p.Nq ? p.Nq - 1 : q);  // a consistent map never clamps
                i = i < 0 ? 0 : (i >= p.Lq ? p.Lq - 1 : i);
                gv = p.g[(int64_t)q * p.B + b];
                qi = q * p.Lq + i;
            }
            u32x4 raw[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int qj = __shfl(qi, j, 16);
                if (j < n) raw[j] = *reinterpret_cast<const u32x4*>(p.Q + (int64_t)qj * 256 + l16 * 16);
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float gj = __shfl(gv, j, 16);
                if (j < n) {
                    float v[8];
                    cvt8<ELEM>(raw[j], v);
                    fma8(acc, gj, v);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) part[grp][l16 * 8 + e] = acc[e];
        __syncthreads();
        if (threadIdx.x < 128) {
            float t = part[0][threadIdx.x];
            for (int gr = 1; gr < kGatherGroups; ++gr) t += part[gr][threadIdx.x];
            p.dD[row * 128 + threadIdx.x] = t;
        }
        __syncthreads();  // part is reused by the next heavy row
    }
}

// Per step of DSTEP documents the gathers of all the group's RPG rows are in
// flight together (RPG * DSTEP = 8 loads: 4 rows x 2 documents, or 1 row x 8
// documents when there are few rows).  Packed corpus (VARLEN): lane j of a
// group holds document b0 + j's first row and length; an empty document gives
// weight 0 and reads a valid row.  Each row sums its terms in ascending b.
template <int ELEM, bool VARLEN, int RPG, int DSTEP>
__global__ __launch_bounds__(kGatherThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void dq_gather(BwdParams p, int rows_per_group) {
    const int l16 = threadIdx.x & 15;
    const int64_t ngroups = (int64_t)gridDim.x * kGatherGroups;
    const int64_t gid = (int64_t)blockIdx.x * kGatherGroups + (threadIdx.x >> 4);
    const int64_t nrows = (int64_t)p.Nq * p.Lq;
    int aoff[RPG], goff[RPG];  // Nq*B*Lq < 2^31 (checked by the host)
    bool ok[RPG];
    float acc[RPG][8];
#pragma unroll
    for (int k = 0; k < RPG; ++k) {
        const int64_t row = gid + k * ngroups;  // q*Lq + i
        ok[k] = k < rows_per_group && row < nrows;
        const int q = ok[k] ? (int)(row / p.Lq) : 0;
        const int i = ok[k] ? (int)(row - (int64_t)q * p.Lq) : 0;
        aoff[k] = q * p.B * p.Lq + i;
        goff[k] = q * p.B;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
    }
    // Straight-line steps: every load is issued unconditionally from a valid
    // address (a missing row or document reads row 0 / the last document) and
    // its term gets weight 0, so no branch separates a load from the next.
    const int b_lo = blockIdx.y * p.dq_docs;
    const int b_hi = (VARLEN && p.T == 0) ? 0 : min(p.B, b_lo + p.dq_docs);  // no rows at all: dQ = 0
    for (int b0 = b_lo; b0 < b_hi; b0 += DSTEP) {
        const int nb = min(DSTEP, b_hi - b0);
        const bool lane_doc = l16 < nb;
        const int bl = b0 + (lane_doc ? l16 : 0);
        int64_t dstart = 0;
        int dlen = p.Ld;
        if constexpr (VARLEN) doc_rows(p, bl, dstart, dlen);
        int araw[RPG];
        float gv[RPG];
#pragma unroll
        for (int k = 0; k < RPG; ++k) {
            araw[k] = p.A[aoff[k] + (int64_t)bl * p.Lq];
            gv[k] = p.g[goff[k] + bl];
        }
        int tok[RPG];
#pragma unroll
        for (int k = 0; k < RPG; ++k) {
            if constexpr (VARLEN) {
                // packed row index (T < 2^31, checked by the host); an empty
                // document, or one starting at T, reads row T-1 with weight 0
                const int r = (int)dstart + clamp_tok(araw[k], dlen > 0 ? dlen : 1);
                tok[k] = r < (int)p.T ? r : (int)p.T - 1;
                gv[k] = (ok[k] && lane_doc && dlen > 0) ? gv[k] : 0.f;
            } else {
                tok[k] = clamp_tok(araw[k], p.Ld);
                gv[k] = (ok[k] && lane_doc) ? gv[k] : 0.f;
            }
        }
        u32x4 raw[RPG][DSTEP];
#pragma unroll
        for (int k = 0; k < RPG; ++k) {
#pragma unroll
            for (int j = 0; j < DSTEP; ++j) {
                const int tj = __shfl(tok[k], j, 16);
                if constexpr (VARLEN) {
                    raw[k][j] = *reinterpret_cast<const u32x4*>(p.D + (int64_t)tj * 256 + l16 * 16);
                } else {
                    // document base is wave-uniform; the row offset fits 32 bits (Ld <= 4096)
                    const char* Db = p.D + (int64_t)min(b0 + j, p.B - 1) * p.Ld * 256;
                    raw[k][j] = *reinterpret_cast<const u32x4*>(Db + (unsigned)(tj * 256 + l16 * 16));
                }
            }
        }
#pragma unroll
        for (int k = 0; k < RPG; ++k) {
#pragma unroll
            for (int j = 0; j < DSTEP; ++j) {
                const float gj = __shfl(gv[k], j, 16);
                float v[8];
                cvt8<ELEM>(raw[k][j], v);
                fma8(acc[k], gj, v);
            }
        }
    }
    float* out = p.dq_split > 1 ? p.dq_part + (int64_t)blockIdx.y * nrows * 128 : p.dQ;
#pragma unroll
    for (int k = 0; k < RPG; ++k) {
        const int64_t row = gid + k * ngroups;
        if (ok[k]) store8(out + row * 128 + l16 * 8, acc[k]);
    }
}

// dQ = sum of the chunks' partial sums in a fixed order: 16 slices of
// consecutive chunks are summed in ascending order by 16 threads each (one
// per float4 of 16 consecutive ones), then the slices in ascending order.
__global__ __launch_bounds__(256) void dq_reduce(BwdParams p) {
    __shared__ f32x4 slice_sum[16][16];  // [slice][element]
    const int64_t n4 = (int64_t)p.Nq * p.Lq * 32;
    const int el = threadIdx.x & 15, sl = threadIdx.x >> 4;
    const int64_t k = (int64_t)blockIdx.x * 16 + el;
    const int per = (p.dq_split + 15) / 16;
    const int c0 = sl * per, c1 = min(p.dq_split, c0 + per);
    const f32x4* part = reinterpret_cast<const f32x4*>(p.dq_part);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (k < n4) {
#pragma unroll 8
        for (int c = c0; c < c1; ++c) {
            const f32x4 v = part[(int64_t)c * n4 + k];
            acc = f32x4{acc[0] + v[0], acc[1] + v[1], acc[2] + v[2], acc[3] + v[3]};
        }
    }
    slice_sum[sl][el] = acc;
    __syncthreads();
    if (sl == 0 && k < n4) {
        f32x4 t = slice_sum[0][el];
        for (int j = 1; j < 16; ++j) {
            const f32x4 v = slice_sum[j][el];
            t = f32x4{t[0] + v[0], t[1] + v[1], t[2] + v[2], t[3] + v[3]};
        }
        reinterpret_cast<f32x4*>(p.dQ)[k] = t;
    }
}

// Atomic-scatter dD, the low-contention alternative to the CSR path: dD is
// cleared, then every source adds g[q,b] * Q[q,i] into its destination row
// with fp32 atomic adds at the device's L2.  A 16-lane group takes one source
// at a time; lane l owns columns e*16 + l (e < 8), so each atomic instruction
// of the group covers 64 contiguous bytes of the row.  The order of the adds
// into one row is not fixed, so results may differ between runs in the last
// bits; rows no source selects are exactly 0.
__global__ __launch_bounds__(256) void zero_rows(float* dst, int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n4; k += stride)
        reinterpret_cast<f32x4*>(dst)[k] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int ELEM, bool VARLEN>
__global__ __launch_bounds__(256) void dd_scatter(BwdParams p) {
    const int l16 = threadIdx.x & 15;
    const int ngroups = gridDim.x * 16;
    const int nsrc = p.Nq * p.B * p.Lq;  // < 2^31 (checked by the host)
    for (int s = blockIdx.x * 16 + (threadIdx.x >> 4); s < nsrc; s += ngroups) {
        const int qb = s / p.Lq;  // q*B + b
        const int i = s - qb * p.Lq;
        const int q = qb / p.B;
        const int b = qb - q * p.B;
        int64_t start;
        int len;
        if constexpr (VARLEN) {
            doc_rows(p, b, start, len);
            if (len == 0) continue;  // uniform per group: an empty document takes no gradient
        } else {
            start = (int64_t)b * p.Ld;
            len = p.Ld;
        }
        const int64_t row = start + clamp_tok(p.A[s], len);
        const float gv = p.g[qb];
        const unsigned short* qrow = reinterpret_cast<const unsigned short*>(p.Q) + ((int64_t)q * p.Lq + i) * 128;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const unsigned short h = qrow[e * 16 + l16];
            if constexpr (ELEM == kBF16)
                v[e] = __uint_as_float((unsigned)h << 16);
            else
                v[e] = (float)__builtin_bit_cast(_Float16, h);
        }
        float* drow = p.dD + row * 128;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            __hip_atomic_fetch_add(drow + e * 16 + l16, gv * v[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// grid and rows per group for a persistent gather over nrows rows
void gather_grid(int64_t nrows, unsigned* blocks, int* rows_per_group) {
    const int64_t full = (int64_t)kGatherBlocks * kGatherGroups;
    int r = (int)((nrows + full - 1) / full);
    if (r < 1) r = 1;
    if (r > kRowsPerGroup) r = kRowsPerGroup;
    const int64_t groups = (nrows + r - 1) / r;
    *blocks = (unsigned)((groups + kGatherGroups - 1) / kGatherGroups);
    *rows_per_group = r;
}

// Documents per dQ chunk: enough chunks that the gather fills the chip
// (kGatherBlocks workgroups) when there are few dQ rows, at least one step of
// documents each (8 with one row per group, else 2).
int dq_split_of(int64_t nrows, int B) {
    unsigned blocks;
    int rpg;
    gather_grid(nrows, &blocks, &rpg);
    int64_t s = ((int64_t)kGatherBlocks + blocks - 1) / blocks;
    const int64_t smax = B / (rpg == 1 ? 8 : 2);
    if (s > smax) s = smax;
    return s < 1 ? 1 : (int)s;
}

size_t dq_part_bytes(int32_t Nq, int32_t Lq, int32_t B) {
    const int64_t nrows = (int64_t)Nq * Lq;
    const int S = dq_split_of(nrows, B);
    return S > 1 ? (size_t)S * nrows * 128 * sizeof(float) : 0;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

template <int ELEM, bool VARLEN>
hipError_t launch_dq(BwdParams p, hipStream_t stream) {
    const int64_t nrows = (int64_t)p.Nq * p.Lq;
    unsigned blocks;
    int rpg;
    gather_grid(nrows, &blocks, &rpg);
    p.dq_split = dq_split_of(nrows, p.B);
    p.dq_docs = (p.B + p.dq_split - 1) / p.dq_split;
    if (rpg == 1)
        hipLaunchKernelGGL((dq_gather<ELEM, VARLEN, 1, 8>), dim3(blocks, p.dq_split), dim3(kGatherThreads), 0, stream,
                           p, rpg);
    else
        hipLaunchKernelGGL((dq_gather<ELEM, VARLEN, kRowsPerGroup, 2>), dim3(blocks, p.dq_split), dim3(kGatherThreads),
                           0, stream, p, rpg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.dq_split == 1) return e;
    hipLaunchKernelGGL(dq_reduce, dim3((unsigned)((nrows * 32 + 15) / 16)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int ELEM, bool VARLEN>
hipError_t launch_bwd_elem(const BwdParams& p, hipStream_t stream) {
    const int nthr = 64 * p.G;
    const unsigned groups = (unsigned)(8 * (((int64_t)p.B + 7) / 8) * p.NG);
    hipError_t e;
    if (VARLEN) {
        hipLaunchKernelGGL(csr_docbase, dim3(1), dim3(1024), 0, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(csr_count, dim3(groups), dim3(nthr), p.Ld * sizeof(int), stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(csr_scan, dim3(p.B), dim3(1024), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(csr_fill, dim3(groups), dim3(nthr), (size_t)p.G * p.Ld * 4, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    unsigned blocks;
    int rpg;
    const int64_t nrows = VARLEN ? p.T : (int64_t)p.B * p.Ld;
    if (nrows > 0) {
        gather_grid(nrows, &blocks, &rpg);
        // packed: the groups split the sources evenly, so the full grid serves any row count
        if (VARLEN) blocks = kGatherBlocks;
        hipLaunchKernelGGL((dd_owner<ELEM, VARLEN>), dim3(blocks), dim3(kGatherThreads), 0, stream, p, rpg);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const unsigned hb = (unsigned)std::min<int64_t>(p.max_heavy, kGatherBlocks);
        if (hb > 0) {
            hipLaunchKernelGGL((dd_heavy<ELEM>), dim3(hb), dim3(kGatherThreads), 0, stream, p);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    return launch_dq<ELEM, VARLEN>(p, stream);
}

template <int ELEM, bool VARLEN>
hipError_t launch_scatter_elem(const BwdParams& p, hipStream_t stream) {
    hipError_t e;
    const int64_t nrows = VARLEN ? p.T : (int64_t)p.B * p.Ld;
    if (nrows > 0) {
        const int64_t n4 = nrows * 32;
        const unsigned zb = (unsigned)std::min<int64_t>((n4 + 255) / 256, 4096);
        hipLaunchKernelGGL(zero_rows, dim3(zb), dim3(256), 0, stream, p.dD, n4);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int64_t nsrc = (int64_t)p.Nq * p.B * p.Lq;
        const unsigned sb = (unsigned)std::min<int64_t>((nsrc + 15) / 16, 8192);
        hipLaunchKernelGGL((dd_scatter<ELEM, VARLEN>), dim3(sb), dim3(256), 0, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    unsigned blocks;
    int rpg;
    return launch_dq<ELEM, VARLEN>(p, stream);
}

// ceil-rounded magic multiplier for floor(n / d), 0 <= n < 2^31:
// shift = ceil(log2 d), magic = ceil(2^(32+shift) / d)
void magic_div(unsigned long long d, unsigned long long* magic, int* shift) {
    int s = 0;
    while ((1ull << s) < d) ++s;
    const unsigned __int128 num = (unsigned __int128)1 << (32 + s);
    *magic = (unsigned long long)((num + d - 1) / d);
    *shift = s;
}

}  // namespace

int bwd_group(int32_t Ld) {
    if (Ld < 1 || Ld > kMaxLdBwd) return 0;
    int G = 16;
    while (G > 1 && (int64_t)G * Ld > kMaxLdBwd) G >>= 1;
    return G;
}

// Workspace layout (each part at a 256-byte boundary): the CSR counts
// [B][NG][Ld] int32, the packed corpus' document bases [B+1] int32, the heavy
// row list (count, then rows) int32, then the dQ chunk partial sums
// [S][Nq*Lq][128] fp32 when dQ is split (S > 1).
namespace {
size_t counts_bytes(int32_t Nq, int32_t B, int32_t Ld) {
    const int G = bwd_group(Ld);
    if (G == 0 || Nq < 1 || B < 1) return 0;
    const int64_t NG = (Nq + G - 1) / G;
    return (size_t)(B * NG * Ld * (int64_t)sizeof(int32_t));
}
// a heavy row has more than kHeavy of the Nq*B*Lq sources
int64_t max_heavy_rows(int32_t Nq, int32_t B, int32_t Lq) { return (int64_t)Nq * B * Lq / (kHeavy + 1); }
size_t heavy_bytes(int32_t Nq, int32_t B, int32_t Lq) {
    return align256((size_t)(1 + max_heavy_rows(Nq, B, Lq)) * sizeof(int32_t));
}
}  // namespace

size_t bwd_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq, int32_t Ld) {
    const size_t c = counts_bytes(Nq, B, Ld);
    if (c == 0 || Lq < 1) return 0;
    return align256(c) + heavy_bytes(Nq, B, Lq) + dq_part_bytes(Nq, Lq, B);
}

size_t bwd_varlen_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq, int32_t max_Ld) {
    const size_t c = counts_bytes(Nq, B, max_Ld);
    if (c == 0 || Lq < 1) return 0;
    return align256(c) + align256((size_t)(B + 1) * sizeof(int32_t)) + heavy_bytes(Nq, B, Lq) +
           dq_part_bytes(Nq, Lq, B);
}

size_t bwd_scatter_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq) {
    if (Nq < 1 || B < 1 || Lq < 1) return 0;
    return std::max<size_t>(256, dq_part_bytes(Nq, Lq, B));
}

hipError_t launch_bwd_scatter(const BwdArgs& a, hipStream_t stream) {
    BwdParams p = {};
    p.Q = static_cast<const char*>(a.Q);
    p.D = static_cast<const char*>(a.D);
    p.A = a.argmax;
    p.g = a.g;
    p.Nq = a.Nq;
    p.Lq = a.Lq;
    p.B = a.B;
    p.Ld = a.Ld;
    p.dQ = a.dQ;
    p.dD = a.dD;
    p.cu = a.cu_seqlens;
    p.T = a.T;
    p.dq_part = static_cast<float*>(a.workspace);
    if (a.cu_seqlens)
        return a.elem == kBF16 ? launch_scatter_elem<kBF16, true>(p, stream) : launch_scatter_elem<kF16, true>(p, stream);
    return a.elem == kBF16 ? launch_scatter_elem<kBF16, false>(p, stream) : launch_scatter_elem<kF16, false>(p, stream);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
    BwdParams p = {};
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
    char* ws = static_cast<char*>(a.workspace);
    p.ws = reinterpret_cast<int32_t*>(ws);
    size_t off = align256(counts_bytes(a.Nq, a.B, a.Ld));
    magic_div((unsigned long long)a.B * a.Lq, &p.magic, &p.shift);
    magic_div((unsigned long long)a.Lq, &p.magic_lq, &p.shift_lq);
    p.max_heavy = max_heavy_rows(a.Nq, a.B, a.Lq);
    if (a.cu_seqlens) {
        p.cu = a.cu_seqlens;
        p.T = a.T;
        p.docbase = reinterpret_cast<int32_t*>(ws + off);
        off += align256((size_t)(a.B + 1) * sizeof(int32_t));
        p.heavy = reinterpret_cast<int32_t*>(ws + off);
        off += heavy_bytes(a.Nq, a.B, a.Lq);
        p.dq_part = reinterpret_cast<float*>(ws + off);
        return a.elem == kBF16 ? launch_bwd_elem<kBF16, true>(p, stream) : launch_bwd_elem<kF16, true>(p, stream);
    }
    p.heavy = reinterpret_cast<int32_t*>(ws + off);
    off += heavy_bytes(a.Nq, a.B, a.Lq);
    p.dq_part = reinterpret_cast<float*>(ws + off);
    return a.elem == kBF16 ? launch_bwd_elem<kBF16, false>(p, stream) : launch_bwd_elem<kF16, false>(p, stream);
}

}  // namespace maxsim

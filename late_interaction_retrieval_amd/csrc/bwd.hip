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
//                  document's rows (LDS atomics; counts are order-free) and
//                  the group's number of sources.
//   2. csr_fill  : per (document, query group), one wave per query: the
//                  document's first slot and row starts from the counts
//                  (row_ptr), then the group's sources ranked by (row, query,
//                  i) in LDS -- within a query 64 at a time in ascending i,
//                  a lane's rank is the number of lower lanes holding its row
//                  -- and written out run by run.  Stable and deterministic.
//   3. dd_owner  : a 16-lane group owns dD rows, walks their sources and
//                  writes each row once (no atomics).
//   4. dq_gather : a 16-lane group owns dQ rows and loops over the B
//                  documents (Algorithm 3 step 3); extra workgroups of the
//                  same launch reduce the dD rows with very many sources
//                  that dd_owner left to them.
// A negative argmax entry (the forward's value for a document with no valid
// token) selects no row.  Entries at or past a document's length break the
// forward's contract; they are clamped into range so that no access leaves
// the buffers.
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
    int32_t* ws;    // [B][NG][Ld] per (document, query group) row counts
    int32_t* gtot;  // [B*NG] per (document, query group) number of sources that select a row
    // floor(n / (B*Lq)) for 0 <= n < 2^31 as (n * magic) >> (32 + shift)
    unsigned long long magic;
    int shift;
    // floor(n / Lq) likewise
    unsigned long long magic_lq;
    int shift_lq;
    // packed corpus: cu_seqlens [B+1] (nullptr: padded documents of Ld rows)
    // and T rows; each document's first CSR slot [B+1] (workspace; nullptr:
    // the fill sums the groups' totals itself)
    const int32_t* cu;
    int64_t T;
    int32_t* docbase;
    // dQ over document chunks: with dq_split > 1 chunk c (blockIdx.y) sums
    // documents [c*dq_docs, (c+1)*dq_docs) into dq_part[c] ([Nq*Lq, 128]),
    // and dq_reduce adds the chunks in ascending order
    int dq_split, dq_docs;
    float* dq_part;
    // dD rows with more than kHeavy sources: dd_owner appends them to this
    // list (count first) and extra workgroups of the dQ launch reduce each
    // with a whole workgroup (heavy_rows)
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

// The row that source s = (q*B + b)*Lq + i selects in document b (of len
// rows), or -1 for none: a negative argmax (what the forward writes for a
// document with no valid token) and every source of a document without rows
// select nothing.  Entries at or past len break the forward's contract and
// are clamped to the last row so that no access leaves the buffers.
__device__ __forceinline__ int src_row(int a, int len) { return (a < 0 || len == 0) ? -1 : (a >= len ? len - 1 : a); }

// Workgroup k of the count and fill grids runs on XCD k % 8; all of document
// b's query groups go to XCD b % 8, so its argmax entries and counts stay in
// one L2 between the two kernels.  The grid has 8 * ceil(B / 8) * NG
// workgroups; those past the last document do nothing.
__device__ __forceinline__ bool doc_group(const BwdParams& p, int& b, int& qg) {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int d = j / p.NG;
    qg = j - d * p.NG;
    b = d * 8 + x;
    return b < p.B;
}

// Sum of v over the workgroup (every thread gets it); red holds one int per wave.
__device__ __forceinline__ int block_sum(int v, int* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    __syncthreads();  // red may still be read by a previous call
    if (lane == 0) red[wave] = v;
    __syncthreads();
    int t = 0;
    for (int w = 0; w < nw; ++w) t += red[w];
    return t;
}

// Exclusive prefix over the workgroup's threads of two values at once, and
// their totals; red holds two ints per wave.
__device__ __forceinline__ void block_exscan2(int x, int y, int* red, int& ex, int& ey, int& tx, int& ty) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int ix = x, iy = y;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int ux = __shfl_up(ix, off), uy = __shfl_up(iy, off);
        if (lane >= off) {
            ix += ux;
            iy += uy;
        }
    }
    __syncthreads();  // red may still be read by a previous call
    if (lane == 63) {
        red[2 * wave] = ix;
        red[2 * wave + 1] = iy;
    }
    __syncthreads();
    int px = 0, py = 0;
    tx = 0;
    ty = 0;
    for (int w = 0; w < nw; ++w) {
        const int a = red[2 * w], c = red[2 * w + 1];
        if (w < wave) {
            px += a;
            py += c;
        }
        tx += a;
        ty += c;
    }
    ex = px + ix - x;
    ey = py + iy - y;
}

// 1. csr_count: per (document, group of G queries), one wave per query, the
// number of the group's sources selecting each of the document's rows (LDS
// histogram; counts do not depend on the order of the increments) and the
// group's number of sources that select a row.  Workgroup 0 also clears the
// heavy-row list that dd_owner appends to after the fill.
__global__ __launch_bounds__(1024) void csr_count(BwdParams p) {
    extern __shared__ int hist[];  // [Ld]
    __shared__ int total;          // the group's sources that select a row
    if (blockIdx.x == 0 && threadIdx.x == 0) p.heavy[0] = 0;
    int b, qg;
    if (!doc_group(p, b, qg)) return;  // uniform
    const int nt = blockDim.x;
    for (int t = threadIdx.x; t < p.Ld; t += nt) hist[t] = 0;
    if (threadIdx.x == 0) total = 0;
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = qg * p.G + wave;
    int64_t st;
    int len;
    doc_rows(p, b, st, len);
    int n = 0;
    if (q < p.Nq) {
        const int32_t* a = p.A + ((int64_t)q * p.B + b) * p.Lq;
        if (p.Lq >= 256 && (p.Lq & 3) == 0 && (reinterpret_cast<uintptr_t>(a) & 15) == 0) {  // uniform
            // long queries: 16-byte loads, up to four per lane in flight before
            // the atomics (one 4-byte load per lane between atomics left the
            // loads serial; training shape 2.5 % faster).  Short ones keep a
            // lane per entry: with a quarter of the lanes busy they measured 4 %
            // slower.
            const int n4 = p.Lq >> 2;
            const int4* a4 = reinterpret_cast<const int4*>(a);
            for (int i0 = 0; i0 < n4; i0 += 256) {  // uniform
                int4 v[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int i = i0 + k * 64 + lane;
                    v[k] = i < n4 ? a4[i] : make_int4(-1, -1, -1, -1);  // -1 selects no row
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int e[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int t = src_row(e[c], len);
                        if (t >= 0) {
                            atomicAdd(&hist[t], 1);
                            ++n;
                        }
                    }
                }
            }
        } else {
            for (int i = lane; i < p.Lq; i += 64) {
                const int t = src_row(a[i], len);
                if (t >= 0) {
                    atomicAdd(&hist[t], 1);
                    ++n;
                }
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off);
    if (lane == 0 && n > 0) atomicAdd(&total, n);
    __syncthreads();
    int32_t* out = p.ws + ((int64_t)b * p.NG + qg) * p.Ld;
    for (int t = threadIdx.x; t < p.Ld; t += nt) out[t] = hist[t];
    if (threadIdx.x == 0) p.gtot[(int64_t)b * p.NG + qg] = total;
}

// With many documents the fill takes each document's first col_idx slot from
// docbase[b] (b = 0 .. B), the exclusive prefix of the documents' source
// counts, formed here by one workgroup of 1024 threads in order; with few,
// every fill workgroup sums the earlier groups' totals itself.
constexpr int kInlineDocTotals = 2048;  // B * NG up to which the fill sums gtot itself

__global__ __launch_bounds__(1024) void csr_docscan(BwdParams p) {
    __shared__ int red[32];
    int carry = 0;
    for (int b0 = 0; b0 <= p.B; b0 += 1024) {
        const int b = b0 + threadIdx.x;
        int n = 0;
        if (b < p.B)
            for (int g = 0; g < p.NG; ++g) n += p.gtot[(int64_t)b * p.NG + g];
        int ex, dummy, tot, dtot;
        block_exscan2(n, 0, red, ex, dummy, tot, dtot);
        if (b <= p.B) p.docbase[b] = carry + ex;
        carry += tot;
    }
}

// 2. csr_fill: per (document, query group), one wave per query.
//   a. The document's first slot (sum of the earlier documents' sources), its
//      row totals (the sum of the groups' counts) and their prefix give every
//      row's first slot: row_ptr, written by the group-0 workgroup.  This
//      group's run of row t starts after the earlier groups' sources of t.
//   b. Within the group the sources are ranked by (row, query, i): per query
//      and row an LDS count, prefix over rows and then queries, and inside a
//      query, 64 sources at a time in ascending i, the rank among the lanes
//      holding the same row (found by an LDS tag per row; only lanes that
//      share a row with another lane of the step take a ballot of that row
//      and count the lower lanes in it).  That is the stable order.
//   c. The sources are placed in LDS in that order and written out by
//      consecutive threads: each row's run of the group is contiguous in
//      col_idx, so a wave's stores cover a few runs instead of 64 scattered
//      words.
// LDS, sized to the shape at launch (fill_lds_bytes): G*Ld int (per query and
// row: counts, then slots), Ld int (per row: global slot minus local slot),
// G*Lq int (the placed sources, packed as row << 14 | query << 10 | i), G*Ld
// bytes (per query and row: a lane tag).  Sized to the largest shapes instead,
// the arrays held one workgroup per CU, and short queries over many short
// documents (4000 workgroups of 512 sources) ran 2.6x slower.
constexpr int kFillIt = kMaxLq / 64;
constexpr int kFillSlots = 16384;  // G * Ld of a query group (bwd_group keeps it within this)
constexpr int kFillPre = 8;        // query groups per document whose counts the fill loads up front

size_t fill_lds_bytes(int G, int Ld, int Lq) {
    return ((size_t)G * Ld + Ld + (size_t)G * Lq) * sizeof(int) + (((size_t)G * Ld + 3) & ~(size_t)3);
}

// KIT: 64-source steps per query (Lq <= 64 * KIT); short queries take fewer
// registers, so more workgroups share a CU.
template <int G, int KIT>
__global__ __launch_bounds__(64 * G) void csr_fill(BwdParams p) {
    extern __shared__ int lds[];
    __shared__ int red[32];
    const int Ld = p.Ld, NG = p.NG;
    int* slot = lds;                                                           // [G][Ld]
    int* delta = slot + G * Ld;                                                // [Ld]
    int* stage = delta + Ld;                                                   // [G*Lq]
    unsigned char* tag = reinterpret_cast<unsigned char*>(stage + G * p.Lq);  // [G][Ld]
    int b, qg;
    if (!doc_group(p, b, qg)) return;  // uniform
    const int tid = threadIdx.x, nt = blockDim.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int q = qg * G + wave;
    int64_t rstart;
    int len;
    doc_rows(p, b, rstart, len);
    const int32_t* a = p.A + ((int64_t)q * p.B + b) * p.Lq;
    int tk[KIT];  // the row each of this lane's sources selects, or -1
#pragma unroll
    for (int k = 0; k < KIT; ++k) {
        const int i = k * 64 + lane;
        tk[k] = (q < p.Nq && i < p.Lq) ? src_row(a[i], len) : -1;
    }
    // The first row chunk's per-group counts (every group of a document up to
    // kFillPre) are loaded now, with the argmax, rather than after the
    // histogram's barrier: with short queries a workgroup holds a few hundred
    // sources and that second round trip was a large part of its time.
    // (Short queries only: long ones have work enough to hide it, and the
    // registers would cost them a workgroup per CU.)
    constexpr int NPRE = KIT <= 4 ? kFillPre : 1;
    const int32_t* cnt = p.ws + (int64_t)b * NG * Ld;
    const bool pre = KIT <= 4 && NG <= NPRE;  // uniform
    int cpre[NPRE];
#pragma unroll
    for (int g = 0; g < NPRE; ++g) cpre[g] = (pre && g < NG && tid < Ld) ? cnt[(int64_t)g * Ld + tid] : 0;
    // the document's first slot
    int dbase;
    if (p.docbase) {
        dbase = p.docbase[b];
    } else {
        int sum = 0;
        for (int k = tid; k < b * NG; k += nt) sum += p.gtot[k];
        dbase = block_sum(sum, red);
    }
    for (int e = tid; e < G * Ld; e += nt) slot[e] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KIT; ++k)
        if (tk[k] >= 0) atomicAdd(&slot[wave * Ld + tk[k]], 1);
    __syncthreads();
    // per row t: local slots of the group's queries, and the global run start
    int carry_lo = 0, carry_row = 0;
    for (int t0 = 0; t0 < Ld; t0 += nt) {  // uniform
        const int t = t0 + tid;
        int gc = 0, rowtot = 0, before = 0;
        if (t < Ld) {
            for (int w = 0; w < G; ++w) gc += slot[w * Ld + t];
            if (pre && t0 == 0) {
#pragma unroll
                for (int g = 0; g < NPRE; ++g) {
                    rowtot += cpre[g];
                    before += g < qg ? cpre[g] : 0;
                }
            } else {
                for (int g = 0; g < NG; ++g) {
                    const int c = cnt[(int64_t)g * Ld + t];
                    rowtot += c;
                    before += g < qg ? c : 0;
                }
            }
        }
        int ex_lo, ex_row, tot_lo, tot_row;
        block_exscan2(gc, rowtot, red, ex_lo, ex_row, tot_lo, tot_row);
        if (t < Ld) {
            int run = carry_lo + ex_lo;
            const int row_first = dbase + carry_row + ex_row;
            delta[t] = row_first + before - run;
            for (int w = 0; w < G; ++w) {
                const int c = slot[w * Ld + t];
                slot[w * Ld + t] = run;
                run += c;
            }
            if (qg == 0 && t < len) p.row_ptr[rstart + t] = row_first;
        }
        carry_lo += tot_lo;
        carry_row += tot_row;
    }
    if (qg == 0 && b == p.B - 1 && tid == 0) {  // one past the last row: the number of sources that select a row
        const int64_t nrows = p.cu ? p.T : (int64_t)p.B * p.Ld;
        p.row_ptr[nrows] = dbase + carry_row;
    }
    __syncthreads();
    if (q < p.Nq) {
        int* myslot = slot + wave * Ld;
        unsigned char* mytag = tag + wave * Ld;
        const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
        for (int k = 0; k < KIT; ++k) {
            if (k * 64 >= p.Lq) break;  // uniform
            const int t = tk[k];
            const bool active = t >= 0;
            // Lanes of this step sharing a row: every active lane writes its id
            // under its row and reads it back (the wave's LDS operations run in
            // order); a lane that reads another id shares its row.  Only for
            // those rows (about 2 of 64 lanes with random rows) the exact rank
            // comes from one ballot of the row; a lane alone in its row has
            // rank 0 and count 1.
            if (active) mytag[t] = (unsigned char)lane;
            // other lanes' writes: the tag must be read back from LDS, not forwarded
            asm volatile("" ::: "memory");
            const bool shared = active && mytag[t] != (unsigned char)lane;
            unsigned long long todo = __ballot(shared);
            int rank = 0, cnt = 1;
            while (todo) {  // uniform
                const int j = __builtin_ctzll(todo);
                const int tj = __builtin_amdgcn_readlane(t, j);
                const bool same = active && t == tj;
                const unsigned long long m = __ballot(same);
                if (same) {
                    rank = __popcll(m & below);
                    cnt = __popcll(m);
                }
                todo &= ~m;
            }
            if (active) {
                // every lane of the row reads the slot before its lowest lane advances it
                const int base = myslot[t];
                stage[base + rank] = (t << 14) | (wave << 10) | (k * 64 + lane);
                if (rank == 0) myslot[t] = base + cnt;
            }
        }
    }
    __syncthreads();
    // the group's carry_lo placed sources, in order; entry e of row t goes to e + delta[t]
    const int64_t s_q0 = ((int64_t)qg * G * p.B + b) * p.Lq;  // source id of (query qg*G, document b, i = 0)
    const int64_t s_qstep = (int64_t)p.B * p.Lq;
    for (int e = tid; e < carry_lo; e += nt) {
        const int v = stage[e];
        const int t = v >> 14;
        p.col_idx[e + delta[t]] = (int)(s_q0 + ((v >> 10) & 15) * s_qstep + (v & 1023));
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
// A dD row with more sources than this is left to heavy_rows: one 16-lane group
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
// Run by the workgroups of the dQ launch past its gather grid (heavy worker
// h0 of hstride), which follows dd_owner on the stream, so the list is
// complete; a separate launch cost about 4.5 us even with no heavy row.
template <int ELEM>
__device__ __forceinline__ void heavy_rows(const BwdParams& p, int h0, int hstride, float (*part)[128]) {
    const int l16 = threadIdx.x & 15, grp = threadIdx.x >> 4;
    const int BLq = p.B * p.Lq;
    const int nsrc = p.Nq * BLq;
    const int count = (int)(p.heavy[0] < p.max_heavy ? p.heavy[0] : p.max_heavy);
    for (int h = h0; h < count; h += hstride) {  // uniform
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
// group holds document b0 + j's first row and length; an empty document, or
// a negative argmax, gives weight 0 and reads a valid row.  Each row sums its
// terms in ascending b.
//
// Workgroups past the gather grid (blockIdx.x >= gather_blocks, every chunk
// row y) reduce the heavy dD rows instead (heavy_rows).
template <int ELEM, bool VARLEN, int RPG, int DSTEP>
__global__ __launch_bounds__(kGatherThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void dq_gather(BwdParams p, int rows_per_group, int gather_blocks) {
    if ((int)blockIdx.x >= gather_blocks) {  // uniform over the workgroup
        __shared__ float part[kGatherGroups][128];
        const int hx = (int)gridDim.x - gather_blocks;  // heavy columns, each gridDim.y workgroups
        heavy_rows<ELEM>(p, ((int)blockIdx.x - gather_blocks) * (int)gridDim.y + (int)blockIdx.y, hx * (int)gridDim.y, part);
        return;
    }
    const int l16 = threadIdx.x & 15;
    const int64_t ngroups = (int64_t)gather_blocks * kGatherGroups;
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
                gv[k] = (ok[k] && lane_doc && dlen > 0 && araw[k] >= 0) ? gv[k] : 0.f;
            } else {
                // a negative argmax (an empty document) selects nothing: weight 0
                tok[k] = clamp_tok(araw[k], p.Ld);
                gv[k] = (ok[k] && lane_doc && araw[k] >= 0) ? gv[k] : 0.f;
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
        const int a = p.A[s];
        if (a < 0) continue;  // uniform per group: selects no row
        const int64_t row = start + clamp_tok(a, len);
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

// heavy_blocks: extra workgroups that reduce the heavy dD rows dd_owner listed
// (0 when there is no list).
template <int ELEM, bool VARLEN>
hipError_t launch_dq(BwdParams p, unsigned heavy_blocks, hipStream_t stream) {
    const int64_t nrows = (int64_t)p.Nq * p.Lq;
    unsigned blocks;
    int rpg;
    gather_grid(nrows, &blocks, &rpg);
    p.dq_split = dq_split_of(nrows, p.B);
    p.dq_docs = (p.B + p.dq_split - 1) / p.dq_split;
    // about heavy_blocks heavy workers in all, spread over the chunk rows
    const unsigned hx = (heavy_blocks + p.dq_split - 1) / p.dq_split;
    const dim3 grid(blocks + hx, p.dq_split);
    if (rpg == 1)
        hipLaunchKernelGGL((dq_gather<ELEM, VARLEN, 1, 8>), grid, dim3(kGatherThreads), 0, stream, p, rpg, (int)blocks);
    else
        hipLaunchKernelGGL((dq_gather<ELEM, VARLEN, kRowsPerGroup, 2>), grid, dim3(kGatherThreads), 0, stream, p, rpg,
                           (int)blocks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.dq_split == 1) return e;
    hipLaunchKernelGGL(dq_reduce, dim3((unsigned)((nrows * 32 + 15) / 16)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int G, int KIT>
hipError_t launch_fill_kit(const BwdParams& p, unsigned groups, hipStream_t stream) {
    hipLaunchKernelGGL((csr_fill<G, KIT>), dim3(groups), dim3(64 * G), fill_lds_bytes(G, p.Ld, p.Lq), stream, p);
    return hipGetLastError();
}
template <int G>
hipError_t launch_fill(const BwdParams& p, unsigned groups, hipStream_t stream) {
    static_assert(kFillIt == 16, "steps per query: 1, 2, 4, 8 or 16");
    if (p.Lq <= 64) return launch_fill_kit<G, 1>(p, groups, stream);
    if (p.Lq <= 128) return launch_fill_kit<G, 2>(p, groups, stream);
    if (p.Lq <= 256) return launch_fill_kit<G, 4>(p, groups, stream);
    if (p.Lq <= 512) return launch_fill_kit<G, 8>(p, groups, stream);
    return launch_fill_kit<G, 16>(p, groups, stream);
}

template <int ELEM, bool VARLEN>
hipError_t launch_bwd_elem(const BwdParams& p, hipStream_t stream) {
    const unsigned groups = (unsigned)(8 * (((int64_t)p.B + 7) / 8) * p.NG);
    hipError_t e;
    hipLaunchKernelGGL(csr_count, dim3(groups), dim3(64 * p.G), p.Ld * sizeof(int), stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.docbase) {
        hipLaunchKernelGGL(csr_docscan, dim3(1), dim3(1024), 0, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    switch (p.G) {
        case 16: e = launch_fill<16>(p, groups, stream); break;
        case 8: e = launch_fill<8>(p, groups, stream); break;
        case 4: e = launch_fill<4>(p, groups, stream); break;
        case 2: e = launch_fill<2>(p, groups, stream); break;
        default: e = launch_fill<1>(p, groups, stream); break;
    }
    if (e != hipSuccess) return e;
    unsigned blocks;
    int rpg;
    const int64_t nrows = VARLEN ? p.T : (int64_t)p.B * p.Ld;
    if (nrows > 0) {
        gather_grid(nrows, &blocks, &rpg);
        // packed: the groups split the sources evenly, so the full grid serves any row count
        if (VARLEN) blocks = kGatherBlocks;
        hipLaunchKernelGGL((dd_owner<ELEM, VARLEN>), dim3(blocks), dim3(kGatherThreads), 0, stream, p, rpg);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const unsigned hb = nrows > 0 ? (unsigned)std::min<int64_t>(p.max_heavy, kGatherBlocks) : 0u;
    return launch_dq<ELEM, VARLEN>(p, hb, stream);
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
    return launch_dq<ELEM, VARLEN>(p, 0u, stream);
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

int bwd_group(int32_t Nq, int32_t Lq, int32_t Ld) {
    if (Ld < 1 || Ld > kMaxLdBwd || Nq < 1) return 0;
    // Groups of 16 queries for long queries; 8 for short ones (Lq <= 256),
    // whose workgroups hold few sources each: there smaller workgroups, more
    // of them per CU, measured 12 % faster at 64 x 32-token queries over 1000
    // documents, and 16 stays 1 % faster for 1024-token queries.
    int G = Lq > 256 ? 16 : 8;
    while (G > 1 && (int64_t)G * Ld > kFillSlots) G >>= 1;  // the fill's per (query, row) slots
    while (G > 1 && G / 2 >= Nq) G >>= 1;                   // no idle query waves beyond Nq
    return G;
}

// Workspace layout, each part at a 256-byte boundary: the CSR counts
// [B][NG][Ld] int32; the query groups' totals [B*NG] int32; the documents'
// first slots [B+1] int32 (used when B*NG > kInlineDocTotals); the heavy-row
// list (count, then rows) int32; the dQ chunk partial sums [S][Nq*Lq][128]
// fp32 when dQ is split (S > 1).  Padded documents and a packed corpus (Ld =
// its longest document) share it.
namespace {
struct WsLayout {
    size_t counts, gtot, docbase, heavy, dq_part, total;
};
// a heavy row has more than kHeavy of the Nq*B*Lq sources
int64_t max_heavy_rows(int32_t Nq, int32_t B, int32_t Lq) { return (int64_t)Nq * B * Lq / (kHeavy + 1); }
bool ws_layout(int32_t Nq, int32_t B, int32_t Lq, int32_t Ld, WsLayout* w) {
    const int G = bwd_group(Nq, Lq, Ld);
    if (G == 0 || B < 1 || Lq < 1) return false;
    const int64_t NG = (Nq + G - 1) / G;
    w->counts = 0;
    w->gtot = w->counts + align256((size_t)(B * NG * Ld * (int64_t)sizeof(int32_t)));
    w->docbase = w->gtot + align256((size_t)(B * NG * (int64_t)sizeof(int32_t)));
    w->heavy = w->docbase + align256((size_t)(B + 1) * sizeof(int32_t));
    w->dq_part = w->heavy + align256((size_t)(1 + max_heavy_rows(Nq, B, Lq)) * sizeof(int32_t));
    w->total = w->dq_part + dq_part_bytes(Nq, Lq, B);
    return true;
}
}  // namespace

size_t bwd_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq, int32_t Ld) {
    WsLayout w;
    return ws_layout(Nq, B, Lq, Ld, &w) ? w.total : 0;
}

size_t bwd_varlen_workspace_bytes(int32_t Nq, int32_t B, int32_t Lq, int32_t max_Ld) {
    return bwd_workspace_bytes(Nq, B, Lq, max_Ld);
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
    p.G = bwd_group(a.Nq, a.Lq, a.Ld);
    p.NG = (a.Nq + p.G - 1) / p.G;
    p.dQ = a.dQ;
    p.dD = a.dD;
    p.row_ptr = a.row_ptr;
    p.col_idx = a.col_idx;
    WsLayout w;
    if (!ws_layout(a.Nq, a.B, a.Lq, a.Ld, &w)) return hipErrorInvalidValue;
    char* ws = static_cast<char*>(a.workspace);
    p.ws = reinterpret_cast<int32_t*>(ws + w.counts);
    p.gtot = reinterpret_cast<int32_t*>(ws + w.gtot);
    p.docbase = (int64_t)a.B * p.NG > kInlineDocTotals ? reinterpret_cast<int32_t*>(ws + w.docbase) : nullptr;
    p.heavy = reinterpret_cast<int32_t*>(ws + w.heavy);
    p.dq_part = reinterpret_cast<float*>(ws + w.dq_part);
    magic_div((unsigned long long)a.B * a.Lq, &p.magic, &p.shift);
    magic_div((unsigned long long)a.Lq, &p.magic_lq, &p.shift_lq);
    p.max_heavy = max_heavy_rows(a.Nq, a.B, a.Lq);
    if (a.cu_seqlens) {
        p.cu = a.cu_seqlens;
        p.T = a.T;
        return a.elem == kBF16 ? launch_bwd_elem<kBF16, true>(p, stream) : launch_bwd_elem<kF16, true>(p, stream);
    }
    return a.elem == kBF16 ? launch_bwd_elem<kBF16, false>(p, stream) : launch_bwd_elem<kF16, false>(p, stream);
}

}  // namespace maxsim

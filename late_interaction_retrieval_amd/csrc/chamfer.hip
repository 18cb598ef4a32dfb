// chamfer.hip -- Chamfer distance on gfx950 (MI355X): the MaxSim machinery
// with a minimum of squared Euclidean distances in place of the maximum of
// inner products (Flash-MaxSim Section 4.2, "Generalization to Chamfer
// Distance").  Forward: for every point of one cloud, the nearest point of
// the other and its index, without the [N, M] distance matrix.  Backward:
// the saved indices inverted into CSR maps (a stable sort of the
// destinations), then one owner per gradient row.
//
// Forward layout.  A 3-float point is too small for the matrix cores, and
// the expanded form |a|^2 + |b|^2 - 2<a, b> loses the small distances that
// decide a nearest neighbour to cancellation, so the distance is formed
// directly on the vector ALU: 3 subtractions, 1 multiply and 2 fused
// multiply-adds, then a compare and two selects.  Each lane keeps 8 (or 4)
// source points in registers; the target points are uniform across the
// wave and arrive by scalar loads, so one load feeds 64 x 8 (or 4) distances.
// The targets of a batch item are split into chunks over workgroups when
// there are too few source tiles to fill the chip; the chunks' minima are
// merged in ascending chunk order.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "internal.h"

namespace maxsim {
namespace {

constexpr int kNnThreads = 256;    // 4 waves
constexpr int kTgtStep = 16;       // targets per scalar-load step
constexpr int kMinChunk = 128;     // targets per chunk, at least

struct NnParams {
    const float* A;  // [Bt, Na, 3] sources
    const float* B;  // [Bt, Nb, 3] targets
    int Bt, Na, Nb;
    int tiles;       // source tiles per batch item
    int chunks;      // target chunks per batch item
    int chunk_len;   // targets per chunk
    float* dist;     // [Bt, Na]  (chunks == 1)
    int32_t* idx;
    float* part_d;   // [chunks][Bt * Na]  (chunks > 1)
    int32_t* part_i;
};

// One direction's workgroup blk of Bt * tiles * chunks; chunk-major inside a
// batch item so that the workgroups sharing a target chunk run together.
template <int kPts>  // source points per lane
__device__ __forceinline__ void nn_tile(const NnParams& p, int blk) {
    constexpr int kSrcTile = kNnThreads * kPts;
    const int per_item = p.tiles * p.chunks;
    const int b = blk / per_item;
    const int rem = blk - b * per_item;
    const int c = rem / p.tiles;
    const int tile = rem - c * p.tiles;
    const int s0 = tile * kSrcTile + threadIdx.x;  // this lane's first source; then +kNnThreads
    const float* __restrict__ A = p.A + (int64_t)b * p.Na * 3;
    const float* __restrict__ T = p.B + (int64_t)b * p.Nb * 3;
    float ax[kPts], ay[kPts], az[kPts], best[kPts];
    int arg[kPts];
#pragma unroll
    for (int r = 0; r < kPts; ++r) {
        const int s = min(s0 + r * kNnThreads, p.Na - 1);  // a lane past the end repeats a valid point
        ax[r] = A[(int64_t)s * 3 + 0];
        ay[r] = A[(int64_t)s * 3 + 1];
        az[r] = A[(int64_t)s * 3 + 2];
        best[r] = __builtin_inff();
        arg[r] = -1;
    }
    const int t_lo = c * p.chunk_len;
    const int t_hi = min(p.Nb, t_lo + p.chunk_len);
    int t = t_lo;
    // full steps: 16 targets (48 floats) by scalar loads, in ascending order
    for (; t + kTgtStep <= t_hi; t += kTgtStep) {
        float tx[kTgtStep], ty[kTgtStep], tz[kTgtStep];
        const float* q = T + (int64_t)t * 3;
#pragma unroll
        for (int k = 0; k < kTgtStep; ++k) {
            tx[k] = q[3 * k];
            ty[k] = q[3 * k + 1];
            tz[k] = q[3 * k + 2];
        }
#pragma unroll
        for (int k = 0; k < kTgtStep; ++k) {
#pragma unroll
            for (int r = 0; r < kPts; ++r) {
                const float dx = ax[r] - tx[k];
                const float dy = ay[r] - ty[k];
                const float dz = az[r] - tz[k];
                const float d = __builtin_fmaf(dz, dz, __builtin_fmaf(dy, dy, dx * dx));
                if (d < best[r]) {
                    best[r] = d;
                    arg[r] = t + k;
                }
            }
        }
    }
    for (; t < t_hi; ++t) {  // the chunk's ragged end
        const float tx = T[(int64_t)t * 3], ty = T[(int64_t)t * 3 + 1], tz = T[(int64_t)t * 3 + 2];
#pragma unroll
        for (int r = 0; r < kPts; ++r) {
            const float dx = ax[r] - tx;
            const float dy = ay[r] - ty;
            const float dz = az[r] - tz;
            const float d = __builtin_fmaf(dz, dz, __builtin_fmaf(dy, dy, dx * dx));
            if (d < best[r]) {
                best[r] = d;
                arg[r] = t;
            }
        }
    }
    const int64_t base = (int64_t)b * p.Na;
    float* od = p.chunks > 1 ? p.part_d + (int64_t)c * p.Bt * p.Na : p.dist;
    int32_t* oi = p.chunks > 1 ? p.part_i + (int64_t)c * p.Bt * p.Na : p.idx;
#pragma unroll
    for (int r = 0; r < kPts; ++r) {
        const int s = s0 + r * kNnThreads;
        if (s < p.Na) {
            od[base + s] = best[r];
            oi[base + s] = arg[r];
        }
    }
}

// Both directions in one launch: workgroups 0 .. g0-1 take p0, the rest p1.
// (The two are independent; together they give the chip twice the resident
// work when one direction alone fills it poorly.)
struct NnPair {
    NnParams d[2];
    int g0;  // workgroups of d[0]
};
template <int kPts>
__global__ __launch_bounds__(kNnThreads) void nn_kernel(NnPair pp) {
    // uniform; indexing the pair loads only the chosen direction's parameters
    // (selecting field by field kept both in scalar registers and pushed the
    // scalar-loaded targets into vector registers)
    const int second = (int)blockIdx.x >= pp.g0 ? 1 : 0;
    const NnParams p = pp.d[second];
    nn_tile<kPts>(p, (int)blockIdx.x - (second ? pp.g0 : 0));
}

// Merge of the chunks' minima in ascending chunk order; a strict compare
// keeps the first index among equal distances.
__device__ __forceinline__ void nn_merge_one(const NnParams& p, int64_t s) {
    const int64_t n = (int64_t)p.Bt * p.Na;
    float best = p.part_d[s];
    int arg = p.part_i[s];
    for (int c = 1; c < p.chunks; ++c) {
        const float d = p.part_d[(int64_t)c * n + s];
        if (d < best) {
            best = d;
            arg = p.part_i[(int64_t)c * n + s];
        }
    }
    p.dist[s] = best;
    p.idx[s] = arg;
}
// elements 0 .. n0-1 of p0, then n1 of p1 (n = 0 for a direction that needs
// no merge)
__global__ __launch_bounds__(256) void nn_merge(NnParams p0, int64_t n0, NnParams p1, int64_t n1) {
    for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < n0 + n1;
         s += (int64_t)gridDim.x * blockDim.x) {
        if (s < n0) {
            nn_merge_one(p0, s);
        } else {
            nn_merge_one(p1, s - n0);
        }
    }
}

// an empty target cloud: +inf and -1 for every source point
__global__ __launch_bounds__(256) void nn_empty(float* dist, int32_t* idx, int64_t n) {
    for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < n; s += (int64_t)gridDim.x * blockDim.x) {
        dist[s] = __builtin_inff();
        idx[s] = -1;
    }
}

void nn_plan_pts(int Bt, int Na, int Nb, int pts, int* tiles, int* chunks, int* chunk_len) {
    const int src_tile = kNnThreads * pts;
    *tiles = (Na + src_tile - 1) / src_tile;
    const int64_t blocks = (int64_t)Bt * *tiles;
    // about 4096 workgroups at most (rounded down: at 100K x 100K points,
    // 2058 workgroups left a nearly empty second round of the 1792 that fit
    // at once, 66 VGPRs; 4067 ran 11 % faster), chunks of kMinChunk at least
    int c = (int)std::min<int64_t>(4096 / blocks, (Nb + kMinChunk - 1) / kMinChunk);
    if (c < 1) c = 1;
    int len = (Nb + c - 1) / c;
    len = (len + kTgtStep - 1) / kTgtStep * kTgtStep;  // whole scalar-load steps except at the very end
    *chunks = (Nb + len - 1) / len;
    if (*chunks < 1) *chunks = 1;
    *chunk_len = len;
}
// 8 source points per lane, or 4 where the 8-point plan fills less than a
// round of the chip (fewer than 2048 workgroups: small clouds or few of
// them): there twice the workgroups, and no idle half tile below 2048
// sources, outweigh the scalar target loads shared by half as many points
// (32 x 2048 x 2048: -11 %, 64 x 1024 x 1024: -40 %; 1 x 100K x 100K, whose
// 8-point plan has 4067 workgroups, ran 3 % slower with 4).
void nn_plan(int Bt, int Na, int Nb, int* pts, int* tiles, int* chunks, int* chunk_len) {
    nn_plan_pts(Bt, Na, Nb, 8, tiles, chunks, chunk_len);
    *pts = 8;
    if ((int64_t)Bt * *tiles * *chunks < 2048) {
        nn_plan_pts(Bt, Na, Nb, 4, tiles, chunks, chunk_len);
        *pts = 4;
    }
}

size_t nn_part_bytes(int Bt, int Na, int Nb) {
    if (Bt < 1 || Na < 1 || Nb < 1) return 0;
    int pts, tiles, chunks, len;
    nn_plan(Bt, Na, Nb, &pts, &tiles, &chunks, &len);
    return chunks > 1 ? (size_t)chunks * Bt * Na * 8 : 0;
}

// One direction's parameters and plan; its chunk minima (when the targets
// are split) at ws.
NnParams nn_params(const float* A, const float* B, int Bt, int Na, int Nb, float* dist, int32_t* idx, void* ws,
                   int* pts) {
    NnParams p{};
    p.A = A;
    p.B = B;
    p.Bt = Bt;
    p.Na = Na;
    p.Nb = Nb;
    nn_plan(Bt, Na, Nb, pts, &p.tiles, &p.chunks, &p.chunk_len);
    p.dist = dist;
    p.idx = idx;
    const int64_t n = (int64_t)Bt * Na;
    p.part_d = static_cast<float*>(ws);
    p.part_i = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + (size_t)p.chunks * n * 4);
    return p;
}

hipError_t launch_nn_pair(const NnParams& p0, const NnParams& p1, int pts, hipStream_t stream) {
    const int g0 = p0.Bt * p0.tiles * p0.chunks, g1 = p1.Bt * p1.tiles * p1.chunks;
    const dim3 grid((unsigned)(g0 + g1));
    NnPair pp;
    pp.d[0] = p0;
    pp.d[1] = p1;
    pp.g0 = g0;
    if (pts == 4) {
        hipLaunchKernelGGL(nn_kernel<4>, grid, dim3(kNnThreads), 0, stream, pp);
    } else {
        hipLaunchKernelGGL(nn_kernel<8>, grid, dim3(kNnThreads), 0, stream, pp);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n0 = p0.chunks > 1 ? (int64_t)p0.Bt * p0.Na : 0;
    const int64_t n1 = p1.chunks > 1 ? (int64_t)p1.Bt * p1.Na : 0;
    if (n0 + n1 == 0) return hipSuccess;
    hipLaunchKernelGGL(nn_merge, dim3((unsigned)std::min<int64_t>((n0 + n1 + 255) / 256, 8192)), dim3(256), 0, stream,
                       p0, n0, p1, n1);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward.  Source s (a point of one cloud, global index b*Na + i) selects
// destination b*Nb + idx[s] of the other cloud.  The CSR map of a direction
// is a stable sort of the sources by destination: an LSD radix sort, 8 bits
// per pass, of (destination, source) pairs, in a fixed order, so the map is
// the same on every run.  Both directions go through one sort: the Q points
// (selecting P destinations 0 .. Bt*N-1) come first, then the P points
// (selecting Q destinations, keyed Bt*N + b*M + j).  Unselected sources
// (idx = -1) get the key nd = Bt*(N+M) and sort to the end.  row_ptr[r] is
// then the lower bound of r in the sorted keys.
// ---------------------------------------------------------------------------
constexpr int kSortThreads = 256;
constexpr int kSortItems = 8;  // per thread per pass
constexpr int kSortTile = kSortThreads * kSortItems;

// elements 0 .. Bt*M-1: the Q points and their P destinations; then the P
// points and their Q destinations (offset by Bt*N); the value is the
// source's global index in its own cloud
__global__ __launch_bounds__(256) void sort_init(const int32_t* idx_q, const int32_t* idx_p, int N, int M,
                                                 int64_t nq, int64_t n, int64_t ndp, int64_t nd, uint32_t* key,
                                                 int32_t* val) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
        const bool qside = e < nq;
        const int64_t s = qside ? e : e - nq;
        const int32_t t = qside ? idx_q[s] : idx_p[s];
        const int Na = qside ? M : N, Nb = qside ? N : M;
        const int64_t b = s / Na;
        key[e] = (t < 0 || t >= Nb) ? (uint32_t)nd : (uint32_t)((qside ? 0 : ndp) + b * Nb + t);
        val[e] = (int32_t)s;
    }
}

// per tile: histogram of the pass's digit -> hist[digit * ntiles + tile]
__global__ __launch_bounds__(kSortThreads) void sort_hist(const uint32_t* key, int64_t n, int shift, int ntiles,
                                                          int32_t* hist) {
    __shared__ int h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int64_t e0 = (int64_t)blockIdx.x * kSortTile;
#pragma unroll
    for (int k = 0; k < kSortItems; ++k) {
        const int64_t e = e0 + k * kSortThreads + threadIdx.x;
        if (e < n) atomicAdd(&h[(key[e] >> shift) & 255u], 1);
    }
    __syncthreads();
    hist[(int64_t)threadIdx.x * ntiles + blockIdx.x] = h[threadIdx.x];
}

// exclusive scan of hist [256 * ntiles] in place (one workgroup, in order):
// each thread takes 16 consecutive entries per round of 16384.  A round goes
// through LDS: coalesced loads and stores on the memory side (a thread's own
// 16 entries read straight from memory were 64 bytes apart across the wave,
// and the one workgroup's load path set the time), and a row of 17 words per
// thread, so the thread's 16 reads hit distinct banks across the wave.
constexpr int kScanRound = 1024 * 16;
__global__ __launch_bounds__(1024) void sort_scan(int32_t* hist, int64_t len) {
    __shared__ int buf[1024 * 17];
    __shared__ int wsum[16];
    __shared__ int carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry_s = 0;
    for (int64_t i0 = 0; i0 < len; i0 += kScanRound) {
        const int64_t cnt = len - i0 < kScanRound ? len - i0 : kScanRound;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int e = k * 1024 + tid;
            buf[(e >> 4) * 17 + (e & 15)] = e < cnt ? hist[i0 + e] : 0;
        }
        __syncthreads();
        int v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = buf[tid * 17 + k];
        int tot = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) tot += v[k];
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
        int run = carry + wpre + x - tot;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            buf[tid * 17 + k] = run;
            run += v[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int e = k * 1024 + tid;
            if (e < cnt) hist[i0 + e] = buf[(e >> 4) * 17 + (e & 15)];
        }
        if (tid == 1023) carry_s = carry + wpre + x;
        __syncthreads();
    }
}

// Stable scatter: a tile's elements are placed in ascending element order.
// Per round of 256 elements (one per thread, thread order = element order):
// a lane's rank among the lanes of its wave with the same digit comes from
// eight ballots; the waves before it add their counts of that digit; the
// earlier rounds of the tile add theirs (running[]).
__global__ __launch_bounds__(kSortThreads) void sort_scatter(const uint32_t* key, const int32_t* val, int64_t n,
                                                             int shift, int ntiles, const int32_t* offs,
                                                             uint32_t* key_out, int32_t* val_out) {
    __shared__ int running[256];
    __shared__ int wcount[kSortThreads / 64][256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    running[tid] = offs[(int64_t)tid * ntiles + blockIdx.x];
    const int64_t e0 = (int64_t)blockIdx.x * kSortTile;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int k = 0; k < kSortItems; ++k) {
#pragma unroll
        for (int w = 0; w < kSortThreads / 64; ++w) wcount[w][tid] = 0;
        __syncthreads();  // also orders running[] after the previous round's update
        const int64_t e = e0 + k * kSortThreads + tid;
        const bool valid = e < n;
        const uint32_t kv = valid ? key[e] : 0u;
        const int dg = (int)((kv >> shift) & 255u);
        unsigned long long m = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const unsigned long long vote = __ballot((dg >> bit) & 1);
            m &= ((dg >> bit) & 1) ? vote : ~vote;
        }
        const int rank = __popcll(m & below);
        if (valid && rank == 0) wcount[wave][dg] = __popcll(m);
        __syncthreads();
        if (valid) {
            int pre = running[dg];
            for (int w = 0; w < wave; ++w) pre += wcount[w][dg];
            key_out[pre + rank] = kv;
            val_out[pre + rank] = val[e];
        }
        __syncthreads();
        int add = 0;
#pragma unroll
        for (int w = 0; w < kSortThreads / 64; ++w) add += wcount[w][tid];
        running[tid] += add;
    }
}

__device__ __forceinline__ int64_t lower_bound(const uint32_t* key, int64_t n, int64_t r) {
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (key[mid] < (uint32_t)r) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// row_ptr_p[r] = lower bound of r (r = 0 .. ndp); row_ptr_q[r] = lower bound
// of ndp + r minus that of ndp (r = 0 .. nd - ndp), so each map starts at 0
__global__ __launch_bounds__(256) void csr_bounds(const uint32_t* key, int64_t n, int64_t ndp, int64_t nd,
                                                  int32_t* row_ptr_p, int32_t* row_ptr_q, int32_t* heavy) {
    if (blockIdx.x == 0 && threadIdx.x == 0) heavy[0] = 0;  // chamfer_rows appends after this kernel
    const int64_t base_q = lower_bound(key, n, ndp);
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r <= nd + 1;
         r += (int64_t)gridDim.x * blockDim.x) {
        if (r <= ndp) {
            row_ptr_p[r] = (int32_t)lower_bound(key, n, r);
        } else {
            const int64_t rq = r - ndp - 1;  // 0 .. nd - ndp
            row_ptr_q[rq] = (int32_t)(lower_bound(key, n, ndp + rq) - base_q);
        }
    }
}

// sorted values -> col_idx_p (the first row_ptr_p[ndp]) and col_idx_q (the next)
__global__ __launch_bounds__(256) void csr_split(const int32_t* val, const int32_t* row_ptr_p,
                                                 const int32_t* row_ptr_q, int64_t ndp, int64_t ndq,
                                                 int32_t* col_idx_p, int32_t* col_idx_q) {
    const int64_t np = row_ptr_p[ndp], nq = row_ptr_q[ndq];
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < np + nq;
         e += (int64_t)gridDim.x * blockDim.x) {
        if (e < np) {
            col_idx_p[e] = val[e];
        } else {
            col_idx_q[e - np] = val[e];
        }
    }
}

// Destination-owned gradient rows.  Row r of cloud X (b*Nx + i) owns
//   2 gx[r] (X[r] - Y[b, idx_x[r]])  +  sum over its CSR sources s of 2 gy[s] (X[r] - Y[s]).
// 4 lanes per row (every point selects one point, so a row has one source on
// average): lane l sums the row's sources l, l+4, ... in ascending order, the
// lanes are added by a fixed butterfly, then the row's own term.
struct RowSide {
    const float* X;
    const float* Y;
    const int32_t* idx_x;
    const float* gx;
    const float* gy;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    int Nx, Ny;
    int64_t nrows;
    float* dX;
};

// A row with more sources than this goes to chamfer_heavy (a whole
// workgroup), so one 4-lane group never walks a long bucket alone.
constexpr int kChLanes = 4;
constexpr int kChHeavy = 256;

// rows of P first (side 0), then rows of Q (side 1), in one launch; heavy
// rows are appended to heavy[1 ..] (count in heavy[0]) and left out here
__global__ __launch_bounds__(256) void chamfer_rows(RowSide s0, RowSide s1, int32_t* heavy, int64_t max_heavy) {
    const int64_t rg = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kChLanes;
    const bool second = rg >= s0.nrows;  // uniform per row group
    const RowSide& sd = second ? s1 : s0;
    const int64_t r = second ? rg - s0.nrows : rg;
    const float* X = sd.X;
    const float* Y = sd.Y;
    const int32_t* idx_x = sd.idx_x;
    const float* gx = sd.gx;
    const float* gy = sd.gy;
    const int32_t* row_ptr = sd.row_ptr;
    const int32_t* col_idx = sd.col_idx;
    const int Nx = sd.Nx, Ny = sd.Ny;
    float* dX = sd.dX;
    const int lr = threadIdx.x % kChLanes;
    const bool ok = r < sd.nrows;
    const int64_t rr = ok ? r : 0;
    // a group past the last row reads nothing (that cloud may be empty)
    const float x0 = ok ? X[rr * 3] : 0.f, x1 = ok ? X[rr * 3 + 1] : 0.f, x2 = ok ? X[rr * 3 + 2] : 0.f;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f;
    const int beg = ok ? row_ptr[rr] : 0, end = ok ? row_ptr[rr + 1] : 0;
    if (end - beg > kChHeavy) {  // uniform per group
        if (lr == 0) {
            const int slot = atomicAdd(&heavy[0], 1);
            if (slot < max_heavy) heavy[1 + slot] = (int32_t)rg;
        }
        return;
    }
    if (ok) {
        for (int e = beg + lr; e < end; e += kChLanes) {
            const int64_t s = col_idx[e];
            const float w = 2.0f * gy[s];
            a0 = __builtin_fmaf(w, x0 - Y[s * 3], a0);
            a1 = __builtin_fmaf(w, x1 - Y[s * 3 + 1], a1);
            a2 = __builtin_fmaf(w, x2 - Y[s * 3 + 2], a2);
        }
    }
#pragma unroll
    for (int off = kChLanes / 2; off >= 1; off >>= 1) {
        a0 += __shfl_xor(a0, off, kChLanes);
        a1 += __shfl_xor(a1, off, kChLanes);
        a2 += __shfl_xor(a2, off, kChLanes);
    }
    if (ok && lr == 0) {
        const int32_t t = idx_x[rr];
        if (t >= 0 && t < Ny) {
            const int64_t b = rr / Nx;
            const float* y = Y + (b * Ny + t) * 3;
            const float w = 2.0f * gx[rr];
            a0 = __builtin_fmaf(w, x0 - y[0], a0);
            a1 = __builtin_fmaf(w, x1 - y[1], a1);
            a2 = __builtin_fmaf(w, x2 - y[2], a2);
        }
        dX[rr * 3] = a0;
        dX[rr * 3 + 1] = a1;
        dX[rr * 3 + 2] = a2;
    }
}

// One heavy row per workgroup at a time: thread t sums the row's sources t,
// t + 256, ... in ascending order, a fixed pairwise tree in LDS adds the
// threads, then the row's own term.  Runs are bit-identical.
__global__ __launch_bounds__(256) void chamfer_heavy(RowSide s0, RowSide s1, const int32_t* heavy, int64_t max_heavy) {
    __shared__ float red[3][256];
    const int tid = threadIdx.x;
    const int count = (int)(heavy[0] < max_heavy ? heavy[0] : max_heavy);
    for (int h = blockIdx.x; h < count; h += gridDim.x) {  // uniform
        const int64_t rg = heavy[1 + h];
        const bool second = rg >= s0.nrows;
        const RowSide& sd = second ? s1 : s0;
        const int64_t r = second ? rg - s0.nrows : rg;
        const float x0 = sd.X[r * 3], x1 = sd.X[r * 3 + 1], x2 = sd.X[r * 3 + 2];
        const int beg = sd.row_ptr[r], end = sd.row_ptr[r + 1];
        float a0 = 0.f, a1 = 0.f, a2 = 0.f;
        for (int e = beg + tid; e < end; e += 256) {
            const int64_t s = sd.col_idx[e];
            const float w = 2.0f * sd.gy[s];
            a0 = __builtin_fmaf(w, x0 - sd.Y[s * 3], a0);
            a1 = __builtin_fmaf(w, x1 - sd.Y[s * 3 + 1], a1);
            a2 = __builtin_fmaf(w, x2 - sd.Y[s * 3 + 2], a2);
        }
        red[0][tid] = a0;
        red[1][tid] = a1;
        red[2][tid] = a2;
        __syncthreads();
        for (int half = 128; half > 0; half >>= 1) {
            if (tid < half) {
                red[0][tid] += red[0][tid + half];
                red[1][tid] += red[1][tid + half];
                red[2][tid] += red[2][tid + half];
            }
            __syncthreads();
        }
        if (tid == 0) {
            a0 = red[0][0];
            a1 = red[1][0];
            a2 = red[2][0];
            const int32_t t = sd.idx_x[r];
            if (t >= 0 && t < sd.Ny) {
                const int64_t b = r / sd.Nx;
                const float* y = sd.Y + (b * sd.Ny + t) * 3;
                const float w = 2.0f * sd.gx[r];
                a0 = __builtin_fmaf(w, x0 - y[0], a0);
                a1 = __builtin_fmaf(w, x1 - y[1], a1);
                a2 = __builtin_fmaf(w, x2 - y[2], a2);
            }
            sd.dX[r * 3] = a0;
            sd.dX[r * 3 + 1] = a1;
            sd.dX[r * 3 + 2] = a2;
        }
        __syncthreads();  // red is reused by the next heavy row
    }
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// workspace of one sort of n elements: keys and values twice, the histogram
size_t sort_bytes(int64_t n) {
    const int64_t ntiles = (n + kSortTile - 1) / kSortTile;
    return 2 * align256((size_t)n * 4) + 2 * align256((size_t)n * 4) + align256((size_t)ntiles * 256 * 4);
}

int key_bits(int64_t nd) {
    int bits = 1;
    while (bits < 32 && ((int64_t)1 << bits) <= nd) ++bits;  // keys take values 0 .. nd
    return bits;
}

// the heavy-row list lives after the sort's buffers in the workspace
int64_t max_heavy_rows(const ChamferArgs& a) {
    return ((int64_t)a.Bt * a.N + (int64_t)a.Bt * a.M) / (kChHeavy + 1);
}
int32_t* heavy_list(const ChamferArgs& a) {
    return reinterpret_cast<int32_t*>(static_cast<char*>(a.workspace) +
                                      sort_bytes((int64_t)a.Bt * a.N + (int64_t)a.Bt * a.M));
}

// Both CSR maps with one sort (see above).
hipError_t build_csr_pair(const ChamferArgs& a, hipStream_t stream) {
    const int64_t nq = (int64_t)a.Bt * a.M, np = (int64_t)a.Bt * a.N;
    const int64_t n = nq + np, ndp = np, nd = np + nq;
    hipError_t e;
    char* w = static_cast<char*>(a.workspace);
    uint32_t* k0 = reinterpret_cast<uint32_t*>(w);
    uint32_t* k1 = reinterpret_cast<uint32_t*>(w + align256((size_t)n * 4));
    int32_t* v0 = reinterpret_cast<int32_t*>(w + 2 * align256((size_t)n * 4));
    int32_t* v1 = reinterpret_cast<int32_t*>(w + 3 * align256((size_t)n * 4));
    int32_t* hist = reinterpret_cast<int32_t*>(w + 4 * align256((size_t)n * 4));
    const unsigned gb = (unsigned)std::min<int64_t>((n + 255) / 256, 4096);
    if (n > 0) {
        const int ntiles = (int)((n + kSortTile - 1) / kSortTile);
        hipLaunchKernelGGL(sort_init, dim3(gb), dim3(256), 0, stream, a.idx_q, a.idx_p, a.N, a.M, nq, n, ndp, nd, k0,
                           v0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int passes = (key_bits(nd) + 7) / 8;
        for (int ps = 0; ps < passes; ++ps) {
            hipLaunchKernelGGL(sort_hist, dim3(ntiles), dim3(kSortThreads), 0, stream, k0, n, 8 * ps, ntiles, hist);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(sort_scan, dim3(1), dim3(1024), 0, stream, hist, (int64_t)ntiles * 256);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(sort_scatter, dim3(ntiles), dim3(kSortThreads), 0, stream, k0, v0, n, 8 * ps, ntiles,
                               hist, k1, v1);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            std::swap(k0, k1);
            std::swap(v0, v1);
        }
    }
    hipLaunchKernelGGL(csr_bounds, dim3((unsigned)std::min<int64_t>((nd + 2 + 255) / 256, 4096)), dim3(256), 0, stream,
                       k0, n, ndp, nd, a.row_ptr_p, a.row_ptr_q, heavy_list(a));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(csr_split, dim3(gb), dim3(256), 0, stream, v0, a.row_ptr_p, a.row_ptr_q, ndp, nd - ndp,
                       a.col_idx_p, a.col_idx_q);
    return hipGetLastError();
}

hipError_t launch_rows_pair(const ChamferArgs& a, hipStream_t stream) {
    RowSide sp{a.P, a.Q, a.idx_p, a.grad_p, a.grad_q, a.row_ptr_p, a.col_idx_p, a.N, a.M, (int64_t)a.Bt * a.N, a.dP};
    RowSide sq{a.Q, a.P, a.idx_q, a.grad_q, a.grad_p, a.row_ptr_q, a.col_idx_q, a.M, a.N, (int64_t)a.Bt * a.M, a.dQ};
    const int64_t nrows = sp.nrows + sq.nrows;
    if (nrows == 0) return hipSuccess;
    const int64_t mh = max_heavy_rows(a);
    hipLaunchKernelGGL(chamfer_rows, dim3((unsigned)((nrows * kChLanes + 255) / 256)), dim3(256), 0, stream, sp, sq,
                       heavy_list(a), mh);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || mh == 0) return e;
    hipLaunchKernelGGL(chamfer_heavy, dim3((unsigned)std::min<int64_t>(mh, 1024)), dim3(256), 0, stream, sp, sq,
                       heavy_list(a), mh);
    return hipGetLastError();
}

}  // namespace

// both directions' chunk minima, side by side (the directions run together)
size_t chamfer_fwd_workspace_bytes(int32_t Bt, int32_t N, int32_t M) {
    return std::max<size_t>(256, align256(nn_part_bytes(Bt, N, M)) + align256(nn_part_bytes(Bt, M, N)));
}

hipError_t launch_chamfer_fwd(const ChamferArgs& a, hipStream_t stream) {
    if (a.Bt == 0 || (a.N == 0 && a.M == 0)) return hipSuccess;
    if (a.N == 0 || a.M == 0) {  // one cloud empty: the other's points get +inf and -1
        const int64_t n = (int64_t)a.Bt * (a.N == 0 ? a.M : a.N);
        hipLaunchKernelGGL(nn_empty, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 4096)), dim3(256), 0, stream,
                           a.N == 0 ? a.dist_q : a.dist_p, a.N == 0 ? a.idx_q : a.idx_p, n);
        return hipGetLastError();
    }
    char* ws = static_cast<char*>(a.workspace);
    int pts0, pts1;
    const NnParams p0 = nn_params(a.P, a.Q, a.Bt, a.N, a.M, a.dist_p, a.idx_p, ws, &pts0);
    const NnParams p1 = nn_params(a.Q, a.P, a.Bt, a.M, a.N, a.dist_q, a.idx_q,
                                  ws + align256(nn_part_bytes(a.Bt, a.N, a.M)), &pts1);
    const int64_t g0 = (int64_t)p0.Bt * p0.tiles * p0.chunks, g1 = (int64_t)p1.Bt * p1.tiles * p1.chunks;
    if (pts0 == pts1 && g0 + g1 <= INT32_MAX) return launch_nn_pair(p0, p1, pts0, stream);
    // different lane plans (or a grid past int range together): one launch per
    // direction (an empty second half)
    NnParams none = p0;
    none.chunks = 1;
    none.tiles = 0;
    hipError_t e = launch_nn_pair(p0, none, pts0, stream);
    if (e != hipSuccess) return e;
    NnParams none1 = p1;
    none1.chunks = 1;
    none1.tiles = 0;
    return launch_nn_pair(p1, none1, pts1, stream);
}

}  // namespace maxsim

namespace maxsim {

size_t chamfer_bwd_workspace_bytes(int32_t Bt, int32_t N, int32_t M) {
    const int64_t n = (int64_t)Bt * N + (int64_t)Bt * M;
    return sort_bytes(n) + align256((size_t)(1 + n / (kChHeavy + 1)) * sizeof(int32_t));
}

hipError_t launch_chamfer_bwd(const ChamferArgs& a, hipStream_t stream) {
    hipError_t e = build_csr_pair(a, stream);
    if (e != hipSuccess) return e;
    return launch_rows_pair(a, stream);
}

}  // namespace maxsim

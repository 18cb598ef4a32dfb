// fwd.hip -- fused MaxSim forward for gfx950 (MI355X).
//
// Computes score(Q, D) = sum_i max_j <Q_i, D_j> for every (query, document)
// pair without writing the similarity tensor (Flash-MaxSim, Section 1 Eq. (1);
// Section 4.1 Algorithm 2 and "Online-Max Recurrence"), and the per query token
// argmax that the backward reuses (Section 4.2).
//
// Design (MI355X-first, not the page's per-pair programs):
//   * A workgroup owns a "slab" of whole queries (up to R query-token rows) and
//     keeps it stationary in VGPRs as the MFMA B operand for its whole life.
//     This is the query-reuse member of the page's kernel family (Section 4.1
//     "Kernel Family"): every document tile it reads is used against all R rows.
//   * Documents stream HBM -> LDS in tiles (256 tokens in a two-buffer ring
//     for fp16/bf16 32x32 blocks; 128 or 64 tokens in a three-buffer ring
//     otherwise) of direct (buffer_load ... lds) loads: the next tiles, possibly
//     of later documents, are in flight while the current one is contracted.
//     LDS rows are XOR-swizzled by 16-byte chunk so the MFMA operand reads are
//     bank-conflict free.
//   * S_t = D_tile Q_slab^T is formed M doc tokens x M query rows at a time.
//     fp16/bf16 use v_mfma_f32_32x32x16 (M = 32; one accumulation chain per
//     query block); int8 uses v_mfma_i32_16x16x64_i8 (M = 16).  Doc tokens are
//     the M dimension of the result, so each lane holds VPL tokens of one query
//     row and the running max / argmax stays in the lane; lanes are merged once
//     per document.  For 32x32 blocks the sub-tiles of a tile form a software
//     pipeline: the MFMAs of sub-tile j are interleaved with the VALU fold of
//     sub-tile j-1, so the matrix pipe and the VALU overlap inside one wave.
//   * The grid is persistent: block -> (slab, document stream) is laid out so
//     the workgroups sharing a document stream sit on the same XCD (blocks are
//     dispatched round-robin over the 8 XCDs) and re-read each tile from that
//     XCD's L2 rather than HBM.  A stream is a contiguous range of documents
//     balanced by work (stream_range) when the grid is one round of
//     workgroups, else every num_streams-th document.
//   * With two tile buffers the first wave of each SIMD issues the tile loads
//     and the second none, and each stage's MFMAs run at raised wave priority,
//     so one wave's non-MFMA work overlaps the other's matrix work.
//   * Masking (Algorithm 2): positions past the document's length are -inf
//     before the maximum (or, where that cannot change the result, rows past
//     the end repeat the tile's first row and are folded unmasked).
//   * int8 (Section 4.3): each value fl32(dot * d_scale) comes from one fused
//     multiply-add on an accumulator started at the bits of 2^23, and each
//     query's exact sum runs in ascending row order at raised wave priority,
//     by a thread per query or, for queries of 64 rows or more, by a wave.
//   * Scores only, 32-token queries, packed corpus (ColBERT re-ranking):
//     fwd_flat_kernel reads each stream's tokens as tiles that run across
//     document boundaries and splits the fold where a document ends.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.h"

namespace maxsim {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct FwdParams {
    const char* Q;
    const char* D;
    const int32_t* lens;
    const int32_t* cu;
    const float* q_scale;
    const float* d_scale;
    int64_t T;
    int Nq, Lq, B, Ld;
    int qps;          // queries per slab (whole queries), or 1 when split
    int split;        // 1: slabs hold whole queries; 2: each query is two half slabs
    int half_rows;    // rows of the first half of a split query
    int num_slabs;
    int num_streams;  // document streams
    int round_robin;  // 1: stream s takes documents s, s + num_streams, ...; 0: a contiguous range (stream_range)
    float* scores;
    int32_t* argmax;
};

// One M x M block of S = D_tile Q^T contracted over the 128-wide embedding.
// Lane l supplies row (l % M) of each operand and one 16-byte chunk of it per
// k-step; NG = 64 / M lane groups (g = l / M) split the k range.  The result
// holds VPL = M*M/64 values per lane: column (query row) l % M and the doc
// tokens tok(g, i), i < VPL.
template <int ELEM, int M>
struct Mma;

template <int ELEM>
struct Mma<ELEM, 16> {  // v_mfma_f32_16x16x32_{f16,bf16}: 8 halves/lane/step, 4 steps
    static constexpr int NG = 4, VPL = 4, KS = 4;
    typedef f32x4 Acc;
    __device__ static __forceinline__ Acc zero() { return Acc{0.f, 0.f, 0.f, 0.f}; }
    __device__ static __forceinline__ Acc mma(u32x4 a, u32x4 b, Acc c) {
        if constexpr (ELEM == kF16) {
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                          __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
        } else {
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                           __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
        }
    }
    __device__ static __forceinline__ int tok(int g, int i) { return 4 * g + i; }
};

template <int ELEM>
struct Mma<ELEM, 32> {  // v_mfma_f32_32x32x16_{f16,bf16}: 8 halves/lane/step, 8 steps
    static constexpr int NG = 2, VPL = 16, KS = 8;
    typedef f32x16 Acc;
    __device__ static __forceinline__ Acc zero() {
        Acc z;
#pragma unroll
        for (int e = 0; e < 16; ++e) z[e] = 0.f;
        return z;
    }
    __device__ static __forceinline__ Acc mma(u32x4 a, u32x4 b, Acc c) {
        if constexpr (ELEM == kF16) {
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                          __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
        } else {
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                           __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
        }
    }
    __device__ static __forceinline__ int tok(int g, int i) { return 8 * (i >> 2) + 4 * g + (i & 3); }
};

template <>
struct Mma<kI8, 16> {  // v_mfma_i32_16x16x64_i8: 16 bytes/lane/step, 2 steps
    static constexpr int NG = 4, VPL = 4, KS = 2;
    typedef i32x4 Acc;
    __device__ static __forceinline__ Acc zero() { return Acc{0, 0, 0, 0}; }
    __device__ static __forceinline__ Acc mma(u32x4 a, u32x4 b, Acc c) {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                                     __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ int tok(int g, int i) { return 4 * g + i; }
};

// LDS slot (in 16-byte units) of chunk c of tile row `row`.  fp16/bf16 rows are
// 256 B = 16 chunks (one full bank sweep): chunk ^ (row & 15).  int8 rows are
// 128 B = 8 chunks, two rows per sweep: chunk ^ ((row >> 1) & 7).  Any 8 or 16
// consecutive rows read at one logical chunk land on distinct bank groups.  The
// map is its own inverse within a row, which the loader uses: the lane that
// fills slot s fetches chunk (s % NCH) ^ f(row) of row s / NCH.
template <int NCH>
__device__ __forceinline__ int swz_chunk(int row, int c) {
    if constexpr (NCH == 16) {
        return c ^ (row & 15);
    } else {
        return c ^ ((row >> 1) & 7);
    }
}
template <int NCH>
__device__ __forceinline__ int swz(int row, int c) {
    return row * NCH + swz_chunk<NCH>(row, c);
}
// The swizzle reads only the row's low four bits, so for an M-row sub-tile
// (M a multiple of 16) swz(sb*M + lm, c) = sb*M*NCH + swz(lm, c): a per-lane
// slot plus a per-sub-tile constant, which the compiler folds into the LDS
// read's immediate offset when the sub-tile index is known.
template <int NCH, int M>
__device__ __forceinline__ int sub_slot(int sb, int lane_slot) {
    static_assert(M % 16 == 0, "sub-tiles span whole swizzle periods");
    return sb * (M * NCH) + lane_slot;
}

// s_waitcnt vmcnt(N) (other counters untouched), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void* lptr_t;
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;  // read-only for the kernel: scalar loads

// Direct HBM -> LDS load (buffer_load ... lds) of `size` bytes per lane (4 or
// 16): lane l's bytes [voff, voff + size) of the nbytes-long range at base
// land at lds + l * size; bytes at or past nbytes read as zero without a
// memory access.  base and nbytes must be wave-uniform (they form the buffer
// descriptor).  The buffer form rather than global_load_lds: the compiler
// counts a FLAT-encoded LDS load as LDS traffic of unknown order while it is
// in flight, and then makes every LDS read wait for all earlier ones
// (lgkmcnt(0)), so a stage's first MFMA waited for all eight of its operand
// reads instead of the first.
__device__ __forceinline__ void buffer_load_lds(const void* base, uint32_t nbytes, uint32_t voff, lptr_t lds, int size) {
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(nbytes);
    // word 3 of a raw (stride 0) gfx9 descriptor: 32-bit data format
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, (int)n, 0x00020000);
    if (size == 16) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, (int)voff, 0, 0, 0);
    } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, (int)voff, 0, 0, 0);
    }
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also orders global
// memory, which makes every wave drain its in-flight HBM -> LDS loads
// (vmcnt(0)) at each barrier and would serialise the tile ring.  Here each wave
// waits for its own LDS reads/writes (lgkmcnt(0)) and the ring's direct loads
// are retired explicitly (wait_vmcnt) before the barrier; the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Row r of the per-document row maxima (and of the int8 query scales) lives
// at r + r/32, so threads reading the rows of consecutive queries (stride Lq)
// do not all hit one bank.
__device__ __forceinline__ int rpad(int r) { return r + (r >> 5); }

template <bool VARLEN>
__device__ __forceinline__ void doc_info(const FwdParams& p, int b, int64_t& start, int& len) {
    if constexpr (VARLEN) {
        const cint_ptr cu = (cint_ptr)p.cu;
        int64_t s0 = cu[b];
        int64_t s1 = cu[b + 1];
        s0 = s0 < 0 ? 0 : (s0 > p.T ? p.T : s0);
        s1 = s1 < s0 ? s0 : (s1 > p.T ? p.T : s1);
        start = s0;
        len = (int)(s1 - s0);
    } else {
        start = (int64_t)b * p.Ld;
        int l = p.lens ? ((cint_ptr)p.lens)[b] : p.Ld;
        len = l < 0 ? 0 : (l > p.Ld ? p.Ld : l);
    }
}

__device__ __forceinline__ unsigned fbits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float bitsf(unsigned x) { return __uint_as_float(x); }

// Lane exchanges without an LDS round trip.  v_permlane32_swap swaps the
// upper 32 lanes of its first operand with the lower 32 of its second;
// v_permlane16_swap swaps the odd 16-lane rows of the first with the even
// rows of the second.  With v as both operands, each returns the lane's own
// value and that of lane l ^ 32 (or l ^ 16), in an order that depends on the
// lane, so their maximum (or minimum) needs no lane select.
__device__ __forceinline__ float xor32_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(fbits(v), fbits(v), false, false);
    return fmaxf(bitsf(r[0]), bitsf(r[1]));
}
__device__ __forceinline__ float xor16_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
    return fmaxf(bitsf(r[0]), bitsf(r[1]));
}
// The same pairings for the unsigned minimum.
__device__ __forceinline__ unsigned xor32_min_u(unsigned v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return r[0] < r[1] ? r[0] : r[1];
}
__device__ __forceinline__ unsigned xor16_min_u(unsigned v) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return r[0] < r[1] ? r[0] : r[1];
}


// Calls f(std::integral_constant<int, j>{}) for j = 0 .. N-1, expanded at
// compile time.
template <int N, int J = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (J < N) {
        f(std::integral_constant<int, J>{});
        static_for<N, J + 1>(f);
    }
}

// Document stream s of S scores the contiguous range [start(s), start(s+1)).
// Padded documents are split by count.  A packed corpus is split by work:
// document b costs its tokens plus DOC_COST (a partial sub-tile and the
// per-document epilogue, in token units), so with key(b) = cu[b] + DOC_COST*b
// (increasing in b), start(s) is the first document whose key reaches
// s*K/S, K = key(B), and every stream gets about K/S, to within one document.
// (Dealing ragged documents round-robin leaves the longest stream 6-11 %
// above the mean at the packed workloads' length mixes, and the grid waits
// for it.)  start(s) is found by the whole workgroup: each round the NT
// threads test evenly spaced entries of the remaining range and a workgroup
// count of those below the target narrows it by a factor of NT, so
// B <= NT^2 needs two rounds of loads.  start(0) = 0 and start(S) = B.  Both
// ends use the same search, so neighbouring streams agree on their common
// boundary.  Every thread of the workgroup must call this (it has barriers).
constexpr int64_t DOC_COST = 32;
template <bool VARLEN, int NT>
__device__ __forceinline__ void stream_range(const FwdParams& p, int s, int& bbeg, int& bend) {
    const int S = p.num_streams;
    if constexpr (!VARLEN) {
        bbeg = (int)((int64_t)s * p.B / S);
        bend = (int)((int64_t)(s + 1) * p.B / S);
    } else {
        const int64_t K = p.T + DOC_COST * p.B;
        const int64_t x0 = (int64_t)s * K / S;
        const int64_t x1 = (int64_t)(s + 1) * K / S;
        // the answer lies in [lo, hi] and key(hi) >= x (key(B) = K >= x)
        int lo0 = 0, hi0 = s == 0 ? 0 : p.B;
        int lo1 = s + 1 == S ? p.B : 0, hi1 = p.B;
        const int t = threadIdx.x;
        while (lo0 < hi0 || lo1 < hi1) {  // uniform
            const int st0 = (hi0 - lo0) / NT + 1, st1 = (hi1 - lo1) / NT + 1;  // (hi - lo) / st < NT
            const int64_t i0 = lo0 + (int64_t)t * st0, i1 = lo1 + (int64_t)t * st1;
            const bool in0 = lo0 < hi0 && i0 <= hi0, in1 = lo1 < hi1 && i1 <= hi1;
            const int64_t v0 = in0 ? p.cu[i0] + DOC_COST * i0 : 0;
            const int64_t v1 = in1 ? p.cu[i1] + DOC_COST * i1 : 0;
            // the samples below x form a prefix t < c; the answer is in (sample c-1, sample c]
            const int c0 = __syncthreads_count(in0 && v0 < x0);
            const int c1 = __syncthreads_count(in1 && v1 < x1);
            if (lo0 < hi0) {
                if (c0 == 0) {
                    hi0 = lo0;
                } else {
                    const int64_t up0 = lo0 + (int64_t)c0 * st0;
                    hi0 = up0 < hi0 ? (int)up0 : hi0;
                    lo0 = lo0 + (c0 - 1) * st0 + 1;
                    lo0 = lo0 > hi0 ? hi0 : lo0;
                }
            }
            if (lo1 < hi1) {
                if (c1 == 0) {
                    hi1 = lo1;
                } else {
                    const int64_t up1 = lo1 + (int64_t)c1 * st1;
                    hi1 = up1 < hi1 ? (int)up1 : hi1;
                    lo1 = lo1 + (c1 - 1) * st1 + 1;
                    lo1 = lo1 > hi1 ? hi1 : lo1;
                }
            }
        }
        bbeg = lo0;
        bend = lo1 < lo0 ? lo0 : lo1;  // only a non-monotone cu_seqlens (unsupported) could invert them
    }
    // the same in every thread: keep them (and what is derived from them) scalar
    bbeg = __builtin_amdgcn_readfirstlane(bbeg);
    bend = __builtin_amdgcn_readfirstlane(bend);
}

// Sum over lanes 0..31 of a wave, left in lanes 16..31 (and the sum over
// lanes 32..63 in lanes 48..63), by DPP.  The adds pair lanes as a butterfly
// xor 1, 2, 4, 8, 16 does.
__device__ __forceinline__ float lanes32_sum(float v) {
    v += bitsf(__builtin_amdgcn_mov_dpp(fbits(v), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    v += bitsf(__builtin_amdgcn_mov_dpp(fbits(v), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    v += bitsf(__builtin_amdgcn_mov_dpp(fbits(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
    v += bitsf(__builtin_amdgcn_mov_dpp(fbits(v), 0x140, 0xF, 0xF, false));  // row_mirror
    // row_bcast:15 into rows 1 and 3 (rows 0 and 2 keep 0)
    v += bitsf(__builtin_amdgcn_update_dpp(0u, fbits(v), 0x142, 0xA, 0xF, false));
    return v;
}

// ELEM: kF16 / kBF16 / kI8.  M: MFMA block edge (16 or 32).  QB: M-row query
// blocks per wave.  WQ x WT waves: WQ along query rows, WT along document
// tokens.  SPW: M-token sub-tiles each wave contracts per tile, NSI of them at
// a time (1 or 2).  NBUF: tile ring depth (2 or 3).  ARGMAX: also track and
// write the argmax.
template <int ELEM, int M, int QB, int WQ, int WT, int SPW, int NSI, int NBUF, bool ARGMAX, bool VARLEN>
__global__ __launch_bounds__(64 * WQ * WT) void fwd_kernel(FwdParams p) {
    using MM = Mma<ELEM, M>;
    using Acc = typename MM::Acc;
    constexpr bool I8 = ELEM == kI8;
    constexpr int NG = MM::NG, VPL = MM::VPL, KS = MM::KS;
    constexpr int NW = WQ * WT;
    constexpr int NT = 64 * NW;
    constexpr int ROWB = I8 ? 128 : 256;  // bytes per token row
    constexpr int NCH = ROWB / 16;        // 16-byte chunks per row
    static_assert(NCH == NG * KS, "each lane group covers KS chunks");
    constexpr int SUBS = SPW * WT;        // M-token sub-tiles per tile
    constexpr int TT = M * SUBS;          // tokens per tile
    constexpr int R = WQ * QB * M;        // slab capacity in query-token rows
    constexpr int RP = R + R / 32;        // padded row-maximum storage
    // fp16/bf16 with 32x32 blocks track the argmax with a packed key: the low
    // KB mantissa bits of each similarity are replaced by its position in the
    // lane (earlier positions get larger codes), so one max over the keys gives
    // both a maximum (to within 2^KB ulp) and where it sits.  The exact maximum
    // is kept separately.  int8 (bit-exact) and 16x16 blocks compare exactly.
    constexpr bool KEYED = ARGMAX && !I8 && M == 32;
    constexpr unsigned KMASK = VPL - 1;
    // int8 with one token-wave: a document's merge parks each row's term
    // v_i = fl32(m_i * q_scale_i) rather than its maximum (no later merge
    // compares maxima), so the serial per-query sums read one value per row.
    constexpr bool I8_TERMS = I8 && WT == 1;

    // Ring of NBUF tile buffers: tile k is contracted while tiles k+1 ..
    // k+NBUF-1 are in flight.
    static_assert(NBUF == 2 || NBUF == 3, "ring depth");
    constexpr int LPW = TT * NCH / (64 * NW);  // 1 KB direct loads per wave per tile
    static_assert(LPW * 64 * NW == TT * NCH, "tile must split into whole 1 KB loads per wave");
    static_assert(!I8 || TT % 64 == 0, "int8 scales load 64 at a time");
    constexpr int SCW = I8 ? TT / 64 : 0;     // waves that also load 64 scales each
    static_assert(SCW <= NW, "scale loads need enough waves");
    __shared__ u32x4 dtile[NBUF][TT * NCH];
    __shared__ __attribute__((aligned(16))) float dsc[I8 ? NBUF : 1][I8 ? TT : 4];
    // Per-document row maxima / argmax of each token-wave, double-buffered by
    // document parity: a document's rows are written at the end of its last
    // step and consumed (sums, argmax stores) at the start of the next step,
    // so the step barrier is the only one.
    __shared__ float rowmax_s[2][WT][RP];
    __shared__ int rowarg_s[ARGMAX ? 2 : 1][ARGMAX ? WT : 1][ARGMAX ? R : 1];
    __shared__ float qsc_s[I8 ? RP : 1];  // int8: the slab's query scales (row r at rpad(r))
    __shared__ int docpf[2][2];          // prefetched document bounds

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: lets branches on it stay scalar
    const int wq = wave % WQ;
    // token-wave index: a compile-time 0 for int8 with one token-wave (the
    // 16-wave argmax workgroups need it to stay within 128 VGPRs; fp16/bf16
    // measured 2-3 % slower with it, so they keep the computed value)
    const int wt = (I8 && WT == 1) ? 0 : wave / WQ;
    const int g = lane / M;    // lane group: k-chunks of the operands, token set of the result
    const int lm = lane % M;   // operand row / result column
    int aslot[KS];             // LDS slot of operand chunk s of row lm of a sub-tile
#pragma unroll
    for (int s = 0; s < KS; ++s) aslot[s] = swz<NCH>(lm, g * KS + s);
    // Operand chunk s of row lm of sub-tile sb in ring slot bf.  int8 reads it
    // at the per-lane slot plus the sub-tile's constant (30 fewer VGPRs, and
    // room for 16-wave workgroups); fp16/bf16 keep the full swizzle per read,
    // which compiles to the same reads with a schedule measured no slower.
    auto opnd = [&](int bf, int sb, int s) -> u32x4 {
        if constexpr (I8) {
            return dtile[bf][sub_slot<NCH, M>(sb, aslot[s])];
        } else {
            return dtile[bf][swz<NCH>(sb * M + lm, g * KS + s)];
        }
    };

    const int blk = blockIdx.x;
    const int xcd = blk & 7;
    const int jx = blk >> 3;
    const int slab = jx % p.num_slabs;
    const int stream = (jx / p.num_slabs) * 8 + xcd;
    if (stream >= p.num_streams || stream >= p.B) return;  // uniform over the workgroup
    int bbeg, bend, bstep;  // this stream's documents: bbeg, bbeg + bstep, ... < bend
    if (p.round_robin) {  // uniform
        bbeg = stream;
        bend = p.B;
        bstep = p.num_streams;
    } else {
        stream_range<VARLEN, NT>(p, stream, bbeg, bend);
        bstep = 1;
    }
    const int Lq = p.Lq;
    // The slab is nq queries x ni of their rows, starting at row i0 of each:
    // whole queries (i0 = 0, ni = Lq) or one half of a split query.  Its rows
    // are contiguous in Q from row q0*Lq + i0.
    int q0, nq, i0, ni;
    if (p.split == 1) {
        q0 = slab * p.qps;
        nq = min(p.qps, p.Nq - q0);
        i0 = 0;
        ni = Lq;
    } else {
        q0 = slab >> 1;
        nq = 1;
        i0 = (slab & 1) ? p.half_rows : 0;
        ni = (slab & 1) ? Lq - p.half_rows : p.half_rows;
    }
    const int nrows = nq * ni;
    const int64_t qrow0 = (int64_t)q0 * Lq + i0;

    // Query slab -> VGPRs.  Lane (g, lm) of block cb holds row (wq*QB+cb)*M+lm,
    // chunks g*KS .. g*KS+KS-1 (k-step s uses chunk g*KS + s; the document
    // operand uses the same chunk map, so every k meets its partner once).
    u32x4 bq[QB][KS];
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) {
        const int r = (wq * QB + cb) * M + lm;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (r < nrows) {
                bq[cb][s] = *reinterpret_cast<const u32x4*>(p.Q + (qrow0 + r) * ROWB + (g * KS + s) * 16);
            } else {
                bq[cb][s] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }

    if constexpr (I8) {
        for (int r = tid; r < nrows; r += NT) qsc_s[rpad(r)] = p.q_scale[qrow0 + r];
    }

    float m[QB];       // running exact maximum per lane and query block
    int code[QB];      // exact path: (global sub-tile << 4) | value slot; keyed path: sub-tile
    float km[QB];      // keyed path: running maximum key
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) {
        m[cb] = -INFINITY;
        km[cb] = -INFINITY;
        code[cb] = -1;
    }

    // Direct HBM -> LDS loads of one tile into ring slot bf.  Every loading
    // wave issues exactly LPL (+1 for the scale waves) loads, so vmcnt bookkeeping is
    // static; lanes whose token is past the document's end fetch the tile's
    // first row instead (in bounds, and a repeat of a value the maximum
    // already sees at a lower index), and the compute masks those tokens
    // where needed.  The descriptor spans the tile's valid rows only, so an
    // empty document's loads read zeros and touch no memory.
    const bool scale_wave = I8 && wave < SCW;
    // With two buffers the tile is loaded by the first wave of each SIMD
    // (waves 0 .. NW/2-1, each twice the even share), and the second wave
    // issues none: issuing a tile's direct loads stalls a wave for about 1000
    // cycles, and when both waves of a SIMD stalled together the matrix pipe
    // stood idle.  The step barrier orders the tile for the waves that read it
    // without having loaded it.
    constexpr bool SPLIT_LOADS = NBUF == 2 && NW == 8;
    constexpr int LW = SPLIT_LOADS ? NW / 2 : NW;  // loading waves
    constexpr int LPL = TT * NCH / (64 * LW);      // 1 KB loads per loading wave per tile
    static_assert(LPL * 64 * LW == TT * NCH, "tile must split into whole 1 KB loads per loading wave");
    static_assert(!I8 || SCW <= LW, "the scale waves are loading waves");
    const bool loader = wave < LW;
    auto issue_tile = [&](int bf, int64_t st, int ln, int tt) {
        if (!loader) return;  // uniform
        const int64_t t0 = st + (int64_t)tt * TT;  // the tile's first row
        int nv = ln - tt * TT;                     // its valid rows
        nv = nv < 0 ? 0 : (nv > TT ? TT : nv);
#pragma unroll
        for (int u = 0; u < LPL; ++u) {
            const int slot0 = (u * LW + wave) * 64;
            const int sl = slot0 + lane;
            const int row = sl / NCH;
            const int c = swz_chunk<NCH>(row, sl % NCH);
            const uint32_t r = row < nv ? row : 0;
            buffer_load_lds(p.D + t0 * ROWB, (uint32_t)nv * ROWB, r * ROWB + c * 16, (lptr_t)&dtile[bf][slot0], 16);
        }
        if constexpr (I8) {
            if (scale_wave) {
                const int row = wave * 64 + lane;
                const uint32_t r = row < nv ? row : 0;
                buffer_load_lds(p.d_scale + t0, (uint32_t)nv * 4, r * 4, (lptr_t)&dsc[bf][wave * 64], 4);
            }
        }
    };
    // End of a step: wait until the next tile has landed.  Vector-memory
    // operations complete in issue order, so allowing only the loads of the
    // NBUF-2 newest tiles to remain retires every older load and store.
    auto wait_next_tile = [&]() {
        if constexpr (NBUF == 2) {
            wait_vmcnt<0>();
        } else if (scale_wave) {
            wait_vmcnt<LPL + 1>();
        } else {
            wait_vmcnt<LPL>();
        }
    };

    // NS consecutive M-token sub-tiles (starting at sb0) against the wave's QB
    // query blocks; their NS*QB accumulation chains are interleaved so the
    // matrix pipe always has independent work.  MASK: some tokens of these
    // sub-tiles lie past the document's end (only the last sub-tiles).  Query
    // rows past the slab's end hold zeros; their results are never read.
    auto subtiles = [&](auto ns_tag, auto mask_tag, int bf, int sb0, int tok0, int ln, int gsub0) {
        constexpr int NS = decltype(ns_tag)::value;
        constexpr bool MASK = decltype(mask_tag)::value;
        static_assert(!I8, "int8 always takes the pipelined path");
        float v[NS][QB][VPL];
        {
            Acc acc[NS][QB];
#pragma unroll
            for (int n = 0; n < NS; ++n)
#pragma unroll
                for (int cb = 0; cb < QB; ++cb) acc[n][cb] = MM::zero();
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                u32x4 a[NS];
#pragma unroll
                for (int n = 0; n < NS; ++n) a[n] = opnd(bf, sb0 + n, s);
#pragma unroll
                for (int cb = 0; cb < QB; ++cb)
#pragma unroll
                    for (int n = 0; n < NS; ++n) acc[n][cb] = MM::mma(a[n], bq[cb][s], acc[n][cb]);
            }
#pragma unroll
            for (int n = 0; n < NS; ++n)
#pragma unroll
                for (int cb = 0; cb < QB; ++cb)
#pragma unroll
                    for (int i = 0; i < VPL; ++i) v[n][cb][i] = acc[n][cb][i];
        }
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const int tk0 = tok0 + n * M;
            const int gsub = gsub0 + n;
#pragma unroll
            for (int cb = 0; cb < QB; ++cb) {
                bool valid[VPL];
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    valid[i] = !MASK || (tk0 + MM::tok(g, i) < ln);
                    if (!valid[i]) v[n][cb][i] = -INFINITY;
                }
                if constexpr (KEYED) {
                    float mx = m[cb];
#pragma unroll
                    for (int i = 0; i < VPL; ++i) mx = fmaxf(mx, v[n][cb][i]);
                    m[cb] = mx;
                    float kt = -INFINITY;
#pragma unroll
                    for (int i = 0; i < VPL; ++i) {
                        const unsigned key = (fbits(v[n][cb][i]) & ~KMASK) | (KMASK - i);
                        kt = fmaxf(kt, valid[i] ? bitsf(key) : -INFINITY);
                    }
                    if (kt > km[cb]) {  // strict: the earlier sub-tile keeps a tie
                        km[cb] = kt;
                        code[cb] = gsub;
                    }
                } else if constexpr (ARGMAX) {
#pragma unroll
                    for (int i = 0; i < VPL; ++i) {
                        if (v[n][cb][i] > m[cb]) {  // strict: the earliest token keeps a tie
                            m[cb] = v[n][cb][i];
                            code[cb] = (gsub << 4) | i;
                        }
                    }
                } else {
                    float mx = m[cb];
#pragma unroll
                    for (int i = 0; i < VPL; ++i) mx = fmaxf(mx, v[n][cb][i]);
                    m[cb] = mx;
                }
            }
        }
    };

    // fp16/bf16 with 32x32 blocks: the sub-tiles of a tile run as a software
    // pipeline.  Stage j issues sub-tile j's MFMA chains (one per query block)
    // while the VALU folds sub-tile j-1's results into the running maximum
    // (and argmax key).  The two touch disjoint registers, and the scheduling
    // hints below interleave them, so the matrix pipe and the VALU work side
    // by side within one wave instead of taking turns.
    // Per k-step the stage issues one MFMA per query block and folds VPL/KS
    // values of each of the previous stage's blocks (a fixed, hand-interleaved
    // order; the scheduling barrier keeps the compiler from regrouping it).
    //
    // int8 values are the exact products fl32(float(dot) * d_scale[token]),
    // formed by one fused multiply-add instead of a convert and a multiply.
    // Each accumulator starts at the integer 0x4B000000, the bits of the
    // float 2^23, so after the contraction (|dot| <= 128 * 127^2 < 2^21) its
    // bits read as the float 2^23 + dot when dot >= 0 and 2^23 + dot/2 when
    // dot < 0 (the binade below 2^23 has half the spacing).  fma(that, s,
    // -2^23 * s) has an exact addend (a power of two times s) and rounds once,
    // to fl32(dot * s), or to fl32(dot * s) / 2 for negative dot, which is
    // exact while d_scale >= 2^-125.  Halving every negative value keeps all
    // orders and ties (the sign is unchanged and all negatives scale alike),
    // so the running maxima and argmax are those of the exact values, and a
    // negative row maximum is doubled back (exactly) before the query scale.
    static_assert(VPL % KS == 0, "fold parts");
    constexpr int FPS = VPL / KS;  // values folded per block per k-step
    auto stage_scales = [&](int bf, int sb) {
        if constexpr (I8) {
            return *reinterpret_cast<const f32x4*>(&dsc[bf][sb * M + 4 * g]);
        } else {
            return f32x4{1.f, 1.f, 1.f, 1.f};
        }
    };
    auto acc_start = [&]() -> Acc {
        if constexpr (I8) {
            return Acc{0x4B000000, 0x4B000000, 0x4B000000, 0x4B000000};
        } else {
            return MM::zero();
        }
    };
    auto value = [&](const Acc& acc, int i, const f32x4& sc) -> float {
        if constexpr (I8) {
            return __builtin_fmaf(__int_as_float(acc[i]), sc[i], -(sc[i] * 8388608.0f));
        } else {
            return acc[i];
        }
    };
    // fold value v at slot i of block cb from global sub-tile gsub (unmasked)
    auto fold_value = [&](int cb, float v, int i, int gsub, float& kt) {
        if constexpr (KEYED) {
            m[cb] = fmaxf(m[cb], v);
            kt = fmaxf(kt, bitsf((fbits(v) & ~KMASK) | (KMASK - i)));
        } else if constexpr (ARGMAX) {
            const bool upd = v > m[cb];  // strict: the earliest token keeps a tie
            m[cb] = upd ? v : m[cb];
            code[cb] = upd ? ((gsub << 4) | i) : code[cb];
        } else {
            m[cb] = fmaxf(m[cb], v);
        }
    };
    auto stage = [&](int bf, int sb, Acc* cur, const Acc* prev, const f32x4& sc_prev, bool has_prev, int gprev) {
        u32x4 a[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) a[s] = opnd(bf, sb, s);
#pragma unroll
        for (int cb = 0; cb < QB; ++cb) cur[cb] = acc_start();
        float kt[QB];
#pragma unroll
        for (int cb = 0; cb < QB; ++cb) kt[cb] = -INFINITY;
        // Raised issue priority while the stage's MFMA / fold interleave runs:
        // the other wave of the SIMD, in its epilogue, boundary folds or load
        // issue, then takes the slots the matrix pipe leaves (INT8 -4 %,
        // others 0.5-1 %).
        __builtin_amdgcn_s_setprio(1);
        // fp16/bf16: each block's fold follows its own MFMA (ColPali and the
        // training forward 1.6-1.9 % faster); int8, VALU-bound, keeps the
        // k-step's MFMAs together and its folds after them (8 % faster so).
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if constexpr (I8) {
#pragma unroll
                for (int cb = 0; cb < QB; ++cb) cur[cb] = MM::mma(a[s], bq[cb][s], cur[cb]);
                if (has_prev) {  // uniform
#pragma unroll
                    for (int cb = 0; cb < QB; ++cb)
#pragma unroll
                        for (int f = 0; f < FPS; ++f) {
                            const int i = s * FPS + f;
                            fold_value(cb, value(prev[cb], i, sc_prev), i, gprev, kt[cb]);
                        }
                }
                __builtin_amdgcn_sched_barrier(0);
            } else {
#pragma unroll
                for (int cb = 0; cb < QB; ++cb) {
                    cur[cb] = MM::mma(a[s], bq[cb][s], cur[cb]);
                    if (has_prev) {  // uniform
#pragma unroll
                        for (int f = 0; f < FPS; ++f) {
                            const int i = s * FPS + f;
                            fold_value(cb, value(prev[cb], i, sc_prev), i, gprev, kt[cb]);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
        if constexpr (KEYED) {
            if (has_prev) {
#pragma unroll
                for (int cb = 0; cb < QB; ++cb) {
                    const bool upd = kt[cb] > km[cb];  // strict: the earlier sub-tile keeps a tie
                    km[cb] = upd ? kt[cb] : km[cb];
                    code[cb] = upd ? gprev : code[cb];
                }
            }
        }
    };
    // Fold a whole block of results (the last stage of a tile, which can be
    // partial: tokens at or past ln are -inf and never win).
    auto fold = [&](auto mask_tag, const Acc* acc, const f32x4& sc, int tok0, int ln, int gsub) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int cb = 0; cb < QB; ++cb) {
            float kt = -INFINITY;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const bool valid = !MASK || (tok0 + MM::tok(g, i) < ln);
                const float v = valid ? value(acc[cb], i, sc) : -INFINITY;
                if constexpr (KEYED) {
                    m[cb] = fmaxf(m[cb], v);
                    kt = fmaxf(kt, valid ? bitsf((fbits(v) & ~KMASK) | (KMASK - i)) : -INFINITY);
                } else {
                    fold_value(cb, v, i, gsub, kt);
                }
            }
            if constexpr (KEYED) {
                const bool upd = kt > km[cb];  // strict: the earlier sub-tile keeps a tie
                km[cb] = upd ? kt : km[cb];
                code[cb] = upd ? gsub : code[cb];
            }
        }
    };
    // Ping-pong accumulators (even / odd stages) and their int8 token scales.
    // They live across steps: when a tile is full and its document goes on
    // in the next tile, its last sub-tile is not drained at the end of the
    // step but folded by the next step's first stage, between its MFMAs (SPW
    // is even, so that sub-tile sits in acc1 as a stage-(-1) result would).
    // (fp16/bf16 only: the int8 path measured no faster with it.)
    Acc acc0[QB], acc1[QB];
    f32x4 sc0, sc1;
    bool carry = false;  // acc1 / sc1 hold the unfolded last sub-tile of the previous tile
    auto compute_tile_pipe = [&](int bf, int tt, int ln, bool last_tile) {
        if (wq * QB * M >= nrows) return;  // uniform: this wave's rows are all past the slab
        const int tok_w = tt * TT + wt * SPW * M;  // first token of this wave's sub-tiles
        int nsub = (ln - tok_w + M - 1) / M;       // sub-tiles holding at least one valid token
        nsub = nsub < 0 ? 0 : (nsub > SPW ? SPW : nsub);
        const bool carried = carry;
        carry = false;
        // stages are expanded at compile time so every accumulator index is static
        static_for<SPW>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if (j >= nsub) return;  // uniform
            Acc* cur = (j & 1) ? acc1 : acc0;
            const Acc* prev = (j & 1) ? acc0 : acc1;
            f32x4& sc_cur = (j & 1) ? sc1 : sc0;
            const f32x4& sc_prev = (j & 1) ? sc0 : sc1;
            const int sb = wt * SPW + j;
            const int gsub = tt * SUBS + sb;
            sc_cur = stage_scales(bf, sb);
            // with one token-wave the previous tile's last sub-tile is gsub - 1 too
            stage(bf, sb, cur, prev, sc_prev, j > 0 || carried, gsub - 1);
            if (!I8 && WT == 1 && SPW % 2 == 0 && j == SPW - 1 && !last_tile) {
                carry = true;  // full tile, the document goes on: the next step folds it
            } else if (j == nsub - 1) {  // drain: fold the last sub-tile (the only one that can be partial)
                // Rows past the document's end were loaded as copies of the
                // tile's first row (issue_tile), so their values repeat that token's
                // under a later index: they change no maximum, and with the
                // strict in-lane update and the lower-index merge they never
                // win an exact argmax either.  Only the keyed argmax, which
                // ranks values within 2^KB ulp by slot, must mask them.
                const int tok0 = tok_w + j * M;
                if (KEYED && tok0 + M > ln) {
                    fold(std::true_type{}, cur, sc_cur, tok0, ln, gsub);
                } else {
                    fold(std::false_type{}, cur, sc_cur, tok0, ln, gsub);
                }
            }
        });
    };

    auto compute_tile = [&](int bf, int tt, int ln, bool last_tile) {
        if constexpr ((!I8 && M == 32 && QB <= 2) || I8) {  // two stages of accumulators fit in registers
            compute_tile_pipe(bf, tt, ln, last_tile);
        } else {
            if (wq * QB * M >= nrows) return;  // uniform: this wave's rows are all past the slab
            const int tok_w = tt * TT + wt * SPW * M;  // first token of this wave's sub-tiles
            int nsub = (ln - tok_w + M - 1) / M;       // sub-tiles holding at least one valid token
            nsub = nsub < 0 ? 0 : (nsub > SPW ? SPW : nsub);
#pragma unroll
            for (int k = 0; k < SPW; k += NSI) {
                if (k >= nsub) break;  // uniform
                const int sb = wt * SPW + k;
                const int tok0 = tok_w + k * M;
                const int gsub = tt * SUBS + sb;
                if (NSI == 2 && k + 1 < nsub) {
                    if (tok0 + 2 * M <= ln) {
                        subtiles(std::integral_constant<int, 2>{}, std::false_type{}, bf, sb, tok0, ln, gsub);
                    } else {
                        subtiles(std::integral_constant<int, 2>{}, std::true_type{}, bf, sb, tok0, ln, gsub);
                    }
                } else {
                    if (tok0 + M <= ln) {
                        subtiles(std::integral_constant<int, 1>{}, std::false_type{}, bf, sb, tok0, ln, gsub);
                    } else {
                        subtiles(std::integral_constant<int, 1>{}, std::true_type{}, bf, sb, tok0, ln, gsub);
                    }
                }
            }
        }
    };

    // 32-token queries in 32x32 blocks (the common ColBERT shape): block cb of a
    // wave is exactly one query, so once its rows are merged the score is the
    // sum over lanes 0..31, formed in registers with DPP (no LDS round trip
    // and nothing left for after the barrier).  lanes32_sum pairs lanes as the
    // butterfly of the general path does, so the result is the same.
    const bool wave_sums = !I8 && M == 32 && Lq == 32 && p.split == 1;

    // End of a document, part 1 (before the step barrier): merge the NG token
    // sets of every query row (lanes lm + M*g) and park the row results.
    // int8 terms with 16-row blocks: after the merge every 16-lane group
    // holds every block's merged maxima, so group g forms and stores the
    // terms of block j + g, four blocks per pass instead of one.
    constexpr bool SPREAD = I8_TERMS && M == 16 && QB % 4 == 0;
    auto epilogue_merge = [&](int par, int b) {
        float mvs[SPREAD ? QB : 1];
        int ids[SPREAD ? QB : 1];
#pragma unroll
        for (int cb = 0; cb < QB; ++cb) {
            float mv = m[cb];
            int idx = -1;
            if constexpr (KEYED) {
                if (code[cb] >= 0) {
                    const int i = (int)(KMASK - (fbits(km[cb]) & KMASK));
                    idx = M * code[cb] + MM::tok(g, i);
                }
            } else if constexpr (ARGMAX) {
                if (code[cb] >= 0) idx = M * (code[cb] >> 4) + MM::tok(g, code[cb] & 15);
            }
#pragma unroll
            for (int off = M; off < 64; off <<= 1) {
                // off 16 through v_permlane16_swap where it measured faster (one
                // token-wave: int8 1-5 %; with four token-waves 12 % slower)
                const bool x16 = WT == 1 && off == 16;
                if constexpr (ARGMAX) {
                    if (off == 32 || x16) {
                        // the larger value, then the lowest index (unsigned:
                        // -1, no candidate, loses) among the lanes holding it
                        const float mx = off == 32 ? xor32_max(mv) : xor16_max(mv);
                        const unsigned c = mv == mx ? (unsigned)idx : 0xFFFFFFFFu;
                        idx = (int)(off == 32 ? xor32_min_u(c) : xor16_min_u(c));
                        mv = mx;
                    } else {
                        const float om = __shfl_xor(mv, off);
                        const int oi = __shfl_xor(idx, off);
                        if (om > mv || (om == mv && (unsigned)oi < (unsigned)idx)) {
                            mv = om;
                            idx = oi;
                        }
                    }
                } else {
                    mv = off == 32 ? xor32_max(mv) : x16 ? xor16_max(mv) : fmaxf(mv, __shfl_xor(mv, off));
                }
            }
            const int r = (wq * QB + cb) * M + lm;
            if constexpr (SPREAD) {
                mvs[cb] = mv;
                ids[cb] = idx;
            } else if (g == 0 && (ARGMAX || !wave_sums)) {  // row maxima for the general sum or the argmax merge
                if constexpr (I8_TERMS) {
                    // v_i = fl32(m_i * q_scale_i) right away (a negative maximum was held halved)
                    rowmax_s[par][0][rpad(r)] = (mv < 0.f ? mv + mv : mv) * qsc_s[rpad(r)];
                } else {
                    rowmax_s[par][wt][rpad(r)] = mv;
                }
                if constexpr (ARGMAX) rowarg_s[par][wt][r] = idx;
            }
            if constexpr (!I8 && M == 32 && WT == 1) {
                if (wave_sums) {  // uniform
                    const float sc = lanes32_sum(mv);
                    const int ql = wq * QB + cb;
                    if (lane == 31 && ql < nq) p.scores[(int64_t)(q0 + ql) * p.B + b] = sc;
                }
            }
            m[cb] = -INFINITY;
            km[cb] = -INFINITY;
            code[cb] = -1;
        }
        if constexpr (SPREAD) {
#pragma unroll
            for (int j = 0; j < QB; j += 4) {
                float v = mvs[j];
                int id = ids[j];
#pragma unroll
                for (int u = 1; u < 4; ++u) {
                    if (g == u) {
                        v = mvs[j + u];
                        id = ids[j + u];
                    }
                }
                const int r = (wq * QB + j + g) * M + lm;
                // v_i = fl32(m_i * q_scale_i) (a negative maximum was held halved)
                rowmax_s[par][0][rpad(r)] = (v < 0.f ? v + v : v) * qsc_s[rpad(r)];
                if constexpr (ARGMAX) rowarg_s[par][wt][r] = id;
            }
        }
    };
    // Row r's maximum / argmax over the token-waves (ties: lower index).
    auto row_max = [&](int par, int r) {
        float mv = rowmax_s[par][0][rpad(r)];
#pragma unroll
        for (int w = 1; w < WT; ++w) mv = fmaxf(mv, rowmax_s[par][w][rpad(r)]);
        if constexpr (I8) mv = mv < 0.f ? mv + mv : mv;  // a negative int8 maximum was held halved
        return mv;
    };
    auto row_arg = [&](int par, int r) {
        float mv = rowmax_s[par][0][rpad(r)];
        int idx = rowarg_s[par][0][r];
#pragma unroll
        for (int w = 1; w < WT; ++w) {
            const float om = rowmax_s[par][w][rpad(r)];
            const int oi = rowarg_s[par][w][r];
            if (om > mv || (om == mv && (unsigned)oi < (unsigned)idx)) {
                mv = om;
                idx = oi;
            }
        }
        return idx;
    };
    // int8 term v_i of row r (in ascending i these form the exact score)
    auto row_term = [&](int par, int r) -> float {
        if constexpr (I8_TERMS) {
            return rowmax_s[par][0][rpad(r)];
        } else {
            return row_max(par, r) * qsc_s[rpad(r)];
        }
    };
    // End of a document, part 2 (after the step barrier): argmax stores and
    // the per-query sums of the row maxima.
    auto epilogue_out = [&](int b, int par) {
        if constexpr (ARGMAX) {
            // r = ql * ni + i; r, ni < 2^11, so the float quotient floors exactly
            const float inv_ni = 1.0f / (float)ni;
            for (int r = tid; r < nrows; r += NT) {
                const int ql = (int)(((float)r + 0.5f) * inv_ni);
                const int i = i0 + r - ql * ni;
                p.argmax[((int64_t)(q0 + ql) * p.B + b) * Lq + i] = row_arg(par, r);
            }
        }
        if constexpr (I8) {
            // Exact epilogue: score = ((v_0 + v_1) + v_2) + ... in fp32, a
            // serial chain per query, run at raised wave priority (it sits on
            // the step's critical path; at the stages' priority the waves in
            // their contraction left it few issue slots: 2-7 % slower).
            __builtin_amdgcn_s_setprio(2);
            if (R >= 64 && ni >= 64) {
                // Long queries: a wave per query reads 64 consecutive terms at
                // once and adds them in order through readlane (lanes past the
                // query add +0, which changes no sum that starts at +0).
                for (int ql = (wave + NW - 1) % NW; ql < nq; ql += NW) {  // uniform per wave
                    const int r0 = ql * ni;
                    float acc = 0.f;
                    for (int c = 0; c < ni; c += 64) {
                        const float t = c + lane < ni ? row_term(par, r0 + c + lane) : 0.f;
#pragma unroll
                        for (int k = 0; k < 64; ++k) acc = acc + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), k));
                    }
                    if (lane == 0) p.scores[(int64_t)(q0 + ql) * p.B + b] = acc;
                }
            } else {
                // A thread per query, on the second wave first (measured
                // faster; the 16-wave argmax kernel excepted), the next 8 rows
                // read while the current 8 are added.  With the argmax the
                // plain loop: at the 128-VGPR limit the read-ahead would spill.
                constexpr bool FIRST_WAVE = ARGMAX && NW == 16;
                for (int ql = FIRST_WAVE ? tid : (tid + NT - (NW > 1 ? 64 : 0)) % NT; ql < nq; ql += NT) {
                    const int r0 = ql * ni;
                    float acc = 0.f;
                    int i = 0;
                    if (I8_TERMS && (ni & 7) == 0) {  // uniform
                        // Groups of 8 rows start at multiples of 8, so none
                        // crosses a 32-row pad step: one address per group
                        // and immediate offsets.  Scores only: the next
                        // group is read while the current one is added.
                        const int ng = ni >> 3;
                        auto ld = [&](float(&v)[8], int gi) {
                            const float* t = &rowmax_s[par][0][rpad(r0 + 8 * gi)];
#pragma unroll
                            for (int k = 0; k < 8; ++k) v[k] = t[k];
                        };
                        auto add = [&](const float(&v)[8]) {
#pragma unroll
                            for (int k = 0; k < 8; ++k) acc = acc + v[k];
                        };
                        float x[8], y[8];
                        if constexpr (ARGMAX) {
                            for (int gi = 0; gi < ng; ++gi) {
                                ld(x, gi);
                                add(x);
                            }
                        } else {
                            ld(x, 0);
                            int gi = 1;
                            for (; gi + 1 < ng; gi += 2) {
                                ld(y, gi);
                                add(x);
                                ld(x, gi + 1);
                                add(y);
                            }
                            if (gi < ng) {
                                ld(y, gi);
                                add(x);
                                add(y);
                            } else {
                                add(x);
                            }
                        }
                        i = ni;
                    } else if (!ARGMAX && ni >= 16) {
                        float cur[8], nxt[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k) cur[k] = row_term(par, r0 + k);
                        for (i = 8; i + 8 <= ni; i += 8) {
#pragma unroll
                            for (int k = 0; k < 8; ++k) nxt[k] = row_term(par, r0 + i + k);
#pragma unroll
                            for (int k = 0; k < 8; ++k) acc = acc + cur[k];
#pragma unroll
                            for (int k = 0; k < 8; ++k) cur[k] = nxt[k];
                        }
#pragma unroll
                        for (int k = 0; k < 8; ++k) acc = acc + cur[k];  // rows i-8 .. i-1
                    }
                    for (; i < ni; ++i) acc = acc + row_term(par, r0 + i);
                    p.scores[(int64_t)(q0 + ql) * p.B + b] = acc;
                }
            }
            __builtin_amdgcn_s_setprio(0);
        } else {
            // P lanes per query (P = ni rounded up to a power of two, at most 64),
            // 64 / P queries per wave pass, butterfly sum inside each lane group.
            // A split query's two halves each add their partial sum to the
            // zero-filled score: two addends, so the result does not depend on
            // which lands first.
            if (WT == 1 && wave_sums) return;  // summed in registers by epilogue_merge
            int P = 1;
            while (P < ni && P < 64) P <<= 1;
            const int qpw = 64 / P;
            const int sub = lane / P, pl = lane % P;
            for (int ql0 = wave * qpw; ql0 < nq; ql0 += NW * qpw) {
                const int ql = ql0 + sub;
                float acc = 0.f;
                if (ql < nq)
                    for (int i = pl; i < ni; i += P) acc += row_max(par, ql * ni + i);
#pragma unroll
                for (int off = 1; off < 64; off <<= 1)
                    if (off < P) acc += __shfl_xor(acc, off);  // uniform guard, constant lane offsets
                if (pl == 0 && ql < nq) {
                    float* dst = p.scores + (int64_t)(q0 + ql) * p.B + b;
                    if (p.split == 1) {
                        *dst = acc;
                    } else {
                        atomicAdd(dst, acc);
                    }
                }
            }
        }
    };

    // Persistent walk over this workgroup's documents, one tile per step, with
    // a look-ahead of two tiles (possibly in later documents).
    struct Cur {
        int b, t, len, ntiles;
        int64_t start;
    };
    auto at_doc = [&](int b) {
        Cur c;
        c.b = b;
        c.t = 0;
        c.start = 0;
        c.len = 0;
        c.ntiles = 0;
        if (b < bend) {
            doc_info<VARLEN>(p, b, c.start, c.len);
            c.ntiles = (c.len + TT - 1) / TT;
        }
        return c;
    };
    // Inside the loop the bounds of the next document travel like tile data:
    // one wave DMAs them (two lanes) into an LDS slot just before issuing a
    // step's tile loads, the step-end wait retires them, and after the barrier
    // every wave reads them from LDS.  No scalar-memory load (whose counter is
    // shared with LDS and returns out of order) and no vector load into
    // registers sits in the loop.  Slot k&1 is written at the end of step k and
    // read at the start of step k+1.
    // (a loading wave when some waves skip the step-end wait: its wait retires the prefetch)
    constexpr bool LATE = I8 && SPLIT_LOADS;
    const bool doc_wave = wave == (LATE ? 0 : NW - 1);
    auto prefetch_doc = [&](int slot, int b) {
        if (doc_wave && b < bend && lane < 2) {
            if constexpr (VARLEN) {
                buffer_load_lds(p.cu + b, 8, lane * 4, (lptr_t)&docpf[slot][0], 4);
            } else if (p.lens) {
                buffer_load_lds(p.lens + b, 4, 0, (lptr_t)&docpf[slot][0], 4);
            }
        }
    };
    auto from_prefetch = [&](int slot, int b) {
        Cur c;
        c.b = b;
        c.t = 0;
        c.start = 0;
        c.len = 0;
        c.ntiles = 0;
        if (b < bend) {
            const int v0 = (VARLEN || p.lens) ? docpf[slot][0] : p.Ld;
            if constexpr (VARLEN) {
                const int v1 = docpf[slot][1];
                int64_t s0 = v0, s1 = v1;
                s0 = s0 < 0 ? 0 : (s0 > p.T ? p.T : s0);
                s1 = s1 < s0 ? s0 : (s1 > p.T ? p.T : s1);
                c.start = s0;
                c.len = (int)(s1 - s0);
            } else {
                c.start = (int64_t)b * p.Ld;
                c.len = v0 < 0 ? 0 : (v0 > p.Ld ? p.Ld : v0);
            }
            c.ntiles = (c.len + TT - 1) / TT;
        }
        return c;
    };
    auto advance = [&](int slot, const Cur& c) {  // the next step; a new document comes from the prefetch
        if (c.t + 1 < c.ntiles) {
            Cur n = c;
            n.t += 1;
            return n;
        }
        return from_prefetch(slot, c.b + bstep);
    };
    // nothing to read at all: every document is empty and D may be absent
    const bool loads = p.T > 0;

    // cs[0] is the tile contracted in this step, cs[j] the one j steps later.
    // The prologue issues tiles 0 .. NBUF-1 (every buffer); at the top of
    // step k >= 1, cs[NBUF-1] = tile k+NBUF-1 goes into the buffer that step
    // k-1 freed.  So at any time the next NBUF-1 tiles are in flight or landed.
    Cur cs[NBUF];
    cs[0] = at_doc(bbeg);
    static_for<NBUF - 1>([&](auto jc) {
        constexpr int j = decltype(jc)::value + 1;
        cs[j] = cs[j - 1];
        if (cs[j].t + 1 < cs[j].ntiles) {
            cs[j].t += 1;
        } else {
            cs[j] = at_doc(cs[j - 1].b + bstep);
        }
    });
    prefetch_doc(1, cs[NBUF - 1].b + bstep);
    if (loads) {
        static_for<NBUF>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if (cs[j].b < bend) issue_tile(j, cs[j].start, cs[j].len, cs[j].t);
        });
        // tile 0 has landed once only the loads of tiles 1 .. NBUF-1 may remain;
        // when the stream ends earlier, fewer were issued: wait for all
        if (cs[NBUF - 1].b < bend) {
            if (scale_wave) {
                wait_vmcnt<(NBUF - 1) * (LPL + 1)>();
            } else if (loader) {
                wait_vmcnt<(NBUF - 1) * LPL>();
            } else {
                wait_vmcnt<0>();
            }
        } else {
            wait_vmcnt<0>();
        }
    }
    lds_barrier();
    int buf = 0;          // ring slot of cs[0]
    int step = 0;
    int par = 0;          // parity of the next document to finish
    int pend = -1;        // document whose outputs are parked in rowmax_s[par ^ 1]
    bool hasn = cs[NBUF - 1].b < bend;  // the newest tile (cs[NBUF-1]) exists
    // int8 with split loads: the waves that issue no tile loads run a step's
    // bookkeeping (the next tile's descriptor, the previous document's
    // stores) after their contraction rather than before it, so each SIMD's
    // matrix pipe has a wave to feed it from the step's start; issuing no
    // loads, they need no wait for the next tile either (int8 scores -1.3 %;
    // fp16/bf16 measured 0.4-0.7 % slower with it and keep the plain order).
    const bool late = LATE && !loader;  // uniform
    auto next_tile = [&]() {
        const bool hasl = cs[NBUF - 2].b < bend;
        cs[NBUF - 1] = hasl ? advance(step & 1, cs[NBUF - 2]) : cs[NBUF - 2];
        hasn = hasl && cs[NBUF - 1].b < bend;
    };
    while (true) {
        const bool has0 = cs[0].b < bend;
        if (!late && pend >= 0) {  // stores first: they must be older than this step's loads
            epilogue_out(pend, par ^ 1);
            pend = -1;
        }
        if (step > 0 && !late) {
            next_tile();
            if (hasn) prefetch_doc((step + 1) & 1, cs[NBUF - 1].b + bstep);
            if (loads && hasn) {
                const int nb = buf + NBUF - 1;
                issue_tile(nb >= NBUF ? nb - NBUF : nb, cs[NBUF - 1].start, cs[NBUF - 1].len, cs[NBUF - 1].t);
            }
        }
        if (!has0) {  // nothing issued or pending past here (has0 false => hasn false)
            if (pend >= 0) epilogue_out(pend, par ^ 1);  // a late wave's last document
            break;
        }
        if (cs[0].t < cs[0].ntiles) compute_tile(buf, cs[0].t, cs[0].len, cs[0].t + 1 >= cs[0].ntiles);
        if (late) {
            if (pend >= 0) {
                epilogue_out(pend, par ^ 1);
                pend = -1;
            }
            if (step > 0) next_tile();
        }
        if (cs[0].t + 1 >= cs[0].ntiles) {
            epilogue_merge(par, cs[0].b);
            pend = cs[0].b;
            par ^= 1;
        }
        if (loads && !late) {
            if (hasn) {
                wait_next_tile();
            } else {
                wait_vmcnt<0>();  // no newer tile: everything outstanding must land
            }
        }
        lds_barrier();
        buf = buf == NBUF - 1 ? 0 : buf + 1;
        ++step;
        static_for<NBUF - 1>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            cs[j] = cs[j + 1];
        });
    }
}

// Packed corpus, 32-token queries, scores only (the ColBERT re-ranking
// shape).  A document's epilogue then needs nothing outside the wave (each
// 32x32 block of a wave is one query: lane merge, DPP sum, one store), so a
// stream reads its contiguous packed token range [cu[bbeg], cu[bend]) as full
// 256-token tiles that run across document boundaries, and the fold splits a
// sub-tile's values where a document ends.  Against tiles aligned to
// documents this drops the partial last sub-tile of every document (about a
// tenth of the MFMA work at 32..300-token documents) and about half of the
// steps with their barriers.  Every maximum and the DPP sum are the same as
// fwd_kernel's, so the scores are bit-identical to it.
template <int ELEM>
__global__ __launch_bounds__(512) void fwd_flat_kernel(FwdParams p) {
    using MM = Mma<ELEM, 32>;
    using Acc = typename MM::Acc;
    constexpr int M = 32, QB = 2, NW = 8, NT = 64 * NW, SPW = 8, TT = M * SPW, NCH = 16;
    constexpr int KS = MM::KS, VPL = MM::VPL, FPS = VPL / KS;
    constexpr int LPW = TT * NCH / NT;  // 1 KB direct loads per wave per tile
    static_assert(LPW * NT == TT * NCH, "tile must split into whole 1 KB loads per wave");
    static_assert(SPW % 2 == 0, "a carried sub-tile sits in acc1");
    constexpr int DCAP = 4096;  // document ends kept in LDS
    __shared__ u32x4 dtile[2][TT * NCH];
    __shared__ int dend_s[DCAP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane / M, lm = lane % M;
    const int blk = blockIdx.x;
    const int xcd = blk & 7;
    const int jx = blk >> 3;
    const int slab = jx % p.num_slabs;
    const int stream = (jx / p.num_slabs) * 8 + xcd;
    if (stream >= p.num_streams || stream >= p.B) return;  // uniform over the workgroup
    int bbeg, bend;
    stream_range<true, NT>(p, stream, bbeg, bend);
    const int q0 = slab * p.qps;
    const int nq = min(p.qps, p.Nq - q0);
    const int nrows = nq * M;
    const int64_t qrow0 = (int64_t)q0 * M;

    u32x4 bq[QB][KS];  // the wave's 64 query rows, as in fwd_kernel
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) {
        const int r = (wave * QB + cb) * M + lm;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bq[cb][s] = r < nrows ? *reinterpret_cast<const u32x4*>(p.Q + (qrow0 + r) * 256 + (g * KS + s) * 16)
                                  : u32x4{0u, 0u, 0u, 0u};
        }
    }

    const cint_ptr cu = (cint_ptr)p.cu;
    auto clamp_t = [&](int64_t v) -> int64_t { return v < 0 ? 0 : (v > p.T ? p.T : v); };
    const int64_t T0 = clamp_t(cu[bbeg]);
    int64_t T1 = clamp_t(cu[bend]);
    T1 = T1 < T0 ? T0 : T1;
    const int ntile = (int)((T1 - T0 + TT - 1) / TT);

    // Tile k: tokens T0 + k*TT ... (past T1: the tile's first row again, in bounds, never folded;
    // past the end of D: zeros, no access).
    // Loaded by the first wave of each SIMD, as in fwd_kernel.
    constexpr int LW = NW / 2, LPL = 2 * LPW;
    const bool loader = wave < LW;
    auto issue_tile = [&](int bf, int k) {
        const int64_t st = T0 + (int64_t)k * TT;
        const int64_t ln = T1 - st;
        if (!loader) return;  // uniform
        const int nv = ln < 0 ? 0 : (ln > TT ? TT : (int)ln);
#pragma unroll
        for (int u = 0; u < LPL; ++u) {
            const int slot0 = (u * LW + wave) * 64;
            const int sl = slot0 + lane;
            const int row = sl / NCH;
            const int c = swz_chunk<NCH>(row, sl % NCH);
            const uint32_t r = row < nv ? row : 0;
            buffer_load_lds(p.D + st * 256, (uint32_t)nv * 256, r * 256 + c * 16, (lptr_t)&dtile[bf][slot0], 16);
        }
    };

    float m[QB];
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) m[cb] = -INFINITY;
    // The ends of the stream's documents go to LDS once, up front: read at a
    // boundary, a scalar load would stall the wave for a memory round trip
    // (its counter is shared with LDS reads, so it cannot be left in flight).
    // A stream of more than DCAP documents reads them from memory instead.
    const int nd = bend - bbeg;
    const bool ends_lds = nd <= DCAP;  // uniform
    if (ends_lds) {
        for (int i = tid; i < nd; i += NT) dend_s[i] = (int)clamp_t(p.cu[bbeg + i + 1]);
    }
    // (read as the same value in every lane: the document walk, and every
    // branch on it, stays scalar)
    auto doc_end = [&](int bb) -> int64_t {
        return ends_lds ? (int64_t)__builtin_amdgcn_readfirstlane(dend_s[bb - bbeg]) : clamp_t(cu[bb + 1]);
    };
    // The document being folded, b, ends at token dend (wave-uniform).
    int b = bbeg;
    int64_t dend = T1;
    auto finish_doc = [&]() {  // document b is complete: merge, sum, store; move to b + 1
#pragma unroll
        for (int cb = 0; cb < QB; ++cb) {
            const float mv = xor32_max(m[cb]);
            const float sc = lanes32_sum(mv);
            const int ql = wave * QB + cb;
            if (lane == 31 && ql < nq) p.scores[(int64_t)(q0 + ql) * p.B + b] = sc;
            m[cb] = -INFINITY;
        }
        ++b;
        if (b < bend) dend = doc_end(b);
    };
    // Fold the values of tokens lo <= t < hi (relative to the sub-tile).
    // Slot i of a lane holds token tok(0, i) + 4g (g = lane / 32), so one
    // word of in-range tokens shifted by 4g gives every slot's test as a bit;
    // each slot's bit becomes an all-ones / all-zeros mask, and each value is
    // one bitfield insert of its bits or those of -inf.
    static_assert(M == 32 && MM::NG == 2, "fold_range assumes the 32x32 layout");
    const uint32_t sh4 = (uint32_t)g * 4u;
    auto fold_range = [&](const Acc* acc, int lo, int hi) {  // 0 <= lo < hi <= 32
        const uint32_t tm = (hi >= 32 ? 0xFFFFFFFFu : (1u << hi) - 1u) & ~((1u << lo) - 1u);
        const uint32_t w = tm >> sh4;  // bit u: token u + 4g lies in range
        uint32_t mk[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int u = MM::tok(0, i);
            mk[i] = (uint32_t)((int32_t)(w << (31 - u)) >> 31);
        }
#pragma unroll
        for (int cb = 0; cb < QB; ++cb) {
            float mx = m[cb];
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                mx = fmaxf(mx, bitsf((fbits(acc[cb][i]) & mk[i]) | (~mk[i] & 0xFF800000u)));
            m[cb] = mx;
        }
    };
    // Fold the sub-tile whose first token is t0, finishing every document
    // that ends inside it (empty ones included).
    auto fold_sub = [&](const Acc* acc, int64_t t0) {
        int lo = 0;
        while (b < bend && dend - t0 < M) {  // uniform
            const int e = (int)(dend - t0);
            if (e > lo) fold_range(acc, lo, e);
            finish_doc();
            lo = e > lo ? e : lo;
        }
        if (b < bend) {
            if (lo == 0) {
#pragma unroll
                for (int cb = 0; cb < QB; ++cb) {
                    float mx = m[cb];
#pragma unroll
                    for (int i = 0; i < VPL; ++i) mx = fmaxf(mx, acc[cb][i]);
                    m[cb] = mx;
                }
            } else {
                fold_range(acc, lo, M);
            }
        }
    };
    // MFMAs of sub-tile sb into cur; when fold_prev, the previous sub-tile
    // (wholly inside document b) is folded between them, as in fwd_kernel.
    // A sub-tile holding a document end is folded afterwards by fold_sub
    // (folding it between the MFMAs, with a branch per k-step, ran slower).
    auto stage = [&](int bf, int sb, Acc* cur, const Acc* prev, bool fold_prev) {
        u32x4 a[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) a[s] = dtile[bf][swz<NCH>(sb * M + lm, g * KS + s)];
#pragma unroll
        for (int cb = 0; cb < QB; ++cb) cur[cb] = MM::zero();
        __builtin_amdgcn_s_setprio(1);  // as in fwd_kernel's stage
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int cb = 0; cb < QB; ++cb) cur[cb] = MM::mma(a[s], bq[cb][s], cur[cb]);
            if (fold_prev) {  // uniform
#pragma unroll
                for (int cb = 0; cb < QB; ++cb)
#pragma unroll
                    for (int f = 0; f < FPS; ++f) m[cb] = fmaxf(m[cb], prev[cb][s * FPS + f]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    if (ntile > 0) issue_tile(0, 0);
    if (ntile > 1) {
        issue_tile(1, 1);
        if (loader) {
            wait_vmcnt<LPL>();  // tile 0 has landed; tile 1 may be in flight
        } else {
            wait_vmcnt<0>();
        }
    } else {
        wait_vmcnt<0>();
    }
    lds_barrier();  // also publishes dend_s
    if (b < bend) dend = doc_end(b);
    Acc acc0[QB], acc1[QB];
    bool carry = false;  // acc1 holds the unfolded last sub-tile of the previous tile
    for (int k = 0; k < ntile; ++k) {
        const int bf = k & 1;
        // tile k+1 goes into the buffer step k-1 read (tile 1 came with the prologue)
        if (k >= 1 && k + 1 < ntile) issue_tile(bf ^ 1, k + 1);
        const int64_t tb = T0 + (int64_t)k * TT;
        const int64_t left = T1 - tb;
        const int nsub = left >= TT ? SPW : (int)((left + M - 1) / M);
        const bool carried = carry;
        carry = false;
        static_for<SPW>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if (j >= nsub) return;  // uniform
            Acc* cur = (j & 1) ? acc1 : acc0;
            const Acc* prev = (j & 1) ? acc0 : acc1;
            const int64_t tprev = tb + (int64_t)(j - 1) * M;  // (for j = 0: the previous tile's last sub-tile)
            const bool has_prev = j > 0 || carried;
            const bool whole = has_prev && b < bend && dend - tprev >= M;  // previous sub-tile inside document b
            stage(bf, j, cur, prev, whole);
            if (has_prev && !whole) fold_sub(prev, tprev);
            if (j == nsub - 1) {
                if (j == SPW - 1 && k + 1 < ntile) {
                    carry = true;  // folded between the next step's first MFMAs (SPW is even: it sits in acc1)
                } else {
                    fold_sub(cur, tb + (int64_t)j * M);
                }
            }
        });
        if (k + 1 < ntile) wait_vmcnt<0>();  // tile k+1 has landed (and this step's stores retired)
        lds_barrier();
    }
    // documents ending on the last sub-tile edge and empty trailing documents
    while (b < bend) finish_doc();
}

// One workgroup of W waves scores up to 32 query rows (rows 0 .. nr-1 from
// `qrows`, 256 bytes apart) against one document (first row st, len tokens).
// The work per document token is tiny, so this is bound by reading D: each
// wave takes SPL 16-token sub-tiles per round and loads them straight from
// HBM into MFMA operand registers (no LDS staging of D), all of a round's
// loads in flight at once.  Lane group g reads 16 contiguous bytes at chunk
// s*4 + g of its row in k-step s, so one load instruction covers 64
// contiguous bytes of 16 rows.  The query rows are read once per workgroup
// into LDS (q_s, 32 rows x 16 chunks, XOR-swizzled by row) and every wave
// takes its MFMA fragments from there: reading them from global memory in
// every wave makes the few cache lines of Q a hot spot that delays the
// document stream.  The first round's document loads are issued before the
// Q barrier.  The argmax is exact (first index on ties).  On return, lanes
// r < nr of wave 0 hold row r's maximum and argmax (other waves' values are
// unspecified); every wave must call it (it contains workgroup barriers).
template <int ELEM, int W, int SPL>
__device__ __forceinline__ void rows_vs_doc(const FwdParams& p, const char* qrows, int nr, int64_t st, int len,
                                            u32x4* q_s, float (*rowmax_s)[32], int (*rowarg_s)[32], float& mv,
                                            int& idx) {
    using MM = Mma<ELEM, 16>;
    using Acc = typename MM::Acc;
    constexpr int M = 16, NG = MM::NG, KS = MM::KS, VPL = MM::VPL, ROWB = 256;
    constexpr int QCH = 32 * 16 / (64 * W);  // query chunks each thread stages
    static_assert(QCH * 64 * W == 32 * 16, "query staging");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane / M, lm = lane % M;
    u32x4 qv[QCH];
#pragma unroll
    for (int k = 0; k < QCH; ++k) {
        const int e = tid + k * 64 * W;
        const int r = e >> 4, c = e & 15;
        qv[k] = r < nr ? *reinterpret_cast<const u32x4*>(qrows + (int64_t)r * ROWB + c * 16) : u32x4{0u, 0u, 0u, 0u};
    }
    const int nsub = (len + M - 1) / M;
    // rows past the document read its first row; an empty document (which
    // may have no rows at all) reads the query rows instead
    const char* fallback = len > 0 ? p.D + st * ROWB : qrows;
    auto load_round = [&](int base, u32x4 (&a)[SPL][KS]) {
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
            const int tok = (base + j) * M + lm;
            const char* src = tok < len ? p.D + (st + tok) * ROWB : fallback;
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) a[j][s2] = *reinterpret_cast<const u32x4*>(src + (s2 * NG + g) * 16);
        }
    };
    // Keep every load of a round in flight together: without this the
    // compiler sinks each sub-tile's loads into the branch that uses them and
    // the round becomes a chain of dependent memory round trips.  (The empty
    // asm reads the registers, so it also waits for the loads.)
    auto pin_round = [&](u32x4 (&a)[SPL][KS]) {
#pragma unroll
        for (int j = 0; j < SPL; ++j)
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) asm volatile("" : "+v"(a[j][s2]));
    };
    u32x4 a[SPL][KS];
    load_round(wave * SPL, a);  // every wave, so the Q write below waits for the Q loads only
#pragma unroll
    for (int k = 0; k < QCH; ++k) {
        const int e = tid + k * 64 * W;
        const int r = e >> 4, c = e & 15;
        q_s[r * 16 + (c ^ (r & 15))] = qv[k];
    }
    __syncthreads();
    u32x4 bq[2][KS];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int r = cb * M + lm;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) bq[cb][s2] = q_s[r * 16 + ((s2 * NG + g) ^ (r & 15))];
    }
    pin_round(a);  // the first round was issued before the Q barrier
    float m[2] = {-INFINITY, -INFINITY};
    int best[2] = {-1, -1};  // token index of the maximum (first on ties)
    for (int base = wave * SPL; base < nsub; base += W * SPL) {  // uniform
        if (base != wave * SPL) {  // later rounds of a long document
            load_round(base, a);
            pin_round(a);
        }
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
            const int sb = base + j;
            if (sb >= nsub) break;  // uniform
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                Acc acc = MM::zero();
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2) acc = MM::mma(a[j][s2], bq[cb][s2], acc);
                // Unmasked: a slot past the document's end holds a copy of
                // its first token (len > 0 here), the same value under a
                // later index, so it changes no maximum, and the strict
                // update and the lower-index merge never let it win the
                // argmax.
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const float v = acc[i];
                    if (v > m[cb]) {  // strict: the earliest token keeps a tie
                        m[cb] = v;
                        best[cb] = sb * M + MM::tok(g, i);
                    }
                }
            }
        }
    }
    // merge the four lane groups of every query row, then the waves
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
        for (int off = M; off < 64; off <<= 1) {
            if (off == 32) {  // the larger value, then the lowest index among the lanes holding it
                const float mx = xor32_max(m[cb]);
                const unsigned c = m[cb] == mx ? (unsigned)best[cb] : 0xFFFFFFFFu;
                best[cb] = (int)xor32_min_u(c);
                m[cb] = mx;
            } else {
                const float om = __shfl_xor(m[cb], off);
                const int oi = __shfl_xor(best[cb], off);
                if (om > m[cb] || (om == m[cb] && (unsigned)oi < (unsigned)best[cb])) {
                    m[cb] = om;
                    best[cb] = oi;
                }
            }
        }
        if (g == 0) {
            rowmax_s[wave][cb * M + lm] = m[cb];
            rowarg_s[wave][cb * M + lm] = best[cb];
        }
    }
    __syncthreads();
    mv = -INFINITY;
    idx = -1;
    if (wave == 0 && lane < nr) {
#pragma unroll
        for (int w = 0; w < W; ++w) {  // ties: the lower token index
            const float om = rowmax_s[w][lane];
            const int oi = rowarg_s[w][lane];
            if (om > mv || (om == mv && (unsigned)oi < (unsigned)idx)) {
                mv = om;
                idx = oi;
            }
        }
    }
    __syncthreads();  // the LDS rows (and q_s) may be reused by the caller
}

// Few query rows in all (Nq * Lq <= 32, e.g. one ColBERT query): one
// workgroup per document scores every row (rows_vs_doc); wave 0 writes the
// argmax and the per-query sums.
template <int ELEM, int W, int SPL, bool ARGMAX, bool VARLEN>
__global__ __launch_bounds__(64 * W) void fwd_tiny_kernel(FwdParams p) {
    __shared__ u32x4 q_s[32 * 16];
    __shared__ float rowmax_s[W][32];
    __shared__ int rowarg_s[W][32];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t st;
    int len;
    doc_info<VARLEN>(p, b, st, len);
    const int nrows = p.Nq * p.Lq;  // <= 32
    float mv;
    int idx;
    rows_vs_doc<ELEM, W, SPL>(p, p.Q, nrows, st, len, q_s, rowmax_s, rowarg_s, mv, idx);
    if (wave != 0) return;
    if (p.Nq == 1) {  // uniform: one query, its rows in lanes 0 .. Lq-1 -> DPP sum, no LDS round trip
        if (ARGMAX && lane < nrows) p.argmax[(int64_t)b * p.Lq + lane] = idx;
        const float sc = lanes32_sum(lane < nrows ? mv : 0.f);
        if (lane == 31) p.scores[b] = sc;
        return;
    }
    if (lane < nrows) rowmax_s[0][lane] = mv;  // only this wave reads it from here on
    __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0): the row maxima are in LDS
    __builtin_amdgcn_wave_barrier();
    const int Lq = p.Lq;
    if (lane < nrows) {
        const int q = lane / Lq, i = lane - q * Lq;
        if (ARGMAX) p.argmax[((int64_t)q * p.B + b) * Lq + i] = idx;
    }
    if (lane < p.Nq) {  // query lane: its Lq (<= 32) row maxima in ascending order
        float v[32];  // all loads issued before the first add
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = i < Lq ? rowmax_s[0][lane * Lq + i] : 0.f;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if (i < Lq) acc += v[i];
        p.scores[(int64_t)lane * p.B + b] = acc;
    }
}

// An explicit list of (query, document) pairs over the packed corpus (the
// rescoring pass of the two-stage scan): one workgroup per pair, the query's
// rows in blocks of 32 (rows_vs_doc each), the block sums added in order.
// scores[p] and argmax[p, Lq] follow the list.
template <int ELEM, int W, int SPL, bool ARGMAX>
__global__ __launch_bounds__(64 * W) void fwd_pairs_kernel(FwdParams p, const int32_t* pq, const int32_t* pb) {
    __shared__ u32x4 q_s[32 * 16];
    __shared__ float rowmax_s[W][32];
    __shared__ int rowarg_s[W][32];
    const int pair = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int q = ((cint_ptr)pq)[pair];
    int b = ((cint_ptr)pb)[pair];
    q = q < 0 ? 0 : (q >= p.Nq ? p.Nq - 1 : q);  // out-of-range pairs break the contract; keep accesses in bounds
    b = b < 0 ? 0 : (b >= p.B ? p.B - 1 : b);
    int64_t st;
    int len;
    doc_info<true>(p, b, st, len);
    const int Lq = p.Lq;
    float total = 0.f;
    for (int r0 = 0; r0 < Lq; r0 += 32) {  // uniform
        const int nr = Lq - r0 < 32 ? Lq - r0 : 32;
        float mv;
        int idx;
        rows_vs_doc<ELEM, W, SPL>(p, p.Q + ((int64_t)q * Lq + r0) * 256, nr, st, len, q_s, rowmax_s, rowarg_s, mv,
                                  idx);
        if (wave == 0) {
            if (ARGMAX && lane < nr) p.argmax[(int64_t)pair * Lq + r0 + lane] = idx;
            // rows of the block in ascending order: every lane gathers them
            // (all shuffles issued before the first add)
            float v[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] = __shfl(mv, i);
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i)
                if (i < nr) part += v[i];
            total += part;
        }
    }
    if (wave == 0 && lane == 0) p.scores[pair] = total;
}

__global__ __launch_bounds__(256) void zero_fill(float* x, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) x[i] = 0.f;
}

template <int ELEM, int M, int QB, int WQ, int WT, int SPW, int NSI, int NBUF, bool ARGMAX, bool VARLEN>
hipError_t launch_cfg(const FwdArgs& a, hipStream_t stream, int target_blocks) {
    constexpr int R = WQ * QB * M;
    FwdParams p;
    p.Q = static_cast<const char*>(a.Q);
    p.D = static_cast<const char*>(a.D);
    p.lens = a.d_lens;
    p.cu = a.cu;
    p.q_scale = a.q_scale;
    p.d_scale = a.d_scale;
    p.T = a.T;
    p.Nq = a.Nq;
    p.Lq = a.Lq;
    p.B = a.B;
    p.Ld = a.Ld;
    if (a.Lq <= R) {
        p.split = 1;
        p.half_rows = a.Lq;
        p.qps = R / a.Lq;
        if (p.qps > a.Nq) p.qps = a.Nq;
        p.num_slabs = (a.Nq + p.qps - 1) / p.qps;
    } else {  // a query longer than the slab: two halves (callers ensure Lq <= 2R)
        p.split = 2;
        p.half_rows = (a.Lq + 1) / 2;
        p.qps = 1;
        p.num_slabs = 2 * a.Nq;
        hipLaunchKernelGGL(zero_fill, dim3((unsigned)(((int64_t)a.Nq * a.B + 255) / 256)), dim3(256), 0, stream,
                           a.scores, (int64_t)a.Nq * a.B);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // blocks = 8 * num_slabs * s8 (the XCD-aware map needs whole groups of 8):
    // as many stream groups as fit in one round of target_blocks, at least one,
    // and no more streams than documents.
    int s8 = target_blocks / (8 * p.num_slabs);
    if (s8 < 1) s8 = 1;
    if (s8 > (a.B + 7) / 8) s8 = (a.B + 7) / 8;
    int streams = 8 * s8;
    if (streams > a.B) streams = a.B;
    p.num_streams = streams;
    // A grid that fits one round of workgroups splits the documents into
    // balanced contiguous ranges; a grid of several rounds is balanced by the
    // hardware's dispatch of later workgroups, and there each workgroup would
    // pay the range search again, so it deals documents round-robin.
    p.round_robin = 8LL * p.num_slabs * s8 > target_blocks;
    p.scores = a.scores;
    p.argmax = a.argmax;
    const long long blocks = 8LL * p.num_slabs * s8;
    hipLaunchKernelGGL((fwd_kernel<ELEM, M, QB, WQ, WT, SPW, NSI, NBUF, ARGMAX, VARLEN>), dim3((unsigned)blocks),
                       dim3(64 * WQ * WT), 0, stream, p);
    return hipGetLastError();
}

// fwd_flat_kernel: 512-row slabs of 16 queries; as many stream groups as fit
// one workgroup per CU, at least one, and no more streams than documents.
template <int ELEM>
hipError_t launch_flat(const FwdArgs& a, hipStream_t stream) {
    FwdParams p{};
    p.Q = static_cast<const char*>(a.Q);
    p.D = static_cast<const char*>(a.D);
    p.cu = a.cu;
    p.T = a.T;
    p.Nq = a.Nq;
    p.Lq = a.Lq;
    p.B = a.B;
    p.Ld = a.Ld;
    p.split = 1;
    p.half_rows = a.Lq;
    p.qps = 16 < a.Nq ? 16 : a.Nq;
    p.num_slabs = (a.Nq + p.qps - 1) / p.qps;
    int s8 = 256 / (8 * p.num_slabs);
    if (s8 < 1) s8 = 1;
    if (s8 > (a.B + 7) / 8) s8 = (a.B + 7) / 8;
    p.num_streams = 8 * s8 < a.B ? 8 * s8 : a.B;
    p.round_robin = 0;  // the kernel walks contiguous token ranges
    p.scores = a.scores;
    const long long blocks = 8LL * p.num_slabs * s8;
    hipLaunchKernelGGL(fwd_flat_kernel<ELEM>, dim3((unsigned)blocks), dim3(512), 0, stream, p);
    return hipGetLastError();
}

template <int ELEM, bool ARGMAX, bool VARLEN>
hipError_t launch_tiny(const FwdArgs& a, hipStream_t stream) {
    FwdParams p{};
    p.Q = static_cast<const char*>(a.Q);
    p.D = static_cast<const char*>(a.D);
    p.lens = a.d_lens;
    p.cu = a.cu;
    p.T = a.T;
    p.Nq = a.Nq;
    p.Lq = a.Lq;
    p.B = a.B;
    p.Ld = a.Ld;
    p.scores = a.scores;
    p.argmax = a.argmax;
    hipLaunchKernelGGL((fwd_tiny_kernel<ELEM, 4, 3, ARGMAX, VARLEN>), dim3((unsigned)a.B), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int ELEM, bool ARGMAX>
hipError_t launch_pairs(const FwdArgs& a, const int32_t* pq, const int32_t* pb, int32_t P, hipStream_t stream) {
    FwdParams p{};
    p.Q = static_cast<const char*>(a.Q);
    p.D = static_cast<const char*>(a.D);
    p.cu = a.cu;
    p.T = a.T;
    p.Nq = a.Nq;
    p.Lq = a.Lq;
    p.B = a.B;
    p.scores = a.scores;
    p.argmax = a.argmax;
    hipLaunchKernelGGL((fwd_pairs_kernel<ELEM, 4, 3, ARGMAX>), dim3((unsigned)P), dim3(256), 0, stream, p, pq, pb);
    return hipGetLastError();
}

template <int ELEM, bool ARGMAX, bool VARLEN>
hipError_t dispatch_shape(const FwdArgs& a, hipStream_t stream) {
    // Few query rows in all (single-query reranking): one 32-row slab, four
    // waves split each document's tokens; many small workgroups fill the chip.
    if ((int64_t)a.Nq * a.Lq <= 32) {
        if constexpr (ELEM != kI8) return launch_tiny<ELEM, ARGMAX, VARLEN>(a, stream);
        return launch_cfg<ELEM, 16, 2, 1, 4, 1, 1, 3, ARGMAX, VARLEN>(a, stream, 2048);
    }
    // Packed corpus, 32-token queries, scores only: tiles across documents.
    if constexpr (!ARGMAX && VARLEN && ELEM != kI8) {
        if (a.Lq == 32) return launch_flat<ELEM>(a, stream);
    }
    // Otherwise one persistent workgroup per CU holding a slab of query rows.
    if constexpr (ELEM == kI8) {
        // 1024-row slabs in 16x16x64 int8 blocks.  Scores only: 8 waves x 128
        // rows.  With the argmax (two compares and selects more per value):
        // 16 waves x 64 rows, 4 waves per SIMD, 6 % faster there (1.2 % slower
        // without it).
        if constexpr (ARGMAX) {
            return launch_cfg<ELEM, 16, 4, 16, 1, 16, 1, 2, ARGMAX, VARLEN>(a, stream, 256);
        } else {
            return launch_cfg<ELEM, 16, 8, 8, 1, 16, 1, 2, ARGMAX, VARLEN>(a, stream, 256);
        }
    } else {
        if (a.Lq > 512 && a.Lq <= 768) {
            // 768-row slabs of whole queries: 8 waves x 96 rows, 2 waves per SIMD
            return launch_cfg<ELEM, 32, 3, 8, 1, 4, 1, 3, ARGMAX, VARLEN>(a, stream, 256);
        }
        // 512-row slabs (whole queries up to 512 tokens, else two halves of a
        // query): 8 waves x 64 rows
        return launch_cfg<ELEM, 32, 2, 8, 1, 8, 2, 2, ARGMAX, VARLEN>(a, stream, 256);
    }
}

template <int ELEM, bool VARLEN>
hipError_t dispatch_argmax(const FwdArgs& a, hipStream_t stream) {
    if (a.argmax) return dispatch_shape<ELEM, true, VARLEN>(a, stream);
    return dispatch_shape<ELEM, false, VARLEN>(a, stream);
}

}  // namespace

hipError_t launch_fwd_pairs(const FwdArgs& a, const int32_t* pq, const int32_t* pb, int32_t P, hipStream_t stream) {
    if (P == 0) return hipSuccess;
    const bool am = a.argmax != nullptr;
    switch (a.elem) {
        case kF16:
            return am ? launch_pairs<kF16, true>(a, pq, pb, P, stream) : launch_pairs<kF16, false>(a, pq, pb, P, stream);
        case kBF16:
            return am ? launch_pairs<kBF16, true>(a, pq, pb, P, stream) : launch_pairs<kBF16, false>(a, pq, pb, P, stream);
        default:
            return hipErrorInvalidValue;
    }
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
    if (a.Nq == 0 || a.B == 0) return hipSuccess;
    switch (a.elem) {
        case kF16:
            return a.varlen ? dispatch_argmax<kF16, true>(a, stream)
                            : dispatch_argmax<kF16, false>(a, stream);
        case kBF16:
            return a.varlen ? dispatch_argmax<kBF16, true>(a, stream)
                            : dispatch_argmax<kBF16, false>(a, stream);
        case kI8:
            return dispatch_argmax<kI8, true>(a, stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace maxsim

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
//   * Documents stream HBM -> LDS in tiles of 64 tokens, double-buffered, the
//     next tile's global loads (possibly of the next document) in flight while
//     the current one is contracted.  LDS rows are XOR-swizzled by 16-byte
//     chunk so the MFMA operand reads are bank-conflict free.
//   * S_t = D_tile Q_slab^T is formed 16 doc tokens x 16 query rows at a time
//     with v_mfma_f32_16x16x32_{f16,bf16} (int8: v_mfma_i32_16x16x64_i8),
//     fp32 (int32) accumulation.  Doc tokens are the M dimension, so each lane
//     holds 4 tokens of one query row and the running max / argmax stays in
//     the lane; lanes are merged once per document (two xor shuffles).
//   * The grid is persistent: block -> (slab, document stream) is laid out so
//     the workgroups sharing a document stream sit on the same XCD (blocks are
//     dispatched round-robin over the 8 XCDs) and re-read each tile from that
//     XCD's L2 rather than HBM.
//   * Masking (Algorithm 2): positions past the document's length are -inf
//     before the maximum; tokens past the end are never loaded.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace maxsim {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
    int qps;          // queries per slab
    int num_slabs;
    int num_streams;  // documents b = stream, stream + num_streams, ...
    float* scores;
    int32_t* argmax;
};

template <int ELEM>
__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (ELEM == kF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
}

__device__ __forceinline__ i32x4 mma16_i8(u32x4 a, u32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                                 __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// LDS slot (in 16-byte units) of chunk c of tile row `row`.  fp16/bf16 rows are
// 256 B = 16 chunks (one full bank sweep): chunk ^ (row & 15).  int8 rows are
// 128 B = 8 chunks, two rows per sweep: chunk ^ ((row >> 1) & 7).  Either way
// the 16 rows read by one 16-lane group land on 16 distinct 16-byte bank groups.
template <int NCH>
__device__ __forceinline__ int swz(int row, int c) {
    if constexpr (NCH == 16) {
        return row * 16 + (c ^ (row & 15));
    } else {
        return row * 8 + (c ^ ((row >> 1) & 7));
    }
}

template <bool VARLEN>
__device__ __forceinline__ void doc_info(const FwdParams& p, int b, int64_t& start, int& len) {
    if constexpr (VARLEN) {
        int64_t s0 = p.cu[b];
        int64_t s1 = p.cu[b + 1];
        s0 = s0 < 0 ? 0 : (s0 > p.T ? p.T : s0);
        s1 = s1 < s0 ? s0 : (s1 > p.T ? p.T : s1);
        start = s0;
        len = (int)(s1 - s0);
    } else {
        start = (int64_t)b * p.Ld;
        int l = p.lens ? p.lens[b] : p.Ld;
        len = l < 0 ? 0 : (l > p.Ld ? p.Ld : l);
    }
}

// ELEM: kF16 / kBF16 / kI8.  QB: 16-row query blocks per wave.  WQ x WT waves:
// WQ along query rows, WT along document tokens.  SPW: 16-token sub-tiles each
// wave contracts per tile.  ARGMAX: also track and write the argmax.
template <int ELEM, int QB, int WQ, int WT, int SPW, bool ARGMAX, bool VARLEN>
__global__ __launch_bounds__(64 * WQ * WT) void fwd_kernel(FwdParams p) {
    constexpr bool I8 = ELEM == kI8;
    constexpr int NW = WQ * WT;
    constexpr int NT = 64 * NW;
    constexpr int ROWB = I8 ? 128 : 256;  // bytes per token row
    constexpr int NCH = ROWB / 16;        // 16-byte chunks per row
    constexpr int KS = NCH / 4;           // MFMA k-steps per row
    constexpr int SUBS = SPW * WT;        // 16-token sub-tiles per tile
    constexpr int TT = 16 * SUBS;         // tokens per tile
    constexpr int R = WQ * QB * 16;       // slab capacity in query-token rows
    constexpr int LPT = TT * NCH / NT;    // 16-byte loads per thread per tile
    static_assert(LPT * NT == TT * NCH, "tile must split evenly over the workgroup");

    __shared__ u32x4 dtile[2][TT * NCH];
    __shared__ float dsc[I8 ? 2 : 1][I8 ? TT : 1];
    __shared__ float rowmax_s[R];
    __shared__ int rowarg_s[ARGMAX ? R : 1];
    __shared__ float xm[WT > 1 ? WT : 1][WT > 1 ? R : 1];
    __shared__ int xi[(WT > 1 && ARGMAX) ? WT : 1][(WT > 1 && ARGMAX) ? R : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wq = wave % WQ;
    const int wt = wave / WQ;
    const int g = lane >> 4;    // lane group: k-chunk of the operands, token quad of the result
    const int l16 = lane & 15;  // operand row / result column

    const int blk = blockIdx.x;
    const int xcd = blk & 7;
    const int jx = blk >> 3;
    const int slab = jx % p.num_slabs;
    const int stream = (jx / p.num_slabs) * 8 + xcd;
    if (stream >= p.num_streams || stream >= p.B) return;  // uniform over the workgroup
    const int q0 = slab * p.qps;
    const int nq = min(p.qps, p.Nq - q0);
    const int nrows = nq * p.Lq;
    const int Lq = p.Lq;

    // Query slab -> VGPRs.  Lane (g, l16) of block cb holds row (wq*QB+cb)*16+l16,
    // chunks g, g+4, g+8, g+12 (k-step s uses chunk g + 4s; the document operand
    // uses the same chunk map, so every k meets its partner exactly once).
    u32x4 bq[QB][KS];
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) {
        const int r = (wq * QB + cb) * 16 + l16;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (r < nrows) {
                bq[cb][s] = *reinterpret_cast<const u32x4*>(
                    p.Q + ((int64_t)q0 * Lq + r) * ROWB + (g + 4 * s) * 16);
            } else {
                bq[cb][s] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }

    float m[QB];
    int code[QB];  // (global 16-token sub-tile << 2) | row within the lane's token quad
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) {
        m[cb] = -INFINITY;
        code[cb] = -1;
    }

    u32x4 pre[LPT];
    float pres = 0.f;

    auto load_tile = [&](int64_t st, int ln, int tt) {
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int ci = tid + u * NT;
            const int row = ci / NCH;
            const int c = ci % NCH;
            const int tok = tt * TT + row;
            if (tok < ln) {
                pre[u] = *reinterpret_cast<const u32x4*>(p.D + (st + tok) * ROWB + c * 16);
            } else {
                pre[u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        if constexpr (I8) {
            if (tid < TT) {
                const int tok = tt * TT + tid;
                pres = tok < ln ? p.d_scale[st + tok] : 0.f;
            }
        }
    };
    auto store_tile = [&](int bf) {
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int ci = tid + u * NT;
            dtile[bf][swz<NCH>(ci / NCH, ci % NCH)] = pre[u];
        }
        if constexpr (I8) {
            if (tid < TT) dsc[bf][tid] = pres;
        }
    };

    auto compute_tile = [&](int bf, int tt, int ln) {
#pragma unroll
        for (int k = 0; k < SPW; ++k) {
            const int sb = wt * SPW + k;
            const int tok0 = tt * TT + sb * 16;
            if (tok0 >= ln) break;  // uniform
            u32x4 a[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) a[s] = dtile[bf][swz<NCH>(sb * 16 + l16, g + 4 * s)];
            f32x4 sc;
            if constexpr (I8) sc = *reinterpret_cast<const f32x4*>(&dsc[bf][sb * 16 + 4 * g]);
            const bool full = tok0 + 16 <= ln;
            const int cbase = (tt * SUBS + sb) << 2;
#pragma unroll
            for (int cb = 0; cb < QB; ++cb) {
                if ((wq * QB + cb) * 16 >= nrows) break;  // uniform: rest of the slab is empty
                float v[4];
                if constexpr (I8) {
                    i32x4 acc = {0, 0, 0, 0};
#pragma unroll
                    for (int s = 0; s < KS; ++s) acc = mma16_i8(a[s], bq[cb][s], acc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = (float)acc[r] * sc[r];
                } else {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s) acc = mma16<ELEM>(a[s], bq[cb][s], acc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = acc[r];
                }
                if (!full) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (tok0 + 4 * g + r >= ln) v[r] = -INFINITY;
                }
                if constexpr (ARGMAX) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (v[r] > m[cb]) {  // strict: the earliest token keeps a tie
                            m[cb] = v[r];
                            code[cb] = cbase | r;
                        }
                    }
                } else {
                    m[cb] = fmaxf(m[cb], fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
                }
            }
        }
    };

    auto epilogue = [&](int b) {
        // Merge the four token quads of every query row (lanes l, l^16, l^32, l^48).
#pragma unroll
        for (int cb = 0; cb < QB; ++cb) {
            float mv = m[cb];
            int idx = -1;
            if constexpr (ARGMAX) {
                if (code[cb] >= 0) idx = 16 * (code[cb] >> 2) + 4 * g + (code[cb] & 3);
            }
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float om = __shfl_xor(mv, off);
                if constexpr (ARGMAX) {
                    const int oi = __shfl_xor(idx, off);
                    if (om > mv || (om == mv && (unsigned)oi < (unsigned)idx)) {
                        mv = om;
                        idx = oi;
                    }
                } else {
                    mv = fmaxf(mv, om);
                }
            }
            const int r = (wq * QB + cb) * 16 + l16;
            if (g == 0 && r < R) {
                if constexpr (WT == 1) {
                    rowmax_s[r] = mv;
                    if constexpr (ARGMAX) rowarg_s[r] = idx;
                } else {
                    xm[wt][r] = mv;
                    if constexpr (ARGMAX) xi[wt][r] = idx;
                }
            }
            m[cb] = -INFINITY;
            code[cb] = -1;
        }
        __syncthreads();
        if constexpr (WT > 1) {
            for (int r = tid; r < R; r += NT) {
                float mv = xm[0][r];
                int idx = 0;
                if constexpr (ARGMAX) idx = xi[0][r];
#pragma unroll
                for (int w = 1; w < WT; ++w) {
                    const float om = xm[w][r];
                    if constexpr (ARGMAX) {
                        const int oi = xi[w][r];
                        if (om > mv || (om == mv && (unsigned)oi < (unsigned)idx)) {
                            mv = om;
                            idx = oi;
                        }
                    } else {
                        mv = fmaxf(mv, om);
                    }
                }
                rowmax_s[r] = mv;
                if constexpr (ARGMAX) rowarg_s[r] = idx;
            }
            __syncthreads();
        }
        if constexpr (ARGMAX) {
            for (int r = tid; r < nrows; r += NT) {
                const int ql = r / Lq;
                const int i = r - ql * Lq;
                p.argmax[((int64_t)(q0 + ql) * p.B + b) * Lq + i] = rowarg_s[r];
            }
        }
        if constexpr (I8) {
            // Exact epilogue: v_i = fl32(m_i * q_scale_i), summed in ascending i.
            for (int ql = tid; ql < nq; ql += NT) {
                const float* qs = p.q_scale + (int64_t)(q0 + ql) * Lq;
                const float* rm = rowmax_s + ql * Lq;
                float acc = 0.f;
                for (int i = 0; i < Lq; ++i) {
                    const float v = rm[i] * qs[i];
                    acc = acc + v;
                }
                p.scores[(int64_t)(q0 + ql) * p.B + b] = acc;
            }
        } else if (Lq < 64) {
            for (int ql = tid; ql < nq; ql += NT) {
                const float* rm = rowmax_s + ql * Lq;
                float acc = 0.f;
                for (int i = 0; i < Lq; ++i) acc += rm[i];
                p.scores[(int64_t)(q0 + ql) * p.B + b] = acc;
            }
        } else {
            for (int ql = wave; ql < nq; ql += NW) {
                const float* rm = rowmax_s + ql * Lq;
                float acc = 0.f;
                for (int i = lane; i < Lq; i += 64) acc += rm[i];
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
                if (lane == 0) p.scores[(int64_t)(q0 + ql) * p.B + b] = acc;
            }
        }
    };

    // Persistent walk over this workgroup's documents, one tile per step.
    int b = stream;
    int64_t start;
    int len;
    doc_info<VARLEN>(p, b, start, len);
    int ntiles = (len + TT - 1) / TT;
    int t = 0;
    load_tile(start, len, 0);
    store_tile(0);
    __syncthreads();
    int buf = 0;
    while (true) {
        int nb = b, nt = t + 1, nlen = len, nntiles = ntiles;
        int64_t nstart = start;
        if (nt >= ntiles) {
            nb = b + p.num_streams;
            nt = 0;
            if (nb < p.B) {
                doc_info<VARLEN>(p, nb, nstart, nlen);
                nntiles = (nlen + TT - 1) / TT;
            }
        }
        const bool has_next = nb < p.B;
        if (has_next) load_tile(nstart, nlen, nt);
        if (t < ntiles) compute_tile(buf, t, len);
        if (t + 1 >= ntiles) epilogue(b);
        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
        if (!has_next) break;
        buf ^= 1;
        b = nb;
        t = nt;
        start = nstart;
        len = nlen;
        ntiles = nntiles;
    }
}

template <int ELEM, int QB, int WQ, int WT, int SPW, bool ARGMAX, bool VARLEN>
hipError_t launch_cfg(const FwdArgs& a, hipStream_t stream, int target_blocks) {
    constexpr int R = WQ * QB * 16;
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
    p.qps = R / a.Lq;
    if (p.qps > a.Nq) p.qps = a.Nq;
    p.num_slabs = (a.Nq + p.qps - 1) / p.qps;
    int streams = (target_blocks + p.num_slabs - 1) / p.num_slabs;
    if (streams > a.B) streams = a.B;
    if (streams < 1) streams = 1;
    p.num_streams = streams;
    p.scores = a.scores;
    p.argmax = a.argmax;
    const int s8 = (streams + 7) / 8;
    const long long blocks = 8LL * p.num_slabs * s8;
    hipLaunchKernelGGL((fwd_kernel<ELEM, QB, WQ, WT, SPW, ARGMAX, VARLEN>), dim3((unsigned)blocks),
                       dim3(64 * WQ * WT), 0, stream, p);
    return hipGetLastError();
}

template <int ELEM, bool ARGMAX, bool VARLEN>
hipError_t dispatch_shape(const FwdArgs& a, hipStream_t stream) {
    // Few query rows in all (single-query reranking): one 32-row slab, four
    // waves split each document's tokens; many small workgroups fill the chip.
    if ((int64_t)a.Nq * a.Lq <= 32) {
        return launch_cfg<ELEM, 2, 1, 4, 1, ARGMAX, VARLEN>(a, stream, 2048);
    }
    // Otherwise a 1024-row slab held by 8 waves, one persistent workgroup per CU.
    return launch_cfg<ELEM, 8, 8, 1, 4, ARGMAX, VARLEN>(a, stream, 256);
}

template <int ELEM, bool VARLEN>
hipError_t dispatch_argmax(const FwdArgs& a, hipStream_t stream) {
    if (a.argmax) return dispatch_shape<ELEM, true, VARLEN>(a, stream);
    return dispatch_shape<ELEM, false, VARLEN>(a, stream);
}

}  // namespace

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

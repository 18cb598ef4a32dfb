/*
 * maxsim_oracle.c -- plain, slow, CPU reference for the fused MaxSim path
 * and its Chamfer-distance generalisation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header or table with the HIP
 * library.
 *
 * Source: "Flash-MaxSim: IO-Aware Fused Kernels for Late-Interaction
 * Scoring" (arXiv 2605.29517).  Every function below cites the passage it
 * follows.  Floating-point inputs (fp16 / bf16) are decoded exactly and all
 * arithmetic is done in fp64; the INT8 path follows its own fp32 epilogue,
 * which is defined here because the page leaves it open.
 *
 * Built with  gcc -O2 -fopenmp -ffp-contract=off  (no fast-math), so every
 * fp operation below is a single IEEE operation in the written order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F16 0
#define ORACLE_BF16 1

/* ------------------------------------------------------------------ */
/* Exact decoders.                                                      */
/* ------------------------------------------------------------------ */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Subnormals are fraction * 2^-24.  Every binary16 value is exactly
 * representable in binary64. */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25);
    }
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent
 * bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 7) & 0xff;
    int frac = h & 0x7f;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -133);
    } else if (expo == 255) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + frac), expo - 134);
    }
    return sign ? -v : v;
}

static double decode(uint16_t h, int dtype) {
    return dtype == ORACLE_BF16 ? oracle_bf16_to_f64(h) : oracle_f16_to_f64(h);
}

/* ------------------------------------------------------------------ */
/* Forward, fp16 / bf16.                                                */
/* ------------------------------------------------------------------ */

/*
 * MaxSim of one (query, document) pair -- paper, Section 1, Eq. (1):
 *     score(Q, D) = sum_i max_j <Q_i, D_j>.
 * q: Lq rows of d decoded values; doc: len rows of d decoded values.
 * The max over j is a strict ">" scan from j = 0 starting at -inf, so the
 * saved index is the first j attaining the maximum (the page saves one
 * argmax index per query token, Section 4.2 "Runtime Inverse-Grid
 * Construction").  With len == 0 the maximum stays -inf and the index -1
 * (the running max starts at -inf, Section 4.1 "Online-Max Recurrence").
 * Writes amax[i] for each query token i and returns the score.
 */
static double pair_score(const double* q, const double* doc, int Lq, int len, int d,
                         int32_t* amax, double* rowmax) {
    double score = 0.0;
    for (int i = 0; i < Lq; ++i) {
        double m = -INFINITY;
        int32_t arg = -1;
        for (int j = 0; j < len; ++j) {
            double s = 0.0;
            for (int k = 0; k < d; ++k) s += q[(int64_t)i * d + k] * doc[(int64_t)j * d + k];
            if (s > m) {
                m = s;
                arg = j;
            }
        }
        if (amax) amax[i] = arg;
        if (rowmax) rowmax[i] = m;
        score += m;
    }
    return score;
}

/*
 * Shared driver: documents are described by (first token, length); the
 * padded layout and the packed cu_seqlens layout only differ in how those
 * two numbers are read (Section 4.3 "Padding-Free Variable-Length": only the
 * real tokens of each document take part).
 */
static void fwd_docs(const uint16_t* Q, const uint16_t* D, int dtype, const int64_t* first,
                     const int32_t* len, int Nq, int Lq, int B, int d, double* scores,
                     int32_t* argmax, double* rowmax) {
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int q = 0; q < Nq; ++q) {
        for (int b = 0; b < B; ++b) {
            double* qd = (double*)malloc(sizeof(double) * (size_t)Lq * d);
            double* dd = (double*)malloc(sizeof(double) * ((size_t)len[b] * d + 1));
            for (int64_t e = 0; e < (int64_t)Lq * d; ++e)
                qd[e] = decode(Q[(int64_t)q * Lq * d + e], dtype);
            for (int64_t e = 0; e < (int64_t)len[b] * d; ++e)
                dd[e] = decode(D[first[b] * d + e], dtype);
            int64_t pair = (int64_t)q * B + b;
            scores[pair] = pair_score(qd, dd, Lq, len[b], d,
                                      argmax ? argmax + pair * Lq : NULL,
                                      rowmax ? rowmax + pair * Lq : NULL);
            free(qd);
            free(dd);
        }
    }
}

/*
 * Padded layout: Q [Nq, Lq, d], D [B, Ld, d]; document b has d_lens[b]
 * valid tokens (all Ld when d_lens is NULL).  Positions j >= d_lens[b] are
 * excluded before the maximum, i.e. they act as -inf (Section 4.1, Algorithm
 * 2 masking step and "Online-Max Recurrence").
 * Outputs: scores [Nq, B] (fp64), argmax [Nq, B, Lq] (may be NULL),
 * rowmax [Nq, B, Lq] (per query token maximum, may be NULL).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_fwd_padded(const uint16_t* Q, const uint16_t* D, const int32_t* d_lens, int dtype,
                      int Nq, int Lq, int B, int Ld, int d, double* scores, int32_t* argmax,
                      double* rowmax) {
    if (Nq < 0 || Lq < 0 || B < 0 || Ld < 0 || d <= 0) return -1;
    int64_t* first = (int64_t*)malloc(sizeof(int64_t) * (B + 1));
    int32_t* len = (int32_t*)malloc(sizeof(int32_t) * (B + 1));
    for (int b = 0; b < B; ++b) {
        first[b] = (int64_t)b * Ld;
        len[b] = d_lens ? d_lens[b] : Ld;
        if (len[b] < 0 || len[b] > Ld) {
            free(first);
            free(len);
            return -1;
        }
    }
    fwd_docs(Q, D, dtype, first, len, Nq, Lq, B, d, scores, argmax, rowmax);
    free(first);
    free(len);
    return 0;
}

/*
 * Packed layout (Section 4.3 "Padding-Free Variable-Length"): D holds the
 * T = cu_seqlens[B] real tokens of all documents back to back, document b
 * being tokens [cu_seqlens[b], cu_seqlens[b+1]).  argmax is local to the
 * document, in [0, length).
 */
int oracle_fwd_varlen(const uint16_t* Q, const uint16_t* D, const int32_t* cu_seqlens, int dtype,
                      int Nq, int Lq, int B, int d, double* scores, int32_t* argmax,
                      double* rowmax) {
    if (Nq < 0 || Lq < 0 || B < 0 || d <= 0 || cu_seqlens[0] != 0) return -1;
    int64_t* first = (int64_t*)malloc(sizeof(int64_t) * (B + 1));
    int32_t* len = (int32_t*)malloc(sizeof(int32_t) * (B + 1));
    for (int b = 0; b < B; ++b) {
        first[b] = cu_seqlens[b];
        len[b] = cu_seqlens[b + 1] - cu_seqlens[b];
        if (len[b] < 0) {
            free(first);
            free(len);
            return -1;
        }
    }
    fwd_docs(Q, D, dtype, first, len, Nq, Lq, B, d, scores, argmax, rowmax);
    free(first);
    free(len);
    return 0;
}

/*
 * <Q[q, i], D[doc b, token j]> in fp64 for j = sel[q, b, i] (the
 * similarity at a given index, e.g. an argmax produced elsewhere).  Documents
 * are packed by cu_seqlens.  Entries with sel < 0 or sel >= length give -inf.
 */
int oracle_sim_at(const uint16_t* Q, const uint16_t* D, const int32_t* cu_seqlens, int dtype,
                  int Nq, int Lq, int B, int d, const int32_t* sel, double* out) {
#pragma omp parallel for schedule(static) collapse(2)
    for (int q = 0; q < Nq; ++q) {
        for (int b = 0; b < B; ++b) {
            int len = cu_seqlens[b + 1] - cu_seqlens[b];
            for (int i = 0; i < Lq; ++i) {
                int64_t o = ((int64_t)q * B + b) * Lq + i;
                int j = sel[o];
                if (j < 0 || j >= len) {
                    out[o] = -INFINITY;
                    continue;
                }
                double s = 0.0;
                for (int k = 0; k < d; ++k)
                    s += decode(Q[((int64_t)q * Lq + i) * d + k], dtype) *
                         decode(D[((int64_t)cu_seqlens[b] + j) * d + k], dtype);
                out[o] = s;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Forward, INT8 x INT8.                                                */
/* ------------------------------------------------------------------ */

/*
 * Section 4.3 "INT8xINT8 Quantization": both Q and D are quantised per
 * token, symmetrically, and the dequantisation is fused into the scoring.
 * The page does not fix the arithmetic; the reading used here is the
 * quantised Eq. (1):
 *     dot_ij = sum_k q_ik * d_jk              (exact integer)
 *     s_ij   = fl32( (float)dot_ij * d_scale_j )
 *     m_i    = max_j s_ij                      (first j on ties)
 *     v_i    = fl32( m_i * q_scale_i )
 *     score  = (((v_0 + v_1) + v_2) + ...)     (fp32, ascending i)
 * |dot_ij| <= 128 * 127 * 127 < 2^24, so (float)dot_ij is exact.  The
 * per-query scale is positive, so applying it after the maximum gives the
 * same value as applying it inside.
 * Q [Nq, Lq, d] int8, q_scale [Nq, Lq]; D packed [T, d] int8, d_scale [T];
 * cu_seqlens [B+1].  Outputs scores [Nq, B] fp32, argmax [Nq, B, Lq].
 */
int oracle_fwd_i8(const int8_t* Q, const float* q_scale, const int8_t* D, const float* d_scale,
                  const int32_t* cu_seqlens, int Nq, int Lq, int B, int d, float* scores,
                  int32_t* argmax) {
    if (Nq < 0 || Lq < 0 || B < 0 || d <= 0 || d > 1024 || cu_seqlens[0] != 0) return -1;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int q = 0; q < Nq; ++q) {
        for (int b = 0; b < B; ++b) {
            int64_t first = cu_seqlens[b];
            int len = cu_seqlens[b + 1] - cu_seqlens[b];
            int64_t pair = (int64_t)q * B + b;
            float score = 0.0f;
            for (int i = 0; i < Lq; ++i) {
                const int8_t* qi = Q + ((int64_t)q * Lq + i) * d;
                float m = -INFINITY;
                int32_t arg = -1;
                for (int j = 0; j < len; ++j) {
                    const int8_t* dj = D + (first + j) * d;
                    int32_t dot = 0;
                    for (int k = 0; k < d; ++k) dot += (int32_t)qi[k] * (int32_t)dj[k];
                    float s = (float)dot * d_scale[first + j];
                    if (s > m) {
                        m = s;
                        arg = j;
                    }
                }
                float v = m * q_scale[(int64_t)q * Lq + i];
                score = score + v;
                if (argmax) argmax[pair * Lq + i] = arg;
            }
            scores[pair] = score;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Backward.                                                            */
/* ------------------------------------------------------------------ */

/*
 * Inverse-grid CSR map, Section 4.2 "Runtime Inverse-Grid Construction" and
 * Algorithm 3 step 1, padded documents of Ld tokens:
 *   source s = (q * B + b) * Lq + i   (flat index into argmax [Nq, B, Lq]),
 *   dst(s)   = b * Ld + argmax[s],
 *   row_ptr  = exclusive prefix sum of bincount(dst) over the B*Ld rows,
 *              length B*Ld + 1, row_ptr[0] = 0,
 *   col_idx  = stable argsort of dst: within each row the sources appear in
 *              ascending s.
 * A negative argmax entry is what the forward writes for a document with no
 * valid token (d_lens[b] = 0: the running maximum never leaves -inf, Section
 * 4.1 "Online-Max Recurrence"); such a source selects no row and appears in
 * no bucket, so row_ptr[B*Ld] is the number of sources with argmax >= 0.
 * The stable argsort is written as a counting sort that visits s in
 * ascending order.  Returns 0, or -1 if some argmax is >= Ld.
 */
int oracle_csr_build(const int32_t* argmax, int Nq, int B, int Lq, int Ld, int32_t* row_ptr,
                     int32_t* col_idx) {
    int64_t nsrc = (int64_t)Nq * B * Lq;
    int64_t ndst = (int64_t)B * Ld;
    int64_t* cnt = (int64_t*)calloc((size_t)ndst + 1, sizeof(int64_t));
    for (int64_t s = 0; s < nsrc; ++s) {
        int64_t b = (s / Lq) % B;
        int32_t t = argmax[s];
        if (t < 0) continue; /* selects no row */
        if (t >= Ld) {
            free(cnt);
            return -1;
        }
        cnt[b * Ld + t] += 1;
    }
    row_ptr[0] = 0;
    for (int64_t r = 0; r < ndst; ++r) row_ptr[r + 1] = (int32_t)(row_ptr[r] + cnt[r]);
    int64_t* cursor = cnt; /* reuse: next free slot of every row */
    for (int64_t r = 0; r < ndst; ++r) cursor[r] = row_ptr[r];
    for (int64_t s = 0; s < nsrc; ++s) { /* ascending s: a stable fill */
        int64_t b = (s / Lq) % B;
        if (argmax[s] < 0) continue;
        int64_t dst = b * Ld + argmax[s];
        col_idx[cursor[dst]] = (int32_t)s;
        cursor[dst] += 1;
    }
    free(cnt);
    return 0;
}

/*
 * Closed-form gradients, Section 4.2 "Closed-Form Gradients", Eqs. (dq) and
 * (dd), with g = dL/dscore [Nq, B] and the saved winner t* = argmax[q, b, i]:
 *   dQ[q, i, :] = sum_b g[q, b] * D[b, t*(q, b, i), :]
 *   dD[b, t, :] = sum over (q, i) with t*(q, b, i) = t of g[q, b] * Q[q, i, :]
 * Written as the plain definition: one pass over every (q, b, i), adding to
 * the selected rows, in fp64.  Rows of dD that no query token selects stay
 * exactly zero.  A source whose argmax is negative (a document with no valid
 * token) selects no row and adds nothing, as in oracle_csr_build.
 * Q [Nq, Lq, d], D [B, Ld, d] (fp16 / bf16), argmax [Nq, B, Lq], g [Nq, B]
 * fp32.  Outputs dQ [Nq, Lq, d], dD [B, Ld, d] fp64.  Returns -1 if some
 * argmax is >= Ld.
 */
int oracle_bwd(const uint16_t* Q, const uint16_t* D, int dtype, const int32_t* argmax,
               const float* g, int Nq, int Lq, int B, int Ld, int d, double* dQ, double* dD) {
    for (int64_t s = 0; s < (int64_t)Nq * B * Lq; ++s)
        if (argmax[s] >= Ld) return -1;
    memset(dQ, 0, sizeof(double) * (size_t)Nq * Lq * d);
    memset(dD, 0, sizeof(double) * (size_t)B * Ld * d);
    for (int q = 0; q < Nq; ++q) {
        for (int b = 0; b < B; ++b) {
            double gqb = (double)g[(int64_t)q * B + b];
            for (int i = 0; i < Lq; ++i) {
                int t = argmax[((int64_t)q * B + b) * Lq + i];
                if (t < 0) continue;
                const uint16_t* qrow = Q + ((int64_t)q * Lq + i) * d;
                const uint16_t* drow = D + ((int64_t)b * Ld + t) * d;
                double* dq = dQ + ((int64_t)q * Lq + i) * d;
                double* ddr = dD + ((int64_t)b * Ld + t) * d;
                for (int k = 0; k < d; ++k) {
                    dq[k] += gqb * decode(drow[k], dtype);
                    ddr[k] += gqb * decode(qrow[k], dtype);
                }
            }
        }
    }
    return 0;
}

/*
 * The backward over a packed (cu_seqlens) corpus: Section 4.2 Algorithm 3
 * with the destination row of source s = (q*B + b)*Lq + i read as
 * dst(s) = cu_seqlens[b] + argmax[s] (the packed row of the selected token;
 * Section 4.3 "Padding-Free Variable-Length" keeps only real tokens).  An
 * empty document (its argmax is -1) has no rows: its sources select nothing,
 * add nothing to dQ and appear in no CSR row.
 *   row_ptr [T + 1]: exclusive prefix sum of the per-row counts (row_ptr[T]
 *                    is the number of sources that select a row),
 *   col_idx [row_ptr[T]]: stable argsort of dst over those sources.
 * Returns 0, or -1 if an argmax of a non-empty document is out of range.
 */
int oracle_csr_build_varlen(const int32_t* argmax, int Nq, int B, int Lq, const int32_t* cu_seqlens,
                            int32_t* row_ptr, int32_t* col_idx) {
    const int64_t nsrc = (int64_t)Nq * B * Lq;
    const int64_t T = cu_seqlens[B];
    int64_t* cnt = (int64_t*)calloc((size_t)T + 1, sizeof(int64_t));
    for (int64_t s = 0; s < nsrc; ++s) {
        const int64_t b = (s / Lq) % B;
        const int len = cu_seqlens[b + 1] - cu_seqlens[b];
        if (len == 0) continue;
        const int32_t t = argmax[s];
        if (t < 0 || t >= len) {
            free(cnt);
            return -1;
        }
        cnt[cu_seqlens[b] + t] += 1;
    }
    row_ptr[0] = 0;
    for (int64_t r = 0; r < T; ++r) row_ptr[r + 1] = (int32_t)(row_ptr[r] + cnt[r]);
    int64_t* cursor = cnt;
    for (int64_t r = 0; r < T; ++r) cursor[r] = row_ptr[r];
    for (int64_t s = 0; s < nsrc; ++s) {
        const int64_t b = (s / Lq) % B;
        if (cu_seqlens[b + 1] == cu_seqlens[b]) continue;
        const int64_t dst = cu_seqlens[b] + argmax[s];
        col_idx[cursor[dst]] = (int32_t)s;
        cursor[dst] += 1;
    }
    free(cnt);
    return 0;
}

/*
 * Closed-form gradients (Section 4.2, Eqs. (dq), (dd)) over a packed corpus:
 *   dQ[q, i, :] = sum over non-empty b of g[q, b] * D_packed[cu[b] + t*, :]
 *   dD[cu[b] + t, :] = sum over (q, i) with t*(q, b, i) = t of g[q, b] * Q[q, i, :]
 * The plain definition in fp64, as oracle_bwd.  D_packed [T, d], dD [T, d].
 */
int oracle_bwd_varlen(const uint16_t* Q, const uint16_t* D, const int32_t* cu_seqlens, int dtype,
                      const int32_t* argmax, const float* g, int Nq, int Lq, int B, int d, double* dQ,
                      double* dD) {
    const int64_t T = cu_seqlens[B];
    for (int q = 0; q < Nq; ++q)
        for (int b = 0; b < B; ++b) {
            const int len = cu_seqlens[b + 1] - cu_seqlens[b];
            for (int i = 0; i < Lq; ++i) {
                const int32_t t = argmax[((int64_t)q * B + b) * Lq + i];
                if (len > 0 && (t < 0 || t >= len)) return -1;
            }
        }
    memset(dQ, 0, sizeof(double) * (size_t)Nq * Lq * d);
    memset(dD, 0, sizeof(double) * (size_t)T * d);
    for (int q = 0; q < Nq; ++q) {
        for (int b = 0; b < B; ++b) {
            if (cu_seqlens[b + 1] == cu_seqlens[b]) continue;
            const double gqb = (double)g[(int64_t)q * B + b];
            for (int i = 0; i < Lq; ++i) {
                const int64_t row = cu_seqlens[b] + argmax[((int64_t)q * B + b) * Lq + i];
                const uint16_t* qrow = Q + ((int64_t)q * Lq + i) * d;
                const uint16_t* drow = D + row * d;
                double* dq = dQ + ((int64_t)q * Lq + i) * d;
                double* ddr = dD + row * d;
                for (int k = 0; k < d; ++k) {
                    dq[k] += gqb * decode(drow[k], dtype);
                    ddr[k] += gqb * decode(qrow[k], dtype);
                }
            }
        }
    }
    return 0;
}

/*
 * Scores of an explicit list of (query, document) pairs over the packed
 * corpus: pair p is query pq[p] against document pb[p] (Eq. (1), the same
 * definition as oracle_fwd_varlen, evaluated only for the listed pairs).
 * This is the rescoring step of the two-stage scan the pages list in the
 * forward kernel family (Section 4.1 "Kernel Family": an INT8 pass ranks the
 * corpus, the candidates are scored again in fp16).
 * Outputs: scores [P] (fp64), argmax [P, Lq] (may be NULL).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_fwd_pairs(const uint16_t* Q, const uint16_t* D, const int32_t* cu_seqlens, int dtype,
                     const int32_t* pq, const int32_t* pb, int P, int Nq, int Lq, int B, int d,
                     double* scores, int32_t* argmax) {
    if (!Q || !cu_seqlens || !pq || !pb || !scores || P < 0 || Nq < 1 || Lq < 1 || B < 1 || d < 1) return -1;
    for (int p = 0; p < P; ++p)
        if (pq[p] < 0 || pq[p] >= Nq || pb[p] < 0 || pb[p] >= B) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int p = 0; p < P; ++p) {
        const int q = pq[p], b = pb[p];
        const int64_t first = cu_seqlens[b];
        const int len = cu_seqlens[b + 1] - cu_seqlens[b];
        double* qd = (double*)malloc(sizeof(double) * (size_t)Lq * d);
        double* dd = (double*)malloc(sizeof(double) * ((size_t)len * d + 1));
        for (int64_t e = 0; e < (int64_t)Lq * d; ++e) qd[e] = decode(Q[(int64_t)q * Lq * d + e], dtype);
        for (int64_t e = 0; e < (int64_t)len * d; ++e) dd[e] = decode(D[first * d + e], dtype);
        scores[p] = pair_score(qd, dd, Lq, len, d, argmax ? argmax + (int64_t)p * Lq : NULL, NULL);
        free(qd);
        free(dd);
    }
    return 0;
}

/*
 * Top-K of each query's row of scores [Nq, B]: the K documents with the
 * largest scores, best first; equal scores are ordered by ascending document
 * index (the selection the two-stage scan keeps, Section 4.1 "Kernel
 * Family").  A full sort per query: plain and slow.
 * Outputs: idx [Nq, K], val [Nq, K].  Returns 0, or -1 on a bad argument.
 */
static const float* topk_row;
static int topk_cmp(const void* a, const void* b) {
    const int32_t i = *(const int32_t*)a, j = *(const int32_t*)b;
    const float si = topk_row[i], sj = topk_row[j];
    if (si > sj) return -1;
    if (si < sj) return 1;
    return (i > j) - (i < j);
}
int oracle_topk(const float* scores, int Nq, int B, int K, int32_t* idx, float* val) {
    if (!scores || !idx || !val || Nq < 1 || B < 1 || K < 1 || K > B) return -1;
    int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
    for (int q = 0; q < Nq; ++q) {
        for (int b = 0; b < B; ++b) order[b] = b;
        topk_row = scores + (int64_t)q * B;
        qsort(order, (size_t)B, sizeof(int32_t), topk_cmp);
        for (int k = 0; k < K; ++k) {
            idx[(int64_t)q * K + k] = order[k];
            val[(int64_t)q * K + k] = topk_row[order[k]];
        }
    }
    free(order);
    return 0;
}

/* Number of OpenMP threads a parallel region of the oracle uses. */
int oracle_num_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/* ------------------------------------------------------------------ */
/* Chamfer distance (Section 4.2, "Generalization to Chamfer Distance"). */
/* ------------------------------------------------------------------ */
/*
 * The same hard-selection structure with a minimum of squared Euclidean
 * distances in place of the maximum of inner products, between two point
 * sets in R^3.  Clouds come in batches: A [Bt, Na, 3] and B [Bt, Nb, 3]
 * (fp32), and batch item b of A is only compared with item b of B.
 */

/* For every point s of A[b]: dist = min over t of |A[b,s] - B[b,t]|^2 and
 * idx = the first t attaining it (fp64 from the fp32 coordinates, the three
 * squares added in x, y, z order).  An empty B gives +inf and -1. */
int oracle_chamfer_nn(const float* A, const float* B, int Bt, int Na, int Nb, double* dist, int32_t* idx) {
    if (Bt < 0 || Na < 0 || Nb < 0) return 1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t s = 0; s < (int64_t)Bt * Na; ++s) {
        const int64_t b = s / Na;
        const float* a = A + s * 3;
        double best = INFINITY;
        int32_t arg = -1;
        for (int t = 0; t < Nb; ++t) {
            const float* p = B + (b * Nb + t) * 3;
            const double dx = (double)a[0] - (double)p[0];
            const double dy = (double)a[1] - (double)p[1];
            const double dz = (double)a[2] - (double)p[2];
            const double dd = dx * dx + dy * dy + dz * dz;
            if (dd < best) {
                best = dd;
                arg = t;
            }
        }
        dist[s] = best;
        idx[s] = arg;
    }
    return 0;
}

/* The inverse map of a nearest-neighbour selection (Section 4.2
 * "Runtime Inverse-Grid Construction" applied to the argmin): source
 * s = b*Na + i selects destination b*Nb + idx[b,i]; row_ptr [Bt*Nb + 1] is
 * the exclusive prefix of the per-destination counts and col_idx lists each
 * destination's sources in ascending s.  Sources with idx = -1 select
 * nothing; col_idx has row_ptr[Bt*Nb] entries. */
int oracle_chamfer_csr(const int32_t* idx, int Bt, int Na, int Nb, int32_t* row_ptr, int32_t* col_idx) {
    if (Bt < 0 || Na < 0 || Nb < 0) return 1;
    const int64_t nd = (int64_t)Bt * Nb;
    int64_t* cnt = calloc(nd + 1, sizeof(int64_t));
    if (!cnt) return 2;
    for (int64_t s = 0; s < (int64_t)Bt * Na; ++s) {
        if (idx[s] < 0) continue;
        if (idx[s] >= Nb) { free(cnt); return 3; }
        cnt[(s / Na) * Nb + idx[s]] += 1;
    }
    int64_t run = 0;
    for (int64_t r = 0; r < nd; ++r) {
        row_ptr[r] = (int32_t)run;
        run += cnt[r];
        cnt[r] = row_ptr[r];  /* now the fill cursor of row r */
    }
    row_ptr[nd] = (int32_t)run;
    for (int64_t s = 0; s < (int64_t)Bt * Na; ++s) {  /* ascending s: a stable fill */
        if (idx[s] < 0) continue;
        const int64_t r = (s / Na) * Nb + idx[s];
        col_idx[cnt[r]] = (int32_t)s;
        cnt[r] += 1;
    }
    free(cnt);
    return 0;
}

/* Gradients of L = sum_i gp[b,i] * distP[b,i] + sum_j gq[b,j] * distQ[b,j]
 * with the selections fixed (the saved argmins), distP from P to its nearest
 * point of Q and distQ from Q to its nearest point of P:
 *   dP[b,i] = 2 gp[b,i] (P[b,i] - Q[b,idx_p[b,i]])
 *           + sum over j with idx_q[b,j] = i of 2 gq[b,j] (P[b,i] - Q[b,j])
 *   dQ[b,j] = 2 gq[b,j] (Q[b,j] - P[b,idx_q[b,j]])
 *           + sum over i with idx_p[b,i] = j of 2 gp[b,i] (Q[b,j] - P[b,i])
 * The sums run over the selecting points in ascending order.  The Chamfer
 * loss of the page is gp = 1/N, gq = 1/M.  Selections of -1 add nothing. */
int oracle_chamfer_bwd(const float* P, const float* Q, int Bt, int N, int M, const int32_t* idx_p,
                       const int32_t* idx_q, const float* gp, const float* gq, double* dP, double* dQ) {
    if (Bt < 0 || N < 0 || M < 0) return 1;
    memset(dP, 0, sizeof(double) * (size_t)Bt * N * 3);
    memset(dQ, 0, sizeof(double) * (size_t)Bt * M * 3);
    for (int b = 0; b < Bt; ++b) {
        /* P's own terms, and what each P point adds to the Q point it selects */
        for (int i = 0; i < N; ++i) {
            const int64_t pi = (int64_t)b * N + i;
            const int32_t j = idx_p[pi];
            if (j < 0) continue;
            if (j >= M) return 3;
            const int64_t qj = (int64_t)b * M + j;
            const double w = 2.0 * (double)gp[pi];
            for (int k = 0; k < 3; ++k) {
                const double diff = (double)P[pi * 3 + k] - (double)Q[qj * 3 + k];
                dP[pi * 3 + k] += w * diff;
                dQ[qj * 3 + k] -= w * diff;
            }
        }
        /* Q's own terms, and what each Q point adds to the P point it selects */
        for (int j = 0; j < M; ++j) {
            const int64_t qj = (int64_t)b * M + j;
            const int32_t i = idx_q[qj];
            if (i < 0) continue;
            if (i >= N) return 3;
            const int64_t pi = (int64_t)b * N + i;
            const double w = 2.0 * (double)gq[qj];
            for (int k = 0; k < 3; ++k) {
                const double diff = (double)Q[qj * 3 + k] - (double)P[pi * 3 + k];
                dQ[qj * 3 + k] += w * diff;
                dP[pi * 3 + k] -= w * diff;
            }
        }
    }
    return 0;
}

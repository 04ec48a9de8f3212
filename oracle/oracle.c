/*
 * oracle.c -- plain, slow, fp64 CPU attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness oracle for the GPU
 * path: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no code, header, table or helper with the GPU
 * library, and the GPU library never calls it.
 *
 * What it computes is the plain definition of softmax attention, row by row,
 * with no tiling, no running statistics and no reordering beyond what the
 * definition states:
 *
 *   s_ij = scale * <q_i, k_j>                      for every allowed key j
 *   m_i  = max_j s_ij
 *   e_ij = exp(s_ij - m_i),  l_i = sum_j e_ij       (stable softmax)
 *   P_ij = e_ij / l_i
 *   O_i  = sum_j P_ij v_j
 *   L_i  = m_i + ln(l_i)
 *
 * Sources (the FlashAttention pages): the naive attention listing on the
 * ai-engineering wiki page, section "The Core Problem" (scores = QK^T/sqrt(d),
 * softmax, weights @ V); tensortonic "FlashAttention" section 1 (weights sum to
 * one and combine the value vectors; a causal mask forbids future positions),
 * section 4 (stable softmax subtracts the row maximum), section 6 (the scale
 * is 1/sqrt(width); causal masking before the softmax) and section 7 (the
 * saved row statistic L = m + log(l) is the log of the full row's exponential
 * sum).  FlashAttention is exact (tensortonic section 8; nexusofnerds FAQ), so
 * the definition is the right oracle for the tiled kernel.
 *
 * Readings where the pages are silent (each listed in the design doc):
 *  - causal allows j <= i (a token may read itself);
 *  - the scale is applied to the dot product, in fp64 here;
 *  - L uses the natural logarithm, in units of scaled scores;
 *  - a row with no allowed key gets O = 0 and L = -inf (reached only when
 *    there are more queries than keys under the bottom-right causal mask);
 *  - queries and keys of different lengths (tensortonic section 9 warns that
 *    the square causal mask is not right for every unequal-length layout):
 *    the queries are the last Nq positions of a sequence whose keys are all
 *    Nk positions, so query i sits at position i + Nk - Nq and, under the
 *    causal mask, reads keys j <= i + Nk - Nq (the mask aligned bottom-right;
 *    for Nq = Nk it is the square mask);
 *  - the backward pass is the exact vector-Jacobian product of this forward
 *    map (the pages give only "weight = exp(s_ij - L_i)" and that each tile
 *    contributes to dQ, dK and dV): with dP_ij = <dO_i, v_j> and
 *    Dsum_i = sum_j P_ij dP_ij,
 *        dS_ij = P_ij (dP_ij - Dsum_i),
 *        dQ_i  = scale * sum_j dS_ij k_j,
 *        dK_j  = scale * sum_i dS_ij q_i,
 *        dV_j  = sum_i P_ij dO_i.
 *
 * Layouts: dense tensors are [B, H, N, D] row-major (tensortonic section 9:
 * [batch, heads, tokens, head_width]); LSE is [B, H, N].  Packed
 * variable-length tensors are [H, total, D] with int32 offsets cu[0..nseq],
 * LSE [H, total]; positions are relative to each sequence start and no
 * attention crosses a sequence boundary (nexusofnerds: variable-length
 * packing).
 *
 * Attention dropout (tensortonic section 7: with dropout enabled the backward
 * pass must reproduce the forward pass's drop decisions from saved generator
 * state; it may not draw a new mask).  The weights become
 * P~_ij = P_ij * keep_ij / (1 - p'), O_i = sum_j P~_ij v_j, while L keeps the
 * log-sum-exp of the undropped scores.  The pages fix no generator, so this
 * library defines the decisions (a reading, listed in the design doc) with the
 * counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011), implemented below
 * from that paper's definition:
 *   - one call maps a 128-bit counter (c0, c1, c2, c3) and a 64-bit key
 *     (k0, k1) to 128 bits through ten rounds; a round forms the 64-bit
 *     products 0xD2511F53 * c0 = (hi0, lo0) and 0xCD9E8D57 * c2 = (hi1, lo1)
 *     and yields (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); between rounds
 *     the key advances by (0x9E3779B9, 0xBB67AE85);
 *   - query i and key j of head bh (= b*H + h) use the call with counter
 *     (j / 4, i / 4, bh, offset mod 2^32) and key (seed mod 2^32,
 *     seed / 2^32); byte j % 4 of output word i % 4 is u;
 *   - key j is kept for query i iff u >= T, T = min(255, round(256 p)), so
 *     the dropout probability is p' = T / 256 and kept weights are scaled by
 *     256 / (256 - T).
 * The generator's output stream is pinned by the known-answer vectors
 * published with Philox4x32-10 (tests/golden/philox4x32_10_kat.txt); the
 * tests also check its statistics and pin every use of it.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared oracle.c -lm   (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static double dot(const double* a, const double* b, int64_t n) {
    double acc = 0.0;
    for (int64_t t = 0; t < n; ++t) acc += a[t] * b[t];
    return acc;
}

/*
 * One query row against keys/values k[0..nk), v[0..nk) (row stride D).
 * s is scratch of length >= nk.  Writes o_i[0..D) and *lse_i.
 */
static void attend_row(const double* q_i, const double* k, const double* v,
                       int64_t nk, int64_t D, double scale, double* s,
                       double* o_i, double* lse_i) {
    for (int64_t d = 0; d < D; ++d) o_i[d] = 0.0;
    if (nk <= 0) {
        *lse_i = -INFINITY;
        return;
    }
    /* scores for every allowed key */
    double m = -INFINITY;
    for (int64_t j = 0; j < nk; ++j) {
        s[j] = scale * dot(q_i, k + j * D, D);
        if (s[j] > m) m = s[j];
    }
    /* stable softmax: shift by the row maximum, exponentiate, sum */
    double l = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    /* normalised weights, then the weighted sum of the value rows */
    for (int64_t j = 0; j < nk; ++j) {
        const double p = s[j] / l;
        const double* v_j = v + j * D;
        for (int64_t d = 0; d < D; ++d) o_i[d] += p * v_j[d];
    }
    *lse_i = m + log(l);
}

/* Number of keys row i may read: all n, or 0..i under the causal mask. */
static int64_t allowed_keys(int64_t i, int64_t n, int causal) {
    return causal ? (i + 1 < n ? i + 1 : n) : n;
}

/* Dense forward: q, k, v, o are [B, H, N, D]; lse is [B, H, N]. */
int oracle_attn_fwd(const double* q, const double* k, const double* v,
                    double* o, double* lse, int64_t B, int64_t H, int64_t N,
                    int64_t D, double scale, int causal) {
    if (B < 0 || H < 0 || N < 0 || D <= 0) return 1;
    const int64_t rows = B * H * N;
    int fail = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r) {
                const int64_t bh = r / N, i = r % N;
                const int64_t base = bh * N * D;
                attend_row(q + base + i * D, k + base, v + base,
                           allowed_keys(i, N, causal), D, scale, s,
                           o + base + i * D, lse + bh * N + i);
            }
            free(s);
        }
    }
    return fail;
}

/*
 * Selected rows of the dense forward.  For t in [0, nrows): head bh[t]
 * (= b*H + h) and query row row[t].  Writes o_rows[t*D..] and lse_rows[t].
 */
int oracle_attn_fwd_rows(const double* q, const double* k, const double* v,
                         const int64_t* bh, const int64_t* row, int64_t nrows,
                         double* o_rows, double* lse_rows, int64_t B, int64_t H,
                         int64_t N, int64_t D, double scale, int causal) {
    for (int64_t t = 0; t < nrows; ++t)
        if (bh[t] < 0 || bh[t] >= B * H || row[t] < 0 || row[t] >= N) return 2;
    int fail = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < nrows; ++t) {
                const int64_t base = bh[t] * N * D, i = row[t];
                attend_row(q + base + i * D, k + base, v + base,
                           allowed_keys(i, N, causal), D, scale, s,
                           o_rows + t * D, lse_rows + t);
            }
            free(s);
        }
    }
    return fail;
}

/*
 * Keys row i of Nq queries may read out of Nk: all of them, or under the
 * causal mask those at positions <= i + Nk - Nq (bottom-right alignment).
 */
static int64_t allowed_keys_qk(int64_t i, int64_t nq, int64_t nk, int causal) {
    if (!causal) return nk;
    const int64_t last = i + nk - nq;  /* last readable key position */
    return last < 0 ? 0 : (last + 1 < nk ? last + 1 : nk);
}

/*
 * Forward with Nq queries against Nk keys: q, o are [B, H, Nq, D], k, v are
 * [B, H, Nk, D], lse is [B, H, Nq].
 */
int oracle_attn_fwd_qk(const double* q, const double* k, const double* v,
                       double* o, double* lse, int64_t B, int64_t H, int64_t Nq,
                       int64_t Nk, int64_t D, double scale, int causal) {
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || D <= 0) return 1;
    const int64_t rows = B * H * Nq;
    int fail = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r) {
                const int64_t bh = r / Nq, i = r % Nq;
                attend_row(q + (bh * Nq + i) * D, k + bh * Nk * D, v + bh * Nk * D,
                           allowed_keys_qk(i, Nq, Nk, causal), D, scale, s,
                           o + (bh * Nq + i) * D, lse + bh * Nq + i);
            }
            free(s);
        }
    }
    return fail;
}

/* Selected rows of oracle_attn_fwd_qk (head bh[t] = b*H + h, query row[t]). */
int oracle_attn_fwd_qk_rows(const double* q, const double* k, const double* v,
                            const int64_t* bh, const int64_t* row, int64_t nrows,
                            double* o_rows, double* lse_rows, int64_t B, int64_t H,
                            int64_t Nq, int64_t Nk, int64_t D, double scale,
                            int causal) {
    for (int64_t t = 0; t < nrows; ++t)
        if (bh[t] < 0 || bh[t] >= B * H || row[t] < 0 || row[t] >= Nq) return 2;
    int fail = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < nrows; ++t) {
                const int64_t i = row[t];
                attend_row(q + (bh[t] * Nq + i) * D, k + bh[t] * Nk * D,
                           v + bh[t] * Nk * D, allowed_keys_qk(i, Nq, Nk, causal), D,
                           scale, s, o_rows + t * D, lse_rows + t);
            }
            free(s);
        }
    }
    return fail;
}

/* Validate packed offsets: cu[0] = 0, non-decreasing, cu[nseq] = total. */
static int check_cu(const int32_t* cu, int64_t nseq, int64_t total) {
    if (nseq < 0 || cu[0] != 0 || cu[nseq] != total) return 3;
    for (int64_t b = 0; b < nseq; ++b)
        if (cu[b + 1] < cu[b]) return 3;
    return 0;
}

/* Sequence that holds packed token t (cu validated). */
static int64_t seq_of(const int32_t* cu, int64_t nseq, int64_t t) {
    int64_t lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/*
 * Packed variable-length forward: q, k, v, o are [H, total, D]; lse is
 * [H, total].  Sequence b holds tokens [cu[b], cu[b+1]); row i of it reads
 * keys of the same sequence only (positions relative to cu[b]).
 */
int oracle_attn_fwd_varlen(const double* q, const double* k, const double* v,
                           double* o, double* lse, const int32_t* cu,
                           int64_t nseq, int64_t H, int64_t total, int64_t D,
                           double scale, int causal) {
    if (check_cu(cu, nseq, total)) return 3;
    int64_t maxlen = 1;
    for (int64_t b = 0; b < nseq; ++b)
        if (cu[b + 1] - cu[b] > maxlen) maxlen = cu[b + 1] - cu[b];
    const int64_t rows = H * total;
    int fail = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)maxlen);
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r) {
                const int64_t h = r / total, t = r % total;
                const int64_t b = seq_of(cu, nseq, t);
                const int64_t start = cu[b], n = cu[b + 1] - cu[b];
                const int64_t base = (h * total + start) * D;
                const int64_t i = t - start;
                attend_row(q + base + i * D, k + base, v + base,
                           allowed_keys(i, n, causal), D, scale, s,
                           o + base + i * D, lse + h * total + t);
            }
            free(s);
        }
    }
    return fail;
}

/* Selected rows of the packed forward: head h[t], packed token tok[t]. */
int oracle_attn_fwd_varlen_rows(const double* q, const double* k,
                                const double* v, const int32_t* cu,
                                int64_t nseq, int64_t H, int64_t total,
                                int64_t D, double scale, int causal,
                                const int64_t* h, const int64_t* tok,
                                int64_t nrows, double* o_rows,
                                double* lse_rows) {
    if (check_cu(cu, nseq, total)) return 3;
    for (int64_t t = 0; t < nrows; ++t)
        if (h[t] < 0 || h[t] >= H || tok[t] < 0 || tok[t] >= total) return 2;
    int64_t maxlen = 1;
    for (int64_t b = 0; b < nseq; ++b)
        if (cu[b + 1] - cu[b] > maxlen) maxlen = cu[b + 1] - cu[b];
    int fail = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)maxlen);
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < nrows; ++t) {
                const int64_t b = seq_of(cu, nseq, tok[t]);
                const int64_t start = cu[b], n = cu[b + 1] - cu[b];
                const int64_t base = (h[t] * total + start) * D;
                const int64_t i = tok[t] - start;
                attend_row(q + base + i * D, k + base, v + base,
                           allowed_keys(i, n, causal), D, scale, s,
                           o_rows + t * D, lse_rows + t);
            }
            free(s);
        }
    }
    return fail;
}

/*
 * Dense backward: the exact gradient of <dout, O> with respect to q, k, v.
 * All tensors [B, H, N, D].  For each head the full N x N weight matrix P and
 * the score gradient dS are held in memory (this is the plain, unfused
 * computation the pages contrast FlashAttention with); rows are processed in
 * parallel for P, dS and dQ, then key columns in parallel for dK and dV.
 */
int oracle_attn_bwd(const double* q, const double* k, const double* v,
                    const double* dout, double* dq, double* dk, double* dv,
                    int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                    int causal) {
    if (B < 0 || H < 0 || N < 0 || D <= 0) return 1;
    if (N == 0) return 0;
    double* P = (double*)malloc(sizeof(double) * (size_t)(N * N));
    double* dS = (double*)malloc(sizeof(double) * (size_t)(N * N));
    if (!P || !dS) {
        free(P);
        free(dS);
        return 1;
    }
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t base = bh * N * D;
        const double *qh = q + base, *kh = k + base, *vh = v + base;
        const double* doh = dout + base;
        double *dqh = dq + base, *dkh = dk + base, *dvh = dv + base;
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t i = 0; i < N; ++i) {
            const int64_t nk = allowed_keys(i, N, causal);
            double* p = P + i * N;
            double* ds = dS + i * N;
            /* forward weights of row i: P_ij = exp(s_ij - m_i) / l_i */
            double m = -INFINITY;
            for (int64_t j = 0; j < nk; ++j) {
                p[j] = scale * dot(qh + i * D, kh + j * D, D);
                if (p[j] > m) m = p[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                p[j] = exp(p[j] - m);
                l += p[j];
            }
            for (int64_t j = 0; j < nk; ++j) p[j] /= l;
            for (int64_t j = nk; j < N; ++j) p[j] = 0.0;
            /* dP_ij = <dO_i, v_j>;  softmax Jacobian: dS = P (dP - sum P dP) */
            double dsum = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                ds[j] = dot(doh + i * D, vh + j * D, D);
                dsum += p[j] * ds[j];
            }
            for (int64_t j = 0; j < nk; ++j) ds[j] = p[j] * (ds[j] - dsum);
            for (int64_t j = nk; j < N; ++j) ds[j] = 0.0;
            /* dQ_i = scale * sum_j dS_ij k_j */
            for (int64_t d = 0; d < D; ++d) dqh[i * D + d] = 0.0;
            for (int64_t j = 0; j < nk; ++j)
                for (int64_t d = 0; d < D; ++d)
                    dqh[i * D + d] += scale * ds[j] * kh[j * D + d];
        }
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t j = 0; j < N; ++j) {
            /* dV_j = sum_i P_ij dO_i ;  dK_j = scale * sum_i dS_ij q_i */
            for (int64_t d = 0; d < D; ++d) {
                dvh[j * D + d] = 0.0;
                dkh[j * D + d] = 0.0;
            }
            for (int64_t i = causal ? j : 0; i < N; ++i) {
                const double pij = P[i * N + j], dsij = dS[i * N + j];
                for (int64_t d = 0; d < D; ++d) {
                    dvh[j * D + d] += pij * doh[i * D + d];
                    dkh[j * D + d] += scale * dsij * qh[i * D + d];
                }
            }
        }
    }
    free(P);
    free(dS);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Dropout: the counter-based generator and the attention with dropped weights.
 * ------------------------------------------------------------------------- */

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
    out[0] = c[0];
    out[1] = c[1];
    out[2] = c[2];
    out[3] = c[3];
}

/* The drop threshold T for probability p (keep iff the decision byte >= T). */
int oracle_dropout_threshold(double p) {
    if (!(p > 0.0)) return 0;
    const double t = floor(p * 256.0 + 0.5);
    return t > 255.0 ? 255 : (int)t;
}

/* keep_ij of query i and key j of head bh (1 = kept). */
static int keep_bit(uint64_t seed, uint64_t offset, int64_t bh, int64_t i, int64_t j,
                    int T) {
    if (T == 0) return 1;
    const uint32_t ctr[4] = {(uint32_t)(j >> 2), (uint32_t)(i >> 2), (uint32_t)bh,
                             (uint32_t)offset};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    const uint32_t u = (out[i & 3] >> (8 * (j & 3))) & 0xFFu;
    return u >= (uint32_t)T;
}

/* The keep mask of head bh for rows [0, nq) and keys [0, nk): keep[i*nk + j]. */
int oracle_dropout_mask(uint8_t* keep, int64_t bh, int64_t nq, int64_t nk, double p,
                        uint64_t seed, uint64_t offset) {
    if (nq < 0 || nk < 0 || !(p >= 0.0 && p < 1.0)) return 1;
    const int T = oracle_dropout_threshold(p);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nq; ++i)
        for (int64_t j = 0; j < nk; ++j)
            keep[i * nk + j] = (uint8_t)keep_bit(seed, offset, bh, i, j, T);
    return 0;
}

/* Dense forward with dropout: O_i = sum_j P_ij keep_ij / (1 - p') v_j;
 * L_i = m_i + ln l_i of the undropped scores.  Slice bh of the B*H slices
 * draws its decisions as head bh_base + bh (0 for a whole batch; a packed
 * sequence b passes b * H + h for its one head). */
int oracle_attn_fwd_dropout_bh(const double* q, const double* k, const double* v, double* o,
                               double* lse, int64_t B, int64_t H, int64_t N, int64_t D,
                               double scale, int causal, double p, uint64_t seed,
                               uint64_t offset, int64_t bh_base) {
    if (B < 0 || H < 0 || N < 0 || D <= 0 || !(p >= 0.0 && p < 1.0)) return 1;
    const int T = oracle_dropout_threshold(p);
    const double inv_keep = 256.0 / (256.0 - T);
    const int64_t rows = B * H * N;
    int fail = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r) {
                const int64_t bh = r / N, i = r % N, base = bh * N * D;
                const double* q_i = q + base + i * D;
                double* o_i = o + base + i * D;
                const int64_t nk = allowed_keys(i, N, causal);
                for (int64_t d = 0; d < D; ++d) o_i[d] = 0.0;
                double m = -INFINITY, l = 0.0;
                for (int64_t j = 0; j < nk; ++j) {
                    s[j] = scale * dot(q_i, k + base + j * D, D);
                    if (s[j] > m) m = s[j];
                }
                for (int64_t j = 0; j < nk; ++j) {
                    s[j] = exp(s[j] - m);
                    l += s[j];
                }
                for (int64_t j = 0; j < nk; ++j) {
                    if (!keep_bit(seed, offset, bh_base + bh, i, j, T)) continue;
                    const double w = s[j] / l * inv_keep;
                    const double* v_j = v + base + j * D;
                    for (int64_t d = 0; d < D; ++d) o_i[d] += w * v_j[d];
                }
                lse[bh * N + i] = nk > 0 ? m + log(l) : -INFINITY;
            }
            free(s);
        }
    }
    return fail;
}

/*
 * Backward with dropout: the exact vector-Jacobian product of
 * oracle_attn_fwd_dropout with the same decisions.  With Z_ij = keep_ij /
 * (1 - p') and G_ij = <dO_i, v_j>:
 *   dV_j = sum_i P_ij Z_ij dO_i,   dP_ij = G_ij Z_ij,
 *   dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik),
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i.
 */
int oracle_attn_bwd_dropout_bh(const double* q, const double* k, const double* v,
                               const double* dout, double* dq, double* dk, double* dv,
                               int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                               int causal, double p, uint64_t seed, uint64_t offset,
                               int64_t bh_base) {
    if (B < 0 || H < 0 || N < 0 || D <= 0 || !(p >= 0.0 && p < 1.0)) return 1;
    if (N == 0) return 0;
    const int T = oracle_dropout_threshold(p);
    const double inv_keep = 256.0 / (256.0 - T);
    double* PZ = (double*)malloc(sizeof(double) * (size_t)(N * N));  /* P_ij Z_ij */
    double* dS = (double*)malloc(sizeof(double) * (size_t)(N * N));
    if (!PZ || !dS) {
        free(PZ);
        free(dS);
        return 1;
    }
    int fail = 0;
    for (int64_t bh = 0; bh < B * H && !fail; ++bh) {
        const int64_t base = bh * N * D;
        const double *qh = q + base, *kh = k + base, *vh = v + base;
        const double* doh = dout + base;
        double *dqh = dq + base, *dkh = dk + base, *dvh = dv + base;
#pragma omp parallel
        {
            double* pr = (double*)malloc(sizeof(double) * (size_t)N);   /* P_i.  */
            double* dpr = (double*)malloc(sizeof(double) * (size_t)N);  /* dP_i. */
            if (!pr || !dpr) {
#pragma omp atomic write
                fail = 1;
            } else {
#pragma omp for schedule(dynamic, 4)
                for (int64_t i = 0; i < N; ++i) {
                    const int64_t nk = allowed_keys(i, N, causal);
                    /* forward weights of row i */
                    double m = -INFINITY, l = 0.0;
                    for (int64_t j = 0; j < nk; ++j) {
                        pr[j] = scale * dot(qh + i * D, kh + j * D, D);
                        if (pr[j] > m) m = pr[j];
                    }
                    for (int64_t j = 0; j < nk; ++j) {
                        pr[j] = exp(pr[j] - m);
                        l += pr[j];
                    }
                    /* dP_ij = <dO_i, v_j> Z_ij;  dsum = sum_j P_ij dP_ij */
                    double dsum = 0.0;
                    for (int64_t j = 0; j < nk; ++j) {
                        pr[j] /= l;
                        const double z =
                            keep_bit(seed, offset, bh_base + bh, i, j, T) ? inv_keep : 0.0;
                        dpr[j] = dot(doh + i * D, vh + j * D, D) * z;
                        PZ[i * N + j] = pr[j] * z;
                        dsum += pr[j] * dpr[j];
                    }
                    for (int64_t j = 0; j < N; ++j) {
                        dS[i * N + j] = j < nk ? pr[j] * (dpr[j] - dsum) : 0.0;
                        if (j >= nk) PZ[i * N + j] = 0.0;
                    }
                    /* dQ_i = scale * sum_j dS_ij k_j */
                    for (int64_t d = 0; d < D; ++d) dqh[i * D + d] = 0.0;
                    for (int64_t j = 0; j < nk; ++j)
                        for (int64_t d = 0; d < D; ++d)
                            dqh[i * D + d] += scale * dS[i * N + j] * kh[j * D + d];
                }
            }
            free(pr);
            free(dpr);
        }
        if (fail) break;
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t j = 0; j < N; ++j) {
            /* dV_j = sum_i P_ij Z_ij dO_i ;  dK_j = scale * sum_i dS_ij q_i */
            for (int64_t d = 0; d < D; ++d) {
                dvh[j * D + d] = 0.0;
                dkh[j * D + d] = 0.0;
            }
            for (int64_t i = causal ? j : 0; i < N; ++i) {
                const double pz = PZ[i * N + j], dsij = dS[i * N + j];
                for (int64_t d = 0; d < D; ++d) {
                    dvh[j * D + d] += pz * doh[i * D + d];
                    dkh[j * D + d] += scale * dsij * qh[i * D + d];
                }
            }
        }
    }
    free(PZ);
    free(dS);
    return fail;
}

/* The dropout entry points over a whole batch: decisions of slice bh drawn as
 * head bh. */
int oracle_attn_fwd_dropout(const double* q, const double* k, const double* v, double* o,
                            double* lse, int64_t B, int64_t H, int64_t N, int64_t D,
                            double scale, int causal, double p, uint64_t seed,
                            uint64_t offset) {
    return oracle_attn_fwd_dropout_bh(q, k, v, o, lse, B, H, N, D, scale, causal, p, seed,
                                      offset, 0);
}
int oracle_attn_bwd_dropout(const double* q, const double* k, const double* v,
                            const double* dout, double* dq, double* dk, double* dv,
                            int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                            int causal, double p, uint64_t seed, uint64_t offset) {
    return oracle_attn_bwd_dropout_bh(q, k, v, dout, dq, dk, dv, B, H, N, D, scale, causal,
                                      p, seed, offset, 0);
}

/*
 * CPU oracle for exact attention — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, double-precision C. Only the test suite, the smoke check and
 * the CPU-baseline leg of the bench load this library; the GPU product path
 * never calls it. It shares no code, header or constant with the HIP kernels.
 *
 * Sources (the text of three public web pages):
 *   [P1] "What the tiling is actually constrained by" (anthology-of-the-sota,
 *        record SOTA-086), section "The formula, which the title only gestures at".
 *   [P2] TensorViz "Compute attention one tile at a time" (flash-attention
 *        model card): the walkthrough step "tiles", the three-tile "schedule"
 *        experiment and the "numericalChecks" list.
 *   [P3] "Flash attention and efficient attention — Hinglish notes" (4.1.14):
 *        "The Standard Attention Problem", "Derivation: Incremental Softmax"
 *        (Steps 1–3), "Worked example Flash Attention Forward Pass",
 *        "Backward Pass: Recomputation", "Worked example Local Attention Window".
 *
 * Tensor layout: every Q/K/V/O/dO/dQ/dK/dV array is [BH][N][d] row-major
 * double (BH = batch*heads flattened); LSE and D are [BH][N].
 *
 * Mask codes: 0 = none, 1 = causal (key j allowed iff j <= query i),
 *             2 = local band (allowed iff |i - j| <= window).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_MASK_NONE 0
#define OR_MASK_CAUSAL 1
#define OR_MASK_LOCAL 2

/* Which (query i, key j) pairs take part. The band form follows P3's
 * "Worked example Local Attention Window" (each token sees itself and its
 * neighbours within the radius); causal is the usual lower-triangular
 * reading, top-left aligned, diagonal included. */
int oracle_allowed(int64_t i, int64_t j, int mask, int64_t window) {
    if (mask == OR_MASK_CAUSAL) return j <= i;
    if (mask == OR_MASK_LOCAL) return (i - j <= window) && (j - i <= window);
    return 1;
}

/* One query row of the dense definition (P3 "The Standard Attention Problem";
 * safe softmax of Step 1): z_j = scale * <q_i, k_j> over allowed j,
 * m = max z, l = sum exp(z - m), P_j = exp(z_j - m) / l, O_i = sum_j P_j v_j,
 * LSE_i = m + ln l. `z` is caller scratch of length N. */
static void dense_row(const double* q, const double* k, const double* v,
                      int64_t N, int64_t d, double scale, int mask, int64_t window,
                      int64_t i, double* z, double* o_row, double* lse_out) {
    const double* qi = q + i * d;
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j) {
        if (!oracle_allowed(i, j, mask, window)) { z[j] = -INFINITY; continue; }
        double s = 0.0;
        for (int64_t c = 0; c < d; ++c) s += qi[c] * k[j * d + c];
        z[j] = scale * s;
        if (z[j] > m) m = z[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < N; ++j)
        if (z[j] != -INFINITY) l += exp(z[j] - m);
    for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        if (z[j] == -INFINITY) continue;
        double p = exp(z[j] - m) / l;
        for (int64_t c = 0; c < d; ++c) o_row[c] += p * v[j * d + c];
    }
    if (lse_out) *lse_out = m + log(l);
}

/* Dense forward over all rows of all heads. */
void oracle_attn_fwd_dense(const double* q, const double* k, const double* v,
                           double* o, double* lse, int64_t BH, int64_t N, int64_t d,
                           double scale, int mask, int64_t window) {
#pragma omp parallel
    {
        double* z = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < BH * N; ++r) {
            int64_t bh = r / N, i = r % N;
            const size_t off = (size_t)bh * N * d;
            dense_row(q + off, k + off, v + off, N, d, scale, mask, window, i, z,
                      o + off + i * d, lse ? lse + bh * N + i : NULL);
        }
        free(z);
    }
}

/* Dense forward for a chosen list of rows (head index bh[r], query index
 * row[r]); used to check sampled outputs at sizes where all rows are too slow.
 * o_rows is [nrows][d], lse_rows is [nrows]. */
void oracle_attn_fwd_dense_rows(const double* q, const double* k, const double* v,
                                int64_t BH, int64_t N, int64_t d, double scale, int mask,
                                int64_t window, const int64_t* bh, const int64_t* row,
                                int64_t nrows, double* o_rows, double* lse_rows) {
    (void)BH;
#pragma omp parallel
    {
        double* z = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            const size_t off = (size_t)bh[r] * N * d;
            dense_row(q + off, k + off, v + off, N, d, scale, mask, window, row[r], z,
                      o_rows + r * d, lse_rows ? lse_rows + r : NULL);
        }
        free(z);
    }
}

/* Tiled online-softmax forward (P3 "Derivation: Incremental Softmax", Steps 2–3
 * and the closing remark that the merge extends to any number of blocks; P2
 * walkthrough step "tiles": a query-major loop over query tiles of Br rows and
 * key tiles of Bc columns that keeps a running maximum, a running denominator
 * and an unnormalized weighted numerator per query row).
 *
 * For each key tile, per row:  m' = max(m, rowmax z_tile);
 *   alpha = exp(m - m')  (0 while m is still -inf);  p = exp(z - m');
 *   l = alpha*l + sum p;  acc = alpha*acc + sum p v;  m = m'.
 * A row whose tile holds no allowed key leaves its state untouched.
 * At the end O = acc / l and LSE = m + ln l.
 *
 * Optional traces (NULL to skip), indexed by key tile t in [0, ceil(N/Bc)):
 *   trace_m, trace_l : [BH][Tc][N]     running max / denominator after tile t
 *   trace_o          : [BH][Tc][N][d]  normalized partial output acc/l after t
 *                                      (NaN while l == 0)
 * Returns 0, or -1 on bad tile sizes / allocation failure. */
int oracle_attn_fwd_tiled(const double* q, const double* k, const double* v,
                          double* o, double* lse, int64_t BH, int64_t N, int64_t d,
                          double scale, int mask, int64_t window, int64_t Br, int64_t Bc,
                          double* trace_m, double* trace_l, double* trace_o) {
    if (Br < 1 || Bc < 1) return -1;
    const int64_t Tr = (N + Br - 1) / Br, Tc = (N + Bc - 1) / Bc;
    int fail = 0;
#pragma omp parallel
    {
        double* S = (double*)malloc((size_t)(Br * Bc) * sizeof(double));
        double* m = (double*)malloc((size_t)Br * sizeof(double));
        double* l = (double*)malloc((size_t)Br * sizeof(double));
        double* acc = (double*)malloc((size_t)(Br * (d > 0 ? d : 1)) * sizeof(double));
        if (!S || !m || !l || !acc) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t task = 0; task < BH * Tr; ++task) {
                const int64_t bh = task / Tr, tr = task % Tr;
                const size_t off = (size_t)bh * N * d;
                const double *Q = q + off, *K = k + off, *V = v + off;
                const int64_t r0 = tr * Br, r1 = (r0 + Br < N) ? r0 + Br : N;
                for (int64_t i = r0; i < r1; ++i) {
                    m[i - r0] = -INFINITY;
                    l[i - r0] = 0.0;
                    for (int64_t c = 0; c < d; ++c) acc[(i - r0) * d + c] = 0.0;
                }
                for (int64_t tc = 0; tc < Tc; ++tc) {
                    const int64_t c0 = tc * Bc, c1 = (c0 + Bc < N) ? c0 + Bc : N;
                    /* score tile, masked entries set to -inf */
                    for (int64_t i = r0; i < r1; ++i)
                        for (int64_t j = c0; j < c1; ++j) {
                            double* s = &S[(i - r0) * Bc + (j - c0)];
                            if (!oracle_allowed(i, j, mask, window)) { *s = -INFINITY; continue; }
                            double dot = 0.0;
                            for (int64_t c = 0; c < d; ++c) dot += Q[i * d + c] * K[j * d + c];
                            *s = scale * dot;
                        }
                    for (int64_t i = r0; i < r1; ++i) {
                        const int64_t ri = i - r0;
                        double tmax = -INFINITY;
                        for (int64_t j = c0; j < c1; ++j)
                            if (S[ri * Bc + (j - c0)] > tmax) tmax = S[ri * Bc + (j - c0)];
                        const double m_new = (tmax > m[ri]) ? tmax : m[ri];
                        if (m_new != -INFINITY) {
                            const double alpha = (m[ri] == -INFINITY) ? 0.0 : exp(m[ri] - m_new);
                            double psum = 0.0;
                            for (int64_t c = 0; c < d; ++c) acc[ri * d + c] *= alpha;
                            for (int64_t j = c0; j < c1; ++j) {
                                const double z = S[ri * Bc + (j - c0)];
                                if (z == -INFINITY) continue;
                                const double p = exp(z - m_new);
                                psum += p;
                                for (int64_t c = 0; c < d; ++c) acc[ri * d + c] += p * V[j * d + c];
                            }
                            l[ri] = alpha * l[ri] + psum;
                            m[ri] = m_new;
                        }
                        if (trace_m) trace_m[(bh * Tc + tc) * N + i] = m[ri];
                        if (trace_l) trace_l[(bh * Tc + tc) * N + i] = l[ri];
                        if (trace_o)
                            for (int64_t c = 0; c < d; ++c)
                                trace_o[((bh * Tc + tc) * N + i) * d + c] =
                                    (l[ri] > 0.0) ? acc[ri * d + c] / l[ri] : NAN;
                    }
                }
                for (int64_t i = r0; i < r1; ++i) {
                    const int64_t ri = i - r0;
                    for (int64_t c = 0; c < d; ++c) o[off + i * d + c] = acc[ri * d + c] / l[ri];
                    if (lse) lse[bh * N + i] = m[ri] + log(l[ri]);
                }
            }
        }
        free(S); free(m); free(l); free(acc);
    }
    return fail ? -1 : 0;
}

/* Dense backward of O = softmax(scale * Q K^T, masked) V for the scalar loss
 * sum(dO * O). The pages state only that the backward recomputes S and P on
 * chip from Q, K, V (P3 "Backward Pass: Recomputation"); the gradient itself
 * follows from the definition by the chain rule:
 *   P     = softmax over allowed j of z_ij = scale <q_i, k_j>
 *   O_i   = sum_j P_ij v_j,          D_i = <dO_i, O_i>
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = <dO_i, v_j>,             dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i
 * The oracle uses its own double O for D. Heads are processed one at a time
 * with full N x N matrices P and dS (so N is kept to a few thousand). Optional
 * outputs o, lse, D (NULL to skip). Returns 0, or -1 on allocation failure. */
int oracle_attn_bwd_dense(const double* q, const double* k, const double* v,
                          const double* dout, double* dq, double* dk, double* dv,
                          int64_t BH, int64_t N, int64_t d, double scale, int mask,
                          int64_t window, double* o, double* lse, double* D) {
    /* Every sum below runs over its index in increasing order, one running
     * double per output element; the loops are nested so that the inner loop
     * walks contiguous memory (a column c, or a block of JB key columns, is
     * carried along), which changes no sum's order and so no result. */
    enum { JB = 8 };
    double* P = (double*)malloc((size_t)(N * N) * sizeof(double));
    double* dS = (double*)malloc((size_t)(N * N) * sizeof(double));
    double* Oh = (double*)malloc((size_t)(N * d) * sizeof(double));
    double* Dh = (double*)malloc((size_t)N * sizeof(double));
    if (!P || !dS || !Oh || !Dh) { free(P); free(dS); free(Oh); free(Dh); return -1; }
    int fail = 0;
    for (int64_t bh = 0; bh < BH && !fail; ++bh) {
        const size_t off = (size_t)bh * N * d;
        const double *Q = q + off, *K = k + off, *V = v + off, *dO = dout + off;
        /* probabilities, output and D, row by row */
#pragma omp parallel for schedule(dynamic, 8)
        for (int64_t i = 0; i < N; ++i) {
            double* Pi = P + i * N;
            double m = -INFINITY;
            for (int64_t j = 0; j < N; ++j) {
                if (!oracle_allowed(i, j, mask, window)) { Pi[j] = -INFINITY; continue; }
                double s = 0.0;
                for (int64_t c = 0; c < d; ++c) s += Q[i * d + c] * K[j * d + c];
                Pi[j] = scale * s;
                if (Pi[j] > m) m = Pi[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < N; ++j)
                if (Pi[j] != -INFINITY) l += exp(Pi[j] - m);
            for (int64_t j = 0; j < N; ++j) Pi[j] = (Pi[j] == -INFINITY) ? 0.0 : exp(Pi[j] - m) / l;
            /* O_i = sum_j P_ij v_j, column c carried along j */
            double* Oi = Oh + i * d;
            for (int64_t c = 0; c < d; ++c) Oi[c] = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                const double p = Pi[j];
                for (int64_t c = 0; c < d; ++c) Oi[c] += p * V[j * d + c];
            }
            double Di = 0.0;
            for (int64_t c = 0; c < d; ++c) Di += dO[i * d + c] * Oi[c];
            Dh[i] = Di;
            if (lse) lse[bh * N + i] = m + log(l);
            /* dS row */
            for (int64_t j = 0; j < N; ++j) {
                double dp = 0.0;
                for (int64_t c = 0; c < d; ++c) dp += dO[i * d + c] * V[j * d + c];
                dS[i * N + j] = Pi[j] * (dp - Di);
            }
        }
#pragma omp parallel
        {
            double* acc = (double*)malloc((size_t)(d > 0 ? d : 1) * sizeof(double));
            double* skb = (double*)malloc((size_t)(JB * (d > 0 ? d : 1)) * sizeof(double));
            double* svb = (double*)malloc((size_t)(JB * (d > 0 ? d : 1)) * sizeof(double));
            if (!acc || !skb || !svb) {
#pragma omp atomic write
                fail = 1;
            }
            /* dQ_i = scale sum_j dS_ij k_j, column c carried along j */
#pragma omp for schedule(static)
            for (int64_t i = 0; i < N; ++i) {
                if (!acc) continue;
                for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
                for (int64_t j = 0; j < N; ++j) {
                    const double ds_ij = dS[i * N + j];
                    for (int64_t c = 0; c < d; ++c) acc[c] += ds_ij * K[j * d + c];
                }
                for (int64_t c = 0; c < d; ++c) dq[off + i * d + c] = scale * acc[c];
            }
            /* dK_j = scale sum_i dS_ij q_i ; dV_j = sum_i P_ij dO_i, for a block
             * of JB keys at a time, each (key, column) carried along i */
#pragma omp for schedule(static)
            for (int64_t j0 = 0; j0 < N; j0 += JB) {
                if (!skb || !svb) continue;
                const int64_t nb = (N - j0 < JB) ? N - j0 : JB;
                for (int64_t t = 0; t < nb * d; ++t) { skb[t] = 0.0; svb[t] = 0.0; }
                for (int64_t i = 0; i < N; ++i) {
                    for (int64_t jj = 0; jj < nb; ++jj) {
                        const int64_t j = j0 + jj;
                        const double ds_ij = dS[i * N + j];
                        const double p_ij = P[i * N + j];
                        double* skj = skb + jj * d;
                        double* svj = svb + jj * d;
                        for (int64_t c = 0; c < d; ++c) {
                            skj[c] += ds_ij * Q[i * d + c];
                            svj[c] += p_ij * dO[i * d + c];
                        }
                    }
                }
                for (int64_t jj = 0; jj < nb; ++jj) {
                    const int64_t j = j0 + jj;
                    const double* skj = skb + jj * d;
                    const double* svj = svb + jj * d;
                    for (int64_t c = 0; c < d; ++c) {
                        dk[off + j * d + c] = scale * skj[c];
                        dv[off + j * d + c] = svj[c];
                    }
                }
            }
            free(acc); free(skb); free(svb);
        }
        if (o) memcpy(o + off, Oh, (size_t)(N * d) * sizeof(double));
        if (D) memcpy(D + bh * N, Dh, (size_t)N * sizeof(double));
    }
    free(P); free(dS); free(Oh); free(Dh);
    return fail ? -1 : 0;
}

/* Backward for chosen rows, by the same chain-rule definition as
 * oracle_attn_bwd_dense but without N x N matrices, so that sampled
 * gradients can be checked at full workload sizes:
 *   dQ of query row (qbh[r], qrow[r]):
 *     dQ_i = scale sum_j P_ij (<dO_i, v_j> - D_i) k_j  over allowed j;
 *   dK, dV of key row (kbh[r], krow[r]):
 *     dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i P_ij (<dO_i, v_j> - D_i) q_i
 *     over the queries i that may see key j;
 * with P_ij = exp(z_ij - LSE_i) and D_i = <dO_i, O_i> from the dense row of
 * query i (dense_row: its own double O and LSE). A key row visits every query
 * that can see it, each through a dense row: O(N^2 d) per key row without a
 * band, O(N + window d) per visited query with one. dq_rows is [nq][d],
 * dk_rows and dv_rows are [nk][d]. Returns 0, or -1 on allocation failure. */
int oracle_attn_bwd_rows(const double* q, const double* k, const double* v,
                         const double* dout, int64_t BH, int64_t N, int64_t d, double scale,
                         int mask, int64_t window, const int64_t* qbh, const int64_t* qrow,
                         int64_t nq, const int64_t* kbh, const int64_t* krow, int64_t nk,
                         double* dq_rows, double* dk_rows, double* dv_rows) {
    (void)BH;
    int fail = 0;
#pragma omp parallel
    {
        double* z = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        double* oi = (double*)malloc((size_t)(d > 0 ? d : 1) * sizeof(double));
        if (!z || !oi) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nq; ++r) {
            if (!z || !oi) continue;
            const size_t off = (size_t)qbh[r] * N * d;
            const double *Q = q + off, *K = k + off, *V = v + off, *dO = dout + off;
            const int64_t i = qrow[r];
            double lse;
            dense_row(Q, K, V, N, d, scale, mask, window, i, z, oi, &lse);
            double Di = 0.0;
            for (int64_t c = 0; c < d; ++c) Di += dO[i * d + c] * oi[c];
            double* out = dq_rows + r * d;
            for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                if (z[j] == -INFINITY) continue;
                double dp = 0.0;
                for (int64_t c = 0; c < d; ++c) dp += dO[i * d + c] * V[j * d + c];
                const double ds = exp(z[j] - lse) * (dp - Di);
                for (int64_t c = 0; c < d; ++c) out[c] += ds * K[j * d + c];
            }
            for (int64_t c = 0; c < d; ++c) out[c] *= scale;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nk; ++r) {
            if (!z || !oi) continue;
            const size_t off = (size_t)kbh[r] * N * d;
            const double *Q = q + off, *K = k + off, *V = v + off, *dO = dout + off;
            const int64_t j = krow[r];
            double* ok = dk_rows + r * d;
            double* ov = dv_rows + r * d;
            for (int64_t c = 0; c < d; ++c) { ok[c] = 0.0; ov[c] = 0.0; }
            for (int64_t i = 0; i < N; ++i) {
                if (!oracle_allowed(i, j, mask, window)) continue;
                double lse;
                dense_row(Q, K, V, N, d, scale, mask, window, i, z, oi, &lse);
                double Di = 0.0, dp = 0.0;
                for (int64_t c = 0; c < d; ++c) {
                    Di += dO[i * d + c] * oi[c];
                    dp += dO[i * d + c] * V[j * d + c];
                }
                const double p = exp(z[j] - lse);
                const double ds = p * (dp - Di);
                for (int64_t c = 0; c < d; ++c) {
                    ov[c] += p * dO[i * d + c];
                    ok[c] += ds * Q[i * d + c];
                }
            }
            for (int64_t c = 0; c < d; ++c) ok[c] *= scale;
        }
        free(z);
        free(oi);
    }
    return fail ? -1 : 0;
}

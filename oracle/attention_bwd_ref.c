/*
 * Oracle for the attention backward pass: explicit gradients in fp64.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests may load this library. It shares no
 * code with the HIP path.
 *
 * The forward is O = P V with P = softmax(S) row by row and S = scale * Q K^T
 * over the visible keys (the definition of the forward oracle,
 * attention_ref.c). For an upstream gradient dO of the same shape as O, the
 * gradients are written out from that definition, in the order the pages give
 * for the FlashAttention-2 backward ("FlashAttention 2 from PyTorch to
 * Triton", What is wrong with this kernel, item 5: the backward recomputes the
 * probabilities from the stored log-sum-exp as P = exp(S - L), and needs the
 * row vector D = rowsum(dO * O); What I am building, on recovering P from L):
 *   1. S_ij = scale * q_i . k_j for visible j (j < Nk, and j <= i + coff if
 *      causal), summed over d in ascending order
 *   2. L_i = m_i + log(sum_j exp(S_ij - m_i)),  P_ij = exp(S_ij - L_i)
 *   3. O_i = sum_j P_ij v_j,  D_i = sum_d dO_i[d] O_i[d]
 *   4. dP_ij = dO_i . v_j
 *   5. dS_ij = P_ij (dP_ij - D_i)
 *   6. dV_j = sum_i P_ij dO_i,  dQ_i = scale * sum_j dS_ij k_j,
 *      dK_j = scale * sum_i dS_ij q_i
 * A query row with no visible key contributes nothing (its P row is 0) and
 * gets dQ_i = 0. Keys no query sees get dK_j = dV_j = 0.
 *
 * Inputs are float32 arrays holding exact input values, widened to double.
 * Layout: q, dout are [BH][Nq][D]; k, v are [BH][Nk][D]; outputs dq [BH][Nq][D],
 * dk and dv [BH][Nk][D], all double. Heads are independent and run in
 * parallel (OpenMP); within a head every sum is sequential, so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

int oracle_attention_bwd(const float *q, const float *k, const float *v, const float *dout,
                         int64_t BH, int64_t Nq, int64_t Nk, int64_t D, double scale,
                         int causal, int64_t coff, double *dq, double *dk, double *dv)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
    if (BH < 1 || Nq < 1 || Nk < 1 || D < 1) return -1;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const float *qh = q + bh * Nq * D, *kh = k + bh * Nk * D, *vh = v + bh * Nk * D;
        const float *doh = dout + bh * Nq * D;
        double *dqh = dq + bh * Nq * D, *dkh = dk + bh * Nk * D, *dvh = dv + bh * Nk * D;
        double *P = (double *)malloc(sizeof(double) * (size_t)(Nq * Nk));
        double *dS = (double *)malloc(sizeof(double) * (size_t)(Nq * Nk));
        double *o = (double *)malloc(sizeof(double) * (size_t)D);
        if (!P || !dS || !o) {
#pragma omp atomic write
            failed = 1;
            free(P);
            free(dS);
            free(o);
            continue;
        }
        for (int64_t i = 0; i < Nq; ++i) {
            int64_t n_vis = Nk;
            if (causal && i + coff + 1 < n_vis) n_vis = i + coff + 1;
            double *Pi = P + i * Nk, *dSi = dS + i * Nk;
            for (int64_t j = 0; j < Nk; ++j) Pi[j] = 0.0, dSi[j] = 0.0;
            if (n_vis <= 0) continue;
            /* steps 1-2: scores, log-sum-exp, probabilities */
            const float *qi = qh + i * D;
            for (int64_t j = 0; j < n_vis; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kh[j * D + d];
                Pi[j] = scale * dot;
            }
            double m = Pi[0];
            for (int64_t j = 1; j < n_vis; ++j)
                if (Pi[j] > m) m = Pi[j];
            double l = 0.0;
            for (int64_t j = 0; j < n_vis; ++j) l += exp(Pi[j] - m);
            const double L = m + log(l);
            for (int64_t j = 0; j < n_vis; ++j) Pi[j] = exp(Pi[j] - L);
            /* step 3: the forward output and D_i = rowsum(dO * O) */
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t j = 0; j < n_vis; ++j)
                for (int64_t d = 0; d < D; ++d) o[d] += Pi[j] * (double)vh[j * D + d];
            const float *doi = doh + i * D;
            double Di = 0.0;
            for (int64_t d = 0; d < D; ++d) Di += (double)doi[d] * o[d];
            /* steps 4-5: dP and dS */
            for (int64_t j = 0; j < n_vis; ++j) {
                double dp = 0.0;
                for (int64_t d = 0; d < D; ++d) dp += (double)doi[d] * (double)vh[j * D + d];
                dSi[j] = Pi[j] * (dp - Di);
            }
        }
        /* step 6: the three products */
        for (int64_t i = 0; i < Nq; ++i)
            for (int64_t d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int64_t j = 0; j < Nk; ++j) acc += dS[i * Nk + j] * (double)kh[j * D + d];
                dqh[i * D + d] = scale * acc;
            }
        for (int64_t j = 0; j < Nk; ++j)
            for (int64_t d = 0; d < D; ++d) {
                double acc_k = 0.0, acc_v = 0.0;
                for (int64_t i = 0; i < Nq; ++i) {
                    acc_k += dS[i * Nk + j] * (double)qh[i * D + d];
                    acc_v += P[i * Nk + j] * (double)doh[i * D + d];
                }
                dkh[j * D + d] = scale * acc_k;
                dvh[j * D + d] = acc_v;
            }
        free(P);
        free(dS);
        free(o);
    }
    return failed ? -2 : 0;
}

/*
 * The same gradients for one head, on selected outputs only: dQ for the query
 * rows rows[0..n_rows) and dK, dV for the key rows cols[0..n_cols). This is
 * the definition above evaluated element by element, so that single outputs
 * of a long sequence can be checked without the Nq x Nk matrices:
 *   - L_i and D_i are computed for every query row first (steps 1-3);
 *   - dQ_r = scale * sum_j P_rj (dP_rj - D_r) k_j, over visible j ascending;
 *   - dV_c = sum_i P_ic dO_i and dK_c = scale * sum_i P_ic (dP_ic - D_i) q_i,
 *     over the query rows i that see key c, ascending.
 * Layout: q, dout [Nq][D]; k, v [Nk][D]; dq_rows [n_rows][D];
 * dk_cols, dv_cols [n_cols][D] (double). Rows and columns run in parallel;
 * every sum is sequential.
 */
int oracle_attention_bwd_sampled(const float *q, const float *k, const float *v,
                                 const float *dout, int64_t Nq, int64_t Nk, int64_t D,
                                 double scale, int causal, int64_t coff,
                                 const int64_t *rows, int64_t n_rows,
                                 const int64_t *cols, int64_t n_cols,
                                 double *dq_rows, double *dk_cols, double *dv_cols)
{
    if (!q || !k || !v || !dout) return -1;
    if (Nq < 1 || Nk < 1 || D < 1 || n_rows < 0 || n_cols < 0) return -1;
    if ((n_rows && (!rows || !dq_rows)) || (n_cols && (!cols || !dk_cols || !dv_cols)))
        return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= Nq) return -1;
    for (int64_t c = 0; c < n_cols; ++c)
        if (cols[c] < 0 || cols[c] >= Nk) return -1;

    double *L = (double *)malloc(sizeof(double) * (size_t)Nq);
    double *Dv = (double *)malloc(sizeof(double) * (size_t)Nq);
    if (!L || !Dv) {
        free(L);
        free(Dv);
        return -2;
    }
    int failed = 0;

    /* steps 1-3 for every row: L_i, and D_i from O_i */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < Nq; ++i) {
        int64_t n_vis = Nk;
        if (causal && i + coff + 1 < n_vis) n_vis = i + coff + 1;
        L[i] = -INFINITY;
        Dv[i] = 0.0;
        if (n_vis <= 0) continue;
        double *s = (double *)malloc(sizeof(double) * (size_t)n_vis);
        double *o = (double *)malloc(sizeof(double) * (size_t)D);
        if (!s || !o) {
#pragma omp atomic write
            failed = 1;
            free(s);
            free(o);
            continue;
        }
        const float *qi = q + i * D;
        for (int64_t j = 0; j < n_vis; ++j) {
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)k[j * D + d];
            s[j] = scale * dot;
        }
        double m = s[0];
        for (int64_t j = 1; j < n_vis; ++j)
            if (s[j] > m) m = s[j];
        double l = 0.0;
        for (int64_t j = 0; j < n_vis; ++j) l += exp(s[j] - m);
        const double Li = m + log(l);
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        for (int64_t j = 0; j < n_vis; ++j) {
            const double p = exp(s[j] - Li);
            for (int64_t d = 0; d < D; ++d) o[d] += p * (double)v[j * D + d];
        }
        const float *doi = dout + i * D;
        double Di = 0.0;
        for (int64_t d = 0; d < D; ++d) Di += (double)doi[d] * o[d];
        L[i] = Li;
        Dv[i] = Di;
        free(s);
        free(o);
    }
    if (failed) {
        free(L);
        free(Dv);
        return -2;
    }

    /* dQ of the selected rows */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t i = rows[r];
        int64_t n_vis = Nk;
        if (causal && i + coff + 1 < n_vis) n_vis = i + coff + 1;
        double *out = dq_rows + r * D;
        for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
        const float *qi = q + i * D, *doi = dout + i * D;
        for (int64_t j = 0; j < n_vis; ++j) {
            double dot = 0.0, dp = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)k[j * D + d];
            for (int64_t d = 0; d < D; ++d) dp += (double)doi[d] * (double)v[j * D + d];
            const double ds = exp(scale * dot - L[i]) * (dp - Dv[i]);
            for (int64_t d = 0; d < D; ++d) out[d] += ds * (double)k[j * D + d];
        }
        for (int64_t d = 0; d < D; ++d) out[d] *= scale;
    }

    /* dK and dV of the selected keys */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < n_cols; ++c) {
        const int64_t j = cols[c];
        double *ok = dk_cols + c * D, *ov = dv_cols + c * D;
        for (int64_t d = 0; d < D; ++d) ok[d] = 0.0, ov[d] = 0.0;
        const float *kj = k + j * D, *vj = v + j * D;
        for (int64_t i = 0; i < Nq; ++i) {
            if (causal && j > i + coff) continue;   /* key j is in row i's future */
            const float *qi = q + i * D, *doi = dout + i * D;
            double dot = 0.0, dp = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[d];
            for (int64_t d = 0; d < D; ++d) dp += (double)doi[d] * (double)vj[d];
            const double p = exp(scale * dot - L[i]);
            const double ds = p * (dp - Dv[i]);
            for (int64_t d = 0; d < D; ++d) {
                ov[d] += p * (double)doi[d];
                ok[d] += ds * (double)qi[d];
            }
        }
        for (int64_t d = 0; d < D; ++d) ok[d] *= scale;
    }
    free(L);
    free(Dv);
    return 0;
}

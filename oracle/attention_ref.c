/*
 * Oracle for the attention forward pass: explicit softmax attention in fp64.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code with the HIP path.
 *
 * What it computes (the plain definition, no tiling, no online softmax):
 *   S = scale * Q K^T, P = softmax(S) over each row, O = P V
 * ("A09 - Advanced Triton & FlashAttention", section 2 First Principles;
 *  "Building a Verifiable FlashAttention Forward from PyTorch to Triton",
 *  Part 1), and the row log-sum-exp LSE_i = m_i + log(l_i) = log sum_j exp(S_ij)
 * ("FlashAttention 2 from PyTorch to Triton", What I am building).
 *
 * For every requested row i of head bh, with keys j in the visible set
 *   J = { j : j < n_kv and (not causal or j <= i + coff) }
 * Causal attention shifts the diagonal by coff: coff = 0 is the top-left
 * alignment (key j visible to query i when j <= i; "Building a Verifiable
 * FlashAttention Forward", Part 1, and the convention the pages attribute to
 * SDPA's is_causal in "How to profile and optimise kernels", Round 4
 * causal tile-skipping); coff = Nk - Nq is the bottom-right alignment that
 * the same passage attributes to the FlashAttention library since 2.1. The
 * query length Nq and the key/value length Nk are separate quantities
 * ("Triton: FlashAttention-2 Forward Pass", Masks and sentinels, on
 * cross-attention): Q and O rows use Nq, K and V rows use Nk.
 *   1. s_j = scale * sum_d q[i][d] * k[j][d], summed over d in ascending order
 *   2. m = max_j s_j, p_j = exp(s_j - m), l = sum_j p_j   (stable softmax,
 *      "Building a Verifiable FlashAttention Forward", Part 2)
 *   3. o[d] = (sum_j p_j v[j][d]) / l,  lse = m + log(l)  (natural log)
 *   4. if J is empty: o = 0 and lse = -inf (a row with no visible key has no
 *      softmax; the pages warn that a finite sentinel would instead average
 *      values it should never see: "FlashAttention 2 from PyTorch to Triton",
 *      What is wrong with this kernel, item 4).
 *
 * Inputs are float32 arrays holding the exact values of the (already rounded)
 * bf16/fp16/fp32 inputs; each element is widened to double exactly before use.
 * Layout: q is contiguous [BH][Nq][D], k and v are [BH][Nk][D]; rows is
 * n_rows pairs (bh, i) with i < Nq.
 * Outputs: o is [n_rows][D] double, lse is [n_rows] double.
 * Rows are independent; OpenMP splits them across threads, each row is
 * computed sequentially, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

int oracle_attention_rows(const float *q, const float *k, const float *v,
                          int64_t BH, int64_t Nq, int64_t Nk, int64_t n_kv, int64_t D,
                          double scale, int causal, int64_t coff, const int64_t *rows,
                          int64_t n_rows, double *o, double *lse)
{
    if (!q || !k || !v || !rows || !o || !lse) return -1;
    if (BH < 1 || Nq < 1 || Nk < 1 || D < 1 || n_kv < 0 || n_kv > Nk || n_rows < 0) return -1;
    for (int64_t r = 0; r < n_rows; ++r) {
        if (rows[2 * r] < 0 || rows[2 * r] >= BH) return -1;
        if (rows[2 * r + 1] < 0 || rows[2 * r + 1] >= Nq) return -1;
    }
    int failed = 0;

#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Nk);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        if (!s || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s || !acc) continue;
            const int64_t bh = rows[2 * r], i = rows[2 * r + 1];
            const float *qi = q + (bh * Nq + i) * D;
            const float *kh = k + bh * Nk * D;
            const float *vh = v + bh * Nk * D;
            double *oi = o + r * D;

            int64_t n_vis = n_kv;                 /* keys 0 .. n_vis-1 are visible */
            if (causal && i + coff + 1 < n_vis) n_vis = i + coff + 1;

            if (n_vis <= 0) {
                for (int64_t d = 0; d < D; ++d) oi[d] = 0.0;
                lse[r] = -INFINITY;
                continue;
            }
            /* step 1: scores */
            for (int64_t j = 0; j < n_vis; ++j) {
                const float *kj = kh + j * D;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[d];
                s[j] = scale * dot;
            }
            /* step 2: stable softmax numerators and denominator */
            double m = s[0];
            for (int64_t j = 1; j < n_vis; ++j)
                if (s[j] > m) m = s[j];
            double l = 0.0;
            for (int64_t j = 0; j < n_vis; ++j) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }
            /* step 3: weighted sum of value rows, one division at the end */
            for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t j = 0; j < n_vis; ++j) {
                const float *vj = vh + j * D;
                for (int64_t d = 0; d < D; ++d) acc[d] += s[j] * (double)vj[d];
            }
            for (int64_t d = 0; d < D; ++d) oi[d] = acc[d] / l;
            lse[r] = m + log(l);
        }
        free(s);
        free(acc);
    }
    return failed ? -2 : 0;
}

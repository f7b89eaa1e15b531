/*
 * fp64 CPU oracle for MLA decode attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may load this code.  It shares nothing with the HIP library: no headers,
 * no helpers, no constants.  It is deliberately plain: one (sequence, query
 * token, head) row at a time, every dot product summed in double, no
 * blocking, no online softmax, no split.
 *
 * What it computes ("FlashMLA-ETAP", gist.science technical summary,
 * Methodology, the ETAP bullet):
 *   standard order   S = Q K^T,  P = softmax(S),  O = P V
 *   transposed order S^T = K Q^T, P^T = softmax(S^T), O^T = V^T P^T, O = (O^T)^T
 * over the shared latent KV cache of MLA (same summary, Integration and
 * Implementation: the low-rank joint compression keeps one latent row per
 * token for all heads).  The head dimension is 576 (arxivlens page,
 * Limitations); keys use all 576 channels, values the first d_v of them.
 *
 * Readings of what the pages leave open:
 *   - softmax runs over keys (for the transposed order: down each column of
 *     S^T), the only axis under which both orders agree;
 *   - S is multiplied by `scale` (the fp32 value given, widened to double)
 *     before the softmax;
 *   - LSE is the natural log of sum_j exp(scale * q.k_j);
 *   - with s_q query tokens the new tokens are the last s_q positions and
 *     token t sees keys 0 .. L - s_q + t (causal);
 *   - an empty key window yields O = 0 and LSE = -inf (a split part that
 *     holds no visible key carries no weight).
 *
 * Inputs are bf16 bit patterns (uint16); they are widened exactly to double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Address of logical key j of sequence b: contiguous [B][cap][d_qk] when
 * block_table is NULL, else pool [pages][page_size][d_qk] through the
 * block table [B][max_pages]. */
static const uint16_t *key_row(const uint16_t *kv, const int32_t *block_table,
                               int b, int64_t j, int d_qk, int64_t cap,
                               int page_size, int max_pages)
{
    if (block_table == NULL)
        return kv + ((int64_t)b * cap + j) * d_qk;
    int64_t page = block_table[(int64_t)b * max_pages + j / page_size];
    return kv + (page * page_size + j % page_size) * d_qk;
}

static int check_args(const int32_t *seqlens, int B, int s_q, int H, int d_qk,
                      int d_v, int64_t cap, const int32_t *block_table,
                      int page_size, int max_pages)
{
    if (B < 0 || s_q < 1 || H < 1 || d_v < 1 || d_v > d_qk)
        return -1;
    for (int b = 0; b < B; b++) {
        if (seqlens[b] < s_q)
            return -1;
        if (block_table == NULL && seqlens[b] > cap)
            return -1;
        if (block_table != NULL &&
            (page_size < 1 || (int64_t)seqlens[b] > (int64_t)max_pages * page_size))
            return -1;
    }
    return 0;
}

/*
 * Standard order, one row at a time.
 *   q      [B][s_q][H][d_qk]   bf16 bits
 *   kv     see key_row()
 *   win_begin/win_end  optional [B] key windows [begin, end): only keys in
 *          the window (and visible to the token) take part -- a split part.
 *   out    [B][s_q][H][d_v]    double
 *   lse    [B][s_q][H]         double
 *   probs  optional [B][s_q][H][probs_stride]: softmax weights per key
 *          (0 for keys the row does not see)
 * Returns 0, or -1 on inconsistent arguments.
 */
int oracle_mla_decode(const uint16_t *q, const uint16_t *kv,
                      const int32_t *block_table, const int32_t *seqlens,
                      const int32_t *win_begin, const int32_t *win_end,
                      int B, int s_q, int H, int d_qk, int d_v, int64_t cap,
                      int page_size, int max_pages, float scale, double *out,
                      double *lse, double *probs, int64_t probs_stride)
{
    if (check_args(seqlens, B, s_q, H, d_qk, d_v, cap, block_table, page_size,
                   max_pages))
        return -1;
    const double sc = (double)scale;
    const int64_t rows = (int64_t)B * s_q * H;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < rows; r++) {
        const int b = (int)(r / ((int64_t)s_q * H));
        const int t = (int)((r / H) % s_q);
        const int64_t L = seqlens[b];
        int64_t lo = 0, hi = L - s_q + t + 1; /* visible keys [0, hi) */
        if (win_begin != NULL && win_begin[b] > lo)
            lo = win_begin[b];
        if (win_end != NULL && win_end[b] < hi)
            hi = win_end[b];
        const uint16_t *qr = q + r * d_qk;
        double *o = out + r * d_v;
        for (int c = 0; c < d_v; c++)
            o[c] = 0.0;
        if (probs != NULL)
            for (int64_t j = 0; j < probs_stride; j++)
                probs[r * probs_stride + j] = 0.0;
        if (hi <= lo) {
            lse[r] = -INFINITY;
            continue;
        }
        const int64_t n = hi - lo;
        double *s = (double *)malloc((size_t)n * sizeof(double));
        if (s == NULL) {
            bad |= 1;
            continue;
        }
        /* S = scale * Q K^T */
        for (int64_t j = 0; j < n; j++) {
            const uint16_t *kr = key_row(kv, block_table, b, lo + j, d_qk, cap,
                                         page_size, max_pages);
            double acc = 0.0;
            for (int c = 0; c < d_qk; c++)
                acc += bf16_to_double(qr[c]) * bf16_to_double(kr[c]);
            s[j] = sc * acc;
        }
        /* P = softmax(S) over keys, with the max subtracted for range */
        double m = s[0];
        for (int64_t j = 1; j < n; j++)
            if (s[j] > m)
                m = s[j];
        double l = 0.0;
        for (int64_t j = 0; j < n; j++) {
            s[j] = exp(s[j] - m);
            l += s[j];
        }
        /* O = P V, V = first d_v channels of the same latent rows */
        for (int64_t j = 0; j < n; j++) {
            const double p = s[j] / l;
            const uint16_t *vr = key_row(kv, block_table, b, lo + j, d_qk, cap,
                                         page_size, max_pages);
            for (int c = 0; c < d_v; c++)
                o[c] += p * bf16_to_double(vr[c]);
            if (probs != NULL && lo + j < probs_stride)
                probs[r * probs_stride + lo + j] = p;
        }
        lse[r] = m + log(l);
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * Transposed order of the same attention, per sequence b with
 * N = L_b keys and N_q = s_q * H query rows:
 *   S^T = K Q^T          in R^{N x N_q}
 *   P^T = softmax(S^T)   column by column (over keys), causal per token
 *   O^T = V^T P^T        in R^{d_v x N_q}
 *   O   = (O^T)^T
 * Arguments as oracle_mla_decode (no windows, no probs).
 */
int oracle_mla_decode_transposed(const uint16_t *q, const uint16_t *kv,
                                 const int32_t *block_table,
                                 const int32_t *seqlens, int B, int s_q, int H,
                                 int d_qk, int d_v, int64_t cap, int page_size,
                                 int max_pages, float scale, double *out,
                                 double *lse)
{
    if (check_args(seqlens, B, s_q, H, d_qk, d_v, cap, block_table, page_size,
                   max_pages))
        return -1;
    const double sc = (double)scale;
    const int nq = s_q * H;
    int bad = 0;

    for (int b = 0; b < B; b++) {
        const int64_t N = seqlens[b];
        double *st = (double *)malloc((size_t)N * nq * sizeof(double)); /* S^T, then P^T */
        double *ot = (double *)malloc((size_t)d_v * nq * sizeof(double)); /* O^T */
        if (st == NULL || ot == NULL) {
            free(st);
            free(ot);
            return -1;
        }
        const uint16_t *qb = q + (int64_t)b * nq * d_qk;

        /* S^T[j][i] = scale * sum_c K[j][c] * Q^T[c][i] */
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < N; j++) {
            const uint16_t *kr = key_row(kv, block_table, b, j, d_qk, cap,
                                         page_size, max_pages);
            for (int i = 0; i < nq; i++) {
                double acc = 0.0;
                for (int c = 0; c < d_qk; c++)
                    acc += bf16_to_double(kr[c]) * bf16_to_double(qb[(int64_t)i * d_qk + c]);
                st[j * nq + i] = sc * acc;
            }
        }
        /* P^T: softmax down each column i, over the keys token i/H sees */
#pragma omp parallel for schedule(static) reduction(| : bad)
        for (int i = 0; i < nq; i++) {
            const int t = i / H;
            const int64_t vis = N - s_q + t + 1;
            double m = st[i];
            for (int64_t j = 1; j < vis; j++)
                if (st[j * nq + i] > m)
                    m = st[j * nq + i];
            double l = 0.0;
            for (int64_t j = 0; j < vis; j++)
                l += exp(st[j * nq + i] - m);
            for (int64_t j = 0; j < N; j++)
                st[j * nq + i] = (j < vis) ? exp(st[j * nq + i] - m) / l : 0.0;
            lse[(int64_t)b * nq + i] = m + log(l);
            if (!(l > 0.0))
                bad |= 1;
        }
        /* O^T[c][i] = sum_j V^T[c][j] * P^T[j][i] */
#pragma omp parallel for schedule(static)
        for (int c = 0; c < d_v; c++) {
            for (int i = 0; i < nq; i++)
                ot[(int64_t)c * nq + i] = 0.0;
            for (int64_t j = 0; j < N; j++) {
                const double v = bf16_to_double(
                    key_row(kv, block_table, b, j, d_qk, cap, page_size, max_pages)[c]);
                for (int i = 0; i < nq; i++)
                    ot[(int64_t)c * nq + i] += v * st[j * nq + i];
            }
        }
        /* O = (O^T)^T */
        for (int i = 0; i < nq; i++)
            for (int c = 0; c < d_v; c++)
                out[((int64_t)b * nq + i) * d_v + c] = ot[(int64_t)c * nq + i];
        free(st);
        free(ot);
    }
    return bad ? -1 : 0;
}

/*
 * Merge attention computed over disjoint key sets of the same rows.  Part s
 * holds O_s (already divided by its own softmax sum l_s) and
 * lse_s = m_s + ln l_s.  The exact merge of the softmax over the union is
 *   lse = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s,
 * evaluated with the largest lse_s subtracted; parts with lse_s = -inf
 * (no key) get weight 0.
 *   lse_parts [n_parts][rows], o_parts [n_parts][rows][d_v]
 */
int oracle_lse_combine(int n_parts, int64_t rows, int d_v,
                       const double *lse_parts, const double *o_parts,
                       double *lse, double *out)
{
    if (n_parts < 1 || rows < 0 || d_v < 1)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        double m = -INFINITY;
        for (int s = 0; s < n_parts; s++)
            if (lse_parts[(int64_t)s * rows + r] > m)
                m = lse_parts[(int64_t)s * rows + r];
        double *o = out + r * d_v;
        for (int c = 0; c < d_v; c++)
            o[c] = 0.0;
        if (m == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double wsum = 0.0;
        for (int s = 0; s < n_parts; s++)
            wsum += exp(lse_parts[(int64_t)s * rows + r] - m);
        const double tot = m + log(wsum);
        for (int s = 0; s < n_parts; s++) {
            const double w = exp(lse_parts[(int64_t)s * rows + r] - tot);
            if (w == 0.0)
                continue;
            const double *os = o_parts + ((int64_t)s * rows + r) * d_v;
            for (int c = 0; c < d_v; c++)
                o[c] += w * os[c];
        }
        lse[r] = tot;
    }
    return 0;
}

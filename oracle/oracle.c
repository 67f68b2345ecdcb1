/*
 * CPU oracle for the DiT long-sequence attention path.  TEST INFRASTRUCTURE ONLY:
 * it is loaded by tests/, by the smoke check and by the bench's cpu_baseline leg,
 * never by the library's product path.  It shares no code, header or constant
 * with the HIP library.
 *
 * Plain, slow, obviously correct: float64 throughout, straight loops in the order
 * of the definitions, OpenMP only over independent output rows.
 *
 * Definitions followed:
 *  - attention per head: o = softmax(q k^T * scale) v with scale = 1/sqrt(d)
 *    (MindIE SD "多卡并行" page, Ring Sequence Parallel section, usage example:
 *    local_attn divides the scores by dim ** 0.5 and applies softmax over keys);
 *    heads are independent ("AIGC 分布式推理：从 Wan2.2 理解 DP/TP/CP/SP/PP",
 *    CP section: head i's softmax uses only head i's Q/K/V) and every query sees
 *    every key (same section; non-causal).
 *  - log-sum-exp of a row: lse = ln sum_j exp(s_j) of the scaled logits s_j.
 *  - LSE merge: the across-rounds online-softmax accumulation of Ring attention
 *    (arganzheng.life, multi-GPU diffusion parallelism, section 4.2 "Ring"): for
 *    parts t over disjoint key sets, L = ln sum_t exp(lse_t) and
 *    o = sum_t exp(lse_t - L) o_t.
 *  - Ulysses seq->head permute: the local data movement of the all-to-all that
 *    turns "N/p tokens x all H heads" into "all N tokens x H/p heads"
 *    (arganzheng.life section 4.1 figure; MindIE SD page, Ulysses section usage
 *    example: split heads into p groups, exchange, concatenate along tokens in
 *    rank order).
 *  - Ulysses head->seq permute: the all-to-all after attention that turns the
 *    output back into "N/p tokens x all heads" (arganzheng.life section 4.1 figure,
 *    the O all-to-all; MindIE SD page, Ulysses usage example: split the attention
 *    output into p token ranges, exchange, concatenate along heads in rank order).
 *  - fused QKV seq->head permute: Q, K and V moved by one all-to-all ("AIGC
 *    分布式推理" CP section: one fused QKV all-to-all plus one for the output per
 *    self-attention).  Reading: each token's row holds its q, k and v of all heads
 *    side by side, as a fused QKV projection writes them, and each head group
 *    receives three separate BSND tensors.
 *
 * Layouts (dense, row-major):  q [B,Nq,H,D], k/v [B,Nkv,H,D], o [B,Nq,H,D],
 * lse [B,H,Nq].  Merge parts: o_parts [P,B,N,H,D], lse_parts [P,B,H,N].
 * Permute: in [p,B,N/p,H,D] -> out [p,B,N,H/p,D].
 * Inverse permute: in [p,B,N,H/p,D] -> out [p,B,N/p,H,D].
 * Fused QKV permute: in [p,B,N/p,3,H,D] -> out [p,3,B,N,H/p,D].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One attention row (b, h, i).  s is caller scratch of Nkv doubles. */
static void attn_row(const double *qrow, const double *kbase, const double *vbase,
                     long row_stride, int Nkv, int D, double scale,
                     double *s, double *orow, double *lse_out)
{
    /* scaled logits s_j = scale * (q . k_j) */
    double m = -INFINITY;
    for (int j = 0; j < Nkv; ++j) {
        const double *kj = kbase + (long)j * row_stride;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += qrow[d] * kj[d];
        s[j] = scale * dot;
        if (s[j] > m)
            m = s[j];
    }
    /* softmax weights exp(s_j - m) / l; subtracting the row max leaves the ratio unchanged */
    double l = 0.0;
    for (int j = 0; j < Nkv; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int d = 0; d < D; ++d)
        orow[d] = 0.0;
    for (int j = 0; j < Nkv; ++j) {
        const double *vj = vbase + (long)j * row_stride;
        for (int d = 0; d < D; ++d)
            orow[d] += s[j] * vj[d];
    }
    for (int d = 0; d < D; ++d)
        orow[d] /= l;
    /* lse = ln sum_j exp(s_j) = m + ln l */
    *lse_out = m + log(l);
}

/* Full attention: o [B,Nq,H,D], lse [B,H,Nq].  Returns 0, or -1 on bad sizes. */
int oracle_attn(const double *q, const double *k, const double *v,
                int B, int Nq, int Nkv, int H, int D, double scale,
                double *o, double *lse)
{
    if (B <= 0 || Nq <= 0 || Nkv <= 0 || H <= 0 || D <= 0)
        return -1;
    long total = (long)B * H * Nq;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Nkv);
#pragma omp for schedule(dynamic, 4)
        for (long r = 0; r < total; ++r) {
            int b = (int)(r / ((long)H * Nq));
            int h = (int)((r / Nq) % H);
            int i = (int)(r % Nq);
            const double *qrow = q + (((long)b * Nq + i) * H + h) * D;
            const double *kb = k + ((long)b * Nkv * H + h) * D;
            const double *vb = v + ((long)b * Nkv * H + h) * D;
            double *orow = o + (((long)b * Nq + i) * H + h) * D;
            attn_row(qrow, kb, vb, (long)H * D, Nkv, D, scale, s,
                     orow, lse + ((long)b * H + h) * Nq + i);
        }
        free(s);
    }
    return 0;
}

/* Attention on a list of rows: rows is [n,3] of (b, h, i); o_rows [n,D], lse_rows [n]. */
int oracle_attn_rows(const double *q, const double *k, const double *v,
                     int B, int Nq, int Nkv, int H, int D, double scale,
                     const int64_t *rows, long n, double *o_rows, double *lse_rows)
{
    if (B <= 0 || Nq <= 0 || Nkv <= 0 || H <= 0 || D <= 0 || n < 0)
        return -1;
    for (long r = 0; r < n; ++r) {
        if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 ||
            rows[3 * r + 1] >= H || rows[3 * r + 2] < 0 || rows[3 * r + 2] >= Nq)
            return -1;
    }
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Nkv);
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < n; ++r) {
            long b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            const double *qrow = q + ((b * Nq + i) * H + h) * D;
            const double *kb = k + (b * Nkv * H + h) * D;
            const double *vb = v + (b * Nkv * H + h) * D;
            attn_row(qrow, kb, vb, (long)H * D, Nkv, D, scale, s,
                     o_rows + r * D, lse_rows + r);
        }
        free(s);
    }
    return 0;
}

/* LSE merge of P parts.  A part whose lse is -inf holds no keys and adds nothing;
 * if every part is -inf the row is empty: o = 0, lse = -inf. */
int oracle_merge(const double *o_parts, const double *lse_parts,
                 int P, int B, int N, int H, int D, double *o, double *lse)
{
    if (P <= 0 || B <= 0 || N <= 0 || H <= 0 || D <= 0)
        return -1;
    long rows = (long)B * N * H;
    long part_o = rows * D;          /* elements of one o part */
    long part_l = (long)B * H * N;   /* elements of one lse part */
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        long b = r / ((long)N * H);
        long n = (r / H) % N;
        long h = r % H;
        long li = (b * H + h) * N + n;
        double M = -INFINITY;
        for (int t = 0; t < P; ++t)
            if (lse_parts[t * part_l + li] > M)
                M = lse_parts[t * part_l + li];
        double *orow = o + r * D;
        if (M == -INFINITY) {
            for (int d = 0; d < D; ++d)
                orow[d] = 0.0;
            lse[li] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int t = 0; t < P; ++t)
            sum += exp(lse_parts[t * part_l + li] - M);
        double L = M + log(sum);
        for (int d = 0; d < D; ++d)
            orow[d] = 0.0;
        for (int t = 0; t < P; ++t) {
            double w = exp(lse_parts[t * part_l + li] - L);
            const double *op = o_parts + t * part_o + r * D;
            for (int d = 0; d < D; ++d)
                orow[d] += w * op[d];
        }
        lse[li] = L;
    }
    return 0;
}

/* Ulysses seq->head permute, element by element:
 *   out[j][b][s*(N/p) + n][hh][d] = in[s][b][n][j*(H/p) + hh][d]
 * for source shard s, destination head group j.  A byte copy of each element. */
int oracle_permute(const void *in, void *out, int p, int B, int N, int H, int D,
                   int elem_bytes)
{
    if (p <= 0 || B <= 0 || N <= 0 || H <= 0 || D <= 0 || elem_bytes <= 0)
        return -1;
    if (N % p != 0 || H % p != 0)
        return -1;
    const unsigned char *src = (const unsigned char *)in;
    unsigned char *dst = (unsigned char *)out;
    long Ns = N / p, Hs = H / p;
    for (long s = 0; s < p; ++s)
        for (long j = 0; j < p; ++j)
            for (long b = 0; b < B; ++b)
                for (long n = 0; n < Ns; ++n)
                    for (long hh = 0; hh < Hs; ++hh)
                        for (long d = 0; d < D; ++d) {
                            long si = (((s * B + b) * Ns + n) * H + (j * Hs + hh)) * D + d;
                            long di = (((j * B + b) * (long)N + (s * Ns + n)) * Hs + hh) * D + d;
                            memcpy(dst + di * elem_bytes, src + si * elem_bytes,
                                   (size_t)elem_bytes);
                        }
    return 0;
}

/* Ulysses head->seq permute (after attention), element by element:
 *   out[s][b][n][j*(H/p) + hh][d] = in[j][b][s*(N/p) + n][hh][d]
 * for head group j (the rank that computed those heads) and token shard s. */
int oracle_head_to_seq(const void *in, void *out, int p, int B, int N, int H, int D,
                       int elem_bytes)
{
    if (p <= 0 || B <= 0 || N <= 0 || H <= 0 || D <= 0 || elem_bytes <= 0)
        return -1;
    if (N % p != 0 || H % p != 0)
        return -1;
    const unsigned char *src = (const unsigned char *)in;
    unsigned char *dst = (unsigned char *)out;
    long Ns = N / p, Hs = H / p;
    for (long s = 0; s < p; ++s)
        for (long j = 0; j < p; ++j)
            for (long b = 0; b < B; ++b)
                for (long n = 0; n < Ns; ++n)
                    for (long hh = 0; hh < Hs; ++hh)
                        for (long d = 0; d < D; ++d) {
                            long si = (((j * B + b) * (long)N + (s * Ns + n)) * Hs + hh) * D + d;
                            long di = (((s * B + b) * Ns + n) * H + (j * Hs + hh)) * D + d;
                            memcpy(dst + di * elem_bytes, src + si * elem_bytes,
                                   (size_t)elem_bytes);
                        }
    return 0;
}

/* Fused QKV seq->head permute, element by element (c = 0, 1, 2 for q, k, v):
 *   out[j][c][b][s*(N/p) + n][hh][d] = in[s][b][n][c][j*(H/p) + hh][d] */
int oracle_qkv_seq_to_head(const void *in, void *out, int p, int B, int N, int H, int D,
                           int elem_bytes)
{
    if (p <= 0 || B <= 0 || N <= 0 || H <= 0 || D <= 0 || elem_bytes <= 0)
        return -1;
    if (N % p != 0 || H % p != 0)
        return -1;
    const unsigned char *src = (const unsigned char *)in;
    unsigned char *dst = (unsigned char *)out;
    long Ns = N / p, Hs = H / p;
    for (long s = 0; s < p; ++s)
        for (long j = 0; j < p; ++j)
            for (long c = 0; c < 3; ++c)
                for (long b = 0; b < B; ++b)
                    for (long n = 0; n < Ns; ++n)
                        for (long hh = 0; hh < Hs; ++hh)
                            for (long d = 0; d < D; ++d) {
                                long si = ((((s * B + b) * Ns + n) * 3 + c) * H + (j * Hs + hh)) * D + d;
                                long di = ((((j * 3 + c) * B + b) * (long)N + (s * Ns + n)) * Hs + hh) * D + d;
                                memcpy(dst + di * elem_bytes, src + si * elem_bytes,
                                       (size_t)elem_bytes);
                            }
    return 0;
}

/* QK-RMSNorm and rotary position embedding on packed q, k, v, written in the fused QKV
 * seq->head layout ("AIGC 分布式推理：从 Wan2.2 理解 DP/TP/CP/SP/PP", TP section: the
 * QK RMSNorm normalises across heads, i.e. over a token's whole H*D hidden vector, and
 * 3D RoPE acts by token position, independent of the head split; CP section: the RoPE
 * cos/sin are sliced with the same token range as the tokens).  For token t = s*(N/p) + n
 * and c = 0 (q) or 1 (k), over the token's H*D values x:
 *     r   = 1 / sqrt(mean(x^2) + eps)
 *     y_e = x_e * r * gamma_c[e]                       e = h*D + d
 *     per head, per pair i < D/2 (elements 2i, 2i+1 of the head):
 *     out_2i   = y_2i cos[t][i] - y_2i+1 sin[t][i]
 *     out_2i+1 = y_2i sin[t][i] + y_2i+1 cos[t][i]
 * and v (c = 2) is copied unchanged.  Layouts: in [p,B,N/p,3,H,D], gamma_q/gamma_k [H*D],
 * cos/sin [N, D/2] (the positions of the whole sequence), out [p,3,B,N,H/p,D]. */
int oracle_qkv_norm_rope(const double *in, const double *gamma_q, const double *gamma_k,
                         const double *cs, const double *sn, double *out,
                         int p, int B, int N, int H, int D, double eps)
{
    if (p <= 0 || B <= 0 || N <= 0 || H <= 0 || D <= 0 || D % 2 != 0 || !(eps >= 0.0))
        return -1;
    if (N % p != 0 || H % p != 0)
        return -1;
    long Ns = N / p, Hs = H / p, HD = (long)H * D;
    long ntok = (long)p * B * Ns;
#pragma omp parallel for schedule(static)
    for (long tk = 0; tk < ntok; ++tk) {
        long s = tk / (B * Ns), b = (tk / Ns) % B, n = tk % Ns;
        long t = s * Ns + n;
        double *y = (double *)malloc(sizeof(double) * HD);
        for (long c = 0; c < 3; ++c) {
            const double *x = in + (((s * B + b) * Ns + n) * 3 + c) * HD;
            if (c < 2) {
                const double *gam = c == 0 ? gamma_q : gamma_k;
                double ss = 0.0;
                for (long e = 0; e < HD; ++e)
                    ss += x[e] * x[e];
                double r = 1.0 / sqrt(ss / (double)HD + eps);
                for (long e = 0; e < HD; ++e)
                    y[e] = x[e] * r * gam[e];
                for (long h = 0; h < H; ++h)
                    for (long i = 0; i < D / 2; ++i) {
                        double a = y[h * D + 2 * i], bb = y[h * D + 2 * i + 1];
                        double co = cs[t * (D / 2) + i], si = sn[t * (D / 2) + i];
                        y[h * D + 2 * i] = a * co - bb * si;
                        y[h * D + 2 * i + 1] = a * si + bb * co;
                    }
            } else {
                for (long e = 0; e < HD; ++e)
                    y[e] = x[e];
            }
            for (long h = 0; h < H; ++h) {
                long j = h / Hs, hh = h % Hs;
                double *dst = out + ((((j * 3 + c) * B + b) * (long)N + t) * Hs + hh) * D;
                for (long d = 0; d < D; ++d)
                    dst[d] = y[h * D + d];
            }
        }
        free(y);
    }
    return 0;
}

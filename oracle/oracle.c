/*
 * oracle.c -- plain fp64 CPU definition of exact attention and its gradients.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (per batch b and query head hq; the key/value head is
 * hk = hq / (Hq/Hkv)):
 *
 *   S_ij = scale * sum_t Q_it K_jt                      (scores, scaled)
 *   S_ij = -inf  for j > i when causal                  (mask after scaling)
 *   L_i  = m_i + ln sum_j exp(S_ij - m_i),  m_i = max_j S_ij
 *   P_ij = exp(S_ij - L_i)
 *   O_i  = sum_j P_ij V_j
 *
 * and, given dO, the gradients of sum(dO * O):
 *
 *   dP_ij = sum_t dO_it V_jt
 *   D_i   = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij K_j
 *   dK_j  = scale * sum_{hq in group} sum_i dS_ij Q_i
 *   dV_j  =         sum_{hq in group} sum_i P_ij dO_i
 *
 * Sources (FlashAttention-2 summary page, zhaifeiyue.github.io, section 3
 * "Target operation" for O = softmax(QK^T)V with optional causal mask and
 * FP16/BF16 inputs; section 4 symbol table for L = m + log(l) and
 * D = rowsum(dO o O); section 4 "checks" for exactness and for GQA/MQA
 * sharing K/V heads with dK/dV summed across the sharing heads; section 3
 * FLOP formula for the five backward matmuls).  The pages do not print the
 * backward formulas beyond D and P = exp(S - L); the ones above follow from
 * differentiating the definition.  The scale multiplies the scores before
 * masking and the softmax; L is a natural-log logsumexp of the scaled,
 * masked scores.
 *
 * This is the definition, evaluated directly: every row of S is formed in
 * full, its true maximum is taken in one pass, and no online or tiled
 * softmax is used.  Sums run in index order in double precision.  No BLAS.
 *
 * Layout: contiguous row-major [B, H, N, d] for Q, K, V, O, dO, dQ, dK, dV
 * (H = Hq for Q/O/dO/dQ, H = Hkv for K/V/dK/dV); [B, Hq, N] for L and D.
 *
 * Block-sparse attention (FlashAttention paper page, aipaper.jasonlin.tech,
 * key contributions and limitations: attention restricted to a predefined
 * block sparsity pattern): every entry point takes a block mask bm, NULL for
 * dense attention, else bytes [nb, nb] with nb = ceil(N / 128), row-major by
 * query block, shared by all batches and heads.  Scores in a zero block are
 * masked (-inf) exactly like scores above the causal diagonal, and both
 * masks may apply at once.  A query row left with no unmasked score has
 * L_i = -inf, O_i = 0, D_i = 0, dQ_i = 0 and adds nothing to dK or dV.
 *
 * Return value of every entry point: 0 on success, -1 on bad sizes
 * (negative sizes, Hq not a multiple of Hkv, d < 1 when there is work).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static int check_sizes(int B, int Hq, int Hkv, int N, int d)
{
    if (B < 0 || Hq < 0 || Hkv < 0 || N < 0 || d < 0) return -1;
    if (Hkv == 0) return (Hq == 0) ? 0 : -1;
    if (Hq % Hkv != 0) return -1;
    if (d < 1 && (long)B * Hq * N > 0) return -1;
    return 0;
}

static const double *head_ptr(const double *X, int b, int h, int H, int N, int d)
{
    return X + (((size_t)b * H + h) * (size_t)N) * (size_t)d;
}

/*
 * Which scores are masked: the causal mask (j > i) and, for block-sparse
 * attention, a block mask bm [nb, nb] of 128 x 128 blocks (row-major, one
 * byte per block, shared by every batch and head): S_ij is masked when
 * bm[(i / 128) * nb + j / 128] == 0.  bm == NULL: no block mask.
 */
#define ORACLE_SPARSE_BLOCK 128
typedef struct {
    int causal;
    const unsigned char *bm;
    int nb;
} mask_t;

static int is_masked(const mask_t *mk, int i, int j)
{
    if (mk->causal && j > i) return 1;
    if (mk->bm && !mk->bm[(size_t)(i / ORACLE_SPARSE_BLOCK) * mk->nb + j / ORACLE_SPARSE_BLOCK]) return 1;
    return 0;
}

/*
 * exp(s - L) for a row with logsumexp L.  A masked score (s = -inf) gives 0,
 * also in a row whose every score is masked (L = -inf), where the difference
 * itself would be undefined.
 */
static double prob(double s, double L)
{
    return s == -INFINITY ? 0.0 : exp(s - L);
}

/* Scaled, masked score S_ij of one query row q (length d) against key row k. */
static double score(const double *q, const double *k, int d, double scale,
                    const mask_t *mk, int i, int j)
{
    if (is_masked(mk, i, j)) return -INFINITY;
    double acc = 0.0;
    for (int t = 0; t < d; ++t) acc += q[t] * k[t];
    return scale * acc;
}

/*
 * Row i of one head: fills s[0..N) with the scaled masked scores and returns
 * L_i = m + ln sum_j exp(s_j - m).  The causal mask alone keeps j = 0; a
 * block mask can mask a whole row, whose logsumexp over no terms is -inf
 * (its output row is then 0 and it contributes nothing to any gradient).
 */
static double row_scores_lse(const double *Qh, const double *Kh, int N, int d,
                             double scale, const mask_t *mk, int i, double *s)
{
    const double *q = Qh + (size_t)i * d;
    double m = -INFINITY;
    for (int j = 0; j < N; ++j) {
        s[j] = score(q, Kh + (size_t)j * d, d, scale, mk, i, j);
        if (s[j] > m) m = s[j];
    }
    if (m == -INFINITY) return -INFINITY;
    double sum = 0.0;
    for (int j = 0; j < N; ++j) sum += exp(s[j] - m);
    return m + log(sum);
}

/* Forward of one query row: O_i (length d) and L_i. */
static double row_forward(const double *Qh, const double *Kh, const double *Vh,
                          int N, int d, double scale, const mask_t *mk, int i,
                          double *s, double *o)
{
    double L = row_scores_lse(Qh, Kh, N, d, scale, mk, i, s);
    for (int t = 0; t < d; ++t) o[t] = 0.0;
    for (int j = 0; j < N; ++j) {
        double p = prob(s[j], L);
        if (p == 0.0) continue;              /* masked (exp(-inf) = 0) */
        const double *v = Vh + (size_t)j * d;
        for (int t = 0; t < d; ++t) o[t] += p * v[t];
    }
    return L;
}

int oracle_fwd(const double *Q, const double *K, const double *V, double *O,
               double *L, int B, int Hq, int Hkv, int N, int d, int causal, const unsigned char *bm,
               double scale)
{
    const mask_t mk = {causal, bm, (N + ORACLE_SPARSE_BLOCK - 1) / ORACLE_SPARSE_BLOCK};
    if (check_sizes(B, Hq, Hkv, N, d)) return -1;
    if ((long)B * Hq * N == 0) return 0;
    const int G = Hq / Hkv;
    const long rows = (long)B * Hq * N;
    #pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        #pragma omp for schedule(dynamic, 16)
        for (long r = 0; r < rows; ++r) {
            int i = (int)(r % N);
            int hq = (int)((r / N) % Hq);
            int b = (int)(r / ((long)N * Hq));
            const double *Qh = head_ptr(Q, b, hq, Hq, N, d);
            const double *Kh = head_ptr(K, b, hq / G, Hkv, N, d);
            const double *Vh = head_ptr(V, b, hq / G, Hkv, N, d);
            double *o = O + (size_t)r * d;
            double l = row_forward(Qh, Kh, Vh, N, d, scale, &mk, i, s, o);
            if (L) L[r] = l;
        }
        free(s);
    }
    return 0;
}

/*
 * Forward of selected rows only: row r of the output is query row ri[r] of
 * head (rb[r], rh[r]).  O_rows is [n, d], L_rows is [n].  Used to check
 * outputs of large problems one row at a time.
 */
int oracle_fwd_rows(const double *Q, const double *K, const double *V,
                    int B, int Hq, int Hkv, int N, int d, int causal, const unsigned char *bm,
                    double scale, int n, const int *rb, const int *rh,
                    const int *ri, double *O_rows, double *L_rows)
{
    const mask_t mk = {causal, bm, (N + ORACLE_SPARSE_BLOCK - 1) / ORACLE_SPARSE_BLOCK};
    if (check_sizes(B, Hq, Hkv, N, d)) return -1;
    for (int r = 0; r < n; ++r)
        if (rb[r] < 0 || rb[r] >= B || rh[r] < 0 || rh[r] >= Hq ||
            ri[r] < 0 || ri[r] >= N) return -1;
    if (n == 0) return 0;
    const int G = Hq / Hkv;
    #pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        #pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < n; ++r) {
            const double *Qh = head_ptr(Q, rb[r], rh[r], Hq, N, d);
            const double *Kh = head_ptr(K, rb[r], rh[r] / G, Hkv, N, d);
            const double *Vh = head_ptr(V, rb[r], rh[r] / G, Hkv, N, d);
            double l = row_forward(Qh, Kh, Vh, N, d, scale, &mk, ri[r], s,
                                   O_rows + (size_t)r * d);
            if (L_rows) L_rows[r] = l;
        }
        free(s);
    }
    return 0;
}

/*
 * Gradients of one key/value head (b, hk) from the row statistics of its G
 * query heads: Lst [G*N] the logsumexp L_i and Dst [G*N] the D_i of each
 * query row.  P_ij = exp(S_ij - L_i), dS_ij = P_ij (dP_ij - D_i).  Two
 * passes over the plain definitions: dQ by rows, then dK/dV by key columns
 * (so no two threads write one location).
 */
static void grads_from_stats(const double *Q, const double *K, const double *V,
                             const double *dO, int Hq, int Hkv, int N, int d,
                             const mask_t *mk, double scale, int b, int hk,
                             const double *Lst, const double *Dst,
                             double *dQg, double *dKh, double *dVh)
{
    const int G = Hq / Hkv;
    const double *Kh = head_ptr(K, b, hk, Hkv, N, d);
    const double *Vh = head_ptr(V, b, hk, Hkv, N, d);

    /* dQ_i = scale * sum_j dS_ij K_j. */
    #pragma omp parallel for schedule(dynamic, 8)
    for (long r = 0; r < (long)G * N; ++r) {
            int g = (int)(r / N), i = (int)(r % N);
            int hq = hk * G + g;
            const double *Qh = head_ptr(Q, b, hq, Hq, N, d);
            const double *q = Qh + (size_t)i * d;
            const double *dOr = head_ptr(dO, b, hq, Hq, N, d) + (size_t)i * d;
            double *dq = dQg + (size_t)r * d;
            for (int t = 0; t < d; ++t) dq[t] = 0.0;
            for (int j = 0; j < N; ++j) {
                double sij = score(q, Kh + (size_t)j * d, d, scale, mk, i, j);
                double p = prob(sij, Lst[r]);
                if (p == 0.0) continue;
                const double *v = Vh + (size_t)j * d;
                double dp = 0.0;
                for (int t = 0; t < d; ++t) dp += dOr[t] * v[t];
                double ds = p * (dp - Dst[r]);
                const double *k = Kh + (size_t)j * d;
                for (int t = 0; t < d; ++t) dq[t] += ds * k[t];
            }
            for (int t = 0; t < d; ++t) dq[t] *= scale;
    }

    /* dK_j = scale * sum_g sum_i dS_ij Q_i ;  dV_j = sum_g sum_i P_ij dO_i. */
    #pragma omp parallel for schedule(dynamic, 8)
    for (int j = 0; j < N; ++j) {
        const double *k = Kh + (size_t)j * d;
        const double *v = Vh + (size_t)j * d;
        double *dk = dKh + (size_t)j * d;
        double *dv = dVh + (size_t)j * d;
        for (int t = 0; t < d; ++t) { dk[t] = 0.0; dv[t] = 0.0; }
        for (int g = 0; g < G; ++g) {
            int hq = hk * G + g;
            const double *Qh = head_ptr(Q, b, hq, Hq, N, d);
            const double *dOh = head_ptr(dO, b, hq, Hq, N, d);
            for (int i = 0; i < N; ++i) {
                const double *q = Qh + (size_t)i * d;
                double sij = score(q, k, d, scale, mk, i, j);
                double p = prob(sij, Lst[(long)g * N + i]);
                if (p == 0.0) continue;
                const double *dOr = dOh + (size_t)i * d;
                double dp = 0.0;
                for (int t = 0; t < d; ++t) dp += dOr[t] * v[t];
                double ds = p * (dp - Dst[(long)g * N + i]);
                for (int t = 0; t < d; ++t) {
                    dv[t] += p * dOr[t];
                    dk[t] += ds * q[t];
                }
            }
        }
        for (int t = 0; t < d; ++t) dk[t] *= scale;
    }
}

/*
 * Backward of one key/value head (b, hk) and the G query heads that share it.
 *   dQg [G, N, d]  dQ of query heads hk*G .. hk*G+G-1
 *   dKh, dVh [N, d]
 *   Lg, Dg [G, N]  the statistics L and D of those query heads (may be NULL)
 * The row statistics L_i and D_i = sum_j P_ij dP_ij first, then the
 * gradients from them (grads_from_stats).
 */
static void bwd_one_kv_head(const double *Q, const double *K, const double *V,
                            const double *dO, int Hq, int Hkv, int N, int d,
                            const mask_t *mk, double scale, int b, int hk,
                            double *dQg, double *dKh, double *dVh,
                            double *Lg, double *Dg)
{
    const int G = Hq / Hkv;
    const double *Kh = head_ptr(K, b, hk, Hkv, N, d);
    const double *Vh = head_ptr(V, b, hk, Hkv, N, d);
    double *Lst = (double *)malloc(sizeof(double) * (size_t)G * N);
    double *Dst = (double *)malloc(sizeof(double) * (size_t)G * N);

    /* Pass 1: L_i and D_i = sum_j P_ij dP_ij for every query row. */
    #pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        #pragma omp for schedule(dynamic, 8)
        for (long r = 0; r < (long)G * N; ++r) {
            int g = (int)(r / N), i = (int)(r % N);
            int hq = hk * G + g;
            const double *Qh = head_ptr(Q, b, hq, Hq, N, d);
            const double *dOr = head_ptr(dO, b, hq, Hq, N, d) + (size_t)i * d;
            double L = row_scores_lse(Qh, Kh, N, d, scale, mk, i, s);
            double D = 0.0;
            for (int j = 0; j < N; ++j) {
                double p = prob(s[j], L);
                if (p == 0.0) continue;
                const double *v = Vh + (size_t)j * d;
                double dp = 0.0;
                for (int t = 0; t < d; ++t) dp += dOr[t] * v[t];
                D += p * dp;
            }
            Lst[r] = L;
            Dst[r] = D;
        }
        free(s);
    }

    grads_from_stats(Q, K, V, dO, Hq, Hkv, N, d, mk, scale, b, hk, Lst, Dst, dQg, dKh, dVh);

    if (Lg) memcpy(Lg, Lst, sizeof(double) * (size_t)G * N);
    if (Dg) memcpy(Dg, Dst, sizeof(double) * (size_t)G * N);
    free(Lst);
    free(Dst);
}

int oracle_bwd(const double *Q, const double *K, const double *V,
               const double *dO, double *dQ, double *dK, double *dV,
               double *D, int B, int Hq, int Hkv, int N, int d, int causal, const unsigned char *bm,
               double scale)
{
    const mask_t mk = {causal, bm, (N + ORACLE_SPARSE_BLOCK - 1) / ORACLE_SPARSE_BLOCK};
    if (check_sizes(B, Hq, Hkv, N, d)) return -1;
    if ((long)B * Hq * N == 0) return 0;
    const int G = Hq / Hkv;
    for (int b = 0; b < B; ++b)
        for (int hk = 0; hk < Hkv; ++hk) {
            size_t qoff = (((size_t)b * Hq + (size_t)hk * G) * N) * d;
            size_t koff = (((size_t)b * Hkv + hk) * (size_t)N) * d;
            double *Dg = D ? D + ((size_t)b * Hq + (size_t)hk * G) * N : NULL;
            bwd_one_kv_head(Q, K, V, dO, Hq, Hkv, N, d, &mk, scale, b, hk,
                            dQ + qoff, dK + koff, dV + koff, NULL, Dg);
        }
    return 0;
}

/*
 * Backward restricted to one key/value head (b, hk): dQg [G,N,d] for query
 * heads hk*G.., dKh/dVh [N,d], and optionally Lg/Dg [G,N].  Used to check
 * single heads of large problems.
 */
int oracle_bwd_head(const double *Q, const double *K, const double *V,
                    const double *dO, int B, int Hq, int Hkv, int N, int d,
                    int causal, const unsigned char *bm, double scale, int b, int hk, double *dQg,
                    double *dKh, double *dVh, double *Lg, double *Dg)
{
    const mask_t mk = {causal, bm, (N + ORACLE_SPARSE_BLOCK - 1) / ORACLE_SPARSE_BLOCK};
    if (check_sizes(B, Hq, Hkv, N, d)) return -1;
    if (b < 0 || b >= B || hk < 0 || hk >= Hkv) return -1;
    if (N == 0) return 0;
    bwd_one_kv_head(Q, K, V, dO, Hq, Hkv, N, d, &mk, scale, b, hk,
                    dQg, dKh, dVh, Lg, Dg);
    return 0;
}

/* ------------------------------------------------------------------------
 * The same definition evaluated at the method's working precision.
 *
 * The method multiplies FP16/BF16 operands with FP32 accumulation (summary
 * page, section 3 "Target operation"); its outputs are stored in bf16.  So
 * the probabilities P enter both P V (forward) and P^T dO (backward) as
 * bf16, dS enters dS^T Q and dS K as bf16, and D = rowsum(dO o O) is formed
 * from the stored bf16 O.  This variant rounds exactly there (values first
 * rounded to fp32, then to bf16, round to nearest even) and keeps every
 * other step of the definition in double:
 *   forward:  p_ij = exp(S_ij - m_i) in [0, 1];  O_i = sum_j bf16(p_ij) V_j
 *             / sum_j p_ij;  O is stored as bf16(O).
 *   backward: D_i = dO_i . bf16(O_i);  P_ij = exp(S_ij - L_i);
 *             dV_j = sum_i bf16(P_ij) dO_i;  dS_ij = P_ij (dP_ij - D_i);
 *             dQ_i = scale sum_j bf16(dS_ij) K_j;  dK_j = scale sum_i bf16(dS_ij) Q_i.
 * The gradients are returned unrounded (double).  It measures how far an
 * exact execution of the method at this precision lands from the exact
 * function; the tests use it to calibrate, never to replace, the reference.
 * ------------------------------------------------------------------------ */
static double round_bf16(double x)
{
    float f = (float)x;
    unsigned int u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u) return (double)f;   /* inf / nan */
    u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Forward row at the working precision: O_i (unrounded) from bf16(p_ij), and L_i. */
static double row_forward_bf16(const double *Qh, const double *Kh, const double *Vh,
                               int N, int d, double scale, const mask_t *mk, int i,
                               double *s, double *o)
{
    const double *q = Qh + (size_t)i * d;
    double m = -INFINITY;
    for (int j = 0; j < N; ++j) {
        s[j] = score(q, Kh + (size_t)j * d, d, scale, mk, i, j);
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int t = 0; t < d; ++t) o[t] = 0.0;
    if (m == -INFINITY) return -INFINITY;    /* every score masked: O_i = 0 */
    for (int j = 0; j < N; ++j) {
        double p = exp(s[j] - m);
        l += p;
        if (p == 0.0) continue;
        double pb = round_bf16(p);
        const double *v = Vh + (size_t)j * d;
        for (int t = 0; t < d; ++t) o[t] += pb * v[t];
    }
    for (int t = 0; t < d; ++t) o[t] /= l;
    return m + log(l);
}

int oracle_fwd_bf16(const double *Q, const double *K, const double *V, double *O,
                    double *L, int B, int Hq, int Hkv, int N, int d, int causal, const unsigned char *bm,
                    double scale)
{
    const mask_t mk = {causal, bm, (N + ORACLE_SPARSE_BLOCK - 1) / ORACLE_SPARSE_BLOCK};
    if (check_sizes(B, Hq, Hkv, N, d)) return -1;
    if ((long)B * Hq * N == 0) return 0;
    const int G = Hq / Hkv;
    const long rows = (long)B * Hq * N;
    #pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        #pragma omp for schedule(dynamic, 16)
        for (long r = 0; r < rows; ++r) {
            int i = (int)(r % N);
            int hq = (int)((r / N) % Hq);
            int b = (int)(r / ((long)N * Hq));
            const double *Qh = head_ptr(Q, b, hq, Hq, N, d);
            const double *Kh = head_ptr(K, b, hq / G, Hkv, N, d);
            const double *Vh = head_ptr(V, b, hq / G, Hkv, N, d);
            double l = row_forward_bf16(Qh, Kh, Vh, N, d, scale, &mk, i, s, O + (size_t)r * d);
            if (L) L[r] = l;
        }
        free(s);
    }
    return 0;
}

/*
 * Working-precision gradients of one key/value head (b, hk) from row
 * statistics Lst (L_i) and Dst (D_i) of its G query heads [G*N]: as
 * grads_from_stats, with P rounded to bf16 in dV and dS rounded to bf16 in
 * dQ and dK.
 */
static void grads_from_stats_bf16(const double *Q, const double *K, const double *V,
                                  const double *dO, int Hq, int Hkv, int N, int d,
                                  const mask_t *mk, double scale, int b, int hk,
                                  const double *Lst, const double *Dst,
                                  double *dQg, double *dKh, double *dVh)
{
    const int G = Hq / Hkv;
    const double *Kh = head_ptr(K, b, hk, Hkv, N, d);
    const double *Vh = head_ptr(V, b, hk, Hkv, N, d);
    /* dQ_i = scale * sum_j bf16(dS_ij) K_j */
    #pragma omp parallel for schedule(dynamic, 8)
    for (long r = 0; r < (long)G * N; ++r) {
        int g = (int)(r / N), i = (int)(r % N);
        int hq = hk * G + g;
        const double *q = head_ptr(Q, b, hq, Hq, N, d) + (size_t)i * d;
        const double *dOr = head_ptr(dO, b, hq, Hq, N, d) + (size_t)i * d;
        double *dq = dQg + (size_t)r * d;
        for (int t = 0; t < d; ++t) dq[t] = 0.0;
        for (int j = 0; j < N; ++j) {
            double p = prob(score(q, Kh + (size_t)j * d, d, scale, mk, i, j), Lst[r]);
            if (p == 0.0) continue;
            const double *v = Vh + (size_t)j * d;
            double dp = 0.0;
            for (int t = 0; t < d; ++t) dp += dOr[t] * v[t];
            double ds = round_bf16(p * (dp - Dst[r]));
            const double *k = Kh + (size_t)j * d;
            for (int t = 0; t < d; ++t) dq[t] += ds * k[t];
        }
        for (int t = 0; t < d; ++t) dq[t] *= scale;
    }
    /* dV_j = sum bf16(P_ij) dO_i ;  dK_j = scale * sum bf16(dS_ij) Q_i */
    #pragma omp parallel for schedule(dynamic, 8)
    for (int j = 0; j < N; ++j) {
        const double *k = Kh + (size_t)j * d;
        const double *v = Vh + (size_t)j * d;
        double *dk = dKh + (size_t)j * d;
        double *dv = dVh + (size_t)j * d;
        for (int t = 0; t < d; ++t) { dk[t] = 0.0; dv[t] = 0.0; }
        for (int g = 0; g < G; ++g) {
            int hq = hk * G + g;
            const double *Qh = head_ptr(Q, b, hq, Hq, N, d);
            const double *dOh = head_ptr(dO, b, hq, Hq, N, d);
            for (int i = 0; i < N; ++i) {
                const double *q = Qh + (size_t)i * d;
                double p = prob(score(q, k, d, scale, mk, i, j), Lst[(long)g * N + i]);
                if (p == 0.0) continue;
                const double *dOr = dOh + (size_t)i * d;
                double dp = 0.0;
                for (int t = 0; t < d; ++t) dp += dOr[t] * v[t];
                double pb = round_bf16(p);
                double ds = round_bf16(p * (dp - Dst[(long)g * N + i]));
                for (int t = 0; t < d; ++t) {
                    dv[t] += pb * dOr[t];
                    dk[t] += ds * q[t];
                }
            }
        }
        for (int t = 0; t < d; ++t) dk[t] *= scale;
    }
}

/* Working-precision backward of one key/value head (b, hk): dQg [G,N,d] of
 * query heads hk*G.., dKh and dVh [N,d]. */
static void bwd_bf16_one_kv_head(const double *Q, const double *K, const double *V,
                                 const double *dO, int Hq, int Hkv, int N, int d,
                                 const mask_t *mk, double scale, int b, int hk,
                                 double *dQg, double *dKh, double *dVh, double *Dg)
{
    const int G = Hq / Hkv;
    const double *Kh = head_ptr(K, b, hk, Hkv, N, d);
    const double *Vh = head_ptr(V, b, hk, Hkv, N, d);
    double *Lst = (double *)malloc(sizeof(double) * (size_t)G * N);
    double *Dst = (double *)malloc(sizeof(double) * (size_t)G * N);
    /* L_i and D_i = dO_i . bf16(O_i), with O_i from the working-precision forward. */
    #pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
        #pragma omp for schedule(dynamic, 8)
        for (long r = 0; r < (long)G * N; ++r) {
            int g = (int)(r / N), i = (int)(r % N);
            int hq = hk * G + g;
            const double *Qh = head_ptr(Q, b, hq, Hq, N, d);
            const double *dOr = head_ptr(dO, b, hq, Hq, N, d) + (size_t)i * d;
            Lst[r] = row_forward_bf16(Qh, Kh, Vh, N, d, scale, mk, i, s, o);
            double D = 0.0;
            for (int t = 0; t < d; ++t) D += dOr[t] * round_bf16(o[t]);
            Dst[r] = D;
        }
        free(s);
        free(o);
    }
    grads_from_stats_bf16(Q, K, V, dO, Hq, Hkv, N, d, mk, scale, b, hk, Lst, Dst, dQg, dKh, dVh);
    if (Dg) memcpy(Dg, Dst, sizeof(double) * (size_t)G * N);
    free(Lst);
    free(Dst);
}

int oracle_bwd_bf16(const double *Q, const double *K, const double *V,
                    const double *dO, double *dQ, double *dK, double *dV, double *D,
                    int B, int Hq, int Hkv, int N, int d, int causal, const unsigned char *bm, double scale)
{
    const mask_t mk = {causal, bm, (N + ORACLE_SPARSE_BLOCK - 1) / ORACLE_SPARSE_BLOCK};
    if (check_sizes(B, Hq, Hkv, N, d)) return -1;
    if ((long)B * Hq * N == 0) return 0;
    const int G = Hq / Hkv;
    for (int b = 0; b < B; ++b)
        for (int hk = 0; hk < Hkv; ++hk) {
            size_t qoff = (((size_t)b * Hq + (size_t)hk * G) * N) * d;
            size_t koff = (((size_t)b * Hkv + hk) * (size_t)N) * d;
            double *Dg = D ? D + ((size_t)b * Hq + (size_t)hk * G) * N : NULL;
            bwd_bf16_one_kv_head(Q, K, V, dO, Hq, Hkv, N, d, &mk, scale, b, hk,
                                 dQ + qoff, dK + koff, dV + koff, Dg);
        }
    return 0;
}

int oracle_bwd_bf16_head(const double *Q, const double *K, const double *V,
                         const double *dO, int B, int Hq, int Hkv, int N, int d,
                         int causal, const unsigned char *bm, double scale, int b, int hk, double *dQg,
                         double *dKh, double *dVh)
{
    const mask_t mk = {causal, bm, (N + ORACLE_SPARSE_BLOCK - 1) / ORACLE_SPARSE_BLOCK};
    if (check_sizes(B, Hq, Hkv, N, d)) return -1;
    if (b < 0 || b >= B || hk < 0 || hk >= Hkv) return -1;
    if (N == 0) return 0;
    bwd_bf16_one_kv_head(Q, K, V, dO, Hq, Hkv, N, d, &mk, scale, b, hk, dQg, dKh, dVh, NULL);
    return 0;
}

/*
 * The backward from a forward's saved outputs, the way the method runs it
 * (summary page, section 4 symbol table: P is rebuilt from the saved
 * logsumexp L, and D = rowsum(dO o O) is formed from the saved O).  For
 * given O [B,Hq,N,d] and L [B,Hq,N]:
 *   P_ij = exp(S_ij - L_i),  D_i = sum_t dO_it O_it,  dS_ij = P_ij (dP_ij - D_i),
 *   dQ, dK, dV as in the definition above, in fp64.
 * With the exact forward's O and L this is oracle_bwd.  With a stored
 * (rounded) O it is the exact gradient the method computes from that O: the
 * difference from oracle_bwd is then the effect of O's rounding through D.
 * A row with L_i = -inf (every score masked) has P_i = 0, dQ_i = 0.
 * oracle_bwd_given_bf16 is the same at the method's working precision: P
 * rounded to bf16 in dV, dS rounded to bf16 in dQ and dK (results unrounded).
 */
static int bwd_given(const double *Q, const double *K, const double *V,
                     const double *O, const double *L, const double *dO,
                     double *dQ, double *dK, double *dV, int B, int Hq, int Hkv,
                     int N, int d, int causal, const unsigned char *bm, double scale,
                     int working_precision)
{
    const mask_t mk = {causal, bm, (N + ORACLE_SPARSE_BLOCK - 1) / ORACLE_SPARSE_BLOCK};
    if (check_sizes(B, Hq, Hkv, N, d)) return -1;
    if ((long)B * Hq * N == 0) return 0;
    const int G = Hq / Hkv;
    double *Dst = (double *)malloc(sizeof(double) * (size_t)G * N);
    for (int b = 0; b < B; ++b)
        for (int hk = 0; hk < Hkv; ++hk) {
            const size_t row0 = ((size_t)b * Hq + (size_t)hk * G) * (size_t)N;
            for (long r = 0; r < (long)G * N; ++r) {
                const double *o = O + (row0 + (size_t)r) * d;
                const double *g = dO + (row0 + (size_t)r) * d;
                double D = 0.0;
                for (int t = 0; t < d; ++t) D += g[t] * o[t];
                Dst[r] = D;
            }
            const double *Lg = L + row0;
            const size_t koff = (((size_t)b * Hkv + hk) * (size_t)N) * d;
            if (working_precision)
                grads_from_stats_bf16(Q, K, V, dO, Hq, Hkv, N, d, &mk, scale, b, hk, Lg, Dst,
                                      dQ + row0 * d, dK + koff, dV + koff);
            else
                grads_from_stats(Q, K, V, dO, Hq, Hkv, N, d, &mk, scale, b, hk, Lg, Dst,
                                 dQ + row0 * d, dK + koff, dV + koff);
        }
    free(Dst);
    return 0;
}

int oracle_bwd_given(const double *Q, const double *K, const double *V,
                     const double *O, const double *L, const double *dO,
                     double *dQ, double *dK, double *dV, int B, int Hq, int Hkv,
                     int N, int d, int causal, const unsigned char *bm, double scale)
{
    return bwd_given(Q, K, V, O, L, dO, dQ, dK, dV, B, Hq, Hkv, N, d, causal, bm, scale, 0);
}

int oracle_bwd_given_bf16(const double *Q, const double *K, const double *V,
                          const double *O, const double *L, const double *dO,
                          double *dQ, double *dK, double *dV, int B, int Hq, int Hkv,
                          int N, int d, int causal, const unsigned char *bm, double scale)
{
    return bwd_given(Q, K, V, O, L, dO, dQ, dK, dV, B, Hq, Hkv, N, d, causal, bm, scale, 1);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

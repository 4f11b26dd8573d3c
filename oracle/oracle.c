/*
 * Reference oracle for exact attention — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 CPU implementation of the unfused three-step definition
 * of scaled-dot-product attention and of its gradients.  It exists so that the
 * HIP kernels of exact_attention_30_amd can be checked against something that
 * shares no code with them.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the library never does.
 *
 * Sources (the four web pages on FlashAttention):
 *   [PAI] "FlashAttention: l'attenzione che non spreca memoria" (book.paithon.it)
 *   [SMB] "L'attention fusionnée" (Smallem series, smallbard.com)
 *   [CTL] "Optimización de Flash Attention para un rendimiento óptimo en
 *          NVIDIA CUDA Tile" (congresoia365.net)
 *   [PDB] "FlashAttention" (note, paweldubiel.com)
 *
 * What is computed (per batch b, query head h, kv head hk = h / (Hq/Hkv)), for
 * Tq query rows against Tk key rows:
 *   s_ij  = scale * <q_i, k_j>, and -inf for a future key j > i + off when causal
 *           ([SMB] «Ce que l'attention écrit en mémoire»; [CTL] «Atención causal»;
 *           off is the query rows' position offset, the cuTile kernel's
 *           input_pos of [CTL] «Parte 1»: query row i stands at position i + off
 *           among the keys)
 *   P_ij  = exp(s_ij - m_i) / l_i with m_i = max_j s_ij, l_i = sum_j exp(s_ij - m_i)
 *           (safe softmax: [PAI] «La online softmax, con i numeri»; [CTL] «Entendiendo
 *           softmax en línea»)
 *   o_i   = sum_j P_ij v_j,   lse_i = m_i + ln l_i   ([SMB] «La passe arrière»)
 * Backward, for the scalar loss sum(O * dO) ([SMB] «La passe arrière»):
 *   dP_ij = <dO_i, v_j>,  c_i = sum_j P_ij dP_ij  (the softmax Jacobian term,
 *           written from its definition; the pages' shortcut c_i = <dO_i, o_i> is
 *           NOT used here, so tests can check it)
 *   dS_ij = P_ij (dP_ij - c_i)
 *   dq_i  = scale * sum_j dS_ij k_j
 *   dk_j  = scale * sum_{h in group} sum_i dS_ij q_i
 *   dv_j  =         sum_{h in group} sum_i P_ij dO_i
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - GQA grouping is consecutive: query head h reads kv head h / (Hq/Hkv).
 *   - lse is in natural-log units of the scaled scores.
 *   - A row with no visible key (causal with i + off < 0) gives o = 0,
 *     lse = -inf and zero gradients.
 *
 * Layouts: row-major, q/o/dO/dq [B][Hq][Tq][D], k/v/dk/dv [B][Hkv][Tk][D],
 * lse/c [B][Hq][Tq].  All arithmetic in double; exp/log from libm.
 * Every loop over keys and over query rows runs in ascending index order, and
 * each output element is written by exactly one thread, so results do not
 * depend on the OpenMP thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

typedef struct {
    int B, Hq, Hkv, Tq, Tk, D;
    double scale;
    int causal;
    int off; /* position of query row 0 among the keys (causal only) */
} shape_t;

static int check_shape(const shape_t* s)
{
    if (s->B < 1 || s->Hq < 1 || s->Hkv < 1 || s->Tq < 0 || s->Tk < 0 || s->D < 1)
        return ORACLE_ERR_ARG;
    if (s->Hq % s->Hkv != 0) return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

static const double* qrow(const double* q, const shape_t* s, int b, int h, int i)
{
    return q + (((size_t)b * s->Hq + h) * s->Tq + i) * s->D;
}

static const double* kvrow(const double* k, const shape_t* s, int b, int hk, int j)
{
    return k + (((size_t)b * s->Hkv + hk) * s->Tk + j) * s->D;
}

static double dot(const double* x, const double* y, int D)
{
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += x[d] * y[d];
    return acc;
}

/* Is key j visible to query i? */
static int visible(const shape_t* s, int i, int j)
{
    return s->causal ? ((long)j <= (long)i + s->off) : 1;
}

/*
 * One query row, step by step as the definition reads.  Fills
 *   p[j]  = P_ij for every key j (0 for an invisible key),
 *   and returns m_i, l_i through pointers.
 * s_buf is scratch of length Tk.
 */
static void softmax_row(const shape_t* s, const double* q_i, const double* k_head, int i,
                        double* s_buf, double* p, double* m_out, double* l_out)
{
    const int T = s->Tk, D = s->D;
    /* step 1: scores */
    for (int j = 0; j < T; ++j)
        s_buf[j] = visible(s, i, j) ? s->scale * dot(q_i, k_head + (size_t)j * D, D) : -INFINITY;
    /* step 2: safe softmax */
    double m = -INFINITY;
    for (int j = 0; j < T; ++j)
        if (s_buf[j] > m) m = s_buf[j];
    double l = 0.0;
    if (m == -INFINITY) { /* no visible key: define P = 0 */
        for (int j = 0; j < T; ++j) p[j] = 0.0;
    } else {
        for (int j = 0; j < T; ++j) {
            p[j] = (s_buf[j] == -INFINITY) ? 0.0 : exp(s_buf[j] - m);
            l += p[j];
        }
        for (int j = 0; j < T; ++j) p[j] /= l;
    }
    *m_out = m;
    *l_out = l;
}

static double lse_of(double m, double l)
{
    return (m == -INFINITY) ? -INFINITY : m + log(l);
}

/* Forward for one (b, h, i): writes o_i (D values) and lse_i. */
static void fwd_one_row(const shape_t* s, const double* q, const double* k, const double* v,
                        int b, int h, int i, double* o_i, double* lse_i, double* om_i,
                        double* s_buf, double* p)
{
    const int G = s->Hq / s->Hkv, hk = h / G, D = s->D, T = s->Tk;
    const double* k_head = kvrow(k, s, b, hk, 0);
    const double* v_head = kvrow(v, s, b, hk, 0);
    double m, l;
    softmax_row(s, qrow(q, s, b, h, i), k_head, i, s_buf, p, &m, &l);
    /* step 3: o_i = sum_j P_ij v_j */
    for (int d = 0; d < D; ++d) o_i[d] = 0.0;
    if (om_i)
        for (int d = 0; d < D; ++d) om_i[d] = 0.0;
    for (int j = 0; j < T; ++j) {
        if (p[j] == 0.0) continue;
        const double* vj = v_head + (size_t)j * D;
        for (int d = 0; d < D; ++d) o_i[d] += p[j] * vj[d];
        if (om_i)
            for (int d = 0; d < D; ++d) om_i[d] += fabs(p[j] * vj[d]);
    }
    *lse_i = lse_of(m, l);
}

/*
 * Backward quantities of one (b, h, i): P row (p), dP row (dp), the row
 * statistics m_i, l_i and the Jacobian term c_i = sum_j P_ij dP_ij.  Returns c_i.
 */
static double bwd_row_terms(const shape_t* s, const double* q, const double* k, const double* v,
                            const double* dout, int b, int h, int i, double* s_buf, double* p,
                            double* dp, double* m_out, double* l_out)
{
    const int G = s->Hq / s->Hkv, hk = h / G, D = s->D, T = s->Tk;
    const double* k_head = kvrow(k, s, b, hk, 0);
    const double* v_head = kvrow(v, s, b, hk, 0);
    const double* do_i = qrow(dout, s, b, h, i);
    softmax_row(s, qrow(q, s, b, h, i), k_head, i, s_buf, p, m_out, l_out);
    double c = 0.0;
    for (int j = 0; j < T; ++j) {
        dp[j] = visible(s, i, j) ? dot(do_i, v_head + (size_t)j * D, D) : 0.0;
        c += p[j] * dp[j];
    }
    return c;
}

/*
 * Per-thread scratch rows: nbuf arrays of length T for each OpenMP thread,
 * taken from one block allocated before the parallel region.
 */
static double* scratch_alloc(int nbuf, int T)
{
    const size_t n = (size_t)omp_get_max_threads() * (size_t)nbuf * (size_t)(T > 0 ? T : 1);
    return (double*)malloc(sizeof(double) * n);
}

static double* scratch_of(double* base, int nbuf, int T, int which)
{
    const size_t row = (size_t)(T > 0 ? T : 1);
    return base + ((size_t)omp_get_thread_num() * (size_t)nbuf + (size_t)which) * row;
}

/* ------------------------------------------------------------------------- */
/* Public C ABI                                                               */
/* ------------------------------------------------------------------------- */

/* Number of OpenMP threads a parallel region of the oracle uses. */
int oracle_threads(void) { return omp_get_max_threads(); }

/*
 * Full forward: o [B,Hq,Tq,D], lse [B,Hq,Tq] for q [B,Hq,Tq,D] and k, v
 * [B,Hkv,Tk,D]; off is the position of query row 0 among the keys (used when
 * causal).  o_mag (nullable) [B,Hq,Tq,D] receives, per output element, the sum
 * of the absolute values of its terms, sum_j |P_ij v_jd|: the scale of the
 * rounding error a finite-precision evaluation of that sum can make.
 */
int oracle_fwd(const double* q, const double* k, const double* v, double* o, double* lse,
               double* o_mag, int B, int Hq, int Hkv, int Tq, int Tk, int D, double scale,
               int causal, int off)
{
    shape_t s = {B, Hq, Hkv, Tq, Tk, D, scale, causal, off};
    if (check_shape(&s) != ORACLE_OK) return ORACLE_ERR_ARG;
    if (Tq == 0) return ORACLE_OK;
    const long rows = (long)B * Hq * Tq;
    double* scr = scratch_alloc(2, Tk);
    if (!scr) return ORACLE_ERR_NOMEM;
#pragma omp parallel for schedule(dynamic, 16)
    for (long r = 0; r < rows; ++r) {
        const int i = (int)(r % Tq), h = (int)((r / Tq) % Hq), b = (int)(r / ((long)Tq * Hq));
        fwd_one_row(&s, q, k, v, b, h, i, o + (size_t)r * D, lse + r,
                    o_mag ? o_mag + (size_t)r * D : NULL, scratch_of(scr, 2, Tk, 0),
                    scratch_of(scr, 2, Tk, 1));
    }
    free(scr);
    return ORACLE_OK;
}

/*
 * Full backward: dq [B,Hq,Tq,D], dk/dv [B,Hkv,Tk,D]; jac (nullable) [B,Hq,Tq]
 * receives c_i.  dq_mag, dk_mag, dv_mag (nullable, shaped like dq, dk, dv)
 * receive per element the sum of the absolute values of its terms
 * (|scale dS_ij k_jd|, |scale dS_ij q_id|, |P_ij dO_id|).
 *
 * Pass 1 (one task per query row) computes dq_i and keeps the row statistics
 * m_i, l_i, c_i.  Pass 2 (one task per key row j of a kv head) sums the
 * contributions of every query row of every query head of the group, in
 * ascending (h, i) order, rebuilding P_ij = exp(s_ij - m_i) / l_i and dP_ij.
 */
int oracle_bwd(const double* q, const double* k, const double* v, const double* dout, double* dq,
               double* dk, double* dv, double* jac, double* dq_mag, double* dk_mag,
               double* dv_mag, int B, int Hq, int Hkv, int Tq, int Tk, int D, double scale,
               int causal, int off)
{
    shape_t s = {B, Hq, Hkv, Tq, Tk, D, scale, causal, off};
    if (check_shape(&s) != ORACLE_OK) return ORACLE_ERR_ARG;
    const int G = Hq / Hkv;
    const long qrows = (long)B * Hq * Tq, krows = (long)B * Hkv * Tk;
    if (Tq == 0 || Tk == 0) { /* no pair of rows: every gradient is zero */
        memset(dq, 0, sizeof(double) * (size_t)qrows * (size_t)D);
        memset(dk, 0, sizeof(double) * (size_t)krows * (size_t)D);
        memset(dv, 0, sizeof(double) * (size_t)krows * (size_t)D);
        if (jac) memset(jac, 0, sizeof(double) * (size_t)qrows);
        return ORACLE_OK;
    }
    double* mst = (double*)malloc(sizeof(double) * (size_t)qrows);
    double* lst = (double*)malloc(sizeof(double) * (size_t)qrows);
    double* cst = (double*)malloc(sizeof(double) * (size_t)qrows);
    double* scr = scratch_alloc(3, Tk);
    if (!mst || !lst || !cst || !scr) {
        free(mst);
        free(lst);
        free(cst);
        free(scr);
        return ORACLE_ERR_NOMEM;
    }

    /* pass 1: per query row */
#pragma omp parallel for schedule(dynamic, 16)
    for (long r = 0; r < qrows; ++r) {
        const int i = (int)(r % Tq), h = (int)((r / Tq) % Hq), b = (int)(r / ((long)Tq * Hq));
        const int hk = h / G;
        double* p = scratch_of(scr, 3, Tk, 1);
        double* dp = scratch_of(scr, 3, Tk, 2);
        double m, l;
        const double c =
            bwd_row_terms(&s, q, k, v, dout, b, h, i, scratch_of(scr, 3, Tk, 0), p, dp, &m, &l);
        mst[r] = m;
        lst[r] = l;
        cst[r] = c;
        double* dq_i = dq + (size_t)r * D;
        double* dqm_i = dq_mag ? dq_mag + (size_t)r * D : NULL;
        for (int d = 0; d < D; ++d) dq_i[d] = 0.0;
        if (dqm_i)
            for (int d = 0; d < D; ++d) dqm_i[d] = 0.0;
        for (int j = 0; j < Tk; ++j) {
            if (!visible(&s, i, j) || m == -INFINITY) continue;
            const double ds = p[j] * (dp[j] - c);
            const double* kj = kvrow(k, &s, b, hk, j);
            for (int d = 0; d < D; ++d) dq_i[d] += ds * kj[d];
            if (dqm_i)
                for (int d = 0; d < D; ++d) dqm_i[d] += fabs(ds * kj[d]);
        }
        for (int d = 0; d < D; ++d) dq_i[d] *= scale;
        if (dqm_i)
            for (int d = 0; d < D; ++d) dqm_i[d] *= fabs(scale);
    }

    /* pass 2: per key row */
#pragma omp parallel for schedule(dynamic, 16)
    for (long r = 0; r < krows; ++r) {
        const int j = (int)(r % Tk), hk = (int)((r / Tk) % Hkv), b = (int)(r / ((long)Tk * Hkv));
        const double* kj = kvrow(k, &s, b, hk, j);
        const double* vj = kvrow(v, &s, b, hk, j);
        double* dk_j = dk + (size_t)r * D;
        double* dv_j = dv + (size_t)r * D;
        double* dkm_j = dk_mag ? dk_mag + (size_t)r * D : NULL;
        double* dvm_j = dv_mag ? dv_mag + (size_t)r * D : NULL;
        for (int d = 0; d < D; ++d) dk_j[d] = dv_j[d] = 0.0;
        if (dkm_j)
            for (int d = 0; d < D; ++d) dkm_j[d] = 0.0;
        if (dvm_j)
            for (int d = 0; d < D; ++d) dvm_j[d] = 0.0;
        for (int g = 0; g < G; ++g) {
            const int h = hk * G + g;
            for (int i = 0; i < Tq; ++i) {
                if (!visible(&s, i, j)) continue;
                const long qr = ((long)b * Hq + h) * Tq + i;
                if (mst[qr] == -INFINITY) continue;
                const double* q_i = qrow(q, &s, b, h, i);
                const double* do_i = qrow(dout, &s, b, h, i);
                const double sij = scale * dot(q_i, kj, D);
                const double pij = exp(sij - mst[qr]) / lst[qr];
                const double dpij = dot(do_i, vj, D);
                const double ds = pij * (dpij - cst[qr]);
                for (int d = 0; d < D; ++d) {
                    dk_j[d] += ds * q_i[d];
                    dv_j[d] += pij * do_i[d];
                }
                if (dkm_j)
                    for (int d = 0; d < D; ++d) dkm_j[d] += fabs(ds * q_i[d]);
                if (dvm_j)
                    for (int d = 0; d < D; ++d) dvm_j[d] += fabs(pij * do_i[d]);
            }
        }
        for (int d = 0; d < D; ++d) dk_j[d] *= scale;
        if (dkm_j)
            for (int d = 0; d < D; ++d) dkm_j[d] *= fabs(scale);
    }
    if (jac) memcpy(jac, cst, sizeof(double) * (size_t)qrows);

    free(mst);
    free(lst);
    free(cst);
    free(scr);
    return ORACLE_OK;
}

static int check_rows(const int64_t* idx, long n, int n0, int n1, int n2)
{
    for (long r = 0; r < n; ++r)
        if (idx[3 * r] < 0 || idx[3 * r] >= n0 || idx[3 * r + 1] < 0 || idx[3 * r + 1] >= n1 ||
            idx[3 * r + 2] < 0 || idx[3 * r + 2] >= n2)
            return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

/*
 * Sampled forward: for each n, idx[3n..3n+2] = (b, h, i) names a query row;
 * o_rows[n*D..] and lse_rows[n] receive its output.  Costs O(T*D) per row, so
 * single rows of very long sequences can be checked.
 */
int oracle_fwd_rows(const double* q, const double* k, const double* v, const int64_t* idx, long n,
                    double* o_rows, double* lse_rows, int B, int Hq, int Hkv, int Tq, int Tk,
                    int D, double scale, int causal, int off)
{
    shape_t s = {B, Hq, Hkv, Tq, Tk, D, scale, causal, off};
    if (check_shape(&s) != ORACLE_OK || check_rows(idx, n, B, Hq, Tq) != ORACLE_OK)
        return ORACLE_ERR_ARG;
    double* scr = scratch_alloc(2, Tk);
    if (!scr) return ORACLE_ERR_NOMEM;
#pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < n; ++r)
        fwd_one_row(&s, q, k, v, (int)idx[3 * r], (int)idx[3 * r + 1], (int)idx[3 * r + 2],
                    o_rows + (size_t)r * D, lse_rows + r, NULL, scratch_of(scr, 2, Tk, 0),
                    scratch_of(scr, 2, Tk, 1));
    free(scr);
    return ORACLE_OK;
}

/* Sampled dq: idx holds (b, h, i) triples as in oracle_fwd_rows. */
int oracle_dq_rows(const double* q, const double* k, const double* v, const double* dout,
                   const int64_t* idx, long n, double* dq_rows, int B, int Hq, int Hkv, int Tq,
                   int Tk, int D, double scale, int causal, int off)
{
    shape_t s = {B, Hq, Hkv, Tq, Tk, D, scale, causal, off};
    if (check_shape(&s) != ORACLE_OK || check_rows(idx, n, B, Hq, Tq) != ORACLE_OK)
        return ORACLE_ERR_ARG;
    const int G = Hq / Hkv;
    double* scr = scratch_alloc(3, Tk);
    if (!scr) return ORACLE_ERR_NOMEM;
#pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < n; ++r) {
        const int b = (int)idx[3 * r], h = (int)idx[3 * r + 1], i = (int)idx[3 * r + 2];
        const int hk = h / G;
        double* p = scratch_of(scr, 3, Tk, 1);
        double* dp = scratch_of(scr, 3, Tk, 2);
        double m, l;
        const double c =
            bwd_row_terms(&s, q, k, v, dout, b, h, i, scratch_of(scr, 3, Tk, 0), p, dp, &m, &l);
        double* dq_i = dq_rows + (size_t)r * D;
        for (int d = 0; d < D; ++d) dq_i[d] = 0.0;
        for (int j = 0; j < Tk; ++j) {
            if (!visible(&s, i, j) || m == -INFINITY) continue;
            const double ds = p[j] * (dp[j] - c);
            const double* kj = kvrow(k, &s, b, hk, j);
            for (int d = 0; d < D; ++d) dq_i[d] += ds * kj[d];
        }
        for (int d = 0; d < D; ++d) dq_i[d] *= scale;
    }
    free(scr);
    return ORACLE_OK;
}

/*
 * Sampled dk/dv: idx holds (b, hk, j) triples naming key rows of a kv head.
 * Every query row that sees key j, of every query head of the group, is
 * rebuilt in full (its softmax needs the whole row), so a key near the end of
 * a causal sequence is cheap and key 0 costs a whole head.  The query rows of
 * one key are spread over the threads and their terms summed afterwards in
 * ascending (h, i) order.
 */
int oracle_dkdv_rows(const double* q, const double* k, const double* v, const double* dout,
                     const int64_t* idx, long n, double* dk_rows, double* dv_rows, int B, int Hq,
                     int Hkv, int Tq, int Tk, int D, double scale, int causal, int off)
{
    shape_t s = {B, Hq, Hkv, Tq, Tk, D, scale, causal, off};
    if (check_shape(&s) != ORACLE_OK || check_rows(idx, n, B, Hkv, Tk) != ORACLE_OK)
        return ORACLE_ERR_ARG;
    const int G = Hq / Hkv;
    double* scr = scratch_alloc(3, Tk);
    /* per (h, i) of one key: dS_ij and P_ij */
    double* dsv = (double*)malloc(sizeof(double) * (size_t)G * (size_t)(Tq > 0 ? Tq : 1));
    double* pv = (double*)malloc(sizeof(double) * (size_t)G * (size_t)(Tq > 0 ? Tq : 1));
    if (!scr || !dsv || !pv) {
        free(scr);
        free(dsv);
        free(pv);
        return ORACLE_ERR_NOMEM;
    }
    for (long r = 0; r < n; ++r) {
        const int b = (int)idx[3 * r], hk = (int)idx[3 * r + 1], j = (int)idx[3 * r + 2];
#pragma omp parallel for schedule(dynamic, 4)
        for (long gi = 0; gi < (long)G * Tq; ++gi) {
            const int g = (int)(gi / Tq), i = (int)(gi % Tq);
            if (!visible(&s, i, j)) {
                dsv[gi] = pv[gi] = 0.0;
                continue;
            }
            double* p = scratch_of(scr, 3, Tk, 1);
            double* dp = scratch_of(scr, 3, Tk, 2);
            double m, l;
            const double c = bwd_row_terms(&s, q, k, v, dout, b, hk * G + g, i,
                                           scratch_of(scr, 3, Tk, 0), p, dp, &m, &l);
            pv[gi] = p[j];
            dsv[gi] = p[j] * (dp[j] - c);
        }
        double* dk_j = dk_rows + (size_t)r * D;
        double* dv_j = dv_rows + (size_t)r * D;
        for (int d = 0; d < D; ++d) dk_j[d] = dv_j[d] = 0.0;
        for (int g = 0; g < G; ++g)
            for (int i = 0; i < Tq; ++i) {
                if (!visible(&s, i, j)) continue;
                const double* q_i = qrow(q, &s, b, hk * G + g, i);
                const double* do_i = qrow(dout, &s, b, hk * G + g, i);
                const long gi = (long)g * Tq + i;
                for (int d = 0; d < D; ++d) {
                    dk_j[d] += dsv[gi] * q_i[d];
                    dv_j[d] += pv[gi] * do_i[d];
                }
            }
        for (int d = 0; d < D; ++d) dk_j[d] *= scale;
    }
    free(scr);
    free(dsv);
    free(pv);
    return ORACLE_OK;
}

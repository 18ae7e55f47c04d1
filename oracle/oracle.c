/*
 * oracle.c -- the reference CPU attention used ONLY as test infrastructure.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * this library.  The product path (the HIP library and its Python binding)
 * never calls it and shares no code, header or constant with it.
 *
 * What it computes is the plain definition of masked softmax attention, in
 * fp64, with an explicit boolean mask per query row and a two-pass softmax
 * (pass 1: the row maximum, pass 2: exponentials and their sum).  There is no
 * tiling, no online rescaling and no fusion: the flash-style method on the
 * pages reaches this same result up to rounding order.
 *
 * Passages followed (page titles as published):
 *  - "[CUDA] Use Triton TMA for long-context causal prefill", Summary: global
 *    causal attention; fully masked rows give finite output (here: exactly 0);
 *    the softmax uses the exact row maximum, no fixed offset.
 *  - same page, Test plan: a dense-mask reference is the correctness yardstick.
 *  - "[executorch][cuda] Add a length-aware Triton SDPA over per-sequence KV
 *    columns", description: the [rows, cols, H, D] column store, the segment
 *    table seq_info = (q_start, q_len, col, kv_end), causal / non-causal /
 *    sliding-window / ring modes, GQA, and zeroed rows that no segment covers.
 *  - same page, stacked commit adding the batched-sequence manifest layout:
 *    a key at position k lives in store row (k mod rows) of its column.
 *  - same page, stacked commit adding the batched sequence cache: a ring layer
 *    holds window + max_write - 1 rows, which fixes the window convention
 *    used here: a query at position p sees keys p-W < k <= p (W keys).
 *
 * Readings where the pages are silent:
 *  - GQA: query head h reads KV head floor(h / (Hq/Hkv)).
 *  - Prefill causality is end-aligned through q_pos0: query row i sits at
 *    absolute position q_pos0 + i and sees keys j <= q_pos0 + i.
 *  - A row whose visible set is empty returns exactly 0 in every element.
 *  - Varlen: query j of a segment sits at position kv_end - q_len + j
 *    (kv_end already counts the step's own tokens).
 *  - Varlen with a window on a non-causal segment: only the lower bound
 *    k > p - W applies.
 *  - Varlen on ring storage: a segment whose visible keys start before
 *    kv_end - R (positions the ring has overwritten) is flagged and skipped.
 *
 * Numbers: bf16 inputs are widened exactly to double; every product, sum and
 * exponential is double precision (libm exp).  Results are double.
 *
 * Parity pins: every function here is pinned by tests that do not re-type
 * its formula (closed forms, invariants, brute force by another route,
 * torch's float64 SDPA with an explicit mask).  Nothing here is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_INVALID 1

/* varlen segment flags (the same bit meanings as the library's error word) */
#define SEGF_QRANGE 1   /* q_start < 0, q_len < 0 or q_start + q_len > T   */
#define SEGF_COL 2      /* col outside [0, cols-1): the last column is scratch */
#define SEGF_KVEND 4    /* kv_end < 0, or kv_end > rows on flat storage     */
#define SEGF_ATTR 8     /* seg_attr ring_rows > rows                         */
#define SEGF_OVERLAP 16 /* a packed row is claimed by two valid segments     */
#define SEGF_SPAN 32    /* ring storage: the visible keys reach back past the
                           R positions the ring still holds                   */

static double widen_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Softmax attention of one query row over n candidate keys.
 *   qrow  : D query values (already widened)
 *   krow/vrow : n pointers to bf16 key / value rows (element stride 1)
 *   mask  : n booleans, 1 = the key is visible to this query
 *   s     : scratch of n doubles
 *   out   : D doubles written
 *   probs : nullable, n doubles: the softmax weight of each candidate
 * An empty visible set writes zeros (and zero weights).
 */
static void attend_row(const double *qrow, int D, int n,
                       const uint16_t *const *krow, const uint16_t *const *vrow,
                       const unsigned char *mask, double scale, double *s,
                       double *out, double *probs)
{
    int any = 0;
    double m = 0.0;
    for (int d = 0; d < D; d++)
        out[d] = 0.0;
    /* scores of visible keys, and pass 1: their maximum */
    for (int j = 0; j < n; j++) {
        if (!mask[j])
            continue;
        double dot = 0.0;
        for (int d = 0; d < D; d++)
            dot += qrow[d] * widen_bf16(krow[j][d]);
        s[j] = scale * dot;
        if (!any || s[j] > m)
            m = s[j];
        any = 1;
    }
    if (probs)
        for (int j = 0; j < n; j++)
            probs[j] = 0.0;
    if (!any)
        return;
    /* pass 2: exponentials relative to the maximum, and their sum */
    double l = 0.0;
    for (int j = 0; j < n; j++) {
        if (!mask[j])
            continue;
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    /* weighted sum of the visible values */
    for (int j = 0; j < n; j++) {
        if (!mask[j])
            continue;
        double w = s[j] / l;
        if (probs)
            probs[j] = w;
        for (int d = 0; d < D; d++)
            out[d] += w * widen_bf16(vrow[j][d]);
    }
}

/*
 * Causal GQA prefill.
 *   q [B,Hq,Lq,D], k/v [B,Hkv,Lkv,D]: bf16 bits, strides in elements
 *   (the innermost stride is the fourth entry and may be anything here).
 *   Query row i sits at position q_pos0 + i and sees key j iff
 *   0 <= j < Lkv, j <= q_pos0 + i and (window <= 0 or j > q_pos0 + i - window).
 *   row_sel / n_sel: the query rows to compute (NULL: all Lq rows).
 *   out [B,Hq,n_sel,D] doubles, contiguous.
 *   probs (nullable) [B,Hq,n_sel,Lkv] doubles: the softmax weights.
 */
int oracle_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   double *out, int B, int Hq, int Hkv, int Lq, int Lkv, int D,
                   double scale, const int64_t *q_str, const int64_t *k_str,
                   const int64_t *v_str, int64_t q_pos0, int window,
                   const int32_t *row_sel, int n_sel, double *probs)
{
    if (!q || !k || !v || !out || !q_str || !k_str || !v_str)
        return ORACLE_INVALID;
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || Lq < 0 || Lkv < 0)
        return ORACLE_INVALID;
    if (Hq % Hkv != 0)
        return ORACLE_INVALID;
    if (!row_sel)
        n_sel = Lq;
    if (n_sel < 0)
        return ORACLE_INVALID;
    for (int r = 0; row_sel && r < n_sel; r++)
        if (row_sel[r] < 0 || row_sel[r] >= Lq)
            return ORACLE_INVALID;
    const int g = Hq / Hkv;
    const long total = (long)B * Hq * n_sel;
    int status = ORACLE_OK;

#pragma omp parallel
    {
        int n = Lkv > 0 ? Lkv : 1;
        double *qrow = malloc(sizeof(double) * D);
        double *s = malloc(sizeof(double) * n);
        unsigned char *mask = malloc(n);
        const uint16_t **krow = malloc(sizeof(uint16_t *) * n);
        const uint16_t **vrow = malloc(sizeof(uint16_t *) * n);
        if (!qrow || !s || !mask || !krow || !vrow) {
#pragma omp atomic write
            status = ORACLE_INVALID;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long idx = 0; idx < total; idx++) {
                int r = (int)(idx % n_sel);
                int h = (int)((idx / n_sel) % Hq);
                int b = (int)(idx / ((long)n_sel * Hq));
                int i = row_sel ? row_sel[r] : r;
                int hk = h / g;
                int64_t p = q_pos0 + i;
                const uint16_t *qp = q + b * q_str[0] + h * q_str[1] + i * q_str[2];
                for (int d = 0; d < D; d++)
                    qrow[d] = widen_bf16(qp[d * q_str[3]]);
                /* the explicit mask row and the key/value rows it refers to */
                for (int j = 0; j < Lkv; j++) {
                    mask[j] = (j <= p) && (window <= 0 || j > p - window);
                    krow[j] = k + b * k_str[0] + hk * k_str[1] + j * k_str[2];
                    vrow[j] = v + b * v_str[0] + hk * v_str[1] + j * v_str[2];
                }
                /* attend_row reads rows with unit stride; gather otherwise */
                double *o = out + idx * D;
                if (k_str[3] == 1 && v_str[3] == 1) {
                    attend_row(qrow, D, Lkv, krow, vrow, mask, scale, s, o,
                               probs ? probs + idx * (long)Lkv : NULL);
                } else {
                    /* rare: non-unit inner stride; copy visible rows densely */
                    uint16_t *kc = malloc(sizeof(uint16_t) * (size_t)n * D);
                    uint16_t *vc = malloc(sizeof(uint16_t) * (size_t)n * D);
                    for (int j = 0; j < Lkv; j++) {
                        for (int d = 0; d < D; d++) {
                            kc[(size_t)j * D + d] = krow[j][d * k_str[3]];
                            vc[(size_t)j * D + d] = vrow[j][d * v_str[3]];
                        }
                        krow[j] = kc + (size_t)j * D;
                        vrow[j] = vc + (size_t)j * D;
                    }
                    attend_row(qrow, D, Lkv, krow, vrow, mask, scale, s, o,
                               probs ? probs + idx * (long)Lkv : NULL);
                    free(kc);
                    free(vc);
                }
            }
        }
        free(qrow);
        free(s);
        free(mask);
        free(krow);
        free(vrow);
    }
    return status;
}

/*
 * Segment checks shared by the varlen oracle's passes.  R is the key-position
 * modulus of the segment (its ring rows, or all rows for flat storage).
 *
 * A ring of R rows, written in position order up to kv_end, still holds
 * positions kv_end - R .. kv_end - 1 only: every older position's row has
 * been overwritten by a newer one (the batched sequence cache sizes a ring
 * layer as window + max_write - 1 rows for exactly this reason).  The
 * earliest key any query of the segment sees is that of its first query,
 * max(0, kv_end - q_len - W + 1) with a window, 0 without; a ring segment
 * whose visible keys start before kv_end - R would read overwritten rows,
 * so it is flagged (SEGF_SPAN) and not attended.
 */
static int segment_flags(const int32_t *si, const int32_t *attr, int T, int rows,
                         int cols, int ring_rows_default, int window_default,
                         int *R_out)
{
    int flags = 0;
    int q_start = si[0], q_len = si[1], col = si[2], kv_end = si[3];
    int ring_rows = attr ? attr[2] : ring_rows_default;
    int W = attr ? attr[1] : window_default;
    if (q_start < 0 || q_len < 0 || (int64_t)q_start + q_len > T)
        flags |= SEGF_QRANGE;
    if (col < 0 || col >= cols - 1)
        flags |= SEGF_COL;
    if (ring_rows > rows)
        flags |= SEGF_ATTR;
    int ring = ring_rows > 0;
    int R = ring ? ring_rows : rows;
    if (kv_end < 0 || (!ring && kv_end > rows))
        flags |= SEGF_KVEND;
    if (ring && q_len > 0 && kv_end > 0) {
        int64_t first = W > 0 ? (int64_t)kv_end - q_len - W + 1 : 0;
        if (first < 0)
            first = 0;
        if ((int64_t)kv_end - first > R)
            flags |= SEGF_SPAN;
    }
    *R_out = R;
    return flags;
}

/*
 * Varlen SDPA over a column store.
 *   q [T,Hq,D] bf16 bits with strides q_str[3];
 *   k/v store [rows, cols, Hkv, D] with strides k_str[4] / v_str[4];
 *   seq_info [S,4] = (q_start, q_len, col, kv_end), host memory;
 *   seg_attr nullable [S,3] = (causal, window, ring_rows); when NULL every
 *   segment takes (causal, window, ring_rows) from the call.
 *   ring_rows <= 0 means flat storage (modulus = rows).
 *   out [T,Hq,D] doubles, contiguous.  err_out receives the OR of segment
 *   flags.  A segment with any flag is not attended; packed rows that no
 *   valid segment covers are 0.  Overlapping valid segments return
 *   ORACLE_INVALID (the result is not defined).
 */
int oracle_varlen(const uint16_t *q, const uint16_t *ks, const uint16_t *vs,
                  double *out, const int32_t *seq_info, int S,
                  const int32_t *seg_attr, int T, int Hq, int Hkv, int D,
                  int rows, int cols, double scale, int causal, int window,
                  int ring_rows, const int64_t *q_str, const int64_t *k_str,
                  const int64_t *v_str, int32_t *err_out)
{
    if (!q || !ks || !vs || !out || !q_str || !k_str || !v_str || !err_out)
        return ORACLE_INVALID;
    if (S < 0 || T < 0 || Hq < 1 || Hkv < 1 || D < 1 || rows < 1 || cols < 2)
        return ORACLE_INVALID;
    if (S > 0 && !seq_info)
        return ORACLE_INVALID;
    if (Hq % Hkv != 0 || S > 2 * (cols - 1))
        return ORACLE_INVALID;
    if (!seg_attr && (ring_rows > rows || (!causal && window > 0)))
        return ORACLE_INVALID;
    const int g = Hq / Hkv;
    int32_t err = 0;

    /* which valid segment owns each packed row (-1: none) */
    int *owner = malloc(sizeof(int) * (T > 0 ? T : 1));
    int *seg_ok = malloc(sizeof(int) * (S > 0 ? S : 1));
    if (!owner || !seg_ok) {
        free(owner);
        free(seg_ok);
        return ORACLE_INVALID;
    }
    for (int t = 0; t < T; t++)
        owner[t] = -1;
    int overlap = 0;
    for (int s = 0; s < S; s++) {
        int R;
        int f = segment_flags(seq_info + 4 * s, seg_attr ? seg_attr + 3 * s : NULL,
                              T, rows, cols, ring_rows, window, &R);
        err |= f;
        seg_ok[s] = (f == 0);
        if (!seg_ok[s])
            continue;
        for (int j = 0; j < seq_info[4 * s + 1]; j++) {
            int t = seq_info[4 * s] + j;
            if (owner[t] >= 0)
                overlap = 1;
            owner[t] = s;
        }
    }
    *err_out = err | (overlap ? SEGF_OVERLAP : 0);
    if (overlap) {
        free(owner);
        free(seg_ok);
        return ORACLE_INVALID;
    }

    for (long x = 0; x < (long)T * Hq * D; x++)
        out[x] = 0.0;

    const long total = (long)T * Hq;
#pragma omp parallel
    {
        int nmax = rows > 0 ? rows : 1;
        /* the largest candidate set is a segment's kv_end keys */
        for (int s = 0; s < S; s++)
            if (seg_ok[s] && seq_info[4 * s + 3] > nmax)
                nmax = seq_info[4 * s + 3];
        double *qrow = malloc(sizeof(double) * D);
        double *sc = malloc(sizeof(double) * nmax);
        unsigned char *mask = malloc(nmax);
        const uint16_t **krow = malloc(sizeof(uint16_t *) * nmax);
        const uint16_t **vrow = malloc(sizeof(uint16_t *) * nmax);
        uint16_t *kc = NULL, *vc = NULL;
        if (k_str[3] != 1 || v_str[3] != 1) {
            kc = malloc(sizeof(uint16_t) * (size_t)nmax * D);
            vc = malloc(sizeof(uint16_t) * (size_t)nmax * D);
        }
#pragma omp for schedule(dynamic, 1)
        for (long idx = 0; idx < total; idx++) {
            int t = (int)(idx / Hq);
            int h = (int)(idx % Hq);
            int s = owner[t];
            if (s < 0)
                continue; /* uncovered: stays 0 */
            const int32_t *si = seq_info + 4 * s;
            int q_start = si[0], q_len = si[1], col = si[2], kv_end = si[3];
            int c = seg_attr ? seg_attr[3 * s + 0] : causal;
            int W = seg_attr ? seg_attr[3 * s + 1] : window;
            int R;
            segment_flags(si, seg_attr ? seg_attr + 3 * s : NULL, T, rows, cols,
                          ring_rows, window, &R);
            int j = t - q_start;
            int64_t p = (int64_t)kv_end - q_len + j;
            int hk = h / g;
            const uint16_t *qp = q + t * q_str[0] + h * q_str[1];
            for (int d = 0; d < D; d++)
                qrow[d] = widen_bf16(qp[d * q_str[2]]);
            for (int key = 0; key < kv_end; key++) {
                mask[key] = (!c || key <= p) && (W <= 0 || key > p - W);
                int64_t r = key % R; /* store row of this key position */
                krow[key] = ks + r * k_str[0] + col * k_str[1] + hk * k_str[2];
                vrow[key] = vs + r * v_str[0] + col * v_str[1] + hk * v_str[2];
                if (kc) {
                    for (int d = 0; d < D; d++) {
                        kc[(size_t)key * D + d] = krow[key][d * k_str[3]];
                        vc[(size_t)key * D + d] = vrow[key][d * v_str[3]];
                    }
                    krow[key] = kc + (size_t)key * D;
                    vrow[key] = vc + (size_t)key * D;
                }
            }
            attend_row(qrow, D, kv_end, krow, vrow, mask, scale, sc,
                       out + idx * D, NULL);
        }
        free(qrow);
        free(sc);
        free(mask);
        free(krow);
        free(vrow);
        free(kc);
        free(vc);
    }
    free(owner);
    free(seg_ok);
    return ORACLE_OK;
}

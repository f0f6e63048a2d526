/*
 * CPU oracle for CSR sparse x dense products with sum / mean / max+argmax
 * reductions (GNN neighbour aggregation).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference: it is
 * built and called by the test suite, by the package smoke check and by the
 * benchmark's CPU-baseline leg, never by the product path.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * Plain, slow, single-threaded, fp32 as the pages fix ("fp32 only", "fp32
 * summation order": graph-spmm kernel card, sections "Requirements and
 * limits" and "Correctness").  Build with -O2 -ffp-contract=off so that the
 * compiler never fuses a multiply into an add unless asked to (fused = 1).
 *
 * Definitions followed (sources are the pages' titles and sections):
 *  - CSR: row i owns entries rowPtr[i] .. rowPtr[i+1]-1 (ParamSpMM, section 2
 *    "Background", CSR format).
 *  - sum: C[i][k] accumulates a_p * B[col_p][k] over the row's entries in
 *    stored order, writing C once at the end (ParamSpMM section 2, Algorithm 1;
 *    GE-SpMM section III-A).
 *  - mean: row-wise mean, empty rows give 0 (graph-spmm card, API table:
 *    spmm_mean).  The divisor is the number of stored entries of the row.
 *  - max: (values, argmax) with the winning neighbour's column id; empty rows
 *    give (0, -1) (graph-spmm card, API table: spmm_max, and "Method").  Ties go
 *    to the first entry in stored order (strict greater-than).
 *  - val == NULL: every stored entry is 1 and no value is read (graph-spmm card,
 *    API table: spmm_sum with val=None; "Method").
 *  - duplicates are not merged: each stored entry counts (graph-spmm card,
 *    "Correctness").
 *  - descriptors: M, mean degree nnz/M and the coefficient of variation of the
 *    row degree (RA-SpMM, abstract and "Structural taxonomy").
 *  - row split: rows longer than a threshold are cut into fixed-length pieces
 *    processed separately (ParamSpMM section 3.2 "workload balancing", PCSR
 *    TRow in section 4.2; graph-spmm card, "Requirements and limits").
 *  - MAC-job gap of thread coarsening (ParamSpMM section 3.3, eq. 1, read with
 *    Table 2: the gap is zero when dim is a multiple of F * omega).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define RED_SUM 0
#define RED_MEAN 1
#define RED_MAX 2

/* One product a_p * b: a single fp32 rounding, or none of its own when fused. */
static float product(const float *val, int64_t p, float b) {
    if (val == NULL) return b;
    return val[p] * b;
}

/*
 * C[r][k] for r over `rows` (all rows when rows == NULL), k in [0, N).
 * C (and argmax, for max) are [nrows, N] row-major, one row per listed row.
 * fused = 0: acc = acc + (a*b), two roundings per entry (the plain definition).
 * fused = 1: acc = fmaf(a, b, acc), one rounding per entry.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_spmm(const int64_t *rowptr, const int64_t *col, const float *val,
                int64_t M, int64_t K, const float *B, int64_t N, int reduce,
                int fused, const int64_t *rows, int64_t nrows, float *C,
                int64_t *argmax) {
    if (M < 0 || K < 0 || N <= 0 || reduce < RED_SUM || reduce > RED_MAX)
        return -1;
    if (rows == NULL) nrows = M;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        if (i < 0 || i >= M) return -1;
        int64_t first = rowptr[i];
        int64_t last = rowptr[i + 1];
        int64_t deg = last - first;
        for (int64_t k = 0; k < N; ++k) {
            float out;
            int64_t arg = -1;
            if (reduce == RED_MAX) {
                if (deg == 0) {
                    out = 0.0f;
                } else {
                    float best = product(val, first, B[col[first] * N + k]);
                    arg = col[first];
                    for (int64_t p = first + 1; p < last; ++p) {
                        float t = product(val, p, B[col[p] * N + k]);
                        if (t > best) {
                            best = t;
                            arg = col[p];
                        }
                    }
                    out = best;
                }
                argmax[r * N + k] = arg;
            } else {
                float acc = 0.0f;
                for (int64_t p = first; p < last; ++p) {
                    float b = B[col[p] * N + k];
                    if (fused && val != NULL)
                        acc = fmaf(val[p], b, acc);
                    else
                        acc = acc + product(val, p, b);
                }
                if (reduce == RED_MEAN)
                    out = (deg == 0) ? 0.0f : acc / (float)deg;
                else
                    out = acc;
            }
            C[r * N + k] = out;
        }
    }
    return 0;
}

/* S[r][k] = sum over the row's entries of |a_p * B[col_p][k]|, in double. */
int oracle_sumabs(const int64_t *rowptr, const int64_t *col, const float *val,
                  int64_t M, const float *B, int64_t N, const int64_t *rows,
                  int64_t nrows, double *S) {
    if (M < 0 || N <= 0) return -1;
    if (rows == NULL) nrows = M;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        if (i < 0 || i >= M) return -1;
        for (int64_t k = 0; k < N; ++k) {
            double s = 0.0;
            for (int64_t p = rowptr[i]; p < rowptr[i + 1]; ++p) {
                double a = val ? (double)val[p] : 1.0;
                s += fabs(a * (double)B[col[p] * N + k]);
            }
            S[r * N + k] = s;
        }
    }
    return 0;
}

/*
 * CSR well-formedness: rowptr[0] == 0, rowptr non-decreasing, every column in
 * [0, K).  Returns -1 when valid, else the first row that breaks a rule
 * (row i for a decrease rowptr[i+1] < rowptr[i] or a bad column in row i;
 * row 0 when rowptr[0] != 0).
 */
int64_t oracle_validate(const int64_t *rowptr, const int64_t *col, int64_t M,
                        int64_t K) {
    if (rowptr[0] != 0) return 0;
    for (int64_t i = 0; i < M; ++i)
        if (rowptr[i + 1] < rowptr[i]) return i;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t p = rowptr[i]; p < rowptr[i + 1]; ++p)
            if (col[p] < 0 || col[p] >= K) return i;
    return -1;
}

/*
 * Row-degree descriptors.  ints = {nnz, dmax, n_empty}; dbl = {mean, cv}
 * with mean = nnz / M and cv = population standard deviation / mean
 * (two-pass: mean first, then the mean squared deviation).  M == 0 or a zero
 * mean gives cv = 0.
 */
void oracle_descriptors(const int64_t *rowptr, int64_t M, int64_t *ints,
                        double *dbl) {
    int64_t nnz = 0, dmax = 0, n_empty = 0;
    for (int64_t i = 0; i < M; ++i) {
        int64_t d = rowptr[i + 1] - rowptr[i];
        nnz += d;
        if (d > dmax) dmax = d;
        if (d == 0) n_empty += 1;
    }
    double mean = (M > 0) ? (double)nnz / (double)M : 0.0;
    double var = 0.0;
    for (int64_t i = 0; i < M; ++i) {
        double dev = (double)(rowptr[i + 1] - rowptr[i]) - mean;
        var += dev * dev;
    }
    var = (M > 0) ? var / (double)M : 0.0;
    ints[0] = nnz;
    ints[1] = dmax;
    ints[2] = n_empty;
    dbl[0] = mean;
    dbl[1] = (mean > 0.0) ? sqrt(var) / mean : 0.0;
}

/*
 * Row split.  Heavy rows are those with degree > T, taken in ascending order;
 * heavy row i is cut into pieces [rowptr[i] + s*L, min(rowptr[i] + (s+1)*L,
 * rowptr[i+1])) for s = 0, 1, ...  Pieces are listed by (row, s).  Every other
 * row is light, listed in ascending order.  Writes at most `cap` pieces and
 * `light_cap` light rows; counts = {n_heavy, n_pieces, n_light}.
 * Returns 0, or -1 for T < 0 or L <= 0.
 */
int oracle_partition(const int64_t *rowptr, int64_t M, int64_t T, int64_t L,
                     int64_t *seg_row, int64_t *seg_begin, int64_t *seg_end,
                     int64_t cap, int64_t *light, int64_t light_cap,
                     int64_t *counts) {
    if (T < 0 || L <= 0) return -1;
    int64_t n_heavy = 0, n_seg = 0, n_light = 0;
    for (int64_t i = 0; i < M; ++i) {
        int64_t deg = rowptr[i + 1] - rowptr[i];
        if (deg > T) {
            n_heavy += 1;
            for (int64_t b = rowptr[i]; b < rowptr[i + 1]; b += L) {
                int64_t e = b + L;
                if (e > rowptr[i + 1]) e = rowptr[i + 1];
                if (n_seg < cap) {
                    seg_row[n_seg] = i;
                    seg_begin[n_seg] = b;
                    seg_end[n_seg] = e;
                }
                n_seg += 1;
            }
        } else {
            if (n_light < light_cap) light[n_light] = i;
            n_light += 1;
        }
    }
    counts[0] = n_heavy;
    counts[1] = n_seg;
    counts[2] = n_light;
    return 0;
}

/*
 * MAC-job gap of a warp that produces F*omega columns per pass over a row,
 * for a dense width dim: the ideal job count min(dim, F*omega) minus the
 * residual warp's job count dim mod (F*omega), taken as 0 when the residual is
 * 0 (no residual warp).
 */
int64_t oracle_mac_gap(int64_t dim, int64_t F, int64_t omega) {
    int64_t span = F * omega;
    int64_t tn = dim < span ? dim : span;
    int64_t tr = dim % span;
    if (tr == 0) return 0;
    return tn - tr;
}

/*
 * Backward pieces and graph construction (graph-spmm kernel card: API table
 * row SparseAdj.from_edge_index; "Requirements and limits": the card is forward
 * only and points to the reversed-edge adjacency A^T for a sum's gradient;
 * "Method": the forward max reports its winning neighbour, which routes the
 * max's gradient).
 */

/*
 * Edge list -> CSR.  Edge e is entry (row[e], col[e]) with value val[e] (or
 * none).  Rows are grouped in ascending order and, within a row, entries keep
 * the order of the edge list (a stable sort by row).  rowptr_out [M+1],
 * col_out [E], val_out [E] (when val != NULL).  Returns -1 when valid, else
 * the first edge whose row is outside [0, M) or column outside [0, K).
 */
int64_t oracle_coo_to_csr(const int64_t *row, const int64_t *col, const float *val,
                          int64_t E, int64_t M, int64_t K, int64_t *rowptr_out,
                          int64_t *col_out, float *val_out) {
    for (int64_t e = 0; e < E; ++e)
        if (row[e] < 0 || row[e] >= M || col[e] < 0 || col[e] >= K) return e;
    for (int64_t i = 0; i <= M; ++i) rowptr_out[i] = 0;
    for (int64_t e = 0; e < E; ++e) rowptr_out[row[e] + 1] += 1;
    for (int64_t i = 0; i < M; ++i) rowptr_out[i + 1] += rowptr_out[i];
    /* place edges in edge order: a running cursor per row keeps them stable */
    int64_t *cursor = (int64_t *)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
    if (!cursor) return -2;
    for (int64_t i = 0; i < M; ++i) cursor[i] = rowptr_out[i];
    for (int64_t e = 0; e < E; ++e) {
        int64_t p = cursor[row[e]]++;
        col_out[p] = col[e];
        if (val) val_out[p] = val[e];
    }
    free(cursor);
    return -1;
}

/*
 * CSR of A [M, K] -> CSR of its transpose [K, M]: entry (i, j, a) of A becomes
 * entry (j, i, a') of the transpose, listed in A's stored order within each
 * transposed row (so rows i ascend).  scale = 0: a' = a (1 when unweighted);
 * scale = 1: a' = a / deg_i in fp32, one division (the mean's backward).
 * rowptr_t [K+1], col_t [nnz], val_t [nnz] (always written).
 */
void oracle_transpose(const int64_t *rowptr, const int64_t *col, const float *val,
                      int64_t M, int64_t K, int scale, int64_t *rowptr_t,
                      int64_t *col_t, float *val_t) {
    for (int64_t j = 0; j <= K; ++j) rowptr_t[j] = 0;
    for (int64_t p = 0; p < rowptr[M]; ++p) rowptr_t[col[p] + 1] += 1;
    for (int64_t j = 0; j < K; ++j) rowptr_t[j + 1] += rowptr_t[j];
    int64_t *cursor = (int64_t *)malloc(sizeof(int64_t) * (size_t)(K > 0 ? K : 1));
    if (!cursor) return;
    for (int64_t j = 0; j < K; ++j) cursor[j] = rowptr_t[j];
    for (int64_t i = 0; i < M; ++i) {
        int64_t deg = rowptr[i + 1] - rowptr[i];
        for (int64_t p = rowptr[i]; p < rowptr[i + 1]; ++p) {
            int64_t q = cursor[col[p]]++;
            float a = val ? val[p] : 1.0f;
            col_t[q] = i;
            val_t[q] = scale ? a / (float)deg : a;
        }
    }
    free(cursor);
}

/*
 * Max-pool backward for an unweighted adjacency: dB[j][k] = sum over rows i
 * with argmax[i][k] == j of dC[i][k], summed in ascending i (fp32).  Rows with
 * argmax -1 (empty) contribute nothing.  dB is [K, N], fully written.
 * Returns 0, or -1 when an argmax entry is outside [-1, K).
 */
int oracle_max_backward(const int64_t *argmax, const float *dC, int64_t M, int64_t K,
                        int64_t N, float *dB) {
    for (int64_t x = 0; x < M * N; ++x)
        if (argmax[x] < -1 || argmax[x] >= K) return -1;
    for (int64_t x = 0; x < K * N; ++x) dB[x] = 0.0f;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < N; ++k) {
            int64_t j = argmax[i * N + k];
            if (j >= 0) dB[j * N + k] = dB[j * N + k] + dC[i * N + k];
        }
    return 0;
}

/*
 * Sparse-matrix features of ParamSpMM section 5.1, Table 3, for the CSR
 * matrix A [M, K] and a vectorized-blocking width V (section 3.1: V
 * consecutive rows form one block, rows V*g .. V*g+V-1).
 *   ints = {n, n_nonempty, nnz, dmax, max_bandwidth, nnz_distinct, nnz_vectors}
 *   dbl  = {delta, mean_deg, mean_deg_nonempty, cv_deg, cv_deg_nonempty,
 *           density, mean_bandwidth, padding_ratio}
 * delta = n_nonempty / n; the "hat" quantities ignore empty rows; cv is the
 * population standard deviation over the mean (two passes); density =
 * nnz / (M * K) with nnz the stored entry count.  Bandwidth of a row: its
 * largest minus its smallest column id (Table 3 footnote: the column distance
 * between the row's first and last nonzero, columns taken in ascending
 * order); averaged over non-empty rows.  nnz_distinct counts distinct
 * (row, col) pairs; a nonzero vector is a column with at least one entry in a
 * block, nnz_vectors counts them over all blocks, and the padding ratio is
 * eq. 2, 1 - nnz_distinct / (nnz_vectors * V) (0 when there are no entries).
 * Returns 0, or -1 for V < 1 or an allocation failure.
 */
static int cmp_i64(const void *a, const void *b) {
    const int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

static int64_t count_distinct(int64_t *buf, int64_t n) {
    if (n == 0) return 0;
    qsort(buf, (size_t)n, sizeof(int64_t), cmp_i64);
    int64_t d = 1;
    for (int64_t i = 1; i < n; ++i)
        if (buf[i] != buf[i - 1]) d += 1;
    return d;
}

int oracle_features(const int64_t *rowptr, const int64_t *col, int64_t M, int64_t K,
                    int64_t V, int64_t *ints, double *dbl) {
    if (V < 1) return -1;
    int64_t nnz = 0, dmax = 0, nonempty = 0, bwmax = 0;
    double bwsum = 0.0;
    int64_t longest = 0;
    for (int64_t i = 0; i < M; ++i) {
        int64_t d = rowptr[i + 1] - rowptr[i];
        nnz += d;
        if (d > dmax) dmax = d;
        if (d > 0) {
            nonempty += 1;
            int64_t lo = col[rowptr[i]], hi = col[rowptr[i]];
            for (int64_t p = rowptr[i]; p < rowptr[i + 1]; ++p) {
                if (col[p] < lo) lo = col[p];
                if (col[p] > hi) hi = col[p];
            }
            bwsum += (double)(hi - lo);
            if (hi - lo > bwmax) bwmax = hi - lo;
        }
    }
    /* degree moments, all rows and non-empty rows, two passes each */
    double mean = M > 0 ? (double)nnz / (double)M : 0.0;
    double mean_ne = nonempty > 0 ? (double)nnz / (double)nonempty : 0.0;
    double var = 0.0, var_ne = 0.0;
    for (int64_t i = 0; i < M; ++i) {
        double d = (double)(rowptr[i + 1] - rowptr[i]);
        var += (d - mean) * (d - mean);
        if (d > 0) var_ne += (d - mean_ne) * (d - mean_ne);
    }
    var = M > 0 ? var / (double)M : 0.0;
    var_ne = nonempty > 0 ? var_ne / (double)nonempty : 0.0;
    /* distinct (row, col) pairs, row by row; nonzero vectors, block by block */
    for (int64_t i = 0; i < M; ++i)
        if (rowptr[i + 1] - rowptr[i] > longest) longest = rowptr[i + 1] - rowptr[i];
    int64_t cap = longest * V > 0 ? longest * V : 1;
    int64_t *buf = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
    if (!buf) return -1;
    int64_t distinct = 0, vectors = 0;
    for (int64_t i = 0; i < M; ++i) {
        int64_t n = 0;
        for (int64_t p = rowptr[i]; p < rowptr[i + 1]; ++p) buf[n++] = col[p];
        distinct += count_distinct(buf, n);
    }
    for (int64_t g = 0; g * V < M; ++g) {
        int64_t n = 0;
        for (int64_t i = g * V; i < g * V + V && i < M; ++i)
            for (int64_t p = rowptr[i]; p < rowptr[i + 1]; ++p) buf[n++] = col[p];
        vectors += count_distinct(buf, n);
    }
    free(buf);
    ints[0] = M;
    ints[1] = nonempty;
    ints[2] = nnz;
    ints[3] = dmax;
    ints[4] = bwmax;
    ints[5] = distinct;
    ints[6] = vectors;
    dbl[0] = M > 0 ? (double)nonempty / (double)M : 0.0;
    dbl[1] = mean;
    dbl[2] = mean_ne;
    dbl[3] = mean > 0.0 ? sqrt(var) / mean : 0.0;
    dbl[4] = mean_ne > 0.0 ? sqrt(var_ne) / mean_ne : 0.0;
    dbl[5] = (M > 0 && K > 0) ? (double)nnz / ((double)M * (double)K) : 0.0;
    dbl[6] = nonempty > 0 ? bwsum / (double)nonempty : 0.0;
    dbl[7] = vectors > 0 ? 1.0 - (double)distinct / ((double)vectors * (double)V) : 0.0;
    return 0;
}

/*
 * Locality reordering.  Reverse Cuthill-McKee (Cuthill and McKee, 1969; the
 * reversal by George, 1971) of a square CSR matrix A [M, M], on the symmetric
 * pattern of A + A^T: the neighbours of a node are the distinct other nodes
 * it shares an entry with in either direction, its degree their count.
 * Cuthill-McKee order: take nodes in ascending (degree, id) order; each one
 * not yet placed starts a component; placing proceeds breadth-first, each
 * placed node appending its unplaced neighbours in ascending (degree, id)
 * order.  perm[i] = the node at position i of the reversed order.
 * Returns 0, or -1 on an allocation failure.
 */
static const int64_t *g_deg;
static int cmp_deg_id(const void *a, const void *b) {
    const int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    if (g_deg[x] != g_deg[y]) return (g_deg[x] > g_deg[y]) - (g_deg[x] < g_deg[y]);
    return (x > y) - (x < y);
}

int oracle_rcm(const int64_t *rowptr, const int64_t *col, int64_t M, int64_t *perm) {
    int64_t nnz = M > 0 ? rowptr[M] : 0;
    int64_t *cnt = (int64_t *)calloc((size_t)M + 1, sizeof(int64_t));
    int64_t *adj = (int64_t *)malloc(sizeof(int64_t) * (size_t)(2 * nnz + 1));
    int64_t *deg = (int64_t *)calloc((size_t)M + 1, sizeof(int64_t));
    int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)(M + 1));
    int64_t *queue = (int64_t *)malloc(sizeof(int64_t) * (size_t)(M + 1));
    int64_t *start = (int64_t *)malloc(sizeof(int64_t) * (size_t)(M + 2));
    char *placed = (char *)calloc((size_t)M + 1, 1);
    if (!cnt || !adj || !deg || !order || !queue || !start || !placed) {
        free(cnt); free(adj); free(deg); free(order); free(queue); free(start); free(placed);
        return -1;
    }
    /* symmetric adjacency lists: both directions of every off-diagonal entry */
    for (int64_t i = 0; i < M; ++i)
        for (int64_t p = rowptr[i]; p < rowptr[i + 1]; ++p)
            if (col[p] != i) {
                cnt[i] += 1;
                cnt[col[p]] += 1;
            }
    start[0] = 0;
    for (int64_t i = 0; i < M; ++i) start[i + 1] = start[i] + cnt[i];
    for (int64_t i = 0; i < M; ++i) cnt[i] = start[i];
    for (int64_t i = 0; i < M; ++i)
        for (int64_t p = rowptr[i]; p < rowptr[i + 1]; ++p)
            if (col[p] != i) {
                adj[cnt[i]++] = col[p];
                adj[cnt[col[p]]++] = i;
            }
    /* distinct neighbours, ascending, compacted in place; degree = their count */
    int64_t w = 0;
    for (int64_t i = 0; i < M; ++i) {
        int64_t n = start[i + 1] - start[i];
        int64_t *l = adj + start[i];
        qsort(l, (size_t)n, sizeof(int64_t), cmp_i64);
        int64_t b = w;
        for (int64_t q = 0; q < n; ++q)
            if (q == 0 || l[q] != l[q - 1]) adj[w++] = l[q];
        start[i] = b;
        deg[i] = w - b;
    }
    start[M] = w;
    for (int64_t i = 0; i < M; ++i) order[i] = i;
    g_deg = deg;
    qsort(order, (size_t)M, sizeof(int64_t), cmp_deg_id);
    int64_t head = 0, tail = 0;
    for (int64_t s = 0; s < M; ++s) {
        int64_t root = order[s];
        if (placed[root]) continue;
        placed[root] = 1;
        queue[tail++] = root;
        while (head < tail) {
            int64_t u = queue[head++];
            int64_t first = tail;
            for (int64_t q = start[u]; q < start[u] + deg[u]; ++q) {
                int64_t v = adj[q];
                if (!placed[v]) {
                    placed[v] = 1;
                    queue[tail++] = v;
                }
            }
            qsort(queue + first, (size_t)(tail - first), sizeof(int64_t), cmp_deg_id);
        }
    }
    for (int64_t i = 0; i < M; ++i) perm[i] = queue[M - 1 - i];
    free(cnt); free(adj); free(deg); free(order); free(queue); free(start); free(placed);
    return 0;
}

/*
 * P A P^T for a square CSR matrix and a permutation perm (perm[i] = the old
 * node placed at i): new row i is old row perm[i] with every column c renamed
 * to its new position inv[c]; each new row lists its entries by ascending new
 * column, equal columns in stored order.  rowptr_p [M+1], col_p [nnz],
 * val_p [nnz] (when val != NULL).  Returns 0, or -1 when perm is not a
 * permutation of [0, M) or on an allocation failure.
 */
typedef struct {
    int64_t c, p;
} cp_pair;
static int cmp_cp(const void *a, const void *b) {
    const cp_pair *x = (const cp_pair *)a, *y = (const cp_pair *)b;
    if (x->c != y->c) return (x->c > y->c) - (x->c < y->c);
    return (x->p > y->p) - (x->p < y->p);
}

int oracle_permute(const int64_t *rowptr, const int64_t *col, const float *val, int64_t M,
                   const int64_t *perm, int64_t *rowptr_p, int64_t *col_p, float *val_p) {
    int64_t *inv = (int64_t *)malloc(sizeof(int64_t) * (size_t)(M + 1));
    if (!inv) return -1;
    for (int64_t i = 0; i < M; ++i) inv[i] = -1;
    for (int64_t i = 0; i < M; ++i) {
        if (perm[i] < 0 || perm[i] >= M || inv[perm[i]] != -1) {
            free(inv);
            return -1;
        }
        inv[perm[i]] = i;
    }
    int64_t longest = 1;
    for (int64_t i = 0; i < M; ++i)
        if (rowptr[i + 1] - rowptr[i] > longest) longest = rowptr[i + 1] - rowptr[i];
    cp_pair *buf = (cp_pair *)malloc(sizeof(cp_pair) * (size_t)longest);
    if (!buf) {
        free(inv);
        return -1;
    }
    rowptr_p[0] = 0;
    for (int64_t i = 0; i < M; ++i) {
        int64_t o = perm[i], n = rowptr[o + 1] - rowptr[o];
        for (int64_t q = 0; q < n; ++q) {
            buf[q].c = inv[col[rowptr[o] + q]];
            buf[q].p = rowptr[o] + q;
        }
        qsort(buf, (size_t)n, sizeof(cp_pair), cmp_cp);
        for (int64_t q = 0; q < n; ++q) {
            col_p[rowptr_p[i] + q] = buf[q].c;
            if (val) val_p[rowptr_p[i] + q] = val[buf[q].p];
        }
        rowptr_p[i + 1] = rowptr_p[i] + n;
    }
    free(buf);
    free(inv);
    return 0;
}

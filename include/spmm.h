/*
 * spmm.h -- C ABI of the MI355X (gfx950) CSR sparse x dense product library
 * for GNN neighbour aggregation: C = A . B with sum, mean or max (+argmax)
 * reductions over each row's stored entries.
 *
 * The interface follows the problem statement shared by the pages:
 *  - A is a fixed graph in CSR form, built once and applied once per layer
 *    (graph-spmm kernel card, "Usage" and the SparseAdj row of its API table;
 *    RA-SpMM, "SpMM formulation": A fixed per graph, B changes per layer, the
 *    feature width N is known only at call time).
 *  - rowptr [M+1] and col [nnz] are int64, the dense operand is fp32
 *    (graph-spmm card, API table footnote and "Requirements and limits").
 *  - B and C are row-major (GE-SpMM, section II-A: GNN feature matrices are
 *    row-major, unlike a column-major vendor product).
 *  - reductions sum / mean / max with the winning neighbour's index, empty rows
 *    giving 0 and (0, -1), val == NULL meaning every stored entry is 1
 *    (graph-spmm card, API table and "Method").
 *
 * Semantics of one output element, for row i with stored entries p in
 * [rowptr[i], rowptr[i+1]) taken in stored order, t_p = a_p * B[col_p][k]
 * (a_p = val[p], or 1 when val == NULL):
 *   SUM  : fp32 sum of t_p.  Rows processed whole are summed in stored order
 *          with one fused multiply-add per entry; rows longer than the split
 *          threshold are summed piece by piece, pieces combined in order.
 *   MEAN : SUM / (number of stored entries), one IEEE fp32 division; 0 if empty.
 *   MAX  : largest t_p (strict '>', so the first of equal values wins) and the
 *          column id col_p of that entry; (0, -1) if the row is empty.
 * NaN products are outside the MAX contract: a row walked whole keeps the
 * stored-order rule exactly (a NaN first entry stays the maximum, later NaNs
 * never win), but for a row cut into pieces (row split, merge path) a NaN
 * that opens a later piece can hide that piece's larger values.
 * Duplicated (row, col) entries each count; columns need not be sorted.
 * Results are bitwise reproducible from run to run: no atomics are used.
 *
 * All functions return a status (or NULL for plan creation) and never abort
 * or throw.  spmm_last_error() returns the calling thread's last status and
 * a message.
 */
#ifndef GNN_SPMM_H
#define GNN_SPMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spmm_plan *spmm_plan_t;

/* Reductions. */
enum spmm_reduce { SPMM_SUM = 0, SPMM_MEAN = 1, SPMM_MAX = 2 };

/* Status codes. */
enum spmm_status {
    SPMM_OK = 0,
    SPMM_E_INVALID_ARG = -1, /* null / host pointer, negative size, bad enum  */
    SPMM_E_BAD_CSR = -2,     /* rowptr not monotone from 0, or col outside [0,K) */
    SPMM_E_OOM = -3,         /* device allocation failed                        */
    SPMM_E_HIP = -4,         /* a HIP runtime call or kernel launch failed      */
    SPMM_E_UNSUPPORTED = -5  /* size beyond the library's 32-bit index limits   */
};

/* Options for spmm_plan_set_option (value 0 / -1 = automatic where noted). */
enum spmm_option {
    SPMM_OPT_SPLIT_T = 1,      /* rows with more than T entries are split; -1 auto */
    SPMM_OPT_SPLIT_L = 2,      /* piece length of split rows; -1 auto             */
    SPMM_OPT_SPLIT_MODE = 3,   /* -1 auto (split only skewed graphs), 0 off, 1 on.
                                  In every mode rows of more than 2^24 entries
                                  are split, and T and L are capped at 2^24   */
    SPMM_OPT_LANES = 4,        /* lanes per row G in {4,8,16,32,64}; 0 auto       */
    SPMM_OPT_COARSEN = 5,      /* vectors per lane F in {1,2}; 0 auto             */
    SPMM_OPT_VEC = 6,          /* floats per vector in {1,2,4}; 0 auto.  4 also
                                  serves any N >= 4 and rows that are only
                                  4-byte aligned: the last vector of a row
                                  ends at column N                           */
    SPMM_OPT_XCD_REMAP = 7,    /* -1 auto, 0 off, 1 on: contiguous rows per XCD  */
    SPMM_OPT_NT_STORE = 8,     /* -1 auto, 0 off, 1 on: non-temporal C stores    */
    SPMM_OPT_TILES = 9,        /* -1 auto (low, even degrees), 0 off, 1 on, 2 on
                                  with 32-bit records: keep 8-row tile records
                                  holding row bounds + indexes               */
    SPMM_OPT_WINDOW = 10,      /* -1 auto (community structure, N > 32), 0 off,
                                  1 on: stage each 256-row block of B in LDS
                                  (a faster kernel when every row's columns
                                  are non-decreasing, bit-identical either way;
                                  that kernel's per-row runs, 8 bytes per row,
                                  are built by -1 with community structure
                                  and by 1, and freed by 0)                   */
    SPMM_OPT_MFMA = 11,        /* matrix-core tiles for community blocks, see
                                  below: 0 off (default), 1 fp16 tiles, 2 split
                                  fp16 tiles (fp32 tolerance)                 */
    SPMM_OPT_VBLOCK = 12,      /* vectorized blocking V = 2, see below: -1 auto
                                  (default): built at plan creation when the
                                  plan is not split, every row is stored with
                                  ascending columns and the padding share is
                                  <= 0.3; 0 off (frees them); 1 build, use when
                                  padding <= 0.3; 2 build, always use          */
    SPMM_OPT_BALANCE = 13,     /* load balance: 0 row split of heavy rows
                                  (default), 1 merge path, see below          */
    SPMM_OPT_PIECE_ORDER = 14, /* 1 (default): the row split's pieces run in
                                  ascending order of their first entry's
                                  column; 0: in partition order.  Same
                                  partition, same bits; rebuilds the split    */
    SPMM_OPT_MEM_LIMIT = 15,   /* bytes of device memory the plan may hold,
                                  counting the temporaries of a call on it;
                                  0 (default): no limit.  See "Device memory"
                                  below                                       */
    SPMM_OPT_SPLIT_FUSED = 16  /* 1 (default): a split product of N <= 256
                                  columns on the row kernel runs its light
                                  rows and its pieces in one dispatch (pieces
                                  first); 0: two dispatches.  Same bits      */
};

/*
 * Device memory.  The pages do not discuss memory limits; the library keeps
 * every device allocation it makes on a ledger so that callers can bound it:
 *  - SPMM_OPT_MEM_LIMIT caps what one plan holds: its own buffers plus the
 *    temporaries (and, for spmm_plan_transpose / spmm_plan_permute, the new
 *    plan's buffers) of any call made on it.  It is checked when a call
 *    allocates, not when the option is set.
 *  - spmm_set_mem_limit caps, for the calling thread, what one call may
 *    allocate (held at once, counted from zero at the start of the call); it
 *    covers the calls that are not made on a plan too (spmm_plan_create,
 *    spmm_coo_to_csr).
 * An allocation that would pass either limit is not made: the call returns
 * SPMM_E_OOM naming the buffer, the bytes asked and the limit, exactly as when
 * the device itself is out of memory.  A failed call frees every buffer it
 * allocated.  A failed spmm_plan_set_option leaves the plan usable: a failed
 * optional structure (tiles, panels, merge segments, fp16 tiles, window runs)
 * is simply absent, and a failed split rebuild puts the previous split
 * parameters back.  spmm_run never allocates.
 */
int spmm_set_mem_limit(int64_t bytes);   /* 0 = no limit; INVALID_ARG if < 0 */

struct spmm_mem_stats {
    int64_t in_use;            /* device bytes the library holds now, all
                                  plans and threads of the process           */
    int64_t last_call_peak;    /* the calling thread's last allocating call:
                                  most bytes it held at once                 */
    int64_t last_call_allocs;  /* ... and the number of allocations it made  */
    int64_t thread_limit;      /* the calling thread's spmm_set_mem_limit    */
};
int spmm_mem_stats(struct spmm_mem_stats *out);

/*
 * SPMM_OPT_BALANCE = 1 (merge-based balancing, RA-SpMM related work: the work
 * is partitioned along a virtual merge path over the CSR stream): setting it
 * builds, synchronously, the start coordinates of segments of 512 items (row
 * ends plus entries) of the merge of rowptr[1..M] with the entry indices,
 * and carry buffers of 2 KB per segment.  Later runs give every wave one
 * segment; rows that end inside a segment they started in are summed in
 * stored order (the same bits as the row kernels), rows spread over several
 * segments are summed piece by piece, pieces folded in order (same fp32
 * contract, deterministic); max ties still go to the first entry.  Setting 0
 * frees the segments and returns to the row split.
 */

/*
 * SPMM_OPT_VBLOCK (ParamSpMM section 3.1 vectorized blocking and section 4.2
 * PCSR, with V = 2): setting 1 or 2 builds, synchronously, a panel copy of
 * the matrix in which rows 2g and 2g+1 share one list of nonzero vectors (a
 * column present in either row; a column stored k and m times in the two rows
 * gives max(k, m) vectors), so each gather of a B row serves both rows.
 * Vectors run in ascending column order: rows stored with ascending columns
 * keep their stored order and give the same bits as without panels; other
 * rows are summed in ascending column order (same fp32 contract, different
 * rounding order), and MAX uses panels only when every row is stored with
 * ascending columns (tie order).  Needs K < 2^30; memory 4 bytes per vector
 * (+ 8 when weighted) + 4 per panel.  With 1, runs use the panels only when
 * the padding share 1 - nnz / (2 * vectors) is at most 0.3; with 2, always.
 * 0 frees them.  Split plans keep their own path unless the value is 2.
 * With -1 (the default) plan creation counts the vectors of a plan whose rows
 * are all stored with ascending columns in one merge pass and builds the
 * panels (two more merge passes and a scan, no sort) when the padding share
 * is at most 0.3, where each gather of a B row serves 1.4 entries or more.
 */

/*
 * SPMM_OPT_MFMA = 1 (RA-SpMM, "Kernel families": a dense tile path for
 * community-structured blocks, which gains by cutting memory traffic rather
 * than by reaching the matrix cores' peak).  Setting it builds, synchronously,
 * one dense 256 x 256 fp16 tile per aligned 256-row block holding the entries
 * whose column lies in the row's own block (duplicates summed in fp32 in
 * stored order, then rounded once to fp16), and a residual CSR of all other
 * entries in stored order; 128 KB of device memory per 256 rows plus the
 * residual.  Later SUM and MEAN runs whose N is a multiple of 4 with 16-byte
 * aligned B and C then compute the in-block part as fp16 x fp16 products with
 * fp32 accumulation on the matrix cores (B rounded to fp16, so |B| must stay
 * below 65504) and add the residual entries in fp32 in stored order.  Results
 * are bitwise reproducible but follow the looser contract of fp16 tiles:
 * |error| <= 2e-3 * sum_p |a_p * B[col_p][k]| + 1e-4 per element.  MAX runs,
 * other N and unaligned pointers keep the fp32 kernels.  Setting 0 frees the
 * tiles.  Returns UNSUPPORTED if an in-block sum of weights exceeds the fp16
 * range.
 * SPMM_OPT_MFMA = 2 builds split tiles instead: each tile is scaled by a power
 * of two (from its largest in-block sum) and stored as an fp16 high half plus
 * an fp16 low half (twice the memory); in the kernel each B slice is scaled
 * by a power of two (from its largest |b|) and split the same way, and three
 * products hi*hi + hi*lo + lo*hi per step leave about 2^-22 relative error
 * per term, so sum and mean meet the fp32 contract, |error| <= 1e-5 *
 * sum_p |a_p * B[col_p][k]| + 1e-6 (not bit-identical to the fp32 kernels).
 * Limit: a weight (feature) more than 2^18 below the largest in-block weight
 * sum of its tile (largest |b| of its 256-row x 64-column block of B) keeps
 * only an absolute accuracy of 2^-39 times that largest value.
 */

/* Descriptors of a plan and of its last routing decision. */
struct spmm_plan_info {
    int64_t M, K, nnz;
    int64_t dmax, n_empty;       /* largest row degree, number of empty rows     */
    double mean_deg;             /* nnz / M (0 when M == 0)                      */
    double cv_deg;               /* population std of row degree / mean_deg      */
    int64_t split_T, split_L;    /* row-split threshold and piece length in use  */
    int64_t n_heavy, n_seg;      /* split rows and pieces (0 when not split)     */
    double split_ratio;          /* (light rows + pieces) / M, ParamSpMM's SR    */
    int32_t has_val;             /* 1 if the plan holds edge values              */
    int32_t index_bits;          /* width of the plan's stored indexes (32)      */
    double plan_ms;              /* wall time of spmm_plan_create                */
    /* routing of the most recent spmm_run / spmm_plan_route call */
    int64_t route_N;
    int32_t route_lanes, route_vec, route_coarsen, route_rows_per_wave;
    int32_t route_slices, route_xcd_remap, route_nt_store, route_split;
    int32_t tiles, tile_cap;     /* row tiles: 0 none, 1 32-bit, 2 16-bit offset
                                    records; entries per record               */
    int32_t route_tiled;
    int32_t route_window;        /* 0 off; 1 window kernel, any column order;
                                    2 window kernel for rows whose columns are
                                    non-decreasing (checked at plan creation) */
    double win_frac;             /* share of entries inside their row's 256-row
                                    block (community structure)               */
    int64_t tile_overflow;       /* tiles that take the CSR path              */
    int64_t mfma_resid_nnz;      /* entries outside their row's block (residual
                                    CSR of the fp16 tile path; 0 when unbuilt) */
    int32_t mfma_tiles;          /* 1 fp16 tiles built, 2 split tiles built    */
    int32_t route_mfma;          /* 1 when the last run used them             */
    int64_t pair_vectors;        /* nonzero vectors of the V = 2 panels (0 when
                                    unbuilt)                                  */
    double pair_padding;         /* 1 - nnz / (2 * pair_vectors)              */
    int32_t pairs_built;         /* 1 built, 2 built and some row unsorted     */
    int32_t route_pairs;         /* 1 when the last run used the panels       */
    int64_t merge_segments;      /* merge-path segments (0 when unbuilt)      */
    int32_t route_merge;         /* 1 when the last run used them             */
    int32_t piece_order;         /* 1 when split pieces run in the order of
                                    their first column (SPMM_OPT_PIECE_ORDER) */
    int64_t generation;          /* bumped by every spmm_plan_set_option call
                                    that freed or replaced a device buffer of
                                    the plan (see spmm_run on graph capture) */
    int64_t device_bytes;        /* device memory the plan holds             */
    int64_t mem_limit;           /* SPMM_OPT_MEM_LIMIT (0: none)             */
    int32_t route_fused_split;   /* 1 when the last run sent light rows and
                                    split pieces in one dispatch              */
};

/*
 * Build a plan for the CSR matrix A [M, K] held on the current HIP device.
 *   rowptr : device int64 [M+1], rowptr[0] == 0, non-decreasing.
 *   col    : device int64 [nnz], values in [0, K); may be NULL when nnz == 0.
 *   val    : device fp32 [nnz], or NULL for an unweighted graph (all ones).
 * nnz is read from rowptr[M].  M, K and nnz must each be below 2^31.
 * The call is synchronous.  It validates the CSR on the GPU, computes the
 * degree descriptors (mean degree and its coefficient of variation, RA-SpMM
 * abstract), narrows indexes to int32, and builds the row split when the
 * graph is skewed.  It copies everything it needs: the caller may free or
 * change its arrays once it returns.  The plan owns its device memory until
 * spmm_plan_destroy.
 * Returns NULL on error (INVALID_ARG, BAD_CSR with the first bad row in the
 * message, OOM, HIP, UNSUPPORTED; see spmm_last_error).
 */
spmm_plan_t spmm_plan_create(const int64_t *rowptr, const int64_t *col, const float *val,
                             int64_t M, int64_t K);

/*
 * C = reduce(A . B) on `stream` (a hipStream_t; NULL = the null stream).
 *   B      : device fp32 [K, N] row-major (may be NULL only when K == 0).
 *   C      : device fp32 [M, N] row-major, fully overwritten.
 *   argmax : device int64 [M, N] or NULL; only allowed with SPMM_MAX, where it
 *            receives the column id of each maximum (-1 for empty rows).
 *   N      : feature width, N >= 1.
 * B, C and argmax need only their element alignment: for N >= 4 the kernels
 * read and write 16 bytes per lane at any 4-byte aligned address (a row's
 * last vector ends at column N), and write no byte outside C and argmax.
 * Asynchronous: it validates its arguments, picks a kernel from the plan's
 * descriptors and N, enqueues the kernels and returns without waiting.  It
 * allocates nothing and enqueues kernels only (no memset or copy), so a call
 * can be captured in a HIP graph on a stream in thread-local capture mode.
 * A captured call holds the kernel choice and the device addresses of its
 * time: it may be replayed while the plan, B and C stay alive AND the plan's
 * generation (spmm_plan_info) is unchanged.  spmm_plan_set_option calls that
 * build, rebuild or free a structure (split parameters, piece order, tiles,
 * window runs, fp16 tiles, panels, merge segments) replace buffers that a
 * captured kernel would still read or write, and bump the generation;
 * capture again after them.  B must not overlap C or argmax.  Runs on one plan must
 * be ordered on one stream (the plan's split buffer is shared); use one plan
 * per stream for concurrency.  Kernel faults surface at the caller's next
 * synchronisation, as usual in HIP.
 * Returns SPMM_OK, INVALID_ARG, UNSUPPORTED or HIP.  M == 0 is a no-op.
 */
int spmm_run(spmm_plan_t plan, const float *B, float *C, int64_t *argmax, int64_t N,
             int reduce, void *stream);

/* Free a plan and its device memory.  No run on it may still be in flight.
 * NULL is accepted (no-op). */
int spmm_plan_destroy(spmm_plan_t plan);

/* Copy the plan's descriptors and last routing decision into *out (host). */
int spmm_plan_info(spmm_plan_t plan, struct spmm_plan_info *out);

/* Fill the routing fields of the plan's info for width N and `reduce`
 * without running anything (B and C assumed 16-byte aligned). */
int spmm_plan_route(spmm_plan_t plan, int64_t N, int reduce);

/*
 * Copy the row split to host arrays.  Pieces are ordered by (row, piece) and
 * piece s of a split row i covers entries [rowptr[i] + s*L, min(rowptr[i] +
 * (s+1)*L, rowptr[i+1])) (ParamSpMM section 3.2 workload balancing, PCSR TRow
 * of section 4.2).  Light rows are the rows that are not split, ascending.
 *   seg_row/seg_begin/seg_end : host int64 [seg_cap] (may be NULL if seg_cap 0)
 *   light                     : host int64 [light_cap] (may be NULL if 0)
 *   counts                    : host int64 [3] = {n_heavy, n_seg, n_light}
 * At most seg_cap / light_cap entries are written.  Synchronous.
 */
int spmm_plan_partition(spmm_plan_t plan, int64_t *seg_row, int64_t *seg_begin,
                        int64_t *seg_end, int64_t seg_cap, int64_t *light,
                        int64_t light_cap, int64_t *counts);

/* Set an option (enum spmm_option).  Changing the split parameters rebuilds
 * the split synchronously; other options apply to later runs.  The caller
 * must not have runs on this plan in flight.  Options that free or replace
 * device buffers bump the plan's generation, which invalidates HIP graphs
 * captured from earlier runs on the plan (see spmm_run).  Returns OK,
 * INVALID_ARG, OOM (see "Device memory"), HIP or UNSUPPORTED. */
int spmm_plan_set_option(spmm_plan_t plan, int option, int64_t value);

/*
 * Edge list -> CSR (graph-spmm kernel card, API table: SparseAdj.from_edge_index
 * sorts an unsorted [2, E] edge list into CSR).  Edge e is the entry
 * (row[e], col[e]) with value val[e] (or no value when val == NULL).  Rows are
 * grouped in ascending order and each row keeps its entries in edge-list
 * order (a stable sort), so the CSR, and every product over it, is
 * deterministic.
 *   row, col          : device int64 [E] (may be NULL when E == 0)
 *   val               : device fp32 [E] or NULL
 *   rowptr_out        : device int64 [M+1], written
 *   col_out, val_out  : device int64 [E] / fp32 [E] (val_out only with val)
 * Synchronous; allocates and frees its own temporary device memory.  Returns
 * BAD_CSR naming the first edge whose row is outside [0, M) or column outside
 * [0, K); E, M and K must be below 2^31.
 */
int spmm_coo_to_csr(const int64_t *row, const int64_t *col, const float *val, int64_t E, int64_t M,
                    int64_t K, int64_t *rowptr_out, int64_t *col_out, float *val_out);

/*
 * spmm_coo_to_csr without any device allocation, for callers that cannot
 * allocate (code under HIP graph capture set-up, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, result and errors as
 * spmm_coo_to_csr (bit-identical output), but its temporaries live in a fixed
 * 32 MiB device workspace that the library reserves on every device it is
 * loaded on, held until the process ends.  Limit: E <= 2^20 edges; larger
 * edge lists return UNSUPPORTED before anything is launched.  Calls on one
 * device share that workspace: the library runs them one at a time (a lock
 * per device), and the workspace keeps the last call's contents, which no
 * call reads.  Synchronous; calls no hipMalloc or hipFree.
 */
int spmm_coo_to_csr_noalloc(const int64_t *row, const int64_t *col, const float *val, int64_t E, int64_t M,
                            int64_t K, int64_t *rowptr_out, int64_t *col_out, float *val_out);

/*
 * Plan of the transpose A^T [K, M] of a plan's matrix (graph-spmm card,
 * "Requirements and limits": the card is forward only and points to A^T,
 * the adjacency with every edge reversed, for the gradient of a sum).  Entry
 * (i, j, a) of A becomes (j, i, a'); within a row of A^T, entries keep A's
 * stored order (rows i ascending).  scale = 0: a' = a (unweighted stays
 * unweighted); scale = 1: a' = a / deg_i in fp32 (1 / deg_i when unweighted),
 * so that spmm_run(A^T, dC, SUM) is the backward of MEAN.  Synchronous;
 * returns a new plan (destroy it separately) or NULL on error.
 */
spmm_plan_t spmm_plan_transpose(spmm_plan_t plan, int scale);

/*
 * Max-pool backward (graph-spmm card, "Method": the forward max reports its
 * winning neighbour, and that index routes the gradient back).  plan_t is the transpose
 * (scale 0) of an UNWEIGHTED adjacency A [M, K]; argmax and dC are the
 * forward's argmax [M, N] (int64) and the output gradient [M, N] (fp32):
 *   dB[j][k] = sum of dC[i][k] over rows i with argmax[i][k] == j,
 * summed in ascending i with no atomics (bitwise reproducible); a duplicated
 * (i, j) edge counts once.  dB [K, N] fp32 is fully written.  Asynchronous on
 * `stream`, allocates nothing.  Returns UNSUPPORTED for a weighted plan_t.
 */
int spmm_max_backward(spmm_plan_t plan_t, const int64_t *argmax, const float *dC, float *dB, int64_t N,
                      void *stream);

/*
 * Sparse-matrix features of ParamSpMM section 5.1, Table 3 (size, degree
 * distribution and data-locality features), for analysing a graph and
 * choosing a layout; V is the width of ParamSpMM's vectorized blocking
 * (section 3.1: blocks of V consecutive rows, rows V*g .. V*g+V-1).
 *   n, n_nonempty, nnz, dmax : rows, rows with entries, stored entries,
 *                              largest row degree
 *   delta                    : n_nonempty / n
 *   mean_deg, cv_deg         : nnz / n and the degree's population
 *                              coefficient of variation over all rows
 *   mean_deg_nonempty, cv_deg_nonempty : the same over non-empty rows
 *   density                  : nnz / (n * K)
 *   mean_bandwidth, max_bandwidth : a row's bandwidth is its largest minus
 *                              its smallest column id (Table 3 footnote);
 *                              mean over non-empty rows, and the maximum
 *   nnz_distinct             : distinct (row, col) pairs
 *   nnz_vectors              : nonzero vectors of V-row blocking: columns
 *                              with at least one entry in a block, summed
 *                              over blocks
 *   padding_ratio            : eq. 2, 1 - nnz_distinct / (nnz_vectors * V)
 *                              (0 when the matrix has no entries)
 *   split_ratio, win_frac    : as in spmm_plan_info
 * 1 <= V <= 64.  Synchronous: sorts a temporary copy of the pattern on the
 * GPU (16 bytes per entry of device memory, freed before returning).
 * Returns OK, INVALID_ARG, OOM or HIP.
 */
struct spmm_features {
    int64_t n, n_nonempty, nnz, dmax;
    double delta, mean_deg, mean_deg_nonempty, cv_deg, cv_deg_nonempty, density;
    double mean_bandwidth;
    int64_t max_bandwidth;
    int64_t V, nnz_distinct, nnz_vectors;
    double padding_ratio;
    double split_ratio, win_frac;
};
int spmm_plan_features(spmm_plan_t plan, int64_t V, struct spmm_features *out);

/* Reordering methods for spmm_plan_reorder. */
enum spmm_reorder_method { SPMM_REORDER_RCM = 1 };

/*
 * Locality reordering (ParamSpMM section 4.4: a reordering that puts nodes
 * with shared neighbours close together complements the kernels and is
 * amortised over the reuses of the graph).  SPMM_REORDER_RCM: reverse
 * Cuthill-McKee (Cuthill and McKee 1969; reversal by George 1971) on the
 * symmetric pattern of A + A^T (distinct neighbours, self loops ignored):
 * nodes taken in ascending (degree, id) order start components, each placed
 * breadth first with every node appending its unplaced neighbours in
 * ascending (degree, id) order; the order is then reversed.  Deterministic.
 *   perm : device int64 [M], written: perm[i] = the node placed at position i.
 * Needs a square plan (M == K).  Synchronous; allocates and frees one block
 * of temporary device memory (about 72 bytes per entry of A and 60 per
 * node).  Returns OK, INVALID_ARG (non-square plan, unknown method, bad
 * pointer), OOM or HIP.
 */
int spmm_plan_reorder(spmm_plan_t plan, int method, int64_t *perm);

/*
 * Plan of P A P^T for a square plan and a permutation perm (device int64
 * [M], perm[i] = the old node placed at position i): new row i is old row
 * perm[i] with every column c renamed to its new position; each new row lists
 * its entries by ascending new column, equal columns in stored order.  Use it
 * with B' = P B (row i of B' = row perm[i] of B); then C' = P C.
 * Synchronous; returns a new plan (destroy it separately) or NULL: INVALID_ARG
 * when perm is not a permutation of [0, M) or the plan is not square.
 */
spmm_plan_t spmm_plan_permute(spmm_plan_t plan, const int64_t *perm);

/* The calling thread's last status; copies its message (NUL-terminated,
 * truncated to cap bytes) into buf when buf != NULL and cap > 0. */
int spmm_last_error(char *buf, int64_t cap);

#ifdef __cplusplus
}
#endif

#endif /* GNN_SPMM_H */

/*
 * lora_oracle.c -- plain CPU reference ("the oracle") for multi-adapter LoRA apply.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
 * bench.py use it.  It shares no code, header, table or helper with the HIP
 * library; the two only ever see the same seeded input buffers.
 *
 * What it computes, and where the pages define it:
 *
 *   Per-row adapted output.  Page "Multi-LoRA Serving: one base, many adapters",
 *   section 2 (mental model, per-row equation) and section 3.1 (LoRA math):
 *   for row i with adapter a(i),
 *        y_i = W x_i + (alpha / r) * B_a (A_a x_i),
 *   with A_a in R^{r x k} (the "shrink" factor) and B_a in R^{d x r} (the
 *   "expand" factor); Delta W = B A is never formed.  The base output W x_i is
 *   already in y (section 2 flowchart: the shared base GEMM runs once, then
 *   add_shrink v = A x, add_expand delta = B v * alpha / r, merge per row).
 *   Rows without an adapter keep the base output (same section: row with
 *   no adapter id; page "LoRA hot-loading and adapter routing", section on
 *   adapter routing: a None id means no LoRA).
 *
 *   Grouping by adapter id.  Page "LoRA hot-loading and adapter routing",
 *   section on batched multi-adapter execution (one group of row indices per
 *   adapter id), and the Multi-LoRA page's flowchart step "group rows by
 *   adapter id".  The pages do not fix the order inside a group; the reading
 *   used here is a stable counting sort: rows in ascending index order within a
 *   group, groups in ascending slot order, and rows with no valid adapter
 *   appended at the end in index order.
 *
 * Precision: every product and sum is taken in IEEE double.  Inputs arrive as
 * fp32 or bf16 bit patterns and are widened exactly (bf16 -> fp32 is a 16-bit
 * left shift, fp32 -> double is exact).  The outputs are unrounded doubles.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *   - scale = alpha_s / r_s with the slot's true rank r_s;
 *   - each output slice q (fused q/k/v, gate/up) has its own A_q, B_q, with the
 *     row's adapter id and scale shared by all slices; slices sit side by side
 *     in y at offsets off_q = d_0 + ... + d_{q-1};
 *   - an id that is neither -1 nor a loaded slot in [0, n_slots) is "bad": it is
 *     counted and its row is left untouched, like a none row.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Widen element idx of a dtype buffer to double (exact for both dtypes). */
static double load_elem(int dtype, const void *base, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* A row is routed to slot s when 0 <= s < n_slots and slot s holds an adapter. */
static int row_is_valid(int32_t id, int n_slots, const int32_t *slot_rank)
{
    return id >= 0 && id < n_slots && slot_rank[id] > 0;
}

/*
 * Segment construction: group rows by adapter id.
 *
 *   perm[n]          row indices, grouped by slot (ascending), stable inside a
 *                    group; rows without a valid adapter follow, in index order
 *   seg_off[N+1]     seg_off[s] = first position of slot s in perm;
 *                    seg_off[N] = number of valid rows
 *   active[N]        slots with at least one row, ascending (first counts[1]
 *                    entries are meaningful, the rest are set to -1)
 *   counts[3]        {valid rows, active slots, bad ids}
 *
 * Returns 0, or -1 on a bad argument.
 */
int oracle_build_segments(const int32_t *ids, int64_t n, int n_slots,
                          const int32_t *slot_rank, int32_t *perm,
                          int32_t *seg_off, int32_t *active, int32_t *counts)
{
    if (n < 0 || n_slots < 1 || (n > 0 && (!ids || !perm)) || !slot_rank ||
        !seg_off || !active || !counts)
        return -1;

    int64_t *count = calloc((size_t)n_slots, sizeof *count);
    int64_t *fill = calloc((size_t)n_slots, sizeof *fill);
    if (!count || !fill) {
        free(count);
        free(fill);
        return -1;
    }

    /* histogram of valid rows per slot; count the bad ids */
    int64_t n_bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (row_is_valid(ids[i], n_slots, slot_rank))
            count[ids[i]] += 1;
        else if (ids[i] != -1)
            n_bad += 1;
    }

    /* exclusive prefix sum of the histogram */
    seg_off[0] = 0;
    for (int s = 0; s < n_slots; ++s)
        seg_off[s + 1] = seg_off[s] + (int32_t)count[s];

    /* stable placement: scan rows in ascending index order */
    for (int64_t i = 0; i < n; ++i) {
        if (row_is_valid(ids[i], n_slots, slot_rank)) {
            int s = ids[i];
            perm[seg_off[s] + fill[s]] = (int32_t)i;
            fill[s] += 1;
        }
    }
    int64_t tail = seg_off[n_slots];
    for (int64_t i = 0; i < n; ++i) {
        if (!row_is_valid(ids[i], n_slots, slot_rank)) {
            perm[tail] = (int32_t)i;
            tail += 1;
        }
    }

    int n_active = 0;
    for (int s = 0; s < n_slots; ++s)
        if (count[s] > 0)
            active[n_active++] = s;
    for (int s = n_active; s < n_slots; ++s)
        active[s] = -1;

    counts[0] = seg_off[n_slots];
    counts[1] = n_active;
    counts[2] = (int32_t)n_bad;
    free(count);
    free(fill);
    return 0;
}

/*
 * Adapted output of selected rows, in double, unrounded.
 *
 *   dtype        ORACLE_F32 or ORACLE_BF16 (x, y_in, A and B all share it)
 *   k            input width; n_slices, slice_d[n_slices]: output slices, D = sum
 *   slot_rank[N] true rank of each slot (0 = empty); slot_alpha[N] its alpha
 *   A_cat, A_off slot s's shrink factor, dense at true rank, [n_slices][r_s][k],
 *                starting at element A_off[s] of A_cat
 *   B_cat, B_off slot s's expand factor, dense at true rank, [D][r_s] (slices
 *                stacked along D), starting at element B_off[s] of B_cat
 *   ids[n]       adapter id per row (-1 = none)
 *   x, ldx       input rows, row i starts at element i * ldx
 *   y_in, ldy    base output rows (W x_i), row i starts at element i * ldy
 *   rows, n_sel  which rows to evaluate (rows == NULL: rows 0 .. n_sel-1)
 *   yref         [n_sel][D] doubles, written
 *   n_threads    OpenMP threads over rows (<= 1: serial)
 *
 * Returns 0, or -1 on a bad argument.
 */
int oracle_apply_rows(int dtype, int64_t k, int n_slices, const int64_t *slice_d,
                      int n_slots, const int32_t *slot_rank, const double *slot_alpha,
                      const void *A_cat, const int64_t *A_off,
                      const void *B_cat, const int64_t *B_off,
                      const int32_t *ids, const void *x, int64_t ldx,
                      const void *y_in, int64_t ldy,
                      const int64_t *rows, int64_t n_sel, double *yref, int n_threads)
{
    if ((dtype != ORACLE_F32 && dtype != ORACLE_BF16) || k < 1 || n_slices < 1 ||
        !slice_d || n_slots < 1 || !slot_rank || !slot_alpha || !ids || !x ||
        !y_in || n_sel < 0 || (n_sel > 0 && !yref))
        return -1;

    int64_t D = 0;
    for (int q = 0; q < n_slices; ++q)
        D += slice_d[q];
    if (ldx < k || ldy < D)
        return -1;

    int max_rank = 0;
    for (int s = 0; s < n_slots; ++s)
        if (slot_rank[s] > max_rank)
            max_rank = slot_rank[s];

    int bad_arg = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 1 ? n_threads : 1)
#endif
    for (int64_t sel = 0; sel < n_sel; ++sel) {
        int64_t i = rows ? rows[sel] : sel;
        double *out = yref + sel * D;

        /* the base output W x_i, already in y */
        for (int64_t c = 0; c < D; ++c)
            out[c] = load_elem(dtype, y_in, i * ldy + c);

        int32_t s = ids[i];
        if (!row_is_valid(s, n_slots, slot_rank))
            continue; /* none row or bad id: base output unchanged */

        int r = slot_rank[s];
        double scale = slot_alpha[s] / (double)r;
        double *v = malloc((size_t)(max_rank > 0 ? max_rank : 1) * sizeof *v);
        if (!v) {
            bad_arg = 1;
            continue;
        }

        int64_t off = 0; /* first output column of slice q */
        for (int q = 0; q < n_slices; ++q) {
            /* add_shrink: v = A_q x_i, one value per rank index j */
            for (int j = 0; j < r; ++j) {
                double acc = 0.0;
                for (int64_t t = 0; t < k; ++t) {
                    double a = load_elem(dtype, A_cat, A_off[s] + ((int64_t)q * r + j) * k + t);
                    double xv = load_elem(dtype, x, i * ldx + t);
                    acc += a * xv;
                }
                v[j] = acc;
            }
            /* add_expand and merge: y += (alpha / r) * B_q v */
            for (int64_t o = 0; o < slice_d[q]; ++o) {
                double acc = 0.0;
                for (int j = 0; j < r; ++j)
                    acc += load_elem(dtype, B_cat, B_off[s] + (off + o) * r + j) * v[j];
                out[off + o] += scale * acc;
            }
            off += slice_d[q];
        }
        free(v);
    }
    return bad_arg ? -1 : 0;
}

/*
 * Parameters held by one adapter on one stack: every slice q has its own
 * A_q (r x k) and B_q (d_q x r), so the total is r * (n_slices * k + D).  For a
 * single slice this is the r(d + k) count of page "Multi-LoRA Serving: one
 * base, many adapters", section 3.1 (LoRA math).  Returns -1 on a bad argument.
 */
int64_t oracle_param_count(int rank, int64_t k, int n_slices, const int64_t *slice_d)
{
    if (rank < 0 || k < 1 || n_slices < 1 || !slice_d)
        return -1;
    int64_t total = 0;
    for (int q = 0; q < n_slices; ++q)
        total += (int64_t)rank * k + slice_d[q] * (int64_t)rank;
    return total;
}

/*
 * Merged weight of one adapter, in double, unrounded.
 *
 * Page "LoRA serving: multi-adapter dynamic loading", section 1 (merge versus
 * keeping the adapter separate): folding one adapter into the base weight,
 * W' = W + (alpha / r) B A, serves that adapter at the base model's cost, and
 * unmerging subtracts the same product.  Page "Multi-LoRA Serving", section
 * 3.1 gives the shapes: B is d x r, A is r x k.  With output slices (fused
 * q/k/v, gate/up) the rows of slice q use that slice's A_q.
 *
 *   dtype            ORACLE_F32 or ORACLE_BF16 (W, A, B share it)
 *   k                input width (columns of W)
 *   n_slices, slice_d[n_slices]   output slices; D = sum, the rows of W
 *   rank, alpha      the slot's true rank and alpha; scale = alpha / rank
 *   A [n_slices][rank][k], B [D][rank]   the slot's factors, dense at true rank
 *   W, ldw           base weight, row o (output feature) starts at element o * ldw
 *   sign             +1 merge, -1 unmerge
 *   Wout [D][k]      doubles, written:
 *                    W[o][i] + sign * scale * sum_j B[o][j] A[q(o)][j][i]
 *   n_threads        OpenMP threads over rows (<= 1: serial)
 *
 * Returns 0, or -1 on a bad argument.
 */
int oracle_merge(int dtype, int64_t k, int n_slices, const int64_t *slice_d, int rank,
                 double alpha, const void *A, const void *B, const void *W, int64_t ldw,
                 int sign, double *Wout, int n_threads)
{
    if ((dtype != ORACLE_F32 && dtype != ORACLE_BF16) || k < 1 || n_slices < 1 || !slice_d ||
        rank < 1 || !A || !B || !W || ldw < k || (sign != 1 && sign != -1) || !Wout)
        return -1;
    int64_t D = 0;
    for (int q = 0; q < n_slices; ++q)
        D += slice_d[q];
    const double scale = alpha / (double)rank;

#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(n_threads > 1 ? n_threads : 1)
#endif
    for (int64_t o = 0; o < D; ++o) {
        /* the slice this output row belongs to */
        int q = 0;
        int64_t off = 0;
        while (q + 1 < n_slices && o >= off + slice_d[q]) {
            off += slice_d[q];
            ++q;
        }
        for (int64_t i = 0; i < k; ++i) {
            double delta = 0.0;
            for (int j = 0; j < rank; ++j)
                delta += load_elem(dtype, B, o * rank + j) *
                         load_elem(dtype, A, ((int64_t)q * rank + j) * k + i);
            Wout[o * k + i] = load_elem(dtype, W, o * ldw + i) + (double)sign * scale * delta;
        }
    }
    return 0;
}

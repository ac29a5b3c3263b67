/*
 * scmp.h -- C ABI of libscmp, the MI355X (gfx950) stochastic-computing (SC)
 * bipolar XNOR matmul with dynamic mixed precision.
 *
 * What the library computes is defined on these pages:
 *  [PAYN]  "Precision As You Need: Stochastic Computing Is a Dense Adaptive
 *          Quantizer" (paper notes): Key design 1 (Sobol-8 cumulative
 *          indicator table, conditional bitstream generator C-BSG, bipolar
 *          XNOR decode equation), Key design 2 (row metrics, threshold
 *          ladder), Key design 3 (early termination per row), Key design 4
 *          (the compensation layer W_b x + b_b run as an SC linear).
 *  [VIT]   scmp_vit README: "Why it works" (per-row bipolar quantisation,
 *          scale = row abs-max / 127), the mixed-precision flag table, the
 *          SC early-termination note for non-power-of-two lengths, and the
 *          head-aligned SC compensator (16 per-head D = 64 SC linears).
 *  [KBAND] pull request "feat(mp): per-group (K-band) stream lengths on the
 *          contraction axis": "How the banding works", "Guards", "Tooling".
 *
 * Conventions shared by every call
 *  - Every pointer named *_dev is a device pointer (HIP global memory) owned
 *    by the caller; it must stay valid until the work queued on `stream`
 *    has finished.  Host pointers are only read during the call.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Every device call is asynchronous on that stream and never
 *    synchronises the device, except scmp_error_flags.
 *  - Calls never allocate device memory, except scmp_build_sobol_table (the
 *    one-time table) which allocates the table it returns.  Scratch memory
 *    comes from the caller (scmp_matmul_workspace_bytes).
 *  - Arguments and plans are validated on the host before any launch.  On
 *    error nothing is launched and the status is returned;
 *    scmp_last_error() then describes the failure (thread-local string).
 *  - Sizes of 0 (G, rows, M or N) are valid and launch nothing.
 *  - Supported precision: 2 <= p <= 8 (q = 2^(p-1) - 1, P = 2^p levels + 1),
 *    1 <= Lmax <= 2^p.  The workloads use p = 8, Lmax = 256.
 *
 * Layouts (row-major, C order)
 *  - Quantised integers: int8 [G][rows][cols], values in [-q, q].
 *  - Scales: float [G][rows][n_chunks] (n_chunks = 1 without chunk_d).
 *  - Packed streams (weight side, optional): uint32 [G][rows][cols][Wl],
 *    Wl = ceil(Lmax / 32); bit b of word w is K[u][32 w + b].
 *  - Row metric, normalised metric: float [G][rows]; rungs: uint8 [G][M];
 *    permutation: int32 [G][M] (sorted position -> row).
 *  - Counts: int32 [G][M][N][n_bands]; outputs C: float with element
 *    (g, i, j) at C_dev[g * batch_stride_c + i * ldc + j].
 */
#ifndef SCMP_H
#define SCMP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SCMP_OK = 0,
  SCMP_ERR_ARG = 1,            /* bad argument: null pointer, bad size or stride */
  SCMP_ERR_CEILING = 2,        /* a (band) length above the ceiling [KBAND] "Guards" */
  SCMP_ERR_ISO_COMPUTE = 3,    /* per-rung iso-compute identity overspent [KBAND] */
  SCMP_ERR_UNSUPPORTED = 4,    /* K-bands on qk/av, K-bands with range MP, range MP [KBAND] "Guards" */
  SCMP_ERR_PLAN_MISMATCH = 5,  /* table priced at another chunk_d or width; shapes vs plan [KBAND] "Guards" */
  SCMP_ERR_NONFINITE = 6,      /* a non-finite input was seen (reported by scmp_error_flags) */
  SCMP_ERR_WORKSPACE = 7,      /* workspace smaller than scmp_matmul_workspace_bytes */
  SCMP_ERR_HIP = 8             /* a HIP runtime call or launch failed */
} scmp_status;

typedef enum { SCMP_OP_LINEAR = 0, SCMP_OP_QK = 1, SCMP_OP_AV = 2 } scmp_op;

/* SC gate of a plan ([PAYN] "Research background and motivation" and Key
 * design 3: one AND gate for unipolar SC, one XNOR gate for bipolar SC;
 * [VIT] SC compensation flags: bipolar or unipolar per-row mode).
 *  BIPOLAR: a stream's level is u = round(P (x + q) / (2 q)); the XNOR
 *           count decodes as s^A s^B q^2 (2 count - L |c|) / L.
 *  UNIPOLAR: sign-magnitude; a stream carries |x| at level
 *           u = round(P |x| / q) (0 -> 0, q -> P) on the same C-BSG streams,
 *           the AND count is taken with the product of the two signs, and
 *           decodes as s^A s^B q^2 count / L. */
typedef enum { SCMP_MODE_BIPOLAR = 0, SCMP_MODE_UNIPOLAR = 1 } scmp_mode;

/* Contraction kernel.  All give bit-identical counts.
 *  AUTO/MFMA: windowed ternary x paired-binary contraction on the fp4
 *             matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4, e2m1 operands
 *             {-1, 0, +1} and {0, 1, 2} at unit scales, float32
 *             accumulators that hold the integer counts exactly while
 *             scmp_plan_info.mfma_exact is 1); the launch form is chosen by
 *             size (persistent when the plan allows it and there are several
 *             output tiles per block, one block per tile otherwise); AUTO
 *             takes the quarter form (below) for persistent plans with
 *             D >= 512 where at least half of the 128-row tiles run streams
 *             of length <= 96 (MFMA never does).  When mfma_exact is 0,
 *             AUTO runs GATHER (bipolar) or BITSERIAL (unipolar) instead and
 *             the MFMA forms return UNSUPPORTED.
 *  MFMA_PERSISTENT: the matrix-core path as a persistent grid taking
 *             output tiles from a work counter; bipolar plans without chunk
 *             scales and with one band only (UNSUPPORTED otherwise).
 *  MFMA_ONEPASS: the matrix-core path with one block per output tile.
 *  MFMA_QUARTER: the persistent grid with the first 16 paired positions
 *             of each index taken 8 at a time (operands from 17 x 17-entry
 *             pair tables of window and pair-sum classes), so that indices
 *             whose windows end by position 8 cost half a step; the same
 *             plans as MFMA_PERSISTENT with the band starting on a multiple
 *             of 32 and D rounded up to 32 at most 4096 (UNSUPPORTED
 *             otherwise).  Its workspace is larger (quarter codes: 1 byte
 *             per row and index, 1 byte per column, index and ladder rung).
 *  BITSERIAL: one bit-select + popcount per 32 stream positions on the
 *             vector ALU; needs the packed weight-side streams.
 *  GATHER:    one lookup per (row, column, index) in a per-length table
 *             T_L[u_A][u_B] of XNOR counts (built into the workspace and
 *             staged whole into LDS); bipolar plans only. */
typedef enum {
  SCMP_ALGO_AUTO = 0,
  SCMP_ALGO_BITSERIAL = 1,
  SCMP_ALGO_MFMA = 2,
  SCMP_ALGO_MFMA_PERSISTENT = 3,
  SCMP_ALGO_MFMA_ONEPASS = 4,
  SCMP_ALGO_GATHER = 5,
  SCMP_ALGO_MFMA_QUARTER = 6
} scmp_algo;

typedef struct scmp_table_s* scmp_table_t; /* opaque, library-owned */
typedef struct scmp_plan_s* scmp_plan_t;   /* opaque, library-owned, host only */

#define SCMP_MAX_RUNGS 8
#define SCMP_MAX_BANDS 16

/* Description of one SC matmul: [PAYN] Key designs 2-3, [VIT] MP flags,
 * [KBAND] "How the banding works" and "Tooling". */
typedef struct {
  int op;                    /* scmp_op */
  int p;                     /* integer bits; must match the table */
  int Lmax;                  /* table length; must match the table */
  int D;                     /* contraction length */
  int chunk_d;               /* 0: one scale per row; >0: one scale per (row, chunk of chunk_d
                                columns), the last chunk may be short; must be a multiple of 32 */
  int n_rungs;               /* 1..SCMP_MAX_RUNGS; 1 = uniform length */
  const int* levels;         /* [n_rungs] stream lengths, strictly descending, >= 1 */
  const double* fractions;   /* [n_rungs] row fractions in the same order, sum 1; NULL = equal */
  int n_bands;               /* 1..SCMP_MAX_BANDS; >1 needs chunk_d > 0 and op LINEAR */
  const int* band_chunks;    /* [n_bands] band widths in whole chunks; NULL = equal split */
  double tilt;               /* straight-line tilt t (used when band_L is NULL) */
  const int* band_L;         /* [n_bands][n_rungs] explicit L[b][k], or NULL */
  int table_chunk_d;         /* chunk_d the explicit band_L was priced at (0 = not stated) */
  int table_D;               /* contraction width band_L was priced at (0 = not stated) */
  int ceiling;               /* largest allowed length; 0 = Lmax; must be <= Lmax */
  int range_mp;              /* nonzero: range-based per-weight-group MP (op LINEAR, two levels,
                                one band); the contraction then runs through scmp_matmul_range */
  int mode;                  /* scmp_mode; 0 = bipolar */
  double range_threshold;    /* range MP: groups with normalised range below it take levels[1] */
  int range_group;           /* range MP: W rows per weight group (0 = 128) */
} scmp_plan_desc;

typedef struct {
  int op, p, Lmax, D, chunk_d, n_chunks, n_rungs, n_bands, ceiling, mode, range_mp, range_group;
  /* 1 when the matrix-core forms hold this plan's counts exactly: they
   * accumulate each segment (D, or one chunk of chunk_d indices) in float32,
   * one index adding at most L + 1 in magnitude, so the plan needs
   * segment * (longest L + 1) < 2^24.  When 0, AUTO runs GATHER (bipolar)
   * or BITSERIAL (unipolar) and the MFMA forms return UNSUPPORTED. */
  int mfma_exact;
} scmp_plan_info;

/* Name of a status code (static string). */
const char* scmp_status_string(int status);

/* Description of the last failure on the calling thread ("" if none). */
const char* scmp_last_error(void);

/* Build the device-resident Sobol table ([PAYN] Key design 1): Sobol points
 * r_l (unscrambled, Gray-code order, r_0 = 0) for l < Lmax, the indicator
 * table K[u][l] = 1[r_l < u] for levels u in [0, 2^p] (row u = b + 1 of the
 * page's 1[r_l <= b]), its prefix sums cum[u][n], and for every length
 * L <= Lmax the paired-position tables the MFMA contraction reads.
 * Allocates device memory (a few MB) owned by the returned table; the
 * build is queued on `stream`.  Errors: ARG (p or Lmax out of range), HIP. */
int scmp_build_sobol_table(int p, int Lmax, void* stream, scmp_table_t* out);

/* Free a table (synchronises the device first).  NULL is ignored. */
int scmp_table_destroy(scmp_table_t table);

/* p and Lmax of a table.  Errors: ARG. */
int scmp_table_info(scmp_table_t table, int* p, int* Lmax);

/* Copy the table to caller buffers (device): r_dev uint16 [Lmax],
 * K_dev uint32 [2^p + 1][ceil(Lmax/32)], cum_dev uint16 [2^p + 1][Lmax + 1].
 * Any pointer may be NULL.  Errors: ARG, HIP. */
int scmp_table_export(scmp_table_t table, uint16_t* r_dev, uint32_t* K_dev, uint16_t* cum_dev,
                      void* stream);

/* Validate a description and build the plan (host only, the "startup" of
 * [KBAND] "Guards").  Band lengths come from band_L or from the straight-
 * line tilt: for rungs below the ceiling raw_b = L_k (1 + t x_b),
 * x_b = (2b - (B-1)) / (B-1), rounded down, single units handed back to the
 * bands with the largest lost fraction (ties to the lower band); rungs at
 * the ceiling stay untilted ([KBAND] "Tooling"); the tilt needs bands of
 * equal column width.
 * Errors: ARG, CEILING (any length above the ceiling), ISO_COMPUTE
 * (sum_b D_b L[b][k] > D L_k), UNSUPPORTED (n_bands > 1 with op QK or AV;
 * range_mp with bands or with op QK / AV; chunk_d not a multiple of 32),
 * PLAN_MISMATCH (table_chunk_d / table_D differ from chunk_d / D). */
int scmp_plan_create(const scmp_plan_desc* desc, scmp_plan_t* out);

/* Free a plan.  NULL is ignored. */
int scmp_plan_destroy(scmp_plan_t plan);

int scmp_plan_query(scmp_plan_t plan, scmp_plan_info* out);

/* L[b][k] as int [n_bands][n_rungs]. */
int scmp_plan_band_lengths(scmp_plan_t plan, int* L_out);

/* Band column boundaries, int [n_bands + 1]. */
int scmp_plan_band_columns(scmp_plan_t plan, int* cols_out);

/* Per-rung budget use sum_b D_b L[b][k] / (D L_k), double [n_rungs]. */
int scmp_plan_budget_use(scmp_plan_t plan, double* use_out);

/* Sorted-position cuts for M rows, int [n_rungs + 1]: cut_0 = 0,
 * cut_(k+1) = floor(F_k M + 0.5) with F_k the running float64 sum of the
 * fractions (last cut M).  Rung k holds sorted positions [cut_k, cut_(k+1)). */
int scmp_plan_row_cuts(scmp_plan_t plan, int M, int* cuts_out);

/* Fused symmetric quantisation and C-BSG encoding ([VIT] "Why it works";
 * [PAYN] Key design 1).  For each of the G x rows rows of X (or each chunk
 * of chunk_d columns when the plan has chunk_d): a = max |x| (float32),
 * s = a / q (IEEE float32 division), x_int = clamp(rint(x / s), -q, q)
 * (float32 division, round half to even); an all-zero row or chunk gives
 * s = 0 and integers 0.  Element (g, r, c) of X is read at
 * X_dev[g * batch_stride + r * row_stride + c * col_stride].
 *   q_dev       int8 [G][rows][cols]               (required)
 *   scales_dev  float [G][rows][n_chunks]          (required)
 *   metric_dev  float [G][rows]: max_c |x| of the whole row; this is the
 *               MP row metric ||X_i||_inf, and max_j A_ij for non-negative
 *               attention rows ([PAYN] Key design 2)            (nullable)
 *   packed_dev  uint32 [G][rows][cols][ceil(Lmax/32)]: the weight side's
 *               full-length counter-domain stream K[u][0..Lmax) with
 *               u = round(P (x_int + q) / (2 q)), or u = round(P |x_int| / q)
 *               for a unipolar plan                             (nullable)
 * cols must equal the plan's D.  Non-finite inputs set a device flag read
 * by scmp_error_flags.  Errors: ARG, PLAN_MISMATCH, HIP. */
int scmp_quantize_encode(scmp_table_t table, scmp_plan_t plan, const float* X_dev, int G, int rows,
                         int cols, int64_t batch_stride, int64_t row_stride, int64_t col_stride,
                         int8_t* q_dev, float* scales_dev, float* metric_dev, uint32_t* packed_dev,
                         void* stream);

/* Row classification ([PAYN] Key design 2): per group g, the normalised
 * metric g_hat = metric / max(metric) (float32; 0 when the max is 0; NaN
 * ranks last), the sorted order by g_hat descending with ties by row index,
 * the rung of each row from the plan's cuts, and thresholds tau_k
 * (k = 1..K-1) = g_hat at sorted position cut_k - 1 (1.0 if none).
 *   metric_dev float [G][M]; ghat_dev float [G][M] (required);
 *   rung_dev uint8 [G][M] (nullable); perm_dev int32 [G][M] (required):
 *   perm[g][pos] = row at sorted position pos; thresholds_dev float
 *   [G][n_rungs - 1] (nullable).  Errors: ARG, HIP. */
int scmp_classify_rows(scmp_plan_t plan, const float* metric_dev, int G, int M, float* ghat_dev,
                       uint8_t* rung_dev, int32_t* perm_dev, float* thresholds_dev, void* stream);

/* Workspace scmp_matmul needs for these sizes (0 for BITSERIAL).  The
 * MFMA path keeps there, per call, the row side encoded at each row's
 * length (two 16-bit window codes per row pair and index), each row tile's
 * largest half-window per index, the per-part or per-chunk n0 sums, the
 * weight side's table offsets (two per column pair and index), index-major
 * copies of both for single-segment plans, sorted-row ids and scales, and
 * a work counter.  GATHER keeps one count table per (band, rung) length,
 * (2^p + 1)^2 uint16 each.  Errors: ARG, PLAN_MISMATCH. */
int scmp_matmul_workspace_bytes(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N,
                                size_t* bytes);

/* The SC matmul C = A x B^T ([PAYN] Key designs 1 and 3; [KBAND] "How the
 * banding works").  Rows of A are taken bucket by bucket in sorted order
 * (rung k = sorted positions [cut_k, cut_(k+1)), all at one length), so
 * every tile runs one stream length.  Row i of rung k contracts index d of
 * band b at L = L[b][k]; A's stream is the L-prefix of its table row and B's
 * stream is generated by two counters gated by A's bits (C-BSG), and the
 * XNOR count is exact.  Per chunk c (the whole row when chunk_d is 0) the
 * decode is s^A_ic s^B_jc q^2 (2 count_ijc - L_c |c|) / L_c, summed over
 * chunks in float32 ([PAYN] Key design 1, decode equation).
 * A unipolar plan (scmp_mode) counts AND instead of XNOR: per index the
 * count is sign(x_A) sign(x_B) cum[u_B][n1_A], and the chunk decode is
 * s^A_ic s^B_jc q^2 count_ijc / L_c.  It runs on the bit-serial kernel or
 * on the one-block-per-tile matrix-core kernel (AUTO and MFMA select it;
 * MFMA_PERSISTENT returns UNSUPPORTED).
 *   qA_dev int8 [G][M][D], sA_dev float [G][M][n_chunks],
 *   permA_dev int32 [G][M] (NULL only for one rung: identity order),
 *   qB_dev int8 [G][N][D], sB_dev float [G][N][n_chunks],
 *   packedB_dev uint32 [G][N][D][ceil(Lmax/32)] (needed by BITSERIAL only),
 *   counts_dev int32 [G][M][N][n_bands] (nullable): per-band XNOR counts
 *   (unipolar: per-band sums of the signed AND counts),
 *   C_dev float (nullable): decoded output at original row order,
 *   workspace_dev / workspace_bytes: scratch of at least
 *   scmp_matmul_workspace_bytes (ignored by BITSERIAL); calls that share a
 *   workspace must be ordered on one stream.
 * At least one of counts_dev and C_dev must be given; ldc >= N.
 * Errors: ARG, PLAN_MISMATCH (table vs plan), WORKSPACE (too small),
 * UNSUPPORTED (MFMA_PERSISTENT with a unipolar plan; a range-MP plan,
 * which runs through scmp_matmul_range), HIP. */
int scmp_matmul(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N,
                const int8_t* qA_dev, const float* sA_dev, const int32_t* permA_dev,
                const int8_t* qB_dev, const uint32_t* packedB_dev, const float* sB_dev,
                int32_t* counts_dev, float* C_dev, int64_t ldc, int64_t batch_stride_c,
                void* workspace_dev, size_t workspace_bytes, void* stream);

/* scmp_matmul for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * product, kernels and results as scmp_matmul, with the scratch memory
 * taken from a static device array of the library (64 MiB per device,
 * held until the process ends) instead of a caller workspace.  The call
 * allocates nothing.  Every call on one device shares that device's array,
 * so calls that overlap on one device (other streams, other threads) race
 * and must be ordered by the caller; the array keeps the last call's
 * contents, and the kernels clear what must start at zero.  Arguments as
 * scmp_matmul, without the workspace.
 * Errors: as scmp_matmul; WORKSPACE when the sizes need more scratch than
 * 64 MiB (scmp_matmul_workspace_bytes tells), nothing launched. */
int scmp_matmul_noalloc(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N,
                        const int8_t* qA_dev, const float* sA_dev, const int32_t* permA_dev,
                        const int8_t* qB_dev, const uint32_t* packedB_dev, const float* sB_dev,
                        int32_t* counts_dev, float* C_dev, int64_t ldc, int64_t batch_stride_c, void* stream);

/* scmp_matmul with a bias added to every row of C: C_ij = (decode as
 * above) + bias_j.  With chunk_d = 64 and one length L this is the
 * head-aligned SC compensator of [VIT] (its head-aligned compensator
 * section): x split into heads of 64 columns, one SC linear per head
 * (per-row scales over the head's columns on both operands, the same Sobol
 * table), the heads' outputs summed and the bias added ([PAYN] Key design
 * 4, the compensation layer W_b x + b_b as an SC linear).
 *   bias_dev float [G][N] (required); other arguments as scmp_matmul.
 * Errors: as scmp_matmul; ARG when bias_dev is NULL. */
int scmp_matmul_bias(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N,
                     const int8_t* qA_dev, const float* sA_dev, const int32_t* permA_dev,
                     const int8_t* qB_dev, const uint32_t* packedB_dev, const float* sB_dev,
                     const float* bias_dev, int32_t* counts_dev, float* C_dev, int64_t ldc,
                     int64_t batch_stride_c, void* workspace_dev, size_t workspace_bytes, void* stream);

/* scmp_matmul with one stream length per group instead of per row: every
 * row of group g runs rung group_rung[g] of the plan's ladder (values past
 * the last rung clamp to it), in original row order.  This is the per-head
 * fixed mixed precision on QK of [VIT] (mixed-precision flag table: QK
 * levels and head fractions, head metric |Q_h|.amax): with G = images x
 * heads, each head's scores Q_h K_h^T all run at the head's length ([PAYN]
 * Key design 3, one L per output row).  The plan's row cuts and fractions
 * are not used here (they rank the heads, see scmp_group_max).  The
 * workspace size is scmp_matmul_workspace_bytes for the same plan, algo
 * and sizes (it covers both row orders).
 *   group_rung_dev uint8 [G] (required); no row permutation; other
 *   arguments as scmp_matmul.
 * Errors: as scmp_matmul; ARG when group_rung_dev is NULL. */
int scmp_matmul_group_rungs(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N,
                            const int8_t* qA_dev, const float* sA_dev, const int8_t* qB_dev,
                            const uint32_t* packedB_dev, const float* sB_dev, const uint8_t* group_rung_dev,
                            int32_t* counts_dev, float* C_dev, int64_t ldc, int64_t batch_stride_c,
                            void* workspace_dev, size_t workspace_bytes, void* stream);

/* Largest value of each group: out_dev[g] = max_i in_dev[g][i] (float32;
 * NaN values are skipped; -inf when all are NaN).  Applied to the row metrics
 * of scmp_quantize_encode over a head's rows it gives the per-head QK
 * metric |Q_h|.amax of [VIT] (mixed-precision flag table); ranking those
 * per image with scmp_classify_rows (M = heads) gives the head rungs.
 *   in_dev float [G][M], out_dev float [G]; M >= 1 when G > 0.
 * Errors: ARG, HIP. */
int scmp_group_max(const float* in_dev, int G, int M, float* out_dev, void* stream);

/* Range-based per-weight-group MP, the weight side's classification
 * ([VIT] mixed-precision flag table: range MP, its two levels and the
 * normalised range threshold, a higher threshold putting more groups at low
 * precision; [KBAND] "Guards": no contraction-axis dispatch).  W's rows
 * (the output columns of C = X W^T) form groups of range_group consecutive
 * rows (the last may be short); a group's range is max - min of its float32
 * weights over all D columns, normalised by the largest group range
 * (float32; 0 when that is 0).  Groups whose normalised range is below
 * range_threshold take levels[1], the others levels[0].  Weights are static,
 * so this runs once when a layer is loaded.
 *   W_dev float [N][D] with row stride w_row_stride (elements, >= D);
 *   norm_dev float [n_groups] (nullable), level_dev uint8 [n_groups]
 *   (nullable); cols_dev int32 [N] (required): the W rows of level 0 in
 *   order, then those of level 1; n_per_level: host int[2], the number of
 *   rows of each level.  Synchronises `stream` (the counts are read back).
 * Errors: ARG (plan without range_mp, sizes), HIP. */
int scmp_range_classify(scmp_plan_t plan, const float* W_dev, int N, int D, int64_t w_row_stride,
                        float* norm_dev, uint8_t* level_dev, int32_t* cols_dev, int* n_per_level,
                        void* stream);

/* Row gather: dst_dev[g][i] = src_dev[g][idx_dev[i]] for rows of row_bytes
 * bytes, g < G, i < n_idx, with src holding n_src rows per g.  Used to
 * store a weight side (qB, sB, packed streams) in the level order of
 * scmp_range_classify.  Indices outside [0, n_src) give zero rows.
 * Errors: ARG, HIP. */
int scmp_gather_rows(const void* src_dev, int G, int n_src, size_t row_bytes, const int32_t* idx_dev, int n_idx,
                     void* dst_dev, void* stream);

/* The range-MP product for the weight rows of one level: every row of A
 * runs at L = levels[level] ([PAYN] Key design 3 with the length set by
 * the weight group) against the N compact weight rows qB / sB / packedB
 * (the level's rows gathered in scmp_range_classify order), and compact
 * column j is written to C column cols_dev[j] (writes outside [0, ldc) are
 * dropped).  Two calls, one per level, give the whole product.  The plan
 * must have range_mp set; rows are in original order (no permutation);
 * counts_dev, when given, is compact: int32 [G][M][N].  Other arguments,
 * workspace and errors as scmp_matmul (ARG when level is not 0 or 1). */
int scmp_matmul_range(scmp_table_t table, scmp_plan_t plan, int algo, int level, int G, int M, int N,
                      const int8_t* qA_dev, const float* sA_dev, const int8_t* qB_dev,
                      const uint32_t* packedB_dev, const float* sB_dev, const int32_t* cols_dev,
                      int32_t* counts_dev, float* C_dev, int64_t ldc, int64_t batch_stride_c,
                      void* workspace_dev, size_t workspace_bytes, void* stream);

/* Diagnostic: synchronise `stream` and return the multiply-accumulates the
 * last MFMA-path contraction with this workspace (scmp_matmul or one of
 * its variants above) issued on the matrix cores
 * (every step of every 128 x 128 tile: four MFMAs per wave, 32 x 32 x 64
 * fp4 MACs each).  The count follows from the data: a step is issued when
 * some row of the tile needs it, up to the tile's largest window at that
 * index, in blocks of 16 paired positions.  *macs receives all of them;
 * fp4_macs (may be NULL) receives the same number (every step is fp4).  Errors: ARG,
 * UNSUPPORTED (BITSERIAL), WORKSPACE, HIP. */
int scmp_matmul_issued_macs(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N,
                            const void* workspace_dev, size_t workspace_bytes, unsigned long long* macs,
                            unsigned long long* fp4_macs, void* stream);

/* Diagnostic: synchronise `stream` and return the multiply-accumulates
 * the exact count needed in the last MFMA-path contraction with this
 * workspace: per output element and contraction index, the bipolar
 * half-window ceil(|n1 - n0| / 2) of paired positions at the row's length
 * (a unipolar plan: the prefix n1), summed over every row, index and band
 * and multiplied by N ([PAYN] Key design 3: the SC cost follows the stream
 * lengths; with the paired windows it follows the windows).  Padding to the
 * tile's largest window and to 16-position blocks is not counted (see
 * scmp_matmul_issued_macs).  Errors: ARG, UNSUPPORTED (BITSERIAL, GATHER),
 * WORKSPACE (no matrix-core call recorded in it), HIP. */
int scmp_matmul_window_macs(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N,
                            const void* workspace_dev, size_t workspace_bytes, unsigned long long* macs,
                            void* stream);

/* Decode counts produced without chunk scales ([PAYN] Key design 1, decode
 * equation): C_ij = s^A_i s^B_j q^2 (2 count_ij - L_i D) / L_i with
 * L_i = L[0][rung_i]; for a unipolar plan C_ij = s^A_i s^B_j q^2 count_ij / L_i.  counts_dev int32 [G][M][N][1]; rung_dev uint8 [G][M]
 * (NULL only for one rung).  Errors: ARG, UNSUPPORTED (plan has chunk_d
 * or bands), HIP. */
int scmp_decode(scmp_plan_t plan, int G, int M, int N, const int32_t* counts_dev,
                const float* sA_dev, const float* sB_dev, const uint8_t* rung_dev, float* C_dev,
                int64_t ldc, int64_t batch_stride_c, void* stream);

/* Synchronise `stream`, return the device error flags raised since the last
 * call (bit 0: a non-finite input to scmp_quantize_encode or
 * scmp_classify_rows) and clear them.  Returns NONFINITE when bit 0 is set,
 * OK otherwise, HIP on a runtime failure. */
int scmp_error_flags(void* stream, int* flags_out);

#ifdef __cplusplus
}
#endif

#endif /* SCMP_H */

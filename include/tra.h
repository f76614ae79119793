/*
 * tra.h - C ABI of the Token Radius Attention (TRA) hot path for AMD Instinct
 * MI355X (gfx950).
 *
 * The method ("Token Radius Attention for Efficient Video Generation", summary
 * page, section 2 "Méthodologie": Intuition I, Intuition II, "Le Pipeline TRA")
 * gives every query token of a T x H x W latent video its own attention
 * support: the query's attention entropy sets a token budget, the budget sets a
 * spatial disk radius, the radius shrinks with temporal distance, and the
 * resulting token-level masks are turned into a block-sparse tile list that a
 * block-sparse attention kernel consumes.  The pages fix the shape of each step
 * but no constants; the constants arrive here through tra_params.
 *
 * Sources cited below:
 *   [TRA] "Token Radius Attention for Efficient Video Generation" (summary page)
 *   [BLOG] "Token Radius Attention视频生成里被忽略但值得关注的高效注意力思路"
 *         (post on fixed-radius token masks)
 *   [RADIAL] "AI视频生成革命！MIT领衔豪华天团让生成效率暴涨370%，成本直降4.4倍"
 *         (news page on Radial attention's static mask)
 *
 * Two calls form the path:
 *   tra_plan_create  entropy -> budget level -> radius table -> CSR tile lists
 *   tra_attention    block-sparse softmax attention with the exact per-token mask
 * and a dense warm-up variant measures the entropy on the full attention
 * (tra_dense_attention, then tra_plan_create_from_entropy).
 * A plan is reusable across calls whose Q/K/V have the plan's shape (the pages'
 * warm-up reuse: entropy is measured once and reused in later denoising steps).
 *
 * Conventions shared by every call:
 *   - Tensors q, k, v, o are DEVICE pointers to contiguous [B, heads, N, d]
 *     arrays, N = T*H*W, token n = (t*H + h)*W + w (frame, then row, then
 *     column), 16-byte aligned, all of the shape's dtype.  The caller owns them.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous on that stream except where noted.
 *   - Errors are reported by status code only; a failing call writes no
 *     output and *out stays NULL.  tra_last_error() gives a message for the
 *     last failure on the calling thread.  A failed allocation returns
 *     TRA_ERR_OOM, a failed kernel launch or runtime call TRA_ERR_HIP.
 *   - Fault injection (tests of the error paths): with the environment
 *     variable TRA_FAULT=alloc[:n] the n-th device or pinned-host allocation
 *     (default the first) of each call fails as if out of memory; with
 *     TRA_FAULT=launch[:n] the n-th kernel launch of each call fails (the
 *     kernel is not launched).
 *   - Supported on the device: dtype TRA_BF16 with head_dim 64 or 128 (bf16
 *     matrix cores), dtype TRA_F32 with head_dim 64 or 128 (fp32 vector path),
 *     8 x 8 tiles (tile_h = tile_w = 8).  T, H, W <= 32767;
 *     B*heads*T*H*W < 2^31; for TRA_BF16 one head's K (T*H*W*head_dim*2 bytes)
 *     below 2^31.  Larger shapes fail with TRA_ERR_SHAPE.  The radius table's
 *     active entries plus two words per level row must fit 64 KB (the
 *     tile-list kernel stages them in LDS); larger tables fail with
 *     TRA_ERR_INVALID_ARG.
 */
#ifndef TRA_H
#define TRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TRA_OK = 0,
  TRA_ERR_INVALID_ARG = 1,   /* bad parameter value or NULL pointer            */
  TRA_ERR_SHAPE = 2,         /* unsupported or inconsistent shape              */
  TRA_ERR_DTYPE = 3,         /* unsupported dtype / head_dim combination        */
  TRA_ERR_PLAN_MISMATCH = 4, /* tensors do not match the plan's shape          */
  TRA_ERR_OOM = 5,           /* device or host allocation failed               */
  TRA_ERR_OVERFLOW = 6,      /* a count exceeds the 32-bit index range         */
  TRA_ERR_HIP = 7,           /* a HIP runtime call or kernel launch failed     */
  TRA_ERR_PLAN_INVALID = 8   /* the plan's last build failed: rebuild it first  */
} tra_status;

typedef enum { TRA_F32 = 0, TRA_BF16 = 1 } tra_dtype;

/* Problem shape.  B batch, heads, T x H x W latent grid, head_dim d. */
typedef struct {
  int32_t B, heads, T, H, W, head_dim;
  int32_t dtype; /* tra_dtype */
} tra_shape;

/*
 * Method constants.
 *   a, c            log-linear entropy -> budget map: ln B = a*H_i + c.  The
 *                   summary page's analytic map B ~ tau*exp(H_i) (Intuition I)
 *                   is a = 1, c = ln tau.
 *   budget_min/max  clamp of the token budget, in tokens (> 0, min <= max).
 *   levels_per_nat  budget quantisation q: level k_i = floor(q*(a*H_i + c)),
 *                   clamped to [ceil(q ln budget_min), floor(q ln budget_max)];
 *                   the quantised budget is exp(k_i/q).
 *   decay           phi in (0, 1]: radius at temporal distance delta is
 *                   r0 * phi^delta (the pages' phi(delta) = exp(-gamma*delta),
 *                   phi = exp(-gamma)).
 *   pool_h, pool_w  key pooling rectangle inside a frame (entropy is taken over
 *                   the mean-pooled keys, ragged rectangles weighted by size).
 *   tile_h, tile_w  query/key tile inside a frame for the block-sparse lists.
 *   radius_override < 0: off.  >= 0: every query uses r0 = radius_override
 *                   (entropy is skipped and every exported level is -1).
 */
typedef struct {
  double a, c, budget_min, budget_max, decay, radius_override;
  int32_t levels_per_nat, pool_h, pool_w, tile_h, tile_w;
  int32_t generator;      /* tra_generator */
  int32_t vote_threshold; /* >= 1: a key tile is listed for a query tile when at
                             least this many of their (query, key) pairs are
                             retained ([TRA] section 2, token voting); 1 = any */
  int32_t block_mask;     /* 0: exact per-token mask inside listed tiles;
                             1: block-only mask, every key of a listed tile
                             (the block-sparse execution the pages feed) */
  int32_t regroup;        /* 0: each 32-query wave of the bf16 attention kernel
                             takes half of one 8 x 8 query tile; 1: the queries
                             of each group of 2 x 2 query tiles are sorted by
                             budget level (ties in raster order within the
                             group) and dealt to the waves in that order, so
                             that a wave's queries have nearly one radius ([TRA] section
                             2, "Exécution Efficace", tile-major layout, read
                             as query regrouping by level).  The tile lists and
                             the retained pairs are the same either way.  bf16
                             only, with the exact mask (block_mask 0) and
                             vote_threshold 1, which define the keys per
                             query rather than per query tile. */
  int32_t group_rows;     /* query-tile rows of the bf16 attention kernel's
                             unit of work, a group of group_rows x 2 query
                             tiles of one frame ([TRA] section 2, "Exécution
                             Efficace": block-sparse execution, key tiles
                             loaded once per group): 2 or 3, or 0 to choose
                             (3 unless that leaves more tile rows of the grid
                             uncovered than 2, regroup is set, or the
                             generator is the 1-D window).  Results are the
                             same for either shape; regroup takes 2. */
} tra_params;

/*
 * Plan generators: which keys a query retains.  All feed the same tile lists
 * and attention kernels.
 *   TRA_GEN_ENTROPY_DISK  the method: per-query budget from the entropy ->
 *                         Euclidean disk per frame with radius r0*phi^delta
 *                         (or the fixed r0 = radius_override when >= 0).
 *   TRA_GEN_MANHATTAN     fixed-radius baseline of the generic radius post
 *                         ([BLOG] section 5.2): keep j iff |t_i-t_j| + |h_i-h_j|
 *                         + |w_i-w_j| <= floor(radius_override); the radius
 *                         table then holds L1 radii floor(R) - delta.
 *   TRA_GEN_RADIAL        Radial attention's static mask ([RADIAL], a spatial
 *                         window that shrinks with temporal distance), read as
 *                         a disk whose area halves per octave band of delta:
 *                         R2[delta] = floor(radius_override^2 / 2^b), b = 0 for
 *                         delta = 0 and floor(log2 delta) + 1 otherwise; frames
 *                         with R2 < 1 are inactive.
 *   TRA_GEN_WINDOW_1D     the 1-D distance ablation ([TRA] section 4): keep j
 *                         iff |n_i - n_j| <= rho along the raster token order,
 *                         rho = floor((B_i - 1)/2) for the query's quantised
 *                         budget B_i (floor(radius_override) when >= 0), so the
 *                         window of 2 rho + 1 tokens holds the budget; every
 *                         radius-table entry of a level is its rho.  Needs at
 *                         most 64 tile columns (W <= 512 with 8-wide tiles),
 *                         vote_threshold 1, and rho < 2^24.
 * The Manhattan and Radial generators need radius_override >= 0 and ignore the
 * entropy (every level is -1).
 */
typedef enum {
  TRA_GEN_ENTROPY_DISK = 0,
  TRA_GEN_MANHATTAN = 1,
  TRA_GEN_RADIAL = 2,
  TRA_GEN_WINDOW_1D = 3
} tra_generator;

typedef struct tra_plan tra_plan; /* opaque; owns its device buffers */

/* Sizes of a plan, all counts per whole plan. */
typedef struct {
  int64_t n_queries;    /* B*heads*N                                             */
  int64_t n_rows;       /* B*heads*n_qtiles: CSR rows, head-major                */
  int64_t nnz;          /* CSR entries (listed query-tile/key-tile pairs)        */
  int32_t n_qtiles;     /* tiles per head = T*ceil(H/tile_h)*ceil(W/tile_w)      */
  int32_t n_pool;       /* pooled keys per head = T*ceil(H/pool_h)*ceil(W/pool_w)*/
  int32_t n_levels;     /* rows of the radius table                              */
  int32_t k_lo;         /* level of table row 0 (-1 under radius_override)       */
  int32_t T;            /* columns of the radius table                           */
  int32_t max_row_len;  /* longest CSR row                                       */
  int32_t group_rows;   /* bf16: query-tile rows per attention group (2 or 3)  */
} tra_plan_info;

/*
 * Host-only validation of a shape and parameter set (no GPU needed).
 * Returns TRA_OK or the status tra_plan_create would fail with.
 */
tra_status tra_params_validate(const tra_shape* shape, const tra_params* params);

/*
 * Host-only radius table (step "budget -> radius", Intuition II and "Le
 * Pipeline TRA"): with S = sum_{delta=-(T-1)}^{T-1} phi^(2|delta|) (the budget
 * is spread over the disks of all frames) and r0^2(k) = exp(k/q)/(pi*S),
 *   R2[k - k_lo][delta] = floor(r0^2(k) * phi^(2*delta)),  delta = 0..T-1,
 * stored as -1 where delta >= 1 and the value is below 1 (frame inactive).
 * r2 receives n_levels*T int32 (host memory, row-major); r0sq, if not NULL,
 * n_levels doubles.  Query `*n_levels` first by passing r2 == NULL.
 */
tra_status tra_radius_table(const tra_shape* shape, const tra_params* params, int32_t* r2,
                            double* r0sq, int32_t* n_levels, int32_t* k_lo);

/*
 * Build a plan from q and k (steps entropy -> level -> radius -> tile lists;
 * [TRA] section 2: Intuition I for entropy -> budget, Intuition II for budget
 * -> radius shrinking with temporal distance, "Exécution Efficace" for the
 * token masks turned into block-sparse tile lists):
 *   Kbar_b = mean of the keys of pool rectangle b, rounded once to the dtype;
 *   H_i    = entropy of softmax_j(q_i . Kbar_{b(j)} / sqrt(d)) over all N keys;
 *   k_i    = clamped level of H_i;
 *   key tile Kb is listed for query tile Qa iff some query i in Qa retains some
 *   key j in Kb: R2[k_i][|t_i-t_j|] >= 0 and
 *   (h_i-h_j)^2 + (w_i-w_j)^2 <= R2[k_i][|t_i-t_j|].
 * The CSR's columns are ascending key-tile ids (tile id = (t*ceil(H/tile_h) +
 * h/tile_h)*ceil(W/tile_w) + w/tile_w) within each head.
 * bf16 plans without a vote threshold build only what the attention kernel
 * reads (levels, per-row runs and counts, and the merged lists of 2 x 2 query
 * tile groups, in a buffer sized at creation for the worst case): the build
 * is asynchronous on `stream`.  Their CSR is completed from the counts and
 * runs on first use by tra_plan_export (row_ptr / col_idx), tra_plan_stats
 * or tra_plan_get_info, which then synchronise.  Other plans (fp32, vote
 * threshold) build the CSR at once and synchronise `stream` once to size it.
 * The calls that copy plan data to the host (tra_plan_export,
 * tra_plan_export_groups, tra_plan_export_regroup, tra_plan_stats,
 * tra_plan_get_info) order themselves after the plan's latest build, on
 * whatever stream it ran; the kernel-launching calls (tra_attention,
 * tra_plan_drift) follow their own stream's order only.
 * An asynchronous rebuild and the attention calls that follow it can be
 * captured in a HIP graph (they launch kernels and record one event, nothing
 * else).  The plan's host-side state (its validity, whether its CSR is
 * complete) follows the calls the host makes, not graph replays: after a
 * replay that rebuilt the plan from other inputs, make an eager rebuild
 * before exporting the CSR.
 * *out receives the plan, which owns all its device memory (including the
 * scratch of tra_plan_stats and tra_plan_drift); on failure nothing is kept
 * and *out stays NULL.
 * Errors: TRA_ERR_INVALID_ARG / SHAPE / DTYPE for inputs the device path does
 * not take (see tra_params_validate), TRA_ERR_OOM, TRA_ERR_HIP,
 * TRA_ERR_OVERFLOW when the tile lists would hold 2^31 entries or more.
 */
tra_status tra_plan_create(const tra_shape* shape, const tra_params* params, const void* q,
                           const void* k, void* stream, tra_plan** out);

/*
 * Block-sparse attention with the plan's exact per-token mask ([TRA] section
 * 2, "Exécution Efficace": the block-sparse backend fed by the tile lists;
 * [BLOG] sections 4.1 and 9: scale 1/sqrt(d), masked keys excluded as -inf
 * before the softmax):
 *   O_i = sum_{j retained by i} softmax_j(q_i . k_j / sqrt(d)) v_j
 * q, k, v, o: device [B, heads, N, d] of the plan's dtype; o must not alias
 * q, k or v.  q and k may differ from the tensors the plan was built from (plan
 * reuse).  Only listed tiles are visited.  The self key is always retained, so
 * every row is well defined.  Asynchronous on `stream`; allocates nothing.
 * The C ABI sees only pointers: tensors of another shape or dtype than the
 * plan's cannot be detected here (call tra_plan_matches first, as the Python
 * binding does).  TRA_ERR_PLAN_INVALID if the plan's last rebuild failed.
 */
tra_status tra_attention(const tra_plan* plan, const void* q, const void* k, const void* v,
                         void* o, void* stream);

/*
 * Re-run the planning steps of tra_plan_create on new q and k into an existing
 * plan (the refresh of a warm-up step), reusing its device buffers; the tile
 * list buffer grows when needed.  The shape and parameters are the plan's.
 * Synchronises `stream` once, except for the asynchronous builds described
 * at tra_plan_create.  On failure the plan is marked invalid: every
 * call that reads it (attention, export, stats, drift) returns
 * TRA_ERR_PLAN_INVALID until a rebuild succeeds.
 */
tra_status tra_plan_rebuild(tra_plan* plan, const void* q, const void* k, void* stream);

/* TRA_OK if `shape` equals the plan's shape, else TRA_ERR_PLAN_MISMATCH.
 * tra_attention trusts its caller on shapes; bindings call this first. */
tra_status tra_plan_matches(const tra_plan* plan, const tra_shape* shape);

/* Sizes of the plan.  For a plan whose CSR is completed on first use (see
 * tra_plan_create) this completes it on the null stream, after the plan's
 * last build, and synchronises. */
tra_status tra_plan_get_info(const tra_plan* plan, tra_plan_info* info);

/*
 * Copy plan contents to HOST memory (any pointer may be NULL to skip):
 *   levels   int16 [n_queries]            budget level k_i (-1 under override)
 *   entropy  float [n_queries]            H_i (0 under override)
 *   r2       int32 [n_levels*T]           radius table
 *   row_ptr  int32 [n_rows + 1]           CSR offsets (global over all heads)
 *   col_idx  int32 [nnz]                  key tile ids (per head)
 *   kbar     [B*heads*n_pool*head_dim] of the dtype: pooled keys, rectangle
 *            (t*ceil(H/pool_h) + r)*ceil(W/pool_w) + c in raster order (the
 *            plan stores the full rectangles first; export reorders)
 * Synchronises `stream`.
 */
tra_status tra_plan_export(const tra_plan* plan, int16_t* levels, float* entropy, int32_t* r2,
                           int32_t* row_ptr, int32_t* col_idx, void* kbar, void* stream);

/*
 * The bf16 attention kernel's unit of work (host copies; synchronises
 * `stream`): a group is group_rows x 2 query tiles of one frame (group_rows
 * from tra_plan_get_info; group id = (b*heads + head, frame, group row, group
 * column) in row-major order), walked over the
 * ascending union of their tile lists.  *n_groups and *n_entries receive the
 * counts (call with NULL arrays first); gptr/glen int32 [n_groups] the offset
 * and length of each group's list in glist; glist int32 [2*n_entries], entry
 * (frame | member << 16 | edge << 31, row0 | col0 << 16), member bit
 * 2*(tile row in group) + (tile column in group) set when that query tile
 * lists the key tile, edge set for a tile cut by the grid's bottom or right
 * edge.  TRA_ERR_DTYPE for fp32 plans (their kernel reads the CSR).
 */
tra_status tra_plan_export_groups(const tra_plan* plan, int64_t* n_groups, int64_t* n_entries, int32_t* gptr,
                                  int32_t* glen, int32_t* glist, void* stream);

/*
 * Query regrouping ([TRA] section 2, "Exécution Efficace"; plans created with
 * params.regroup = 1; host copy, synchronises `stream`): for each group, in
 * the order of tra_plan_export_groups, its 256 query positions as slots
 * (row * 16 + column inside the group's 16 x 16 positions) in the order the
 * attention kernel deals them to its waves, 32 per wave: ascending budget
 * level, ties by slot, positions outside the grid last.  perm: uint8
 * [n_groups * 256].  TRA_ERR_INVALID_ARG for a plan created without regroup
 * or a NULL argument.
 */
tra_status tra_plan_export_regroup(const tra_plan* plan, uint8_t* perm, void* stream);

/*
 * Exact pair counts of a plan (synchronises `stream`; counters live in the
 * plan, so nothing is allocated, and two stats or drift calls on one plan
 * must not overlap):
 *   retained  sum over queries of the keys each attends to (the FLOPs that
 *             count: 4*d per pair): the keys it retains; with vote_threshold
 *             > 1 only those inside its tile's listed tiles (the votes of the
 *             kept tiles); with block_mask, every key of the listed tiles
 *   listed    sum over CSR entries of (valid queries x valid keys) of the pair
 *             of tiles: the pairs a tile-granular kernel visits
 */
tra_status tra_plan_stats(const tra_plan* plan, int64_t* retained, int64_t* listed, void* stream);

/*
 * Plan drift (plans are reused across denoising steps, [TRA] section 2
 * "Reutilisation Inter-Etapes"): the number of queries whose budget level
 * would change if the plan were rebuilt from q and k.  Runs the pooling and
 * entropy steps on q and k into scratch memory the plan owns (nothing is
 * allocated per call; two stats or drift calls on one plan must not overlap)
 * and compares the levels with the plan's; the plan's tile lists and levels
 * are not modified.  Under radius_override every level is -1 and the drift is
 * 0.  Synchronises `stream`.
 */
tra_status tra_plan_drift(const tra_plan* plan, const void* q, const void* k, int64_t* changed,
                          void* stream);

/*
 * tra_plan_drift for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same count, computed in a static device buffer of the library instead of the
 * plan's scratch.  That buffer holds tra_drift_noalloc_max_bytes() bytes (32
 * MiB) per GPU, kept until the process ends; a plan whose drift needs more
 * (pooled keys plus 2 bytes per query, each part rounded to 256 bytes) is
 * refused with TRA_ERR_SHAPE.  Calls that overlap on one GPU share the buffer
 * and race: serialise them.  Must be called with the plan's device current.
 * Synchronises `stream`.
 */
tra_status tra_plan_drift_noalloc(const tra_plan* plan, const void* q, const void* k, int64_t* changed,
                                  void* stream);
size_t tra_drift_noalloc_max_bytes(void);

/*
 * Dense warm-up pass ([TRA] section 2, "Le Pipeline TRA", entropy-to-budget
 * step: the entropy is measured on the full attention of dense warm-up steps):
 *   O_i = sum_j softmax_j(q_i . k_j / sqrt(d)) v_j over all N keys of the head,
 *   H_i = -sum_j p_ij ln p_ij of that same softmax (when entropy != NULL).
 * q, k, v, o: device [B, heads, N, d] of the shape's dtype (same limits as
 * tra_plan_create); o must not alias q, k or v.  entropy: device float
 * [B*heads*N] or NULL (then only O is computed).  bf16 runs on matrix cores
 * with fp32 softmax and fp64 entropy sums; fp32 inputs use fp64 scores.
 * Asynchronous on `stream`; allocates nothing.
 */
tra_status tra_dense_attention(const tra_shape* shape, const void* q, const void* k, const void* v,
                               void* o, float* entropy, void* stream);

/*
 * Build a plan whose budget levels come from given per-query entropies
 * (device float [B*heads*N], e.g. those of tra_dense_attention) instead of
 * the pooled-key estimate: k_i = clamped level of entropy[i], then the same
 * radius table and tile lists as tra_plan_create.  The entropies are copied
 * into the plan (tra_plan_export returns them); the plan's pooled keys are
 * zero.  Under radius_override the entropies are ignored.  Synchronises
 * `stream` once.
 */
tra_status tra_plan_create_from_entropy(const tra_shape* shape, const tra_params* params,
                                        const float* entropy, void* stream, tra_plan** out);

/* tra_plan_rebuild with levels from given entropies (see
 * tra_plan_create_from_entropy).  Pooled keys keep their last values. */
tra_status tra_plan_rebuild_from_entropy(tra_plan* plan, const float* entropy, void* stream);

/*
 * Rebuild a plan from saved contents (checkpoint / resume of a plan that a
 * reuse schedule keeps across denoising steps: "Token Radius Attention for
 * Efficient Video Generation", summary page, section 2, "Reutilisation
 * Inter-Etapes").  All arrays are HOST memory, in tra_plan_export's layout:
 *   levels   int16 [B*heads*N]   budget level of each query (required); every
 *            value must lie in [k_lo, k_lo + n_levels - 1] of the radius
 *            table these params give, or be -1 under radius_override
 *   entropy  float [B*heads*N]   stored for export only (NULL: zeros)
 *   kbar     pooled keys [B*heads*n_pool*head_dim] of the dtype, stored for
 *            export and drift (NULL: zeros)
 * The radius table is recomputed from the params, and the tile lists (CSR,
 * votes, group lists) are built from the levels by the same kernels as
 * tra_plan_create, so a plan exported and imported with the same shape and
 * params attends exactly like the original.  TRA_ERR_INVALID_ARG (nothing
 * allocated) for a NULL levels array or a level outside the table; the
 * usual statuses otherwise.  Synchronises `stream`.
 */
tra_status tra_plan_import(const tra_shape* shape, const tra_params* params, const int16_t* levels,
                           const float* entropy, const void* kbar, void* stream, tra_plan** out);

/* Frees the plan.  hipFree waits for the device's outstanding work before it
 * releases memory, so destroying a plan synchronises the device. */
void tra_plan_destroy(tra_plan* plan);

/*
 * Reuse schedule across denoising steps ([TRA] section 2, "Le Pipeline TRA":
 * entropy measured during dense warm-up steps, then reused by the sparse
 * steps that follow, relying on the stability of the entropy across steps).
 * One call per denoising step, in order; each computes that step's attention
 * output o from its q, k, v (device [B, heads, N, d] of the shape's dtype):
 *   step < warmup_steps - 1        TRA_STEP_DENSE: dense attention
 *   step == warmup_steps - 1       TRA_STEP_DENSE_REPLAN: dense attention with
 *                                  exact entropies, plan built from them
 *   later                          TRA_STEP_SPARSE: sparse attention under the
 *                                  plan, unless a refresh is due, which runs as
 *                                  TRA_STEP_DENSE_REPLAN instead
 * A refresh is due after refresh_every sparse steps (0 = never), and on the
 * step after a sparse step whose drift exceeded drift_threshold * B*heads*N
 * queries.  Drift (tracked when drift_threshold >= 0) is the number of queries
 * whose pooled-key budget level differs from the level the pooled estimate
 * gave on the inputs of the last re-plan step; measuring it costs one pooling
 * and entropy pass and one stream synchronisation per sparse step.
 * The schedule owns its plan and buffers; tra_schedule_step returns the
 * step's mode and drift (-1 if not measured) in *info (may be NULL).
 */
typedef struct {
  int32_t warmup_steps;   /* >= 1 */
  int32_t refresh_every;  /* >= 0 */
  double drift_threshold; /* fraction of queries; < 0: no drift tracking */
} tra_schedule_params;

typedef enum { TRA_STEP_DENSE = 0, TRA_STEP_DENSE_REPLAN = 1, TRA_STEP_SPARSE = 2 } tra_step_mode;

typedef struct {
  int32_t step, mode; /* mode: tra_step_mode */
  int64_t drift;
} tra_step_info;

typedef struct tra_schedule tra_schedule;

tra_status tra_schedule_create(const tra_shape* shape, const tra_params* params, const tra_schedule_params* sp,
                               tra_schedule** out);
tra_status tra_schedule_step(tra_schedule* sched, const void* q, const void* k, const void* v, void* o,
                             void* stream, tra_step_info* info);
/* The schedule's current plan (borrowed; NULL before the first re-plan step). */
tra_status tra_schedule_plan(const tra_schedule* sched, const tra_plan** plan);
void tra_schedule_destroy(tra_schedule* sched);

const char* tra_status_string(tra_status s);

/* Message describing the last failing call on this thread ("" if none). */
const char* tra_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TRA_H */

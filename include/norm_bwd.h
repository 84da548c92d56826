/*
 * norm_bwd.h -- C ABI of the LayerNorm / RMSNorm backward library for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed. "Norm backward in Triton -- the dγ/dβ reduction",
 * section "The gradients (the half-page you reverse)": for every row r of
 * x[M, N] with the forward's saved per-row statistics mean[r] and
 * rstd[r] = 1/sigma_r,
 *
 *     xhat  = (x - mean) * rstd          (RMSNorm: xhat = x * rstd)
 *     dyhat = dy * gamma
 *     dx    = rstd * (dyhat - mean_j(dyhat) - xhat * mean_j(dyhat * xhat))
 *             (RMSNorm has no mean_j(dyhat) term)
 *     dgamma[j] = sum over all rows of dy * xhat
 *     dbeta[j]  = sum over all rows of dy
 *
 * How. The per-feature sums run over the token axis, the same axis dx is
 * parallel over ("Norm & activation backward", section "Half two: dγ and dβ
 * reduce across the whole batch", its strategy table). This library takes the
 * deterministic two-pass route from that table: kernel A computes dx and, for
 * each of G disjoint row groups (group g = the rows r with r mod G == g; on
 * the two-rows-per-wave layout, the adjacent row pairs (2q, 2q + 1) with
 * q mod G == g), the group's partial dgamma/dbeta in registers, stored once
 * into a caller-provided fp32 workspace[G, N]; kernel B sums the groups in
 * one fixed order. There are
 * no atomics, so dx, dgamma and dbeta are bitwise identical across calls with
 * equal arguments (same kind, M, N, dtypes, groups, and pointer alignment
 * class) on the same device type. The group count never depends on the GPU's
 * compute-unit count.
 *
 * Memory. Every pointer is a device pointer owned by the caller. The library
 * allocates nothing. Tensors are dense row-major: x, dy, dx are [M, N] with
 * row stride N elements; gamma, dgamma, dbeta are [N]; mean, rstd are fp32 [M].
 * Outputs must not overlap any input, each other, or the workspace.
 *
 * Streams and errors. All calls that launch work are asynchronous on
 * `stream` (a hipStream_t passed as void*, NULL = the default stream); results
 * are valid once the caller synchronises that stream. Arguments are checked
 * on the host before anything is launched: on a non-zero status nothing was
 * enqueued, except NORM_BWD_ERR_HIP, which reports a failed launch.
 * Before launching, the library reads (and so clears) the calling thread's
 * pending HIP error with hipGetLastError, so that a launch failure it reports
 * is its own. norm_bwd_last_error() gives a message for the calling thread's
 * last failure. Nothing aborts, and nothing prints unless the environment
 * variable NORM_BWD_LOG is set to a non-empty value other than "0" when the
 * first failure occurs: then every failing call also writes its message to
 * stderr.
 */
#ifndef NORM_BWD_H
#define NORM_BWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define NORM_BWD_OK 0
#define NORM_BWD_ERR_INVALID_ARG 1   /* NULL pointer, negative size, bad eps, overlap, misaligned plan */
#define NORM_BWD_ERR_UNSUPPORTED 2   /* dtype code, dtype pair, or N beyond the fused path's limit */
#define NORM_BWD_ERR_WORKSPACE 3     /* workspace NULL or smaller than required */
#define NORM_BWD_ERR_HIP 4           /* a HIP launch failed (hipGetLastError) */

/* Element types (x, dy, gamma, dx use io_dtype; dgamma, dbeta use wgrad_dtype). */
#define NORM_BWD_F32 0
#define NORM_BWD_F16 1   /* IEEE binary16 */
#define NORM_BWD_BF16 2  /* bfloat16 */

/* Normalisation kinds. */
#define NORM_BWD_LAYERNORM 0
#define NORM_BWD_RMSNORM 1

/*
 * Largest N the fused path takes (rows held in registers). "Aligned" means N
 * is a multiple of 16 / element size and x, dy, gamma, dx start on 16-byte
 * boundaries; other rows use one element per lane. Wider rows (up to
 * INT32_MAX) take the wide-row path in norm_bwd_layernorm, norm_bwd_rmsnorm,
 * norm_bwd_ex (automatic groups) and the forward: one workgroup per row
 * computes dx or y, holding the row in its registers when it fits (aligned
 * rows up to 65536 16-bit or 32768 fp32 elements) and otherwise streaming it
 * in chunks, and the column walk (see norm_bwd_wgrad) forms dgamma/dbeta,
 * with no workspace beyond the recomputed statistics (4 or 8 bytes per row)
 * in recompute mode. The
 * explicit-plan entry points (norm_bwd_make_plan, norm_bwd_execute*) cover
 * the fused path only and return NORM_BWD_ERR_UNSUPPORTED beyond it.
 */
#define NORM_BWD_MAX_N_16BIT 32768          /* fp16/bf16, aligned, dbeta NULL */
#define NORM_BWD_MAX_N_16BIT_DBETA 16384    /* fp16/bf16, aligned, dbeta requested */
#define NORM_BWD_MAX_N_F32 16384            /* fp32, aligned */
#define NORM_BWD_MAX_N_UNALIGNED 8192

/*
 * LayerNorm backward ("Norm backward in Triton -- the dγ/dβ reduction",
 * "The gradients"; the same dx and dgamma/dbeta are the Phobos tutorial
 * "05: Layer norm" kernels ln_bwd_dx and ln_bwd_dwdb).
 *
 *   x, dy, gamma   [M,N], [M,N], [N] in io_dtype (read)
 *   mean, rstd     fp32 [M], the forward's saved statistics (read); or both
 *                  NULL: recompute mode, in which each row's statistics are
 *                  computed from x in fp32 as the forward does (mean =
 *                  sum(x)/N, then var = sum((x - mean)^2)/N, rstd =
 *                  1/sqrt(var + eps)) before the gradient. This follows the
 *                  option of recomputing sigma on chip rather than reading
 *                  it ("Norm & activation backward", "Half one"). Exactly
 *                  one of them NULL is NORM_BWD_ERR_INVALID_ARG.
 *   M, N           rows and features, >= 0. M = 0 writes zeros to dgamma and
 *                  dbeta (the empty sum); N = 0 does nothing.
 *   io_dtype       NORM_BWD_F32 / F16 / BF16
 *   wgrad_dtype    NORM_BWD_F32 or io_dtype: dgamma/dbeta are accumulated in
 *                  fp32 and rounded (to nearest even) once at the end
 *   eps            the forward's epsilon; checked (finite, >= 0); used only
 *                  in recompute mode (a saved rstd already contains it).
 *                  With eps = 0 a constant row has rstd = inf, and its dx is
 *                  not finite, as the formula gives.
 *   dx             [M,N] io_dtype (written, rounded to nearest even)
 *   dgamma         [N] wgrad_dtype (written)
 *   dbeta          [N] wgrad_dtype (written), or NULL to skip it
 *   workspace      at least norm_bwd_workspace_bytes(NORM_BWD_LAYERNORM, M, N,
 *                  io_dtype, dbeta != NULL) bytes of device memory, 16-byte
 *                  aligned; its prior contents are never read
 *   stream         hipStream_t or NULL
 * Returns a status code.
 */
int norm_bwd_layernorm(const void *x, const void *dy, const void *gamma,
                       const float *mean, const float *rstd, int64_t M,
                       int64_t N, int io_dtype, int wgrad_dtype, float eps,
                       void *dx, void *dgamma, void *dbeta, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * RMSNorm backward ("Norm backward in Triton", "The gradients": no mean, so
 * xhat = x * rstd and dx loses the mean_j(dyhat) term). Same arguments as
 * norm_bwd_layernorm without `mean`. dbeta may be NULL (RMSNorm has no bias);
 * when given it receives the column sum of dy, which does not depend on the
 * normalisation. rstd = NULL selects recompute mode (rstd = 1/sqrt(sum(x^2)/N
 * + eps) per row, from x).
 */
int norm_bwd_rmsnorm(const void *x, const void *dy, const void *gamma,
                     const float *rstd, int64_t M, int64_t N, int io_dtype,
                     int wgrad_dtype, float eps, void *dx, void *dgamma,
                     void *dbeta, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * Workspace size in bytes that norm_bwd_layernorm / norm_bwd_rmsnorm (and
 * norm_bwd_ex with automatic groups) need for (kind, M, N, io_dtype), in
 * either statistics mode: on the fused path the larger of the two automatic
 * plans' groups * N * 4 bytes per gradient vector (two vectors when
 * with_dbeta != 0), and never less than the wide-row path's recomputed
 * statistics (M * 4 bytes, LayerNorm M * 8). Returns (size_t)-1 for invalid
 * arguments, including M * N * 4 above 2^62 (which every entry point
 * rejects). Host-only; launches nothing.
 */
size_t norm_bwd_workspace_bytes(int kind, int64_t M, int64_t N, int io_dtype,
                                int with_dbeta);

/*
 * Extended backward: everything norm_bwd_layernorm / norm_bwd_rmsnorm do, plus
 * row strides, an explicit group count and accumulation into existing weight
 * gradients. Accumulating is what a training step needs when several
 * micro-batches (or a parameter shared between layers) add into one gradient
 * buffer ("Matmul backward in Triton", "Accumulate into the grad buffer, never
 * overwrite"); the row stride follows the row-stride argument of the
 * kernels in "Norm backward in Triton" (stride_row).
 *
 *   kind, io_dtype, wgrad_dtype, M, N, eps, gamma, mean, rstd, dgamma, dbeta,
 *   workspace, workspace_bytes, stream: as for norm_bwd_layernorm (mean is
 *   ignored for RMSNorm; mean = rstd = NULL selects recompute mode).
 *   flags     NORM_BWD_ACCUMULATE: dgamma[j] (and dbeta[j]) become
 *             old + (this call's sum), added in fp32 after the fixed-order
 *             group sum and rounded once to wgrad_dtype; M = 0 leaves them
 *             unchanged. Without it they are overwritten. Other bits:
 *             NORM_BWD_ERR_INVALID_ARG.
 *   groups    0 = automatic (the workspace must then hold
 *             norm_bwd_workspace_bytes(kind, M, N, io_dtype, dbeta != NULL)),
 *             else as norm_bwd_make_plan (the workspace must hold
 *             norm_bwd_make_plan(kind, M, N, io_dtype, dbeta != NULL,
 *             groups).workspace_bytes)
 *   ldx, lddy, lddx  row strides of x, dy and dx in elements (0 = N, else
 *             >= N). Row r of x starts at x + r * ldx. Elements between rows
 *             are neither read nor written. 16-byte vector access is used only
 *             when every row start is 16-byte aligned; otherwise one element
 *             per lane (same results up to summation order).
 *   Outputs may not overlap any input's or output's span (first row start to
 *   last row end). Returns a status code; checks as for the other entry
 *   points.
 */
#define NORM_BWD_ACCUMULATE 1u

typedef struct norm_bwd_args {
    int32_t kind;
    int32_t io_dtype;
    int32_t wgrad_dtype;
    uint32_t flags;
    int64_t M, N;
    int64_t groups;
    const void *x;
    int64_t ldx;
    const void *dy;
    int64_t lddy;
    const void *gamma;
    const float *mean;
    const float *rstd;
    void *dx;
    int64_t lddx;
    void *dgamma;
    void *dbeta;
    void *workspace;
    size_t workspace_bytes;
    void *stream;
    float eps;
    int32_t reserved;  /* must be 0 */
} norm_bwd_args_t;

int norm_bwd_ex(const norm_bwd_args_t *args);

/*
 * norm_bwd_ex for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, results and checks, with the workspace taken from a
 * static array of NORM_BWD_STATIC_SCRATCH_BYTES in the library's device code
 * instead of args->workspace. Nothing is allocated by this call, by the
 * library or by any routine it calls.
 *
 *   args      as for norm_bwd_ex, except that args->workspace must be NULL
 *             and args->workspace_bytes 0 (else NORM_BWD_ERR_INVALID_ARG).
 *   The problem's workspace (norm_bwd_workspace_bytes for automatic groups,
 *   norm_bwd_make_plan(...).workspace_bytes for explicit groups, as for
 *   norm_bwd_ex) must fit in NORM_BWD_STATIC_SCRATCH_BYTES, else
 *   NORM_BWD_ERR_WORKSPACE, with nothing launched.
 *   The stream must belong to the calling thread's current device
 *   (NORM_BWD_ERR_INVALID_ARG otherwise); NULL is that device's default
 *   stream.
 * Each device holds one copy of the array, from the first call on it until
 * the process ends. Calls on one device share it: two calls whose work
 * overlaps in time on one device (on different streams, or from different
 * threads without ordering) race on it and their results are undefined.
 * Calls ordered on one stream are safe; each call writes every byte of the
 * workspace it reads, so no state carries over between calls.
 */
#define NORM_BWD_STATIC_SCRATCH_BYTES (32u << 20)   /* 32 MiB per device */

int norm_bwd_ex_static(const norm_bwd_args_t *args);

/*
 * Weight gradients alone, by a column walk: dgamma[j] = sum over rows of
 * dy * xhat (and dbeta[j] = sum of dy) without dx and without a workspace.
 * Each workgroup owns a tile of adjacent columns and walks all M rows, as the
 * Phobos tutorial's ln_bwd_dwdb does ("05: Layer norm"), so no two workgroups
 * write the same column. For callers that need only the weight gradients; it
 * reads x and dy once more where the fused path reads them once for dx too.
 *
 *   kind, x, dy, mean, rstd, M, N, io_dtype, wgrad_dtype, dgamma, dbeta as for
 *   norm_bwd_layernorm (contiguous [M,N]; the saved statistics are required;
 *   dbeta may be NULL). Any N up to INT32_MAX (no register-resident rows).
 *   flags   NORM_BWD_ACCUMULATE: old + sum, as for norm_bwd_ex.
 * The summation order depends on M, N and io_dtype only (reproducible), and
 * differs from the fused path's. Returns a status code.
 */
int norm_bwd_wgrad(int kind, const void *x, const void *dy, const float *mean,
                   const float *rstd, int64_t M, int64_t N, int io_dtype,
                   int wgrad_dtype, void *dgamma, void *dbeta, unsigned flags,
                   void *stream);

/*
 * (Declared above.) norm_bwd_workspace_bytes returns enough for the automatic
 * plan of either statistics mode: LayerNorm in recompute mode plans more row
 * groups on one row per wave (a second workgroup per compute unit hides its
 * second exchange per row), so for LayerNorm it is max(saved-statistics
 * plan, recompute plan).
 */

/*
 * An execution plan: the row grouping and the launch geometry of kernel A.
 * Produced by norm_bwd_make_plan; a caller may change `groups` (then call
 * norm_bwd_make_plan again with it) or the geometry fields for tuning, and
 * norm_bwd_execute re-validates every field. Results depend on groups,
 * rows_in_flight and rows_per_wave (dgamma/dbeta order) and on vec, chunks,
 * waves_per_row, rows_per_wave (order of the in-row sums), never on the
 * device.
 *
 * Two lane layouts. rows_per_wave = 1: a row is split over waves_per_row
 * waves of 64 lanes, each lane holding chunks vectors of vec elements.
 * rows_per_wave = 2 (16-byte vectors only, waves_per_row = 1, chunks 1 or
 * 3, N = 32 * vec * chunks exactly): rows go in adjacent pairs (2q, 2q + 1),
 * group g is the pairs with q mod groups == g (groups at most ceil(M / 2),
 * rows_per_group = 2 * ceil(ceil(M / 2) / groups)), and each 32-lane half of
 * a wave holds one row of a pair; threads = 32 * rows_in_flight (at most
 * 512).
 */
typedef struct norm_bwd_plan {
    int32_t kind;            /* NORM_BWD_LAYERNORM / RMSNORM */
    int32_t io_dtype;        /* element type of x, dy, gamma, dx */
    int32_t with_dbeta;      /* 1: kernel A also sums dy for dbeta */
    int32_t vec;             /* elements per lane per load (16 bytes, or 1) */
    int64_t M, N;            /* problem size */
    int64_t groups;          /* G: row groups = workspace rows; group g = rows r, r mod G == g
                                (two rows per wave: row pairs q, q mod G == g) */
    int64_t rows_per_group;  /* ceil(M / G): the most rows any group holds
                                (two rows per wave: 2 * ceil(ceil(M / 2) / G)) */
    int32_t chunks;          /* C: loads of `vec` elements per lane per row slice */
    int32_t waves_per_row;   /* S: 64-lane waves sharing one row */
    int32_t rows_in_flight;  /* P: rows a workgroup processes at once */
    int32_t threads;         /* 64 * S * P, kernel A's workgroup size */
    int32_t grid;            /* kernel A workgroups (groups are strided over them) */
    int32_t lds_bytes;       /* kernel A dynamic LDS: S * C * 64 * vec * 4 when P > 1
                                (one row per wave), else 0 */
    int32_t rows_per_wave;   /* 1, or 2: each 32-lane half of a wave takes a row */
    size_t workspace_bytes;  /* with_dbeta ? 2 : 1, times groups * N * 4 */
} norm_bwd_plan_t;

/*
 * Fill *plan for (kind, M, N, io_dtype, with_dbeta). groups = 0 chooses the
 * automatic group count: 256, at most ceil(M / 4) -- a function of the
 * problem only, never of the device. (The entry points that recompute
 * LayerNorm statistics on one row per wave plan their own: 512-thread
 * workgroups and about 4096 waves in flight, at most ceil(M / 4) groups,
 * above 256 rounded down to a multiple of 256; RMSNorm recompute, and
 * LayerNorm recompute on two rows per wave, take the groups as here.)
 * groups > 0 asks for that many row groups, clamped to M so that no group is
 * empty. The lane
 * layout takes at most 32 bytes of each operand per lane, then the fewest
 * waves per row (a power of two), except that widths which waves of 32-byte
 * lanes cover exactly take that many waves (5120 16-bit elements: 5). The
 * rows in flight per workgroup are the fewest whose x and dy reach 16 KiB,
 * and at least two where a group holds more than 2 MiB of each operand
 * (rows_per_group * N * element size), as far as 16 waves, the kernel's
 * launch bound and 63 KiB of LDS allow. Rows that 64-lane waves would cover
 * with idle lanes and 32 lanes cover exactly (N = 32 * vec * 1 or 3: 256 or
 * 768 16-bit, 128 or 384 fp32 elements) take two rows per wave instead, with
 * the fewest rows in flight whose x and dy reach 8 KiB (RMSNorm) or 16 KiB
 * (LayerNorm; recompute mode: 16 KiB in both kinds, and LayerNorm
 * recompute keeps 256 groups there). A plan is for saved statistics. The
 * plan assumes 16-byte aligned base pointers; norm_bwd_execute rejects a
 * plan whose vec the pointers do not allow.
 * Host-only. Returns a status code.
 */
int norm_bwd_make_plan(int kind, int64_t M, int64_t N, int io_dtype,
                       int with_dbeta, int64_t groups, norm_bwd_plan_t *plan);

/*
 * Run kernel A then kernel B of `plan` on `stream` (the whole backward pass).
 * mean is ignored for RMSNorm. dbeta must be non-NULL exactly when
 * plan->with_dbeta. Other arguments as for norm_bwd_layernorm, except that
 * the saved statistics are required (there is no eps argument, so no
 * recompute mode: use norm_bwd_layernorm / norm_bwd_rmsnorm for that).
 */
int norm_bwd_execute(const norm_bwd_plan_t *plan, const void *x,
                     const void *dy, const void *gamma, const float *mean,
                     const float *rstd, int wgrad_dtype, void *dx,
                     void *dgamma, void *dbeta, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * Kernel A alone: writes dx and the per-group partial sums into
 * workspace[groups, N] (dgamma partials), followed by workspace[groups, N]
 * (dbeta partials) when plan->with_dbeta. For callers that overlap the
 * group reduction with other work, and for timing each kernel.
 */
int norm_bwd_execute_partials(const norm_bwd_plan_t *plan, const void *x,
                              const void *dy, const void *gamma,
                              const float *mean, const float *rstd, void *dx,
                              void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * Kernel B alone: dgamma[j] = sum over g of workspace[g, j] (and dbeta from
 * the second plane when dbeta != NULL), summed in one fixed order that
 * depends only on `groups`, rounded to wgrad_dtype. groups = 0 writes zeros.
 * The workspace holds fp32 [with_dbeta ? 2 : 1][groups][N] as kernel A
 * writes it. groups * N * 8 above 2^62 is NORM_BWD_ERR_INVALID_ARG; a
 * workspace shorter than the partials is NORM_BWD_ERR_WORKSPACE.
 */
int norm_bwd_reduce_partials(int64_t groups, int64_t N, int wgrad_dtype,
                             const void *workspace, size_t workspace_bytes,
                             void *dgamma, void *dbeta, void *stream);

/*
 * Forward pass that produces the saved statistics the backward consumes
 * ("05: Layer norm", the Phobos tutorial's ln_fwd; RMSNorm per "Norm backward
 * in Triton", "The gradients"). For each row of x[M, N]:
 *   LayerNorm: mean = sum(x)/N, var = sum((x - mean)^2)/N (biased),
 *              rstd = 1/sqrt(var + eps), y = gamma * (x - mean) * rstd + beta
 *   RMSNorm:   rstd = 1/sqrt(sum(x^2)/N + eps), y = gamma * x * rstd
 * computed in fp32 from the io_dtype inputs; y is rounded to nearest even.
 *   x [M,N], gamma [N], beta [N] or NULL (read, io_dtype)
 *   y [M,N] io_dtype (written); mean, rstd fp32 [M] (written; either may be
 *   NULL to skip it)
 * The row sums run on the backward's lane layout for N, so that recompute
 * mode (same x, same eps, 16-byte aligned pointers in both calls) forms the
 * statistics this forward stores bit for bit; widths of the two-rows-per-wave
 * layout take it here too.
 * Any N up to INT32_MAX (wider than the fused limits without dbeta: the
 * row-loop forward, three passes over each row). Asynchronous on `stream`;
 * checked on the host first (status codes as above). Allocates nothing.
 */
int norm_fwd_layernorm(const void *x, const void *gamma, const void *beta,
                       int64_t M, int64_t N, int io_dtype, float eps, void *y,
                       float *mean, float *rstd, void *stream);
int norm_fwd_rmsnorm(const void *x, const void *gamma, int64_t M, int64_t N,
                     int io_dtype, float eps, void *y, float *rstd,
                     void *stream);

/* Static text for a status code. */
const char *norm_bwd_status_string(int status);

/* Message describing the calling thread's most recent failure ("" if none). */
const char *norm_bwd_last_error(void);

/*
 * Measurement aid, not part of the backward pass: copy `bytes` (a multiple
 * of 16, 16-byte aligned pointers) from src to dst with a plain streaming
 * kernel on `stream`. Used to calibrate hardware byte counters and to measure
 * the achievable HBM copy bandwidth next to the norm kernels.
 */
int norm_bwd_probe_copy(const void *src, void *dst, size_t bytes, void *stream);

/*
 * Measurement aid, not part of the backward pass: the streaming ceiling for
 * kernel A's access mix (the dx pass reads x and dy and writes dx once each:
 * "Norm backward in Triton", "Worked numbers", counts exactly these bytes).
 * c = a + b over `bytes` bytes of each operand, taken as 32-bit words, with
 * 16-byte non-temporal loads and stores, on `stream`. Moves 3 * bytes.
 *   a, b     read; c written; 16-byte aligned device pointers; c may not
 *            overlap a or b (a and b may be the same buffer)
 *   bytes    bytes per operand, a multiple of 16
 *   grid     workgroups of 256 threads (1 .. 2^20), or 0 for one pass over
 *            the data (each thread handles `unroll` vectors once)
 *   unroll   16-byte vectors per operand each thread loads before it stores
 *            (1, 2, 4 or 8)
 * Returns a status code; NORM_BWD_ERR_INVALID_ARG for arguments outside these
 * ranges, with nothing launched.
 */
int norm_bwd_probe_triad(const void *a, const void *b, void *c, size_t bytes, int grid,
                         int unroll, void *stream);

/*
 * Measurement aid, not part of the backward pass: the triad above in one pass
 * with 16-byte raw buffer loads and stores under a chosen cache policy, to
 * find which policy streams kernel A's 2-read:1-write mix fastest.
 *   a, b, c       as for norm_bwd_probe_triad
 *   bytes         bytes per operand: a multiple of 4096 * unroll, at most
 *                 NORM_BWD_PROBE_POLICY_MAX_BYTES (32-bit buffer offsets)
 *   unroll        16-byte vectors per operand per thread: 1, 2 or 4
 *   load_policy, store_policy
 *                 cache-policy bits of the gfx950 vector memory
 *                 instructions, any OR of 1 (sc0), 2 (nt) and 16 (sc1);
 *                 0 is the default policy
 * Returns a status code; NORM_BWD_ERR_INVALID_ARG for arguments outside these
 * ranges, with nothing launched.
 */
#define NORM_BWD_PROBE_POLICY_MAX_BYTES (0xFFFFFFFFu - 16383u)
int norm_bwd_probe_triad_policy(const void *a, const void *b, void *c, size_t bytes,
                                int unroll, int load_policy, int store_policy, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NORM_BWD_H */

/*
 * gba.h -- C ABI of the MI355X (gfx950) fused GEMM + bias + activation library.
 *
 * The operation is the tiled GEMM of "writing-tilelang-kernels" (skillsmp.com),
 * sections "Kernel Anatomy" and "GEMM (Minimal)": A is (M,K), B is (K,N), C is
 * (M,N), all row-major, fp16 inputs, float accumulator in registers, one write
 * of C. "TileLang: Write, Autotune, and Ship Fused Tensor-Core Kernels from
 * Python" (saipien.org), section "Why tile-level control matters", adds the
 * fused epilogue: a bias add and an activation applied while the accumulator
 * is still in registers, so the M x N intermediate never goes back to HBM.
 *
 * Conventions shared by every entry point:
 *   - All array arguments are DEVICE pointers owned by the caller. The library
 *     allocates nothing on the compute path and keeps no pointer after a call.
 *   - Layouts are dense row-major with leading dimensions K (A, and W of the
 *     _nt calls), N (B, C, X, Y).
 *   - dtype (gba_dtype) applies to A, B, bias and C alike; accumulation is fp32.
 *   - Pointers must be 16-byte aligned, and K and N multiples of 8 (the 16-byte
 *     row-alignment rule of "writing-tilelang-kernels", Common Pitfalls);
 *     otherwise GBA_ERR_ALIGN. M is arbitrary.
 *   - M == 0 or N == 0: nothing to do, GBA_OK, no launch. K == 0: the empty
 *     sum, C = act(bias) (or act(0)). Negative sizes, or K > 2^21, N > 2^23,
 *     M > 2^31 - 1 (the kernels' 32-bit tile offsets): GBA_ERR_SHAPE.
 *   - Argument errors are reported synchronously, before any launch. Work is
 *     enqueued on the calling thread's stream (gba_set_stream) and runs
 *     asynchronously; a device fault surfaces at the caller's next sync.
 *   - A launch failure returns GBA_ERR_HIP; gba_last_hip_error() gives the code.
 *   - The device must be gfx950 (MI355X/MI350X); otherwise GBA_ERR_DEVICE.
 */
#ifndef GBA_H
#define GBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GBA_DTYPE_F16 = 0, GBA_DTYPE_BF16 = 1 } gba_dtype;

/* Epilogue activations. ReLU and sigmoid: "writing-tilelang-kernels",
 * Pre-flight Checklist ("ReLU/sigmoid epilogue after GEMM") and Key API
 * Patterns (T.max, T.sigmoid). GELU: "TileLang: Write, Autotune, and Ship Fused
 * Tensor-Core Kernels from Python", Why tile-level control matters; this
 * library's GELU is the erf form, GELU(z) = z * Phi(z) = 0.5 z (1 + erf(z/sqrt2)).
 * Softplus: the Elementwise (2D) template of "writing-tilelang-kernels", Quick
 * Templates, log(1 + exp(z)) in the float accumulator type. GELU_TANH: the
 * tanh form of GELU (Hendrycks and Gimpel, 2016). */
typedef enum {
    GBA_ACT_NONE = 0,
    GBA_ACT_RELU = 1,     /* max(z, 0) */
    GBA_ACT_SIGMOID = 2,  /* 1 / (1 + exp(-z)) */
    GBA_ACT_GELU = 3,     /* z * Phi(z), erf form */
    GBA_ACT_SOFTPLUS = 4, /* log(1 + exp(z)) */
    GBA_ACT_GELU_TANH = 5 /* 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) */
} gba_act;

typedef enum {
    GBA_OK = 0,
    GBA_ERR_NULL = 1,     /* a required pointer is NULL */
    GBA_ERR_SHAPE = 2,    /* negative or too-large size */
    GBA_ERR_DTYPE = 3,    /* dtype not a gba_dtype */
    GBA_ERR_ACT = 4,      /* act not a gba_act */
    GBA_ERR_ALIGN = 5,    /* pointer not 16-byte aligned, or K / N not a multiple of 8 */
    GBA_ERR_ALIAS = 6,    /* output overlaps an input it may not overlap */
    GBA_ERR_DEVICE = 7,   /* no HIP device, or not gfx950 */
    GBA_ERR_HIP = 8,      /* a HIP runtime call failed; see gba_last_hip_error() */
    GBA_ERR_SCHEDULE = 9, /* schedule not among the compiled-in ones */
    GBA_ERR_CACHE = 10,   /* schedule cache could not be written (tuning still done) */
    GBA_TUNE_INCOMPLETE = 11, /* gba_autotune stopped at its candidate budget (GBA_TUNE_BUDGET);
                                 its progress is kept, a later call resumes */
    GBA_ERR_SCRATCH = 12  /* gemm_bias_act_noalloc: the split-K partials would exceed its
                             static scratch (gba_noalloc_scratch_bytes) */
} gba_status;

/* A GEMM schedule: one compiled-in kernel instance plus its launch mapping.
 * bm x bn is the output tile of one workgroup, bk the K depth of one LDS stage,
 * wm x wn the grid of 64-lane waves over the tile, stages the LDS ring depth.
 * raster 0 maps workgroup ids to tiles row by row; raster 1 first gathers the
 * tiles each of the 8 XCDs runs into one contiguous block, then walks them in
 * groups of group_m tile rows so that neighbouring workgroups share A and B
 * panels in that XCD's L2 ("use_swizzle ... L2 cache locality",
 * "writing-tilelang-kernels", Key API Patterns). kernel selects the main-loop
 * design; the compiled-in ones are:
 *   0 = tiles staged through registers into LDS (B transposed on the way), at
 *       the pages' 128x128x32 starting tile;
 *   3 = direct global->LDS loads into a `stages`-deep ring, every instruction
 *       of an MFMA step placed by hand (global->LDS loads issued by the first
 *       `loaders` waves, spread over `spread` steps; the next step's LDS reads
 *       between the 16x16x32 MFMAs), one tile per workgroup;
 *   4 = kernel 3's loop run persistently: one workgroup per CU walks tiles w,
 *       w + G, ... (G = min(tiles, CUs)) as one stream of K slices, so the next
 *       tile's first slices load during the current tile's last steps and
 *       epilogue (the built-in choice for 256x256 tiles). With K <= bk it hands
 *       the call to the 128x128 four-stage kernel 3, which feeds every output
 *       element the same MFMAs in the same order.
 * (Ids 1 and 2, earlier designs that never won, are no longer compiled in.)
 * loaders and spread are 0 for kernel 0. */
typedef struct {
    int32_t bm, bn, bk;
    int32_t wm, wn;
    int32_t stages;
    int32_t raster;
    int32_t group_m;
    int32_t kernel;
    int32_t loaders;
    int32_t spread;
} gba_schedule;

/* C = act(A.B + bias).
 * A: [M,K], B: [K,N], bias: [N] or NULL (no bias), C: [M,N], all `dtype`.
 * act: gba_act. C must not overlap A, B or bias (GBA_ERR_ALIAS). */
int gemm_bias_act(const void *A, const void *B, const void *bias, void *C, int64_t M,
                  int64_t N, int64_t K, int act, int dtype);

/* C = A.B rounded to `dtype`: the first kernel of the unfused pair used as the
 * HBM-traffic baseline ("TileLang: Write, Autotune, and Ship Fused Tensor-Core
 * Kernels from Python", Why tile-level control matters: fused vs unfused,
 * intermediate M x N round trip of 2*M*N*2 bytes). Same rules as gemm_bias_act. */
int gemm(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int dtype);

/* Y = act(X + bias) elementwise over [M,N]: the second kernel of the unfused
 * pair (an elementwise 2-D kernel, cf. the "Elementwise (2D)" template of
 * "writing-tilelang-kernels", Quick Templates). X and Y: [M,N]; bias: [N] or
 * NULL. Y may equal X exactly (in place) but may not partially overlap it;
 * Y may not overlap bias. */
int bias_act(const void *X, const void *bias, void *Y, int64_t M, int64_t N, int act,
             int dtype);

/* C = act(A.W^T + bias) with the second operand stored as W: [N,K] row-major
 * (K-contiguous rows, the layout of a linear layer's weight): the transpose_B
 * form of the tile GEMM ("writing-tilelang-kernels", Key API Patterns,
 * T.gemm(..., transpose_B=True)). A: [M,K], bias: [N] or NULL, C: [M,N].
 * Everything else as gemm_bias_act: same dtype rule, the 16-byte alignment rule
 * with K and N multiples of 8, same errors; C may not overlap A, W or bias.
 * Kernels 3 and 4 have this path; a forced schedule of another kernel makes the
 * call return GBA_ERR_SCHEDULE. The result is bitwise that of gemm_bias_act on
 * the same schedule with B = W^T. */
int gemm_bias_act_nt(const void *A, const void *W, const void *bias, void *C, int64_t M,
                     int64_t N, int64_t K, int act, int dtype);

/* C = A.W^T rounded to `dtype`, W: [N,K] (gemm with transpose_B). */
int gemm_nt(const void *A, const void *W, void *C, int64_t M, int64_t N, int64_t K, int dtype);

/* gemm_bias_act_ex / gba_workspace_size flags. */
enum {
    GBA_TRANSPOSE_B = 1, /* B is W, stored [N,K], as in gemm_bias_act_nt */
    GBA_INPUT_FP8 = 2,   /* gba_workspace_size only: for gemm_bias_act_fp8_ex */
    GBA_TRANSPOSE_A = 4  /* A is At, stored [K,M]: C = act(At^T.B + bias) */
};

/* gemm_bias_act (or, with GBA_TRANSPOSE_B, gemm_bias_act_nt) with an optional
 * caller-owned device workspace for split-K, and the first operand in either
 * layout.
 * GBA_TRANSPOSE_A: the first operand is At: [K,M] row-major (M-contiguous
 * rows) and the product is At^T.B (or At^T.W^T with GBA_TRANSPOSE_B): the
 * transpose_A form of the tile GEMM ("writing-tilelang-kernels", Key API
 * Patterns, T.gemm(..., transpose_A=True)). M must then be a multiple of 8 as
 * well (16-byte rows of At; else GBA_ERR_ALIGN) and at most 2^23 (like N; else
 * GBA_ERR_SHAPE). Kernels 3 and 4 at the built-in tiles have this path (see
 * gba_list_schedule); a forced schedule without it returns GBA_ERR_SCHEDULE.
 * The result is bitwise that of the [M,K] path on the same schedule with
 * A = At^T: both feed the matrix cores the same operands in the same order. When the chosen schedule's tiles
 * leave compute units idle and K is deep enough for the split to pay for its
 * extra traffic (e.g. 256x256x4096: 16 tiles of 64x64 for 256 CUs; not
 * 1024^3, where the fp32 partials' round trip costs more than it saves), K is
 * split S ways: a first kernel writes the S fp32 partial sums
 * [S][M][N] into the workspace, and a second adds them in split order and
 * applies bias, act and the rounding (the fused epilogue, one pass over C).
 * gba_workspace_size gives the bytes that enable the split (0: no split for
 * this shape); a NULL or smaller workspace runs the one-kernel path. The
 * workspace needs no initialisation and holds nothing between calls; it must
 * be 16-byte aligned and overlap none of A, B, bias, C (GBA_ERR_ALIGN /
 * GBA_ERR_ALIAS). Calls sharing a workspace must be ordered on one stream.
 * The split changes the fp32 summation order, not the tolerance; results are
 * deterministic. Unknown flag bits: GBA_ERR_SHAPE. */
int gemm_bias_act_ex(const void *A, const void *B, const void *bias, void *C, int64_t M,
                     int64_t N, int64_t K, int act, int dtype, int flags, void *workspace,
                     size_t workspace_bytes);

/* gemm_bias_act_ex for callers that cannot allocate device memory: code
 * recorded under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. It takes no workspace; when the call splits K (the same
 * choice as gemm_bias_act_ex with a large enough workspace, and the same
 * result, bitwise), the fp32 partials go to a static device array of the
 * library, gba_noalloc_scratch_bytes() = 16 MiB, one per GPU, held until the
 * process ends. It calls no allocating routine: the array's address is taken
 * (hipGetSymbolAddress) on the first call on each device. Splits whose
 * partials (S * M * N * 4 bytes) would exceed the array return GBA_ERR_SCRATCH
 * before any launch; with 64 x 64 or 128 x 128 tiles and at most CUs / tiles
 * splits the partials take at most CUs * 128 * 128 * 4 bytes, so that bound is
 * never reached on a 256-CU device. The array needs no clearing: the
 * first pass writes every partial it reads back. All calls on one GPU share
 * the array, so calls that overlap on that GPU (different streams, or
 * different host threads without ordering) race; order them on one stream.
 * Arguments, flags and errors otherwise as gemm_bias_act_ex. */
int gemm_bias_act_noalloc(const void *A, const void *B, const void *bias, void *C, int64_t M,
                          int64_t N, int64_t K, int act, int dtype, int flags);
size_t gba_noalloc_scratch_bytes(void);

/* The plan of a gemm_bias_act_ex call with these arguments, these
 * GBA_TRANSPOSE_A / GBA_TRANSPOSE_B flags and a workspace of at least
 * gba_workspace_size bytes: *splits K ranges computed with the tile schedule
 * *sched (*splits = 1: one kernel, *sched as gba_get_schedule_ex). The split's
 * schedule can differ from the one-kernel choice: where the built-in choice is
 * the 64x64 tile, the 128x128 tile's split is taken when the cost model
 * predicts it faster. Launches nothing. Errors as gba_get_schedule_ex, and
 * GBA_ERR_NULL for a NULL output. */
int gba_split_plan(int64_t M, int64_t N, int64_t K, int act, int dtype, int flags,
                   gba_schedule *sched, int *splits);

/* Workspace bytes gemm_bias_act_ex (with GBA_INPUT_FP8: gemm_bias_act_fp8_ex)
 * would use for these arguments (0 if it would not split), written to *bytes. */
int gba_workspace_size(int64_t M, int64_t N, int64_t K, int act, int dtype, int flags,
                       size_t *bytes);

/* 8-bit float input formats (OCP OFP8): E4M3 (largest finite 448, no
 * infinities) and E5M2 (largest finite 57344). */
typedef enum { GBA_FP8_E4M3 = 0, GBA_FP8_E5M2 = 1 } gba_fp8_format;

/* C = act(scale * A.W^T + bias) with 8-bit float inputs: the FP8 GEMM named
 * in "tilelang" (skillsmp.com), Documentation Structure (float8_e4m3/e5m2 in
 * the type system, an FP8 GEMM among the GEMM examples), with the fused
 * epilogue of gemm_bias_act.
 * A: [M,K] and W: [N,K] (the transpose_B layout), both 8-bit in format `fmt`
 * (gba_fp8_format), row-major, K-contiguous; scale: the fp32 dequantization
 * factor of the product (e.g. the product of the per-tensor scales of A and
 * W), applied before the bias; bias: [N] or NULL and C: [M,N], both `dtype`
 * (fp16/bf16). Accumulation is fp32 on the 16x16x128 8-bit matrix cores.
 * K must be a multiple of 16 (16-byte rows) and N of 8; pointers 16-byte
 * aligned (GBA_ERR_ALIGN). fmt not a gba_fp8_format: GBA_ERR_DTYPE. A
 * non-finite scale: GBA_ERR_SHAPE. C may not overlap A, W or bias. One
 * compiled-in schedule (persistent 256x256 tiles); forced schedules do not
 * apply. Other rules as gemm_bias_act. */
int gemm_bias_act_fp8_nt(const void *A, const void *W, const void *bias, void *C, int64_t M,
                         int64_t N, int64_t K, float scale, int act, int fmt, int dtype);

/* gemm_bias_act_fp8_nt with an optional split-K workspace, as gemm_bias_act_ex:
 * when the 256x256 tiles leave compute units idle and K is deep enough (e.g.
 * 128 x 4096 x 14336: 16 tiles for 256 CUs), the first pass writes
 * scale * partial sums of K ranges ([S][M][N] fp32) and the second adds them in
 * split order, then bias, act and rounding. Size from gba_workspace_size with
 * GBA_INPUT_FP8; NULL or smaller: the one-kernel path. */
int gemm_bias_act_fp8_ex(const void *A, const void *W, const void *bias, void *C, int64_t M,
                         int64_t N, int64_t K, float scale, int act, int fmt, int dtype,
                         void *workspace, size_t workspace_bytes);

/* Stream for this thread's later calls (a hipStream_t); NULL = default stream. */
int gba_set_stream(void *hip_stream);

/* Force a schedule for this thread's later GEMM calls (NULL: back to the cache
 * or the built-in heuristic). GBA_ERR_SCHEDULE if no compiled-in kernel has
 * this (bm, bn, bk, wm, wn, stages, kernel, loaders, spread), or raster/group_m
 * are out of range. */
int gba_set_schedule(const gba_schedule *s);

/* The schedule a gemm_bias_act (gemm_bias_act_nt; gemm_bias_act_ex with these
 * GBA_TRANSPOSE_A / GBA_TRANSPOSE_B flags) call with these arguments would use
 * now. Unknown flag bits: GBA_ERR_SHAPE. */
int gba_get_schedule(int64_t M, int64_t N, int64_t K, int act, int dtype, gba_schedule *out);
int gba_get_schedule_nt(int64_t M, int64_t N, int64_t K, int act, int dtype, gba_schedule *out);
int gba_get_schedule_ex(int64_t M, int64_t N, int64_t K, int act, int dtype, int flags,
                        gba_schedule *out);

/* gba_autotune flags. */
enum {
    GBA_TUNE_ALL_GROUPS = 1,   /* also try every raster group size in {1,2,4,8,16} */
    GBA_TUNE_TRANSPOSE_B = 2,  /* tune gemm_bias_act_nt: B is W, stored [N,K] */
    GBA_TUNE_TRANSPOSE_A = 4   /* A is At, stored [K,M] (gemm_bias_act_ex, GBA_TRANSPOSE_A) */
};

/* Compiled-in kernel instances: count, and the i-th one (raster/group_m are
 * their defaults). */
int gba_num_schedules(void);
int gba_list_schedule(int i, gba_schedule *out);

/* Autotuner ("TileLang: Write, Autotune, and Ship Fused Tensor-Core Kernels from
 * Python", section Autotuning: how it works and how much it costs): for every
 * compiled-in instance (with a path for the operand layouts that
 * GBA_TUNE_TRANSPOSE_A / _B select) whose LDS ring (bm*bk + bk*bn) * 2 * stages
 * fits the 160 KiB LDS of a CU, and each raster variant, run 10 untimed and 50
 * timed launches on the caller's buffers, keep the median time, and pick the
 * fastest. C holds the winner's result on return. flags: GBA_TUNE_* bits.
 * best / best_ms may be NULL. Synchronous: it waits for its own launches.
 *
 * Persistence (the page's on-disk cache, kept across runs and CI; disabled as
 * a whole by GBA_DISABLE_CACHE=1):
 *   - The winner is stored in $GBA_CACHE_DIR/schedules.json (default
 *     ~/.cache/gba) under the key (arch, CU count, gba_build_id(), dtype, act,
 *     operand layouts, M, N, K), and used by later calls in any process.
 *     Entries of other builds stay in the file and are never used by this one.
 *   - Writers merge into the file under an exclusive lock and replace it by
 *     rename: concurrent processes lose no entries and readers never see a
 *     partial file. A process re-reads the file when GBA_CACHE_DIR changes.
 *   - Each timed candidate is appended to $GBA_CACHE_DIR/tuning.json as it
 *     finishes. A call with the same key first takes the candidates already
 *     there (an interrupted run's) instead of timing them again; the journal
 *     entries of a key are removed when its tuning completes.
 *   - GBA_TUNE_BUDGET=n (environment) limits a call to timing n new
 *     candidates: if some remain, it returns GBA_TUNE_INCOMPLETE with the best
 *     so far in best / best_ms and in C, writes nothing to schedules.json, and
 *     the next call resumes.
 * Returns GBA_ERR_CACHE (with best filled and C written) if the cache or the
 * journal could not be written. */
int gba_autotune(const void *A, const void *B, const void *bias, void *C, int64_t M,
                 int64_t N, int64_t K, int act, int dtype, int flags, gba_schedule *best,
                 double *best_ms);

/* Per-candidate results of this thread's last gba_autotune call (the page's
 * tuning cost accounting): their number, and the i-th candidate's schedule,
 * median ms, and whether it came from the tuning journal (1) rather than being
 * timed by that call (0). Any pointer may be NULL; i out of range:
 * GBA_ERR_SHAPE. */
int gba_autotune_num_trials(void);
int gba_autotune_trial(int i, gba_schedule *sched, double *ms, int *resumed);

/* Identifies the kernels compiled into this library (a hash of its sources);
 * part of every schedule-cache key. */
const char *gba_build_id(void);

/* Read or seed the schedule cache without a device (e.g. to ship schedules
 * tuned elsewhere, or to inspect them): the entry gba_autotune would write for
 * a gemm_bias_act_ex call with these sizes, act, dtype and GBA_TRANSPOSE_A /
 * GBA_TRANSPOSE_B flags on a device of this arch (gcnArchName, e.g.
 * "gfx950:sramecc+:xnack-") and CU count, for this build.
 * gba_cache_lookup: GBA_OK with *sched (and *ms, the tuned median; either may
 * be NULL) if the cache holds such an entry; GBA_ERR_SCHEDULE if it does not or
 * the cache is disabled. gba_cache_store: merges the entry into the file as
 * gba_autotune does (GBA_ERR_SCHEDULE if sched is not compiled in,
 * GBA_ERR_CACHE if the file cannot be written, GBA_OK and nothing written if
 * the cache is disabled). Both: NULL arch: GBA_ERR_NULL; an arch string with
 * '"', '|' or a newline, or longer than 64: GBA_ERR_DEVICE; cus <= 0,
 * negative sizes, unknown flags, or (store) a negative or non-finite ms:
 * GBA_ERR_SHAPE; bad act / dtype as gemm_bias_act. */
int gba_cache_lookup(const char *arch, int cus, int64_t M, int64_t N, int64_t K, int act,
                     int dtype, int flags, gba_schedule *sched, double *ms);
int gba_cache_store(const char *arch, int cus, int64_t M, int64_t N, int64_t K, int act,
                    int dtype, int flags, const gba_schedule *sched, double ms);

/* Device-side epilogue probe: y[i] = act(z[i]) in fp32, computed by the same
 * device function the GEMM epilogue uses. z, y: device float arrays of n. */
int gba_epilogue_probe(const float *z, float *y, int64_t n, int act);

/* Shader-clock probe, for reporting the clock a measurement ran at: n_wg
 * workgroups of one wave each spin for spin_us microseconds of the device's
 * constant-rate wall clock; workgroup i writes out[2i] = elapsed core clock
 * cycles (s_memtime) and out[2i+1] = elapsed wall-clock ticks (s_memrealtime).
 * The core clock in MHz is out[2i] / out[2i+1] * (*wall_khz) / 1000. Enqueued on
 * the library's stream (gba_set_stream) right after the work to be described, it
 * reads the clock that work ended at. out: device array of 2 * n_wg uint64,
 * owned by the caller; *wall_khz (host): the wall clock's rate. Errors: NULL
 * pointers: GBA_ERR_NULL; n_wg outside 1..65536 or spin_us outside 1..100000:
 * GBA_ERR_SHAPE. */
int gba_clock_probe(uint64_t *out, int n_wg, int spin_us, int *wall_khz);

const char *gba_status_string(int status);
int gba_last_hip_error(void);
const char *gba_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GBA_H */

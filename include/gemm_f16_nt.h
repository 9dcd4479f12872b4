/*
 * gemm_f16_nt.h -- C ABI of the MI355X (gfx950) dense fp16 NT GEMM library
 * (libgemm_f16.so).
 *
 * The operation (Tilus tutorial "Hopper matmul", page "2. Multi-Stage
 * Software Pipelining", The Full Kernel; page "6. Register Reallocation,
 * Multicast, and a Persistent Kernel", opening paragraphs):
 *
 *     C[i][j] = fp16_rne( sum_k A[i][k] * B[j][k] )      (accumulated in fp32)
 *
 *   A  fp16 [M, K] row-major (leading dimension K)
 *   B  fp16 [N, K] row-major (leading dimension K); the product uses B^T
 *   C  fp16 [M, N] row-major (leading dimension N)
 *
 * The pages' kernels take (m_size, n_size, k_size, a_ptr, b_ptr, c_ptr): dense
 * matrices, no leading-dimension, alpha or beta arguments.  This interface
 * keeps that and adds the HIP stream to enqueue on.  fp16 data travel as raw
 * 16-bit IEEE binary16 storage.  The fp32 accumulator is rounded once, to
 * nearest with ties to even; results beyond the fp16 range become +-inf and
 * fp16 subnormals are kept.  C is write-only (beta = 0): it is never read.
 *
 * Threading: every entry point may be called from any host thread.  The only
 * global state is a lazily built, mutex-protected cache of per-device
 * properties (compute-unit count).
 */
#ifndef GEMM_F16_NT_H
#define GEMM_F16_NT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
    GEMM_F16_OK = 0,
    /* a dimension < 0; a NULL pointer for a matrix with elements; C
     * overlapping A or B; an unknown configuration id */
    GEMM_F16_INVALID_ARG = 1,
    /* valid but outside what the kernels handle: A, B or C not 2-byte aligned
     * (not fp16 element addresses), M, N or K above 2^31 - 1, or more than
     * 2^31 - 1 output tiles; also a forced configuration that cannot take the
     * arguments (see gemm_f16_nt_with_config) */
    GEMM_F16_UNSUPPORTED = 2,
    /* the HIP runtime reported an error for the kernel launch (the status
     * hipLaunchKernel returns; the thread's last-error state is left as it
     * was) or when querying the current device */
    GEMM_F16_LAUNCH_FAILED = 3,
    /* gemm_f16_nt_splitk_noalloc only: the planned fp32 partials need more
     * than the library's fixed 64 MiB scratch array */
    GEMM_F16_SCRATCH_LIMIT = 4
};

/*
 * C = A * B^T on `stream` (0 = the null stream), on the current HIP device.
 *
 * A, B and C are device pointers owned by the caller; they must stay valid
 * until the enqueued work has finished.  The library allocates nothing and
 * uses no workspace (gemm_f16_nt_splitk below is the variant that takes
 * one).  The call returns once the kernel is enqueued; a fault
 * inside the kernel surfaces at the caller's next synchronisation.
 *
 * M = 0 or N = 0: nothing to compute, returns GEMM_F16_OK without a launch.
 * K = 0: C is filled with +0 (the empty sum).
 * Any K and any 2-byte alignment of A, B and C are accepted.  The fast
 * kernels load with 16-byte direct-to-LDS DMA and need K a multiple of 8, at
 * most 2^21, and A and B 16-byte aligned; other arguments run the general
 * kernel (register-staged loads), which gives the same results, more slowly.
 * Results are deterministic: no atomics, and each element's K order depends
 * only on K, never on the element's position or on the launch shape.
 */
int gemm_f16_nt(int64_t M, int64_t N, int64_t K,
                const void *A, const void *B, void *C,
                hipStream_t stream);

/* A static, human-readable name for a status code. */
const char *gemm_f16_nt_status_string(int status);

/*
 * The current HIP device's compute-unit count, as the planners of the
 * launching entry points use it (read once per device and cached; safe from
 * any thread).  GEMM_F16_INVALID_ARG for NULL; GEMM_F16_LAUNCH_FAILED if the
 * HIP runtime cannot report it.
 */
int gemm_f16_device_cus(int32_t *cus);

/*
 * Argument check used by every GEMM entry point; pure host function, touches
 * no device and dereferences nothing.  Returns a status code.
 */
int gemm_f16_nt_validate(int64_t M, int64_t N, int64_t K,
                         const void *A, const void *B, const void *C);

/*
 * The launch plan the library would use for (M, N, K) on a device with
 * `num_cus` compute units, for 16-byte aligned A and B (otherwise the general
 * kernel, the last configuration, runs).  Pure host function (no device
 * access): used by tests and by the benchmark to report what runs.
 */
typedef struct {
    int32_t config_id;   /* index into the compiled kernel table           */
    int32_t block_m;     /* output tile rows (M)                           */
    int32_t block_n;     /* output tile columns (N)                        */
    int32_t block_k;     /* K depth of one LDS stage                        */
    int32_t waves;       /* 64-lane wavefronts per workgroup               */
    int32_t stages;      /* LDS ring depth                                 */
    int32_t swizzle;     /* raster group width in N tiles (1 = plain rows) */
    int32_t tiles_m;     /* ceil(M / block_m)                              */
    int32_t tiles_n;     /* ceil(N / block_n)                              */
    int32_t grid;        /* persistent workgroups launched                 */
    int64_t tiles;       /* tiles_m * tiles_n                              */
    int32_t lds_bytes;   /* LDS used by one workgroup: the ring, plus the
                            staged epilogue's second buffer where it has one */
    int32_t xcds;        /* XCD count the tile order is arranged for       */
    int32_t epilogue;    /* 0: stores straight from the MFMA registers;
                            1: C staged through LDS for row-contiguous stores */
    int32_t b_layout;    /* B in memory: 0 = [N, K] (gemm_f16_nt, gemm_f16_tt),
                            1 = [K, N] (gemm_f16_nn, gemm_f16_tn) */
    int32_t a_layout;    /* A in memory: 0 = [M, K] (gemm_f16_nt, gemm_f16_nn),
                            1 = [K, M] (gemm_f16_tn, gemm_f16_tt) */
} gemm_f16_nt_plan_t;

int gemm_f16_nt_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                     gemm_f16_nt_plan_t *plan);

/* Number of kernel configurations compiled into the library, and the static
 * description of configuration `config_id` (tiles_m, tiles_n, tiles and grid
 * are left 0).  Pure host functions. */
int gemm_f16_nt_num_configs(void);
int gemm_f16_nt_config_info(int32_t config_id, gemm_f16_nt_plan_t *info);

/*
 * gemm_f16_nt with an explicit kernel configuration, raster group width,
 * persistent grid size and epilogue (config_id < 0: the planner's choice;
 * grid <= 0: one workgroup per compute unit, capped by the tile count;
 * swizzle <= 0: the configuration's default;
 * epilogue < 0: the library's choice, 0: direct stores, 1: staged through
 * LDS -- GEMM_F16_UNSUPPORTED if the configuration has no room for it).  A
 * direct-to-LDS configuration forced on arguments only the general kernel
 * takes (K not a multiple of 8 or above 2^21, A or B not 16-byte aligned)
 * returns GEMM_F16_UNSUPPORTED.  Otherwise the same semantics, ownership
 * and status codes as gemm_f16_nt; the result is
 * identical for every configuration, swizzle, grid and epilogue, because the
 * K order of each element does not depend on them.  For tests and tuning
 * sweeps.
 */
int gemm_f16_nt_with_config(int64_t M, int64_t N, int64_t K,
                            const void *A, const void *B, void *C,
                            hipStream_t stream, int32_t config_id,
                            int32_t swizzle, int32_t grid, int32_t epilogue);

/*
 * The other operand layouts (the pages only build the NT form).  All four
 * compute C[i][j] = fp16_rne( sum_k a(i, k) * b(k, j) ), accumulated in fp32,
 * C fp16 [M, N] row-major, with
 *
 *   gemm_f16_nn:  a(i, k) = A[i][k], A [M, K];  b(k, j) = B[k][j], B [K, N]
 *   gemm_f16_tn:  a(i, k) = A[k][i], A [K, M];  b(k, j) = B[k][j], B [K, N]
 *   gemm_f16_tt:  a(i, k) = A[k][i], A [K, M];  b(k, j) = B[j][k], B [N, K]
 *
 * (gemm_f16_nt: A [M, K], B [N, K]), every array row-major.  The same kernels
 * as gemm_f16_nt, with a tile of an operand stored [K, M] or [K, N] kept in
 * that form in LDS and its MFMA fragments read through gfx950's transposing
 * LDS read.  Each element's K order is the same as gemm_f16_nt's, so each
 * result equals gemm_f16_nt on the explicitly transposed operands bit for
 * bit.  The direct-to-LDS kernels of these layouts need K at most 2^21; for
 * an operand stored with K contiguous, K a multiple of 8; for one stored
 * [K, M] or [K, N], M or N a multiple of 8 and K * M * 2 or K * N * 2 below
 * 2^31; and A and B 16-byte aligned.  Other arguments run the layout's
 * general kernel (register-staged loads along each operand's contiguous
 * dimension, any sizes and 2-byte alignment), with the same results, more
 * slowly; a forced direct-to-LDS configuration on such arguments is
 * GEMM_F16_UNSUPPORTED.  K = 0 writes +0 without reading A or B.  Ownership,
 * asynchrony, threading and the other status codes as for gemm_f16_nt; a
 * configuration id of another layout is GEMM_F16_INVALID_ARG (each
 * configuration's a_layout and b_layout say which it is).  The _plan
 * functions are the pure host planners.
 */
int gemm_f16_nn(int64_t M, int64_t N, int64_t K,
                const void *A, const void *B, void *C,
                hipStream_t stream);
int gemm_f16_nn_with_config(int64_t M, int64_t N, int64_t K,
                            const void *A, const void *B, void *C,
                            hipStream_t stream, int32_t config_id,
                            int32_t swizzle, int32_t grid, int32_t epilogue);
int gemm_f16_nn_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                     gemm_f16_nt_plan_t *plan);
int gemm_f16_tn(int64_t M, int64_t N, int64_t K,
                const void *A, const void *B, void *C,
                hipStream_t stream);
int gemm_f16_tn_with_config(int64_t M, int64_t N, int64_t K,
                            const void *A, const void *B, void *C,
                            hipStream_t stream, int32_t config_id,
                            int32_t swizzle, int32_t grid, int32_t epilogue);
int gemm_f16_tn_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                     gemm_f16_nt_plan_t *plan);
int gemm_f16_tt(int64_t M, int64_t N, int64_t K,
                const void *A, const void *B, void *C,
                hipStream_t stream);
int gemm_f16_tt_with_config(int64_t M, int64_t N, int64_t K,
                            const void *A, const void *B, void *C,
                            hipStream_t stream, int32_t config_id,
                            int32_t swizzle, int32_t grid, int32_t epilogue);
int gemm_f16_tt_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                     gemm_f16_nt_plan_t *plan);

/*
 * Split over K, for shapes whose output tiles leave most compute units idle
 * (a small M x N with a long K).  The pages split the work over output tiles
 * only, and note what an under-filled last round of tiles costs (Tilus
 * tutorial "Hopper matmul", page "6. Register Reallocation, Multicast, and a
 * Persistent Kernel", the results and the closing caution on other shapes).
 * Here K is also cut into `splits` ranges of whole K slices, one work unit
 * per (range, output tile); each unit writes its fp32 partial sums to a
 * caller-provided workspace, and a second kernel on the same stream forms
 *
 *     C[i][j] = fp16_rne( P_0[i][j] + P_1[i][j] + ... )      (fp32, in range order)
 *
 * so results are deterministic, but they differ from gemm_f16_nt's in the
 * fp32 rounding of the sum (exact for sums that fp32 represents exactly,
 * e.g. small integers).
 *
 * gemm_f16_nt_splitk_plan: pure host function.  For (M, N, K) on `num_cus`
 * compute units and 16-byte aligned A and B, writes the kernel configuration
 * (plan, with grid = the persistent grid over all units), the effective split
 * count (*splits_out, at most `splits`: ranges are whole K slices) and the
 * workspace size in bytes (*workspace_bytes, 0 when there is no split).
 * splits <= 0 lets the library choose (it weighs the rounds of MFMA work
 * against the partial-sum traffic; where gemm_f16_nt's plan streams B, or A,
 * through registers for a few rows of A or columns of B, it splits that plan
 * by a rule of its own or keeps it unsplit); splits = 1 is gemm_f16_nt's
 * plan.
 * GEMM_F16_INVALID_ARG for NULL outputs, negative sizes, num_cus <= 0 or
 * splits > 64.
 *
 * gemm_f16_nt_splitk: C = A * B^T with K split as the plan above says, for
 * the current device.  `workspace` is caller-owned device memory, 16-byte
 * aligned (else GEMM_F16_UNSUPPORTED), of at least the planned bytes, not
 * overlapping A, B or C (else GEMM_F16_INVALID_ARG); its contents on entry
 * do not matter and are overwritten.  It may be NULL when the plan has no
 * split.  Concurrent calls need separate workspaces unless they are ordered
 * on one stream.  Arguments only the general kernel takes (K not a multiple
 * of 8 or above 2^21, A or B not 16-byte aligned), K = 0, and a plan with
 * one split run gemm_f16_nt itself, with the same result.  Otherwise the
 * same semantics, ownership and status codes as gemm_f16_nt, plus
 * GEMM_F16_INVALID_ARG for splits > 64.
 *
 * gemm_f16_nt_splitk_with_config: the same with the kernel configuration
 * fixed (config_id < 0: the planner's choice), for tests and sweeps.  Its
 * effective split count follows the forced configuration's K slice, so the
 * workspace the plan above reports may not suffice for it;
 * gemm_f16_splitk_workspace_bytes gives a size that does.
 *
 * gemm_f16_splitk_workspace_bytes: pure host function.  The workspace bytes
 * that any configuration of any layout needs for at most `splits` ranges of
 * an M x N output: splits slices of M N fp32 partials, each rounded up to 64
 * elements (0 for splits <= 1).  GEMM_F16_INVALID_ARG for NULL output,
 * negative sizes or splits outside 0..64; GEMM_F16_UNSUPPORTED for M or N
 * above 2^31 - 1.
 */
int gemm_f16_splitk_workspace_bytes(int64_t M, int64_t N, int32_t splits,
                                    int64_t *workspace_bytes);
int gemm_f16_nt_splitk_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                            int32_t splits, gemm_f16_nt_plan_t *plan,
                            int32_t *splits_out, int64_t *workspace_bytes);
int gemm_f16_nt_splitk(int64_t M, int64_t N, int64_t K,
                       const void *A, const void *B, void *C,
                       int32_t splits, void *workspace, int64_t workspace_bytes,
                       hipStream_t stream);
int gemm_f16_nt_splitk_with_config(int64_t M, int64_t N, int64_t K,
                                   const void *A, const void *B, void *C,
                                   int32_t splits, void *workspace,
                                   int64_t workspace_bytes, hipStream_t stream,
                                   int32_t config_id);

/*
 * gemm_f16_nt_splitk_noalloc: gemm_f16_nt_splitk for callers that cannot
 * allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  It takes no workspace: the fp32
 * partials go to a fixed array inside the library (64 MiB per GPU, held by
 * each GPU the library runs on until the process ends), and the call itself
 * allocates nothing.  Same plan, kernels and result bits as
 * gemm_f16_nt_splitk(M, N, K, A, B, C, splits, <workspace>, ..., stream)
 * with a large enough workspace, and the same status codes, plus
 * GEMM_F16_SCRATCH_LIMIT when the planned partials (the workspace bytes
 * gemm_f16_nt_splitk_plan reports) exceed 64 MiB: pass a smaller `splits`.
 * The array needs no clearing (every partial it holds is written before it
 * is read), but every call on one GPU shares it: calls that may overlap on
 * one GPU (different streams, or other host threads) race, and must be
 * ordered by the caller, e.g. on one stream.
 */
int gemm_f16_nt_splitk_noalloc(int64_t M, int64_t N, int64_t K,
                               const void *A, const void *B, void *C,
                               int32_t splits, hipStream_t stream);

/*
 * The split over K for the other layouts: the same semantics, planner,
 * workspace rules and status codes as the gemm_f16_nt_splitk functions
 * above, for the operands stored as gemm_f16_nn, gemm_f16_tn and gemm_f16_tt
 * take them.  Arguments only the layout's general kernel takes run it
 * without a split (as gemm_f16_nt_splitk does for NT), and K = 0 writes +0.
 */
int gemm_f16_nn_splitk_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                            int32_t splits, gemm_f16_nt_plan_t *plan,
                            int32_t *splits_out, int64_t *workspace_bytes);
int gemm_f16_nn_splitk(int64_t M, int64_t N, int64_t K,
                       const void *A, const void *B, void *C,
                       int32_t splits, void *workspace, int64_t workspace_bytes,
                       hipStream_t stream);
int gemm_f16_nn_splitk_with_config(int64_t M, int64_t N, int64_t K,
                                   const void *A, const void *B, void *C,
                                   int32_t splits, void *workspace,
                                   int64_t workspace_bytes, hipStream_t stream,
                                   int32_t config_id);
int gemm_f16_tn_splitk_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                            int32_t splits, gemm_f16_nt_plan_t *plan,
                            int32_t *splits_out, int64_t *workspace_bytes);
int gemm_f16_tn_splitk(int64_t M, int64_t N, int64_t K,
                       const void *A, const void *B, void *C,
                       int32_t splits, void *workspace, int64_t workspace_bytes,
                       hipStream_t stream);
int gemm_f16_tn_splitk_with_config(int64_t M, int64_t N, int64_t K,
                                   const void *A, const void *B, void *C,
                                   int32_t splits, void *workspace,
                                   int64_t workspace_bytes, hipStream_t stream,
                                   int32_t config_id);
int gemm_f16_tt_splitk_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                            int32_t splits, gemm_f16_nt_plan_t *plan,
                            int32_t *splits_out, int64_t *workspace_bytes);
int gemm_f16_tt_splitk(int64_t M, int64_t N, int64_t K,
                       const void *A, const void *B, void *C,
                       int32_t splits, void *workspace, int64_t workspace_bytes,
                       hipStream_t stream);
int gemm_f16_tt_splitk_with_config(int64_t M, int64_t N, int64_t K,
                                   const void *A, const void *B, void *C,
                                   int32_t splits, void *workspace,
                                   int64_t workspace_bytes, hipStream_t stream,
                                   int32_t config_id);

/*
 * Autotuning (the pages pick each kernel version's tile sizes, stage count
 * and K depth by timing a search space of compile-time configurations:
 * Tilus tutorial "Hopper matmul", page "2. Multi-Stage Software Pipelining",
 * Multi-Stage Shared Memory and the results; page "3. Warp Specialization",
 * the results; page "6. Register Reallocation, Multicast, and a Persistent
 * Kernel", the closing caution on other shapes).  Here the search space
 * is the library's compiled configurations of one operand layout, each run
 * unsplit and, where the unsplit grid leaves the GPU under-filled, with K
 * split several ways.
 *
 * `layout` = 2 * (A stored [K, M]) + (B stored [K, N]): 0 NT (gemm_f16_nt),
 * 1 NN (gemm_f16_nn), 2 TT (gemm_f16_tt), 3 TN (gemm_f16_tn).
 *
 * One candidate: a configuration id and an effective split count (1 = no
 * split).  Replaying it is gemm_f16_<layout>_splitk_with_config(M, N, K, A,
 * B, C, splits, workspace, workspace_bytes, stream, config_id), whose result
 * for one split equals that of gemm_f16_<layout>_with_config.
 */
typedef struct gemm_f16_tune_entry_t {
    int32_t config_id;
    int32_t splits;     /* effective split count, 1 = no split */
    int32_t status;     /* status of the candidate's calls (gemm_f16_autotune) */
    float ms;           /* average time per call in ms, -1 when not timed */
} gemm_f16_tune_entry_t;

/*
 * gemm_f16_autotune_candidates: pure host function.  Lists the candidates
 * gemm_f16_autotune would time for (M, N, K) on `num_cus` compute units, in
 * the order it times them: every configuration of `layout` that can take the
 * arguments (only the layout's general kernel when they do not suit the
 * direct-to-LDS configurations; `aligned` != 0 says A and B are 16-byte
 * aligned), each unsplit and then with each distinct effective split count
 * (K per range at least 256) while the unsplit tiles fill fewer than 4 rounds
 * of the grid, up to 16 rounds of work units, whose fp32 partials fit in
 * `workspace_bytes`.  Writes the first min(count, max_entries) candidates to
 * `entries` (status 0, ms -1), the count to *n_entries, and to
 * *workspace_needed the workspace bytes that the largest split candidate
 * needs regardless of `workspace_bytes` (0 without split candidates).
 * M, N or K = 0: no candidates.  GEMM_F16_INVALID_ARG for a layout outside
 * 0..3, negative sizes or workspace_bytes, num_cus <= 0, max_entries < 0,
 * entries NULL with max_entries > 0, or NULL n_entries or workspace_needed.
 *
 * gemm_f16_autotune: times every candidate above on the caller's buffers and
 * the current device, on `stream`: one untimed call, then `iters` calls
 * between two HIP events; `ms` is the event time over `iters`.  Before the
 * first candidate is timed, it runs for about 50 ms (in batches of `iters`),
 * so that the GPU's clock has ramped up from idle.  It blocks
 * until each candidate's events have completed (so it is not for graph
 * capture).  `workspace` (caller-owned device memory, 16-byte aligned, not
 * overlapping A, B or C; NULL when workspace_bytes = 0) bounds the split
 * candidates as above.  Candidates that a layout's kernels reject record
 * GEMM_F16_UNSUPPORTED and are skipped; any other failure stops the search
 * and is returned.  On success *best is the fastest candidate and C holds its
 * result (it is run once more last; C's contents are otherwise those of the
 * last call).  `entries` receives up to max_entries timed candidates in
 * order, *n_entries (may be NULL) their count.  M or N = 0: no call, *best =
 * {-1, 1, 0, 0}; K = 0: C is filled with +0 and *best = {-1, 1, 0, 0}.
 * GEMM_F16_INVALID_ARG for a layout outside 0..3, iters outside 1..10000,
 * NULL best, entries NULL with max_entries > 0, or the arguments
 * gemm_f16_<layout> rejects; the library allocates no device memory.
 */
int gemm_f16_autotune_candidates(int32_t layout, int64_t M, int64_t N, int64_t K,
                                 int32_t num_cus, int32_t aligned, int64_t workspace_bytes,
                                 gemm_f16_tune_entry_t *entries, int32_t max_entries,
                                 int32_t *n_entries, int64_t *workspace_needed);
int gemm_f16_autotune(int32_t layout, int64_t M, int64_t N, int64_t K,
                      const void *A, const void *B, void *C,
                      void *workspace, int64_t workspace_bytes, int32_t iters,
                      hipStream_t stream, gemm_f16_tune_entry_t *best,
                      gemm_f16_tune_entry_t *entries, int32_t max_entries,
                      int32_t *n_entries);

/*
 * The tile order the kernel walks (Tilus tutorial "Hopper matmul", page
 * "4. Pipeline Abstraction and Two Consumer Warp Groups", Tile
 * Rasterization; page "6. ...", Persistent Tile Loop), exposed so that host
 * tests run the very same function the device runs.  Pure host function.
 * `slot` = round * grid + workgroup.  Writes the output tile (tile_m, tile_n)
 * that this slot computes; returns GEMM_F16_INVALID_ARG when slot is out of
 * [0, plan->tiles).
 */
int gemm_f16_nt_tile_of_slot(const gemm_f16_nt_plan_t *plan, int64_t slot,
                             int32_t *tile_m, int32_t *tile_n);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F16_NT_H */

/*
 * sgemm.h -- FP32 GEMM for AMD Instinct MI355X (gfx950), C ABI.
 *
 * Operation (page "GEMM 优化之路", problem statement and performance limit):
 *
 *     C = alpha * A * B + beta * C
 *
 * with A of size M x K, B of size K x N and C of size M x N, all row-major
 * FP32.  This ABI adds explicit leading dimensions (the page uses K, N, N):
 *     A(i,k) = A[i*lda + k],  B(k,j) = B[k*ldb + j],  C(i,j) = C[i*ldc + j].
 * sgemm_run_ex also takes transposed storage (the A^T*B and A*B^T cases of
 * the gsyq.cn GEMM guide, section 6.4 step 8): with transa = SGEMM_OP_T, A is
 * stored K x M and A(i,k) = A[k*lda + i]; with transb = SGEMM_OP_T, B is
 * stored N x K and B(k,j) = B[j*ldb + k].
 * Only the M x N window of C is written; every other element of the C buffer
 * is left untouched.
 *
 * Conventions (the page always evaluates beta*C; the library follows BLAS):
 *   - beta == 0: C is not read, so it may hold anything, NaN included.
 *   - K == 0: C = beta*C (zeros when beta == 0).
 *   - M == 0 or N == 0: nothing is launched; the call returns SGEMM_OK.
 *   - The summation order inside each output is unspecified but fixed: the
 *     same inputs on the same device give the same bits on every call.
 *     Accuracy: |C - exact| <= 4*max(K,1)*2^-24*(|alpha|*sum_k|a_ik*b_kj|
 *     + |beta*c_ij|) elementwise; results are exact whenever every partial
 *     sum is an integer below 2^24.
 *
 * Memory: A, B and C are device pointers owned by the caller, who also owns
 * the stream.  C must not overlap A or B.  The library allocates no device
 * memory.  The handle holds host-side state (device id, CU count, kernel
 * choice) and, only if the caller sets one with sgemm_set_workspace, the
 * address and size of a caller-owned device workspace.  Only two kinds of
 * plan touch that workspace: STREAM_K launches (partial tiles) and SMALL_M
 * launches with more than one K range (partial sums of the ranges); every
 * other plan neither reads nor writes it.  Problems such as 128^3, 1024^3,
 * 4096^3, 1000 x 1500 x 777 and 4096 x 11008 x 4096 plan one output tile per
 * workgroup (TILES) and never use it, with or without a workspace.
 *
 * Errors: every function returns SGEMM_OK (0) or a negative status; no
 * function aborts or prints.  Argument errors are found on the host before
 * any HIP call.  sgemm_run is asynchronous: a fault during execution shows
 * up at the next synchronisation of the stream, as for any HIP kernel.
 *
 * Threading: sgemm_run does not modify the handle.  Calls on one handle may
 * overlap in time (several host threads, or several streams) only when the
 * handle has no workspace: with one, STREAM_K and multi-range SMALL_M plans
 * of overlapping calls write the same partial-sum slots and corrupt each
 * other's results, so calls that may overlap need separate handles, each
 * with its own workspace (or none).  sgemm_set_variant / sgemm_set_kernel /
 * sgemm_set_workspace / sgemm_destroy must not race with sgemm_run on the
 * same handle.
 */
#ifndef SGEMM_H_
#define SGEMM_H_

#include <hip/hip_runtime_api.h> /* hipStream_t */
#include <stddef.h>                /* size_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sgemm_handle_s* sgemm_handle_t;

enum sgemm_status {
  SGEMM_OK = 0,
  SGEMM_ERR_HANDLE = -1, /* null handle, or null out-pointer in sgemm_create */
  SGEMM_ERR_SIZE = -2,   /* M, N or K negative */
  SGEMM_ERR_LD = -3,     /* lda < max(1,K), ldb < max(1,N) or ldc < max(1,N) */
  SGEMM_ERR_NULL = -4,   /* null A/B/C where it would be read or written */
  SGEMM_ERR_HIP = -5,    /* a HIP runtime call failed (launch, device query) */
  SGEMM_ERR_DEVICE = -6, /* no device, not gfx950, or not the handle's device */
  SGEMM_ERR_VALUE = -7,  /* unknown variant or kernel id */
  SGEMM_ERR_ALIAS = -8,  /* the C window overlaps the A or B window */
  SGEMM_ERR_UNSUPPORTED = -9, /* forced kernel cannot run these arguments */
  SGEMM_ERR_SCRATCH = -10  /* sgemm_run_ex_noalloc: forced kernel needs more
                              than SGEMM_SCRATCH_BYTES of scratch */
};

/* Operand storage for sgemm_run_ex: as stated (N) or transposed (T). */
enum sgemm_op {
  SGEMM_OP_N = 0,
  SGEMM_OP_T = 1
};

/* Kernel families.  MFMA uses the FP32 matrix cores (v_mfma_f32_32x32x2_f32);
 * VALU uses per-lane FMA outer products on the vector ALUs (stored operands
 * only, no transposes).  AUTO = MFMA. */
enum sgemm_variant {
  SGEMM_VARIANT_AUTO = 0,
  SGEMM_VARIANT_MFMA = 1,
  SGEMM_VARIANT_VALU = 2
};

/* Problem sizes a kernel takes (sgemm_kernel_info).  Every tile shape comes
 * in these instances; sgemm_run uses the first that fits.
 *   ALIGNED: M % bm == N % bn == K % bk == 0 (the VALU kernel also needs lda
 *            and ldb multiples of 4 and 16-byte aligned A and B).  All
 *            operand tiles move by direct global-to-LDS loads.
 *   EDGE:    any M, N, K with M >= 4 when A is stored transposed and N >= 4
 *            when B is stored as stated (the extents along which 16-byte
 *            pieces run).  Whole K steps use direct loads (rows and columns
 *            past the edge read the last valid one, or the piece that
 *            straddles the edge is read as it is; either only feeds outputs
 *            that are never stored); a partial last K step, and the last K
 *            row when a piece can straddle, go through registers with zero
 *            fill.
 *   GUARDED: any sizes; every operand tile goes through registers with zero
 *            fill past the edges ("GEMM 优化之路", exercise 2).
 * MFMA kernels need only 4-byte aligned A and B (16-byte global loads on
 * gfx950 take any 4-byte aligned address). */
enum sgemm_mode {
  SGEMM_MODE_ALIGNED = 0,
  SGEMM_MODE_EDGE = 1,
  SGEMM_MODE_GUARDED = 2
};

/* How a kernel spreads work over workgroups (sgemm_kernel_schedule).
 *   TILES:    one output tile per workgroup, all of K.
 *   STREAM_K: a grid of (CUs x a small count) workgroups that each take an
 *             equal, contiguous share of the tiles x K-steps iteration space,
 *             so a tile count that is not a multiple of the CU count leaves
 *             no CU idle.  A tile split between workgroups is written as
 *             partial sums to the handle's workspace (sgemm_set_workspace)
 *             and a second kernel adds them in K order and applies alpha and
 *             beta: the result is deterministic.  Chosen only when the
 *             handle has a workspace of sgemm_workspace_size bytes (the
 *             load-balancing schedule of the tiles-and-K-steps split; the
 *             pages' "split-K" next step).
 *   SMALL_M:  M <= the kernel's bm (1, 2, 4, 8 or 16): vector-ALU kernels
 *             that stream B once with 16-byte loads, for decode-like
 *             products.
 *             B stored K x N: either one pass (bm 1, 2, 4 or 8; bn = 32
 *             columns of C per workgroup over all of K, its waves on
 *             contiguous runs of K, sums added in a fixed order, no
 *             workspace) or, bm 4, 8 or 16, 256 columns of C per workgroup
 *             and K split over enough workgroups to give every CU one; with
 *             more than one K range the ranges' sums go to the workspace and
 *             a second kernel adds them in range order and applies alpha and
 *             beta (deterministic); without a workspace (or when it is too
 *             small) the ranges are merged until they fit, down to one.
 *             B stored N x K (bm 1, 2, 4 or 8): one pass, bn = 8 (bm <= 2)
 *             or 4 columns of C per workgroup over all of K, its waves on
 *             contiguous runs of K and the lanes along K, sums added in a
 *             fixed order, no workspace.  Chosen for the AUTO and VALU
 *             variants only. */
enum sgemm_schedule {
  SGEMM_SCHEDULE_TILES = 0,
  SGEMM_SCHEDULE_STREAM_K = 1,
  SGEMM_SCHEDULE_SMALL_M = 2
};

/* Create a handle bound to the current HIP device, which must be gfx950.
 * On success *out receives the handle.  Returns SGEMM_ERR_HANDLE if out is
 * NULL, SGEMM_ERR_DEVICE or SGEMM_ERR_HIP if the device cannot be used. */
int sgemm_create(sgemm_handle_t* out);

/* Enqueue C = alpha*A*B + beta*C on `stream` (0 = the null stream) and
 * return without waiting.  The current device must be the handle's device.
 * Sizes and leading dimensions are in elements.  Arguments are checked as in
 * sgemm_validate before anything is launched. */
int sgemm_run(sgemm_handle_t h, int M, int N, int K, float alpha,
              const float* A, int lda, const float* B, int ldb, float beta,
              float* C, int ldc, hipStream_t stream);

/* As sgemm_run, with operand storage transa / transb (SGEMM_OP_N or
 * SGEMM_OP_T, else SGEMM_ERR_VALUE).  Leading dimensions must cover the
 * stored rows: lda >= max(1, transa ? M : K), ldb >= max(1, transb ? K : N).
 * SGEMM_ERR_UNSUPPORTED if the handle's variant or forced kernel has no
 * kernel for this storage (the VALU family reads stored operands only). */
int sgemm_run_ex(sgemm_handle_t h, int transa, int transb, int M, int N,
                 int K, float alpha, const float* A, int lda, const float* B,
                 int ldb, float beta, float* C, int ldc, hipStream_t stream);

/* Free the handle.  NULL is a no-op returning SGEMM_OK.  A workspace set on
 * the handle stays the caller's to free. */
int sgemm_destroy(sgemm_handle_t h);

/* Device memory the stream-K kernels (partial tiles) and the small-M kernels
 * (partial sums of K ranges) may use: `bytes` at `workspace` (16-byte
 * aligned, on the handle's device, owned by the caller and kept alive while
 * calls that may use it are in flight).  NULL with bytes 0 removes it.
 * Without a workspace of at least sgemm_workspace_size bytes no stream-K
 * kernel is planned (a forced one returns SGEMM_ERR_UNSUPPORTED); the
 * small-M kernels split K only as far as the workspace holds.  Calls on one handle share the workspace: calls
 * that may overlap in time (different streams) need handles with separate
 * workspaces.  SGEMM_ERR_NULL for NULL with bytes > 0, SGEMM_ERR_VALUE for a
 * misaligned pointer. */
int sgemm_set_workspace(sgemm_handle_t h, void* workspace, size_t bytes);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * call as sgemm_run_ex, with the same checks, results and determinism, but
 * the stream-K and small-M kernels keep their partial sums in a buffer of
 * the library's own -- a fixed device array of SGEMM_SCRATCH_BYTES (16 MiB)
 * per GPU, set up by sgemm_create and held until the process ends -- in
 * place of the handle's workspace, which this call ignores.  It calls no
 * allocating routine.  Plans are made for that buffer's size (stream-K with
 * 64 x 64 tiles, small-M K splits up to 16 MiB of partial sums); a forced
 * stream-K kernel that needs more returns SGEMM_ERR_SCRATCH before anything
 * is launched.  Every call on one GPU shares that GPU's buffer and leaves
 * its contents behind (no kernel needs it zeroed): calls that may overlap
 * in time on one GPU (several streams or host threads) race on it and must
 * not be made.  SGEMM_ERR_HIP if the buffer's set-up failed on this device.
 * Other statuses as sgemm_run_ex. */
#define SGEMM_SCRATCH_BYTES (16u << 20)
int sgemm_run_ex_noalloc(sgemm_handle_t h, int transa, int transb, int M, int N,
                         int K, float alpha, const float* A, int lda, const float* B,
                         int ldb, float beta, float* C, int ldc, hipStream_t stream);

/* Bytes of workspace that let every stream-K kernel run on the handle's
 * device (two partial tiles per stream-K workgroup; 64 MiB on 256 CUs). */
int sgemm_workspace_size(sgemm_handle_t h, size_t* bytes);

/* ---- host-only helpers (no HIP call, no device needed) ---------------- */

/* The argument checks of sgemm_run: sizes, leading dimensions, null
 * pointers (only where an operand is actually touched) and C overlapping
 * A or B.  Returns SGEMM_OK or the status sgemm_run would return. */
int sgemm_validate(int M, int N, int K, const float* A, int lda,
                   const float* B, int ldb, float beta, const float* C,
                   int ldc);
/* The checks of sgemm_run_ex (storage flags, stored shapes). */
int sgemm_validate_ex(int transa, int transb, int M, int N, int K,
                      const float* A, int lda, const float* B, int ldb,
                      float beta, const float* C, int ldc);

/* Static text for a status code ("unknown status" for other values). */
const char* sgemm_status_string(int status);

/* Kernel table.  Ids run from 0 to sgemm_num_kernels()-1. */
int sgemm_num_kernels(void);
const char* sgemm_kernel_name(int kernel_id); /* NULL for a bad id */
/* Tile shape and properties of a kernel; any out-pointer may be NULL.
 * bk is the K granularity (K values per LDS stage).  *mode receives the
 * SGEMM_MODE_* of the instance (which sizes it takes).  transa / transb give
 * the operand storage the kernel reads. */
int sgemm_kernel_info(int kernel_id, int* variant, int* bm, int* bn, int* bk,
                      int* threads, int* mode, int* transa, int* transb);

/* How sgemm_run splits a call: it returns the number of launches (1 or 2)
 * or a negative status.  kernels[0] (and kernels[1], else -1) receive the
 * kernel ids; *n_split receives the first column of the second launch (N
 * when there is one launch).  A second launch covers columns
 * [n_split, N) after the first covers [0, n_split); it is used when whole
 * rounds of a large tile plus a finer tile for the rest beat one launch.
 * kernels and n_split may be NULL.  Pure function of its inputs. */
int sgemm_plan(int variant, int M, int N, int K, const float* A, int lda,
               const float* B, int ldb, const float* C, int ldc,
               int* kernels, int* n_split);
/* sgemm_plan for sgemm_run_ex's operand storage.  sgemm_plan and
 * sgemm_plan_ex plan for 256 CUs and no workspace (so never stream-K). */
int sgemm_plan_ex(int variant, int transa, int transb, int M, int N, int K,
                  const float* A, int lda, const float* B, int ldb,
                  const float* C, int ldc, int* kernels, int* n_split);
/* Exactly the plan sgemm_run_ex follows on handle h: its variant, forced
 * kernel, CU count and workspace.  Returns the number of launches (0 when M
 * or N is 0) or the status sgemm_run_ex would return; launches nothing. */
int sgemm_plan_handle(sgemm_handle_t h, int transa, int transb, int M, int N,
                      int K, const float* A, int lda, const float* B, int ldb,
                      const float* C, int ldc, int* kernels, int* n_split);

/* SGEMM_SCHEDULE_* of a kernel, or SGEMM_ERR_VALUE for a bad id. */
int sgemm_kernel_schedule(int kernel_id);

/* The kernel of sgemm_run's first launch for these arguments and variant
 * (SGEMM_VARIANT_*), or a negative status.  Pure function of its inputs. */
int sgemm_select_kernel(int variant, int M, int N, int K, const float* A,
                        int lda, const float* B, int ldb, const float* C,
                        int ldc);

/* Diagnostics: the workgroup -> output-tile mapping of the kernels with
 * square tiles (XCD-contiguous renumbering, then bands of tile rows sized so
 * one XCD's share of the tiles is a near-square block; kernels whose tiles
 * are taller than wide use shorter bands, so that the block stays no taller
 * than wide in elements).  nwg must equal tiles_m*tiles_n; for wg in
 * [0, nwg) it stores the tile's row and column indices. */
void sgemm_tile_coords(int wg, int nwg, int tiles_m, int tiles_n, int* tm,
                       int* tn);

/* Diagnostics: launch `workgroups` workgroups of 256 lanes that each run
 * `iterations` rounds of eight independent v_mfma_f32_32x32x2_f32 with no
 * memory traffic (4096 flops per MFMA per wave, 4 waves per workgroup), then
 * write one float per lane to `out` (device memory of workgroups*256 floats,
 * owned by the caller).  Timing it on `stream` gives the matrix-core rate
 * the device sustains, the ceiling for the SGEMM kernels.  Asynchronous;
 * returns SGEMM_ERR_SIZE / SGEMM_ERR_NULL / SGEMM_ERR_HIP on bad input or a
 * failed launch. */
int sgemm_diag_mfma_chain(int workgroups, int iterations, float* out,
                          hipStream_t stream);

/* Diagnostics: the shader clock the product itself runs at.  The same
 * call as sgemm_run_ex (same checks, same plan on handle h), when that plan
 * is one launch of a one-tile-per-workgroup MFMA kernel; the first lane of
 * workgroup w also stores the shader cycle counter and the constant-rate
 * wall clock when the workgroup starts and after all its waves are done:
 * stamps[4*w .. 4*w+3] = {cycles_start, cycles_end, wall_start, wall_end}.
 * (cycles_end - cycles_start) / (wall_end - wall_start) * the wall clock's
 * rate (sgemm_diag_wall_clock_khz) is the clock that tile ran at.  `stamps`
 * is caller-owned device memory of 4*stamp_slots long longs.  Returns the
 * number of workgroups stamped (> 0), SGEMM_ERR_NULL for null stamps,
 * SGEMM_ERR_SIZE if stamp_slots is smaller than that number,
 * SGEMM_ERR_UNSUPPORTED for an empty problem or any other plan, or the
 * status sgemm_run_ex would return.  Asynchronous. */
int sgemm_diag_run_clocked(sgemm_handle_t h, int transa, int transb, int M, int N,
                           int K, float alpha, const float* A, int lda,
                           const float* B, int ldb, float beta, float* C, int ldc,
                           long long* stamps, int stamp_slots, hipStream_t stream);

/* The current device's wall-clock counter rate in kHz (the rate of the
 * counter sgemm_diag_run_clocked reads as wall time).  SGEMM_ERR_NULL for a null
 * out-pointer, SGEMM_ERR_DEVICE / SGEMM_ERR_HIP if it cannot be queried. */
int sgemm_diag_wall_clock_khz(int* khz);

/* ---- products with 16-bit or 8-bit A and B --------------------------------
 *
 * Operation (the gsyq.cn GEMM guide, section 5.1: matrix units multiply
 * 16-bit inputs and accumulate in FP32):
 *
 *     C = alpha * op(A) * op(B) + beta * C
 *
 * with A and B stored in a 16-bit or 8-bit format (dtype) and C, alpha, beta
 * FP32.  Storage, leading dimensions (in elements), transa / transb, the
 * M x N window of C, the beta == 0 and K == 0 conventions and the
 * determinism of sgemm_run_ex hold unchanged.  A and B hold bit patterns:
 * SGEMM_DTYPE_BF16 is bfloat16 (the upper half of an IEEE binary32),
 * SGEMM_DTYPE_F16 IEEE binary16, SGEMM_DTYPE_FP8_E4M3 and _E5M2 the OCP
 * 8-bit formats.  Every product of two such values is exact in FP32, so for
 * the 16-bit formats the accuracy statement of sgemm_run holds as it is:
 * |C - exact| <= 4*max(K,1)*2^-24*(|alpha|*sum_k|a_ik*b_kj| + |beta*c_ij|)
 * against the exact product of the stored values.  The 8-bit formats carry
 * no such bound: their matrix instructions sum each block of consecutive
 * products (64 in the tile kernels' 32x32x64 instruction, 128 in the
 * small-M kernels' 16x16x128 one) in a fixed-point window below the block's
 * largest product before the FP32 accumulation, and their rounding there is
 * not documented.  For them the library gives only a measured envelope: on
 * uniform, one-signed, small-normal and seven-binade inputs the error stayed
 * under 2^-11 of each 64-product block's largest product, and the tests
 * accept the bound above plus 2^-9*|alpha|*ceil(K/64)*max_k|a_ik|*max_k|b_kj|.  What is exact: integer
 * inputs in [-4, 4] (every product and block sum far inside the window) give
 * bit-exact results, as for FP32; a block that holds products of very
 * different size (448*448 beside 1*1) may lose the small ones.  Infinities
 * and NaNs in A or B
 * propagate as the matrix unit's FP32 arithmetic makes them; finite inputs
 * whose products or sums overflow FP32 give infinities.  Every format takes
 * every storage; an operand stored with its outer index contiguous (A as
 * K x M, B as K x N) is read through the LDS transposing reads, which for
 * 8-bit formats costs some speed (4096^3: ~75 us against ~67 us with A
 * stored M x K and B N x K).
 *
 * Memory: A and B are device pointers to 2-byte (16-bit formats) or 1-byte
 * elements, 16-bit ones at least 2-byte aligned (SGEMM_ERR_VALUE otherwise);
 * no kernel needs more.  Kernels (sgemm_lowp_kernel_info): ALIGNED takes M
 * and N multiples of the tile (64, 128 or 256) and K a multiple of the K
 * step (bk: 64 for 16-bit formats, 128 for 8-bit ones); EDGE any sizes with
 * M of at least one 16-byte piece (8 elements of a 16-bit format, 16 of an
 * 8-bit one) when A is stored K x M and N likewise when B is stored K x N;
 * GUARDED (64 x 64 only) any sizes; the one-pass small-M kernels (bm = bn =
 * 16, bk = one 16 x 16 MFMA block: 32 k of a 16-bit format, 128 of an 8-bit
 * one) take M <= 16 with B stored N x K, any N, K and alignment.
 * Ownership, streams, errors and threading as for sgemm_run; the handle's
 * workspace, when set, also serves the split-K kernels of products with few
 * rows (sgemm_lowp_kernel_schedule). */
enum sgemm_dtype {
  SGEMM_DTYPE_BF16 = 1,
  SGEMM_DTYPE_F16 = 2,
  SGEMM_DTYPE_FP8_E4M3 = 3, /* OCP 8-bit: 4 exponent bits, bias 7, no inf */
  SGEMM_DTYPE_FP8_E5M2 = 4  /* OCP 8-bit: 5 exponent bits, bias 15 */
};

/* Enqueue the 16-bit or 8-bit product on `stream` and return without
 * waiting.  SGEMM_ERR_VALUE for an unknown dtype or storage flag or a
 * misaligned A or B; SGEMM_ERR_UNSUPPORTED when a forced kernel
 * (sgemm_set_lowp_kernel) cannot run the arguments; other statuses as
 * sgemm_run_ex. */
int sgemm_run_lowp(sgemm_handle_t h, int dtype, int transa, int transb, int M,
                   int N, int K, float alpha, const void* A, int lda,
                   const void* B, int ldb, float beta, float* C, int ldc,
                   hipStream_t stream);

/* The argument checks of sgemm_run_lowp (host only, no HIP call). */
int sgemm_validate_lowp(int dtype, int transa, int transb, int M, int N, int K,
                        const void* A, int lda, const void* B, int ldb,
                        float beta, const float* C, int ldc);

/* Kernel table of the 16-bit and 8-bit products (ids 0 ..
 * sgemm_lowp_num_kernels()-1).  *mode is SGEMM_MODE_ALIGNED,
 * SGEMM_MODE_EDGE or SGEMM_MODE_GUARDED; bk is the K step (64 for 16-bit
 * formats, 128 for 8-bit ones; the one-pass small-M kernels: one MFMA
 * block, 32 or 128). */
int sgemm_lowp_num_kernels(void);
const char* sgemm_lowp_kernel_name(int kernel_id); /* NULL for a bad id */
int sgemm_lowp_kernel_info(int kernel_id, int* dtype, int* bm, int* bn,
                           int* bk, int* threads, int* mode, int* transa,
                           int* transb);

/* SGEMM_SCHEDULE_* of a kernel of the 16-bit/8-bit table (SGEMM_ERR_VALUE
 * for a bad id).  SGEMM_SCHEDULE_SMALL_M marks two kinds of kernels for
 * products with few rows, used when 64 x 64 tiles would fill at most half
 * the CUs:
 *   one pass ("_G16x16_..._small"): M <= 16 and B stored N x K.  Each
 *     workgroup takes 16 columns of C over all of K; its waves feed 16 x 16
 *     MFMAs straight from memory (no LDS tiles), split K and add their
 *     partial blocks through LDS in wave order.  No workspace, one launch,
 *     deterministic.  Taken first, with or without a workspace (16-bit
 *     formats with more than four rows: only when split K does not run).
 *   split K ("_sk_edge"): M <= 64, any storage, a workspace on the handle
 *     (sgemm_set_workspace).  K is split into ranges of whole K steps (at
 *     least four each) so that the workgroups reach two per CU, each range's
 *     partial sums go to the workspace ([split][M][N rounded up to 4]
 *     floats), and a second kernel adds them in range order and applies
 *     alpha and beta (deterministic).  Without a workspace they are not used
 *     (a forced one returns SGEMM_ERR_UNSUPPORTED). */
int sgemm_lowp_kernel_schedule(int kernel_id);

/* The launch sgemm_run_lowp makes on handle h: *kernel receives the kernel
 * id and *splits the number of K ranges (1 unless a split-K kernel splits
 * K); either may be NULL.  Returns SGEMM_OK, or the status sgemm_run_lowp
 * would return (SGEMM_ERR_UNSUPPORTED for an empty problem); launches
 * nothing. */
int sgemm_lowp_plan_handle(sgemm_handle_t h, int dtype, int transa, int transb,
                           int M, int N, int K, const void* A, int lda,
                           const void* B, int ldb, const float* C, int ldc,
                           int* kernel, int* splits);

/* The kernel sgemm_run_lowp picks for these arguments on a 256-CU device
 * with no workspace (never a split-K kernel; the one-pass small-M kernel
 * where it applies), or a negative status.  Pure function of its inputs. */
int sgemm_lowp_select_kernel(int dtype, int transa, int transb, int M, int N,
                             int K, const void* A, int lda, const void* B,
                             int ldb, const float* C, int ldc);

/* Diagnostics: as sgemm_diag_mfma_chain with v_mfma_f32_32x32x16_bf16
 * (dtype SGEMM_DTYPE_BF16) or v_mfma_f32_32x32x16_f16 (SGEMM_DTYPE_F16),
 * 32768 flops per MFMA per wave, or v_mfma_scale_f32_32x32x64_f8f6f4 with
 * unit scales (SGEMM_DTYPE_FP8_E4M3 / SGEMM_DTYPE_FP8_E5M2), 131072 flops
 * per MFMA per wave; eight independent accumulators, no memory traffic: the
 * ceiling for the 16-bit and 8-bit product kernels.  SGEMM_ERR_VALUE for
 * another dtype. */
int sgemm_diag_mfma_chain_lowp(int dtype, int workgroups, int iterations,
                               float* out, hipStream_t stream);

/* Force one 16-bit product kernel on this handle (kernel_id >= 0) or go back
 * to automatic selection (-1).  A forced kernel whose mode, format or
 * storage cannot take the arguments makes sgemm_run_lowp return
 * SGEMM_ERR_UNSUPPORTED. */
int sgemm_set_lowp_kernel(sgemm_handle_t h, int kernel_id);

/* ---- handle options ----------------------------------------------------- */

/* Choose the kernel family used by sgemm_run on this handle. */
int sgemm_set_variant(sgemm_handle_t h, int variant);

/* Force one kernel of the table (kernel_id >= 0), or go back to automatic
 * selection (-1).  A forced kernel makes sgemm_run return
 * SGEMM_ERR_UNSUPPORTED for arguments its mode or storage cannot handle. */
int sgemm_set_kernel(sgemm_handle_t h, int kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_H_ */

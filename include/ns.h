/*
 * ns.h -- C ABI of the MI355X (gfx950) Newton-Schulz orthogonalisation library.
 *
 * The operation is the one defined on the DMuon documentation page
 * "Newton-Schulz 变体" (Newton-Schulz variants):
 *
 *   - section "精度流水线" (precision pipeline): X = G / (||G||_F + eps) in
 *     fp32, then X is cast to fp16 and iterated in fp16;
 *   - section "直接空间 NS（经典）" (direct space): per step
 *     X <- a_k X + b_k (X X^T) X + c_k (X X^T)^2 X on the full matrix;
 *   - section "Gram 空间 NS（Dao-AILab）" (Gram space), equations Z_k and
 *     Q_{k+1}: R = X X^T, Z_k = b_k R_k + c_k R_k^2,
 *     Q_{k+1} = Z_k Q_k + a_k Q_k, R evolved by recurrence, output Q X;
 *   - section "重启机制" (restart mechanism): before each listed step index
 *     Q is applied to X and R is rebuilt from X;
 *   - section "系数集" (coefficient sets): tables of (a_k, b_k, c_k) rows.
 *
 * The library computes on the short side: a matrix with more rows than
 * columns is transposed on the way in and back on the way out, so every
 * Gram matrix is min(m, n) square.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   Layout      Matrices are row-major: element (i, j) of an (m, n) matrix
 *               with leading dimension ld sits at base[i * ld + j]
 *               (ld counted in elements, ld >= n).
 *   Ownership   Every device pointer (inputs, outputs, workspace) belongs to
 *               the caller; the library never allocates or frees device
 *               memory. Host arrays (coeffs, restarts, the ns_matrix array)
 *               are read during the call only.
 *   Streams     `stream` is a hipStream_t passed as void* (NULL = the null
 *               stream). Calls enqueue work and return; results are valid
 *               once the stream reaches them. Outputs must not overlap
 *               inputs or the workspace; a matrix whose output range
 *               overlaps its own input range is refused (NS_ERR_INVALID_ARG),
 *               other overlaps are the caller's to avoid. Concurrent calls on
 *               different streams need different workspaces.
 *   Workspace   Device memory of the size the matching *_workspace_size
 *               function reports, 256-byte aligned (NS_ERR_WORKSPACE
 *               otherwise), with no required contents: every call writes
 *               what it reads. The call also writes its launch descriptors
 *               there, and the integer counters (reset by every call) with
 *               which the workgroups of a launch claim its last tiles.
 *   Graphs      A call enqueues kernel launches only (its descriptor tables
 *               travel as kernel arguments of small fill launches; there are
 *               no host-to-device copies, memsets or host waits), so it can
 *               be captured into a HIP graph and replayed, provided the
 *               captured buffers stay allocated and timing is disabled.
 *   Errors      Return codes only: nothing is printed and nothing is thrown.
 *               Argument checks run on the host before any device work; on
 *               any error other than NS_ERR_HIP nothing has been enqueued.
 *               Before launching, every byte range the planned kernels can
 *               read or write is checked on the host against the workspace
 *               buffers and the caller's matrices (NS_ERR_INTERNAL if one
 *               falls outside; ns_plan_check exposes the same check).
 *               NaN or Inf in the input propagate to the output.
 *   Device      The current HIP device must be a gfx950 GPU, otherwise
 *               NS_ERR_UNSUPPORTED.
 *   Determinism The same inputs on the same device give bitwise identical
 *               outputs: fixed tile and reduction order, no float atomics
 *               (which workgroup computes a claimed tile varies from run to
 *               run, how it is computed does not).
 *   Precision   Every stored intermediate is fp16; products accumulate in
 *               fp32; scalar epilogues are evaluated in fp32 and rounded
 *               once.
 */
#ifndef NSMI_NS_H
#define NSMI_NS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NS_OK = 0,
  NS_ERR_INVALID_ARG = 1,  /* a size, pointer, dtype or parameter is invalid */
  NS_ERR_UNSUPPORTED = 2,  /* no HIP device, or the device is not gfx950    */
  NS_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required   */
  NS_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed    */
  NS_ERR_INTERNAL = 5      /* the launch plan failed the library's own
                              bounds check (a library defect); nothing was
                              enqueued                                       */
} ns_status;

typedef enum { NS_DT_F32 = 0, NS_DT_BF16 = 1, NS_DT_F16 = 2 } ns_dtype;

/* Axis 1 of the page's section "后端分发" (backend dispatch): the algorithm.
 * Axis 2 (which SYRK kernel) has a single value here: this library's gfx950
 * MFMA kernels. */
typedef enum { NS_GRAM = 0, NS_DIRECT = 1 } ns_backend;

#define NS_MAX_STEPS 16

/* Iteration parameters (the page's NewtonSchulz(coefficients=...,
 * restart_iterations=...) arguments plus the normalisation eps).
 *   num_steps     K, 1 <= K <= NS_MAX_STEPS.
 *   coeffs        host array of 3*K floats a_0, b_0, c_0, a_1, ...; row k is
 *                 used at step k. Must be finite.
 *   restarts      host array of num_restarts step indices in [0, K-1]
 *                 (gram only, ignored by direct). Index 0 is a no-op,
 *                 duplicates are ignored. May be NULL if num_restarts == 0.
 *   eps           added to the Frobenius norm; finite and >= 0.            */
typedef struct {
  int num_steps;
  const float* coeffs;
  const int* restarts;
  int num_restarts;
  float eps;
} ns_params;

/* One matrix of a call.
 *   g, g_dtype, m, n, ldg   input G (device), fp32 / bf16 / fp16, (m, n)
 *                           row-major, m >= 1, n >= 1, ldg >= n.
 *   out, out_dtype, ldo     output (device), same (m, n) orientation as G,
 *                           fp16 (the iteration dtype) / bf16 / fp32 (both
 *                           taken from the fp32 accumulator of the last
 *                           product), ldo >= n.                              */
typedef struct {
  const void* g;
  ns_dtype g_dtype;
  int64_t m, n, ldg;
  void* out;
  ns_dtype out_dtype;
  int64_t ldo;
} ns_matrix;

/* Largest side accepted for m or n. */
#define NS_MAX_DIM 65536

/* Bytes of device workspace that ns_gram / ns_direct / ns_batched need for
 * these matrices (count >= 1; `mats[i].g/out` are not read). Pure host
 * computation. Writes *bytes. */
ns_status ns_workspace_size(const ns_matrix* mats, int count, ns_backend backend,
                            const ns_params* params, size_t* bytes);

/* Precision pipeline step 1 and 2 on one matrix: x = fp16(g / (||g||_F + eps))
 * with the norm accumulated in fp32 and the quotient rounded to nearest even.
 *   x, ldx           device output. If transpose_tall != 0 and m > n, x is
 *                    the (n, m) transpose of the result (the short-side
 *                    orientation the iteration uses); otherwise (m, n).
 *                    ldx >= number of columns of x.
 *   norm_out         device float receiving ||g||_F, or NULL.
 *   ws, ws_bytes     device workspace of ns_normalize_workspace_size bytes.
 */
ns_status ns_normalize_workspace_size(int64_t m, int64_t n, size_t* bytes);
ns_status ns_normalize(const void* g, ns_dtype g_dtype, int64_t m, int64_t n,
                       int64_t ldg, void* x, int64_t ldx, int transpose_tall,
                       float eps, float* norm_out, void* ws, size_t ws_bytes,
                       void* stream);

/* Direct-space NS on one matrix (the page's direct_newton_schulz /
 * NewtonSchulz("direct")). Restarts in params are ignored. */
ns_status ns_direct(const ns_matrix* mat, const ns_params* params, void* ws,
                    size_t ws_bytes, void* stream);

/* Gram-space NS on one matrix (the page's newton_schulz /
 * NewtonSchulz("gram")), with restarts. */
ns_status ns_gram(const ns_matrix* mat, const ns_params* params, void* ws,
                  size_t ws_bytes, void* stream);

/* NS on `count` independent matrices of mixed shapes, one kernel launch per
 * stage over all of them (tiles of larger matrices scheduled first). Each
 * output is bitwise equal to what ns_gram / ns_direct gives for that matrix
 * alone. count == 0 is a no-op. `mats` is a host array. */
ns_status ns_batched(const ns_matrix* mats, int count, ns_backend backend,
                     const ns_params* params, void* ws, size_t ws_bytes,
                     void* stream);

/* ns_batched without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments (minus the workspace),
 * results and errors as ns_batched, each output bitwise equal to it; the
 * workspace is instead a static device array of NS_NOALLOC_SCRATCH_BYTES
 * bytes inside the library, one per device, held until the process ends.
 * A call whose ns_workspace_size exceeds that returns NS_ERR_WORKSPACE
 * before any device work. The call allocates no device memory and no
 * pinned host memory, creates no events and never times its launches (its
 * first call on a device resolves the array's address there once).
 * Every call on a device shares that device's array, which keeps the last
 * call's contents (nothing in it needs clearing: each call writes all it
 * reads), so calls that overlap on one device race: order them on one
 * stream. */
#define NS_NOALLOC_SCRATCH_BYTES (128u << 20)
ns_status ns_batched_noalloc(const ns_matrix* mats, int count, ns_backend backend,
                             const ns_params* params, void* stream);

/* Column-sharded Gram NS on one matrix, the tensor-parallel route of the
 * pages (Newton-Schulz reference page, section "Gram 空间 NS": R is a sum of
 * local Gram matrices, so TP is exact through one all-reduce; article page,
 * section "6. 与TP的结合", distributed mode: the norm from a scalar
 * all-reduce of per-shard sums, and one Gram all-reduce per restart),
 * emulated on one device with `shards` virtual shards:
 *   * the working matrix X (s x l, short side first: columns of a wide G,
 *     rows of a tall G) is split into `shards` column blocks, shard i
 *     holding l / shards columns (one more for i < l % shards), each in its
 *     own buffers;
 *   * ||G||_F is formed over the whole matrix and shared by the shards;
 *   * every shard forms its partial Gram matrix R_i = X_i X_i^T (fp16, all
 *     shards in one launch); the all-reduce is a shard-order sum of the R_i
 *     accumulated in fp32 and rounded once to fp16;
 *   * the s x s Gram-space iteration runs once (every rank would hold an
 *     identical copy); at a restart each shard applies Q to its own columns
 *     and the partial Grams are reduced again; the output of shard i,
 *     Q X_i, fills its own columns (wide) or rows (tall) of `out`.
 * In exact arithmetic the result equals ns_gram's; with shards == 1 it is
 * bitwise equal to ns_gram. 1 <= shards <= NS_MAX_SHARDS and
 * shards <= max(m, n), else NS_ERR_INVALID_ARG; other arguments, the
 * workspace and errors as for ns_gram (the size comes from
 * ns_gram_sharded_workspace_size; `mat->g/out` are not read by it). */
#define NS_MAX_SHARDS 64
ns_status ns_gram_sharded_workspace_size(const ns_matrix* mat, int shards,
                                         const ns_params* params, size_t* bytes);
ns_status ns_gram_sharded(const ns_matrix* mat, int shards, const ns_params* params,
                          void* ws, size_t ws_bytes, void* stream);

/* One Muon optimizer step around the NS call, Gram backend, for a batch of
 * matrices (one launch per stage, like ns_batched). The article page
 * (section "1. Introduction", "2. Muon执行过程") says a Muon step keeps a
 * momentum M of the gradient, orthogonalises M approximately and uses the
 * result as the update direction; its formula itself is missing from the
 * extracted text, and the pages give only lr = 0.02 as an example. This
 * entry takes the plainest reading of that description:
 *   M <- beta * M + G                 (momentum, elementwise)
 *   W <- W - lr * scale * NS(M)       (NS = the Gram iteration of ns_gram
 *                                      on the updated M, same params)
 * with beta, lr and a per-matrix scale chosen by the caller (no value of
 * them is fixed by the pages; scale = 1 gives the plain update).
 * Fusion: the momentum update runs inside the norm pass (M read, updated
 * with one fp32 fma per element, rounded to M's type and written back, and
 * the norm taken of the stored values); the parameter update runs in the
 * epilogue of the final product (W read as C and written as D, the fp32
 * product Q X scaled by -lr * scale and added before W's one rounding), so
 * NS(M) is never stored.
 *   grad      (m, n) row-major, fp32/bf16/fp16, leading dim ld_grad, read;
 *   momentum  (m, n) row-major, any of the three types, ld_momentum, read
 *             and written;
 *   param     (m, n) row-major, any of the three types, ld_param, read and
 *             written.
 * The three buffers of a matrix must not overlap each other or another
 * matrix's. Validation, workspace (ns_muon_workspace_size; pointers are not
 * read by it), streams, errors and determinism as for ns_batched; beta,
 * lr and every scale must be finite. */
typedef struct {
  const void* grad;
  ns_dtype grad_dtype;
  int64_t m, n, ld_grad;
  void* momentum;
  ns_dtype momentum_dtype;
  int64_t ld_momentum;
  void* param;
  ns_dtype param_dtype;
  int64_t ld_param;
  float scale;
} ns_muon_matrix;
ns_status ns_muon_workspace_size(const ns_muon_matrix* mats, int count,
                                 const ns_params* params, size_t* bytes);
ns_status ns_muon_step(const ns_muon_matrix* mats, int count, const ns_params* params,
                       float beta, float lr, void* ws, size_t ws_bytes, void* stream);

/* Building blocks of the iteration, exposed for kernel-level testing.
 * All operands are fp16 row-major device matrices; products accumulate in
 * fp32 and the scaled sum is rounded once to fp16.
 *
 * ns_syrk: r = x x^T for x (s, l); r is (s, s) with leading dimension s and
 * is exactly symmetric (lower-triangle tiles computed, then mirrored). This
 * is the Gram product R = X X^T of the page's Gram-space section.
 * Requires s % 256 == 0 and l % 128 == 0 (dense: leading dims l and s).
 *
 * ns_gemm_nt: d = alpha * (a b^T) + beta * c + gamma * I for a (M, K) and
 * b (N, K) (so b^T is K x N), c and d (M, N); c may be NULL when beta == 0.
 * symmetric != 0 computes only the lower-triangle tiles (requires M == N)
 * and mirrors them, so d is exactly symmetric; use it only when the result
 * is symmetric in exact arithmetic. Requires M % 256 == 0, N % 256 == 0,
 * K % 128 == 0, dense leading dimensions (K for a and b, N for c and d).
 *
 * Both take a device workspace of at least NS_UNIT_WORKSPACE_BYTES bytes
 * (it holds the launch descriptor). */
#define NS_UNIT_WORKSPACE_BYTES 4096
ns_status ns_syrk(const void* x, int64_t s, int64_t l, void* r, void* ws,
                  size_t ws_bytes, void* stream);
ns_status ns_gemm_nt(const void* a, const void* b, const void* c, void* d,
                     int64_t M, int64_t N, int64_t K, float alpha, float beta,
                     float gamma, int symmetric, void* ws, size_t ws_bytes,
                     void* stream);

/* One product of the grouped GEMM kernel with every option the iteration's
 * stages use, exposed for kernel-level testing of that path (the building
 * blocks above use only row-major operands and none of the second outputs).
 * The kernel computes, for i < M, j < N (fp32, rounded once per output):
 *   v = alpha * sum_k A[i][k] B[j][k] + beta * C[i][j] + (i == j < diag_n ? gamma : 0)
 *   d[i][j]  = v                                (type d_dtype, leading dim ldd)
 *   d2[i][j] = v + (i == j < diag_n ? delta : 0)           (fp16, leading dim N)
 *   dt[j][i] = v                                 (fp16, leading dim M)
 *   a (M, K) and b (N, K): fp16, leading dimension K; or, with a_kmajor
 *             (b_kmajor), a stored as its (K, M) transpose with leading
 *             dimension M (b as (K, N), leading dimension N), which needs
 *             the row-pair layout (a_pairs / b_pairs = 1); at most one
 *             operand K-major, not in the symmetric mode, and not b with
 *             c_is_bt. This is how the Gram iteration multiplies by X
 *             without a transposed copy of it;
 *   c (M, N): type c_dtype, leading dimension ldc, or NULL (then beta is
 *             not used);
 *   *_pairs:  1 = the row-pair layout the iteration keeps its fp16 buffers
 *             in (rows even, leading dimension a multiple of 32): element
 *             (i, j) at (i / 2) * 2 ld + (j / 32) * 64 + (i % 2) * 32 + j % 32;
 *             0 = row-major. d_pairs applies to d, d2 and dt;
 *   symmetric: M == N, only tiles on or below the diagonal are computed and
 *             each is also stored mirrored, so d (and d2) come out exactly
 *             symmetric; requires fp16 c and d, no dt;
 *   c_is_bt:  the caller guarantees c[i][j] == b[j][i] (needs M <= K,
 *             alpha != 0); beta * c is then taken from the B slices the
 *             product already streams instead of being read again;
 *   valid_m, valid_n: stores (and reads of c) are clipped to this block when
 *             the output is not an fp16 tile-aligned buffer; d2 and dt
 *             need the unclipped fp16 path (valid block == M x N, fp16 d,
 *             16-byte aligned, ldd % 8 == 0) or the symmetric mode.
 * M, N multiples of 256, K a multiple of 128, all sides <= NS_MAX_DIM.
 * Problems share one launch, ordered as the iteration's stages order them
 * (longer K first); the workspace holds the launch descriptors
 * (ns_gemm_grouped_workspace_size). tile_edge selects the kernel: 256 (the
 * 256 x 256 tile kernel), 64 (the 64 x 64 tile kernel the stages use when
 * they have fewer than 64 tiles of 256 x 256; it gives the same bits), or
 * 0 (that same rule). Asynchronous on `stream`; errors as for every entry
 * point. */
typedef struct {
  const void* a;
  const void* b;
  const void* c;
  void* d;
  void* d2;
  void* dt;
  int64_t M, N, K, ldc, ldd;
  int64_t valid_m, valid_n, diag_n;
  ns_dtype c_dtype, d_dtype;
  int symmetric, c_is_bt;
  int a_pairs, b_pairs, c_pairs, d_pairs;
  int a_kmajor, b_kmajor;
  float alpha, beta, gamma, delta;
} ns_gemm_problem;
ns_status ns_gemm_grouped_workspace_size(int count, size_t* bytes);
ns_status ns_gemm_grouped(const ns_gemm_problem* probs, int count, int tile_edge, void* ws,
                          size_t ws_bytes, void* stream);

/* Host-side self-check of a call's launch plan (testing and diagnostics;
 * needs no device, launches nothing and dereferences no pointer). Builds the
 * plan that ns_batched (entry NS_CHECK_BATCHED; mats is an ns_matrix array),
 * ns_gram_sharded (NS_CHECK_SHARDED; one ns_matrix, `shards` shards) or
 * ns_muon_step (NS_CHECK_MUON; mats is an ns_muon_matrix array) would
 * launch for these arguments with its workspace at address `ws`, and runs
 * the bounds check every call runs before launching: each byte range a
 * kernel of the plan can read or write, derived from its descriptors the
 * way the kernels address memory, must lie inside one workspace buffer of
 * the plan's layout or one caller matrix, with write permission where it is
 * written; and each GEMM launch's workgroups must be dealt one-to-one onto
 * its tiles.
 * ws_bytes == 0 takes the required size. `plant` != 0 first plants
 * one of these mistakes into the plan, so a test can see the check catch it
 * (NS_ERR_UNSUPPORTED if the plan has no place for it):
 *   1 a caller's C read over the whole padded tile instead of its real block
 *   2 a caller's output written over the whole padded tile
 *   3 a product reading one K block past its operands
 *   4 the cast writing 64 rows past its padded block
 *   5 the norm pass reading one row past the input
 *   6 a shard reduction running one block past its parts
 *   7 a product reading its K-major operand from one K block further on
 *   8 the tile deal of a launch claiming one tile more than the launch has
 * Returns NS_OK, NS_ERR_INTERNAL (first violation described in msg, if msg
 * is not NULL, truncated to msg_len bytes), or the status the entry point's
 * argument checks give. */
typedef enum { NS_CHECK_BATCHED = 0, NS_CHECK_SHARDED = 1, NS_CHECK_MUON = 2 } ns_check_entry;
ns_status ns_plan_check(ns_check_entry entry, const void* mats, int count, ns_backend backend,
                        int shards, const ns_params* params, void* ws, size_t ws_bytes,
                        int plant, char* msg, size_t msg_len);

/* Kernel timing (measurement aid). While enabled, every launch made by
 * ns_normalize / ns_gram / ns_gram_sharded / ns_direct / ns_batched /
 * ns_muon_step is bracketed by two HIP events on the caller's stream. ns_timing_read waits for the recorded
 * events, reports the totals since the last read, and clears them. The
 * algorithmic work counts exclude zero padding:
 *   gemm_flops   2 m n k per general product; s (s + 1) k per symmetric
 *                product (SYRK and the Gram-space products);
 *   norm_bytes   HBM bytes the normalisation must move: the input read
 *                twice (norm pass, scale pass) and two fp16 copies written;
 *                for ns_muon_step the momentum pass also reads the
 *                gradient and writes the momentum; the norm_* fields also
 *                count the shard reductions of ns_gram_sharded (every part
 *                read once, the sum written).
 * Enabling or disabling is global to the process; disabled by default. */
typedef struct {
  double gemm_ms;
  int64_t gemm_launches;
  double gemm_flops;
  double norm_ms;
  int64_t norm_launches;
  double norm_bytes;
} ns_timing_report;
ns_status ns_timing_enable(int enable);
ns_status ns_timing_read(ns_timing_report* report);

/* Human-readable status name; never NULL. */
const char* ns_status_string(ns_status s);

/* One-line summary of the algorithm axis and kernel set for the current
 * device (the counterpart of the page's get_ns_backend(), section
 * "查询当前后端"), e.g. "Gram NS / direct NS · kernel=hip-mfma-f16
 * (gfx950, 256 CUs)". Never NULL; valid until the next call. */
const char* ns_backend_info(void);

/* Structured diagnostics (the counterpart of the page's
 * get_backend_status(), section "查询当前后端"): which device the calls
 * would run on and which kernel set, so that "auto" is never ambiguous.
 * Caller-owned struct, filled on the host; never launches work.
 *   device_found     1 if the current HIP device is a gfx950, else 0
 *                    (then every compute call returns NS_ERR_UNSUPPORTED);
 *   device_index     current HIP device, -1 if none;
 *   arch             gcnArchName of the current device ("" if none);
 *   compute_units    CU count of the current device (0 if none);
 *   clock_mhz        maximum engine clock reported by HIP (0 if none);
 *   deterministic    always 1: fixed tile order, fixed reduction order and
 *                    no floating-point atomics, so reruns on the same device
 *                    and build are bitwise identical (the page's bit-exact
 *                    option is therefore always on);
 *   gemm_tile        edge of the GEMM workgroup tile;
 *   version          NS_VERSION of the library;
 *   kernel           static name of the kernel set (never NULL).
 * Returns NS_ERR_INVALID_ARG for a NULL pointer, else NS_OK (also when no
 * device is present: the struct then says so). */
#define NS_VERSION 1
typedef struct {
  int device_found;
  int device_index;
  char arch[64];
  int compute_units;
  int clock_mhz;
  int deterministic;
  int gemm_tile;
  int version;
  const char* kernel;
} ns_backend_status_t;
ns_status ns_backend_status(ns_backend_status_t* out);

#ifdef __cplusplus
}
#endif

#endif /* NSMI_NS_H */

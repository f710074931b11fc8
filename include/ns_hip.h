/*
 * ns_hip.h - C ABI of the MI355X (gfx950) Newton–Schulz orthogonalization
 * library, libns_hip.so.
 *
 * The operation is Muon's quintic Newton–Schulz iteration applied to one
 * matrix or to a stack of independent matrices [batch, rows, cols]:
 *
 *   X  <- X / (||X||_F + 1e-7)            per matrix (slice)
 *   work on Xᵀ if rows > cols              (result returned untransposed)
 *   repeat ns_steps times:
 *     A = X Xᵀ,   B = b A + c A A,   X = a X + B X
 *
 * Sources (page title, section):
 *   - prime-rl PR #3873 (Muon optimizer-step speedups), "Summary" item 1:
 *     X Xᵀ and b A + c A A on a symmetric GEMM that computes one triangle and
 *     mirrors it; a X + B X as one GEMM with the scalar folded in; fp32
 *     alpha/beta epilogue (microbenchmark note under the NS table).
 *   - same page, "Summary" item 2: a 3-D stack is a batch along its leading
 *     axis; each slice is orthogonalized on its own.
 *   - param-decomp PR #978 "stacked-NS Muon", section "What": same-shape
 *     leaves batched into one NS; ns_steps (default 5); ns_dtype float32 or
 *     bfloat16.
 *   - Megatron-LM PR #6381 "Add --muon-use-syrk option ...", "Summary": the
 *     Gram product is symmetric, so a SYRK needs about half a GEMM's FLOPs;
 *     "Version compatibility": a requested fast path that cannot run must be
 *     a hard error, never a silent fallback (hence the status codes below).
 *
 * Conventions for every entry point:
 *   - Pointers named in/out/x/... are DEVICE pointers on the calling thread's
 *     current HIP device, 16-byte aligned, to contiguous row-major data.
 *     The caller owns them; the library never frees or retains them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is enqueued on it; calls return after enqueueing, without a
 *     host synchronisation.
 *   - Argument errors are detected on the host before anything is enqueued;
 *     no partial work is left behind.  Every call returns an ns_status.
 *   - No entry point falls back to another implementation.
 *   - Calls that share a device AND a stream share one library-owned
 *     workspace and are ordered by that stream; calls on different streams
 *     get different workspaces.
 */
#ifndef NS_HIP_H
#define NS_HIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
typedef enum {
  NS_OK = 0,
  NS_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, ns_steps < 0,
                             rows*cols >= 2^31, partial overlap in/out    */
  NS_ERR_DTYPE = 2,       /* dtype is not NS_DTYPE_F32 / NS_DTYPE_BF16    */
  NS_ERR_ALIGNMENT = 3,   /* a pointer not 16-byte aligned; for the stage
                             exports also rows or cols not a multiple of 8 */
  NS_ERR_ARCH = 4,        /* current device is not gfx950                 */
  NS_ERR_OOM = 5,         /* workspace allocation failed                  */
  NS_ERR_HIP = 6,         /* a HIP runtime call or launch failed;
                             details in ns_last_error()                   */
  NS_ERR_SCRATCH = 7      /* ns_orthogonalize_noalloc: the call needs more
                             than NS_NOALLOC_SCRATCH_BYTES of workspace    */
} ns_status;

/* Storage and compute dtype of every matrix of one call. */
enum {
  NS_DTYPE_F32 = 0,  /* fp32 storage, fp32 MFMA, fp32 epilogues           */
  NS_DTYPE_BF16 = 1  /* bf16 storage, bf16 MFMA with fp32 accumulation,
                        fp32 epilogues, fp32 diagonals (see below)        */
};

/*
 * ns_orthogonalize - the whole method on a stack of matrices.
 *
 *   in, out   device pointers to [batch, rows, cols] row-major, `dtype`.
 *             out may be the same pointer as in (in-place); any other
 *             overlap is NS_ERR_INVALID_ARG.  out always has the input's
 *             orientation (tall inputs are NOT returned transposed).
 *   batch     number of independent slices (0..65535; 0 enqueues nothing).
 *   rows,cols slice shape, each > 0.  When rows or cols is not a multiple
 *             of 8 the call zero-pads each slice to multiples of 8 in the
 *             workspace, runs on the padded copy and copies the caller's
 *             block back (zero rows and columns add only zero singular
 *             values, so the result is NS of the caller's matrix); the pad
 *             and unpad passes cost two extra copies of the stack.
 *   dtype     NS_DTYPE_F32 or NS_DTYPE_BF16.
 *   ns_steps  number of quintic steps (>= 0; 0 returns X / (||X||_F + eps)).
 *   a, b, c   quintic coefficients (Muon's usual: 3.4445, -4.7750, 2.0315).
 *   stream    hipStream_t as void*.
 *
 * Each slice is normalised by its own Frobenius norm.  An all-zero slice
 * yields zeros.  NaN/Inf inputs propagate; they are not checked.  The sum
 * of squares and the first Gram product accumulate the raw input in fp32
 * (the 1/||X|| scaling is applied in their epilogues), so a slice whose
 * ||X||_F exceeds about 1.8e19 (its sum of squares past the fp32 range)
 * gives no meaningful result (NaN or zeros).
 * Internally the Gram matrix A and the polynomial C = aI + bA + cAA are held
 * as an off-diagonal matrix (zero diagonal) in `dtype` plus an fp32 diagonal
 * vector; only lower-triangle tiles of both are computed.  C is mirrored;
 * A is mirrored too, except on large bf16 stacks, where it is kept as its
 * lower block triangle and the polynomial reads the rest transposed.
 * The workspace (ns_workspace_bytes) is allocated on first use per
 * (device, stream) and grown when needed.  Growing allocates a new buffer
 * without synchronising; the replaced one stays allocated (work queued
 * earlier may still use it) until ns_release_workspace.  Once the workspace
 * of (device, stream) is at least this call's size, a call makes no
 * allocation and no synchronisation: it enqueues only kernels (and, in place
 * with an odd step count, one device copy), so it can be captured into a
 * HIP graph, provided the capture runs on that same stream and workspace
 * poisoning is off.
 */
int ns_orthogonalize(const void* in, void* out, int64_t batch, int64_t rows,
                     int64_t cols, int dtype, int ns_steps, float a, float b,
                     float c, void* stream);

/* Bytes of library workspace one ns_orthogonalize call of this shape needs. */
size_t ns_workspace_bytes(int64_t batch, int64_t rows, int64_t cols, int dtype);

/*
 * ns_orthogonalize_noalloc - ns_orthogonalize for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Same arguments, checks, kernels and results as ns_orthogonalize (bitwise),
 * but the workspace is a fixed device array inside the library, one copy
 * per GPU, of NS_NOALLOC_SCRATCH_BYTES (256 MiB), held from the moment the
 * library's code is loaded on that GPU until the process ends.  The call
 * makes no device allocation (no hipMalloc, no hipFree, no allocating
 * library routine) and no synchronisation; the caller still provides in and
 * out.  A shape whose ns_workspace_bytes() exceeds NS_NOALLOC_SCRATCH_BYTES
 * is rejected with NS_ERR_SCRATCH before anything is enqueued (256 MiB
 * covers, e.g., bf16 4096 x 4096, 4096 x 14336 and 16 x 1536 x 2048).
 *
 * Every call on a GPU uses that GPU's one array and leaves its last contents
 * there; nothing in it has to start at zero (every kernel writes what a later
 * one reads).  Calls that overlap in time on one GPU - on different streams,
 * or from different threads without ordering - race on the array; order
 * them on one stream.  Kernel timing (ns_timing_*) does not apply to this
 * entry point.  Workspace poisoning (ns_set_workspace_poison) does, with
 * a memset of the array.
 */
#define NS_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int ns_orthogonalize_noalloc(const void* in, void* out, int64_t batch,
                             int64_t rows, int64_t cols, int dtype,
                             int ns_steps, float a, float b, float c,
                             void* stream);

/*
 * ns_orthogonalize_grouped - the same method on several stacks of different
 * shapes in one call (param-decomp PR #978, "What": same-shape leaves are
 * batched into one NS; here leaves of different shapes share the launches
 * too, and prime-rl PR #3873, "Summary" item 2: each slice on its own).
 *
 *   n_groups  number of stacks, 0..NS_MAX_GROUPS (0 enqueues nothing).
 *   in, out   HOST arrays of n_groups DEVICE pointers; stack g is
 *             [batch[g], rows[g], cols[g]] row-major at in[g], result at
 *             out[g], with ns_orthogonalize's rules for each pair
 *             (out[g] == in[g] allowed, any other overlap is an error).
 *             No out[g] may overlap another stack's in or out.
 *   batch, rows, cols
 *             HOST arrays of n_groups sizes, each checked as in
 *             ns_orthogonalize (batch[g] == 0: stack g is skipped and
 *             its pointers are not read, so they may be NULL).
 *   dtype, ns_steps, a, b, c, stream
 *             as in ns_orthogonalize, shared by every stack.
 *
 * The host arrays are read during the call only.  Each step runs at most
 * five launches whatever the number of stacks (Gram of the wide stacks,
 * Gram of the tall ones, one poly over all, update of the wide, update of
 * the tall; each split per 16 stacks), so many small leaves fill the GPU
 * together.  Every slice's result is bitwise the one ns_orthogonalize gives
 * for it.  ns_steps == 0 runs the stacks one after another.  Errors in any
 * stack are reported before anything is enqueued, with the stack's index in
 * ns_last_error().
 */
#define NS_MAX_GROUPS 4096
int ns_orthogonalize_grouped(int n_groups, const void* const* in, void* const* out,
                             const int64_t* batch, const int64_t* rows,
                             const int64_t* cols, int dtype, int ns_steps,
                             float a, float b, float c, void* stream);

/* Bytes of library workspace one ns_orthogonalize_grouped call needs (0 for
 * invalid arguments). */
size_t ns_workspace_bytes_grouped(int n_groups, const int64_t* batch,
                                  const int64_t* rows, const int64_t* cols,
                                  int dtype);

/* Free every cached workspace (all devices and streams), replaced ones
 * included.  Synchronises each device that held one.  Must not run while
 * another thread is inside a call.  Returns NS_OK or NS_ERR_HIP. */
int ns_release_workspace(void);

/* Number of workspace allocations (hipMalloc) the library has made since it
 * was loaded.  A call whose workspace is warm leaves it unchanged. */
int64_t ns_workspace_allocations(void);

/* ---- diagnostics --------------------------------------------------------- */

/* Static description of a status code. */
const char* ns_status_string(int status);

/* Text of the last error raised on the calling thread ("" if none). */
const char* ns_last_error(void);

/* Writes (NUL-terminated, truncated to n) a description of the kernels and
 * tile shapes the last successful call on this thread enqueued, so that a
 * caller can tell which path ran.  Returns the full length. */
int ns_query_last_config(char* buf, size_t n);

/*
 * Per-kernel timing with HIP events on the launch stream.
 * ns_timing_enable(mask): from now on, every launch of a kernel whose kind
 * bit is set in `mask` (1 << NS_KIND_*) records two hipEvents in its own
 * dispatch packet (hipExtLaunchKernel: the kernel's start and end), so no
 * packet goes between the kernels of a call; 0 disables.  The events are
 * timing-only (no system-scope fence); the stream must be synchronised
 * before their results are read on the host.  A timed dispatch still
 * releases its events at its end, which delays the next kernel by a few
 * microseconds: time a sample of the launches (ns_timing_sample) where the
 * call's own duration matters.
 * ns_timing_sample(every, offset): time only launch i of each kind (counted
 * from the last reset) with i % every == offset; every = 1, offset = 0 (the
 * default) times them all.  NS_ERR_INVALID_ARG unless 0 <= offset < every.
 * ns_timing_reset() drops the records and restarts the launch counts.
 * ns_timing_query(kind, &total_ms, &launches) waits for the recorded events
 * and returns the summed kernel time and the number of launches recorded.
 */
enum {
  NS_KIND_SUMSQ = 0,   /* per-slice sum of squares (norm, pass 1)        */
  NS_KIND_SCALE = 1,   /* scale and cast (norm, pass 2)                   */
  NS_KIND_GRAM = 2,    /* lower-triangle X Xᵀ (mirrored or lower-only)    */
  NS_KIND_POLY = 3,    /* lower-triangle C = aI + bA + cAA with mirror     */
  NS_KIND_UPDATE = 4,  /* X' = C X (or X C for tall), diagonal folded     */
  NS_KIND_COUNT = 5
};
int ns_timing_enable(int mask);
int ns_timing_sample(int every, int offset);
int ns_timing_reset(void);
int ns_timing_query(int kind, double* total_ms, int64_t* launches);

/*
 * Diagnostic: with on != 0, every later ns_orthogonalize and
 * ns_orthogonalize_grouped call first fills its whole workspace with 0xFF
 * bytes (NaN in bf16 and in fp32) on its stream, so that any kernel reading
 * a workspace element that no earlier kernel of the call wrote turns the
 * result into NaN.  0 turns it off (the default).  For tests: it costs one
 * fill of the workspace per call, enqueued as a memset, so keep it off
 * while a stream is being captured into a graph.  Returns NS_OK.
 */
int ns_set_workspace_poison(int on);

/*
 * Roofline calibration on the current device (a measurement helper; no step
 * of the method): every wave of two workgroups per CU runs `iters` (a
 * multiple of 4, at most 2^30) rounds of four back-to-back MFMAs on
 * registers only, v_mfma_f32_32x32x16_bf16 (dtype 1) or
 * v_mfma_f32_32x32x2_f32 (dtype 0), with operands that change from one
 * instruction to the next.  Writes the achieved dense rate in TFLOP/s (HIP
 * events on `stream`) and the average shader clock in MHz over the loop
 * (s_memtime against the constant-rate s_memrealtime).  Allocates and frees
 * its own small buffers and synchronises with the stream; about 0.1 s at
 * iters = 2^20.  Errors: NS_ERR_DTYPE, NS_ERR_INVALID_ARG (null outputs,
 * iters out of range), NS_ERR_ARCH, NS_ERR_HIP.
 */
int ns_peak_mfma(int dtype, int64_t iters, double* tflops, double* clock_mhz, void* stream);

/* ---- single stages (the same kernels ns_orthogonalize runs) ------------- */
/* Shapes: a slice of x is rows x cols, both multiples of 8 (the stages do
 * not pad); m = min(rows, cols).  The Gram side is the short one: A = X Xᵀ
 * when rows <= cols, A = Xᵀ X when rows > cols. */

/* X0 = x / (||x||_F + 1e-7) per slice, same shape, layout and dtype.
 * norms (optional, may be NULL): fp32 [batch] receives ||x||_F per slice.
 * x0 may equal x. */
int ns_stage_normalize(const void* x, void* x0, float* norms, int64_t batch,
                       int64_t rows, int64_t cols, int dtype, void* stream);

/* Gram of each slice: a_off [batch, m, m] (dtype) receives the off-diagonal
 * entries with exact zeros on the diagonal and is bitwise symmetric;
 * a_diag fp32 [batch, m] receives the diagonal. */
int ns_stage_gram(const void* x, void* a_off, float* a_diag, int64_t batch,
                  int64_t rows, int64_t cols, int dtype, void* stream);

/* C = a I + b A + c A A from A = a_off + diag(a_diag), stored the same way:
 * c_off [batch, m, m] (zero diagonal, bitwise symmetric), c_diag fp32
 * [batch, m].  a_off must be symmetric with a zero diagonal. */
int ns_stage_poly(const void* a_off, const float* a_diag, void* c_off,
                  float* c_diag, int64_t batch, int64_t m, int dtype, float a,
                  float b, float c, void* stream);

/* One update with C = c_off + diag(c_diag):
 *   rows <= cols:  x_out = C x         (C is rows x rows)
 *   rows >  cols:  x_out = x C         (C is cols x cols)
 * x_out must not overlap x. */
int ns_stage_update(const void* x, const void* c_off, const float* c_diag,
                    void* x_out, int64_t batch, int64_t rows, int64_t cols,
                    int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NS_HIP_H */

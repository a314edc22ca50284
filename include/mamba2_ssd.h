/*
 * mamba2_ssd.h -- C ABI of the Mamba-2 chunked SSD forward pass on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (NVIDIA developer blog "Accelerating Mamba-2 with
 * high-performance forward-pass kernels in NVIDIA CUDA Tile", section
 * "Mamba-2 architecture", the core recurrence): for every batch row b and
 * head h, with g = h / (nheads / ngroups) the head's group,
 *
 *     state_t[p, n] = exp(A[h] * dt[b,t,h]) * state_{t-1}[p, n]
 *                     + dt[b,t,h] * x[b,t,h,p] * B[b,t,g,n]
 *     y[b,t,h,p]    = sum_n C[b,t,g,n] * state_t[p, n] + D[h] * x[b,t,h,p]
 *
 * starting from state_{-1} = init_state[b,h] (zeros when NULL). The state is
 * held headdim-major ([headdim][dstate]). The library evaluates it chunk by
 * chunk through the log-space cumulative-decay "jump" formulas of the same
 * section, in four kernels enqueued on the caller's stream:
 *
 *   ssd_chunk_cumsum  chunk-local inclusive cumsum of A*dt, times log2(e)
 *                     (blog section "Kernel 1")
 *   ssd_chunk_state   each chunk's own state contribution, an MFMA
 *                     contraction over the chunk's tokens (the inner
 *                     product of the "Kernel 2: fwd_pass_state" section)
 *   ssd_state_pass    the sequential pass over chunk checkpoints
 *                     (the chunk loop of the same section)
 *   (for bf16 io and many (batch, head) pairs the chunk states are computed
 *   inside the state pass instead: one kernel with the structure of the
 *   blog's "Kernel 2", the per-chunk states never reaching memory --
 *   ssd_chunk_state_pass for headdim 64, chunk 256, or
 *   ssd_chunk_state_pass_rows for dstate 128 or 256; mamba2_ssd_fwd_path
 *   tells which kernel sequence a call takes, and a field of io_dtype can
 *   force one)
 *   ssd_chunk_scan    the per-chunk outputs: decayed carried-state term,
 *                     masked decayed C.B^T product with dt*x, and D*x
 *                     (blog section "Kernel 3: compute_out")
 *
 * Conventions for every entry point:
 *  - All arrays are dense, row-major, with the layouts given below; there
 *    are no strides. Pointers passed to mamba2_ssd_fwd are device pointers
 *    (hipMalloc'd or torch CUDA tensors); the caller owns them. The library
 *    never allocates or frees memory and keeps no state between calls.
 *  - dt must be >= 0 (already through softplus; no bias or softplus is
 *    applied inside) and A must be < 0 (the blog's "every A is negative").
 *    These are documented preconditions, not checked on the device.
 *  - Status codes are the MAMBA2_SSD_* values below: 0 on success, negative
 *    on failure. Validation runs on the host before anything is enqueued;
 *    on a validation error nothing is launched and no output is touched.
 *  - mamba2_ssd_fwd is asynchronous: it returns once the kernels are
 *    enqueued. Faults inside a kernel surface at the caller's next
 *    synchronisation, not as a return code.
 */
#ifndef MAMBA2_SSD_H_
#define MAMBA2_SSD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MAMBA2_SSD_OK                0
#define MAMBA2_SSD_ERR_NULL_POINTER (-1) /* a required pointer is NULL               */
#define MAMBA2_SSD_ERR_BAD_DIM      (-2) /* a size is <= 0 (< 0 for batch, seqlen),
                                            overflows, exceeds a grid limit, or one
                                            chunk of x (or of B, C) spans >= 2 GiB   */
#define MAMBA2_SSD_ERR_GROUPS       (-3) /* nheads is not a multiple of ngroups       */
#define MAMBA2_SSD_ERR_CHUNK        (-4) /* chunk is not one of 64, 128, 256          */
#define MAMBA2_SSD_ERR_UNSUPPORTED  (-5) /* (headdim, dstate, io dtype) not built     */
#define MAMBA2_SSD_ERR_WORKSPACE    (-6) /* workspace NULL or smaller than required   */
#define MAMBA2_SSD_ERR_ALIAS        (-7) /* an output overlaps another array          */
#define MAMBA2_SSD_ERR_HIP          (-8) /* a kernel launch failed; see
                                            mamba2_ssd_last_hip_error()               */
#define MAMBA2_SSD_ERR_ALIGN        (-9) /* a pointer lacks the alignment an entry
                                            point documents                           */

/* ---- io dtypes: the element type of x, B, C and y ---------------------- */
#define MAMBA2_SSD_F32  0   /* IEEE binary32                                    */
#define MAMBA2_SSD_BF16 1   /* bfloat16 (upper half of a binary32)              */

/* Layout flag, OR-ed into the io_dtype argument of the forward entry points
 * (mamba2_ssd_supported, _workspace_layout_query, _fwd_workspace_bytes,
 * _check_args, _fwd, _fwd_timed, _fwd_path, _fused_state_pass): dt is given head-major,
 * float [batch][nheads][seqlen], instead of token-major [batch][seqlen][nheads].
 * This is the [batch, head, token] global-memory layout the blog's
 * "Mamba-2 performance optimizations" section recommends for dt and the
 * decay cumsum (contiguous per-head reads); results are identical in both
 * layouts. Any other bit above the low byte gives MAMBA2_SSD_ERR_UNSUPPORTED.
 * The decode step (mamba2_ssd_step) takes no flags: its dt is [batch][nheads]. */
#define MAMBA2_SSD_DT_HEAD_MAJOR 0x100

/* Kernel sequence, a field OR-ed into the io_dtype argument of the forward
 * entry points (bits 12-13). Every sequence computes the same function (the
 * results agree to fp32 rounding); they differ in how the chunk states reach
 * the outputs. AUTO (0) lets the library choose by shape; the others force
 * one sequence, and a shape the forced sequence does not support gives
 * MAMBA2_SSD_ERR_UNSUPPORTED from every forward entry point.
 *   FOUR     ssd_chunk_cumsum, ssd_chunk_state, ssd_state_pass,
 *            ssd_chunk_scan (every supported shape)
 *   THREE    ssd_chunk_cumsum, ssd_chunk_state_pass(_rows), ssd_chunk_scan
 *            (bf16; headdim 64 and chunk 256, or dstate 128 or 256)
 *   CHAINED  ssd_chunk_cumsum, then one kernel that computes each chunk's
 *            state contribution, the pass and the outputs, handing the
 *            carried state from each chunk to the next through the
 *            workspace (bf16, headdim 64, dstate 64 or 128, chunk 256)
 * The workspace size depends on the sequence: query it with the same
 * io_dtype value that is passed to the call. */
#define MAMBA2_SSD_PATH_AUTO    0x0000
#define MAMBA2_SSD_PATH_FOUR    0x1000
#define MAMBA2_SSD_PATH_THREE   0x2000
#define MAMBA2_SSD_PATH_CHAINED 0x3000
#define MAMBA2_SSD_PATH_MASK    0x3000

/* Problem sizes. batch and seqlen may be 0 (nothing to compute: with
 * seqlen == 0 final_state receives init_state, or zeros). seqlen need not be
 * a multiple of chunk: the last chunk is then ragged and behaves as if
 * padded with tokens whose x, dt, B and C are zero (the blog's kernel loads
 * use zero padding), which neither decay nor feed the state. */
typedef struct {
  int64_t batch;    /* B  */
  int64_t seqlen;   /* T  */
  int64_t nheads;   /* H  */
  int64_t headdim;  /* P: 64 or 128                         */
  int64_t dstate;   /* N: 64, 128 or 256                    */
  int64_t ngroups;  /* G: H % G == 0; heads h*H/G .. (h+1)*H/G-1 share group h */
  int64_t chunk;    /* Q: 64, 128 or 256                    */
} mamba2_ssd_dims;

/* Where each intermediate lives inside the caller's workspace. nchunks =
 * ceil(seqlen / chunk); Tp = nchunks * chunk. Offsets are in bytes from the
 * workspace base and 256-byte aligned. The contents after a call are
 * documented so tests can check each kernel's output:
 *   gcum    float [batch][nheads][Tp]  chunk-local inclusive cumsum of
 *                                      A*dt, times log2(e); padded tokens
 *                                      repeat the last real value
 *   dtt     float [batch][nheads][Tp]  dt transposed, padded tokens 0
 *   wst     float [batch][nheads][Tp]  dt_t * 2^(G'_last - G'_t), the weight
 *                                      of token t in its chunk's state
 *   states  float [batch][nheads][nchunks][headdim][dstate]
 *                                      each chunk's own contribution S_k
 *                                      (FOUR only; no bytes on the other
 *                                      sequences)
 *   hprev   [batch][nheads][nchunks][headdim][dstate] states h entering
 *           each chunk; io = F32: float; io = BF16: bf16 pairs, 4 bytes per
 *           element: for each row and each aligned group of 8 dstate
 *           columns, the 8 values bf16(h) followed by the 8 values
 *           bf16(h - bf16(h)), so hi + lo carries h to about 16 bits
 *           (FOUR and THREE; no bytes on CHAINED)
 *   chain   float [batch][nheads][headdim][dstate] (CHAINED only): the
 *           carried state handed from each chunk to the next
 *   sync    int32 (CHAINED only): a work counter and one progress flag per
 *           (batch, head), cleared by ssd_chunk_cumsum
 * A region a sequence does not use has no bytes: its offset equals the next
 * region's. */
typedef struct {
  size_t total_bytes;
  size_t gcum_offset;
  size_t dtt_offset;
  size_t wst_offset;
  size_t states_offset;
  size_t hprev_offset;
  size_t chain_offset;
  size_t sync_offset;
  int64_t nchunks;
  int32_t path;       /* the MAMBA2_SSD_PATH_* sequence the layout is for */
} mamba2_ssd_workspace_layout;

/* 1 if (headdim, dstate, chunk, io_dtype) has compiled kernels, else 0.
 * Host only; needs no GPU. */
int mamba2_ssd_supported(int64_t headdim, int64_t dstate, int64_t chunk, int io_dtype);

/* Fill *out with the workspace layout for these sizes. Host only.
 * Returns a status code (the dimension checks of mamba2_ssd_check_args). */
int mamba2_ssd_workspace_layout_query(const mamba2_ssd_dims* dims, int io_dtype,
                                      mamba2_ssd_workspace_layout* out);

/* Workspace bytes mamba2_ssd_fwd needs, or 0 if the sizes are invalid.
 * Host only. */
size_t mamba2_ssd_fwd_workspace_bytes(const mamba2_ssd_dims* dims, int io_dtype);

/* Every host-side check of mamba2_ssd_fwd, without touching the GPU: sizes,
 * support, required pointers, alignment, workspace size and aliasing.
 * Pointers are only compared, never dereferenced, so any values may be
 * passed.
 * Alignment (MAMBA2_SSD_ERR_ALIGN): x, B, C, y, init_state and final_state
 * on 16 bytes, dt, A and D on 4, the workspace on 256 (the kernels move
 * these arrays in 16-byte pieces; hipMalloc and torch allocations satisfy
 * this; a view at an odd element offset may not).
 * Aliasing rules: init_state may be the same pointer as final_state (an
 * in-place state update); apart from that, y, final_state and the
 * workspace must not overlap any other array. Inputs may overlap each
 * other. Arrays that are empty (batch or seqlen 0) may be NULL. */
int mamba2_ssd_check_args(const mamba2_ssd_dims* dims, int io_dtype,
                          const void* x, const float* dt, const float* A,
                          const void* B, const void* C, const float* D,
                          const float* init_state, const void* y, const float* final_state,
                          const void* workspace, size_t workspace_bytes);

/* The forward pass.
 *   x           io    [batch][seqlen][nheads][headdim]
 *   dt          float [batch][seqlen][nheads]          (>= 0)
 *   A           float [nheads]                         (< 0)
 *   B, C        io    [batch][seqlen][ngroups][dstate]
 *   D           float [nheads]
 *   init_state  float [batch][nheads][headdim][dstate], or NULL for zeros
 *   y           io    [batch][seqlen][nheads][headdim]  (written)
 *   final_state float [batch][nheads][headdim][dstate], or NULL to skip
 *   workspace   device memory of at least mamba2_ssd_fwd_workspace_bytes;
 *               contents on entry are ignored; concurrent calls need
 *               separate workspaces
 *   stream      a hipStream_t, or NULL for the default stream
 * Arithmetic: fp32 accumulation and an fp32 carried state everywhere. With
 * io = BF16 the products run on bf16 MFMA: x, B and C enter exactly, and each
 * operand that is not an input (w*x in the chunk-state contraction, the
 * decayed masked C.B^T times dt, and the carried state) enters as a pair of
 * bf16 numbers hi + lo, about 16 significant bits, in two MFMAs. y is
 * rounded to bf16 nearest-even once at the end; final_state is fp32. With
 * io = F32 every product is an fp32 MFMA.
 * Returns a status code; see the conventions above. */
int mamba2_ssd_fwd(const mamba2_ssd_dims* dims, int io_dtype,
                   const void* x, const float* dt, const float* A,
                   const void* B, const void* C, const float* D,
                   const float* init_state, void* y, float* final_state,
                   void* workspace, size_t workspace_bytes, void* stream);

/* The kernel sequence mamba2_ssd_fwd takes for these sizes and io_dtype
 * (including its path field): MAMBA2_SSD_PATH_FOUR, _THREE or _CHAINED, or a
 * negative status when the arguments are invalid or the forced sequence
 * does not support the shape. AUTO chooses CHAINED where it supports the
 * shape, else THREE when its (batch, head, dstate group) walks alone fill
 * the GPU, else FOUR. Host only. */
int mamba2_ssd_fwd_path(const mamba2_ssd_dims* dims, int io_dtype);

/* 1 if mamba2_ssd_fwd with these sizes computes the chunk states inside
 * another kernel (sequences THREE and CHAINED: the workspace holds no states
 * region), 0 if it runs ssd_chunk_state and ssd_state_pass (FOUR), or if
 * the arguments are invalid. Host only. */
int mamba2_ssd_fused_state_pass(const mamba2_ssd_dims* dims, int io_dtype);

/* mamba2_ssd_fwd that also records caller-created events on `stream`, so
 * each kernel can be timed where it runs: events[0] before ssd_chunk_cumsum,
 * events[1] before ssd_chunk_state, events[2] before ssd_state_pass,
 * events[3] before ssd_chunk_scan and events[4] after it. On THREE,
 * events[1]..events[2] enclose ssd_chunk_state_pass and events[2]..events[3]
 * nothing; on CHAINED, events[1]..events[2] enclose the chained kernel and
 * the later spans nothing. `events` points to
 * 5 hipEvent_t handles (passed as void*) owned by the caller; NULL makes the
 * call identical to mamba2_ssd_fwd. The kernels and their order are the
 * same; a failed event record returns MAMBA2_SSD_ERR_HIP. */
int mamba2_ssd_fwd_timed(const mamba2_ssd_dims* dims, int io_dtype,
                         const void* x, const float* dt, const float* A,
                         const void* B, const void* C, const float* D,
                         const float* init_state, void* y, float* final_state,
                         void* workspace, size_t workspace_bytes, void* stream,
                         void* const* events);

/* ---- forward pass without caller memory -----------------------------------
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Identical
 * to mamba2_ssd_fwd (same arguments apart from the workspace, same kernels,
 * same results bit for bit) except that the workspace is a device array
 * inside the library, MAMBA2_SSD_NOALLOC_MAX_WORKSPACE bytes per GPU, held
 * from the library's load until the process ends. Calls whose workspace
 * (mamba2_ssd_fwd_workspace_bytes with the same io_dtype) exceeds it return
 * MAMBA2_SSD_ERR_WORKSPACE before anything is launched. The call allocates
 * nothing (no hipMalloc, no library allocator); on its first use on a GPU it
 * looks up the array's address there (hipGetSymbolAddress).
 * The array is shared by every call on the same GPU and keeps the last
 * call's contents (every region a call reads is written by that call first,
 * so nothing has to start at zero). Calls that overlap in time on one GPU
 * (on different streams, or from different threads) race on it and give
 * undefined results; serialise them. The stream's device (the current
 * device for a NULL stream) selects the array. */
#define MAMBA2_SSD_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)

int mamba2_ssd_fwd_noalloc(const mamba2_ssd_dims* dims, int io_dtype,
                           const void* x, const float* dt, const float* A,
                           const void* B, const void* C, const float* D,
                           const float* init_state, void* y, float* final_state,
                           void* stream);

/* ---- one decode step ----------------------------------------------------
 *
 * The recurrent form of the same layer (blog section "Mamba-2 architecture":
 * the core recurrence, which the blog notes suits token-by-token inference):
 * each of `batch` sequences advances by one token, for every head h, with
 * g = h / (nheads / ngroups),
 *
 *     state[b,h,p,n] <- exp(A[h] * dt[b,h]) * state[b,h,p,n]
 *                       + dt[b,h] * x[b,h,p] * B[b,g,n]
 *     y[b,h,p]        = sum_n C[b,g,n] * state[b,h,p,n] + D[h] * x[b,h,p]
 *
 * (y reads the updated state, as in the forward pass). The state is the
 * final_state of mamba2_ssd_fwd (same layout), updated in place, so a
 * prefill followed by steps continues the same sequence. One kernel reads
 * and writes the state once: the step is bound by HBM bandwidth. */
typedef struct {
  int64_t batch;    /* sequences, each advanced by one token (0 = nothing to do) */
  int64_t nheads;   /* H  */
  int64_t headdim;  /* P: any >= 1                                           */
  int64_t dstate;   /* N: 64, 128 or 256                                     */
  int64_t ngroups;  /* G: H % G == 0, heads grouped as in mamba2_ssd_fwd     */
} mamba2_ssd_step_dims;

/* 1 if mamba2_ssd_step has kernels for (dstate, io_dtype), else 0. Host only. */
int mamba2_ssd_step_supported(int64_t dstate, int io_dtype);

/* Every host-side check of mamba2_ssd_step, without touching the GPU:
 * sizes (batch * nheads * headdim rows and batch * ngroups * dstate must
 * stay below 2^31), support, required pointers, alignment (state 16 bytes;
 * B and C 16 bytes for F32, 8 for BF16) and aliasing (state and y must not
 * overlap each other or any input). Pointers are only compared. */
int mamba2_ssd_step_check_args(const mamba2_ssd_step_dims* dims, int io_dtype,
                               const void* x, const float* dt, const float* A,
                               const void* B, const void* C, const float* D,
                               const float* state, const void* y);

/* One decode step.
 *   x      io    [batch][nheads][headdim]
 *   dt     float [batch][nheads]              (>= 0)
 *   A, D   float [nheads]                     (A < 0)
 *   B, C   io    [batch][ngroups][dstate]
 *   state  float [batch][nheads][headdim][dstate]  read and written in place
 *   y      io    [batch][nheads][headdim]     (written)
 *   stream a hipStream_t, or NULL for the default stream
 * Arithmetic in fp32 (exp(A dt) on the hardware base-2 exponential); y is
 * rounded to the io dtype (bf16 nearest-even) once at the end. Asynchronous,
 * like mamba2_ssd_fwd; returns a status code. */
int mamba2_ssd_step(const mamba2_ssd_step_dims* dims, int io_dtype,
                    const void* x, const float* dt, const float* A,
                    const void* B, const void* C, const float* D,
                    float* state, void* y, void* stream);

/* ---- backward pass -------------------------------------------------------
 *
 * Every input's gradient for a loss whose gradients with respect to the
 * forward outputs are dy (with respect to y) and dfinal (with respect to
 * final_state; NULL means zero). The forward pass is the recurrence at the
 * top of this header; its gradient follows the chunked form differentiated
 * block by block, with the state's adjoint running the chunk pass backwards
 * in time (the "Part 3" derivation of Sasha Rush's "Mamba: The Hard Way"
 * shows this reversal for the scalar scan: the derivative is the same scan
 * run in the other direction, and the coefficient gradients need the forward
 * and backward states together). The forward intermediates are recomputed
 * inside the call; nothing from a forward call is needed.
 *
 * Inputs: dims, io (MAMBA2_SSD_F32 or MAMBA2_SSD_BF16, no layout flags), x,
 * dt, A, B, C, D, init_state (nullable) exactly as for mamba2_ssd_fwd; dy
 * [batch][seqlen][nheads][headdim] in the io dtype; dfinal (nullable) float
 * [batch][nheads][headdim][dstate].
 * Outputs, all float32, dense, caller-owned, written whole:
 *   dx  [batch][seqlen][nheads][headdim]   ddt [batch][seqlen][nheads]
 *   dB  [batch][seqlen][ngroups][dstate]   dC  like dB (sums over the
 *                                          heads of each group)
 *   dA  [nheads]   dD [nheads]             (sums over batch rows and tokens)
 *   dinit [batch][nheads][headdim][dstate] (nullable: not written)
 * Arithmetic: fp32 accumulation everywhere. With bf16 io, headdim 64,
 * chunk 256 and dstate 64 or 128 the products run on the bf16 MFMA: bf16
 * inputs enter exactly, fp32 intermediates (decayed blocks, states, scaled
 * rows) as bf16 (hi, lo) pairs, about 2^-17 relative per operand; other
 * shapes and fp32 io use fp32 operands.
 * Workspace: mamba2_ssd_bwd_workspace_bytes(dims, io) bytes, device memory,
 * 256-byte aligned; it holds the chunk cumsums, the chunk states and their
 * adjoints, the per-group C.B^T-weighted sums and the per-token partial
 * results; for shapes off the bf16 path above also padded fp32 copies of
 * the inputs and the per-head C.B^T and dy.x^T blocks (batch 4, seqlen
 * 8192, 80 heads, headdim 64, dstate 128, chunk 256: 2.6 GB with bf16 io,
 * 9.9 GB with fp32 io). Sizes are those of mamba2_ssd_fwd, plus
 * batch * nchunks * nheads <= 65535.
 * Errors: as mamba2_ssd_check_args (NULL_POINTER for a missing required
 * pointer: A, D, dA, dD always; x, dt, B, C, dy, dx, ddt, dB, dC when
 * batch * seqlen > 0), ALIAS when an output overlaps an input, another
 * output or the workspace, ALIGN for a workspace that is not 256-byte
 * aligned, UNSUPPORTED for flag bits in io. Validation runs
 * on the host before any launch; the call is asynchronous on `stream`. */
size_t mamba2_ssd_bwd_workspace_bytes(const mamba2_ssd_dims* dims, int io_dtype);

int mamba2_ssd_bwd_check_args(const mamba2_ssd_dims* dims, int io_dtype,
                              const void* x, const float* dt, const float* A,
                              const void* B, const void* C, const float* D,
                              const float* init_state, const void* dy, const float* dfinal,
                              const float* dx, const float* ddt, const float* dA,
                              const float* dB, const float* dC, const float* dD,
                              const float* dinit, const void* workspace,
                              size_t workspace_bytes);

int mamba2_ssd_bwd(const mamba2_ssd_dims* dims, int io_dtype,
                   const void* x, const float* dt, const float* A,
                   const void* B, const void* C, const float* D,
                   const float* init_state, const void* dy, const float* dfinal,
                   float* dx, float* ddt, float* dA, float* dB, float* dC, float* dD,
                   float* dinit, void* workspace, size_t workspace_bytes, void* stream);

/* Static string naming a status code. Never NULL. */
const char* mamba2_ssd_status_string(int status);

/* Text of the last HIP error this thread saw inside mamba2_ssd_fwd,
 * mamba2_ssd_bwd or mamba2_ssd_step (MAMBA2_SSD_ERR_HIP), or "" if none. Valid until the thread's next call. */
const char* mamba2_ssd_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA2_SSD_H_ */

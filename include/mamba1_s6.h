/*
 * mamba1_s6.h -- C ABI of the Mamba-1 selective scan (S6) on AMD Instinct
 * MI355X (gfx950), the state-space family's other member.
 *
 * The operation (Sasha Rush, "Mamba: The Hard Way", Part 5 "Mamba / S6"):
 * for every batch row b, channel d and state n, with the continuous-time
 * parameters discretized per step,
 *
 *     a_t = exp(delta[b,d,t] * A[d,n]),   b_t = B[b,n,t] * delta[b,d,t]
 *     h[b,d,n] <- a_t * h[b,d,n] + b_t * x[b,d,t]
 *     y[b,d,t]  = sum_n C[b,n,t] * h[b,d,n]
 *
 * starting from h0 (zeros when NULL); the state after the last token goes to
 * hT when it is not NULL. No skip term and no gate (the page runs the scan
 * with neither). A is shared by every batch row.
 *
 * Layouts, all float32, dense, row-major, caller-owned device memory:
 *   x, delta, y   [batch][channels][seqlen]
 *   B, C          [batch][dstate][seqlen]
 *   A             [channels][dstate]
 *   h0, hT        [batch][channels][dstate]
 * delta >= 0 and A < 0 are documented preconditions, not checked on device.
 *
 * The scan runs chunk-parallel in one pass over x and delta (chunks of 64
 * tokens: each chunk's own scan from a zero state, its entering state from
 * the summaries the earlier chunks publish, then the chunk again from that
 * state), through a caller-provided workspace of
 * mamba1_s6_workspace_bytes(dims) bytes that holds those summaries and the
 * chunks' progress flags (cleared by the call itself). Two calls that share
 * a workspace must not overlap in time. Status codes are the MAMBA2_SSD_*
 * values of mamba2_ssd.h; validation runs on the host before any launch and
 * the call is asynchronous on `stream`.
 */
#ifndef MAMBA1_S6_H_
#define MAMBA1_S6_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t batch;     /* >= 0 */
  int64_t seqlen;    /* >= 0 */
  int64_t channels;  /* D > 0 */
  int64_t dstate;    /* N: 1, 2, 4, 8 or 16 */
} mamba1_s6_dims;

/* 1 if dstate has compiled kernels, else 0. Host only. */
int mamba1_s6_supported(int64_t dstate);

/* Workspace bytes for these sizes (0 when the sizes are invalid). Host only. */
size_t mamba1_s6_workspace_bytes(const mamba1_s6_dims* dims);

/* Host-only validation of a call: NULL_POINTER (a required pointer missing:
 * A always; x, delta, B, C, y when batch * seqlen > 0), BAD_DIM (a size out
 * of range or a grid limit: batch <= 65535, ceil(seqlen / 64) <= 65535),
 * UNSUPPORTED (dstate), WORKSPACE, ALIGN (a float array not 4-byte
 * aligned, or the workspace not 256-byte aligned when batch > 0), ALIAS (y
 * or hT overlapping an input, each other or the workspace; hT may equal h0
 * exactly). */
int mamba1_s6_check_args(const mamba1_s6_dims* dims, const float* x, const float* delta,
                         const float* A, const float* B, const float* C, const float* h0,
                         const float* y, const float* hT, const void* workspace,
                         size_t workspace_bytes);

/* The scan; returns a status code after enqueueing its kernels (the clearing
 * of the workspace's counter and flags, then the one-pass scan). */
int mamba1_s6_fwd(const mamba1_s6_dims* dims, const float* x, const float* delta,
                  const float* A, const float* B, const float* C, const float* h0,
                  float* y, float* hT, void* workspace, size_t workspace_bytes, void* stream);

/* ---- backward pass -------------------------------------------------------
 *
 * Every input's gradient of the scan above for a loss whose gradients with
 * respect to its outputs are dy (like y) and dhT (like hT; NULL means zero).
 * The state's adjoint g runs the same scan backwards in time ("Mamba: The
 * Hard Way", Part 3, applied to each scalar chain of Part 5):
 *
 *     g_t = C[b,n,t] dy[b,d,t] + a_{t+1} g_{t+1}      (after the last token: dhT)
 *     dx[b,d,t]     = sum_n g_t B[b,n,t] delta_t
 *     ddelta[b,d,t] = sum_n g_t (A[d,n] a_t h_{t-1} + B[b,n,t] x_t)
 *     dA[d,n]       = sum_{b,t} g_t delta_t a_t h_{t-1}
 *     dB[b,n,t]     = sum_d g_t delta_t x_t,   dC[b,n,t] = sum_d dy_t h_t
 *     dh0[b,d,n]    = a_0 g_0
 *
 * Inputs: dims, x, delta, A, B, C, h0 (nullable) exactly as for
 * mamba1_s6_fwd; dy [batch][channels][seqlen]; dhT (nullable)
 * [batch][channels][dstate]. Outputs, float32, dense, caller-owned, written
 * whole: dx, ddelta like x; dA like A; dB, dC like B; dh0 like h0 (nullable:
 * not written). dstate 1, 2, 4, 8 or 16.
 * The call runs the forward scan for the chunks' end states (no y), which
 * also forms each chunk's own adjoint record from dy; then the chunks'
 * entering adjoints, the per-chunk gradients (each chunk's states recomputed
 * from its entering state) and the sums over batch rows, chunks and channel
 * blocks, in fixed orders (deterministic). fp32 arithmetic throughout.
 * Workspace: mamba1_s6_bwd_workspace_bytes(dims) bytes of device memory
 * (the forward's, plus per-chunk adjoints and partial sums); two calls that
 * share it must not overlap in time.
 * Errors: as mamba1_s6_check_args (NULL_POINTER: A, dA always; x, delta, B,
 * C, dy, dx, ddelta, dB, dC when batch * seqlen > 0; ALIGN as there), ALIAS
 * when an output overlaps an input, another output or the workspace. Validation runs on
 * the host before any launch; the call is asynchronous on `stream`. */
size_t mamba1_s6_bwd_workspace_bytes(const mamba1_s6_dims* dims);

int mamba1_s6_bwd_check_args(const mamba1_s6_dims* dims, const float* x, const float* delta,
                             const float* A, const float* B, const float* C, const float* h0,
                             const float* dy, const float* dhT, const float* dx, const float* ddelta,
                             const float* dA, const float* dB, const float* dC, const float* dh0,
                             const void* workspace, size_t workspace_bytes);

int mamba1_s6_bwd(const mamba1_s6_dims* dims, const float* x, const float* delta, const float* A,
                  const float* B, const float* C, const float* h0, const float* dy, const float* dhT,
                  float* dx, float* ddelta, float* dA, float* dB, float* dC, float* dh0,
                  void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA1_S6_H_ */

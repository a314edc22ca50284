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
 * UNSUPPORTED (dstate), WORKSPACE, ALIAS (y or hT overlapping an input,
 * each other or the workspace; hT may equal h0 exactly). */
int mamba1_s6_check_args(const mamba1_s6_dims* dims, const float* x, const float* delta,
                         const float* A, const float* B, const float* C, const float* h0,
                         const float* y, const float* hT, const void* workspace,
                         size_t workspace_bytes);

/* The scan; returns a status code after enqueueing its three kernels. */
int mamba1_s6_fwd(const mamba1_s6_dims* dims, const float* x, const float* delta,
                  const float* A, const float* B, const float* C, const float* h0,
                  float* y, float* hT, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA1_S6_H_ */

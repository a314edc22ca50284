// Host-side description of one backward call (ssd_bwd.hip): sizes, the
// caller's device pointers and the workspace carve-up. Validated by the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ssd_launch.h"

namespace ssd {

// Byte offsets of the backward workspace's arrays (all fp32, 256-byte aligned).
struct BwdLayout {
  size_t gcum, dtt, wst, E;             // [bt][H][Tp]
  size_t Xp, dYp;                       // [bt][Tp][H][P], zero padded (empty on the fused path)
  size_t Bp, Cp;                        // [bt][Tp][G][N], zero padded
  size_t S, hprev, dhn;                 // [bt][H][nc][P][N]
  size_t CB;                            // [bt][nc][G][Q][Q] (C B^T, then the group's sum of W2s)
  size_t DX, W1;                        // [bt][nc][H][Q][Q] (fused path: DX = per-segment W2 sums, W1 empty)
  size_t U, V;                          // [bt][nc][H][Q][P] (fused path: transposed dHn, Hprev fragments)
  size_t dXp;                           // [bt][Tp][H][P]
  size_t dBh, dCh;                      // [bt][Tp][G][N]
  size_t rowZ, colZ, colW;              // [bt][H][Tp]
  size_t dA_part, dD_part;              // [bt][H][nc]
  size_t total;
};

// (io selects the layout: the fused path of bwd_fused.hip needs less)
BwdLayout bwd_layout(int64_t bt, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q, int64_t nc, int io);

struct BwdProblem {
  int64_t bt, T, H, P, N, G, Q, nc, Tp;
  int io;                               // 0 = fp32, 1 = bf16 (x, B, C, dy)
  const void* x; const float* dt; const float* A; const void* B; const void* C; const float* D;
  const float* init;                    // may be null
  const void* dy;
  const float* dfinal;                  // may be null
  float* dx; float* ddt; float* dA; float* dB; float* dC; float* dD;
  float* dinit;                         // may be null
  // workspace arrays (see BwdLayout)
  float *gcum, *dtt, *wst, *E, *Xp, *dYp, *Bp, *Cp, *S, *hprev, *dhn, *CB, *DX, *W1, *U, *V, *dXp, *dBh,
      *dCh, *rowZ, *colZ, *colW, *dA_part, *dD_part;
};

// Enqueues the backward kernels after the cumsum (which the caller runs into
// gcum, dtt and wst first).
hipError_t launch_ssd_bwd(BwdProblem p, hipStream_t stream);

// The fused causal part (bwd_fused.hip): for the shapes it supports it
// replaces the C B^T and dY X^T products, the masks and decays, the W1^T dY
// product and the group sums of W2, writing dXp, rowZ, colZ, colW and CB
// (the group's W2 sum) as those steps do; w2part holds the per-segment sums
// ([bt][nc][G][nseg][Q][Q]).
bool bwd_fused_supported(int io, int64_t P, int64_t N, int64_t Q);
int bwd_fused_segments(int64_t bt, int64_t nc, int64_t H, int64_t G);
hipError_t launch_bwd_fused_qq(const BwdProblem& p, float* w2part, int nseg, hipStream_t stream);
// The same shapes: U = B dHn^T and V = C Hprev^T formed on the fly with dx,
// ddt and the dA / dD parts (in place of the U, V products and finish_chunk).
// It also writes dHn and Hprev transposed, [n][p] in bf16 (hi, lo) pairs,
// into the U and V regions, for:
hipError_t launch_bwd_fused_finish(const BwdProblem& p, hipStream_t stream);
// out[t][g][n] = sum over the group's heads of scale_t^h X_t^h S^h (the
// carried-state parts of dB and dC; ST: the transposed states above).
hipError_t launch_bwd_fused_headsum(const BwdProblem& p, const void* X, const float* scale, const void* ST,
                                    float* out, hipStream_t stream);

}  // namespace ssd

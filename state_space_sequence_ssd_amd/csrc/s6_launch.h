// Host-side description of one selective-scan call (s6_scan.hip). Device
// pointers, validated by the ABI (s6_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

struct S6Problem {
  int64_t bt, L, D, N;          // batch, seqlen, channels, dstate
  const float* x;               // [bt][D][L]
  const float* delta;           // [bt][D][L]
  const float* A;               // [D][N]
  const float* B;               // [bt][N][L]
  const float* C;               // [bt][N][L]
  const float* h0;              // [bt][D][N] or null (zeros)
  float* y;                     // [bt][D][L]
  float* hT;                    // [bt][D][N] or null (not written)
  float* aggS;                  // workspace: [bt][nchunks][D][N] each chunk's end state from zero
  float* aggD;                  // workspace: [bt][nchunks][D] each chunk's sum of delta
  float* incl;                  // workspace: [bt][nchunks][D][N] each chunk's end state
  int* sync;                    // workspace: s6_sync_words int32 (ticket counter, error word, flags)
  // the backward pass's forward sweep (y, hT null): with dy set, each chunk's
  // adjoint record O [bt][nchunks][D][N] and delta sum SD [bt][nchunks][D]
  const float* dy = nullptr;    // [bt][D][L]
  float* O = nullptr;
  float* SD = nullptr;
};

// One backward call (s6_bwd.hip): the inputs above, the upstream gradients,
// the outputs and the workspace arrays it fills after the forward scan has
// left every chunk's end state in `incl`.
struct S6BwdProblem {
  int64_t bt, L, D, N;
  const float* x;               // [bt][D][L]
  const float* delta;           // [bt][D][L]
  const float* A;               // [D][N]
  const float* B;               // [bt][N][L]
  const float* C;               // [bt][N][L]
  const float* h0;              // [bt][D][N] or null (zeros)
  const float* dy;              // [bt][D][L]
  const float* dhT;             // [bt][D][N] or null (zeros)
  float* dx;                    // [bt][D][L]
  float* ddelta;                // [bt][D][L]
  float* dA;                    // [D][N]
  float* dB;                    // [bt][N][L]
  float* dC;                    // [bt][N][L]
  float* dh0;                   // [bt][D][N] or null (not written)
  const float* incl;            // [bt][nchunks][D][N] chunk end states (forward workspace)
  float* O;                     // [bt][nchunks][D][N] each chunk's adjoint leaving its first token
  float* SD;                    // [bt][nchunks][D] each chunk's sum of delta
  float* R;                     // [bt][nchunks][D][N] the adjoint entering each chunk from the right
  float* dA_part;               // [bt][nchunks][D][N]
  float* dB_part;               // [bt][channel blocks][N][L]
  float* dC_part;               // [bt][channel blocks][N][L]
};

int64_t s6_chunk_tokens();      // tokens per chunk of the parallel scan
int64_t s6_bwd_channel_block();   // channels per block of the backward's dB, dC partial sums
bool s6_bwd_has(int64_t N);
hipError_t launch_s6_bwd(const S6BwdProblem& p, hipStream_t stream);
int64_t s6_sync_words(int64_t bt, int64_t D, int64_t L, int64_t N);
bool s6_has(int64_t N);
hipError_t launch_s6(const S6Problem& p, hipStream_t stream);

}  // namespace ssd

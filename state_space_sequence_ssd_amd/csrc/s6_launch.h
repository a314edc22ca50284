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
};

int64_t s6_chunk_tokens();      // tokens per chunk of the parallel scan
int64_t s6_sync_words(int64_t bt, int64_t D, int64_t L);
bool s6_has(int64_t N);
hipError_t launch_s6(const S6Problem& p, hipStream_t stream);

}  // namespace ssd

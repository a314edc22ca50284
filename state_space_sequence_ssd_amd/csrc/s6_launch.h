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
  float* S;                     // workspace: [bt][D][nchunks][N]
  float* sumd;                  // workspace: [bt][D][nchunks]
  float* hin;                   // workspace: [bt][D][nchunks][N]
};

int64_t s6_chunk_tokens();      // tokens per chunk of the parallel scan
bool s6_has(int64_t N);
hipError_t launch_s6(const S6Problem& p, hipStream_t stream);

}  // namespace ssd

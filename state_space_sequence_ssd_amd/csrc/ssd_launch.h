// Host-side description of one forward call, shared by the C ABI and the
// kernel launchers. All pointers are device pointers, validated by the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

struct Problem {
  int64_t bt, T, H, P, N, G, Q;  // batch, seqlen, nheads, headdim, dstate, ngroups, chunk
  int64_t nc, Tp;                // nchunks, nchunks * chunk
  int io;                        // 0 = fp32, 1 = bf16 (x, B, C, y)
  int dt_head_major;             // dt is [bt][H][T] instead of [bt][T][H]
  const void* x;
  const float* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const float* init;             // may be null (zeros)
  void* y;
  float* final_state;            // may be null (not written)
  float* gcum;                   // workspace: [bt][H][Tp]
  float* dtt;                    // workspace: [bt][H][Tp]
  float* wst;                    // workspace: [bt][H][Tp]
  float* states;                 // workspace: [bt][H][nc][P][N]
  void* hprev;                   // workspace: [bt][H][nc][P][N] fp32, or bf16 (hi, lo) pairs
  float* chain;                  // workspace (chained path): [bt][H][P][N] carried state slots
  int* sync;                     // workspace (chained path): ticket counter, error word, flags per (bt, H)
  int nsync;                     // int32 words of sync (0 = none); ssd_chunk_cumsum clears them
};

// One decode step (see ssd_step.hip). Device pointers, validated by the ABI.
struct StepProblem {
  int64_t bt, H, P, N, G;        // batch, nheads, headdim, dstate, ngroups
  int io;                        // 0 = fp32, 1 = bf16 (x, B, C, y)
  const void* x;                 // [bt][H][P]
  const float* dt;               // [bt][H]
  const float* A;                // [H]
  const void* B;                 // [bt][G][N]
  const void* C;                 // [bt][G][N]
  const float* D;                // [H]
  float* state;                  // [bt][H][P][N], read and written
  void* y;                       // [bt][H][P]
};

// Each launcher enqueues one kernel on `stream` and returns the launch status.
hipError_t launch_chunk_cumsum(const Problem& p, hipStream_t stream);
hipError_t launch_chunk_state(const Problem& p, hipStream_t stream);
hipError_t launch_state_pass(const Problem& p, hipStream_t stream);
hipError_t launch_chunk_scan(const Problem& p, hipStream_t stream);
hipError_t launch_ssd_step(const StepProblem& p, hipStream_t stream);
// The chunk states and the state pass in one kernel (chunk_state.hip): the
// shapes it supports, and the sizes for which the forward call prefers it.
bool chunk_state_pass_fits(const Problem& p);
bool chunk_state_pass_pays(const Problem& p);
hipError_t launch_chunk_state_pass(const Problem& p, hipStream_t stream);
// States, pass and outputs in one kernel, the carried state handed from
// chunk to chunk through memory (chunk_chained.hip); the cumsum kernel clears
// its counters.
bool chunk_chained_fits(const Problem& p);
hipError_t launch_chunk_chained(const Problem& p, hipStream_t stream);
// The C.B^T-resident scan (chunk_scan_resident.hip) and the shapes it takes.
bool chunk_scan_resident_fits(const Problem& p);
hipError_t launch_chunk_scan_resident(const Problem& p, hipStream_t stream);

// Compile-time instantiation tables (host queries, no GPU needed).
bool chunk_state_has(int io, int64_t P, int64_t N, int64_t Q);
bool chunk_scan_has(int io, int64_t P, int64_t N, int64_t Q);
bool step_has(int io, int64_t N);

// Grid-dimension limits the launchers rely on (y and z <= 65535).
constexpr int64_t kMaxGridYZ = 65535;

}  // namespace ssd

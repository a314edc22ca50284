// Device helpers of the kernel that hands the carried state from chunk to
// chunk through memory (ssd_chunk_chained): direct global->LDS loads,
// wave-uniform buffer resources, the progress flags of the hand-off, and the
// piece swizzle of the B tile in LDS.
//
// The hand-off protocol (the blog's "Kernel 2: fwd_pass_state" walks a head's
// chunks in order inside one program; here the chunks of a head are spread
// over workgroups, each waiting for its predecessor). Work items ("tickets")
// are numbered chunk-major and claimed in order from a counter by persistent
// workgroups. The tile of chunk k of a head stores h_{k+1} with
// device-coherent stores, waits for them to complete, and then raises the
// head's progress flag to k+1; the tile of chunk k+1 polls that flag with
// device-coherent loads and reads the state the same way. A tile waits only
// on a lower ticket, claimed by a workgroup that is already running and that
// only waits on lower tickets itself, so every wait ends; the polls are
// bounded all the same (on the bound the error word is set and the wait
// gives up). ssd_chunk_cumsum clears the counter and the flags.
#pragma once

#include "ssd_device.h"

namespace ssd {
namespace lookback {

// Layout of the sync region (int32 words): words 0-1 the 64-bit ticket
// counter, word 2 the error word, from word 64 one progress flag per
// (batch, head).
constexpr int kSyncErr = 2;
constexpr int kSyncFlags = 64;
constexpr int kMaxPolls = 1 << 18;      // bound of one wait (each poll sleeps, then reloads)

// 16-byte piece c of a B row t (N bf16, N / 8 pieces) is stored at piece
// c ^ bswz(t): the transposing reads of the chunk-state product (4 rows x 2
// adjacent pieces per 16 lanes) and the row fragment reads of C.B^T (16 rows
// x 1 piece per 16 lanes) both hit 16 distinct 16-byte bank groups. Period:
// N / 8 rows.
template <int N>
__device__ __forceinline__ constexpr uint32_t bswz(uint32_t t) {
  constexpr uint32_t H = N / 16;
  return 2 * (t % H) + (t / H) % 2;
}

// Direct global->LDS load of 16 bytes per lane from a wave-uniform base plus
// a per-lane offset; lane i's bytes land at lds + 16 i (lds wave-uniform, in
// M0). SC1: device-coherent (the load misses any cache that could hold a
// stale copy written by another XCD).
template <bool SC1>
__device__ __forceinline__ void dma16(const void* sbase_in, uint32_t voff, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  // the base is wave-uniform by construction; say so, so it goes in SGPRs
  const uint64_t a = reinterpret_cast<uint64_t>(sbase_in);
  const void* sbase = reinterpret_cast<const void*>(
      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
      (uint32_t)__builtin_amdgcn_readfirstlane((int)a));
  if constexpr (SC1)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 sc1" ::"s"(m0), "v"(voff), "s"(sbase)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}

// The same through a buffer resource: lane i's 16 bytes at byte voff + soff
// of the resource land at lds + 16 i; offsets at or past the resource's
// size load zeros (the zero padding of a ragged chunk, with no branches).
template <bool SC1>
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  if constexpr (SC1)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen sc1 lds" ::"s"(m0), "v"(voff), "s"(r), "s"(so)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0), "v"(voff), "s"(r), "s"(so)
                 : "memory", "m0");
}

// A buffer resource built from wave-uniform values read back as such (so it
// sits in SGPRs even where the compiler has kept its inputs in VGPRs).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t urs(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const void* b = reinterpret_cast<const void*>(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                                                (uint32_t)__builtin_amdgcn_readfirstlane((int)a));
  return make_rsrc(b, (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes));
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)v));
}

__device__ __forceinline__ void vm_wait0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void vm_lds_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Flags are read and written with relaxed device-scope atomics
// (device-coherent on every XCD); ordering against the state itself comes
// from the state's stores completing (vmcnt) before the flag is raised.
__device__ __forceinline__ int load_flag(const int* f) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void store_flag(int* f, int v) {
  __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (the whole wave) until *f >= want; on the bound, record the error word.
__device__ __forceinline__ void wait_flag(const int* f, int want, int* sync) {
  int v = load_flag(f);
  int polls = 0;
  while (v < want) {
    __builtin_amdgcn_s_sleep(2);
    if (++polls > kMaxPolls) {
      store_flag(sync + kSyncErr, 1);
      break;
    }
    v = load_flag(f);
  }
}

// Claim the next ticket (one lane calls it).
__device__ __forceinline__ int64_t claim_ticket(int* sync) {
  return __hip_atomic_fetch_add(reinterpret_cast<long long*>(sync), 1LL, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace lookback
}  // namespace ssd

// Device helpers shared by the selective-scan kernels (s6_scan.hip,
// s6_bwd.hip): a wave's 64 channel rows of a chunk's 64 (or 32) tokens
// through LDS.
#pragma once

#include "lookback_device.h"
#include "ssd_device.h"

namespace ssd {
namespace s6 {

// A wave's 64 channel rows of TOK tokens (TOK = 64: 256 bytes per row, or
// 32: 128 bytes) in LDS: 16-byte piece q (tokens 4 q .. 4 q + 3) of row r
// sits at piece q ^ (r % (TOK / 4)), so both the coalesced transfers (whole
// rows, 1 KB per instruction) and each lane's walk along its own row hit
// distinct 16-byte bank groups.
template <int TOK = 64>
__device__ __forceinline__ uint32_t tile_off(uint32_t r, uint32_t q) {
  static_assert(TOK == 64 || TOK == 32, "tile rows of 64 or 32 tokens");
  return r * (TOK * 4) + ((q ^ (r & (TOK / 4 - 1))) << 4);
}

// rows [rows0 .. rows0 + 63] of a [rows][L] array, tokens t0 .. t0 + TOK - 1,
// into the wave's tile by direct global->LDS loads (rows at or past
// `rows_valid` read as zeros; the caller masks tokens past the sequence)
template <int TOK = 64>
__device__ __forceinline__ void tile_load(const float* src, int64_t row0, int rows_valid, int64_t L, int64_t t0,
                                          unsigned char* tile, int lane) {
  constexpr int P = TOK / 4;   // 16-byte pieces per row; 64 / P rows per instruction
  asm volatile("" : "+v"(lane));   // per-lane offsets formed here, not kept live across the ticket
  const __amdgpu_buffer_rsrc_t r = lookback::urs(src + row0 * L, (uint32_t)((int64_t)rows_valid * L * 4));
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const uint32_t row = (uint32_t)((64 / P) * i + lane / P), q = (uint32_t)(lane % P) ^ (row % P);
    lookback::bdma16<false>(r, (uint32_t)(row * L + t0 + 4 * q) * 4, 0, tile + i * 1024);
  }
}

// The same with 4-byte loads, for rows that are not 16-byte aligned: lane l
// takes token t0 + l of each row (zeros past the sequence or the rows).
template <int TOK = 64>
__device__ __forceinline__ void tile_load_scalar(const float* src, int64_t row0, int rows_valid, int64_t L,
                                                 int64_t t0, int nt, unsigned char* tile, int lane) {
  asm volatile("" : "+v"(lane));
#pragma unroll 8
  for (int r = 0; r < 64; ++r) {
    const float v = (r < rows_valid && lane < nt && lane < TOK) ? src[(row0 + r) * L + t0 + lane] : 0.f;
    if (lane < TOK)
      *reinterpret_cast<float*>(tile + tile_off<TOK>((uint32_t)r, (uint32_t)lane >> 2) + (lane & 3) * 4) = v;
  }
}


// A lane's whole row (its channel, TOK tokens) into registers through the
// wave's tile: zeros past the sequence (nt tokens) and for lanes at or past
// `rows_valid`. VEC: direct 16-byte loads of whole rows (rows 16-byte
// aligned; nt a multiple of 4 when the chunk is ragged).
template <bool VEC, int TOK = 64>
__device__ __forceinline__ void rows_in(const float* src, int64_t row0, int rows_valid, int64_t L, int64_t t0,
                                        int nt, unsigned char* tile, int lane, float* v) {
  if constexpr (VEC) {
    if (rows_valid > 0) tile_load<TOK>(src, row0, rows_valid < 64 ? rows_valid : 64, L, t0, tile, lane);
  } else {
    tile_load_scalar<TOK>(src, row0, rows_valid, L, t0, nt, tile, lane);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const bool row_in = ln < rows_valid;
#pragma unroll
  for (int q = 0; q < TOK / 4; ++q) {
    const float4 w = *reinterpret_cast<const float4*>(tile + tile_off<TOK>((uint32_t)ln, (uint32_t)q));
    const bool in = row_in && (!VEC || 4 * q < nt);
    v[4 * q] = in ? w.x : 0.f;
    v[4 * q + 1] = in ? w.y : 0.f;
    v[4 * q + 2] = in ? w.z : 0.f;
    v[4 * q + 3] = in ? w.w : 0.f;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read out before the tile is refilled
}

// The inverse: each lane's row of TOK values out through the wave's tile, as
// whole rows (rows at or past `rows_valid` and tokens past nt are not
// written).
template <bool VEC, int TOK = 64>
__device__ __forceinline__ void rows_out(float* dst, int64_t row0, int rows_valid, int64_t L, int64_t t0, int nt,
                                         unsigned char* tile, int lane, const float* v) {
  constexpr int P = TOK / 4;
  int ln = lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int q = 0; q < P; ++q)
    *reinterpret_cast<float4*>(tile + tile_off<TOK>((uint32_t)ln, (uint32_t)q)) =
        make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if constexpr (!VEC) {
#pragma unroll 8
    for (int r = 0; r < 64; ++r) {
      const float w = ln < TOK ? *reinterpret_cast<const float*>(tile + tile_off<TOK>((uint32_t)r, (uint32_t)ln >> 2) +
                                                                 (ln & 3) * 4)
                               : 0.f;
      if (r < rows_valid && ln < nt && ln < TOK) dst[(row0 + r) * L + t0 + ln] = w;
    }
  } else if (rows_valid > 0) {
    const __amdgpu_buffer_rsrc_t rd =
        lookback::urs(dst + row0 * L, (uint32_t)((int64_t)(rows_valid < 64 ? rows_valid : 64) * L * 4));
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const uint32_t r = (uint32_t)((64 / P) * i + ln / P), q = (uint32_t)(ln % P) ^ (r % P);
      const u32x4 w = *reinterpret_cast<const u32x4*>(tile + r * (TOK * 4) + ((uint32_t)(ln % P) << 4));
      if ((int)(4 * q) < nt) __builtin_amdgcn_raw_buffer_store_b128(w, rd, (r * (uint32_t)L + (uint32_t)t0 + 4 * q) * 4, 0, 0);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read out before the tile is refilled
}

}  // namespace s6
}  // namespace ssd

// The Mamba-1 selective scan (S6): one scalar state per (batch row, channel
// d, state n), discretized per step ("Mamba: The Hard Way", Part 5):
//
//   h[n] <- exp(delta_t A[d, n]) h[n] + delta_t B[n, t] x_t,   y_t = sum_n C[n, t] h[n]
//
// Layouts: x, delta, y [batch][channels][seqlen]; B, C [batch][dstate][seqlen];
// A [channels][dstate]; states [batch][channels][dstate]; all fp32.
//
// The sequence is cut into chunks of kChunk tokens. One kernel, s6_onepass,
// takes work items ("tickets") (chunk c, batch row b, block of 256 channels),
// numbered chunk-major and claimed in order by persistent workgroups; a lane
// owns one channel and holds its chunk's x and delta in registers, so each is
// read from memory once:
//   1. the chunk is scanned from a zero state: its end state S and its sum of
//      delta, published (device-coherent stores, then flag 1 for the block);
//   2. the state entering the chunk is found by looking back over the earlier
//      chunks of the same rows: a chunk whose flag is 2 has published its
//      inclusive end state P and ends the walk; a chunk with flag 1
//      contributes its S and its decay exp(A sum(delta)) (the chunk's decays
//      multiply to that) and the walk goes on. The walk never passes chunk 0:
//      there it waits for flag 2, which chunk 0 raises without waiting on
//      anything (it alone reads h0, before any inclusive state exists, so hT
//      may be h0);
//   3. the inclusive end state is published (flag 2) and the chunk is
//      scanned again from the entering state, writing y.
// A tile waits only for flag 1 of lower tickets, which their workgroups
// raise before they wait on anything, or for flag 2 of chunk 0: every wait
// ends (the polls are bounded all the same, recording an error word). The
// "Part 2/3" view of the page is the same: a scan splits into blocks whose
// summaries combine associatively. A small kernel clears the counter and
// flags first.
#include "lookback_device.h"
#include "ssd_device.h"
#include "s6_device.h"
#include "s6_launch.h"

namespace ssd {

namespace {

constexpr int kChunk = 64;    // tokens per chunk
constexpr int kLanes = 256;   // threads per workgroup (4 waves)

// Lanes per channel: dstate 16 splits each channel's states over a lane
// pair (8 each), which keeps two waves per SIMD; the pair's partial outputs
// are added by one DPP step. Channels per workgroup: kLanes / NL.
template <int N> struct Lanes { static constexpr int NL = N >= 16 ? 2 : 1, NS = N / NL, CB = kLanes / NL; };
constexpr int kSyncWords = 64;   // sync region head: ticket counter (0-1), error word (2)
constexpr int kMaxPolls = 1 << 20;

// A lane's N-float chunk summary (N consecutive floats at byte `off` of a
// wave-uniform resource), stored or loaded device-coherent in 16-, 8- or
// 4-byte pieces, so the writes through to memory are whole lines per wave.
template <int N>
__device__ __forceinline__ void st_state(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* v) {
  if constexpr (N == 1) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), r, off, 0, 16);
  } else if constexpr (N == 2) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(v[0]), __float_as_uint(v[1])}, r, off, 0, 16);
  } else {
#pragma unroll
    for (int q = 0; q < N / 4; ++q)
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                                                   __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3])},
                                             r, off + 16 * q, 0, 16);
  }
}
template <int N>
__device__ __forceinline__ void ld_state(__amdgpu_buffer_rsrc_t r, uint32_t off, float* v) {
  if constexpr (N == 1) {
    v[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 16));
  } else if constexpr (N == 2) {
    const auto w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 16);
    v[0] = __uint_as_float(w[0]);
    v[1] = __uint_as_float(w[1]);
  } else {
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * q, 0, 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = __uint_as_float(w[e]);
    }
  }
}

__device__ __forceinline__ int flag_of(const int* f) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// wait (the whole wave) until *f >= want; returns the value seen
__device__ __forceinline__ int wait_flag(const int* f, int want, int* sync) {
  int v = flag_of(f);
  for (int polls = 0; v < want; ++polls) {
    if (polls > kMaxPolls) {
      __hip_atomic_store(sync + 2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
    v = flag_of(f);
  }
  return v;
}

__global__ void s6_clear(int* sync, int64_t words) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    sync[i] = 0;
}

// seqlen 0: the final state is the initial one (or zeros)
__global__ void s6_pass_state(const float* h0, float* hT, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) hT[i] = h0 ? h0[i] : 0.f;
}

// BWD: the backward pass's forward sweep. No y and no final state; instead,
// from dy, each chunk's adjoint record for the backward pass: O, the
// adjoint that the chunk's own dy leaves at its first token,
// sum_t (a_t0 ... a_t) C_t dy_t per state, and the chunk's sum of delta SD
// (so the backward pass needs no reverse sweep of its own per chunk).
template <int N, bool VEC, bool BWD>
__global__ __launch_bounds__(kLanes) __attribute__((amdgpu_waves_per_eu(2))) void s6_onepass(const float* __restrict__ x, const float* __restrict__ dl,
                                                     const float* __restrict__ A, const float* __restrict__ Bm,
                                                     const float* __restrict__ Cm, const float* h0, float* y,
                                                     float* hT, float* aggS, float* aggD, float* incl, int* sync,
                                                     const float* __restrict__ dy, float* __restrict__ Oc,
                                                     float* __restrict__ SD, int64_t L, int D, int64_t nc,
                                                     int64_t ntickets) {
  __shared__ __attribute__((aligned(16))) float sB[N][kChunk];
  __shared__ __attribute__((aligned(16))) float sC[N][kChunk];
  __shared__ __attribute__((aligned(1024))) unsigned char sT[kLanes / 64][64 * 256];   // per wave: x, delta, then y
  __shared__ int64_t sTicket;
  constexpr int NL = Lanes<N>::NL, NS = Lanes<N>::NS, CB = Lanes<N>::CB, RW = 64 / NL;   // RW: rows per wave
  const int tid = threadIdx.x;
  const int sub = tid % NL;   // the lane's states: sub NS .. sub NS + NS - 1
  // (the wave index read back as uniform: the tile addresses it forms stay in
  // scalar registers)
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  unsigned char* const tile = sT[wave];
  const int ncb = (D + CB - 1) / CB;
  const int64_t per = ntickets / nc;   // tickets per chunk = batch rows * channel blocks
  int* const flags = sync + kSyncWords;

  if (tid == 0) sTicket = __hip_atomic_fetch_add(reinterpret_cast<long long*>(sync), 1LL, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int64_t ticket = sTicket;
  while (ticket < ntickets) {
    const int64_t c = ticket / per;
    const int64_t u = ticket % per;
    const int64_t b = u / ncb;
    const int cb = (int)(u % ncb);
    const int d = cb * CB + tid / NL;
    const bool valid = d < D;
    const int64_t t0 = c * kChunk;
    const int nt = L - t0 < kChunk ? (int)(L - t0) : kChunk;

    for (int idx = tid; idx < N * kChunk; idx += kLanes) {
      const int n = idx / kChunk, k = idx % kChunk;
      const int64_t o = (b * N + n) * L + t0 + k;
      sB[n][k] = k < nt ? Bm[o] : 0.f;
      sC[n][k] = k < nt ? Cm[o] : 0.f;
    }
    // the lane's x and delta (zeros past the sequence or the channels)
    float xr[kChunk], dr[kChunk];
    const int64_t wrow0 = b * D + cb * CB + wave * RW;   // the wave's first row
    const int wrows = D - (cb * CB + wave * RW);          // its rows inside the array (may be <= 0)
    {
      // whole rows through the wave's tile: x, then delta (the tile is the
      // wave's own, so no workgroup barrier; a direct load has landed in LDS
      // once vmcnt says so)
      float* const dst[2] = {xr, dr};
      const float* const srcs[2] = {x, dl};
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        if constexpr (VEC) {
          if (wrows > 0) s6::tile_load(srcs[a], wrow0, wrows < RW ? wrows : RW, L, t0, tile, lane);
        } else {
          s6::tile_load_scalar(srcs[a], wrow0, wrows < RW ? wrows : RW, L, t0, nt, tile, lane);
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        int ln = lane / NL;   // the lane's channel row (a lane pair reads the same row)
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int q = 0; q < kChunk / 4; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(tile + s6::tile_off((uint32_t)ln, (uint32_t)q));
          // (past the sequence the direct loads read the next row: masked here;
          // nt is a multiple of 4 on that path)
          const bool in = !VEC || 4 * q < nt;
          dst[a][4 * q] = in ? v.x : 0.f;
          dst[a][4 * q + 1] = in ? v.y : 0.f;
          dst[a][4 * q + 2] = in ? v.z : 0.f;
          dst[a][4 * q + 3] = in ? v.w : 0.f;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read out before the tile is refilled
      }
    }
    if constexpr (BWD) {
      // dy stays in the tile, read 4 tokens at a time by its lane (past the
      // sequence it holds the next row's tokens, which meet C = 0 there)
      if constexpr (VEC) {
        if (wrows > 0) s6::tile_load(dy, wrow0, wrows < RW ? wrows : RW, L, t0, tile, lane);
      } else {
        s6::tile_load_scalar(dy, wrow0, wrows < RW ? wrows : RW, L, t0, nt, tile, lane);
      }
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    }
    float a2[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) a2[n] = valid ? A[(int64_t)d * N + sub * NS + n] * kLog2e : 0.f;
    __syncthreads();   // B and C staged

    // 1. the chunk from a zero state. Past the sequence x, delta, B and C are
    // zero, so padded tokens leave h unchanged (exp2(0) = 1, no input).
    float h[NS], pa[NS], oa[NS];   // (BWD: the running decay product and O)
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      h[n] = 0.f;
      pa[n] = 1.f;
      oa[n] = 0.f;
    }
    float dsum = 0.f;
    int lnb = lane / NL;
    asm volatile("" : "+v"(lnb));
#pragma unroll
    for (int t4 = 0; t4 < kChunk; t4 += 4) {
      float u[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u[j] = dr[t4 + j] * xr[t4 + j];
        dsum += dr[t4 + j];
      }
      float gj[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BWD) {
        const float4 g4 = *reinterpret_cast<const float4*>(tile + s6::tile_off((uint32_t)lnb, (uint32_t)(t4 / 4)));
        gj[0] = g4.x;
        gj[1] = g4.y;
        gj[2] = g4.z;
        gj[3] = g4.w;
      }
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        const float4 b4 = *reinterpret_cast<const float4*>(&sB[sub * NS + n][t4]);
        const float bj[4] = {b4.x, b4.y, b4.z, b4.w};
        if constexpr (BWD) {
          const float4 c4 = *reinterpret_cast<const float4*>(&sC[sub * NS + n][t4]);
          const float cj[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float a = exp2_hw(dr[t4 + j] * a2[n]);
            h[n] = fmaf(a, h[n], u[j] * bj[j]);
            pa[n] *= a;
            oa[n] = fmaf(pa[n], cj[j] * gj[j], oa[n]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) h[n] = fmaf(exp2_hw(dr[t4 + j] * a2[n]), h[n], u[j] * bj[j]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one group of tokens at a time: bounded live ranges
    }
    if constexpr (BWD) {
      // (through resources over the block's valid records: no branch, which
      // the compiler would otherwise sink the O chain into)
      const int64_t rec0 = (b * nc + c) * D + cb * CB;
      const uint32_t nrec = (uint32_t)(D - cb * CB < CB ? D - cb * CB : CB);
      st_state<NS>(lookback::urs(Oc + rec0 * N, nrec * N * 4), (uint32_t)tid * NS * 4, oa);
      st_state<1>(lookback::urs(SD + rec0, nrec * 4), (uint32_t)(tid / NL) * 4, &dsum);
    }
    int* const myflag = flags + (b * nc + c) * ncb + cb;

    // 2. the entering state
    float hin[NS];
    if (c == 0) {
#pragma unroll
      for (int n = 0; n < NS; ++n) hin[n] = (h0 && valid) ? h0[(b * D + d) * N + sub * NS + n] : 0.f;
    } else {
      {
        // the workgroup's CB records (those of channels past D are dropped;
        // a lane pair's two lanes write the same delta sum)
        const int64_t rec0 = (b * nc + c) * D + cb * CB;
        const uint32_t nrec = (uint32_t)(D - cb * CB < CB ? D - cb * CB : CB);
        st_state<NS>(lookback::urs(aggS + rec0 * N, nrec * N * 4), (uint32_t)tid * NS * 4, h);
        st_state<1>(lookback::urs(aggD + rec0, nrec * 4), (uint32_t)(tid / NL) * 4, &dsum);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();   // every lane's aggregate is out
      if (tid == 0) __hip_atomic_store(myflag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // hin = acc + lam * (inclusive state of the chunk where the walk ends)
      float acc[NS], lam[NS];
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        acc[n] = 0.f;
        lam[n] = 1.f;
      }
      // (the flag of chunk j - 1 is read together with chunk j's summary: one
      // round trip per chunk walked)
      int fseen = flag_of(flags + (b * nc + c - 1) * ncb + cb);
      for (int64_t j = c - 1;; --j) {
        const int* fj = flags + (b * nc + j) * ncb + cb;
        const int want = j == 0 ? 2 : 1;
        const int f = fseen >= want ? fseen : wait_flag(fj, want, sync);
        const int64_t rj = (b * nc + j) * D + cb * CB;   // chunk j's records of this block
        const uint32_t nrec = (uint32_t)(D - cb * CB < CB ? D - cb * CB : CB);
        if (f >= 2 || j == 0) {   // (at chunk 0 only after a wait that hit its bound is f < 2)
          float pj[NS];
          ld_state<NS>(lookback::urs(incl + rj * N, nrec * N * 4), (uint32_t)tid * NS * 4, pj);
#pragma unroll
          for (int n = 0; n < NS; ++n) hin[n] = valid ? fmaf(lam[n], pj[n], acc[n]) : 0.f;
          break;
        }
        float sj[NS], sd;
        ld_state<NS>(lookback::urs(aggS + rj * N, nrec * N * 4), (uint32_t)tid * NS * 4, sj);
        ld_state<1>(lookback::urs(aggD + rj, nrec * 4), (uint32_t)(tid / NL) * 4, &sd);
        fseen = flag_of(fj - ncb);   // chunk j - 1 (j >= 1 here)
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          acc[n] = fmaf(lam[n], sj[n], acc[n]);
          lam[n] *= exp2_hw(a2[n] * sd);
        }
      }
    }
    // 3. the inclusive end state, published; hT after the last chunk
    {
      const bool last = c + 1 == nc;
      float hout[NS];
#pragma unroll
      for (int n = 0; n < NS; ++n) hout[n] = fmaf(exp2_hw(a2[n] * dsum), hin[n], h[n]);
      if (!last) {
        const int64_t rec0 = (b * nc + c) * D + cb * CB;
        const uint32_t nrec = (uint32_t)(D - cb * CB < CB ? D - cb * CB : CB);
        st_state<NS>(lookback::urs(incl + rec0 * N, nrec * N * 4), (uint32_t)tid * NS * 4, hout);
      } else if (hT && valid) {
#pragma unroll
        for (int n = 0; n < NS; ++n) hT[(b * D + d) * N + sub * NS + n] = hout[n];
      }
      if (!last) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) __hip_atomic_store(myflag, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // ... and the chunk again from the entering state: y replaces x (unless
    // no y is asked for: the backward pass runs this kernel for the chunks'
    // end states alone). (The
    // decays are recomputed: kept from the first scan they would take 64 N
    // registers per lane, so the operands are laundered to stop the compiler
    // from keeping them.)
    if (!BWD && y) {
#pragma unroll
    for (int t = 0; t < kChunk; ++t) asm volatile("" : "+v"(dr[t]));
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      asm volatile("" : "+v"(a2[n]));
      h[n] = hin[n];
    }
#pragma unroll
    for (int t4 = 0; t4 < kChunk; t4 += 4) {
      float u[4], yv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) u[j] = dr[t4 + j] * xr[t4 + j];
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        const float4 b4 = *reinterpret_cast<const float4*>(&sB[sub * NS + n][t4]);
        const float4 c4 = *reinterpret_cast<const float4*>(&sC[sub * NS + n][t4]);
        const float bj[4] = {b4.x, b4.y, b4.z, b4.w}, cj[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h[n] = fmaf(exp2_hw(dr[t4 + j] * a2[n]), h[n], u[j] * bj[j]);
          yv[j] = fmaf(cj[j], h[n], yv[j]);
        }
      }
      if constexpr (NL == 2) {
        // the pair's partial sums over their states: each lane adds its
        // partner's (lanes 2i, 2i + 1; DPP quad permutation 1, 0, 3, 2)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          yv[j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(yv[j]), 0xB1, 0xF, 0xF, false));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) xr[t4 + j] = yv[j];
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      // through the tile: each lane writes its row (a lane pair its two
      // halves), then whole rows go out
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const uint32_t row = (uint32_t)(ln / NL);
#pragma unroll
      for (int q = 0; q < kChunk / 4; ++q)
        if (NL == 1 || q / (kChunk / 4 / NL) == sub)
          *reinterpret_cast<float4*>(tile + s6::tile_off(row, (uint32_t)q)) =
              make_float4(xr[4 * q], xr[4 * q + 1], xr[4 * q + 2], xr[4 * q + 3]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (!VEC) {
        // lane l stores token t0 + l of each row
#pragma unroll 8
        for (int r = 0; r < RW; ++r) {
          const float v = *reinterpret_cast<const float*>(tile + s6::tile_off((uint32_t)r, (uint32_t)ln >> 2) + (ln & 3) * 4);
          if (r < wrows && ln < nt) y[(wrow0 + r) * L + t0 + ln] = v;
        }
      } else if (wrows > 0) {
        const __amdgpu_buffer_rsrc_t ry =
            lookback::urs(y + wrow0 * L, (uint32_t)((int64_t)(wrows < RW ? wrows : RW) * L * 4));
#pragma unroll
        for (int i = 0; i < RW / 4; ++i) {
          const uint32_t r = (uint32_t)(4 * i + (ln >> 4)), q = (uint32_t)(ln & 15) ^ (r & 15);
          const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * 256 + ((uint32_t)(ln & 15) << 4));
          if ((int)(4 * q) < nt) __builtin_amdgcn_raw_buffer_store_b128(v, ry, (r * (uint32_t)L + (uint32_t)t0 + 4 * q) * 4, 0, 0);
        }
      }
    }
    }
    // the next ticket (the B, C tiles are free once every lane is past them)
    __syncthreads();
    if (tid == 0) sTicket = __hip_atomic_fetch_add(reinterpret_cast<long long*>(sync), 1LL, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    ticket = sTicket;
  }
}

template <int N, bool VEC, bool BWD>
int onepass_slots() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    dev = 0;
  }
  if (!cached[dev]) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, s6_onepass<N, VEC, BWD>, kLanes, 0) != hipSuccess || cus <= 0 ||
        per_cu <= 0) {
      (void)hipGetLastError();
      cus = 256;
      per_cu = 1;
    }
    cached[dev] = cus * per_cu;
  }
  return cached[dev];
}

template <int N>
hipError_t launch_n(const S6Problem& p, hipStream_t s) {
  const int64_t nc = (p.L + kChunk - 1) / kChunk;
  const int64_t rows = p.bt * p.D;
  if (rows == 0) return hipSuccess;
  if (nc == 0) {
    if (p.hT && p.hT != p.h0) {
      const int64_t n = rows * N;
      hipLaunchKernelGGL(s6_pass_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p.h0, p.hT, n);
    }
    return hipGetLastError();
  }
  // whole 16-byte pieces of x, delta and y through LDS when every row starts
  // 16-byte aligned (and 64 rows of one array stay below 2 GB of offsets)
  const int vec = (p.L % 4 == 0 && p.L <= ((int64_t)1 << 22) && (reinterpret_cast<uintptr_t>(p.x) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.delta) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.y) & 15) == 0 && (reinterpret_cast<uintptr_t>(p.dy) & 15) == 0)
                      ? 1 : 0;
  const int64_t ncb = (p.D + Lanes<N>::CB - 1) / Lanes<N>::CB;
  const int64_t ntickets = nc * p.bt * ncb;
  const int64_t words = kSyncWords + ntickets;
  const int64_t cblocks = (words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024;
  hipLaunchKernelGGL(s6_clear, dim3((unsigned)cblocks), dim3(256), 0, s, p.sync, words);
  const auto go = [&](auto kernel, int slots) {
    const int64_t grid = ntickets < slots ? ntickets : slots;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kLanes), 0, s, p.x, p.delta, p.A, p.B, p.C, p.h0, p.y,
                       p.hT, p.aggS, p.aggD, p.incl, p.sync, p.dy, p.O, p.SD, p.L, (int)p.D, nc, ntickets);
  };
  if (p.dy) {
    if (vec)
      go(s6_onepass<N, true, true>, onepass_slots<N, true, true>());
    else
      go(s6_onepass<N, false, true>, onepass_slots<N, false, true>());
  } else if (vec) {
    go(s6_onepass<N, true, false>, onepass_slots<N, true, false>());
  } else {
    go(s6_onepass<N, false, false>, onepass_slots<N, false, false>());
  }
  return hipGetLastError();
}

}  // namespace

int64_t s6_sync_words(int64_t bt, int64_t D, int64_t L, int64_t N) {
  const int64_t nc = (L + kChunk - 1) / kChunk;
  const int64_t cbk = N >= 16 ? Lanes<16>::CB : kLanes;   // channels per workgroup
  return kSyncWords + nc * bt * ((D + cbk - 1) / cbk);
}

int64_t s6_chunk_tokens() { return kChunk; }

bool s6_has(int64_t N) { return N == 1 || N == 2 || N == 4 || N == 8 || N == 16; }

hipError_t launch_s6(const S6Problem& p, hipStream_t s) {
  switch (p.N) {
    case 1: return launch_n<1>(p, s);
    case 2: return launch_n<2>(p, s);
    case 4: return launch_n<4>(p, s);
    case 8: return launch_n<8>(p, s);
    case 16: return launch_n<16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd

// ssd_chunk_chained: the chunk states, the pass over them and the outputs in
// one kernel (bf16 io, headdim 64, chunk 256, dstate 64 or 128). For every
// (batch, chunk k, head) tile, with G' the chunk-local cumsum of A*dt times
// log2 e (from ssd_chunk_cumsum) and h_k the state entering chunk k:
//
//   S_k     = sum_t w_t x_t (x) B_t,   w_t = dt_t 2^(G'_last - G'_t)   (the chunk's own state)
//   h_{k+1} = 2^(G'_last) h_k + S_k                                    (the jump over the chunk)
//   y_t     = 2^(G'_t) C_t . h_k + sum_{j<=t} (C_t . B_j) 2^(G'_t - G'_j) dt_j x_j + D x_t
//
// (CUDA Tile Mamba-2 blog, section "Mamba-2 architecture": the jump formula
// and the decayed block output; "Kernel 2: fwd_pass_state" and "Kernel 3:
// compute_out" are the two halves fused here.)
//
// Why one kernel. Split into a state pass and an output kernel, the path
// writes every chunk's entering state to memory and reads it back, and reads
// x twice: about 1 GB of traffic per call at the 2.7B-like layer on top of
// the 0.7 GB that x, y, B, C and dt themselves need. Here every tile reads
// x once and writes y once; the only state that moves is h_k itself, handed
// from the tile of chunk k-1 to the tile of chunk k of the same head.
//
// The hand-off. Work items ("tickets") are (chunk k, batch b, block of HB
// heads of one group), numbered chunk-major and claimed in order from a
// counter by persistent workgroups. A tile needs h_k, which the tile of
// chunk k-1 of the same head publishes: it stores h_{k+1} to that head's slot
// in the workspace (device-coherent stores, so the value is visible to any
// XCD), waits for the stores to complete, and then raises the head's progress
// flag to k+1. The consumer polls the flag with device-coherent loads and
// then reads the slot the same way. The ticket a tile waits on has a lower
// number, so it was claimed by a workgroup that is already running and that
// only waits on lower tickets itself: every wait ends. (The polls are bounded
// all the same: a poll that outlives its bound records an error word in the
// workspace and goes on.) The counter and flags are cleared by
// ssd_chunk_cumsum, which runs first on the same stream.
//
// A ticket's heads share B and C (one group), so the workgroup computes the
// causal C.B^T blocks once per ticket and keeps them in AGPRs, as the
// resident scan does. Per head:
//   phase A   S_k^T = B^T (w o X): wave w takes headdim half w & 1 and the
//             dstate blocks NBW (w >> 1) + i, i < NBW = N / 64. B^T and X^T fragments
//             come from LDS by gfx950's transposing reads; w o X enters as a
//             bf16 (hi, lo) pair, two MFMAs against the exact bf16 B.
//   chain     h_k lands in LDS (fp32, padded rows) by direct global->LDS
//             loads; each wave reads its part in the accumulator layout of
//             S_k^T, forms h_{k+1} with fmaf and stores it, then rewrites
//             its part of h_k in place as bf16 (hi, lo) pairs, the operand
//             format of the carried-state product.
//   outputs   the resident scan's per-head work: carried-state term h_k.C^T
//             scaled by 2^(G'_t), then the intra-chunk block pairs (decay,
//             mask, dt and the hi/lo split applied to the resident C.B^T),
//             products formed transposed (y^T = x^T M^T), D x on the
//             diagonal, y out through LDS as 16-byte row pieces.
// The next head's x tile and G', dt rows (and before a new ticket its B tile)
// are loaded among this head's carried-state MFMAs and pairs.
#include "lookback_device.h"
#include "ssd_device.h"
#include "ssd_launch.h"

#include <type_traits>

namespace ssd {

namespace {

using namespace lookback;

template <int N>
struct CCfg {
  static constexpr int P = 64, Q = 256, NTB = 8, WAVES = 4, THREADS = 256;
  static constexpr int KS = N / 16;             // bf16 MFMA k-steps over dstate
  static constexpr int NBW = N / 64;            // dstate blocks per wave in phase A
  static constexpr int XBYTES = Q * P * 2;      // x tile, 128-byte rows
  static constexpr int GBYTES = 2 * Q * 4;      // G' row, then dt row
  static constexpr int HRB = N * 4 + 16;        // state row: N fp32 (or N bf16 pairs) + one pad piece
  static constexpr int HROWP = HRB / 16;
  static constexpr int HBYTES = P * HRB;
  static constexpr int BRB = N * 2;             // B row, unpadded, pieces swizzled
  static constexpr int NPC = BRB / 16;          // 16-byte pieces per B row
  static constexpr int BBYTES = Q * BRB;
  static constexpr int IX = XBYTES / 1024, IG = GBYTES / 1024, IH = HBYTES / 1024, IB = BBYTES / 1024;
  static constexpr int LX = IX / WAVES, LB = IB / WAVES;
  static constexpr int LH = (IH + WAVES - 1) / WAVES;
  static_assert(HBYTES % 1024 == 0 && IX % WAVES == 0 && IB % WAVES == 0, "whole direct-load instructions");
  static_assert(BBYTES + XBYTES + GBYTES + HBYTES + 4 * 4096 + 3 * Q * 4 + 64 <= 160 * 1024, "LDS");
};

__device__ __forceinline__ float to_agpr(float v) {
  float a;
  asm("v_accvgpr_write_b32 %0, %1" : "=a"(a) : "v"(v));
  return a;
}
__device__ __forceinline__ float from_agpr(float a) {
  float v;
  asm("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// The intra-chunk pairs of wave W, in emission order e = 0..11 (as the
// resident scan: slot 0 and slots 1..3 of t-block W, then slots 1..8 of
// t-block 7 - W).
__host__ __device__ constexpr bool pair_kept(int e, int W) {
  return !((e >= 4 && e < 7 && e - 3 <= W) || (e >= 1 && e < 4 && e > W));
}
__host__ __device__ constexpr int pair_jb(int e) { return e < 4 ? e : 8 - (e - 3); }
__host__ __device__ constexpr bool pair_diag(int e, int W) { return pair_jb(e) == (e < 4 ? W : 7 - W); }
__host__ __device__ constexpr int kept_index(int e, int W) {
  int n = 0;
  for (int f = 0; f < e; ++f)
    if (pair_kept(f, W)) ++n;
  return n;
}
__host__ __device__ constexpr int next_pair(int e, int W) {
  for (int f = e + 1; f < 12; ++f)
    if (pair_kept(f, W)) return f;
  return -1;
}

template <int N>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ssd_chunk_chained(const bf16* __restrict__ x, const bf16* __restrict__ Bm, const bf16* __restrict__ Cm,
                       const float* __restrict__ gcum, const float* __restrict__ dtt, const float* __restrict__ Dp,
                       const float* init, bf16* __restrict__ y, float* final_state, float* chain, int* sync,
                       int64_t Tlen, int H, int G, int64_t nc, int64_t Tp, int HB, int64_t ntickets) {
  using Cf = CCfg<N>;
  using I = Io<bf16>;
  using Frag = bf16x8;
  constexpr int P = 64, Q = 256, KS = Cf::KS, HRB = Cf::HRB, BRB = Cf::BRB, NBW = Cf::NBW;
  typedef short s16x4 __attribute__((ext_vector_type(4)));

  __shared__ __attribute__((aligned(1024))) unsigned char sB[Cf::BBYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char sX[Cf::XBYTES + Cf::GBYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char sH[Cf::HBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char sY[4 * 4096];
  __shared__ __attribute__((aligned(16))) float sW[Q];    // dt_j 2^(G'_end(block of j) - G'_j) <= dt_j
  __shared__ __attribute__((aligned(16))) float sE[Q];    // 2^(G'_t) <= 1
  __shared__ __attribute__((aligned(16))) float sWs[Q];   // dt_t 2^(G'_last - G'_t) <= dt_t
  __shared__ int64_t sTicket;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  __builtin_assume(wave >= 0 && wave < 4);
  const int lane = tid % 64;
  const int tb0 = wave, tb1 = 7 - wave;
  const int NHB = H / HB;
  const uint32_t xrb = (uint32_t)H * P * 2;       // x / y row stride in bytes
  const float* sG = reinterpret_cast<const float*>(sX + Cf::XBYTES);
  const float* sDt = sG + Q;

  // x tile direct loads: instruction kk (8 rows) puts lane l at row
  // 8 kk + l / 8, 16-byte piece (l % 8) with the 64-byte halves swapped in
  // rows with bit 1 set. B tile direct loads: instruction kk puts lane l at
  // row RPI kk + t_l, stored piece c_s = l % PPR, which holds logical piece
  // c_s ^ bswz(row); the swizzle of row RPI (wave + 4 i) + t_l equals that of
  // RPI wave + t_l (bswz has period 16 rows for N = 128 and 8 for N = 64), so
  // a lane's source offset is one constant for all of its B loads. The
  // per-lane offsets are derived where a group of loads is issued, from a
  // laundered lane id, so they do not stay live across the head.
  constexpr int PPR = BRB / 16, RPI = 1024 / BRB;
  const uint32_t bstride = (uint32_t)G * N * 2;
  struct LoadLane {
    uint32_t jl, xpiece, x_lane, b_tl, b_cs, b_lane;
  };
  auto load_lane = [&]() {
    int ll = lane;
    asm volatile("" : "+v"(ll));
    LoadLane L;
    L.jl = (uint32_t)ll >> 3;
    L.xpiece = (((uint32_t)ll & 7) ^ ((L.jl & 2) << 1)) * 16;
    L.x_lane = L.jl * xrb + L.xpiece;
    L.b_tl = (uint32_t)ll / PPR;
    L.b_cs = (uint32_t)ll % PPR;
    L.b_lane = L.b_tl * bstride + ((L.b_cs ^ bswz<N>((uint32_t)(RPI * wave) + L.b_tl)) * 16);
    return L;
  };

  // resources over one head's chunk of x (rows past the sequence read as
  // zeros), over the chunk's B rows of one group, and over one state
  auto x_rsrc = [&](int b, int k, int h, int nvalid) {
    const bf16* xs = x + (((int64_t)b * Tlen + (int64_t)k * Q) * H + h) * P;
    return urs(xs, (uint32_t)(nvalid - 1) * xrb + P * 2);
  };
  auto b_rsrc = [&](const bf16* bt, int nvalid) { return urs(bt, (uint32_t)(nvalid - 1) * bstride + N * 2); };
  // one of the LX x-row loads (instruction i of this wave)
  auto issue_x_one = [&](const LoadLane& L, __amdgpu_buffer_rsrc_t rx, int i) {
    int w = wave;
    asm volatile("" : "+s"(w));
    const int kk = w + 4 * i;
    bdma16<false>(rx, L.x_lane, (uint32_t)(kk * 8) * xrb, sX + kk * 1024);
  };
  // the G' row (wave 0) or dt row (wave 1) of head h of (b, k)
  auto issue_gd = [&](int b, int k, int h) {
    if (wave < Cf::IG) {
      const float* src = (wave == 0 ? gcum : dtt) + ((int64_t)b * H + h) * Tp + (int64_t)k * Q;
      bdma16<false>(urs(src, Q * 4), (uint32_t)lane * 16, 0, sX + Cf::XBYTES + wave * 1024);
    }
  };
  // one of the LB B-row loads (instruction i of this wave), swizzled pieces
  auto issue_B_one = [&](const LoadLane& L, __amdgpu_buffer_rsrc_t rb, int i) {
    int w = wave;
    asm volatile("" : "+s"(w));
    const int kk = w + 4 * i;
    bdma16<false>(rb, L.b_lane, (uint32_t)(RPI * kk) * bstride, sB + kk * 1024);
  };
  // one of the LH state-row loads (instruction i of this wave) of h_k into sH;
  // the pad piece of each row reads past the resource (zeros)
  auto issue_h_one = [&](__amdgpu_buffer_rsrc_t rh, bool coherent, int i) {
    int w = wave;
    asm volatile("" : "+s"(w));
    const int kk = w + 4 * i;
    if (kk < Cf::IH) {
      int ll = lane;
      asm volatile("" : "+v"(ll));
      const uint32_t o = (uint32_t)kk * 1024 + (uint32_t)ll * 16;
      const uint32_t r = o / HRB, c = (o % HRB) / 16;
      const uint32_t voff = c < (uint32_t)(N / 4) ? r * (N * 4) + c * 16 : 0x7ffffff0u;
      if (coherent) bdma16<true>(rh, voff, 0, sH + kk * 1024);
      else bdma16<false>(rh, voff, 0, sH + kk * 1024);
    }
  };
  auto h_rsrc = [&](const float* src) { return urs(src, (uint32_t)(P * N * 4)); };
  auto issue_x = [&](int b, int k, int h, int nvalid) {
    const LoadLane L = load_lane();
    const __amdgpu_buffer_rsrc_t rx = x_rsrc(b, k, h, nvalid);
#pragma unroll
    for (int i = 0; i < Cf::LX; ++i) issue_x_one(L, rx, i);
    issue_gd(b, k, h);
  };
  auto issue_B = [&](const bf16* bt, int nvalid) {
    const LoadLane L = load_lane();
    const __amdgpu_buffer_rsrc_t rb = b_rsrc(bt, nvalid);
#pragma unroll
    for (int i = 0; i < Cf::LB; ++i) issue_B_one(L, rb, i);
  };
  auto issue_h = [&](const float* src, bool coherent) {
    const __amdgpu_buffer_rsrc_t rh = h_rsrc(src);
#pragma unroll
    for (int i = 0; i < Cf::LH; ++i) issue_h_one(rh, coherent, i);
  };

  float cbc[9][16];   // resident C.B^T blocks of the ticket's (b, k, group), in AGPRs
  Frag cf[2][KS];     // C fragments of the wave's t-blocks, in AGPRs

  const int64_t per = ntickets / nc;                          // tickets per chunk = batch * NHB
  if (tid == 0) sTicket = __hip_atomic_fetch_add(reinterpret_cast<long long*>(sync), 1LL, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
  lds_barrier();
  // wave-uniform: the addresses derived from it are scalar operands
  int64_t ticket = uniform64(sTicket);
  bool prefetched = false;   // the ticket's B tile and first x tile were issued during the previous ticket
  int flag_raw = 0;          // the next head's progress flag, polled during the previous head

  for (;;) {
    if (ticket >= ntickets) break;
    const int k = (int)(ticket / per);
    const int u = (int)(ticket % per);
    const int b = u / NHB;
    const int hb = u % NHB;
    const int h0 = hb * HB;
    const int grp = h0 / (H / G);
    const int64_t t0 = (int64_t)k * Q;
    const int nvalid = (int)(Tlen - t0 < Q ? Tlen - t0 : Q);
    const bf16* bt = Bm + (((int64_t)b * Tlen + t0) * G + grp) * N;
    const bf16* ct = Cm + (((int64_t)b * Tlen + t0) * G + grp) * N;
    int64_t next_ticket = ntickets;

    // ---- ticket set-up: B tile, the first head's x, C fragments, C.B^T
    if (!prefetched) {
      issue_B(bt, nvalid);
      issue_x(b, k, h0, nvalid);
    }
    {
      int lt = lane;
      asm volatile("" : "+v"(lt));
      const int m = lt & 31, g = lt >> 5;
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int tr = (uu ? tb1 : tb0) * 32 + m;
        const bool valid = tr < nvalid;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          u32x4 c4 = __builtin_bit_cast(u32x4, I::load_row(ct + (int64_t)tr * G * N + s * 16 + 8 * g, valid));
          asm("" : "=a"(c4) : "0"(c4));
          cf[uu][s] = __builtin_bit_cast(Frag, c4);
        }
      }
    }
    vm_lds_barrier();
    {
      int lt = lane;
      asm volatile("" : "+v"(lt));
      const int m = lt & 31, g = lt >> 5;
      const uint32_t sw = bswz<N>((uint32_t)m);   // the row swizzle of rows 32 jb + m
#pragma unroll
      for (int e = 0; e < 12; ++e) {
        const int sl = e < 4 ? e : e - 3;
        const int uu = e < 4 ? 0 : 1;
        if (e >= 4 && e < 7 && sl <= wave) continue;
        if (e >= 1 && e < 4 && sl > wave) continue;
        const int jb = uu ? 8 - sl : sl;
        const unsigned char* brow = sB + (jb * 32 + m) * BRB;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s)
          I::mma(acc, *reinterpret_cast<const Frag*>(brow + (((uint32_t)(2 * s + g)) ^ sw) * 16), cf[uu][s]);
#pragma unroll
        for (int r = 0; r < 16; ++r) cbc[sl][r] = to_agpr(acc[r]);
      }
    }

    for (int j = 0; j < HB; ++j) {
      const int h = h0 + j;
      const int64_t bh = (int64_t)b * H + h;
      int lt = lane;
      asm volatile("" : "+v"(lt));
      const int m = lt & 31, g = lt >> 5;
      // this head's x has landed (and the previous head's flag poll); the 8 y
      // stores of the previous head may still be in flight
      asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (j == HB - 1 && tid == 0)
        sTicket = __hip_atomic_fetch_add(reinterpret_cast<long long*>(sync), 1LL, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      {
        const float gi = sG[tid];
        sW[tid] = sDt[tid] * exp2_hw(sG[tid | 31] - gi);
        sWs[tid] = sDt[tid] * exp2_hw(sG[Q - 1] - gi);
        sE[tid] = exp2_hw(gi);
      }
      const float gt0 = sG[tb0 * 32 + m], gt1 = sG[tb1 * 32 + m];
      const float glast = sG[Q - 1];
      const float Dh = Dp[h];
      // h_k: from the initial state (or zeros) at chunk 0, else from the
      // previous chunk's tile once its flag is up (polled during the
      // previous head; a poll that missed is repeated at the chain step)
      bool h_issue = k == 0 ? init != nullptr : __builtin_amdgcn_readfirstlane(flag_raw) >= (int)k;
      if (k == 0 && !init)
        for (int o = tid * 16; o < Cf::HBYTES; o += 256 * 16) *reinterpret_cast<u32x4*>(sH + o) = u32x4{0u, 0u, 0u, 0u};
      const float* hsrc = k == 0 ? init + bh * (int64_t)(P * N) : chain + bh * (int64_t)(P * N);
      const __amdgpu_buffer_rsrc_t rh = h_rsrc(hsrc);
      lds_barrier();
      if (j == HB - 1) next_ticket = uniform64(sTicket);   // claimed above, visible after the barrier

      // transposing x reads: lane s supplies row 4 (s / 32) + (s % 16) / 4 of
      // a 16-row step, headdim columns 16 ((s / 16) % 2) + 4 (s % 4) + 32 pe
      // (the 64-byte half flipped in rows with bit 1 set); xtr ^ 64 is pe = 1
      const uint32_t xtr = (uint32_t)(4 * g + ((lt & 15) >> 2)) * 128 +
                           (((uint32_t)(32 * ((lt >> 4) & 1) + 8 * (lt & 3))) ^ (uint32_t)(64 * ((lt & 15) >> 3)));
      // x^T fragment of headdim block pe over tokens 16 s + drow(e, g)
      auto load_xs = [&](int pe, int s) -> Frag {
        uint64_t h2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const unsigned char* a = sX + (pe ? (xtr ^ 64u) : xtr) + (16 * s + 8 * hh) * 128;
          h2[hh] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                    (__attribute__((address_space(3))) s16x4*)(a)));
        }
        const u32x4 w4 = {(uint32_t)h2[0], (uint32_t)(h2[0] >> 32), (uint32_t)h2[1], (uint32_t)(h2[1] >> 32)};
        return __builtin_bit_cast(Frag, w4);
      };

      // ---- phase A: S_k^T[n][p] = sum_t B[t][n] (w_t x[t][p]); rows n of
      // dstate blocks NBW (w >> 1) + i, columns p of headdim block w & 1.
      // Each step's fragments are read while the previous step computes;
      // h_k's direct loads (when issued here) go one per step among the MFMAs.
      const int pe_a = wave & 1, nb0 = NBW * (wave >> 1);
      f32x16 sacc[NBW];
#pragma unroll
      for (int i = 0; i < NBW; ++i) sacc[i] = f32x16{};
      {
        // B^T fragment reads: lane supplies row 16 s + 8 hh + 4 g + (l % 16) / 4,
        // the 8 bytes of dstate columns 32 nb + 16 ((l / 16) % 2) + 4 (l % 4) ..
        // (row 16 s + t_r has the swizzle of row t_r: bswz has period 16 or 8)
        const uint32_t a_ = (uint32_t)((lt & 15) >> 2);
        const uint32_t piece0 = (uint32_t)(2 * ((lt >> 4) & 1) + ((lt & 3) >> 1));
        const uint32_t half = (uint32_t)(lt & 1) * 8;
        uint32_t btoff[2][NBW];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < NBW; ++i) {
            const uint32_t tr = (uint32_t)(8 * hh + 4 * g) + a_;
            btoff[hh][i] = tr * BRB + (((uint32_t)(4 * (nb0 + i)) + piece0) ^ bswz<N>(tr)) * 16 + half;
          }
        auto load_bt = [&](int i, int s) -> Frag {
          uint64_t h2[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const unsigned char* adr = sB + btoff[hh][i] + 16 * s * BRB;
            h2[hh] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                      (__attribute__((address_space(3))) s16x4*)(adr)));
          }
          const u32x4 w4 = {(uint32_t)h2[0], (uint32_t)(h2[0] >> 32), (uint32_t)h2[1], (uint32_t)(h2[1] >> 32)};
          return __builtin_bit_cast(Frag, w4);
        };
        // software pipeline over the 16 steps: at step s the fragments of step
        // s + 2 are read, the (hi, lo) split of step s + 1 is formed, and the
        // MFMAs of step s run (their split was formed one step earlier)
        Frag xf[3], bfr[3][NBW];
        float4 wq[3][2];
        Frag shi[2], slo[2];
        auto ldA = [&](int s, int sl) {
          xf[sl] = load_xs(pe_a, s);
#pragma unroll
          for (int i = 0; i < NBW; ++i) bfr[sl][i] = load_bt(i, s);
          wq[sl][0] = *reinterpret_cast<const float4*>(&sWs[16 * s + 4 * g]);
          wq[sl][1] = *reinterpret_cast<const float4*>(&sWs[16 * s + 8 + 4 * g]);
        };
        // w o x of one step as a bf16 (hi, lo) pair; each hi value is taken as
        // a bit slice of the packed pair
        auto splitA = [&](int sl, Frag& hi, Frag& lo) {
          const float wv[8] = {wq[sl][0].x, wq[sl][0].y, wq[sl][0].z, wq[sl][0].w,
                               wq[sl][1].x, wq[sl][1].y, wq[sl][1].z, wq[sl][1].w};
          const u32x4 xd = __builtin_bit_cast(u32x4, xf[sl]);
          u32x4 uh, ul;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v0 = wv[2 * i] * bf16lo(xd[i]), v1 = wv[2 * i + 1] * bf16hi(xd[i]);
            uint32_t hh = pack_bf16x2(v0, v1);
            asm volatile("" : "+v"(hh));
            uh[i] = hh;
            ul[i] = pack_bf16x2(v0 - __uint_as_float(hh << 16), v1 - __uint_as_float(hh & 0xffff0000u));
          }
          hi = __builtin_bit_cast(Frag, uh);
          lo = __builtin_bit_cast(Frag, ul);
        };
        ldA(0, 0);
        ldA(1, 1);
        splitA(0, shi[0], slo[0]);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          if (s + 2 < 16) ldA(s + 2, (s + 2) % 3);
          if (h_issue && s < Cf::LH) issue_h_one(rh, k > 0, s);
#pragma unroll
          for (int i = 0; i < NBW; ++i) I::mma(sacc[i], bfr[s % 3][i], shi[s & 1]);
#pragma unroll
          for (int i = 0; i < NBW; ++i) I::mma(sacc[i], bfr[s % 3][i], slo[s & 1]);
          if (s + 1 < 16) splitA((s + 1) % 3, shi[(s + 1) & 1], slo[(s + 1) & 1]);
          // interleave this step's MFMAs with the next step's split
#pragma unroll
          for (int q = 0; q < 2 * NBW; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 40 / (2 * NBW), 0);   // then VALU
          }
        }
      }

      // ---- chain: h_k in sH, h_{k+1} out, h_k rewritten as (hi, lo) pairs
      if (!h_issue && k > 0) {
        wait_flag(sync + kSyncFlags + bh, (int)k, sync);
        issue_h(hsrc, true);
      }
      vm_lds_barrier();
      // h_{k+1} (this wave's part), stored among the pairs below
      u32x4 hn[NBW][4];
      {
        const float alpha = exp2_hw(glast);
        const int p = 32 * pe_a + m;
        float4 hk[NBW][4];
#pragma unroll
        for (int i = 0; i < NBW; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            hk[i][q] = *reinterpret_cast<const float4*>(sH + p * HRB + 4 * (32 * (nb0 + i) + 8 * q + 4 * g));
#pragma unroll
        for (int i = 0; i < NBW; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 a = hk[i][q];
            hn[i][q] = u32x4{__float_as_uint(fmaf(alpha, a.x, sacc[i][4 * q])),
                             __float_as_uint(fmaf(alpha, a.y, sacc[i][4 * q + 1])),
                             __float_as_uint(fmaf(alpha, a.z, sacc[i][4 * q + 2])),
                             __float_as_uint(fmaf(alpha, a.w, sacc[i][4 * q + 3]))};
          }
        // h_k as (hi, lo) bf16 pairs, in place: group n / 8 of row p holds 8
        // hi values then 8 lo values (the same 32 bytes its fp32 values took)
#pragma unroll
        for (int i = 0; i < NBW; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 a = hk[i][q];
            const uint32_t h01 = pack_bf16x2(a.x, a.y), h23 = pack_bf16x2(a.z, a.w);
            const uint32_t l01 = pack_bf16x2(a.x - bf16lo(h01), a.y - bf16hi(h01));
            const uint32_t l23 = pack_bf16x2(a.z - bf16lo(h23), a.w - bf16hi(h23));
            unsigned char* grp8 = sH + p * HRB + (4 * (nb0 + i) + q) * 32 + 8 * g;
            *reinterpret_cast<uint2*>(grp8) = make_uint2(h01, h23);
            *reinterpret_cast<uint2*>(grp8 + 16) = make_uint2(l01, l23);
          }
      }
      lds_barrier();

      // the next head: the next of this ticket, or the first of the next ticket
      bool has_next = true, new_ticket = false;
      int nk = k, nb = b;
      int nh = h + 1, nvn = nvalid;
      const bf16* nbt = bt;
      if (j + 1 == HB) {
        new_ticket = true;
        has_next = next_ticket < ntickets;
        if (has_next) {
          nk = (int)(next_ticket / per);
          const int nu = (int)(next_ticket % per);
          nb = nu / NHB;
          nh = (nu % NHB) * HB;
          const int64_t nt0 = (int64_t)nk * Q;
          nvn = (int)(Tlen - nt0 < Q ? Tlen - nt0 : Q);
          nbt = Bm + (((int64_t)nb * Tlen + nt0) * G + nh / (H / G)) * N;
        }
      }

      // after pair number idx (0..8) of the pairs below: this wave's stores of
      // h_{k+1} (spread over the first five pairs, so the write path drains
      // between them) and, before a new ticket, its loads of that ticket's B
      // tile (B of this ticket is no longer read)
      const bool last_chunk = k + 1 == nc;
      float* hdst = last_chunk ? final_state : chain;
      auto pair_hook = [&](int idx) {
        constexpr int NS = NBW * 4;
        if (hdst) {
          const __amdgpu_buffer_rsrc_t rs = urs(hdst + bh * (int64_t)(P * N), (uint32_t)(P * N * 4));
          int ll = lane;
          asm volatile("" : "+v"(ll));
          const int p = 32 * pe_a + (ll & 31), gg = ll >> 5;
#pragma unroll
          for (int si = 0; si < NS; ++si) {
            if (si < idx * NS / 5 || si >= (idx + 1) * NS / 5) continue;
            const int i = si / 4, q = si % 4;
            const uint32_t off = (uint32_t)(p * N + 32 * (nb0 + i) + 8 * q + 4 * gg) * 4;
            if (last_chunk) __builtin_amdgcn_raw_buffer_store_b128(hn[i][q], rs, off, 0, 0);
            else __builtin_amdgcn_raw_buffer_store_b128(hn[i][q], rs, off, 0, 16);   // sc1
          }
        }
        if (has_next && new_ticket) {
          const LoadLane LB_ = load_lane();
          const __amdgpu_buffer_rsrc_t rbn = b_rsrc(nbt, nvn);
#pragma unroll
          for (int q = 0; q < Cf::LB; ++q)
            if (q >= idx * Cf::LB / 9 && q < (idx + 1) * Cf::LB / 9) issue_B_one(LB_, rbn, q);
        }
      };

      f32x16 acc[2][2];
#pragma unroll
      for (int uu = 0; uu < 2; ++uu)
#pragma unroll
        for (int pe = 0; pe < 2; ++pe) acc[uu][pe] = f32x16{};

      // ---- intra-chunk pairs, slot by slot, specialised per wave
      auto pairs = [&](auto wtag) {
        constexpr int W = decltype(wtag)::value;
        auto load_x = [&](int jb, Frag (*d)[2]) {
#pragma unroll
          for (int pe = 0; pe < 2; ++pe)
#pragma unroll
            for (int js = 0; js < 2; ++js) d[pe][js] = load_xs(pe, 2 * jb + js);
        };
        auto load_w = [&](int jb, float4* wv, float& ge) {
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) wv[c4] = *reinterpret_cast<const float4*>(&sW[jb * 32 + 8 * c4 + 4 * g]);
          ge = sG[jb * 32 + 31];
        };
        Frag d[2][2];
        float4 wv[4];
        float ge = 0.f;
        load_x(0, d);
        if (!pair_diag(0, W)) load_w(0, wv, ge);
#pragma unroll
        for (int e = 0; e < 12; ++e) {
          const int sl = e < 4 ? e : e - 3;
          const int uu = e < 4 ? 0 : 1;
          if (!pair_kept(e, W)) continue;
          const int jb = uu ? 8 - sl : sl;
          const int tbk = uu ? 7 - W : W;
          const bool diag = jb == tbk;
          const float gtu = uu ? gt1 : gt0;
          const int j0 = jb * 32;
          Frag dn[2][2];
          float4 wvn[4];
          float gen = 0.f;
          const int en = next_pair(e, W);
          if (en >= 0) load_x(pair_jb(en), dn);
          if (en >= 0 && !pair_diag(en, W)) load_w(pair_jb(en), wvn, gen);
          float v[16];
          if (!diag) {
            const float a = exp2_hw(gtu - ge);
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
              v[4 * c4 + 0] = from_agpr(cbc[sl][4 * c4 + 0]) * (wv[c4].x * a);
              v[4 * c4 + 1] = from_agpr(cbc[sl][4 * c4 + 1]) * (wv[c4].y * a);
              v[4 * c4 + 2] = from_agpr(cbc[sl][4 * c4 + 2]) * (wv[c4].z * a);
              v[4 * c4 + 3] = from_agpr(cbc[sl][4 * c4 + 3]) * (wv[c4].w * a);
            }
          } else {
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
              const float4 g4 = *reinterpret_cast<const float4*>(&sG[j0 + 8 * c4 + 4 * g]);
              const float4 d4 = *reinterpret_cast<const float4*>(&sDt[j0 + 8 * c4 + 4 * g]);
              const float gq[4] = {g4.x, g4.y, g4.z, g4.w}, dq[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int q = 4 * c4 + i, jr = drow(q, g);
                const float val = from_agpr(cbc[sl][q]) * exp2_hw(gtu - gq[i]) * dq[i];
                v[q] = (m > jr) ? val : ((m == jr) ? val + Dh : 0.f);
              }
            }
          }
#pragma unroll
          for (int js = 0; js < 2; ++js) {
            u32x4 uh, ul;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              uint32_t hh = pack_bf16x2(v[js * 8 + 2 * i], v[js * 8 + 2 * i + 1]);
              asm volatile("" : "+v"(hh));
              uh[i] = hh;
              ul[i] = pack_bf16x2(v[js * 8 + 2 * i] - __uint_as_float(hh << 16),
                                  v[js * 8 + 2 * i + 1] - __uint_as_float(hh & 0xffff0000u));
            }
            const Frag ahi = __builtin_bit_cast(Frag, uh), alo = __builtin_bit_cast(Frag, ul);
#pragma unroll
            for (int pe = 0; pe < 2; ++pe) {
              I::mma(acc[uu][pe], d[pe][js], ahi);
              I::mma(acc[uu][pe], d[pe][js], alo);
            }
          }
          pair_hook(kept_index(e, W));
#pragma unroll
          for (int pe = 0; pe < 2; ++pe)
#pragma unroll
            for (int js = 0; js < 2; ++js) d[pe][js] = dn[pe][js];
          if (en >= 0 && !pair_diag(en, W)) {
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) wv[c4] = wvn[c4];
            ge = gen;
          }
        }
      };
      switch (wave) {
        case 0: pairs(std::integral_constant<int, 0>{}); break;
        case 1: pairs(std::integral_constant<int, 1>{}); break;
        case 2: pairs(std::integral_constant<int, 2>{}); break;
        default: pairs(std::integral_constant<int, 3>{}); break;
      }
      __builtin_amdgcn_sched_barrier(0);

      // h_{k+1} is stored (each wave waits for its stores, issued among the
      // first pairs), and every wave is done with x: raise the flag; the next
      // head's x may load
      vm_lds_barrier();
      if (tid == 0) __hip_atomic_store(sync + kSyncFlags + bh, (int)(k + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

      // ---- carried state: tmp[u][pe] = h_k . C^T (rows p, columns t), then
      // acc += 2^(G'_t) tmp. The next head's x, G' and dt (and for a new
      // ticket its B tile) are issued among these MFMAs.
      {
        constexpr int HBK = KS / 4, NBLK = 2 * HBK;
        constexpr int NPF = Cf::LX + 1;               // x rows, G'/dt row
        const LoadLane LL = load_lane();
        const __amdgpu_buffer_rsrc_t rxn = x_rsrc(nb, nk, nh, nvn);
        auto prefetch = [&](int q0, int q1) {
          if (!has_next) return;
#pragma unroll
          for (int q = 0; q < NPF; ++q) {
            if (q < q0 || q >= q1) continue;
            if (q < Cf::LX) issue_x_one(LL, rxn, q);
            else issue_gd(nb, nk, nh);
          }
        };
        f32x16 tmp[2][2];
#pragma unroll
        for (int uu = 0; uu < 2; ++uu)
#pragma unroll
          for (int pe = 0; pe < 2; ++pe) tmp[uu][pe] = f32x16{};
        Frag hf[2][2][4];
        auto load_h = [&](int blk, Frag (*dst)[4]) {
          const int pe = blk / HBK, s0 = (blk % HBK) * 4;
          const unsigned char* hp = sH + (pe * 32 + m) * HRB;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dst[0][i] = *reinterpret_cast<const Frag*>(hp + (2 * (s0 + i) + g) * 32);
            dst[1][i] = *reinterpret_cast<const Frag*>(hp + (2 * (s0 + i) + g) * 32 + 16);
          }
        };
        load_h(0, hf[0]);
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) {
          if (blk + 1 < NBLK) load_h(blk + 1, hf[(blk + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          const int pe = blk / HBK, s0 = (blk % HBK) * 4;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) {
              I::mma(tmp[uu][pe], hf[blk & 1][0][i], cf[uu][s0 + i]);
              I::mma(tmp[uu][pe], hf[blk & 1][1][i], cf[uu][s0 + i]);
            }
          prefetch(blk * NPF / NBLK, (blk + 1) * NPF / NBLK);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
          const float sc = sE[(uu ? tb1 : tb0) * 32 + m];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc[uu][0][r] = fmaf(sc, tmp[uu][0][r], acc[uu][0][r]);
            acc[uu][1][r] = fmaf(sc, tmp[uu][1][r], acc[uu][1][r]);
          }
        }
      }
      // the next head's flag, read at its start (after the y stores below)
      if (has_next && nk > 0)
        flag_raw = __hip_atomic_load(sync + kSyncFlags + (int64_t)nb * H + nh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

      // ---- y through LDS in 16-byte row pieces (as the resident scan)
      {
        unsigned char* ys_lds = sY + wave * 4096;
        const uint32_t wrow = (uint32_t)m * 128 + 8 * (uint32_t)g, wsw = (uint32_t)(m >> 1) & 7;
        const int pr = lane / 8, pc = lane % 8;
        uint32_t plane = (uint32_t)pr * xrb + (uint32_t)pc * 16;
        uint32_t xrbs = xrb;
        asm volatile("" : "+v"(plane), "+s"(xrbs));
        unsigned char* yt = reinterpret_cast<unsigned char*>(y + (((int64_t)b * Tlen + t0) * H + h) * P);
        const __amdgpu_buffer_rsrc_t yr = urs(yt, (uint32_t)nvalid * xrbs);
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
#pragma unroll
          for (int pe = 0; pe < 2; ++pe)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const uint2 v2 = make_uint2(pack_bf16x2(acc[uu][pe][4 * c], acc[uu][pe][4 * c + 1]),
                                          pack_bf16x2(acc[uu][pe][4 * c + 2], acc[uu][pe][4 * c + 3]));
              *reinterpret_cast<uint2*>(ys_lds + wrow + (((uint32_t)(4 * pe + c)) ^ wsw) * 16) = v2;
            }
          const uint32_t row0 = (uint32_t)((uu ? tb1 : tb0) * 32);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t rsw = (uint32_t)(4 * (i & 1) + (pr >> 1));
            const u32x4 v = *reinterpret_cast<const u32x4*>(ys_lds + (8 * i + pr) * 128 + ((uint32_t)pc ^ rsw) * 16);
            __builtin_amdgcn_raw_buffer_store_b128(v, yr, plane + (row0 + 8 * i) * xrbs, 0, 0);
          }
        }
      }
    }
    ticket = next_ticket;
    prefetched = true;
  }
}

int chained_heads_per_ticket(const Problem& p, int cus) {
  const int64_t hpg = p.H / p.G;
  for (int hb : {4, 2, 1})
    if (hpg % hb == 0 && (hb == 1 || p.bt * p.nc * (p.H / hb) >= 3 * (int64_t)cus)) return hb;
  return 1;
}

template <int N>
int chained_grid() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    dev = 0;
  }
  if (!cached[dev]) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ssd_chunk_chained<N>, 256, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0) {
      (void)hipGetLastError();
      cus = 256;
      per_cu = 1;
    }
    cached[dev] = cus * per_cu;
  }
  return cached[dev];
}

template <int N>
hipError_t launch_chained(const Problem& p, hipStream_t stream) {
  const int slots = chained_grid<N>();
  const int HB = chained_heads_per_ticket(p, slots);
  const int64_t ntickets = p.bt * p.nc * (p.H / HB);
  const int64_t grid = ntickets < slots ? ntickets : slots;
  hipLaunchKernelGGL((ssd_chunk_chained<N>), dim3((unsigned)grid), dim3(256), 0, stream, (const bf16*)p.x,
                     (const bf16*)p.B, (const bf16*)p.C, p.gcum, p.dtt, p.D, p.init, (bf16*)p.y, p.final_state,
                     p.chain, p.sync, p.T, (int)p.H, (int)p.G, p.nc, p.Tp, HB, ntickets);
  return hipGetLastError();
}

}  // namespace

bool chunk_chained_fits(const Problem& p) {
  return p.io == 1 && p.P == 64 && p.Q == 256 && (p.N == 64 || p.N == 128) && p.nc > 0;
}

hipError_t launch_chunk_chained(const Problem& p, hipStream_t stream) {
  if (p.bt == 0 || p.nc == 0) return hipSuccess;
  return p.N == 64 ? launch_chained<64>(p, stream) : launch_chained<128>(p, stream);
}

}  // namespace ssd

// ssd_chunk_scan, C.B^T-resident form (bf16 io, headdim 64, chunk 256,
// dstate 64 or 128): the same outputs as chunk_scan.hip,
//
//   y[t, p] = 2^(G'_t) sum_n C[t, n] Hprev[p, n]
//           + sum_{j <= t} (C_t . B_j) 2^(G'_t - G'_j) dt_j x[j, p] + D x[t, p]
//
// (CUDA Tile Mamba-2 blog, section "Mamba-2 architecture", the decayed block
// output; section "Kernel 3: compute_out").
//
// What changes. C_t . B_j depends on (batch, chunk, group) only, not on the
// head; every head of a group reuses the same causal Q x Q block. A
// persistent workgroup walks consecutive heads of one chunk, so it computes
// the chunk's C.B^T once, keeps it in registers (each wave holds its 9
// causal 32x32 blocks, 144 fp32 per lane), and per head only applies the
// head's decay and dt, splits, and multiplies with x. That removes the per
// head C.B^T products (a third of the MFMAs of the per-head form).
//
// Per head ("tile"), the operands that change are x (32 KB), the carried
// state Hprev (32 KB of bf16 hi/lo pairs) and the head's G', dt rows (2 KB).
// They are brought into one of two LDS buffers by direct global->LDS loads
// while the previous tile computes; a tile needs two workgroup barriers, not
// one per 32-token block.
//
// Waves. 4 waves; wave w owns the 32-row t-blocks w and 7 - w, i.e. the
// causal (t-block, j-block) pairs (w, 0..w) and (7 - w, 0..7 - w): 9 pairs
// for every wave. Pair blocks sit in 9 register slots: slot k holds (w, k)
// for k <= w and (7 - w, 8 - k) for k > w. Slots 0 and 4..8 therefore
// belong to one t-block whatever the wave; slots 1..3 are emitted once per
// t-block behind a wave-uniform branch, so the accumulator each product
// feeds is always known at compile time.
//
// Products are formed transposed, y^T = x^T M^T and y_state^T = Hprev C^T:
// the accumulators hold headdim rows p and token columns t, so x enters as
// the MFMA's first operand (rows p, contraction over j). gfx950's transposing
// LDS read (ds_read_b64_tr_b16) gathers such a fragment straight from the
// row-major x tile: within 16 lanes, lane i supplies the address of row
// i / 4 at columns 4 (i % 4) .. + 3, and lane 4a + b receives column b of
// the rows supplied by lanes a, a + 4, a + 8, a + 12. No byte shuffles are
// needed to split column pairs.
//
// LDS layouts (all reads conflict-free):
//  - x tile: 256 rows of 128 bytes, unpadded; in rows whose index has bit 1
//    set the two 64-byte halves are swapped, so the four rows of a
//    half-wave's transposing read (64 bytes each) fill the four 64-byte
//    quarters of the 256-byte bank space. A wave-instruction of the direct
//    load fills 8 whole rows, so its per-lane source offset is one constant
//    and the row block is a scalar.
//  - Hprev: slot rows of N*4 bytes plus one 16-byte pad piece, slot p
//    holding headdim row p (fragment reads of 16 consecutive lanes hit 16
//    distinct bank groups).
//  - B tile (C.B^T phase only, in the other buffer): rows padded by one
//    16-byte piece.
#include "ssd_device.h"
#include "ssd_launch.h"

#include <type_traits>

namespace ssd {

namespace {

template <int N>
struct RCfg {
  static constexpr int P = 64, Q = 256, NTB = 8, WAVES = 4, THREADS = 256;
  static constexpr int KS = N / 16;            // bf16 MFMA k-steps over dstate
  static constexpr int NPAIR = NTB + 1;        // causal block pairs per wave
  static constexpr int XRB = P * 2;            // x row bytes in LDS (unpadded)
  static constexpr int XBYTES = Q * XRB;       // 32 KB
  static constexpr int HROWP = N / 4 + 1;      // Hprev pieces per padded slot row
  static constexpr int HRB = HROWP * 16;
  static constexpr int HBYTES = (P * HROWP * 16 + 1023) / 1024 * 1024;
  static constexpr int GBYTES = 2 * Q * 4;     // G' row, then dt row
  static constexpr int HOFF = XBYTES, GOFF = XBYTES + HBYTES;
  static constexpr int IX = XBYTES / 1024;     // wave-instructions of one tile's loads
  static constexpr int IH = HBYTES / 1024;
  static constexpr int IG = GBYTES / 1024;
  static constexpr int LX = IX / WAVES;        // per wave
  static constexpr int LR = (IH + IG + WAVES - 1) / WAVES;
  static constexpr int LT = LX + LR;           // tile loads per wave
  static constexpr int RB = N * 2 / 16;        // pieces per B row
  static constexpr int BROWP = RB + 1;
  static constexpr int BRB = BROWP * 16;
  static constexpr int BBYTES = (Q * BRB + 1023) / 1024 * 1024;
  static constexpr int IB = BBYTES / 1024;
  static constexpr int LB = (IB + WAVES - 1) / WAVES;
  // one tile buffer; the C.B^T phase puts the B tile in one as well
  static constexpr int BUF = GOFF + GBYTES > BBYTES ? GOFF + GBYTES : BBYTES;
  static_assert(IX % WAVES == 0, "x loads split evenly");
  static_assert(2 * BUF + 2 * Q * 4 + 4 * 4096 <= 160 * 1024, "LDS");
  static_assert(LT <= 40 && LB + LT + 2 * KS <= 63, "vmcnt accounting");
};

// Direct global->LDS load, 16 bytes per lane, from a wave-uniform base plus a
// per-lane 32-bit offset (the scalar-base form of the instruction). Lane i's
// bytes land at lds + 16 i; lds must be wave-uniform (it goes in M0).
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// Values pinned in the accumulation registers (AGPRs): the resident C.B^T
// blocks live there between tiles, leaving the VGPRs to the per-pair
// working set; they are read back one 32x32 block at a time.
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

template <int VM>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One (batch, chunk, head) tile's addresses; all wave-uniform.
struct RTile {
  int64_t b, k, bk;
  int h, nvalid;
  int64_t ckey;
  const unsigned char* x;      // first x row of the tile
  unsigned char* y;
  const bf16* bt;              // first B row
  const bf16* ct;              // first C row
  const unsigned char* gc;     // G' row (Q floats)
  const unsigned char* dtc;    // dt row
  const unsigned char* hs;     // Hprev block (P rows of 4N bytes)
  float Dh;
};

template <int N>
__device__ __forceinline__ RTile make_rtile(int64_t b, int64_t k, int64_t bk, int h, const bf16* x, const bf16* Bm,
                                            const bf16* Cm, const float* gcum, const float* dtt, const float* Dp,
                                            const void* hprev, bf16* y, int64_t Tlen, int H, int G, int64_t nc,
                                            int64_t Tp) {
  constexpr int P = 64, Q = 256;
  RTile t;
  const int grp = h / (H / G);
  const int64_t t0 = k * Q;
  t.b = b;
  t.k = k;
  t.bk = bk;
  t.h = h;
  t.nvalid = (int)(Tlen - t0 < Q ? Tlen - t0 : Q);
  t.ckey = bk * G + grp;
  t.x = reinterpret_cast<const unsigned char*>(x + ((b * Tlen + t0) * H + h) * P);
  t.y = reinterpret_cast<unsigned char*>(y + ((b * Tlen + t0) * H + h) * P);
  t.bt = Bm + ((b * Tlen + t0) * G + grp) * N;
  t.ct = Cm + ((b * Tlen + t0) * G + grp) * N;
  t.gc = reinterpret_cast<const unsigned char*>(gcum + (b * H + h) * Tp + t0);
  t.dtc = reinterpret_cast<const unsigned char*>(dtt + (b * H + h) * Tp + t0);
  t.hs = static_cast<const unsigned char*>(hprev) + ((b * H + h) * nc + k) * (int64_t)(P * N) * 4;
  t.Dh = Dp[h];
  return t;
}

// The intra-chunk pairs of wave W, in emission order e = 0..11 (slot sl,
// t-block choice u): which emissions the wave keeps, the j-block of an
// emission, and the wave's next kept emission after e (-1: none).
__host__ __device__ constexpr bool pair_kept(int e, int W) {
  return !((e >= 4 && e < 7 && e - 3 <= W) || (e >= 1 && e < 4 && e > W));
}
__host__ __device__ constexpr int pair_jb(int e) { return e < 4 ? e : 8 - (e - 3); }
__host__ __device__ constexpr bool pair_diag(int e, int W) { return pair_jb(e) == (e < 4 ? W : 7 - W); }
__host__ __device__ constexpr int next_pair(int e, int W) {
  for (int f = e + 1; f < 12; ++f)
    if (pair_kept(f, W)) return f;
  return -1;
}
static_assert(pair_kept(0, 0) && pair_kept(0, 3) && pair_jb(0) == 0, "every wave starts at j-block 0");

template <int N>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ssd_chunk_scan_resident(const bf16* __restrict__ x, const bf16* __restrict__ Bm, const bf16* __restrict__ Cm,
                             const float* __restrict__ gcum, const float* __restrict__ dtt,
                             const float* __restrict__ Dp, const void* __restrict__ hprev, bf16* __restrict__ y,
                             int64_t Tlen, int H, int G, int64_t nc, int64_t Tp, int64_t ntiles, int xcd) {
  using Cf = RCfg<N>;
  using I = Io<bf16>;
  using Frag = bf16x8;
  constexpr int P = 64, Q = 256, KS = Cf::KS, LX = Cf::LX, LR = Cf::LR, LB = Cf::LB;
  constexpr int IH = Cf::IH, IG = Cf::IG;

  __shared__ __attribute__((aligned(1024))) unsigned char lds[2][Cf::BUF];
  __shared__ __attribute__((aligned(16))) float sW[Q];   // dt_j * 2^(G'_end(block of j) - G'_j) <= dt_j
  __shared__ __attribute__((aligned(16))) float sE[Q];   // 2^(G'_t) <= 1
  __shared__ __attribute__((aligned(16))) unsigned char ystage[4 * 4096];   // per wave: one 32 x 64 bf16 y block

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  __builtin_assume(wave >= 0 && wave < 4);
  const int lane = tid % 64;
  const int tb0 = wave, tb1 = 7 - wave;

  // this workgroup's contiguous range of tiles, heads fastest; with xcd set,
  // the tiles of XCD group x are the chunks (batch*nchunks index) = x mod 8,
  // walked by the workgroups that the dispatcher deals to XCD x
  int64_t lo, hi;
  {
    const int64_t grid = gridDim.x, w = blockIdx.x;
    if (xcd) {
      const int64_t n8 = ntiles / 8, xg = w % 8, lw = w / 8, per = grid / 8;
      lo = xg * n8 + lw * n8 / per;
      hi = xg * n8 + (lw + 1) * n8 / per;
    } else {
      lo = w * ntiles / grid;
      hi = (w + 1) * ntiles / grid;
    }
  }
  if (lo >= hi) return;   // whole workgroup

  // first tile: walk position lo -> (bk, h) -> (b, k)
  int64_t bk;
  int h;
  if (xcd) {
    const int64_t n8 = ntiles / 8, xg = lo / n8, i = lo % n8;
    bk = xg + 8 * (i / H);
    h = (int)(i % H);
  } else {
    bk = lo / H;
    h = (int)(lo % H);
  }
  const int64_t bkstep = xcd ? 8 : 1;
  int64_t b = bk / nc, k = bk % nc;

  // per-lane load offsets, fixed for the whole walk
  const uint32_t xrb = (uint32_t)H * P * 2;                  // x / y row stride in bytes
  const int jl = lane >> 3;                                   // x row (within 8) this lane loads
  const uint32_t xpiece = (uint32_t)((lane & 7) ^ ((jl & 2) << 1)) * 16;   // its 16 bytes, halves swapped
  const uint32_t xlane = (uint32_t)jl * xrb + xpiece;
  uint32_t roff[LR];    // Hprev (or G', dt) load offsets of the rest list
#pragma unroll
  for (int i = 0; i < LR; ++i) {
    int rho = wave + i * 4;
    if (rho >= IH + IG) rho %= IH + IG;     // spare: repeats a load
    if (rho < IH) {
      const int s = rho * 64 + lane;
      int r = s / Cf::HROWP, c = s % Cf::HROWP;
      if (r >= P) r = P - 1;                // tail of the last instruction
      if (c >= Cf::HROWP - 1) c = 0;        // pad piece
      roff[i] = (uint32_t)(r * N * 4 + c * 16);
    } else {
      roff[i] = (uint32_t)(lane * 16);
    }
  }

  float cbc[9][16];   // resident C.B^T blocks (slots, see above), in AGPRs
  Frag cf[2][KS];     // C fragments of the wave's t-blocks, in AGPRs
  int64_t ckey_cached = -1;
  int ys = 0;     // y stores issued after the current tile's loads: none, or 8
  int buf = 0;

  // Issue the loads of one tile into LDS buffer `dst`.
  // (The per-lane and per-instruction offsets below are derived from values
  // laundered per call, so they are not hoisted out of the walk and kept
  // alive in registers across it.)
  // Loads q0 .. q1 - 1 of the tile's LT: x first, then Hprev, G' and dt.
  auto issue_part = [&](const RTile& t, unsigned char* dst, int q0, int q1) {
    const bool full = t.nvalid == Q;
    uint32_t xl = xlane, xr = xrb, xpc = xpiece;
    int jll = jl;
    asm volatile("" : "+v"(xl), "+v"(jll), "+v"(xpc), "+s"(xr));
#pragma unroll
    for (int i = 0; i < LX; ++i) {
      if (i < q0 || i >= q1) continue;
      const int kk = wave + 4 * i;           // 8 x rows per instruction
      if (full) {
        lds_dma16_s(t.x + (uint32_t)(kk * 8) * xr, xl, dst + kk * 1024);
      } else {
        const int row = min(kk * 8 + jll, t.nvalid - 1);
        lds_dma16_s(t.x, (uint32_t)row * xr + xpc, dst + kk * 1024);
      }
    }
#pragma unroll
    for (int i = 0; i < LR; ++i) {
      if (LX + i < q0 || LX + i >= q1) continue;
      int rho = wave + i * 4;
      if (rho >= IH + IG) rho %= IH + IG;
      if (rho < IH)
        lds_dma16_s(t.hs, roff[i], dst + Cf::HOFF + rho * 1024);
      else
        lds_dma16_s(rho == IH ? t.gc : t.dtc, roff[i], dst + Cf::GOFF + (rho - IH) * 1024);
    }
  };
  auto issue_tile = [&](const RTile& t, unsigned char* dst) { issue_part(t, dst, 0, Cf::LT); };

  for (int64_t pos = lo; pos < hi; ++pos) {
    // lane-derived values are re-derived per tile from a laundered lane id:
    // hoisted out of the walk, they would outgrow the register file
    int lt = lane;
    asm volatile("" : "+v"(lt));
    const int m = lt & 31, g = lt >> 5;
    // transposing x reads: lane s supplies row 4 (s / 32) + (s % 16) / 4 of a
    // 16-row step, headdim columns 16 ((s / 16) % 2) + 4 (s % 4) + 32 pe (the
    // 64-byte half flipped in rows with bit 1 set); xtr ^ 64 is the pe = 1 read
    const uint32_t xtr = (uint32_t)(4 * g + ((lt & 15) >> 2)) * 128 +
                         (((uint32_t)(32 * ((lt >> 4) & 1) + 8 * (lt & 3))) ^ (uint32_t)(64 * ((lt & 15) >> 3)));
    const RTile t = make_rtile<N>(b, k, bk, h, x, Bm, Cm, gcum, dtt, Dp, hprev, y, Tlen, H, G, nc, Tp);
    unsigned char* cur = lds[buf];
    unsigned char* oth = lds[buf ^ 1];

    if (t.ckey != ckey_cached) {
      // C.B^T phase: every earlier load and store of this wave is done and
      // every wave has left the previous tile
      wait_vm_barrier<0>();
      // C rows of the wave's t-blocks as MFMA fragments
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tr = (u ? tb1 : tb0) * 32 + m;
        const bool valid = tr < t.nvalid;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          u32x4 c4 = __builtin_bit_cast(u32x4, I::load_row(t.ct + (int64_t)tr * G * N + s * 16 + 8 * g, valid));
          asm("" : "=a"(c4) : "0"(c4));     // held in AGPRs; the MFMA reads them there
          cf[u][s] = __builtin_bit_cast(Frag, c4);
        }
      }
      // the chunk's B rows into the other buffer (padded rows), rows past
      // the sequence clamped to its last row
      int lanel = lane;   // laundered: these offsets are recomputed per phase, not kept across the walk
      asm volatile("" : "+v"(lanel));
#pragma unroll
      for (int i = 0; i < LB; ++i) {
        int kk = wave + 4 * i;
        if (kk >= Cf::IB) kk %= Cf::IB;
        const int s = kk * 64 + lanel;
        int r = s / Cf::BROWP, c = s % Cf::BROWP;
        if (r >= Q) r = Q - 1;
        if (c >= Cf::RB) c = 0;
        const int row = min(r, t.nvalid - 1);
        lds_dma16_s(t.bt, (uint32_t)((int64_t)row * G * N * 2 + c * 16), oth + kk * 1024);
      }
      issue_tile(t, cur);
      // B and C landed once only this tile's LT loads remain
      wait_vm_barrier<Cf::LT>();
      const unsigned char* bb = oth + m * Cf::BRB + g * 16;
#pragma unroll
      for (int e = 0; e < 12; ++e) {
        // emitted (slot, t-block) combinations: slot 0 (u = 0), slots 1..3
        // for u = 0 and for u = 1, slots 4..8 (u = 1)
        const int sl = e < 4 ? e : (e < 7 ? e - 3 : e - 3);
        const int u = e < 4 ? 0 : 1;
        if (e >= 4 && e < 7 && sl <= wave) continue;   // slot belongs to t-block w
        if (e >= 1 && e < 4 && sl > wave) continue;    // slot belongs to t-block 7 - w
        const int jb = u ? 8 - sl : sl;
        const unsigned char* bj = bb + jb * 32 * Cf::BRB;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) I::mma(acc, *reinterpret_cast<const Frag*>(bj + s * 32), cf[u][s]);
#pragma unroll
        for (int r = 0; r < 16; ++r) cbc[sl][r] = to_agpr(acc[r]);
      }
      lds_barrier();      // the B tile is read; its buffer may be refilled
      ckey_cached = t.ckey;
      ys = 0;
    }

    // this tile's loads have landed once only the previous tile's y stores remain
    if (ys) wait_vm_barrier<8>();
    else wait_vm_barrier<0>();
    const float* sG = reinterpret_cast<const float*>(cur + Cf::GOFF);
    const float* sDt = sG + Q;
    {
      const float gi = sG[tid];
      sW[tid] = sDt[tid] * exp2_hw(sG[tid | 31] - gi);   // exponent <= 0
      sE[tid] = exp2_hw(gi);
    }
    const float gt0 = sG[tb0 * 32 + m], gt1 = sG[tb1 * 32 + m];
    lds_barrier();

    // next tile: advance the walk; prefetch it when it shares this chunk's C.B^T
    const bool has_next = pos + 1 < hi;
    if (has_next) {
      if (++h == H) {
        h = 0;
        bk += bkstep;
        k += bkstep;
        while (k >= nc) {
          k -= nc;
          ++b;
        }
      }
    }
    bool prefetch = false;
    RTile nt = t;
    if (has_next) {
      nt = make_rtile<N>(b, k, bk, h, x, Bm, Cm, gcum, dtt, Dp, hprev, y, Tlen, H, G, nc, Tp);
      prefetch = nt.ckey == ckey_cached;
    }
    // (its loads are issued among the carried-state MFMAs below: a wave that
    // waits to issue a direct load leaves the MFMAs it has issued running)

    // carried state: acc[u][pe] = Hprev . C^T, row p = 32 pe + drow(r, g),
    // column t = 32 tb + m, then columns scaled by 2^(G'_t)
    f32x16 acc[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int pe = 0; pe < 2; ++pe) acc[u][pe] = f32x16{};
    // Hprev fragments in blocks of 4 k-steps, each block read while the
    // previous one's MFMAs run
    constexpr int HB = KS / 4;   // blocks per column half
    Frag hf[2][2][4];            // [buffer][hi, lo][k-step in block]
    auto load_h = [&](int blk, Frag (*dst)[4]) {
      const int pe = blk / HB, s0 = (blk % HB) * 4;
      const unsigned char* hp = cur + Cf::HOFF + (pe * 32 + m) * Cf::HRB;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[0][i] = *reinterpret_cast<const Frag*>(hp + (2 * (s0 + i) + g) * 32);
        dst[1][i] = *reinterpret_cast<const Frag*>(hp + (2 * (s0 + i) + g) * 32 + 16);
      }
    };
    load_h(0, hf[0]);
#pragma unroll
    for (int blk = 0; blk < 2 * HB; ++blk) {
      if (blk + 1 < 2 * HB) load_h(blk + 1, hf[(blk + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const int pe = blk / HB, s0 = (blk % HB) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          I::mma(acc[u][pe], hf[blk & 1][0][i], cf[u][s0 + i]);
          I::mma(acc[u][pe], hf[blk & 1][1][i], cf[u][s0 + i]);
        }
      if (prefetch) issue_part(nt, oth, blk * Cf::LT / (2 * HB), (blk + 1) * Cf::LT / (2 * HB));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float sc = sE[(u ? tb1 : tb0) * 32 + m];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[u][0][r] *= sc;
        acc[u][1][r] *= sc;
      }
    }

    // intra-chunk pairs, slot by slot, specialised per wave (straight-line code)
    const unsigned char* xt = cur;
    auto pairs = [&](auto wtag) {
      constexpr int W = decltype(wtag)::value;
      // x^T fragments of j-block jb: d[pe][js] holds headdim row 32 pe + m and,
      // in k-slot e, token j = 32 jb + 16 js + 4 g + 8 (e / 4) + e % 4 (the
      // order of the decayed block's k-slots below); two transposing reads each
      auto load_x = [&](int jb, Frag (*d)[2]) {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int pe = 0; pe < 2; ++pe)
#pragma unroll
          for (int js = 0; js < 2; ++js) {
            uint64_t h2[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const unsigned char* a = xt + (pe ? (xtr ^ 64u) : xtr) + (jb * 32 + 16 * js + 8 * hh) * 128;
              h2[hh] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                        (__attribute__((address_space(3))) s16x4*)(a)));
            }
            const u32x4 w4 = {(uint32_t)h2[0], (uint32_t)(h2[0] >> 32), (uint32_t)h2[1], (uint32_t)(h2[1] >> 32)};
            d[pe][js] = __builtin_bit_cast(Frag, w4);
          }
      };
      // each pair's x rows are read one pair ahead, so their LDS latency
      // hides behind the previous pair's work
      // an off-diagonal pair's weights w_j and G'_end of its j-block, also
      // read one pair ahead
      auto load_w = [&](int jb, float4* wv, float& ge) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) wv[c4] = *reinterpret_cast<const float4*>(&sW[jb * 32 + 8 * c4 + 4 * g]);
        ge = sG[jb * 32 + 31];
      };
      Frag d[2][2];
      float4 wv[4];
      float ge = 0.f;
      load_x(0, d);   // the first pair of every wave is (t-block W, j-block 0)
      if (!pair_diag(0, W)) load_w(0, wv, ge);
#pragma unroll
    for (int e = 0; e < 12; ++e) {
      const int sl = e < 4 ? e : e - 3;       // the same emission order as the C.B^T phase
      const int u = e < 4 ? 0 : 1;
      if (!pair_kept(e, W)) continue;
      const int jb = u ? 8 - sl : sl;
      const int tb = u ? 7 - W : W;
      const bool diag = jb == tb;
      const float gtu = u ? gt1 : gt0;
      const int j0 = jb * 32;
      Frag dn[2][2];
      float4 wvn[4];
      float gen = 0.f;
      const int en = next_pair(e, W);
      if (en >= 0) load_x(pair_jb(en), dn);
      if (en >= 0 && !pair_diag(en, W)) load_w(pair_jb(en), wvn, gen);
      float v[16];
      if (!diag) {
        // every t is past the whole j-block: 2^(G'_t - G'_j) = 2^(G'_t - G'_end) 2^(G'_end - G'_j)
        const float a = exp2_hw(gtu - ge);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          v[4 * c4 + 0] = from_agpr(cbc[sl][4 * c4 + 0]) * (wv[c4].x * a);
          v[4 * c4 + 1] = from_agpr(cbc[sl][4 * c4 + 1]) * (wv[c4].y * a);
          v[4 * c4 + 2] = from_agpr(cbc[sl][4 * c4 + 2]) * (wv[c4].z * a);
          v[4 * c4 + 3] = from_agpr(cbc[sl][4 * c4 + 3]) * (wv[c4].w * a);
        }
      } else {
        // diagonal block: direct decay; the causal mask is a select. The
        // skip term D x_t is the product of this block's diagonal with x,
        // so D joins the diagonal entries here and rides in the same MFMAs
        // (instead of a read-modify-write of the accumulators).
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          // rows drow(4 c4 + i, g) = 8 c4 + 4 g + i: four consecutive G', dt
          const float4 g4 = *reinterpret_cast<const float4*>(&sG[j0 + 8 * c4 + 4 * g]);
          const float4 d4 = *reinterpret_cast<const float4*>(&sDt[j0 + 8 * c4 + 4 * g]);
          const float gq[4] = {g4.x, g4.y, g4.z, g4.w}, dq[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int q = 4 * c4 + i, jr = drow(q, g);
            const float val = from_agpr(cbc[sl][q]) * exp2_hw(gtu - gq[i]) * dq[i];
            v[q] = (m > jr) ? val : ((m == jr) ? val + t.Dh : 0.f);
          }
        }
      }
      // (hi, lo) bf16 split of the decayed block, two MFMAs per x fragment
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        u32x4 uh, ul;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t hh = pack_bf16x2(v[js * 8 + 2 * i], v[js * 8 + 2 * i + 1]);
          asm volatile("" : "+v"(hh));    // keep the pair packed: the hi parts below are bit slices of it
          uh[i] = hh;
          ul[i] = pack_bf16x2(v[js * 8 + 2 * i] - __uint_as_float(hh << 16),
                              v[js * 8 + 2 * i + 1] - __uint_as_float(hh & 0xffff0000u));
        }
        const Frag ahi = __builtin_bit_cast(Frag, uh), alo = __builtin_bit_cast(Frag, ul);
#pragma unroll
        for (int pe = 0; pe < 2; ++pe) {
          I::mma(acc[u][pe], d[pe][js], ahi);
          I::mma(acc[u][pe], d[pe][js], alo);
        }
      }
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

    // y goes out through LDS in 16-byte row pieces: per t-block, the wave
    // writes its 32 x 64 block (bf16, 128-byte rows) into its own staging
    // area, 8 bytes (headdim columns 32 pe + 8 c + 4 g .. + 3 of its token
    // row m) at a time, reads it back as 16-byte pieces and stores 4 of them
    // per lane, through a buffer resource over the tile's valid rows (rows
    // past a ragged sequence are dropped by its range check). In staging row
    // t, 16-byte piece c sits at c ^ ((t / 2) % 8), which spreads the 32
    // rows a half-wave writes over the banks. One wave's LDS operations run
    // in order, so the staging area needs no barrier.
    {
      unsigned char* ys_lds = ystage + wave * 4096;
      const uint32_t wrow = (uint32_t)m * 128 + 8 * (uint32_t)g, wsw = (uint32_t)(m >> 1) & 7;
      const int pr = lane / 8, pc = lane % 8;   // piece i * 64 + lane: row 8 i + pr, 16-byte piece pc
      uint32_t plane = (uint32_t)pr * xrb + (uint32_t)pc * 16;
      uint32_t xrbs = xrb;
      asm volatile("" : "+v"(plane), "+s"(xrbs));
      const __amdgpu_buffer_rsrc_t yr = make_rsrc(t.y, (uint32_t)t.nvalid * xrbs);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int pe = 0; pe < 2; ++pe)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint2 v2 = make_uint2(pack_bf16x2(acc[u][pe][4 * c], acc[u][pe][4 * c + 1]),
                                        pack_bf16x2(acc[u][pe][4 * c + 2], acc[u][pe][4 * c + 3]));
            *reinterpret_cast<uint2*>(ys_lds + wrow + (((uint32_t)(4 * pe + c)) ^ wsw) * 16) = v2;
          }
        const uint32_t row0 = (uint32_t)((u ? tb1 : tb0) * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t rsw = (uint32_t)(4 * (i & 1) + (pr >> 1));   // ((8 i + pr) / 2) % 8
          const u32x4 v = *reinterpret_cast<const u32x4*>(ys_lds + (8 * i + pr) * 128 + ((uint32_t)pc ^ rsw) * 16);
          __builtin_amdgcn_raw_buffer_store_b128(v, yr, plane + (row0 + 8 * i) * xrbs, 0, 0);
        }
      }
    }
    const bool full = t.nvalid == Q;
    ys = (prefetch && full) ? 1 : 0;
    buf ^= 1;
  }
}

template <int N>
int64_t resident_grid(int64_t ntiles) {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    dev = 0;
  }
  if (!cached[dev]) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ssd_chunk_scan_resident<N>, 256, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0) {
      (void)hipGetLastError();
      cus = 256;
      per_cu = 1;
    }
    cached[dev] = cus * per_cu;
  }
  int64_t grid = cached[dev] < ntiles ? cached[dev] : ntiles;
  if (grid >= 8) grid -= grid % 8;
  return grid;
}

template <int N>
hipError_t launch_resident(const Problem& p, hipStream_t stream) {
  const int64_t ntiles = p.bt * p.nc * p.H;
  if (ntiles == 0) return hipSuccess;
  const int64_t grid = resident_grid<N>(ntiles);
  const int xcd = (grid % 8 == 0 && (p.bt * p.nc) % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((ssd_chunk_scan_resident<N>), dim3((unsigned)grid), dim3(256), 0, stream,
                     (const bf16*)p.x, (const bf16*)p.B, (const bf16*)p.C, p.gcum, p.dtt, p.D,
                     (const void*)p.hprev, (bf16*)p.y, p.T, (int)p.H, (int)p.G, p.nc, p.Tp, ntiles, xcd);
  return hipGetLastError();
}

}  // namespace

bool chunk_scan_resident_fits(const Problem& p) {
  return p.io == 1 && p.P == 64 && p.Q == 256 && (p.N == 64 || p.N == 128);
}

hipError_t launch_chunk_scan_resident(const Problem& p, hipStream_t stream) {
  return p.N == 64 ? launch_resident<64>(p, stream) : launch_resident<128>(p, stream);
}

}  // namespace ssd

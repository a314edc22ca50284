// The causal (Q x Q) part of the backward pass, fused: for bf16 io, headdim
// 64, chunk 256 and dstate 64 or 128, one kernel takes a chunk's heads from
// the inputs to the per-token results that the rest of the pass consumes,
//
//   dXp  = (L o CB o dt_j)^T dY             (the causal part of dx)
//   colW_j = sum_i L_ij CB_ij DX_ij,  colZ_j = dt_j colW_j
//   rowZ_i = sum_j L_ij CB_ij DX_ij dt_j     (the time-gradient sums)
//   W2g  = sum over a group's heads of L o DX o dt_j
//
// with CB = C B^T, DX = dY X^T and L_ij = 2^(G'_i - G'_j) (i >= j, else 0):
// the causal block of the CUDA Tile Mamba-2 blog's decayed block output
// (section "Mamba-2 architecture") differentiated with respect to x, B, C
// and the decays; C B^T stays on chip as in its section "Kernel 3:
// compute_out". No Q x Q block reaches memory except the group's W2g sum.
//
// Work split. A workgroup takes one (batch row, chunk, group, segment of the
// group's heads) and walks the segment's heads. C.B^T depends on the group
// only: its 36 causal 32x32 blocks are computed once and stay in the
// accumulation registers (AGPRs). Wave w owns the 32-token column blocks w
// and 7 - w: the causal blocks (ib, jb) with jb in that pair, 9 for every
// wave. Owning whole columns keeps dx (a sum over rows i) and colW inside the
// wave; row sums (rowZ) go through LDS.
//
// Per head and block: DX = dY[ib] X[jb]^T on the bf16 MFMA (exact products,
// fp32 sums), then L, the three weighted blocks and the sums on the VALU,
// then dx[jb] += W1^T dY[ib] with W1 split into a bf16 (hi, lo) pair against
// the exact dY. The accumulator layout of a block (lane = column j,
// registers = rows i) is already the first operand of that product, so W1
// never moves; dY enters through gfx950's transposing LDS read.
//
// Decays. Off the diagonal L_ij = Eloc_i F_j with Eloc_i = 2^(G'_i -
// G'_(32 ib - 1)) (one per row, computed once per head) and F_j = 2^(G'_(32 ib
// - 1) - G'_j): both exponents are <= 0, so neither factor overflows and the
// product underflows only where L itself does. Diagonal blocks take
// 2^(G'_i - G'_j) directly.
#include "lookback_device.h"
#include "ssd_bwd.h"
#include "ssd_device.h"

namespace ssd {

namespace {

constexpr int kP = 64, kQ = 256;
constexpr int kTile = kQ * kP * 2;              // one bf16 tile, 32 KB
constexpr int kBuf = 2 * kTile + 2 * kQ * 4;    // dY, X, G', dt of one head
constexpr int kZs = 40;                         // scratch row stride, floats

// Piece swizzle of the dY and X tiles (rows of 128 bytes, 8 pieces of 16):
// logical piece q of row i sits at piece q ^ fsw(i). 16 consecutive rows at
// one piece (the row fragment reads) and 4 rows at 4 adjacent pieces (the
// transposing reads) both fall on 16 distinct 16-byte bank groups.
__device__ __forceinline__ constexpr uint32_t fsw(uint32_t i) { return (((i >> 1) & 1u) << 2) | ((i >> 2) & 3u); }
__device__ __forceinline__ uint32_t toff(uint32_t i, uint32_t q) { return i * 128u + ((q ^ fsw(i)) << 4); }

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

template <int NVM>
__device__ __forceinline__ void vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NVM) : "memory");
}

template <int V> struct IC { static constexpr int value = V; };
template <bool V> struct BC { static constexpr bool value = V; };

template <int I, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(IC<I>{});
    static_for<I + 1, E>(f);
  }
}

// Stores each wave issues after a head's prefetch: 2 x (8 dx pieces + colW +
// colZ) + rowZ. A head waits for its tiles with vmcnt(kStoresAfter), a lower
// bound, so every load issued before those stores has landed.
constexpr int kStoresAfter = 16;

// W2 = false: dXp, rowZ, colZ, colW. W2 = true: only the segment's W2 sums
// (the two do not fit one kernel's registers: C.B^T and the W2 sums are 144
// values per lane each).
template <int N, bool W2>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ssd_bwd_qq(const bf16* __restrict__ x, const bf16* __restrict__ dy, const bf16* __restrict__ Bm,
                const bf16* __restrict__ Cm, const float* __restrict__ gcum, const float* __restrict__ dtt,
                float* __restrict__ dXp, float* __restrict__ rowZ, float* __restrict__ colZ,
                float* __restrict__ colW, float* __restrict__ w2part, int64_t Tlen, int H, int G, int64_t nc,
                int64_t Tp, int nseg) {
  using Frag = bf16x8;
  constexpr int KS = N / 16;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2][kBuf];
  __shared__ __attribute__((aligned(16))) float sEl[kQ];
  __shared__ __attribute__((aligned(16))) float sRow[4][kQ];
  __shared__ __attribute__((aligned(16))) float sZ[4][32 * kZs];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(w >= 0 && w < 4);
  const int hf = lane >> 5, jl = lane & 31;

  int64_t wi = blockIdx.x;
  const int seg = (int)(wi % nseg);
  wi /= nseg;
  const int grp = (int)(wi % G);
  const int64_t bkg = wi;              // (b * nc + k) * G + grp
  wi /= G;
  const int64_t k = wi % nc, b = wi / nc;
  const int hpg = H / G, hs = (hpg + nseg - 1) / nseg;
  const int h0 = grp * hpg + seg * hs;
  const int h1 = min(h0 + hs, (grp + 1) * hpg);
  const int64_t t0 = k * kQ;
  const int nvalid = (int)(Tlen - t0 < kQ ? Tlen - t0 : kQ);
  const uint32_t xrs = (uint32_t)(H * kP * 2);                       // bytes between token rows of x, dy
  const uint32_t tbytes = (uint32_t)(nvalid - 1) * xrs + kP * 2;     // a head's rows in the chunk

  // A head's tiles into LDS buffer bi: wave w fills rows 64 w .. 64 w + 63 of
  // dY and X (8 direct loads each, rows past the sequence as zeros), waves 0
  // and 1 the G' and dt rows.
  auto load_tiles = [&](int h, int bi) __attribute__((always_inline)) {
    unsigned char* base = lds[bi];
    const int64_t row0 = (b * Tlen + t0) * H + h;
    const __amdgpu_buffer_rsrc_t rdy = lookback::urs(dy + row0 * kP, tbytes);
    const __amdgpu_buffer_rsrc_t rx = lookback::urs(x + row0 * kP, tbytes);
    const uint32_t r = (uint32_t)lane >> 3, qp = (uint32_t)lane & 7;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t blk = 8u * w + m, row = 8u * blk + r;
      const uint32_t voff = row * xrs + ((qp ^ fsw(row)) << 4);
      lookback::bdma16<false>(rdy, voff, 0, base + 1024 * blk);
      lookback::bdma16<false>(rx, voff, 0, base + kTile + 1024 * blk);
    }
    if (w < 2) {
      const float* src = (w == 0 ? gcum : dtt) + ((b * H + h) * Tp + t0);
      lookback::dma16<false>(src, (uint32_t)lane * 16u, base + 2 * kTile + w * 1024);
    }
  };

  if (h0 >= h1) return;   // (the host never launches an empty segment)
  load_tiles(h0, 0);

  // ---- C.B^T blocks of the wave's 9 pairs, into AGPRs
  // slot s: (ib, jb) = (w + s, w) for s < 8 - w, else (s - 1, 7 - w)
  float cbr[W2 ? 1 : 9][16];
  if constexpr (!W2) {
    const uint32_t brs = (uint32_t)(G * N * 2);
    const uint32_t bbytes = (uint32_t)(nvalid - 1) * brs + N * 2;
    const int64_t brow0 = (b * Tlen + t0) * G + grp;
    const __amdgpu_buffer_rsrc_t rb = lookback::urs(Bm + brow0 * N, bbytes);
    const __amdgpu_buffer_rsrc_t rc = lookback::urs(Cm + brow0 * N, bbytes);
    auto ldfr = [&](__amdgpu_buffer_rsrc_t r, int blk, Frag* f) __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const uint32_t off = (uint32_t)(32 * blk + jl) * brs + (uint32_t)(16 * kk + 8 * hf) * 2;
        f[kk] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
      }
    };
    Frag b0[KS], b1[KS];
    ldfr(rb, w, b0);
    ldfr(rb, 7 - w, b1);
    static_for<0, 9>([&](auto st) __attribute__((always_inline)) {
      constexpr int s = decltype(st)::value;
      const bool c0 = s < 8 - w;
      const int ib = c0 ? w + s : s - 1;
      Frag cf[KS];
      ldfr(rc, ib, cf);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cf[kk], c0 ? b0[kk] : b1[kk], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) cbr[s][r] = to_agpr(acc[r]);
    });
  }

  float w2s[W2 ? 9 : 1][16];
  if constexpr (W2) {
#pragma unroll
    for (int s = 0; s < 9; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) w2s[s][r] = 0.f;
  }

  for (int h = h0, it = 0; h < h1; ++h, ++it) {
    const int bi = it & 1;
    if (it == 0 || W2)
      vm_barrier<0>();
    else
      vm_barrier<kStoresAfter>();
    if (h + 1 < h1) load_tiles(h + 1, bi ^ 1);
    const unsigned char* cur = lds[bi];
    const float* gL = reinterpret_cast<const float*>(cur + 2 * kTile);
    const float* dL = gL + kQ;
    {
      const float ga = tid >= 32 ? gL[(tid & ~31) - 1] : 0.f;
      sEl[tid] = exp2_hw(gL[tid] - ga);
      *reinterpret_cast<float4*>(&sRow[w][4 * lane]) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    lookback::lds_barrier();

    const int64_t hrow = (b * H + h) * Tp + t0;   // this head's token vectors
    float* zs = sZ[w];

    // Lane-dependent offsets, derived here from a lane id the compiler
    // cannot see through, so that it does not precompute every pair's
    // addresses before the loop and keep them all live.
    uint32_t lid = (uint32_t)lane;
    asm volatile("" : "+v"(lid));
    const uint32_t jlv = lid & 31u, hfv = lid >> 5;
    // row fragment (row 32 blk + jl, piece 2 kk + hf) of a swizzled tile:
    // byte 4096 blk + (fb ^ 32 kk)
    const uint32_t fb = jlv * 128u + ((hfv ^ fsw(jlv)) << 4);
    // transposing read: lane u = a + 4 m of a 16-lane group supplies row m of
    // the group's 4 rows (32 ib + 16 ks + 8 hh + 4 hf + m), columns
    // 32 pb + 16 c + 4 a .. + 3 (c: the group's 16-column half); byte
    // 4096 ib + 2048 ks + 1024 hh + (tb ^ 64 pb ^ 32 hh)
    const uint32_t tra = lid & 3u, trm = (lid >> 2) & 3u, trc = (lid >> 4) & 1u;
    const uint32_t tlp = (2u * trc + (tra >> 1)) ^ (((trm >> 1) << 2) | hfv);
    const uint32_t tb = (4u * hfv + trm) * 128u + (tlp << 4) + 8u * (tra & 1u);
    // scratch: lane (hf, jl) writes column jl of rows drow(r, hf), reads row
    // jl from column 16 hf
    const uint32_t zwb = 4u * hfv * kZs + jlv, zrb = jlv * kZs + 16u * hfv;

    // column-block state
    Frag xf[4];
    float gj = 0.f, dtj = 0.f, colw = 0.f;
    f32x16 dxa[2];
    auto load_col = [&](int jb) __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        xf[kk] = *reinterpret_cast<const Frag*>(cur + kTile + 4096 * jb + (fb ^ (32u * kk)));
      gj = gL[32 * jb + jlv];
      dtj = dL[32 * jb + jlv];
      colw = 0.f;
      dxa[0] = f32x16{};
      dxa[1] = f32x16{};
    };
    auto flush = [&](int jb) __attribute__((always_inline)) {
      if constexpr (W2) return;
      const float cw = colw + __shfl_xor(colw, 32);
      if (hfv == 0) {
        colW[hrow + 32 * jb + jlv] = cw;
        colZ[hrow + 32 * jb + jlv] = cw * dtj;
      }
      // dx rows j = 32 jb + row, 32 columns per half, through the scratch as
      // 16-byte pieces (a wave's LDS operations complete in order)
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) zs[zwb + (8 * (r / 4) + r % 4) * kZs] = dxa[pb][r];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int row = 8 * c + (int)(lid >> 3), c4 = 4 * (int)(lid & 7);
          const float4 v = *reinterpret_cast<const float4*>(&zs[row * kZs + c4]);
          *reinterpret_cast<float4*>(dXp + ((b * Tp + t0 + 32 * jb + row) * H + h) * kP + 32 * pb + c4) = v;
        }
      }
    };

    auto pair = [&](auto stag, auto dtag, int ib) __attribute__((always_inline)) {
      constexpr int s = decltype(stag)::value;
      constexpr bool DIAG = decltype(dtag)::value;
      // each pair's work stays between its own scheduling fences: hoisting the
      // next pairs' LDS reads would only add live registers
      __builtin_amdgcn_sched_barrier(0);
      // DX block = dY[ib] X[jb]^T
      f32x16 dxv = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const Frag a = *reinterpret_cast<const Frag*>(cur + 4096 * ib + (fb ^ (32u * kk)));
        dxv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xf[kk], dxv, 0, 0, 0);
      }
      // decays of the block's 16 rows in this lane's column
      float ln[16];
      if constexpr (DIAG) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 g4 = *reinterpret_cast<const float4*>(&gL[32 * ib + 8 * q + 4 * hfv]);
          const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q + e;
            const float l = exp2_hw(gv[e] - gj);
            ln[r] = (uint32_t)(8 * q + e) + 4u * hfv >= jlv ? l : 0.f;
          }
        }
      } else {
        const float F = exp2_hw(gL[32 * ib - 1] - gj);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 e4 = *reinterpret_cast<const float4*>(&sEl[32 * ib + 8 * q + 4 * hfv]);
          ln[4 * q] = e4.x * F;
          ln[4 * q + 1] = e4.y * F;
          ln[4 * q + 2] = e4.z * F;
          ln[4 * q + 3] = e4.w * F;
        }
      }
      if constexpr (W2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) w2s[s][r] += (ln[r] * dtj) * dxv[r];
        return;
      }
      float w1[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float cb = from_agpr(cbr[W2 ? 0 : s][r]);
        const float d = dxv[r];
        const float u = ln[r] * (cb * d);
        colw += u;
        zs[zwb + (8 * (r / 4) + r % 4) * kZs] = u * dtj;
        const float ld = ln[r] * dtj;
        w1[r] = ld * cb;
      }
      // row sums of Z over the block's 32 columns: lane (hf, jl) adds row jl,
      // columns 16 hf .. 16 hf + 15, then the two halves
      {
        float rs = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float4 v = *reinterpret_cast<const float4*>(&zs[zrb + 4 * c]);
          rs += (v.x + v.y) + (v.z + v.w);
        }
        rs += __shfl_xor(rs, 32);
        if (hfv == 0) sRow[w][32 * ib + jlv] += rs;
      }
      // dx[jb] += W1^T dY[ib]: k-slot e of half hf and step ks is row
      // 16 ks + 8 (e / 4) + 4 hf + e % 4 of the block on both sides
      typedef short s16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        Frag hi, lo;
        Io<bf16>::split(&w1[8 * ks], hi, lo);
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
          uint64_t h2[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const unsigned char* a = cur + 4096 * ib + 2048 * ks + 1024 * hh + (tb ^ (64u * pb + 32u * hh));
            h2[hh] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                      (__attribute__((address_space(3))) s16x4*)(a)));
          }
          const u32x4 w4 = {(uint32_t)h2[0], (uint32_t)(h2[0] >> 32), (uint32_t)h2[1], (uint32_t)(h2[1] >> 32)};
          const Frag bfr = __builtin_bit_cast(Frag, w4);
          dxa[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, bfr, dxa[pb], 0, 0, 0);
          dxa[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, bfr, dxa[pb], 0, 0, 0);
        }
      }
    };

    // the wave's 9 pairs: column block w (slots 0 .. 7 - w), then 7 - w
    load_col(w);
    static_for<0, 9>([&](auto st) __attribute__((always_inline)) {
      constexpr int s = decltype(st)::value;
      if constexpr (s == 0) {
        pair(IC<0>{}, BC<true>{}, w);
      } else if constexpr (s <= 4) {
        pair(IC<s>{}, BC<false>{}, w + s);
      } else {
        if (s < 8 - w) {
          pair(IC<s>{}, BC<false>{}, w + s);
        } else if (s == 8 - w) {
          flush(w);
          load_col(7 - w);
          pair(IC<s>{}, BC<true>{}, s - 1);
        } else {
          pair(IC<s>{}, BC<false>{}, s - 1);
        }
      }
    });
    flush(7 - w);

    // rowZ: the four waves' partial row sums
    if constexpr (!W2) {
      lookback::lds_barrier();
      rowZ[hrow + tid] = ((sRow[0][tid] + sRow[1][tid]) + sRow[2][tid]) + sRow[3][tid];
    }
  }

  if constexpr (W2) {
    // this segment's sum of L o DX o dt_j over its heads, causal 32x32 blocks
    float* o = w2part + ((bkg * nseg + seg) * kQ) * kQ;
    static_for<0, 9>([&](auto st) __attribute__((always_inline)) {
      constexpr int s = decltype(st)::value;
      const bool c0 = s < 8 - w;
      const int ib = c0 ? w + s : s - 1, jb = c0 ? w : 7 - w;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[(32 * ib + drow(r, hf)) * kQ + 32 * jb + jl] = w2s[s][r];
    });
  }
}

// W2g[bkg] = the sum of the segments' blocks on and below the diagonal; the
// 32x32 blocks above it inside a 64x64 diagonal tile are cleared (the causal
// products that read W2g run over whole 64-wide tiles).
__global__ void w2_segment_sum(const float* __restrict__ part, float* __restrict__ out, int nseg, int64_t total4) {
  constexpr int64_t QQ = (int64_t)kQ * kQ;
  for (int64_t i4 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i4 < total4; i4 += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = 4 * i4, bkg = e / QQ, o = e % QQ;
    const int i = (int)(o / kQ), j = (int)(o % kQ);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i / 32 >= j / 32) {
      const float* src = part + bkg * nseg * QQ + o;
      for (int s = 0; s < nseg; ++s) {
        const float4 v = *reinterpret_cast<const float4*>(src + s * QQ);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
    } else if (i / 64 != j / 64) {
      continue;   // never read
    }
    *reinterpret_cast<float4*>(out + e) = acc;
  }
}


// ---------------------------------------------------------------- finish
// Per (batch row, chunk, head): the carried-state terms and the per-token
// results,
//
//   U = B dHn^T,  V = C Hprev^T                 (rows: tokens, columns: headdim)
//   dx_t   = dXp_t + w_t U_t + D dY_t
//   avec_t = dY_t . V_t,  bvec_t = x_t . U_t,  ddx_t = dY_t . x_t
//   dG_t   = E_t avec_t + rowZ_t - colZ_t - w_t bvec_t   (+ at the chunk's
//            last token: 2^(G'_last) <dHn, Hprev> + sum_j w_j bvec_j)
//   ddt_t  = colW_t + 2^(G'_last - G'_t) bvec_t + A sum_{j >= t} dG_j
//   dA part = sum_t dG_t cumdt_t,  dD part = sum_t ddx_t
//
// with E_t = 2^(G'_t), w_t = dt_t 2^(G'_last - G'_t) and dHn the adjoint of
// the state leaving the chunk (the chain rule through G_t = A sum_{s <= t}
// dt_s of the blog's decays, section "Mamba-2 architecture").
//
// The two fp32 states are read once per workgroup as whole rows, split into
// bf16 (hi, lo) planes in LDS (their inner product taken on the way), and
// every wave takes its MFMA fragments from there. Wave v owns the 32 tokens
// of block v: U and V on the bf16 MFMA against the exact bf16 B and C rows,
// lane = headdim column and registers = tokens, so x, dy, dXp and dx are read
// and written as whole rows. The per-token dot products go through LDS; the
// chunk's scans are wave scans joined through LDS.
template <int N>
struct FinCfg {
  static constexpr int RP = N / 8;                 // 16-byte pieces per bf16 state row
  static constexpr int PLANE = kP * N * 2;         // bytes of one bf16 plane
  static constexpr int LDS = 4 * PLANE;            // dHn hi, lo, Hprev hi, lo
};
// piece q of state row p (RP pieces) sits at piece q ^ (p % min(RP, 16)):
// with RP >= 16 the fragment reads (16 rows, one piece each) hit 16 distinct
// 16-byte bank groups
template <int RP>
__device__ __forceinline__ uint32_t spiece(uint32_t p, uint32_t q) {
  return q ^ (p & (uint32_t)((RP < 16 ? RP : 16) - 1));
}

template <int N>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void ssd_bwd_state_finish(
    const bf16* __restrict__ x, const bf16* __restrict__ dy, const bf16* __restrict__ Bm, const bf16* __restrict__ Cm,
    const float* __restrict__ Ap, const float* __restrict__ Dp, const float* __restrict__ gcum,
    const float* __restrict__ dtt, const float* __restrict__ wst, const float* __restrict__ hprev,
    const float* __restrict__ dhn, const float* __restrict__ dXp, const float* __restrict__ rowZ,
    const float* __restrict__ colZ, const float* __restrict__ colW, float* __restrict__ dx, float* __restrict__ ddt,
    float* __restrict__ dA_part, float* __restrict__ dD_part, uint4* __restrict__ dhnT, uint4* __restrict__ hpT,
    int64_t Tlen, int H, int G, int64_t nc, int64_t Tp, int64_t nbk) {
  using Frag = bf16x8;
  using Cf = FinCfg<N>;
  constexpr int KS = N / 16, RP = Cf::RP;
  __shared__ __attribute__((aligned(16))) unsigned char sS[Cf::LDS];
  __shared__ __attribute__((aligned(16))) float sZ[8][32 * kZs];
  __shared__ float sA[kQ], sB[kQ], sD[kQ];
  __shared__ float sRed[4][8];
  __shared__ float sTot[2][4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int v = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave 0..7 = token block
  const int hf = lane >> 5, jl = lane & 31;
  // XCD-aware order: workgroup tau runs on XCD tau % 8, and the heads of one
  // (b, k) share an XCD, so its B, C rows and DX blocks are read into one L2
  const int64_t tau = blockIdx.x, xcd = tau % 8, slot = tau / 8;
  const int64_t bk = (slot / H) * 8 + xcd;
  if (bk >= nbk) return;
  const int h = (int)(slot % H);
  const int64_t k = bk % nc, b = bk / nc;
  const int grp = h / (H / G);
  const int64_t t0 = k * kQ;
  const int nvalid = (int)(Tlen - t0 < kQ ? Tlen - t0 : kQ);
  const int64_t hrow = (b * H + h) * Tp + t0;

  // ---- the states: whole rows in, bf16 (hi, lo) planes out, and <dHn, Hprev>
  float dot = 0.f;
  {
    const float* ds = dhn + ((b * H + h) * nc + k) * (int64_t)(kP * N);
    const float* hs = hprev + ((b * H + h) * nc + k) * (int64_t)(kP * N);
    constexpr int NV = kP * N / 4 / 512;   // 16-byte pieces per thread and state
    float4 dv[NV], hv[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      dv[j] = *reinterpret_cast<const float4*>(ds + 4 * (tid + 512 * j));
      hv[j] = *reinterpret_cast<const float4*>(hs + 4 * (tid + 512 * j));
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = 4 * (tid + 512 * j), pr = e / N, n0 = e % N;
      dot = fmaf(dv[j].x, hv[j].x, fmaf(dv[j].y, hv[j].y, fmaf(dv[j].z, hv[j].z, fmaf(dv[j].w, hv[j].w, dot))));
      const uint32_t off = (uint32_t)pr * (N * 2) + (spiece<RP>(pr, n0 / 8) << 4) + (uint32_t)(n0 % 8) * 2;
      auto put = [&](const float4& q, int plane) {
        const uint32_t h01 = pack_bf16x2(q.x, q.y), h23 = pack_bf16x2(q.z, q.w);
        const uint32_t l01 = pack_bf16x2(q.x - bf16lo(h01), q.y - bf16hi(h01));
        const uint32_t l23 = pack_bf16x2(q.z - bf16lo(h23), q.w - bf16hi(h23));
        *reinterpret_cast<uint2*>(sS + plane * Cf::PLANE + off) = make_uint2(h01, h23);
        *reinterpret_cast<uint2*>(sS + (plane + 1) * Cf::PLANE + off) = make_uint2(l01, l23);
      };
      put(dv[j], 0);
      put(hv[j], 2);
    }
  }
  // B and C rows of the wave's tokens (exact bf16 fragments)
  Frag bfr[KS], cfr[KS];
  {
    const uint32_t brs = (uint32_t)(G * N * 2);
    const uint32_t bbytes = (uint32_t)(nvalid - 1) * brs + N * 2;
    const int64_t brow0 = (b * Tlen + t0) * G + grp;
    const __amdgpu_buffer_rsrc_t rb = lookback::urs(Bm + brow0 * N, bbytes);
    const __amdgpu_buffer_rsrc_t rc = lookback::urs(Cm + brow0 * N, bbytes);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint32_t off = (uint32_t)(32 * v + jl) * brs + (uint32_t)(16 * kk + 8 * hf) * 2;
      bfr[kk] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
      cfr[kk] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0));
    }
  }
  __syncthreads();

  // ---- the states transposed into bf16 (hi, lo) MFMA fragments (column n,
  // 8 consecutive headdim rows per lane), in the order the head-summed dB and
  // dC products read them: each 16-lane group
  // gathers 16 columns of 8 rows with the transposing LDS read (lane
  // u = a + 4 m supplies row m of 4, columns 4 a .. 4 a + 3; lane u receives
  // column u of the 4 rows)
  {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const int gi = v * 4 + (lane >> 4), u = lane & 15, ta = u & 3, tm = u >> 2;
    const int64_t tb = ((b * H + h) * nc + k) * (int64_t)N;   // first (n) row of this tile
#pragma unroll
    for (int j = 0; j < N / 64; ++j) {
      const int it = gi + 32 * j, pg = it % 8, nblk = it / 8;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        uint64_t q[2][2];   // [plane hi/lo][row half]
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t row = (uint32_t)(8 * pg + 4 * hh + tm);
          const uint32_t off = row * (N * 2) + (spiece<RP>(row, (uint32_t)(2 * nblk + (ta >> 1))) << 4) + 8u * (ta & 1);
#pragma unroll
          for (int pl = 0; pl < 2; ++pl)
            q[pl][hh] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(sS + (2 * st + pl) * Cf::PLANE + off)));
        }
        // fragment order: [n block of 32][k-step][plane][lane], lane = 32 (pg % 2) + n % 32
        const int n = 16 * nblk + u;
        uint4* dst = (st == 0 ? dhnT : hpT) + (((tb / 32 + n / 32) * 4 + pg / 2) * 2) * 64 + 32 * (pg % 2) + n % 32;
        dst[0] = make_uint4((uint32_t)q[0][0], (uint32_t)(q[0][0] >> 32), (uint32_t)q[0][1], (uint32_t)(q[0][1] >> 32));
        dst[64] = make_uint4((uint32_t)q[1][0], (uint32_t)(q[1][0] >> 32), (uint32_t)q[1][1], (uint32_t)(q[1][1] >> 32));
      }
    }
  }

  // ---- U and V for token block v, both headdim halves
  f32x16 U[2], V[2];
  U[0] = U[1] = V[0] = V[1] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const uint32_t pr = (uint32_t)(32 * pb + jl);
      const uint32_t off = pr * (N * 2) + (spiece<RP>(pr, (uint32_t)(2 * kk + hf)) << 4);
      const Frag dh = *reinterpret_cast<const Frag*>(sS + off);
      const Frag dl = *reinterpret_cast<const Frag*>(sS + Cf::PLANE + off);
      const Frag hh = *reinterpret_cast<const Frag*>(sS + 2 * Cf::PLANE + off);
      const Frag hl = *reinterpret_cast<const Frag*>(sS + 3 * Cf::PLANE + off);
      U[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk], dh, U[pb], 0, 0, 0);
      U[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk], dl, U[pb], 0, 0, 0);
      V[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cfr[kk], hh, V[pb], 0, 0, 0);
      V[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cfr[kk], hl, V[pb], 0, 0, 0);
    }
  }

  // ---- per token: dx, and the three dot products over headdim
  {
    const uint32_t xrs = (uint32_t)(H * kP * 2);
    const uint32_t xbytes = (uint32_t)(nvalid - 1) * xrs + kP * 2;
    const int64_t row0 = (b * Tlen + t0) * H + h;
    const __amdgpu_buffer_rsrc_t rx = lookback::urs(x + row0 * kP, xbytes);
    const __amdgpu_buffer_rsrc_t ry = lookback::urs(dy + row0 * kP, xbytes);
    const __amdgpu_buffer_rsrc_t ro = lookback::urs(dx + row0 * kP, (uint32_t)(nvalid - 1) * (xrs * 2) + kP * 4);
    const float Dh = Dp[h];
    // every load before any store (a load issued behind a store waits for it)
    float xv[2][16], yv[2][16], dp[2][16], wv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * v + drow(r, hf);
      wv[r] = wst[hrow + i];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        const uint32_t eo = (uint32_t)i * xrs + (uint32_t)(32 * pb + jl) * 2;
        xv[pb][r] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rx, eo, 0, 0) << 16);
        yv[pb][r] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(ry, eo, 0, 0) << 16);
        dp[pb][r] = dXp[((b * Tp + t0 + i) * H + h) * kP + 32 * pb + jl];
      }
    }
    float pa[16], pbv[16], pd[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * v + drow(r, hf);
      pa[r] = 0.f;
      pbv[r] = 0.f;
      pd[r] = 0.f;
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        const uint32_t eo = (uint32_t)i * xrs + (uint32_t)(32 * pb + jl) * 2;
        const float u = U[pb][r], vv = V[pb][r];
        buf_store_dword(__float_as_uint(dp[pb][r] + wv[r] * u + Dh * yv[pb][r]), ro, 2 * eo);
        pa[r] = fmaf(yv[pb][r], vv, pa[r]);
        pbv[r] = fmaf(xv[pb][r], u, pbv[r]);
        pd[r] = fmaf(yv[pb][r], xv[pb][r], pd[r]);
      }
    }
    // row sums over the 32 lanes of a half through the wave's scratch (a
    // wave's LDS operations complete in order): lane (hf, jl) adds row jl,
    // columns 16 hf .. 16 hf + 15, then the two halves
    float* zs = sZ[v];
    auto rowsum = [&](const float* val, float* out) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) zs[drow(r, hf) * kZs + jl] = val[r];
      float rs = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 t4 = *reinterpret_cast<const float4*>(&zs[jl * kZs + 16 * hf + 4 * c]);
        rs += (t4.x + t4.y) + (t4.z + t4.w);
      }
      rs += __shfl_xor(rs, 32);
      if (hf == 0) out[32 * v + jl] = rs;
    };
    rowsum(pa, sA);
    rowsum(pbv, sB);
    rowsum(pd, sD);
  }
  for (int off = 32; off >= 1; off /= 2) dot += __shfl_xor(dot, off);
  if (lane == 0) sRed[3][v] = dot;
  __syncthreads();

  // ---- the chunk's scans, one token per thread of waves 0-3
  const bool scan = v < 4;
  const int t = tid & (kQ - 1);
  float dg = 0.f, bv = 0.f, gt = 0.f, dtv = 0.f, glast = 0.f;
  auto wave_sum = [&](float val) {
    for (int off = 32; off >= 1; off /= 2) val += __shfl_xor(val, off);
    return val;
  };
  if (scan) {
    gt = gcum[hrow + t];
    dtv = dtt[hrow + t];
    glast = gcum[hrow + kQ - 1];
    const float wt = wst[hrow + t];
    bv = sB[t];
    dg = exp2_hw(gt) * sA[t] + rowZ[hrow + t] - colZ[hrow + t] - wt * bv;
    const float s0 = wave_sum(wt * bv), s1 = wave_sum(sD[t]);
    if (lane == 0) {
      sRed[0][v] = s0;
      sRed[1][v] = s1;
    }
  }
  __syncthreads();
  float suf = 0.f, pre = 0.f;
  if (scan) {
    const float swb = ((sRed[0][0] + sRed[0][1]) + sRed[0][2]) + sRed[0][3];
    float dotv = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) dotv += sRed[3][u];
    if (t == kQ - 1) dg += exp2_hw(glast) * dotv + swb;
    // suffix sums of dG (within the wave, then the later waves' totals) and
    // prefix sums of dt
    suf = dg;
    pre = dtv;
    for (int off = 1; off < 64; off *= 2) {
      const float sd = __shfl_down(suf, off), su = __shfl_up(pre, off);
      if (lane + off < 64) suf += sd;
      if (lane >= off) pre += su;
    }
    if (lane == 0) sTot[0][v] = suf;
    if (lane == 63) sTot[1][v] = pre;
  }
  __syncthreads();
  if (scan) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u > v) suf += sTot[0][u];
      if (u < v) pre += sTot[1][u];
    }
    if (t0 + t < Tlen) ddt[(b * Tlen + t0 + t) * H + h] = colW[hrow + t] + exp2_hw(glast - gt) * bv + Ap[h] * suf;
    const float s2 = wave_sum(dg * pre);
    if (lane == 0) sRed[2][v] = s2;
  }
  __syncthreads();
  if (tid == 0) {
    dA_part[(b * H + h) * nc + k] = ((sRed[2][0] + sRed[2][1]) + sRed[2][2]) + sRed[2][3];
    dD_part[(b * H + h) * nc + k] = ((sRed[1][0] + sRed[1][1]) + sRed[1][2]) + sRed[1][3];
  }
}

// ---------------------------------------------------------------- head sums
// The carried-state parts of dB and dC, summed over a group's heads:
//
//   dB_t += sum_h w_t^h  x_t^h  dHn^h      dC_t += sum_h E_t^h dY_t^h Hprev^h
//
// (per chunk; rows t of the chunk, columns n), i.e. one product per chunk
// with a contraction over (head, headdim). The row scale times x is split
// into a bf16 (hi, lo) pair; the states arrive as (hi, lo) MFMA fragments
// from the finishing kernel; three MFMAs per step (hi.hi, hi.lo, lo.hi).
// A workgroup computes a 64 x 64 tile (tokens x dstate columns), one 32 x 32
// block per wave, walking the group's heads; each head's x rows, state
// fragments and scale row come in by direct global->LDS loads one head
// ahead. The eight tiles of a (batch row, chunk, group) run on one XCD, so
// its x rows and states are read from HBM once.
template <int N>
struct HsCfg {
  static constexpr int TT = 128;                   // tokens per tile
  static constexpr int RB = N == 128 ? 2 : 1;      // 32-row blocks per wave
  static constexpr int NB = N / 32;                // 32-column blocks per tile (2 per wave)
  static constexpr int XB = TT * 128;              // x rows of the tile, one head
  static constexpr int SB = NB * 4 * 2 * 1024;     // state fragments of the tile's column blocks
  static constexpr int GB = 1024;                  // the head's scale row (the whole chunk)
  static constexpr int BUF = XB + SB + GB;
  static constexpr int NI = BUF / 1024;            // direct loads per head
  static constexpr int ITEMS = kQ / TT;            // tiles per (batch row, chunk, group)
};

template <int N>
__global__ __launch_bounds__(256) void ssd_bwd_headsum(const bf16* __restrict__ X, const float* __restrict__ scale,
                                                       const uint4* __restrict__ ST, float* __restrict__ out,
                                                       int64_t Tlen, int H, int G, int64_t nc, int64_t Tp,
                                                       int64_t nbkg) {
  using Frag = bf16x8;
  using Cf = HsCfg<N>;
  constexpr int RB = Cf::RB;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2][Cf::BUF];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, jl = lane & 31;
  // XCD-aware order: workgroup tau runs on XCD tau % 8; the tiles of one
  // (b, k, g) share an XCD
  const int64_t tau = blockIdx.x, xcd = tau % 8, slot = tau / 8;
  const int64_t bkg = (slot / Cf::ITEMS) * 8 + xcd;
  if (bkg >= nbkg) return;
  const int itile = (int)(slot % Cf::ITEMS);
  const int grp = (int)(bkg % G);
  const int64_t k = (bkg / G) % nc, b = bkg / G / nc;
  const int64_t t0 = k * kQ;
  const int nvalid = (int)(Tlen - t0 < kQ ? Tlen - t0 : kQ);
  const int hpg = H / G;
  const uint32_t xrs = (uint32_t)(H * kP * 2);
  // the tile's rows t0 + TT itile + 0 .. TT - 1 of X (rows past the sequence: zeros)
  const int rows = nvalid - Cf::TT * itile;
  const uint32_t xbytes = rows > 0 ? (uint32_t)(rows - 1) * xrs + (uint32_t)(H * kP * 2) : 0u;
  const bf16* xt = X + (b * Tlen + t0 + (rows > 0 ? Cf::TT * itile : 0)) * H * kP;
  // wave w: rows rb0 .. rb0 + 32 RB - 1, columns of blocks cb0, cb0 + 1
  const int rb0 = RB == 2 ? 64 * (w >> 1) : 32 * w;
  const int cb0 = RB == 2 ? 2 * (w & 1) : 0;

  auto load_head = [&](int hl, int bi) __attribute__((always_inline)) {
    const int h = grp * hpg + hl;
    unsigned char* base = lds[bi];
    const __amdgpu_buffer_rsrc_t rx = lookback::urs(xt, xbytes);
    for (int m = w; m < Cf::NI; m += 4) {
      if (m < Cf::XB / 1024) {
        // x rows 8 m .. 8 m + 7; piece q of row r at q ^ ((r >> 1) & 7)
        const uint32_t r = 8u * m + ((uint32_t)lane >> 3), qp = (uint32_t)lane & 7;
        const uint32_t q = qp ^ ((r >> 1) & 7u);
        lookback::bdma16<false>(rx, r * xrs + (uint32_t)h * (kP * 2) + q * 16u, 0, base + 1024 * m);
      } else if (m < (Cf::XB + Cf::SB) / 1024) {
        // state fragments: (column block c, k-step kk, plane pl), 1 KB each
        const int f = m - Cf::XB / 1024;
        const uint4* src = ST + (((b * H + h) * nc + k) * (N / 32) * 8 + f) * 64;
        lookback::dma16<false>(src, (uint32_t)lane * 16u, base + 1024 * m);
      } else {
        lookback::dma16<false>(scale + (b * H + h) * Tp + t0, (uint32_t)lane * 16u, base + 1024 * m);
      }
    }
  };

  f32x16 acc[RB][2];
#pragma unroll
  for (int a = 0; a < RB; ++a) acc[a][0] = acc[a][1] = f32x16{};
  load_head(0, 0);
  for (int hl = 0; hl < hpg; ++hl) {
    const int bi = hl & 1;
    lookback::vm_lds_barrier();
    if (hl + 1 < hpg) load_head(hl + 1, bi ^ 1);
    const unsigned char* cur = lds[bi];
    const float* scl = reinterpret_cast<const float*>(cur + Cf::XB + Cf::SB) + Cf::TT * itile;
    float sc[RB];
#pragma unroll
    for (int a = 0; a < RB; ++a) sc[a] = scl[rb0 + 32 * a + jl];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t q = (uint32_t)(2 * kk + hf);
      Frag ah[RB], al[RB], bh[2], bl[2];
#pragma unroll
      for (int a = 0; a < RB; ++a) {
        const uint32_t ar = (uint32_t)(rb0 + 32 * a + jl);
        const u32x4 xr = *reinterpret_cast<const u32x4*>(cur + ar * 128u + ((q ^ ((ar >> 1) & 7u)) << 4));
        float xv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[2 * e] = sc[a] * bf16lo(xr[e]);
          xv[2 * e + 1] = sc[a] * bf16hi(xr[e]);
        }
        Io<bf16>::split(xv, ah[a], al[a]);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const unsigned char* sf = cur + Cf::XB + (((cb0 + c) * 4 + kk) * 2) * 1024 + 16 * lane;
        bh[c] = *reinterpret_cast<const Frag*>(sf);
        bl[c] = *reinterpret_cast<const Frag*>(sf + 1024);
      }
#pragma unroll
      for (int a = 0; a < RB; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[a], bh[c], acc[a][c], 0, 0, 0);
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[a], bl[c], acc[a][c], 0, 0, 0);
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[a], bh[c], acc[a][c], 0, 0, 0);
        }
    }
  }
  // rows TT itile + rb0 + 32 a + drow(r, hf), columns 32 (cb0 + c) + jl
#pragma unroll
  for (int a = 0; a < RB; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float* o = out + ((b * Tp + t0 + Cf::TT * itile + rb0 + 32 * a) * G + grp) * (int64_t)N + 32 * (cb0 + c) + jl;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[(int64_t)drow(r, hf) * G * N] = acc[a][c][r];
    }
}

}  // namespace

bool bwd_fused_supported(int io, int64_t P, int64_t N, int64_t Q) {
  return io == 1 && P == kP && Q == kQ && (N == 64 || N == 128);
}

int bwd_fused_segments(int64_t bt, int64_t nc, int64_t H, int64_t G) {
  const int64_t hpg = H / G, items = bt * nc * G;
  if (items <= 0 || hpg <= 0) return 1;
  // about 256 workgroups or more, each walking at least one head
  int64_t nseg = (256 + items - 1) / items;
  if (nseg > hpg) nseg = hpg;
  if (nseg < 1) nseg = 1;
  const int64_t hs = (hpg + nseg - 1) / nseg;
  return (int)((hpg + hs - 1) / hs);   // no empty segment
}

hipError_t launch_bwd_fused_qq(const BwdProblem& p, float* w2part, int nseg, hipStream_t s) {
  const int64_t items = p.bt * p.nc * p.G * nseg;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffff) return hipErrorInvalidValue;
  const bf16* x = static_cast<const bf16*>(p.x);
  const bf16* dy = static_cast<const bf16*>(p.dy);
  const bf16* Bm = static_cast<const bf16*>(p.B);
  const bf16* Cm = static_cast<const bf16*>(p.C);
  auto launch = [&](auto ntag, auto wtag) {
    constexpr int NN = decltype(ntag)::value;
    constexpr bool WW = decltype(wtag)::value;
    hipLaunchKernelGGL((ssd_bwd_qq<NN, WW>), dim3((unsigned)items), dim3(256), 0, s, x, dy, Bm, Cm, p.gcum, p.dtt,
                       p.dXp, p.rowZ, p.colZ, p.colW, w2part, p.T, (int)p.H, (int)p.G, p.nc, p.Tp, nseg);
  };
  if (p.N == 64) {
    launch(IC<64>{}, BC<false>{});
    launch(IC<64>{}, BC<true>{});
  } else {
    launch(IC<128>{}, BC<false>{});
    launch(IC<128>{}, BC<true>{});
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total4 = p.bt * p.nc * p.G * (int64_t)kQ * kQ / 4;
  const int64_t g = (total4 + 255) / 256;
  hipLaunchKernelGGL(w2_segment_sum, dim3((unsigned)(g < 65536 ? g : 65536)), dim3(256), 0, s, w2part, p.CB, nseg,
                     total4);
  return hipGetLastError();
}

hipError_t launch_bwd_fused_headsum(const BwdProblem& p, const void* X, const float* scale, const void* ST,
                                    float* out, hipStream_t s) {
  const int64_t nbkg = p.bt * p.nc * p.G;
  const int64_t items = (nbkg + 7) / 8 * 8 * (kQ / 128);
  if (nbkg <= 0 || p.H <= 0) return hipSuccess;
  if (items > 0x7fffffff) return hipErrorInvalidValue;
  if (p.N == 64)
    hipLaunchKernelGGL(ssd_bwd_headsum<64>, dim3((unsigned)items), dim3(256), 0, s, (const bf16*)X, scale,
                       (const uint4*)ST, out, p.T, (int)p.H, (int)p.G, p.nc, p.Tp, nbkg);
  else
    hipLaunchKernelGGL(ssd_bwd_headsum<128>, dim3((unsigned)items), dim3(256), 0, s, (const bf16*)X, scale,
                       (const uint4*)ST, out, p.T, (int)p.H, (int)p.G, p.nc, p.Tp, nbkg);
  return hipGetLastError();
}

hipError_t launch_bwd_fused_finish(const BwdProblem& p, hipStream_t s) {
  const int64_t nbk = p.bt * p.nc;
  const int64_t items = (nbk + 7) / 8 * 8 * p.H;   // (b, k) padded to a multiple of 8
  if (nbk <= 0 || p.H <= 0) return hipSuccess;
  if (items > 0x7fffffff) return hipErrorInvalidValue;
  const bf16* x = static_cast<const bf16*>(p.x);
  const bf16* dy = static_cast<const bf16*>(p.dy);
  const bf16* Bm = static_cast<const bf16*>(p.B);
  const bf16* Cm = static_cast<const bf16*>(p.C);
  if (p.N == 64)
    hipLaunchKernelGGL(ssd_bwd_state_finish<64>, dim3((unsigned)items), dim3(512), 0, s, x, dy, Bm, Cm, p.A, p.D,
                       p.gcum, p.dtt, p.wst, p.hprev, p.dhn, p.dXp, p.rowZ, p.colZ, p.colW, p.dx, p.ddt, p.dA_part,
                       p.dD_part, (uint4*)p.U, (uint4*)p.V, p.T, (int)p.H, (int)p.G, p.nc, p.Tp, nbk);
  else
    hipLaunchKernelGGL(ssd_bwd_state_finish<128>, dim3((unsigned)items), dim3(512), 0, s, x, dy, Bm, Cm, p.A, p.D,
                       p.gcum, p.dtt, p.wst, p.hprev, p.dhn, p.dXp, p.rowZ, p.colZ, p.colW, p.dx, p.ddt, p.dA_part,
                       p.dD_part, (uint4*)p.U, (uint4*)p.V, p.T, (int)p.H, (int)p.G, p.nc, p.Tp, nbk);
  return hipGetLastError();
}

}  // namespace ssd

// ssd_chunk_state: each chunk's own contribution to the state,
//
//   S_k[p, n] = sum_{t in chunk k} x[t, p] * w_t * B[t, n],
//   w_t = dt_t * 2^(G'_last - G'_t)   (computed by ssd_chunk_cumsum)
//
// i.e. (exp(G_last - G) o dt o B)^T X of the CUDA Tile Mamba-2 blog's jump
// formula (section "Mamba-2 architecture"; the MMA in "Kernel 2:
// fwd_pass_state"), held headdim-major. Here it is computed for every chunk
// in parallel, and the sequential part lives in ssd_state_pass.
//
// One wave computes one (batch, head, chunk) tile's rows of one headdim
// column group against NGW dstate column groups with 32x32 MFMAs; the
// contraction runs over the chunk's tokens in steps of 2*KPL, with the loads
// of the next few steps in flight (a small ring of registers) while this
// step's MFMAs run. Loads go through buffer resources: the token-row part of
// each address is a scalar offset, and in a ragged last chunk the rows past
// the sequence load as zeros. The scale w_t
// is applied to x (w and x are both per head, while B is shared by the
// heads of a group). With bf16 io the product w*x is not a bf16 number, so
// it enters the MFMA as a bf16 (hi, lo) pair in two MFMAs against the exact
// bf16 B (the blog instead rounds its scaled operand to bf16 once; that
// rounding alone breaks a 1e-2 + 2e-2|y| elementwise bound where large terms
// cancel). Accumulation is fp32 and S is stored fp32 into the workspace.
//
// Operand loads: the contraction index (token) is the slow index of both x
// and B in memory, so each lane loads one dword per token row; a 32-lane
// half reads a whole 128-byte row. Element e of a dword feeds the MFMA block
// of parity e (see ssd_device.h), so both operands arrive without any
// transpose through LDS.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

template <typename T, int P, int N>
struct StateCfg {
  static constexpr int E = Io<T>::E;
  static constexpr int CG = 32 * E;                 // columns per column group
  static constexpr int NPG = P / CG;                // headdim column groups
  static constexpr int NNG = N / CG;                // dstate column groups
  // dstate groups per wave: one 32x32 block pair set per wave (64 fp32
  // accumulators) unless that needs more than 8 waves per tile
  static constexpr int NGW = (NPG * NNG > 8) ? (NPG * NNG) / 8 : 1;
  static constexpr int NGS = NNG / NGW;
  static constexpr int WPT = NPG * NGS;             // waves per (b, h, chunk) tile
  static constexpr int TPW = WPT >= 4 ? 1 : 4 / WPT;   // tiles per workgroup
  static constexpr int THREADS = 64 * WPT * TPW;
  static_assert(WPT >= 1 && WPT <= 8, "tile does not fit a workgroup");
};

// One k-step's operands for a lane: KPL token rows of x and of each of the
// wave's NGW dstate column groups of B (one dword each), and KPL weights.
template <typename T, int NGW>
struct Step {
  static constexpr int KPL = Io<T>::KPL;
  uint32_t xd[KPL];
  uint32_t bd[NGW][KPL];
  float w[KPL];
};

// Loads of k-step s. The lane's tokens are t = s*2*KPL + KPL*g + i. With
// FULL (every token of the chunk inside the sequence) the row term of each
// address is wave-uniform and goes in the scalar offset; otherwise the
// whole offset is in the vector operand, so rows past the sequence fall
// outside the resource and load as zeros.
template <typename T, int NGW, bool FULL>
__device__ __forceinline__ void load_step(Step<T, NGW>& st, int s, __amdgpu_buffer_rsrc_t rx,
                                          __amdgpu_buffer_rsrc_t rb, const float* wc, uint32_t xlane,
                                          uint32_t blane, uint32_t xsb, uint32_t bsb, int g) {
  constexpr int KPL = Io<T>::KPL, CGB = 32 * 4;   // bytes per column group
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const uint32_t trow = (uint32_t)(s * 2 * KPL + i);   // plus KPL*g, in the lane term
    if constexpr (FULL) {
      st.xd[i] = buf_load_dword(rx, xlane, trow * xsb);
#pragma unroll
      for (int j = 0; j < NGW; ++j) st.bd[j][i] = buf_load_dword(rb, blane + j * CGB, trow * bsb);
    } else {
      st.xd[i] = buf_load_dword(rx, xlane + trow * xsb, 0);
#pragma unroll
      for (int j = 0; j < NGW; ++j) st.bd[j][i] = buf_load_dword(rb, blane + j * CGB + trow * bsb, 0);
    }
  }
  const float* wp = wc + s * 2 * KPL + KPL * g;   // the workspace covers the padded chunk
  if constexpr (KPL % 4 == 0) {
#pragma unroll
    for (int i = 0; i < KPL; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(wp + i);
      st.w[i] = v.x; st.w[i + 1] = v.y; st.w[i + 2] = v.z; st.w[i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < KPL; ++i) st.w[i] = wp[i];
  }
}

template <typename T, int P, int N, int Q, bool FULL>
__device__ __forceinline__ void state_tile(const T* __restrict__ x, const T* __restrict__ Bm,
                                           const float* __restrict__ wst, float* __restrict__ states,
                                           int64_t Tlen, int H, int G, int64_t nc, int64_t Tp, int h, int k,
                                           int64_t b, int pg, int ng0, int m, int g) {
  using I = Io<T>;
  using Cfg = StateCfg<T, P, N>;
  constexpr int E = I::E, KPL = I::KPL, CG = Cfg::CG, NGW = Cfg::NGW;
  constexpr int KSTEPS = Q / (2 * KPL);
  constexpr int D = KPL == 1 ? 4 : 3;   // k-steps of loads in flight (ring of registers)
  static_assert(KPL != 1 || 8 % D == 0, "ring index must stay static under the partial unroll");

  const int grp = h / (H / G);
  const int64_t t0 = (int64_t)k * Q;
  const int nvalid = (int)(Tlen - t0 < Q ? Tlen - t0 : Q);
  const float* wc = wst + ((int64_t)b * H + h) * Tp + t0;
  const uint32_t xsb = (uint32_t)((int64_t)H * P * sizeof(T)), bsb = (uint32_t)((int64_t)G * N * sizeof(T));
  const T* xt = x + ((b * Tlen + t0) * H + h) * P + pg * CG;
  const T* bt = Bm + ((b * Tlen + t0) * G + grp) * N + ng0 * CG;
  // bytes the tile may read: rows 0..nvalid-1, each CG (x) or NGW*CG (B) columns
  const uint32_t xbytes = (uint32_t)(nvalid - 1) * xsb + CG * sizeof(T);
  const uint32_t bbytes = (uint32_t)(nvalid - 1) * bsb + NGW * CG * sizeof(T);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xt, xbytes), rb = make_rsrc(bt, bbytes);
  const uint32_t xlane = m * 4 + KPL * g * xsb, blane = m * 4 + KPL * g * bsb;

  f32x16 acc[E][NGW][E];
#pragma unroll
  for (int a = 0; a < E; ++a)
#pragma unroll
    for (int j = 0; j < NGW; ++j)
#pragma unroll
      for (int c = 0; c < E; ++c) acc[a][j][c] = f32x16{};

  Step<T, NGW> ring[D];
#pragma unroll
  for (int s = 0; s < D - 1; ++s)
    if (s < KSTEPS) load_step<T, NGW, FULL>(ring[s], s, rx, rb, wc, xlane, blane, xsb, bsb, g);
#pragma unroll (KPL == 1 ? 8 : KSTEPS)
  for (int s = 0; s < KSTEPS; ++s) {
    if (s + D - 1 < KSTEPS)   // in flight while this step's MFMAs run
      load_step<T, NGW, FULL>(ring[(s + D - 1) % D], s + D - 1, rx, rb, wc, xlane, blane, xsb, bsb, g);
    const Step<T, NGW>& cur = ring[s % D];
    typename I::Frag ahi[E], alo[E];
#pragma unroll
    for (int pe = 0; pe < E; ++pe) {
      float v[KPL];
#pragma unroll
      for (int i = 0; i < KPL; ++i) v[i] = cur.w[i] * I::elem(cur.xd[i], pe);
      I::split(v, ahi[pe], alo[pe]);
    }
#pragma unroll
    for (int j = 0; j < NGW; ++j)
#pragma unroll
      for (int ne = 0; ne < E; ++ne) {
        const typename I::Frag bf = I::from_dwords(cur.bd[j], ne);   // B is exact in the io dtype
#pragma unroll
        for (int pe = 0; pe < E; ++pe) {
          I::mma(acc[pe][j][ne], ahi[pe], bf);
          if constexpr (I::SPLIT) I::mma(acc[pe][j][ne], alo[pe], bf);
        }
      }
  }

  // S[p][n]: D row r -> p = pg*CG + E*drow(r, g) + pe, col -> n = (ng0+j)*CG + E*m + ne
  float* sb = states + (((int64_t)b * H + h) * nc + k) * (int64_t)(P * N);
#pragma unroll
  for (int pe = 0; pe < E; ++pe)
#pragma unroll
    for (int j = 0; j < NGW; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = pg * CG + E * drow(r, g) + pe;
        float* dst = sb + p * N + (ng0 + j) * CG + E * m;
        if constexpr (E == 2)
          *reinterpret_cast<float2*>(dst) = make_float2(acc[pe][j][0][r], acc[pe][j][1][r]);
        else
          *dst = acc[pe][j][0][r];
      }
}

template <typename T, int P, int N, int Q>
__global__ __launch_bounds__((StateCfg<T, P, N>::THREADS)) void ssd_chunk_state(
    const T* __restrict__ x, const T* __restrict__ Bm, const float* __restrict__ wst,
    float* __restrict__ states, int64_t Tlen, int H, int G, int64_t nc, int64_t Tp) {
  using Cfg = StateCfg<T, P, N>;
  // wave-uniform (scalar) wave index: the buffer resources built from it
  // must be provably uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int m = lane % 32, g = lane / 32;
  const int tile = wave / Cfg::WPT, sub = wave % Cfg::WPT;
  const int pg = sub / Cfg::NGS, ng0 = (sub % Cfg::NGS) * Cfg::NGW;
  const int h = blockIdx.x * Cfg::TPW + tile;
  if (h >= H) return;
  const int k = blockIdx.y;
  const int64_t b = blockIdx.z;
  if ((int64_t)(k + 1) * Q <= Tlen)
    state_tile<T, P, N, Q, true>(x, Bm, wst, states, Tlen, H, G, nc, Tp, h, k, b, pg, ng0, m, g);
  else
    state_tile<T, P, N, Q, false>(x, Bm, wst, states, Tlen, H, G, nc, Tp, h, k, b, pg, ng0, m, g);
}

// ---------------------------------------------------------------------------
// ssd_chunk_state_pass: the chunk states and the pass over them in one kernel
// (the structure of the blog's "Kernel 2: fwd_pass_state": one program walks
// a head's chunks in order, computes each chunk's contribution with an MMA
// and jumps the carried state over the chunk), for bf16 io with headdim 64.
// One wave owns one (batch, head, 64-column dstate group): it holds the state
// h for 64 x 64 entries in the MFMA accumulator layout, and for each chunk k
//   hprev[k] = h (as bf16 (hi, lo) pairs, the state pass's format),
//   S_k      = X_k^T (w o B_k)  (the tile product above, same operands),
//   h        = 2^(G'_last,k) h + S_k   (fmaf, as the state pass does),
// then writes final = h. The per-chunk states never reach memory: this
// saves writing and re-reading them (4 P N bytes each way per chunk). The
// loads of x, B and w run a ring of RING k-steps (16 tokens each) that
// continues across chunk boundaries; the ring size divides the k-steps of a
// chunk so every slot index stays static. The chunks of one head are
// sequential here, so this form needs many (batch, head) pairs to fill the
// GPU; the host takes it only then.
template <int N, int Q>
struct FusedCfg {
  static constexpr int P = 64, KSTEPS = Q / 16;
  static constexpr int HALF = KSTEPS / 2;     // k-steps per wave per chunk
  static constexpr int RING = 4;              // k-steps staged in LDS per wave
  static constexpr int NNG = N / 64;          // dstate groups per (batch, head)
  static_assert(KSTEPS == 16, "a wave stores its 16 hprev state rows over its 8 k-steps of a chunk");
};

// Direct global->LDS load of 16 bytes per lane from a wave-uniform base plus a
// per-lane offset; lane i's bytes land at lds + 16 i (lds wave-uniform, in M0).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// A workgroup of two waves per (batch, head, 64-column dstate group). Wave kh
// takes k-steps 8 kh .. 8 kh + 7 of every chunk (16 tokens each), so the
// chunk's product S_k is the sum of the two waves' partial sums. After a
// chunk, wave kh hands the other wave its partial sum of the state rows of
// parity 1 - kh through LDS and adds the other's partial of parity kh: each
// wave then holds S_k, and owns the state h, for the rows of its own parity
// (p = 2 drow(r, g) + kh), which it updates and stores to hprev. Each
// wave's 16-row steps of x (all 64 headdim columns) and B (the group's 64
// columns) go to its own RING LDS slots by four 1-KB direct loads, RING-1
// steps ahead, and each chunk's 256 weights w by one more. Within a slot, row
// r sits at row slot r ^ ((r >> 3) & 1), so the two half-waves of a dword
// read (rows 8g + i) hit different halves of the bank space. A wave stores
// hprev with one 16-byte store per lane per k-step, issued after that step's
// loads; so before step t is read, the operations issued after its loads
// number at least 1 + 5 (RING - 1) = 16 (12 for the first RING - 1 steps).
template <int N, int Q>
__global__ __launch_bounds__(128) void ssd_chunk_state_pass(
    const bf16* __restrict__ x, const bf16* __restrict__ Bm, const float* __restrict__ wst,
    const float* __restrict__ gcum, const float* init, void* __restrict__ hprev, float* final_state,
    int64_t Tlen, int H, int G, int64_t nc, int64_t Tp, int xcd) {
  using I = Io<bf16>;
  using Fc = FusedCfg<N, Q>;
  constexpr int P = 64, KPL = 8, HALF = Fc::HALF, RING = Fc::RING, NNG = Fc::NNG;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[2][RING][4096];   // per wave: x rows, then B rows
  __shared__ __attribute__((aligned(1024))) float wbuf[2][2][Q];                 // per wave, by chunk parity
  __shared__ __attribute__((aligned(1024))) float4 xch[2][8][64];                // partial sums handed over

  const int kh = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64, m = lane % 32, g = lane / 32;
  // workgroup -> (batch*head, dstate group). With xcd set (batch*heads a
  // multiple of 8), the groups of one head are 8 workgroups apart: the
  // dispatcher deals workgroups to the 8 XCDs in turn, so they run on the
  // same XCD at about the same time and the second read of the head's x
  // rows hits that XCD's L2.
  const int64_t wid = blockIdx.x;
  int ng;
  int64_t bh;
  if (xcd) {
    ng = (int)((wid / 8) % NNG);
    bh = (wid / (8 * NNG)) * 8 + wid % 8;
  } else {
    ng = (int)(wid % NNG);
    bh = wid / NNG;
  }
  const int h = (int)(bh % H);
  const int64_t b = bh / H;
  const int grp = h / (H / G);
  const uint32_t xsb = (uint32_t)H * P * 2, bsb = (uint32_t)G * N * 2;
  const int64_t nsteps = nc * HALF;   // this wave's k-steps over the walk
  // per-lane load offsets within a step: instruction q (rows 8q..8q+7 of the
  // step) puts lane l at row slot 8q + l/8, which holds row 8q + ((l/8) ^ q)
  const int rq0 = (lane >> 3), rq1 = 8 + ((lane >> 3) ^ 1);
  const uint32_t piece = (uint32_t)(lane & 7) * 16;
  // LDS read offsets: row 8g + i of a step sits at slot 8g + (i ^ g), i.e.
  // +1 slot for even i and -1 for odd i in the upper half-wave
  const int rde = (8 * g + g) * 128 + 4 * m, rdo = (8 * g - g) * 128 + 4 * m;

  // issue the loads of this wave's k-step t (chunk t / HALF, chunk step
  // 8 kh + t % HALF) into its slot, and at its first step of a chunk the
  // chunk's weights
  auto issue = [&](int64_t t) {
    const int64_t k = t / HALF;
    const int s = (int)(t - k * HALF) + HALF * kh;
    const int64_t t0 = k * Q;
    const int nv = (int)(Tlen - t0 < Q ? Tlen - t0 : Q);
    const unsigned char* xs = reinterpret_cast<const unsigned char*>(x + ((b * Tlen + t0) * H + h) * P);
    const unsigned char* bs = reinterpret_cast<const unsigned char*>(Bm + ((b * Tlen + t0) * G + grp) * N + ng * 64);
    unsigned char* slot = ring[kh][t % RING];
    if (s == HALF * kh) dma16(wst + bh * Tp + t0, (uint32_t)lane * 16, wbuf[kh][k & 1]);
    const int r0 = s * 16;
    if (r0 + 16 <= nv) {
      dma16(xs + (uint32_t)r0 * xsb, (uint32_t)rq0 * xsb + piece, slot);
      dma16(xs + (uint32_t)r0 * xsb, (uint32_t)rq1 * xsb + piece, slot + 1024);
      dma16(bs + (uint32_t)r0 * bsb, (uint32_t)rq0 * bsb + piece, slot + 2048);
      dma16(bs + (uint32_t)r0 * bsb, (uint32_t)rq1 * bsb + piece, slot + 3072);
    } else {
      // rows past the sequence: the last row again (finite; its weight is 0)
      const uint32_t a0 = (uint32_t)min(r0 + rq0, nv - 1), a1 = (uint32_t)min(r0 + rq1, nv - 1);
      dma16(xs, a0 * xsb + piece, slot);
      dma16(xs, a1 * xsb + piece, slot + 1024);
      dma16(bs, a0 * bsb + piece, slot + 2048);
      dma16(bs, a1 * bsb + piece, slot + 3072);
    }
  };

  // this wave's state rows: hs[ne][r], p = 2 drow(r, g) + kh, n = 64 ng + 2m + ne
  f32x16 hs[2];
  if (init) {
    const float* ip = init + bh * (int64_t)(P * N) + ng * 64 + 2 * m;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float2 v = *reinterpret_cast<const float2*>(ip + (2 * drow(r, g) + kh) * N);
      hs[0][r] = v.x;
      hs[1][r] = v.y;
    }
  } else {
    hs[0] = f32x16{};
    hs[1] = f32x16{};
  }
  // hprev[k] goes out through LDS: after each state update the wave writes
  // its 32 state rows (p = 2 j + kh, j = 0..31) as (hi, lo) pairs in the
  // stored format into its half of xch (one 256-byte row per j: column n of
  // the group at (n/8)*32 + (n%8)*2 bytes, lo 16 bytes after hi), and during
  // the next chunk each k-step stores 4 of these rows with one 16-byte store
  // per lane. In memory, row p of chunk k holds this group's columns in the
  // 256 bytes at p * 4N + 256 ng.
  unsigned char* stg = reinterpret_cast<unsigned char*>(xch[kh][0]);
  const uint32_t sw_off = (uint32_t)(m / 4) * 32 + (uint32_t)(m % 4) * 4;
  auto stage = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t d = pack_bf16x2(hs[0][r], hs[1][r]);
      const uint32_t lo = pack_bf16x2(hs[0][r] - bf16lo(d), hs[1][r] - bf16hi(d));
      unsigned char* row = stg + drow(r, g) * 256 + sw_off;
      *reinterpret_cast<uint32_t*>(row) = d;
      *reinterpret_cast<uint32_t*>(row + 16) = lo;
    }
  };
  const uint32_t st_row = (uint32_t)(lane >> 4), st_piece = (uint32_t)(lane & 15) * 16;
  unsigned char* hbase = static_cast<unsigned char*>(hprev) + bh * nc * (int64_t)(P * N) * 4;
  stage();

  for (int64_t t = 0; t < RING - 1 && t < nsteps; ++t) issue(t);
  if (init) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // h is complete before the first split

  for (int64_t k = 0; k < nc; ++k) {
    f32x16 acc[2][2];
#pragma unroll
    for (int pe = 0; pe < 2; ++pe)
#pragma unroll
      for (int ne = 0; ne < 2; ++ne) acc[pe][ne] = f32x16{};
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(hbase + k * (int64_t)(P * N) * 4, (uint32_t)(P * N * 4));
    const float* wk = wbuf[kh][k & 1] + HALF * kh * 16;
#pragma unroll
    for (int si = 0; si < HALF; ++si) {
      const int64_t t = k * HALF + si;
      // the slot refilled below was read one step ago
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (t + RING - 1 < nsteps) issue(t + RING - 1);
      // hprev[k] = h: staged rows j = 4 si .. 4 si + 3, 16 bytes per lane,
      // streamed (the next kernel reads them, long after they leave the caches)
      {
        const uint32_t j = (uint32_t)(4 * si) + st_row;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + j * 256 + st_piece);
        __builtin_amdgcn_raw_buffer_store_b128(v, rh, (2 * j + kh) * (4 * N) + ng * 256 + st_piece, 0, 2);
      }
      // step t has landed once the operations issued after it are outstanding at most
      if (t + RING - 1 >= nsteps) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      else if (t < RING - 1) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      const unsigned char* sb = ring[kh][t % RING];
      uint32_t xd[KPL], bd[KPL];
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        xd[i] = *reinterpret_cast<const uint32_t*>(sb + i * 128 + ((i & 1) ? rdo : rde));
        bd[i] = *reinterpret_cast<const uint32_t*>(sb + 2048 + i * 128 + ((i & 1) ? rdo : rde));
      }
      const float4 w0 = *reinterpret_cast<const float4*>(wk + si * 16 + 8 * g);
      const float4 w1 = *reinterpret_cast<const float4*>(wk + si * 16 + 8 * g + 4);
      const float wv[KPL] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      typename I::Frag ahi[2], alo[2];
#pragma unroll
      for (int pe = 0; pe < 2; ++pe) {
        float v[KPL];
#pragma unroll
        for (int i = 0; i < KPL; ++i) v[i] = wv[i] * I::elem(xd[i], pe);
        I::split(v, ahi[pe], alo[pe]);
      }
#pragma unroll
      for (int ne = 0; ne < 2; ++ne) {
        const typename I::Frag bf = I::from_dwords(bd, ne);
#pragma unroll
        for (int pe = 0; pe < 2; ++pe) {
          I::mma(acc[pe][ne], ahi[pe], bf);
          I::mma(acc[pe][ne], alo[pe], bf);
        }
      }
    }
    // hand over the partial sum of the other wave's rows, take ours
    // (fixed-index branches: a selected register index would go to scratch)
    float4* mine = xch[kh][0] + lane;
    const float4* theirs = xch[kh ^ 1][0] + lane;
    f32x16 part[2];
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ne = i / 4, r0 = (i % 4) * 4;
        mine[i * 64] = make_float4(acc[1][ne][r0], acc[1][ne][r0 + 1], acc[1][ne][r0 + 2], acc[1][ne][r0 + 3]);
      }
      part[0] = acc[0][0];
      part[1] = acc[0][1];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ne = i / 4, r0 = (i % 4) * 4;
        mine[i * 64] = make_float4(acc[0][ne][r0], acc[0][ne][r0 + 1], acc[0][ne][r0 + 2], acc[0][ne][r0 + 3]);
      }
      part[0] = acc[1][0];
      part[1] = acc[1][1];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ne = i / 4, r0 = (i % 4) * 4;
      const float4 o = theirs[i * 64];
      part[ne][r0] += o.x;
      part[ne][r0 + 1] += o.y;
      part[ne][r0 + 2] += o.z;
      part[ne][r0 + 3] += o.w;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // read before the next hand-over
    // h = 2^(G'_last,k) h + S_k
    const float sc = exp2_hw(gcum[bh * Tp + k * Q + (Q - 1)]);
#pragma unroll
    for (int ne = 0; ne < 2; ++ne)
#pragma unroll
      for (int r = 0; r < 16; ++r) hs[ne][r] = fmaf(sc, hs[ne][r], part[ne][r]);
    if (k + 1 < nc) stage();   // hprev[k + 1]; xch is free again after the second barrier
  }
  if (final_state) {
    float* fp = final_state + bh * (int64_t)(P * N) + ng * 64 + 2 * m;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      *reinterpret_cast<float2*>(fp + (2 * drow(r, g) + kh) * N) = make_float2(hs[0][r], hs[1][r]);
  }
}

template <int N, int Q>
hipError_t launch_fused(const Problem& p, hipStream_t stream) {
  const int64_t groups = p.bt * p.H * FusedCfg<N, Q>::NNG;
  const int xcd = (p.bt * p.H) % 8 == 0 ? 1 : 0;
  hipLaunchKernelGGL((ssd_chunk_state_pass<N, Q>), dim3((unsigned)groups), dim3(128), 0, stream, (const bf16*)p.x,
                     (const bf16*)p.B, p.wst, p.gcum, p.init, p.hprev, p.final_state, p.T, (int)p.H, (int)p.G,
                     p.nc, p.Tp, xcd);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// ssd_chunk_state_pass_rows: the same outputs as ssd_chunk_state_pass above,
// for bf16 io with dstate 128 or 256, any supported headdim and chunk. A
// workgroup owns one (batch, head, 128-column dstate slice); its
// P/16 waves each own 16 headdim rows and walk the chunks together, all of
// them reading the same x and B tiles from one LDS ring. For each chunk k a
// wave computes
//   hprev[k] = h   (bf16 (hi, lo) pairs, the state pass's format),
//   S_k^T    = B_k^T (w o X_k)   (128 dstate rows x 16 headdim columns),
//   h        = 2^(G'_last,k) h + S_k   (fmaf, as the state pass does),
// then writes final = h. The per-chunk states never reach memory.
//
// Operands. The 16x16x32 bf16 MFMA takes both operands from the ring through
// gfx950's transposing LDS read (ds_read_b64_tr_b16): the contraction index,
// the token, is the slow index of x and B in memory. The product is formed
// transposed, dstate as the MFMA rows and headdim as its columns, so a lane's
// four accumulator registers hold four consecutive dstate columns of one
// headdim row; a swap between neighbouring 16-lane rows (v_permlane16_swap)
// then gives each lane a whole 16-byte piece of the stored (hi, lo) format.
// The weight w_t is applied to x, each value once per wave, and w o x enters
// as a bf16 (hi, lo) pair in two MFMAs against the exact bf16 B
// (Io<bf16>::split). In a k-step of 32 tokens, lane group q = lane / 16 holds
// tokens 8 q .. 8 q + 7 in its k-slots, the MFMA's own layout.
//
// Ring. A k-step's slot holds the step's 32 x rows (2P bytes each), its 32 B
// rows of the workgroup's dstate slice (256 bytes each) and its 32 weights.
// The 32-byte segments of every row sit XOR-swizzled by row bits, so the
// eight rows a half-wave's transposing read touches land in eight different
// bank groups. Each wave loads its share of every step (one x piece, 8 / W
// B pieces and part of the weights) D - 1 steps ahead by direct global->LDS
// loads, waits for them, and a workgroup barrier per step makes every share
// visible and frees the slot read a step earlier. Past the end of the walk
// the waves load the last step again, into slots no one reads, so the vector
// memory operations a step issues depend only on its place in the chunk, and
// each wait count is a compile-time constant of that place (they complete in
// order).
template <int P, int Q>
struct SpCfg {
  static constexpr int W = P / 16;            // waves per workgroup
  static constexpr int KS = Q / 32;           // k-steps per chunk
  static constexpr int PPS = 8 / KS;          // hprev stores per wave per k-step (8 per chunk)
  // Headdim 128: a chunk's 8 hprev stores per wave go out together at its
  // first step, so each row's 512 bytes leave at once. Spread over the steps,
  // each step writing one 128-byte strip of 128 rows, the writes ran at half
  // the rate there (grouped wide-state layer 805 against 700 us); at headdim 64
  // (130M-like) the spread stores are faster (57 against 63 us).
  static constexpr bool BURST = P == 128;
  static constexpr int XRB = 2 * P;           // x row bytes
  static constexpr int XOFF = 0, BOFF = 32 * XRB, WOFF = BOFF + 32 * 256, SLOT = WOFF + 128;
  static constexpr int XL = 32 * XRB / 1024;  // x loads per step (one per wave)
  static constexpr int BL = 8 / W;            // B loads per wave per step
  static constexpr int LPS = 1 + BL + 1;      // loads per wave per step (x, B, w)
  static constexpr int D = P == 64 ? 6 : 4;   // ring slots
  // vector memory operations issued after a step's loads when it is waited
  // for, at the top of iteration s of a chunk: the loads of the D - 2
  // iterations after the one that issued them, and the stores of that
  // iteration and those D - 2 (PPS each, or 8 at each chunk start when the
  // stores go out together); for the steps loaded before the walk, at least
  // the loads of D - 2 issues
  static constexpr int VM_FIRST = (D - 2) * LPS;
  static constexpr int vm_at(int s) {
    int stores = 0;
    for (int u = s - (D - 1); u <= s - 1; ++u)
      stores += BURST ? ((((u % KS) + KS) % KS == 0) ? 8 : 0) : PPS;
    return (D - 2) * LPS + stores;
  }
  static_assert(XL == W, "one x load per wave per step");
  static_assert(KS >= 1 && 8 % KS == 0, "8 hprev stores per chunk");
  static_assert((D - 2) * LPS + (BURST ? 8 * ((D + KS - 2) / KS) : (D - 1) * PPS) <= 63, "vmcnt range");
  static_assert(D * SLOT <= 80 * 1024, "two workgroups per CU");
};

// 32-byte segment swizzle of a ring row: segment c of row r sits at c ^ f(r).
// Eight rows of a half-wave's transposing read (rows 8 q + 4 hh + 0..3 for
// q = 0, 1, or 2, 3) get eight different bank groups: in 256-byte rows the
// bank group is the position itself; in 128-byte rows it is the position
// plus 4 (r % 2).
__device__ __forceinline__ constexpr uint32_t swz256(uint32_t r) { return (r & 3) | ((r >> 1) & 4); }
__device__ __forceinline__ constexpr uint32_t swz128(uint32_t r) { return ((r >> 1) & 1) | ((r >> 2) & 2); }

template <int P, int N, int Q>
__global__ __launch_bounds__(64 * (P / 16)) void ssd_chunk_state_pass_rows(
    const bf16* __restrict__ x, const bf16* __restrict__ Bm, const float* __restrict__ wst,
    const float* __restrict__ gcum, const float* init, void* __restrict__ hprev, float* final_state,
    int64_t Tlen, int H, int G, int64_t nc, int64_t Tp, int xcd) {
  using Sc = SpCfg<P, Q>;
  using I = Io<bf16>;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int W = Sc::W, KS = Sc::KS, PPS = Sc::PPS, D = Sc::D, NG = N / 128, XRB = Sc::XRB;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[D][Sc::SLOT];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64, q = lane / 16, li = lane % 16;
  // workgroup -> (batch, group, head of the group, dstate slice). Every head
  // and slice of a (batch, group) reads the group's B rows; with xcd set
  // (batch * groups a multiple of 8) they take consecutive workgroup slots
  // of one XCD (the dispatcher deals workgroups to the 8 XCDs in turn), so
  // those rows, and each head's x rows for its second slice, come from that
  // XCD's L2.
  const int64_t wid = blockIdx.x, hpg = H / G, members = hpg * NG;
  int64_t set, member;
  if (xcd) {
    const int64_t j = wid / 8;
    member = j % members;
    set = (j / members) * 8 + wid % 8;
  } else {
    member = wid % members;
    set = wid / members;
  }
  const int ng = (int)(member % NG);
  const int grp = (int)(set % G);
  const int64_t b = set / G;
  const int h = (int)(grp * hpg + member / NG);
  const int64_t bh = b * H + h;
  const uint32_t xsb = (uint32_t)H * P * 2, bsb = (uint32_t)G * N * 2;
  const int64_t nsteps = nc * KS;
  const bf16* xs0 = x + (b * Tlen * H + h) * P;                 // token 0 of the head
  const bf16* bs0 = Bm + (b * Tlen * G + grp) * N + ng * 128;
  const float* ws0 = wst + bh * Tp;

  // this wave's loads of a step: x piece `wave` (rows 1024/XRB * wave ..),
  // B pieces BL * wave .. (4 rows each), weights 32/W floats
  constexpr int XRPL = 1024 / XRB;                               // x rows per load
  const uint32_t xr = (uint32_t)(XRPL * wave + lane / (XRB / 16));
  const uint32_t xps = (uint32_t)(lane % (XRB / 16));            // 16-byte LDS piece in the row
  const uint32_t xsw = P == 64 ? swz128(xr) : swz256(xr);
  const uint32_t xsrc = ((((xps >> 1) ^ xsw)) << 5) + ((xps & 1) << 4);
  const uint32_t bps = (uint32_t)(lane % 16);
  constexpr int WLANES = 8 / W;                                  // 16-byte weight pieces per wave
  auto issue = [&](int64_t u) {
    unsigned char* sp = ring[u % D];
    const int64_t tb = 32 * u;
    if (lane < WLANES) dma16(ws0 + tb + 4 * WLANES * wave, (uint32_t)lane * 16, sp + Sc::WOFF + 16 * WLANES * wave);
    if (tb + 32 <= Tlen) {
      dma16(xs0 + tb * H * P, xr * xsb + xsrc, sp + Sc::XOFF + 1024 * wave);
#pragma unroll
      for (int j = 0; j < Sc::BL; ++j) {
        const uint32_t br = (uint32_t)(4 * (Sc::BL * wave + j) + lane / 16);
        dma16(bs0 + tb * G * N, br * bsb + ((((bps >> 1) ^ swz256(br))) << 5) + ((bps & 1) << 4),
              sp + Sc::BOFF + 1024 * (Sc::BL * wave + j));
      }
    } else {
      // rows past the sequence: the last row again (finite; its weight is 0)
      const int64_t base = tb < Tlen - 1 ? tb : Tlen - 1;
      const int64_t rx = tb + xr < Tlen - 1 ? tb + xr : Tlen - 1;
      dma16(xs0 + base * H * P, (uint32_t)(rx - base) * xsb + xsrc, sp + Sc::XOFF + 1024 * wave);
#pragma unroll
      for (int j = 0; j < Sc::BL; ++j) {
        const uint32_t br = (uint32_t)(4 * (Sc::BL * wave + j) + lane / 16);
        const int64_t rb = tb + br < Tlen - 1 ? tb + br : Tlen - 1;
        dma16(bs0 + base * G * N, (uint32_t)(rb - base) * bsb + ((((bps >> 1) ^ swz256(br))) << 5) + ((bps & 1) << 4),
              sp + Sc::BOFF + 1024 * (Sc::BL * wave + j));
      }
    }
  };

  // transposing reads: lane supplies row 8 q + 4 hh + li / 4, columns
  // 16 c + 4 (li % 4) of 32-byte segment c (this wave's headdim segment for x,
  // dstate block jj for B)
  const uint32_t rr = (uint32_t)(8 * q + li / 4);                // row for hh = 0; hh = 1 adds 4
  const uint32_t col8 = (uint32_t)(li % 4) * 8;
  uint32_t xtr[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const uint32_t r = rr + 4 * hh;
    xtr[hh] = r * XRB + (((uint32_t)wave ^ (P == 64 ? swz128(r) : swz256(r))) << 5) + col8;
  }
  const uint32_t brow0 = rr * 256 + col8, bsw0 = swz256(rr), bsw1 = swz256(rr + 4);

  // the state: lane holds headdim row p = 16 wave + li and, in hs[jj][i],
  // dstate column 128 ng + 16 jj + 4 q + i
  const int p = 16 * wave + li;
  f32x4 hs[8];
  if (init) {
    const float* ip = init + bh * (int64_t)(P * N) + p * N + ng * 128 + 4 * q;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const float4 v = *reinterpret_cast<const float4*>(ip + 16 * jj);
      hs[jj] = f32x4{v.x, v.y, v.z, v.w};
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) hs[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  unsigned char* hbase = static_cast<unsigned char*>(hprev) + bh * nc * (int64_t)(P * N) * 4;
  // piece (jj, q / 2) of row p: dstate columns 128 ng + 16 jj + 8 (q / 2) ..
  // + 7; lane groups q = 0, 2 store its hi halves, q = 1, 3 its lo halves
  const uint32_t hrow = (uint32_t)p * (4 * N) + (uint32_t)(16 * ng + q / 2) * 32 + (uint32_t)(q % 2) * 16;
  // one block's piece of hprev[k] = h (the state entering the chunk)
  auto store_block = [&](__amdgpu_buffer_rsrc_t rh, int jj) {
    const uint32_t a0 = pack_bf16x2(hs[jj][0], hs[jj][1]);
    const uint32_t a1 = pack_bf16x2(hs[jj][2], hs[jj][3]);
    const uint32_t l0 = pack_bf16x2(hs[jj][0] - bf16lo(a0), hs[jj][1] - bf16hi(a0));
    const uint32_t l1 = pack_bf16x2(hs[jj][2] - bf16lo(a1), hs[jj][3] - bf16hi(a1));
    const auto s0 = __builtin_amdgcn_permlane16_swap(a0, l0, false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(a1, l1, false, false);
    const u32x4 vv = {s0[0], s1[0], s0[1], s1[1]};
    __builtin_amdgcn_raw_buffer_store_b128(vv, rh, hrow + (uint32_t)jj * 64, 0, 0);
  };

  for (int64_t u = 0; u < D - 1; ++u) issue(u < nsteps ? u : nsteps - 1);

  for (int64_t k = 0; k < nc; ++k) {
    f32x4 acc[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(hbase + k * (int64_t)(P * N) * 4, (uint32_t)(P * N * 4));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int64_t t = k * KS + s;
      // this wave's loads of step t have landed and its reads of step t - 1
      // are done; after the barrier, so are every wave's
      if (t < D - 1) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(Sc::VM_FIRST) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(Sc::vm_at(s)) : "memory");
      issue(t + D - 1 < nsteps ? t + D - 1 : nsteps - 1);
      if constexpr (Sc::BURST)
        if (s == 0) {
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) store_block(rh, jj);
        }
      const unsigned char* sp = ring[t % D];
      uint64_t x2[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        x2[hh] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                  (__attribute__((address_space(3))) s16x4*)(sp + Sc::XOFF + xtr[hh])));
      const float4 w0 = *reinterpret_cast<const float4*>(sp + Sc::WOFF + 32 * q);
      const float4 w1 = *reinterpret_cast<const float4*>(sp + Sc::WOFF + 32 * q + 16);
      bf16x8 bfr[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const uint64_t b0 = __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(sp + Sc::BOFF + brow0 + ((jj ^ bsw0) << 5))));
        const uint64_t b1 = __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(sp + Sc::BOFF + brow0 + 4 * 256 + ((jj ^ bsw1) << 5))));
        const u32x4 w4 = {(uint32_t)b0, (uint32_t)(b0 >> 32), (uint32_t)b1, (uint32_t)(b1 >> 32)};
        bfr[jj] = __builtin_bit_cast(bf16x8, w4);
      }
      const uint32_t xd[4] = {(uint32_t)x2[0], (uint32_t)(x2[0] >> 32), (uint32_t)x2[1], (uint32_t)(x2[1] >> 32)};
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = wv[e] * I::elem(xd[e / 2], e % 2);
      bf16x8 xhi, xlo;
      I::split(v, xhi, xlo);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) acc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[jj], xhi, acc[jj], 0, 0, 0);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) acc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[jj], xlo, acc[jj], 0, 0, 0);
      // hprev[k] = h: blocks s*PPS .. s*PPS + PPS - 1
      if constexpr (!Sc::BURST) {
#pragma unroll
        for (int i = 0; i < PPS; ++i) store_block(rh, s * PPS + i);
      }
    }
    // h = 2^(G'_last,k) h + S_k
    const float sc = exp2_hw(gcum[bh * Tp + k * Q + (Q - 1)]);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) hs[jj][i] = fmaf(sc, hs[jj][i], acc[jj][i]);
  }
  if (final_state) {
    float* fp = final_state + bh * (int64_t)(P * N) + p * N + ng * 128 + 4 * q;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      *reinterpret_cast<float4*>(fp + 16 * jj) = make_float4(hs[jj][0], hs[jj][1], hs[jj][2], hs[jj][3]);
  }
  // the ring's last loads land in this workgroup's LDS: they must finish before it exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int P, int N, int Q>
hipError_t launch_rows(const Problem& p, hipStream_t stream) {
  constexpr int NG = N / 128;
  const int64_t groups = p.bt * p.H * NG;
  const int xcd = (p.bt * p.G) % 8 == 0 ? 1 : 0;
  hipLaunchKernelGGL((ssd_chunk_state_pass_rows<P, N, Q>), dim3((unsigned)groups), dim3(64 * (P / 16)), 0, stream,
                     (const bf16*)p.x, (const bf16*)p.B, p.wst, p.gcum, p.init, p.hprev, p.final_state, p.T,
                     (int)p.H, (int)p.G, p.nc, p.Tp, xcd);
  return hipGetLastError();
}

template <typename T, int P, int N, int Q>
hipError_t launch_one(const Problem& p, hipStream_t stream) {
  using Cfg = StateCfg<T, P, N>;
  const dim3 grid((unsigned)((p.H + Cfg::TPW - 1) / Cfg::TPW), (unsigned)p.nc, (unsigned)p.bt);
  hipLaunchKernelGGL((ssd_chunk_state<T, P, N, Q>), grid, dim3(Cfg::THREADS), 0, stream, (const T*)p.x,
                     (const T*)p.B, p.wst, p.states, p.T, (int)p.H, (int)p.G, p.nc, p.Tp);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const Problem& p, hipStream_t s) {
#define SSD_CASE(PP, NN, QQ) \
  if (p.P == PP && p.N == NN && p.Q == QQ) return launch_one<T, PP, NN, QQ>(p, s);
#define SSD_Q(PP, NN) SSD_CASE(PP, NN, 64) SSD_CASE(PP, NN, 128) SSD_CASE(PP, NN, 256)
  SSD_Q(64, 64) SSD_Q(64, 128) SSD_Q(64, 256) SSD_Q(128, 64) SSD_Q(128, 128) SSD_Q(128, 256)
#undef SSD_Q
#undef SSD_CASE
  return hipErrorInvalidValue;
}

}  // namespace

bool chunk_state_has(int io, int64_t P, int64_t N, int64_t Q) {
  return (io == 0 || io == 1) && (P == 64 || P == 128) && (N == 64 || N == 128 || N == 256) &&
         (Q == 64 || Q == 128 || Q == 256);
}

hipError_t launch_chunk_state(const Problem& p, hipStream_t stream) {
  return p.io == 1 ? dispatch<bf16>(p, stream) : dispatch<float>(p, stream);
}

bool chunk_state_pass_fits(const Problem& p) {
  // bf16, at least one chunk; headdim 64 and chunk 256 (ssd_chunk_state_pass,
  // dstate 64, 128 or 256), or dstate 128 or 256 (ssd_chunk_state_pass_rows)
  if (p.io != 1 || p.nc <= 0) return false;
  return (p.P == 64 && p.Q == 256 && (p.N == 64 || p.N == 128 || p.N == 256)) ||
         ((p.P == 64 || p.P == 128) && (p.N == 128 || p.N == 256));
}

namespace {
// The two-wave form walks (batch, head, 64-column dstate group)s; it takes
// headdim 64, chunk 256 when those walks alone fill the GPU.
bool two_wave_form(const Problem& p) {
  return p.P == 64 && p.Q == 256 && (p.N == 64 || !(p.bt * p.H * (p.N / 64) < 512));
}
}  // namespace

bool chunk_state_pass_pays(const Problem& p) {
  // Each walk is sequential over the chunks, so the one-kernel forms need
  // many of them. Measured on MI355X (us, against ssd_chunk_state +
  // ssd_state_pass): two-wave form at the 2.7B-like layer (640 walks) 291
  // against 329; the row form with 192 (batch, head) workgroups (130M-like)
  // 58 against 63, with 256 (grouped wide state, headdim 128, dstate 256,
  // chunk 128) 821 against 1693, with 80 (long prefill) 1232 against 674.
  if (two_wave_form(p)) return p.bt * p.H * (p.N / 64) >= 512;
  return p.bt * p.H * (p.N / 128) >= 128;
}

hipError_t launch_chunk_state_pass(const Problem& p, hipStream_t stream) {
  if (two_wave_form(p)) {
#define SSD_CASE(NN, QQ) \
  if (p.N == NN && p.Q == QQ) return launch_fused<NN, QQ>(p, stream);
    SSD_CASE(64, 256) SSD_CASE(128, 256) SSD_CASE(256, 256)
#undef SSD_CASE
    return hipErrorInvalidValue;
  }
#define SSD_CASE(PP, NN, QQ) \
  if (p.P == PP && p.N == NN && p.Q == QQ) return launch_rows<PP, NN, QQ>(p, stream);
#define SSD_Q(PP, NN) SSD_CASE(PP, NN, 64) SSD_CASE(PP, NN, 128) SSD_CASE(PP, NN, 256)
  SSD_Q(64, 128) SSD_Q(64, 256) SSD_Q(128, 128) SSD_Q(128, 256)
#undef SSD_Q
#undef SSD_CASE
  return hipErrorInvalidValue;
}

}  // namespace ssd

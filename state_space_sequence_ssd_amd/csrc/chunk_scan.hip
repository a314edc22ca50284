// ssd_chunk_scan: the outputs of every chunk,
//
//   y[t, p] = 2^(G'_t) * sum_n C[t, n] * Hprev[p, n]
//           + sum_{j <= t} (sum_n C[t, n] B[j, n]) * 2^(G'_t - G'_j) * dt_j * x[j, p]
//           + D * x[t, p]
//
// i.e. Y = exp(G) o (C h^T) + (exp(G - G^T) o (C B^T) o M)(dt o X) + D X of
// the CUDA Tile Mamba-2 blog (section "Mamba-2 architecture", the decayed
// block output; section "Kernel 3: compute_out" fuses the three terms and
// keeps C.B^T out of global memory, as here).
//
// Work split. A workgroup owns one (batch, head, chunk) tile: Q rows t x
// headdim columns. The rows form Q/32 blocks of 32. A wave owns either the
// block pair {i, Q/32-1-i} (so every wave has the same number of causal
// (t-block, j-block) pairs) or, when two blocks' C fragments would not fit
// in registers, a single block; and one or more headdim column groups. Its
// accumulators hold those rows x columns in fp32.
//
// Flow:
//  1. Each wave loads the C rows of its t-blocks once as MFMA fragments
//     (contiguous along dstate); they are the B operand of C.B^T and the A
//     operand of the carried-state term. G' and dt of the chunk go to LDS.
//  2. acc = C . Hprev^T (MFMA over dstate), each row t then scaled by
//     2^(G'_t) <= 1. With bf16 io, Hprev arrives as the (hi, lo) bf16 pairs
//     ssd_state_pass wrote (two MFMAs against the exact bf16 C).
//  3. The chunk's tokens are walked in 32-token j-blocks. The block's B rows
//     and x rows are loaded once per workgroup into an LDS ring with direct
//     global->LDS loads (no registers involved), 2-3 blocks ahead of use;
//     one barrier per block. For each owned t-block >= j: CB^T = B . C^T for
//     the block (MFMA over dstate); its D layout gives lane l the column t =
//     l%32 and 16 rows j, exactly the lanes and registers the A operand of
//     the next product needs once the contraction index j is permuted to the
//     D row order (the x operand below uses the same order). The decay
//     2^(G'_t - G'_j) and dt_j are applied, the causal mask is a select (not a
//     multiply: entries above the diagonal can hold 2^(+large)), and with
//     bf16 io the result enters as a (hi, lo) bf16 pair in two MFMAs against
//     the exact bf16 x. On the diagonal block D*x is added from LDS.
//  4. y = acc rounded to the io dtype, one dword per lane per row (whole
//     128-byte rows per half-wave).
//
// Precision note: the blog rounds the carried state and the decayed matrix
// to the input type; where large terms cancel, that rounding alone breaks a
// 1e-2 + 2e-2|y| elementwise bound, so every MFMA operand that is not an
// input keeps about 16 significant bits here.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

template <typename T, int P, int N, int Q>
struct ScanCfg {
  static constexpr int E = Io<T>::E;
  static constexpr int KPL = Io<T>::KPL;
  static constexpr int CG = 32 * E;
  static constexpr int NPG = P / CG;                    // headdim column groups
  static constexpr int NTB = Q / 32;                    // 32-row blocks
  static constexpr int CF_VGPR = (N / (2 * KPL)) * (KPL == 8 ? 4 : 1);   // C fragments of one t-block
  static constexpr int TBW = (2 * CF_VGPR <= 64) ? 2 : 1;             // t-blocks per wave
  static constexpr int NTG = NTB / TBW;
  static constexpr int PGW0 = 64 / (TBW * E * 16);                    // keep 64 accumulators per wave
  static constexpr int PGW = PGW0 < 1 ? 1 : (PGW0 > NPG ? NPG : PGW0);
  static constexpr int NPS = NPG / PGW;
  static constexpr int WAVES = NTG * NPS;
  static constexpr int THREADS = 64 * WAVES;
  // j-block staging through LDS with direct global->LDS loads (16 bytes per
  // lane, lane i of a wave-instruction lands at base + 16 i): a block is the
  // 32 B rows followed by the 32 x rows, in 16-byte pieces.
  static constexpr int RB = N * (int)sizeof(T) / 16;    // pieces per B row
  static constexpr int RX = P * (int)sizeof(T) / 16;    // pieces per x row
  static constexpr int IB = 32 * RB / 64, IX = 32 * RX / 64;   // wave-instructions per block
  static constexpr int LB = (IB + WAVES - 1) / WAVES, LX = (IX + WAVES - 1) / WAVES;
  static constexpr int LOADS = LB + LX;                 // per wave per block
  static constexpr int BBYTES = 32 * RB * 16, XBYTES = 32 * RX * 16;
  static constexpr int BLOCK = BBYTES + XBYTES;
  static constexpr int NBUF = BLOCK <= 16384 ? 4 : 3;   // blocks in the LDS ring
  static_assert(NTB % TBW == 0 && NPG % PGW == 0, "tile split");
  static_assert(WAVES >= 1 && WAVES <= 8, "tile does not fit a workgroup");
  static_assert(RB >= 8 && RX >= 8, "row narrower than the swizzle");
};

// LDS placement (in 16-byte pieces) of B row m, piece c: the piece index is
// XORed with a row-dependent value so that the 16 lanes of one 16-byte
// fragment read (rows m..m+15, same piece) hit 16 different bank groups.
template <int RB>
__device__ __forceinline__ int bslot(int m, int c) {
  const int f = RB >= 16 ? (m & 15) : ((m >> 1) & (RB - 1));
  return m * RB + (c ^ f);
}
// x rows: the two half-waves read rows j and j+4 of the same columns; rows
// with bit 2 set are moved to the other half of the banks (for 8-piece rows
// by swapping row parity, for wider rows by XORing the piece with 8).
template <int RX>
__device__ __forceinline__ int xslot(int j, int c) {
  const int b2 = (j >> 2) & 1;
  if constexpr (RX == 8)
    return (j ^ b2) * 8 + c;
  else
    return j * RX + (c ^ (b2 << 3));
}

// Wait until at most VM vector-memory operations of this wave are in flight
// and its LDS operations are done, then meet the workgroup at the barrier.
// The memory clobber keeps the compiler from moving LDS accesses across it.
template <int VM>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}

// Direct global->LDS loads of j-block jb (B rows, then x rows) into one ring
// slot. Every wave issues LB + LX 16-byte-per-lane loads; instruction kk
// fills LDS bytes [kk*1024, kk*1024 + 1024) of its part, lane i the 16 bytes
// at kk*1024 + 16 i, so the global piece each lane fetches is chosen to
// realise the swizzled placement of bslot / xslot. Rows past the sequence are
// clamped to its last row (a valid address); their products are masked out by
// the caller. `wave` must be wave-uniform (it feeds the LDS address in M0).
template <typename Cfg, typename T>
__device__ __forceinline__ void issue_block(unsigned char* slot_base, const T* bbase, const T* xbase,
                                            int64_t brow, int64_t xrow, int jb, int nvalid, int wave, int lane) {
  constexpr int RB = Cfg::RB, RX = Cfg::RX, EPC = 16 / (int)sizeof(T);
#pragma unroll
  for (int i = 0; i < Cfg::LB; ++i) {
    const int kk = (wave + i * Cfg::WAVES) % Cfg::IB;   // spare instructions repeat a piece
    const int s = kk * 64 + lane;
    const int mr = s / RB, pc = s % RB;
    const int f = RB >= 16 ? (mr & 15) : ((mr >> 1) & (RB - 1));
    const int row = min(jb * 32 + mr, nvalid - 1);
    __builtin_amdgcn_global_load_lds(bbase + row * brow + (pc ^ f) * EPC, slot_base + kk * 1024, 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < Cfg::LX; ++i) {
    const int kk = (wave + i * Cfg::WAVES) % Cfg::IX;
    const int s = kk * 64 + lane;
    const int pr = s / RX, pc = s % RX;
    const int b2 = (pr >> 2) & 1;
    const int jr = RX == 8 ? (pr ^ b2) : pr;
    const int c = RX == 8 ? pc : (pc ^ (b2 << 3));
    const int row = min(jb * 32 + jr, nvalid - 1);
    __builtin_amdgcn_global_load_lds(xbase + row * xrow + c * EPC, slot_base + Cfg::BBYTES + kk * 1024, 16, 0, 0);
  }
}

template <typename T, int P, int N, int Q>
__global__ __launch_bounds__((ScanCfg<T, P, N, Q>::THREADS)) __attribute__((amdgpu_waves_per_eu(2)))
void ssd_chunk_scan(const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
                    const float* __restrict__ gcum, const float* __restrict__ dtt, const float* __restrict__ Dp,
                    const void* __restrict__ hprev, T* __restrict__ y, int64_t Tlen, int H, int G, int64_t nc,
                    int64_t Tp) {
  using I = Io<T>;
  using Frag = typename I::Frag;
  using Cfg = ScanCfg<T, P, N, Q>;
  constexpr int E = I::E, KPL = I::KPL, CG = Cfg::CG, NTB = Cfg::NTB, TBW = Cfg::TBW;
  constexpr int PGW = Cfg::PGW, NPS = Cfg::NPS, WAVES = Cfg::WAVES;
  constexpr int RB = Cfg::RB, RX = Cfg::RX, NBUF = Cfg::NBUF, LOADS = Cfg::LOADS;
  constexpr int KS = N / (2 * KPL);    // MFMA steps over dstate
  constexpr int JS = 32 / (2 * KPL);   // MFMA steps over a 32-token j-block
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte piece

  __shared__ __attribute__((aligned(16))) unsigned char ring[NBUF][Cfg::BLOCK];
  __shared__ __attribute__((aligned(16))) float sG[Q];
  __shared__ __attribute__((aligned(16))) float sDt[Q];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int m = lane % 32, g = lane / 32;
  const int tg = wave / NPS, pg0 = (wave % NPS) * PGW;
  int tbs[TBW];
  tbs[0] = tg;
  if constexpr (TBW == 2) tbs[1] = NTB - 1 - tg;
  const int h = blockIdx.x;
  const int k = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int grp = h / (H / G);
  const int64_t t0 = (int64_t)k * Q;
  const int nvalid = (int)(Tlen - t0 < Q ? Tlen - t0 : Q);   // >= 1

  const float* gc = gcum + ((int64_t)b * H + h) * Tp + t0;
  const float* dtc = dtt + ((int64_t)b * H + h) * Tp + t0;
  const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N;
  const T* xbase = x + ((b * Tlen + t0) * H + h) * P;
  T* ybase = y + ((b * Tlen + t0) * H + h) * P;
  const T* bbase = Bm + ((b * Tlen + t0) * G + grp) * N;
  const T* cbase = Cm + ((b * Tlen + t0) * G + grp) * N;
  const int64_t hoff = (((int64_t)b * H + h) * nc + k) * (int64_t)(P * N);

  // 1. C fragments of the wave's t-blocks: row t = 32*tb + m, dstate k-step s
  Frag cf[TBW][KS];
#pragma unroll
  for (int u = 0; u < TBW; ++u) {
    const int t = tbs[u] * 32 + m;
    const bool valid = t < nvalid;
#pragma unroll
    for (int s = 0; s < KS; ++s) cf[u][s] = I::load_row(cbase + t * brow + s * 2 * KPL + KPL * g, valid);
  }
  for (int i = tid; i < Q; i += 64 * WAVES) {
    sG[i] = gc[i];
    sDt[i] = dtc[i];
  }

  // 2. carried state: acc[u][q][pe] = C . Hprev^T, col -> p = (pg0+q)*CG + E*m + pe
  f32x16 acc[TBW][PGW][E];
#pragma unroll
  for (int u = 0; u < TBW; ++u)
#pragma unroll
    for (int q = 0; q < PGW; ++q)
#pragma unroll
      for (int pe = 0; pe < E; ++pe) acc[u][q][pe] = f32x16{};
#pragma unroll
  for (int q = 0; q < PGW; ++q)
#pragma unroll
    for (int pe = 0; pe < E; ++pe) {
      const int p = (pg0 + q) * CG + E * m + pe;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Frag hhi, hlo;
        if constexpr (I::SPLIT) {
          // (hi, lo) pairs: 8 hi then 8 lo bf16 per aligned group of 8 columns
          const bf16* hp = static_cast<const bf16*>(hprev) + 2 * hoff + (int64_t)p * 2 * N + (2 * s + g) * 16;
          hhi = I::load_row(reinterpret_cast<const T*>(hp), true);
          hlo = I::load_row(reinterpret_cast<const T*>(hp + 8), true);
        } else {
          hhi = I::load_row(static_cast<const T*>(hprev) + hoff + (int64_t)p * N + s * 2 * KPL + KPL * g, true);
        }
#pragma unroll
        for (int u = 0; u < TBW; ++u) {
          I::mma(acc[u][q][pe], cf[u][s], hhi);
          if constexpr (I::SPLIT) I::mma(acc[u][q][pe], cf[u][s], hlo);
        }
      }
    }

  // the first NBUF-1 j-blocks go in flight now (issued after the C and Hprev
  // loads, so waiting for those does not wait for these)
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    if (i < NTB) issue_block<Cfg>(ring[i], bbase, xbase, brow, xrow, i, nvalid, wave, lane);

  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // sG, sDt visible
#pragma unroll
  for (int u = 0; u < TBW; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float sc = exp2_hw(sG[tbs[u] * 32 + drow(r, g)]);
#pragma unroll
      for (int q = 0; q < PGW; ++q)
#pragma unroll
        for (int pe = 0; pe < E; ++pe) acc[u][q][pe][r] *= sc;
    }

  // 3. intra-chunk, causal over 32-token j-blocks
  float gt[TBW];
#pragma unroll
  for (int u = 0; u < TBW; ++u) gt[u] = sG[tbs[u] * 32 + m];
  const float Dh = Dp[h];
  int tmax = tbs[0];
  if constexpr (TBW == 2) tmax = tbs[1];

  for (int jb = 0; jb < NTB; ++jb) {
    // block jb has landed once at most (blocks issued after it) x LOADS remain
    const int after = NTB - 1 - jb < NBUF - 2 ? NTB - 1 - jb : NBUF - 2;
    if (after <= 0) wait_vm_barrier<0>();
    else if (after == 1) wait_vm_barrier<LOADS>();
    else wait_vm_barrier<2 * LOADS>();
    if (jb + NBUF - 1 < NTB)
      issue_block<Cfg>(ring[(jb + NBUF - 1) % NBUF], bbase, xbase, brow, xrow, jb + NBUF - 1, nvalid, wave, lane);
    if (jb > tmax) continue;

    const unsigned char* sb = ring[jb % NBUF];
    const unsigned char* sx = sb + Cfg::BBYTES;
    const int j0 = jb * 32;
    const float* gjb = sG + j0;
    const float* djb = sDt + j0;
#pragma unroll
    for (int u = 0; u < TBW; ++u) {
      const int tb = tbs[u];
      if (tb < jb) continue;
      // CB^T for (j-block, t-block): A = B rows j (from LDS), B operand = C^T
      f32x16 cb = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int byte = (s * 2 * KPL + KPL * g) * (int)sizeof(T);
        const Frag bfr = *reinterpret_cast<const Frag*>(sb + bslot<RB>(m, byte / 16) * 16 + byte % 16);
        I::mma(cb, bfr, cf[u][s]);
      }
      // decay, dt, causal mask (and rows past the sequence), as a select
      float v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int jr = drow(q, g);
        const bool keep = ((tb > jb) || (m >= jr)) && (j0 + jr < nvalid);
        const float val = cb[q] * exp2_hw(gt[u] - gjb[jr]) * djb[jr];
        v[q] = keep ? val : 0.f;
      }
#pragma unroll
      for (int js = 0; js < JS; ++js) {
        Frag ahi, alo;
        I::split(&v[js * KPL], ahi, alo);
#pragma unroll
        for (int q = 0; q < PGW; ++q) {
          // x rows of this step, exact in the io dtype, in the same permuted j order
          const int byte = ((pg0 + q) * CG + E * m) * (int)sizeof(T);
          uint32_t d[KPL];
#pragma unroll
          for (int i = 0; i < KPL; ++i)
            d[i] = *reinterpret_cast<const uint32_t*>(sx + xslot<RX>(drow(js * KPL + i, g), byte / 16) * 16 +
                                                      byte % 16);
#pragma unroll
          for (int pe = 0; pe < E; ++pe) {
            const Frag xf = I::from_dwords(d, pe);
            I::mma(acc[u][q][pe], ahi, xf);
            if constexpr (I::SPLIT) I::mma(acc[u][q][pe], alo, xf);
          }
        }
      }
      if (tb == jb) {
        // D x for the block's own rows, from the staged x rows
#pragma unroll
        for (int q = 0; q < PGW; ++q) {
          const int byte = ((pg0 + q) * CG + E * m) * (int)sizeof(T);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t xd =
                *reinterpret_cast<const uint32_t*>(sx + xslot<RX>(drow(r, g), byte / 16) * 16 + byte % 16);
#pragma unroll
            for (int pe = 0; pe < E; ++pe) acc[u][q][pe][r] += Dh * I::elem(xd, pe);
          }
        }
      }
    }
  }

  // 4. y
#pragma unroll
  for (int u = 0; u < TBW; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = tbs[u] * 32 + drow(r, g);
      if (t < nvalid) {
#pragma unroll
        for (int q = 0; q < PGW; ++q)
          I::store_pair(ybase + t * xrow + (pg0 + q) * CG + E * m, acc[u][q][0][r], acc[u][q][E - 1][r]);
      }
    }
}

template <typename T, int P, int N, int Q>
hipError_t launch_one(const Problem& p, hipStream_t stream) {
  using Cfg = ScanCfg<T, P, N, Q>;
  const dim3 grid((unsigned)p.H, (unsigned)p.nc, (unsigned)p.bt);
  hipLaunchKernelGGL((ssd_chunk_scan<T, P, N, Q>), grid, dim3(Cfg::THREADS), 0, stream, (const T*)p.x,
                     (const T*)p.B, (const T*)p.C, p.gcum, p.dtt, p.D, (const void*)p.hprev, (T*)p.y, p.T,
                     (int)p.H, (int)p.G, p.nc, p.Tp);
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

bool chunk_scan_has(int io, int64_t P, int64_t N, int64_t Q) {
  return (io == 0 || io == 1) && (P == 64 || P == 128) && (N == 64 || N == 128 || N == 256) &&
         (Q == 64 || Q == 128 || Q == 256);
}

hipError_t launch_chunk_scan(const Problem& p, hipStream_t stream) {
  return p.io == 1 ? dispatch<bf16>(p, stream) : dispatch<float>(p, stream);
}

}  // namespace ssd

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
  // j-block staging: direct global->LDS loads, 16 bytes per lane, lane i of
  // a wave-instruction landing at base + 16 i. A block holds its 32 B rows
  // padded to RB+1 pieces (16 bytes each) and its 32 x rows padded to RX+2
  // pieces; pad pieces receive a copy of a real piece and are never read.
  // With those strides the 16 lanes of a 16-byte B fragment read (rows
  // m..m+15) and the two half-waves of a dword x read (rows j and j+4) fall
  // on distinct LDS banks, and every read address is a per-lane base plus a
  // compile-time offset.
  static constexpr int RB = N * (int)sizeof(T) / 16;    // pieces per B row
  static constexpr int RX = P * (int)sizeof(T) / 16;    // pieces per x row
  static constexpr int BROWP = RB + 1, XROWP = RX + 2;  // padded row strides, in pieces
  static constexpr int IB = (32 * BROWP + 63) / 64, IX = (32 * XROWP + 63) / 64;   // wave-instructions
  static constexpr int ITOT = IB + IX;
  static constexpr int LOADS = (ITOT + WAVES - 1) / WAVES;   // per wave per block (spares repeat)
  static constexpr int BBYTES = IB * 1024, XBYTES = IX * 1024;
  // per-lane load offsets kept in registers for whole-chunk blocks (see
  // plan_block) only when they are few; otherwise each block recomputes them
  static constexpr bool PLAN = LOADS <= 4;
  static constexpr int BLOCK = BBYTES + XBYTES;
  // The carried state Hprev (P rows of 4N bytes: fp32, or the bf16 (hi, lo)
  // pairs) is the B operand every wave needs in full. When it fits, it is
  // brought into LDS once per workgroup by direct loads, its rows reordered
  // so that the 16 lanes of a fragment read hit distinct banks; otherwise
  // each wave loads it from global memory.
  static constexpr int HROWP = N / 4 + 1;                // padded row, in 16-byte pieces
  static constexpr int HBYTES = P * HROWP * 16;
  static constexpr bool HLDS = HBYTES <= 36 * 1024;
  static constexpr int IH = HLDS ? (HBYTES + 1023) / 1024 : 0;
  static constexpr int HLOADS = (IH + WAVES - 1) / WAVES;   // per wave (spares repeat)
  static constexpr int HALLOC = HLDS ? IH * 1024 : 16;
  static constexpr int NBUF = HLDS ? 3 : (BLOCK <= 16384 ? 4 : 3);   // blocks in the LDS ring
  // Otherwise, with bf16 (hi, lo) Hprev, the carried-state product streams
  // Hprev through the ring in pieces of two MFMA k-steps (32 dstate columns:
  // 128 bytes of each row), read once per workgroup: slot rows of 144 bytes
  // (one 16-byte pad piece) in the row order of the HLDS case, so the 16
  // lanes of a fragment read hit 16 distinct bank groups.
  static constexpr bool STAGE = !HLDS && E == 2;
  static constexpr int SROW = 144;                       // slot row bytes: 8 data pieces + 1 pad
  static constexpr int NPC = N / 32;                     // pieces (two k-steps each)
  static constexpr int IHP = P * 9 / 64;                 // wave-instructions per piece
  static constexpr int HPL = (IHP + WAVES - 1) / WAVES;  // per wave (spares repeat)
  static_assert(NTB % TBW == 0 && NPG % PGW == 0, "tile split");
  static_assert(!STAGE || (NBUF == 3 && P * SROW <= BLOCK && (P * 9) % 64 == 0 && NTB >= 2), "staged Hprev pieces");
  static_assert(WAVES >= 1 && WAVES <= 8, "tile does not fit a workgroup");
};

// Wait until at most VM vector-memory operations of this wave are in flight
// and its LDS operations are done, then meet the workgroup at the barrier.
// The memory clobber keeps the compiler from moving LDS accesses across it.
template <int VM>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}

// Direct global->LDS loads of j-block jb into one ring slot: LOADS
// wave-instructions per wave; instruction kk (0 <= kk < ITOT) fills bytes
// [kk*1024, kk*1024 + 1024) of the slot, lane i the 16 bytes at kk*1024 +
// 16 i, so each lane fetches the global piece that belongs at its slot.
// Rows past the sequence are clamped to its last row (a valid address): those
// tokens have dt = 0 in the workspace, which zeroes their products. `wave`
// must be wave-uniform (it feeds the LDS address in M0).
template <typename Cfg, typename T>
__device__ __forceinline__ void issue_block(unsigned char* slot_base, const T* bbase, const T* xbase,
                                            int64_t brow, int64_t xrow, int jb, int nvalid, int wave, int lane) {
  constexpr int EPC = 16 / (int)sizeof(T);
#pragma unroll
  for (int i = 0; i < Cfg::LOADS; ++i) {
    const int kk = (wave + i * Cfg::WAVES) % Cfg::ITOT;   // spare instructions repeat one
    if (kk < Cfg::IB) {
      const int s = kk * 64 + lane;
      int r = s / Cfg::BROWP, c = s % Cfg::BROWP;
      if (r >= 32) r = 31;            // tail of the last instruction
      if (c >= Cfg::RB) c = 0;        // pad piece
      const int row = min(jb * 32 + r, nvalid - 1);
      lds_dma16(bbase + row * brow + c * EPC, slot_base + kk * 1024);
    } else {
      const int kx = kk - Cfg::IB;
      const int s = kx * 64 + lane;
      int r = s / Cfg::XROWP, c = s % Cfg::XROWP;
      if (r >= 32) r = 31;
      if (c >= Cfg::RX) c = 0;
      const int row = min(jb * 32 + r, nvalid - 1);
      lds_dma16(xbase + row * xrow + c * EPC, slot_base + Cfg::BBYTES + kx * 1024);
    }
  }
}

// The same loads for a j-block whose 32 rows all lie inside the sequence:
// `off` holds, per load instruction, this lane's byte offset from the
// block's first row (fixed for the whole chunk, see plan_block), and the
// block base is wave-uniform, so each load is a scalar base plus a vector
// offset with no per-block address arithmetic.
template <typename Cfg, typename T>
__device__ __forceinline__ void plan_block(uint32_t* off, int64_t brow, int64_t xrow, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < Cfg::LOADS; ++i) {
    const int kk = (wave + i * Cfg::WAVES) % Cfg::ITOT;
    const bool isb = kk < Cfg::IB;
    const int s = (isb ? kk : kk - Cfg::IB) * 64 + lane;
    const int rowp = isb ? Cfg::BROWP : Cfg::XROWP, rdat = isb ? Cfg::RB : Cfg::RX;
    int r = s / rowp, c = s % rowp;
    if (r >= 32) r = 31;     // tail of the last instruction
    if (c >= rdat) c = 0;    // pad piece
    off[i] = (uint32_t)(r * (isb ? brow : xrow) * (int64_t)sizeof(T) + c * 16);
  }
}

template <typename Cfg>
__device__ __forceinline__ void issue_block_full(unsigned char* slot_base, const unsigned char* bblk,
                                                 const unsigned char* xblk, const uint32_t* off, int wave) {
#pragma unroll
  for (int i = 0; i < Cfg::LOADS; ++i) {
    const int kk = (wave + i * Cfg::WAVES) % Cfg::ITOT;
    if (kk < Cfg::IB)
      lds_dma16(bblk + off[i], slot_base + kk * 1024);
    else
      lds_dma16(xblk + off[i], slot_base + Cfg::BBYTES + (kk - Cfg::IB) * 1024);
  }
}

// Per-lane (row, byte column) of each of the wave's LOADS load instructions
// within a j-block, packed as row << 16 | column byte offset (see
// issue_block for the slot layout).
template <typename Cfg>
__device__ __forceinline__ void plan_block_rc(uint32_t* rc, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < Cfg::LOADS; ++i) {
    const int kk = (wave + i * Cfg::WAVES) % Cfg::ITOT;
    const bool isb = kk < Cfg::IB;
    const int s = (isb ? kk : kk - Cfg::IB) * 64 + lane;
    const int rowp = isb ? Cfg::BROWP : Cfg::XROWP, rdat = isb ? Cfg::RB : Cfg::RX;
    int r = s / rowp, c = s % rowp;
    if (r >= 32) r = 31;     // tail of the last instruction
    if (c >= rdat) c = 0;    // pad piece
    rc[i] = (uint32_t)(r << 16) | (uint32_t)(c * 16);
  }
}

// issue_block from a plan: bt and xt are the tile's first B and x rows (as
// bytes), bsb and xsb their row strides in bytes; rows past the sequence are
// clamped to its last row, as in issue_block. Offsets are 32-bit (one chunk
// of x spans less than 2 GiB).
template <typename Cfg>
__device__ __forceinline__ void issue_block_rc(unsigned char* slot_base, const unsigned char* bt,
                                               const unsigned char* xt, uint32_t bsb, uint32_t xsb,
                                               const uint32_t* rc, int jb, int nvalid, int wave) {
#pragma unroll
  for (int i = 0; i < Cfg::LOADS; ++i) {
    const int kk = (wave + i * Cfg::WAVES) % Cfg::ITOT;
    const int row = min(jb * 32 + (int)(rc[i] >> 16), nvalid - 1);
    if (kk < Cfg::IB)
      lds_dma16(bt + ((uint32_t)row * bsb + (rc[i] & 0xffffu)), slot_base + kk * 1024);
    else
      lds_dma16(xt + ((uint32_t)row * xsb + (rc[i] & 0xffffu)), slot_base + Cfg::BBYTES + (kk - Cfg::IB) * 1024);
  }
}

// Direct global->LDS loads of the chunk's Hprev (HLDS case). LDS row slot r
// holds headdim row p: with two bf16 columns per dword (E = 2) slot
// q*64 + pe*32 + m holds p = q*64 + 2m + pe, so the lanes of one fragment
// read (consecutive m) read consecutive slots; with fp32, slot p holds p.
template <typename Cfg, typename T>
__device__ __forceinline__ void issue_hprev(unsigned char* dst, const unsigned char* hsrc, int wave, int lane) {
  constexpr int HROWP = Cfg::HROWP, P = Cfg::NPG * Cfg::CG;
  constexpr int ROWB = (HROWP - 1) * 16;   // 4N bytes of data per row
#pragma unroll
  for (int i = 0; i < Cfg::HLOADS; ++i) {
    const int kk = (wave + i * Cfg::WAVES) % Cfg::IH;
    const int s = kk * 64 + lane;
    int r = s / HROWP, c = s % HROWP;
    if (r >= P) r = P - 1;        // tail of the last instruction
    if (c >= HROWP - 1) c = 0;    // pad piece
    int p = r;
    if constexpr (Cfg::E == 2) p = (r / 64) * 64 + 2 * (r % 32) + (r / 32) % 2;
    lds_dma16(hsrc + (int64_t)p * ROWB + c * 16, dst + kk * 1024);
  }
}

// Direct global->LDS loads of Hprev piece c (dstate columns 32 c .. 32 c + 31
// of every headdim row, bf16 (hi, lo) pairs: bytes 128 c .. 128 c + 127 of
// each 4N-byte row) into a ring slot: slot row r (144 bytes) holds headdim
// row (r / 64) * 64 + 2 (r % 32) + (r / 32) % 2, its ninth piece a copy of
// the first (never read).
template <typename Cfg>
__device__ __forceinline__ void issue_hpiece(unsigned char* dst, const unsigned char* hsrc, int c, int wave,
                                             int lane) {
  constexpr int ROWB = (Cfg::HROWP - 1) * 16;
#pragma unroll
  for (int i = 0; i < Cfg::HPL; ++i) {
    const int kk = (wave + i * Cfg::WAVES) % Cfg::IHP;
    const int s = kk * 64 + lane;
    const int r = s / 9;
    int pc = s % 9;
    if (pc == 8) pc = 0;   // pad piece
    const int p = (r / 64) * 64 + 2 * (r % 32) + (r / 32) % 2;
    lds_dma16(hsrc + (int64_t)p * ROWB + c * 128 + pc * 16, dst + kk * 1024);
  }
}

template <typename T, int P, int N, int Q>
__global__ __launch_bounds__((ScanCfg<T, P, N, Q>::THREADS)) __attribute__((amdgpu_waves_per_eu(2)))
void ssd_chunk_scan(const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
                    const float* __restrict__ gcum, const float* __restrict__ dtt, const float* __restrict__ Dp,
                    const void* __restrict__ hprev, T* __restrict__ y, int64_t Tlen, int H, int G, int64_t nc,
                    int64_t Tp, int xcd) {
  using I = Io<T>;
  using Frag = typename I::Frag;
  using Cfg = ScanCfg<T, P, N, Q>;
  static_assert(!Cfg::HLDS, "Hprev that fits in LDS takes the persistent form below");
  constexpr int E = I::E, KPL = I::KPL, CG = Cfg::CG, NTB = Cfg::NTB, TBW = Cfg::TBW;
  constexpr int PGW = Cfg::PGW, NPS = Cfg::NPS, WAVES = Cfg::WAVES;
  constexpr int NBUF = Cfg::NBUF, LOADS = Cfg::LOADS;
  constexpr int BRB = Cfg::BROWP * 16, XRB = Cfg::XROWP * 16;   // padded row bytes
  constexpr int KS = N / (2 * KPL);    // MFMA steps over dstate
  constexpr int JS = 32 / (2 * KPL);   // MFMA steps over a 32-token j-block

  __shared__ __attribute__((aligned(16))) unsigned char ring[NBUF][Cfg::BLOCK];
  __shared__ __attribute__((aligned(16))) float sG[Q];
  __shared__ __attribute__((aligned(16))) float sDt[Q];
  __shared__ __attribute__((aligned(16))) float sW[Q];   // dt_j * 2^(G'_end(block of j) - G'_j) <= dt_j

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int m = lane % 32, g = lane / 32;
  const int tg = wave / NPS, pg0 = (wave % NPS) * PGW;
  int tbs[TBW];
  tbs[0] = tg;
  if constexpr (TBW == 2) tbs[1] = NTB - 1 - tg;
  // workgroup -> (batch, chunk, head). The heads of one group read the same
  // B and C rows; with xcd set (batch * chunks * groups a multiple of 8) a
  // group's heads take consecutive workgroup slots of one XCD (the
  // dispatcher deals workgroups to the 8 XCDs in turn), so those rows come
  // from that XCD's L2 after the first head.
  const int64_t L = blockIdx.x, hpg = H / G;
  int64_t set, member;
  if (xcd) {
    const int64_t j = L / 8;
    member = j % hpg;
    set = (j / hpg) * 8 + L % 8;
  } else {
    member = L % hpg;
    set = L / hpg;
  }
  const int h = (int)((set % G) * hpg + member);
  const int k = (int)((set / G) % nc);
  const int64_t b = set / (G * nc);
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
  const bool full = Cfg::PLAN && nvalid == Q;   // every j-block lies inside the sequence
  uint32_t boffs[LOADS];
  if constexpr (Cfg::PLAN) plan_block<Cfg, T>(boffs, brow, xrow, wave, lane);
  const int64_t bblk_bytes = 32 * brow * (int64_t)sizeof(T), xblk_bytes = 32 * xrow * (int64_t)sizeof(T);

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
    const float gi = gc[i], di = dtc[i];
    sG[i] = gi;
    sDt[i] = di;
    sW[i] = di * exp2_hw(gc[(i | 31)] - gi);   // exponent <= 0: the block's last G' is its smallest
  }

  // Hprev bytes of this chunk: P rows of 4N bytes
  const unsigned char* hsrc = static_cast<const unsigned char*>(hprev) + hoff * 4;
  // the first NBUF-1 j-blocks go in flight now; with staged Hprev its first
  // two pieces go first, and the j-blocks follow the last pieces
  constexpr int JOFF = Cfg::STAGE ? Cfg::NPC % NBUF : 0;   // ring slot of j-block 0
  auto issue_j = [&](int jn) {
    const int sn = (jn + JOFF) % NBUF;
    if (full)
      issue_block_full<Cfg>(ring[sn], reinterpret_cast<const unsigned char*>(bbase) + jn * bblk_bytes,
                            reinterpret_cast<const unsigned char*>(xbase) + jn * xblk_bytes, boffs, wave);
    else
      issue_block<Cfg>(ring[sn], bbase, xbase, brow, xrow, jn, nvalid, wave, lane);
  };
  if constexpr (Cfg::STAGE) {
    issue_hpiece<Cfg>(ring[0], hsrc, 0, wave, lane);
    if (Cfg::NPC > 1) issue_hpiece<Cfg>(ring[1], hsrc, 1, wave, lane);
    else issue_j(0);
  }
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    if (!Cfg::STAGE && i < NTB) {
      if (full)
        issue_block_full<Cfg>(ring[i], reinterpret_cast<const unsigned char*>(bbase) + i * bblk_bytes,
                              reinterpret_cast<const unsigned char*>(xbase) + i * xblk_bytes, boffs, wave);
      else
        issue_block<Cfg>(ring[i], bbase, xbase, brow, xrow, i, nvalid, wave, lane);
    }

  // 2. carried state: acc[u][q][pe] = C . Hprev^T, col -> p = (pg0+q)*CG + E*m + pe
  f32x16 acc[TBW][PGW][E];
#pragma unroll
  for (int u = 0; u < TBW; ++u)
#pragma unroll
    for (int q = 0; q < PGW; ++q)
#pragma unroll
      for (int pe = 0; pe < E; ++pe) acc[u][q][pe] = f32x16{};
  if constexpr (Cfg::STAGE) {
    // piece c is in slot c % 3; at its turn the item after it (piece c + 1,
    // or j-block 0 after the last piece) is still in flight, and the slot
    // read one turn earlier takes item c + 2 (a piece, then j-blocks 0, 1)
#pragma unroll
    for (int c = 0; c < Cfg::NPC; ++c) {
      if (c + 1 < Cfg::NPC) wait_vm_barrier<Cfg::HPL>();
      else wait_vm_barrier<LOADS>();
      if (c + 2 < Cfg::NPC) issue_hpiece<Cfg>(ring[(c + 2) % NBUF], hsrc, c + 2, wave, lane);
      else if (c + 2 - Cfg::NPC < NBUF - 1) issue_j(c + 2 - Cfg::NPC);
      const unsigned char* hb = ring[c % NBUF];
      // one k-step at a time: its fragments are read while the previous
      // k-step's MFMAs run, and no more of them stay live
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        Frag hhi[PGW][E], hlo[PGW][E];
#pragma unroll
        for (int q = 0; q < PGW; ++q)
#pragma unroll
          for (int pe = 0; pe < E; ++pe) {
            const unsigned char* hp = hb + ((pg0 + q) * 64 + pe * 32 + m) * Cfg::SROW + (2 * sl + g) * 32;
            hhi[q][pe] = *reinterpret_cast<const Frag*>(hp);
            hlo[q][pe] = *reinterpret_cast<const Frag*>(hp + 16);
          }
#pragma unroll
        for (int q = 0; q < PGW; ++q)
#pragma unroll
          for (int pe = 0; pe < E; ++pe)
#pragma unroll
            for (int u = 0; u < TBW; ++u) {
              I::mma(acc[u][q][pe], cf[u][2 * c + sl], hhi[q][pe]);
              I::mma(acc[u][q][pe], cf[u][2 * c + sl], hlo[q][pe]);
            }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (!Cfg::STAGE) {
    // fp32 Hprev, too large for LDS: each wave loads its fragments from
    // global memory (the fp32 MFMA takes the state whole, no split)
    static_assert(!I::SPLIT, "bf16 Hprev is staged");
#pragma unroll
    for (int q = 0; q < PGW; ++q)
#pragma unroll
      for (int pe = 0; pe < E; ++pe) {
        const int p = (pg0 + q) * CG + E * m + pe;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const Frag hhi =
              I::load_row(static_cast<const T*>(hprev) + hoff + (int64_t)p * N + s * 2 * KPL + KPL * g, true);
#pragma unroll
          for (int u = 0; u < TBW; ++u) I::mma(acc[u][q][pe], cf[u][s], hhi);
        }
      }
  }

  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // sG, sDt, sW visible
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
  // per-lane LDS read bases: B fragment rows m (16-byte pieces 2s+g), x dword
  // rows drow(., g) (column (pg0+q)*CG + E*m)
  const int boff = m * BRB + g * 16 * (KPL == 8 ? 1 : 0) + (KPL == 8 ? 0 : g * 4);
  const int xoff = 4 * g * XRB + (pg0 * CG + E * m) * (int)sizeof(T);

  for (int jb = 0; jb < NTB; ++jb) {
    // block jb has landed once at most (blocks issued after it) x LOADS remain
    const int after = NTB - 1 - jb < NBUF - 2 ? NTB - 1 - jb : NBUF - 2;
    if (after <= 0) wait_vm_barrier<0>();
    else if (after == 1) wait_vm_barrier<LOADS>();
    else wait_vm_barrier<2 * LOADS>();
    if (jb + NBUF - 1 < NTB) issue_j(jb + NBUF - 1);
    if (jb > tmax) continue;

    const unsigned char* sb = ring[(jb + JOFF) % NBUF] + boff;
    const unsigned char* sx = ring[(jb + JOFF) % NBUF] + Cfg::BBYTES + xoff;
    const int j0 = jb * 32;
    // this lane half's 16 j rows are rows drow(q, g) of the block (D row order)
    float wj[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 wv = *reinterpret_cast<const float4*>(&sW[j0 + 8 * c + 4 * g]);
      wj[4 * c + 0] = wv.x; wj[4 * c + 1] = wv.y; wj[4 * c + 2] = wv.z; wj[4 * c + 3] = wv.w;
    }
    // x fragments (exact in the io dtype), contraction index in the same j order
    Frag xf[PGW][E][JS];
#pragma unroll
    for (int q = 0; q < PGW; ++q)
#pragma unroll
      for (int js = 0; js < JS; ++js) {
        uint32_t d[KPL];
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const int q2 = js * KPL + i;   // drow(q2, g) = 8*(q2/4) + 4g + q2%4; the 4g is in xoff
          d[i] = *reinterpret_cast<const uint32_t*>(sx + (8 * (q2 / 4) + q2 % 4) * XRB + q * CG * (int)sizeof(T));
        }
#pragma unroll
        for (int pe = 0; pe < E; ++pe) xf[q][pe][js] = I::from_dwords(d, pe);
      }
    const float gend = sG[j0 + 31];
#pragma unroll
    for (int u = 0; u < TBW; ++u) {
      const int tb = tbs[u];
      if (tb < jb) continue;
      // CB^T for (j-block, t-block): A = B rows j (from LDS), B operand = C^T
      f32x16 cb = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const Frag bfr = *reinterpret_cast<const Frag*>(sb + s * 2 * KPL * (int)sizeof(T));
        I::mma(cb, bfr, cf[u][s]);
      }
      float v[16];
      if (tb > jb) {
        // every t is past the whole j-block: 2^(G'_t - G'_j) = 2^(G'_t - G'_end) 2^(G'_end - G'_j),
        // both factors <= 1; the second (times dt_j) is the table sW
        const float a = exp2_hw(gt[u] - gend);
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = cb[q] * (wj[q] * a);
      } else {
        // diagonal block: direct decay, causal mask as a select (entries above the
        // diagonal can hold 2^(+large))
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int jr = drow(q, g);
          const float val = cb[q] * exp2_hw(gt[u] - sG[j0 + jr]) * sDt[j0 + jr];
          v[q] = (m >= jr) ? val : 0.f;
        }
      }
#pragma unroll
      for (int js = 0; js < JS; ++js) {
        Frag ahi, alo;
        I::split(&v[js * KPL], ahi, alo);
#pragma unroll
        for (int q = 0; q < PGW; ++q)
#pragma unroll
          for (int pe = 0; pe < E; ++pe) {
            I::mma(acc[u][q][pe], ahi, xf[q][pe][js]);
            if constexpr (I::SPLIT) I::mma(acc[u][q][pe], alo, xf[q][pe][js]);
          }
      }
      if (tb == jb) {
        // D x for the block's own rows, from the staged x rows
#pragma unroll
        for (int q = 0; q < PGW; ++q)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t xd = *reinterpret_cast<const uint32_t*>(
                sx + (8 * (r / 4) + r % 4) * XRB + q * CG * (int)sizeof(T));
#pragma unroll
            for (int pe = 0; pe < E; ++pe) acc[u][q][pe][r] += Dh * I::elem(xd, pe);
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

// Everything one (batch, head, chunk) tile needs to find its data; all of it
// is wave-uniform and lives in scalar registers.
template <typename T>
struct Tile {
  int h, nvalid;
  float Dh;
  int64_t ckey;   // identifies the C rows (batch, chunk, group)
  const T* xbase;
  const T* bbase;
  const T* cbase;
  T* ybase;
  const float* gc;
  const float* dtc;
  const unsigned char* hsrc;
};

// Tile number gi of the persistent walk. Tiles are numbered (batch*chunk,
// head) with heads fastest; with xcd set (the grid and batch*nchunks are
// multiples of 8), the numbering first groups the chunks by index mod 8, and
// workgroup w, dealt round-robin to XCD w mod 8, walks a contiguous range of
// its XCD's group. So a workgroup visits consecutive heads of one chunk
// (its C fragments stay in registers across them), and each chunk's B and C
// rows are read into one XCD's L2 only.
template <typename T, int P, int N, int Q>
__device__ __forceinline__ Tile<T> make_tile(int64_t gi, bool xcd, int64_t ntiles, const T* x, const T* Bm,
                                             const T* Cm, const float* gcum, const float* dtt, const float* Dp,
                                             const void* hprev, T* y, int64_t Tlen, int H, int G, int64_t nc,
                                             int64_t Tp) {
  int64_t bk;
  int h;
  if (xcd) {
    const int64_t n8 = ntiles / 8, xg = gi / n8, i = gi % n8;
    bk = xg + 8 * (i / H);
    h = (int)(i % H);
  } else {
    bk = gi / H;
    h = (int)(gi % H);
  }
  const int64_t k = bk % nc, b = bk / nc;
  const int grp = h / (H / G);
  const int64_t t0 = k * Q;
  Tile<T> t;
  t.h = h;
  t.ckey = bk * G + grp;
  t.nvalid = (int)(Tlen - t0 < Q ? Tlen - t0 : Q);
  t.Dh = Dp[h];
  t.xbase = x + ((b * Tlen + t0) * H + h) * P;
  t.ybase = y + ((b * Tlen + t0) * H + h) * P;
  t.bbase = Bm + ((b * Tlen + t0) * G + grp) * N;
  t.cbase = Cm + ((b * Tlen + t0) * G + grp) * N;
  t.gc = gcum + (b * H + h) * Tp + t0;
  t.dtc = dtt + (b * H + h) * Tp + t0;
  t.hsrc = static_cast<const unsigned char*>(hprev) + (((b * H + h) * nc + k) * (int64_t)(P * N)) * 4;
  return t;
}

// vmcnt's largest count.
__device__ __forceinline__ constexpr int cap63(int n) { return n < 63 ? n : 63; }

// Persistent form of the kernel above, used when the carried state fits in
// LDS. Each workgroup walks a contiguous range of tiles (see make_tile); one
// stream of direct global->LDS loads runs across tile boundaries: while a
// tile's j-blocks are consumed, the next tile's Hprev (into the LDS buffer
// freed once this tile's carried-state product is done) and its first two
// j-blocks (into the ring slots as they free) are already in flight, and
// the next tile's G' and dt are loaded into registers behind this tile's y
// stores. The arithmetic
// is the kernel above's, step for step.
//
// Load accounting: every wave issues LOADS instructions per j-block and
// HLOADS per Hprev, in program order; vector memory operations complete in
// issue order, so "item X has landed" is "at most (operations issued after
// X) remain". The counts used below include only this stream's own loads,
// a lower bound whenever the compiler adds loads or stores of its own.
template <typename T, int P, int N, int Q>
__global__ __launch_bounds__((ScanCfg<T, P, N, Q>::THREADS)) __attribute__((amdgpu_waves_per_eu(2)))
void ssd_chunk_scan_persistent(const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
                               const float* __restrict__ gcum, const float* __restrict__ dtt,
                               const float* __restrict__ Dp, const void* __restrict__ hprev, T* __restrict__ y,
                               int64_t Tlen, int H, int G, int64_t nc, int64_t Tp, int64_t ntiles, int xcd) {
  using I = Io<T>;
  using Frag = typename I::Frag;
  using Cfg = ScanCfg<T, P, N, Q>;
  constexpr int E = I::E, KPL = I::KPL, CG = Cfg::CG, NTB = Cfg::NTB, TBW = Cfg::TBW;
  constexpr int PGW = Cfg::PGW, NPS = Cfg::NPS;
  constexpr int LOADS = Cfg::LOADS, HLOADS = Cfg::HLOADS;
  constexpr int BRB = Cfg::BROWP * 16, XRB = Cfg::XROWP * 16;
  constexpr int KS = N / (2 * KPL);
  constexpr int JS = 32 / (2 * KPL);
  static_assert(Cfg::HLDS && Cfg::NBUF == 3, "persistent form: Hprev in LDS, three ring slots");
  static_assert(Q <= Cfg::THREADS, "one token of G' per thread");
  constexpr int NYS = TBW * 16 * PGW;   // y store instructions per wave of a full tile

  __shared__ __attribute__((aligned(16))) unsigned char ring[3][Cfg::BLOCK];
  __shared__ __attribute__((aligned(16))) unsigned char sH[Cfg::HALLOC];
  __shared__ __attribute__((aligned(16))) float sG[Q];
  __shared__ __attribute__((aligned(16))) float sDt[Q];
  __shared__ __attribute__((aligned(16))) float sW[Q];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int tg = wave / NPS, pg0 = (wave % NPS) * PGW;
  int tbs[TBW];
  tbs[0] = tg;
  if constexpr (TBW == 2) tbs[1] = NTB - 1 - tg;
  int tmax = tbs[0];
  if constexpr (TBW == 2) tmax = tbs[1];
  const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N;
  uint32_t brc[LOADS];
  plan_block_rc<Cfg>(brc, wave, threadIdx.x % 64);
  const uint32_t bsb = (uint32_t)(brow * (int64_t)sizeof(T)), xsb = (uint32_t)(xrow * (int64_t)sizeof(T));
  const bool use_xcd = xcd != 0;

  // this workgroup's contiguous range [pos, last) of the tile numbering
  int64_t pos, last;
  if (use_xcd) {
    const int64_t n8 = ntiles / 8, g8 = gridDim.x / 8, xg = blockIdx.x % 8, idx = blockIdx.x / 8;
    pos = xg * n8 + idx * n8 / g8;
    last = xg * n8 + (idx + 1) * n8 / g8;
  } else {
    pos = blockIdx.x * ntiles / gridDim.x;
    last = (blockIdx.x + 1) * ntiles / gridDim.x;
  }
  if (pos >= last) return;
  Tile<T> cur = make_tile<T, P, N, Q>(pos, use_xcd, ntiles, x, Bm, Cm, gcum, dtt, Dp, hprev, y, Tlen, H, G, nc, Tp);

  // j-block jb of tile t into ring slot `slot`
#define SSD_ISSUE(slot, t, jb)                                                                              \
  issue_block_rc<Cfg>(ring[slot], reinterpret_cast<const unsigned char*>((t).bbase),                        \
                      reinterpret_cast<const unsigned char*>((t).xbase), bsb, xsb, brc, jb, (t).nvalid, wave)

  // stream head: Hprev and j-blocks 0, 1 of the first tile; its G' and dt
  int tid = threadIdx.x, lane = tid % 64;
  issue_hprev<Cfg, T>(sH, cur.hsrc, wave, lane);
  SSD_ISSUE(0, cur, 0);
  SSD_ISSUE(1, cur, 1);
  int slot0 = 0;   // ring slot of the current tile's j-block 0
  float pre_g = 0.f, pre_d = 0.f, pre_l = 0.f;
  if (tid < Q) {
    pre_g = cur.gc[tid];
    pre_d = cur.dtc[tid];
    pre_l = cur.gc[tid | 31];
  }

  Frag cf[TBW][KS];
  int64_t cf_key = -1;
  // 1 when the previous tile issued exactly NYS y stores per wave (a full
  // tile): the waits below then count them, so they do not also wait for
  // the stores' write acknowledgements (vmcnt covers loads and stores alike)
  int ys = 0;
  while (true) {
    // Lane-derived addresses are rebuilt for every tile: an opaque copy of
    // the thread index keeps the compiler from hoisting them out of the tile
    // loop, where they would all stay live across it.
    asm volatile("" : "+v"(tid));
    lane = tid % 64;
    const int m = lane % 32, g = lane / 32;
    const int boff = m * BRB + g * 16 * (KPL == 8 ? 1 : 0) + (KPL == 8 ? 0 : g * 4);
    const int xoff = 4 * g * XRB + (pg0 * CG + E * m) * (int)sizeof(T);
    const int64_t npos = pos + 1;
    const bool has_next = npos < last;
    // (the last tile describes itself as its successor; nothing is loaded for it)
    const Tile<T> nxt = make_tile<T, P, N, Q>(has_next ? npos : pos, use_xcd, ntiles, x, Bm, Cm, gcum, dtt, Dp,
                                              hprev, y, Tlen, H, G, nc, Tp);

    // 1. C fragments of the wave's t-blocks, unless the previous tile had the same C rows
    if (cur.ckey != cf_key) {
      cf_key = cur.ckey;
#pragma unroll
      for (int u = 0; u < TBW; ++u) {
        const int t = tbs[u] * 32 + m;
        const bool valid = t < cur.nvalid;
#pragma unroll
        for (int s = 0; s < KS; ++s) cf[u][s] = I::load_row(cur.cbase + t * brow + s * 2 * KPL + KPL * g, valid);
      }
      // consume the fragments here, so the compiler's wait for these loads
      // stays on this (rare) path instead of draining the whole load queue
      // before every tile's first product
#pragma unroll
      for (int u = 0; u < TBW; ++u)
#pragma unroll
        for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(cf[u][s]));
      ys = 0;   // that wait also waited for the stores
    }
    // every wave is past the previous tile's reads of sG, sDt and sW
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (tid < Q) {
      sG[tid] = pre_g;
      sDt[tid] = pre_d;
      sW[tid] = pre_d * exp2_hw(pre_l - pre_g);   // exponent <= 0
    }

    // 2. carried state. Hprev has landed once at most the two j-blocks
    // issued after it remain -- after the previous tile's C.Hprev came all
    // NTB of its j-block issues and its y stores (the barrier also publishes
    // sG, sDt, sW).
    f32x16 acc[TBW][PGW][E];
#pragma unroll
    for (int u = 0; u < TBW; ++u)
#pragma unroll
      for (int q = 0; q < PGW; ++q)
#pragma unroll
        for (int pe = 0; pe < E; ++pe) acc[u][q][pe] = f32x16{};
    if (ys) wait_vm_barrier<cap63(NTB * LOADS + NYS)>();
    else wait_vm_barrier<2 * LOADS>();
#pragma unroll
    for (int q = 0; q < PGW; ++q)
#pragma unroll
      for (int pe = 0; pe < E; ++pe) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          Frag hhi, hlo;
          const int slot = E == 2 ? (pg0 + q) * 64 + pe * 32 + m : (pg0 + q) * CG + E * m + pe;
          const unsigned char* hp = sH + slot * (Cfg::HROWP * 16);
          if constexpr (I::SPLIT) {
            hhi = *reinterpret_cast<const Frag*>(hp + (2 * s + g) * 32);
            hlo = *reinterpret_cast<const Frag*>(hp + (2 * s + g) * 32 + 16);
          } else {
            hhi = *reinterpret_cast<const Frag*>(hp + (s * 2 * KPL + KPL * g) * 4);
          }
#pragma unroll
          for (int u = 0; u < TBW; ++u) {
            I::mma(acc[u][q][pe], cf[u][s], hhi);
            if constexpr (I::SPLIT) I::mma(acc[u][q][pe], cf[u][s], hlo);
          }
        }
      }
    // every wave is done with sH: the next tile's Hprev may land there
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (has_next) issue_hprev<Cfg, T>(sH, nxt.hsrc, wave, lane);
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
    for (int jb = 0; jb < NTB; ++jb) {
      // block jb has landed once only the stream items issued after it remain:
      // the next j-block (issued one iteration earlier, or before this tile
      // for jb = 0) and, for jb <= 1, the next tile's Hprev
      // (and, for jb <= 1 after a full tile, that tile's NYS y stores)
      const bool blk_after = jb == 0 || jb + 1 < NTB || has_next;
      const bool h_after = jb <= 1 && has_next;
      if (jb <= 1 && ys) {
        if (blk_after && h_after) wait_vm_barrier<cap63(LOADS + HLOADS + NYS)>();
        else if (blk_after) wait_vm_barrier<cap63(LOADS + NYS)>();
        else if (h_after) wait_vm_barrier<cap63(HLOADS + NYS)>();
        else wait_vm_barrier<cap63(NYS)>();
      } else {
        if (blk_after && h_after) wait_vm_barrier<LOADS + HLOADS>();
        else if (blk_after) wait_vm_barrier<LOADS>();
        else if (h_after) wait_vm_barrier<HLOADS>();
        else wait_vm_barrier<0>();
      }
      {
        const int jn = jb + 2, sn = (slot0 + jn) % 3;
        if (jn < NTB) SSD_ISSUE(sn, cur, jn);
        else if (has_next) SSD_ISSUE(sn, nxt, jn - NTB);
      }
      if (jb > tmax) continue;

      const unsigned char* sb = ring[(slot0 + jb) % 3] + boff;
      const unsigned char* sx = ring[(slot0 + jb) % 3] + Cfg::BBYTES + xoff;
      const int j0 = jb * 32;
      float wj[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 wv = *reinterpret_cast<const float4*>(&sW[j0 + 8 * c + 4 * g]);
        wj[4 * c + 0] = wv.x; wj[4 * c + 1] = wv.y; wj[4 * c + 2] = wv.z; wj[4 * c + 3] = wv.w;
      }
      Frag xf[PGW][E][JS];
#pragma unroll
      for (int q = 0; q < PGW; ++q)
#pragma unroll
        for (int js = 0; js < JS; ++js) {
          uint32_t d[KPL];
#pragma unroll
          for (int i = 0; i < KPL; ++i) {
            const int q2 = js * KPL + i;
            d[i] = *reinterpret_cast<const uint32_t*>(sx + (8 * (q2 / 4) + q2 % 4) * XRB + q * CG * (int)sizeof(T));
          }
#pragma unroll
          for (int pe = 0; pe < E; ++pe) xf[q][pe][js] = I::from_dwords(d, pe);
        }
      const float gend = sG[j0 + 31];
#pragma unroll
      for (int u = 0; u < TBW; ++u) {
        const int tb = tbs[u];
        if (tb < jb) continue;
        f32x16 cb = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const Frag bfr = *reinterpret_cast<const Frag*>(sb + s * 2 * KPL * (int)sizeof(T));
          I::mma(cb, bfr, cf[u][s]);
        }
        float v[16];
        if (tb > jb) {
          const float a = exp2_hw(gt[u] - gend);
#pragma unroll
          for (int q = 0; q < 16; ++q) v[q] = cb[q] * (wj[q] * a);
        } else {
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int jr = drow(q, g);
            const float val = cb[q] * exp2_hw(gt[u] - sG[j0 + jr]) * sDt[j0 + jr];
            v[q] = (m >= jr) ? val : 0.f;
          }
        }
#pragma unroll
        for (int js = 0; js < JS; ++js) {
          Frag ahi, alo;
          I::split(&v[js * KPL], ahi, alo);
#pragma unroll
          for (int q = 0; q < PGW; ++q)
#pragma unroll
            for (int pe = 0; pe < E; ++pe) {
              I::mma(acc[u][q][pe], ahi, xf[q][pe][js]);
              if constexpr (I::SPLIT) I::mma(acc[u][q][pe], alo, xf[q][pe][js]);
            }
        }
        if (tb == jb) {
#pragma unroll
          for (int q = 0; q < PGW; ++q)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const uint32_t xd = *reinterpret_cast<const uint32_t*>(
                  sx + (8 * (r / 4) + r % 4) * XRB + q * CG * (int)sizeof(T));
#pragma unroll
              for (int pe = 0; pe < E; ++pe) acc[u][q][pe][r] += cur.Dh * I::elem(xd, pe);
            }
        }
      }
    }

    // the next tile's G' and dt, in flight behind this tile's y stores
    if (has_next && tid < Q) {
      pre_g = nxt.gc[tid];
      pre_d = nxt.dtc[tid];
      pre_l = nxt.gc[tid | 31];
    }

    // 4. y
#pragma unroll
    for (int u = 0; u < TBW; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = tbs[u] * 32 + drow(r, g);
        if (t < cur.nvalid) {
#pragma unroll
          for (int q = 0; q < PGW; ++q)
            I::store_pair(cur.ybase + t * xrow + (pg0 + q) * CG + E * m, acc[u][q][0][r], acc[u][q][E - 1][r]);
        }
      }
    ys = cur.nvalid == Q ? 1 : 0;
    if (!has_next) break;
    slot0 = (slot0 + NTB) % 3;
    pos = npos;
    cur = nxt;
  }
#undef SSD_ISSUE
}

// Workgroups of the persistent form that fit on the current device at once
// (cached per device; a failed query falls back to 256).
template <typename T, int P, int N, int Q>
int64_t persistent_grid(int64_t ntiles) {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    dev = 0;
  }
  if (!cached[dev]) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ssd_chunk_scan_persistent<T, P, N, Q>,
                                                     ScanCfg<T, P, N, Q>::THREADS, 0) != hipSuccess ||
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

template <typename T, int P, int N, int Q>
hipError_t launch_one(const Problem& p, hipStream_t stream) {
  using Cfg = ScanCfg<T, P, N, Q>;
  if constexpr (Cfg::HLDS && Cfg::NBUF == 3) {
    const int64_t ntiles = p.bt * p.nc * p.H;
    if (ntiles == 0) return hipSuccess;
    const int64_t grid = persistent_grid<T, P, N, Q>(ntiles);
    const int xcd = (grid % 8 == 0 && (p.bt * p.nc) % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((ssd_chunk_scan_persistent<T, P, N, Q>), dim3((unsigned)grid), dim3(Cfg::THREADS), 0,
                       stream, (const T*)p.x, (const T*)p.B, (const T*)p.C, p.gcum, p.dtt, p.D,
                       (const void*)p.hprev, (T*)p.y, p.T, (int)p.H, (int)p.G, p.nc, p.Tp, ntiles, xcd);
  } else {
    const int64_t tiles = p.H * p.nc * p.bt;
    const int xcd = (p.bt * p.nc * p.G) % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL((ssd_chunk_scan<T, P, N, Q>), dim3((unsigned)tiles), dim3(Cfg::THREADS), 0, stream,
                       (const T*)p.x, (const T*)p.B, (const T*)p.C, p.gcum, p.dtt, p.D, (const void*)p.hprev,
                       (T*)p.y, p.T, (int)p.H, (int)p.G, p.nc, p.Tp, xcd);
  }
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
  if (chunk_scan_resident_fits(p)) return launch_chunk_scan_resident(p, stream);
  return p.io == 1 ? dispatch<bf16>(p, stream) : dispatch<float>(p, stream);
}

}  // namespace ssd

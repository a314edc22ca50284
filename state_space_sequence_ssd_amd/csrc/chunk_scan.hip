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
// Work split. A (batch, head, chunk) tile is Q rows of t x headdim columns.
// Its rows form Q/32 blocks of 32; wave w owns the block pair {w, Q/32-1-w},
// so every wave has the same number of causal (t-block, j-block) pairs.
// Accumulators hold the wave's 64 rows x its headdim column groups in fp32.
//
// Per wave:
//  1. C rows of both t-blocks are loaded once as MFMA fragments (contiguous
//     along dstate); they serve as the B operand of C.B^T and as the A operand
//     of the carried-state term.
//  2. acc = C . Hprev^T (MFMA over dstate), then each row t scaled by
//     2^(G'_t) <= 1. Hprev is fp32; with bf16 io it enters as a bf16 (hi, lo)
//     pair in two MFMAs against the exact bf16 C.
//  3. For each 32-token j-block up to the wave's last t-block: CB^T = B . C^T
//     for the j-block (MFMA over dstate). Its D layout gives lane l the
//     column t = l%32 and 16 rows j; exactly the lanes and registers the A
//     operand of the next product needs, once the contraction index j is
//     permuted to the D row order (the B operand below uses the same order).
//     The decay 2^(G'_t - G'_j) and dt_j are applied and the causal mask is a
//     select (not a multiply: entries above the diagonal can hold
//     2^(+large)); with bf16 io the result enters as a bf16 (hi, lo) pair in
//     two MFMAs against the exact bf16 x. (The blog rounds the carried state
//     and this matrix to the input type; where large terms cancel that
//     rounding alone breaks a 1e-2 + 2e-2|y| elementwise bound, so here every
//     MFMA operand that is not an input keeps about 16 significant bits.)
//  4. y = acc + D x, rounded to the io dtype, stored one dword per lane per
//     row (whole 128-byte rows per half-wave).
//
// x fragments are loaded one dword per lane per token row (see
// ssd_device.h); no LDS is used and there are no barriers.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

template <typename T, int P, int Q>
struct ScanCfg {
  static constexpr int E = Io<T>::E;
  static constexpr int CG = 32 * E;
  static constexpr int NPG = P / CG;          // headdim column groups
  static constexpr int NTB = Q / 32;          // 32-row blocks
  static constexpr int NPAIR = NTB / 2;       // balanced block pairs
  static constexpr int PGW = (NPAIR * NPG) / 4 > 1 ? (NPAIR * NPG) / 4 : 1;   // column groups per wave
  static constexpr int NPS = NPG / PGW;
  static constexpr int WPT = NPAIR * NPS;     // waves per tile
  static constexpr int TPW = 4 / WPT;         // tiles per 256-thread workgroup
  static_assert(NTB >= 2 && NTB % 2 == 0, "chunk must be a multiple of 64");
  static_assert(WPT >= 1 && WPT <= 4 && 4 % WPT == 0, "tile does not fit a workgroup");
};

template <typename T, int P, int N, int Q>
__global__ __launch_bounds__(256) void ssd_chunk_scan(const T* __restrict__ x,
                                                      const T* __restrict__ Bm,
                                                      const T* __restrict__ Cm,
                                                      const float* __restrict__ gcum,
                                                      const float* __restrict__ dtt,
                                                      const float* __restrict__ Dp,
                                                      const float* __restrict__ hprev,
                                                      T* __restrict__ y,
                                                      int64_t Tlen, int H, int G, int64_t nc, int64_t Tp) {
  using I = Io<T>;
  using Frag = typename I::Frag;
  using Cfg = ScanCfg<T, P, Q>;
  constexpr int E = I::E, KPL = I::KPL, CG = Cfg::CG, NTB = Cfg::NTB;
  constexpr int PGW = Cfg::PGW, NPS = Cfg::NPS, WPT = Cfg::WPT, TPW = Cfg::TPW;
  constexpr int KS = N / (2 * KPL);    // MFMA steps over dstate
  constexpr int JS = 32 / (2 * KPL);   // MFMA steps over a 32-token j-block

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int m = lane % 32, g = lane / 32;
  const int tile = wave / WPT, sub = wave % WPT;
  const int pair = sub / NPS, pg0 = (sub % NPS) * PGW;
  const int h = blockIdx.x * TPW + tile;
  if (h >= H) return;
  const int k = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int grp = h / (H / G);
  const int64_t t0 = (int64_t)k * Q;
  const int64_t nvalid = Tlen - t0;
  const int tbs[2] = {pair, NTB - 1 - pair};

  const float* gc = gcum + ((int64_t)b * H + h) * Tp + t0;
  const float* dtc = dtt + ((int64_t)b * H + h) * Tp + t0;
  const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N;
  const T* xbase = x + ((b * Tlen + t0) * H + h) * P;
  T* ybase = y + ((b * Tlen + t0) * H + h) * P;
  const T* bbase = Bm + ((b * Tlen + t0) * G + grp) * N;
  const T* cbase = Cm + ((b * Tlen + t0) * G + grp) * N;
  const float* hp = hprev + (((int64_t)b * H + h) * nc + k) * (int64_t)(P * N);

  // 1. C fragments of both t-blocks: row t = 32*tb + m, dstate k-step s
  Frag cf[2][KS];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = tbs[u] * 32 + m;
    const bool valid = t < nvalid;
#pragma unroll
    for (int s = 0; s < KS; ++s) cf[u][s] = I::load_row(cbase + t * brow + s * 2 * KPL + KPL * g, valid);
  }

  // 2. carried state: acc[u][pgl][pe] = C . Hprev^T, col -> p = (pg0+pgl)*CG + E*m + pe
  f32x16 acc[2][PGW][E];
#pragma unroll
  for (int u = 0; u < 2; ++u)
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
        Frag hhi, hlo;   // the fp32 carried state as a bf16 pair (C is exact)
        I::load_split(hp + p * N + s * 2 * KPL + KPL * g, hhi, hlo);
        I::mma(acc[0][q][pe], cf[0][s], hhi);
        I::mma(acc[1][q][pe], cf[1][s], hhi);
        if constexpr (I::SPLIT) {
          I::mma(acc[0][q][pe], cf[0][s], hlo);
          I::mma(acc[1][q][pe], cf[1][s], hlo);
        }
      }
    }
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float sc = exp2_hw(gc[tbs[u] * 32 + drow(r, g)]);
#pragma unroll
      for (int q = 0; q < PGW; ++q)
#pragma unroll
        for (int pe = 0; pe < E; ++pe) acc[u][q][pe][r] *= sc;
    }

  // 3. intra-chunk, causal over 32-token j-blocks
  const float gt[2] = {gc[tbs[0] * 32 + m], gc[tbs[1] * 32 + m]};
  for (int jb = 0; jb <= tbs[1]; ++jb) {
    const int j0 = jb * 32;
    Frag bfr[KS];
    {
      const int j = j0 + m;
      const bool valid = j < nvalid;
#pragma unroll
      for (int s = 0; s < KS; ++s) bfr[s] = I::load_row(bbase + j * brow + s * 2 * KPL + KPL * g, valid);
    }
    // this lane half's 16 j rows, in D row order: j(q) = j0 + drow(q, g)
    float gj[16], dj[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 gv = *reinterpret_cast<const float4*>(gc + j0 + 8 * c + 4 * g);
      const float4 dv = *reinterpret_cast<const float4*>(dtc + j0 + 8 * c + 4 * g);
      gj[4 * c + 0] = gv.x; gj[4 * c + 1] = gv.y; gj[4 * c + 2] = gv.z; gj[4 * c + 3] = gv.w;
      dj[4 * c + 0] = dv.x; dj[4 * c + 1] = dv.y; dj[4 * c + 2] = dv.z; dj[4 * c + 3] = dv.w;
    }
    // x fragments (exact in the io dtype), contraction index in the same j(q) order
    Frag xf[PGW][E][JS];
#pragma unroll
    for (int q = 0; q < PGW; ++q)
#pragma unroll
      for (int js = 0; js < JS; ++js) {
        uint32_t d[KPL];
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const int j = j0 + drow(js * KPL + i, g);
          d[i] = j < nvalid
                     ? *(reinterpret_cast<const uint32_t*>(xbase + j * xrow + (pg0 + q) * CG) + m)
                     : 0u;
        }
#pragma unroll
        for (int pe = 0; pe < E; ++pe) xf[q][pe][js] = I::from_dwords(d, pe);
      }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tb = tbs[u];
      if (tb < jb) continue;
      f32x16 cb = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) I::mma(cb, bfr[s], cf[u][s]);
      float v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const bool keep = (tb > jb) || (m >= drow(q, g));
        const float val = cb[q] * exp2_hw(gt[u] - gj[q]) * dj[q];
        v[q] = keep ? val : 0.f;
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
    }
  }

  // 4. y = acc + D x
  const float Dh = Dp[h];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = tbs[u] * 32 + drow(r, g);
      if (t < nvalid) {
#pragma unroll
        for (int q = 0; q < PGW; ++q) {
          const int64_t off = t * xrow + (pg0 + q) * CG + E * m;
          const uint32_t xd = *reinterpret_cast<const uint32_t*>(xbase + off);
          I::store_pair(ybase + off, acc[u][q][0][r] + Dh * I::elem(xd, 0),
                        acc[u][q][E - 1][r] + Dh * I::elem(xd, E - 1));
        }
      }
    }
}

template <typename T, int P, int N, int Q>
hipError_t launch_one(const Problem& p, hipStream_t stream) {
  constexpr int TPW = ScanCfg<T, P, Q>::TPW;
  const dim3 grid((unsigned)((p.H + TPW - 1) / TPW), (unsigned)p.nc, (unsigned)p.bt);
  hipLaunchKernelGGL((ssd_chunk_scan<T, P, N, Q>), grid, dim3(256), 0, stream, (const T*)p.x, (const T*)p.B,
                     (const T*)p.C, p.gcum, p.dtt, p.D, p.hprev, (T*)p.y, p.T, (int)p.H, (int)p.G,
                     p.nc, p.Tp);
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

// The backward pass of the selective scan (S6): every input's gradient for
// upstream gradients dy (like y) and dhT (like the final state). Per scalar
// chain (batch row b, channel d, state n), with a_t = exp(delta_t A[d, n]),
// u_t = B[n, t] delta_t x_t and h_t = a_t h_{t-1} + u_t, the state's adjoint
// runs the same scan backwards in time ("Mamba: The Hard Way", Part 3, on
// the chains of Part 5):
//
//   g_t = C[n, t] dy_t + a_{t+1} g_{t+1}         (after the last token: dhT)
//   dx_t = sum_n g_t B delta_t,   ddelta_t = sum_n g_t (A a_t h_{t-1} + B x_t)
//   dA  += g_t delta_t a_t h_{t-1},   dh0 = a_0 g_0
//   dB[n, t] = sum_d g_t delta_t x_t,   dC[n, t] = sum_d dy_t h_t
//
// Chunks of 64 tokens, as in the forward pass:
//   1. the forward sweep (s6_onepass in its backward mode) leaves every
//      chunk's end state and, from dy, the chunk's own adjoint record: O_c,
//      the adjoint its dy alone leaves at its first token (times that
//      token's decay), sum_t (a_t0 ... a_t) C_t dy_t, and the chunk's sum of
//      delta (its decays multiply to exp(A sum));
//   2. s6_bwd_carry: the adjoint entering each chunk from the right,
//      R_{c-1} = O_c + exp(A sum_c delta) R_c from R_last = dhT, and dh0;
//   3. s6_bwd_chunk: per chunk and 64 channels (one wave) and group of up
//      to 4 states (one pass per group, each adding its terms of dx and
//      ddelta to the earlier passes'), the states recomputed forward from
//      the entering state (kept every 8 tokens), then per 8-token piece, last
//      first, the piece's states again and the backward step for each token,
//      which gives dx, ddelta and the per-chunk parts of dA, dB and dC (the
//      dB and dC parts summed over the wave's 64 channels in registers, by
//      lane swaps and DPP);
//   4. s6_bwd_reduce: dA over batch rows and chunks, dB and dC over channel
//      blocks (fixed orders: deterministic).
// Lanes are channels, as in the forward pass; each lane holds its chunk's x
// and delta in registers, read as whole rows through a per-wave LDS tile
// that then keeps dy.
#include "lookback_device.h"
#include "ssd_device.h"
#include "s6_device.h"
#include "s6_launch.h"

namespace ssd {

namespace {

constexpr int kChunk = 64;      // tokens per chunk (the forward pass's)
constexpr int kBwdLanes = 64;   // channels per workgroup of the chunk kernel (one wave)

// piece length of the recomputation: the states of S tokens are held at once
template <int N> struct BwdPiece { static constexpr int S = 8; };

// 2. per (batch row, channel, state): the adjoint entering each chunk from
// the right, R[c]; dh0 at the end. Chunks are walked from the last, their
// records read eight chunks ahead; threads take consecutive (channel, state)
// pairs, so every record read and written is coalesced.
template <int N>
__global__ __launch_bounds__(256) void s6_bwd_carry(const float* __restrict__ A, const float* __restrict__ O,
                                                    const float* __restrict__ SD, const float* __restrict__ dhT,
                                                    float* __restrict__ R, float* __restrict__ dh0, int64_t bt, int D,
                                                    int64_t nc) {
  // i = (b * D + d) * N + n; grid-stride, the grid being capped at 65536
  // workgroups
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < bt * D * N;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bd = i / N;
    const int n = (int)(i % N);
    const int64_t b = bd / D;
    const int d = (int)(bd % D);
    const float a2 = A[(int64_t)d * N + n] * kLog2e;
    float r = dhT ? dhT[i] : 0.f;
    constexpr int CR = 8;
    for (int64_t c1 = nc - 1; c1 >= 0; c1 -= CR) {
      float ov[CR], sv[CR];
#pragma unroll
      for (int j = 0; j < CR; ++j) {
        const int64_t c = c1 - j;
        const int64_t rec = (b * nc + (c >= 0 ? c : 0)) * D + d;
        ov[j] = c >= 0 ? O[rec * N + n] : 0.f;
        sv[j] = c >= 0 ? SD[rec] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < CR; ++j) {
        const int64_t c = c1 - j;
        if (c < 0) break;
        const int64_t rec = (b * nc + c) * D + d;
        R[rec * N + n] = r;
        r = fmaf(exp2_hw(a2 * sv[j]), r, ov[j]);
      }
    }
    if (dh0) dh0[i] = r;
  }
}

// Sums over a wave's 64 lanes in registers. halve<M>(a, b, hi): lanes
// whose bit M is clear (hi false) return a plus their partner's a, the
// others b plus their partner's b; partners differ in bit M: M = 32 and 16
// through gfx950's half swaps (v_permlane32_swap, v_permlane16_swap), M = 8
// a rotation by 8 within 16 lanes, M = 4 the mirror within 8 lanes, M = 2
// and 1 quad permutations (DPP).
template <int M>
__device__ __forceinline__ float dpp_partner(float v) {
  static_assert(M == 8 || M == 4 || M == 2 || M == 1, "DPP partners within 16 lanes");
  constexpr int ctrl = M == 8 ? 0x128 : M == 4 ? 0x141 : M == 2 ? 0x4E : 0xB1;
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}
template <int M>
__device__ __forceinline__ float halve(float a, float b, bool hi) {
  if constexpr (M == 32 || M == 16) {
    const auto r = M == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                           : __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const float keep = hi ? b : a, send = hi ? a : b;
    return keep + dpp_partner<M>(send);
  }
}
// R values per lane down to one by halving over lane bits BIT, BIT - 1, ...:
// afterwards value k sits in the lanes whose bits BIT .. BIT - log2(R) + 1,
// read from the highest, spell k, summed over the lanes that differ only in
// those bits.
template <int R, int BIT>
__device__ __forceinline__ void halve_all(float* v, unsigned lane) {
  if constexpr (R > 1) {
    const bool hi = ((lane >> BIT) & 1u) != 0;
#pragma unroll
    for (int k = 0; k < R / 2; ++k) v[k] = halve<(1 << BIT)>(v[k], v[k + R / 2], hi);
    halve_all<R / 2, BIT - 1>(v, lane);
  }
}
constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

constexpr int kHalf = 32;   // tokens per half chunk: the chunk kernel holds one half in registers

// The states at the start of each S-token piece of one half chunk (tokens
// tb .. tb + 31 of the chunk), from h at the half's start; h leaves as the
// state after the half.
template <int N, int S>
__device__ __forceinline__ void half_forward(const float* xr, const float* dr, const float* a2,
                                             const float (*sB)[kChunk], int tb, float* h, float (*ck)[N]) {
#pragma unroll
  for (int j = 0; j < kHalf / S; ++j) {
    // one piece at a time: hoisted, the decays of the whole half would be
    // live at once
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < N; ++n) ck[j][n] = h[n];
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int t = S * j + i;
      const float u = dr[t] * xr[t];
#pragma unroll
      for (int n = 0; n < N; ++n) h[n] = fmaf(exp2_hw(dr[t] * a2[n]), h[n], u * sB[n][tb + t]);
    }
  }
}

// The backward steps over one half chunk, its pieces last first. g is the
// adjoint entering the half from the right and leaves as the adjoint of the
// state before the half; dA accumulates; each piece's dB and dC values are
// summed over the wave's lanes and written by the lanes that hold them
// (part + tb + token). The outputs dx, ddelta replace x, delta in xr, dr.
//
// The pieces run as a loop that is not unrolled (unrolled, the compiler
// interleaves the pieces and keeps far more live than one piece needs): the
// current piece always sits in the last S entries of xr, dr and in the last
// checkpoint; after it, its outputs take its place and the arrays rotate
// right by one piece, so after all pieces every output is back at its
// token's position.
template <int N, int S>
__device__ __forceinline__ void half_backward(float* xr, float* dr, float (*ck)[N], const float* an, const float* a2,
                                              float* g, float* dA, const float (*sB)[kChunk],
                                              const float (*sC)[kChunk], const float (*sY)[64], int tb, int lane,
                                              float* part, bool writer, int isum, int nth) {
  constexpr int NP = kHalf / S;
  constexpr int T1 = ilog2(2 * N), T2 = ilog2(S), T3 = 6 - T1 - T2;
  static_assert((1 << T1) == 2 * N && (1 << T2) == S && T3 >= 0 && T3 <= 2, "piece sums fill the lanes");
  const unsigned ul = (unsigned)lane;
#pragma unroll 1
  for (int m = 0; m < NP; ++m) {
    const int j = NP - 1 - m;   // the piece's position in the half
    constexpr int P0 = kHalf - S;
    // the piece's entering states, recomputed (the decays are recomputed
    // again in the backward steps: holding them would cost S N registers)
    float hp[S][N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = ck[NP - 1][n];
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int t = tb + S * j + i;
      const float u = dr[P0 + i] * xr[P0 + i];
#pragma unroll
      for (int n = 0; n < N; ++n) {
        hp[i][n] = h[n];
        h[n] = fmaf(exp2_hw(dr[P0 + i] * a2[n]), h[n], u * sB[n][t]);
      }
    }
    // the backward steps, last token first; each step's dB (g_t delta_t x_t)
    // and dC (dy_t h_t) values are halved over the lanes at once
    float pr[S];
#pragma unroll
    for (int i = S - 1; i >= 0; --i) {
      const int t = tb + S * j + i;
      const float gyt = sY[S * j + i][lane];
      const float dxt = dr[P0 + i] * xr[P0 + i];
      float s1 = 0.f, s2 = 0.f, v[2 * N];
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const float av = exp2_hw(dr[P0 + i] * a2[n]);
        const float gn = fmaf(sC[n][t], gyt, g[n]);     // dL/dh_t
        const float ah = av * hp[i][n];
        const float bnt = sB[n][t];
        v[N + n] = gyt * fmaf(dxt, bnt, ah);            // dy_t h_t
        s1 = fmaf(gn, bnt, s1);
        const float ga = gn * ah;
        s2 = fmaf(ga, an[n], s2);
        dA[n] = fmaf(dr[P0 + i], ga, dA[n]);
        v[n] = gn * dxt;                                 // g_t delta_t x_t
        g[n] = av * gn;                                  // dL/dh_{t-1} from step t
      }
      halve_all<2 * N, 5>(v, ul);
      pr[i] = v[0];
      const float xt = xr[P0 + i];
      xr[P0 + i] = dr[P0 + i] * s1;   // dx_t
      dr[P0 + i] = fmaf(xt, s1, s2);  // ddelta_t
    }
    halve_all<S, 5 - T1>(pr, ul);
    float tot = pr[0];
    if constexpr (T3 >= 2) tot += dpp_partner<2>(tot);
    if constexpr (T3 >= 1) tot += dpp_partner<1>(tot);
    {
      const int t = S * j + isum;
      if (writer && t < nth) part[tb + t] = tot;
    }
    // rotate: the outputs to the front, the next piece to the back
    {
      float tx[S], td[S];
#pragma unroll
      for (int i = 0; i < S; ++i) {
        tx[i] = xr[P0 + i];
        td[i] = dr[P0 + i];
      }
#pragma unroll
      for (int k = kHalf - 1; k >= S; --k) {
        xr[k] = xr[k - S];
        dr[k] = dr[k - S];
      }
#pragma unroll
      for (int i = 0; i < S; ++i) {
        xr[i] = tx[i];
        dr[i] = td[i];
      }
#pragma unroll
      for (int q = NP - 1; q >= 1; --q)
#pragma unroll
        for (int n = 0; n < N; ++n) ck[q][n] = ck[q - 1][n];
    }
  }
}

// dy of one half chunk into the wave's token-major array sY[token][lane]
// (zeros past the sequence and for lanes past D), through the staging tile
template <bool VEC>
__device__ __forceinline__ void half_dy(const float* dy, int64_t row0, int rows_valid, int64_t L, int64_t t0h,
                                        int nth, unsigned char* tile, int lane, float (*sY)[64]) {
  float gy[kHalf];
  s6::rows_in<VEC, kHalf>(dy, row0, rows_valid, L, t0h, nth, tile, lane, gy);
#pragma unroll
  for (int t = 0; t < kHalf; ++t) sY[t][lane] = gy[t];
}

// A half chunk's outputs out as whole rows; with ACC, added to what an
// earlier state group's pass left there (fixed order: deterministic)
template <bool VEC, bool ACC>
__device__ __forceinline__ void half_out(float* dst, int64_t row0, int rows_valid, int64_t L, int64_t t0h, int nth,
                                         unsigned char* tile, int lane, float* v) {
  if constexpr (ACC) {
    float prev[kHalf];
    s6::rows_in<VEC, kHalf>(dst, row0, rows_valid, L, t0h, nth, tile, lane, prev);
#pragma unroll
    for (int t = 0; t < kHalf; ++t) v[t] = prev[t] + v[t];
  }
  s6::rows_out<VEC, kHalf>(dst, row0, rows_valid, L, t0h, nth, tile, lane, v);
}

// 3. per (batch row, chunk, 64 channels; one wave): dx, ddelta and the
// chunk's parts of dA, dB and dC for the states n0 .. n0 + N - 1 of NT (N <=
// 4; larger dstates run one pass per group of 4 states, each adding its dx,
// ddelta terms to the earlier passes': ACC). The chunk is taken in halves
// of 32 tokens, the second first: forward over the first half (its piece
// checkpoints kept), forward over the second, backward over the second, then
// the first half's x and delta read again and its backward steps. At most
// 256 registers and 18 KB of LDS: two waves per SIMD.
template <int N, int NT, bool VEC, bool ACC>
__global__ __launch_bounds__(kBwdLanes) __attribute__((amdgpu_waves_per_eu(2))) void s6_bwd_chunk(
    const float* __restrict__ x, const float* __restrict__ dl, const float* __restrict__ A,
    const float* __restrict__ Bm, const float* __restrict__ Cm, const float* __restrict__ dy, const float* h0,
    const float* __restrict__ incl, const float* __restrict__ R, float* dx, float* ddl,
    float* __restrict__ dA_part, float* __restrict__ dB_part, float* __restrict__ dC_part, int64_t L, int D,
    int64_t nc, int n0) {
  static_assert(N <= 4 && NT % N == 0, "at most 4 states per pass");
  constexpr int S = BwdPiece<N>::S, NP = kHalf / S;
  constexpr int T1 = ilog2(2 * N), T3 = 6 - T1 - ilog2(S);
  __shared__ __attribute__((aligned(16))) float sB[N][kChunk];
  __shared__ __attribute__((aligned(16))) float sC[N][kChunk];
  __shared__ __attribute__((aligned(16))) float sY[kHalf][64];
  __shared__ __attribute__((aligned(1024))) unsigned char sT[64 * kHalf * 4];
  const int lane = threadIdx.x;
  const int ncb = (D + kBwdLanes - 1) / kBwdLanes;
  const int64_t c = blockIdx.y;
  const int64_t b = blockIdx.x / ncb;
  const int cb = (int)(blockIdx.x % ncb);
  const int d = cb * kBwdLanes + lane;
  const bool valid = d < D;
  const int64_t t0 = c * kChunk;
  const int nt = L - t0 < kChunk ? (int)(L - t0) : kChunk;
  const int nt0 = nt < kHalf ? nt : kHalf, nt1 = nt > kHalf ? nt - kHalf : 0;
  for (int idx = lane; idx < N * kChunk; idx += kBwdLanes) {
    const int n = idx / kChunk, k = idx % kChunk;
    const int64_t o = (b * NT + n0 + n) * L + t0 + k;
    sB[n][k] = k < nt ? Bm[o] : 0.f;
    sC[n][k] = k < nt ? Cm[o] : 0.f;
  }
  const int64_t wrow0 = b * D + cb * kBwdLanes;
  const int wrows = D - cb * kBwdLanes;
  float xr[kHalf], dr[kHalf];
  s6::rows_in<VEC, kHalf>(x, wrow0, wrows, L, t0, nt0, sT, lane, xr);
  s6::rows_in<VEC, kHalf>(dl, wrow0, wrows, L, t0, nt0, sT, lane, dr);
  float an[N], a2[N], h[N], g[N], dA[N];
  {
    const int64_t rec = (b * nc + c) * D + d;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      an[n] = valid ? A[(int64_t)d * NT + n0 + n] : 0.f;
      a2[n] = an[n] * kLog2e;
      g[n] = valid ? R[rec * NT + n0 + n] : 0.f;
      dA[n] = 0.f;
      if (!valid)
        h[n] = 0.f;
      else if (c == 0)
        h[n] = h0 ? h0[((int64_t)b * D + d) * NT + n0 + n] : 0.f;
      else
        h[n] = incl[(rec - D) * NT + n0 + n];   // chunk c - 1's end state
    }
  }
  __syncthreads();   // B and C staged
  // where this lane's piece sum lands: value v (dB of state v, or dC of
  // state v - N) of token i of the piece; lanes with nonzero low bits hold
  // copies
  const unsigned ul = (unsigned)lane;
  const int vsum = (int)(ul >> (6 - T1)), isum = (int)((ul >> T3) & (S - 1));
  const bool writer = (ul & ((1u << T3) - 1)) == 0;
  float* const part = (vsum < N ? dB_part : dC_part) + ((b * ncb + cb) * NT + n0 + vsum % N) * L + t0;

  float ck0[NP][N];
  half_forward<N, S>(xr, dr, a2, sB, 0, h, ck0);   // h: the state after the first half
  if (nt1 > 0) {
    float ck1[NP][N];
    s6::rows_in<VEC, kHalf>(x, wrow0, wrows, L, t0 + kHalf, nt1, sT, lane, xr);
    s6::rows_in<VEC, kHalf>(dl, wrow0, wrows, L, t0 + kHalf, nt1, sT, lane, dr);
    half_forward<N, S>(xr, dr, a2, sB, kHalf, h, ck1);
    half_dy<VEC>(dy, wrow0, wrows, L, t0 + kHalf, nt1, sT, lane, sY);
    half_backward<N, S>(xr, dr, ck1, an, a2, g, dA, sB, sC, sY, kHalf, lane, part, writer, isum, nt1);
    half_out<VEC, ACC>(dx, wrow0, wrows, L, t0 + kHalf, nt1, sT, lane, xr);
    half_out<VEC, ACC>(ddl, wrow0, wrows, L, t0 + kHalf, nt1, sT, lane, dr);
  }
  if (nt1 > 0) {
    s6::rows_in<VEC, kHalf>(x, wrow0, wrows, L, t0, nt0, sT, lane, xr);
    s6::rows_in<VEC, kHalf>(dl, wrow0, wrows, L, t0, nt0, sT, lane, dr);
  }
  half_dy<VEC>(dy, wrow0, wrows, L, t0, nt0, sT, lane, sY);
  half_backward<N, S>(xr, dr, ck0, an, a2, g, dA, sB, sC, sY, 0, lane, part, writer, isum, nt0);
  half_out<VEC, ACC>(dx, wrow0, wrows, L, t0, nt0, sT, lane, xr);
  half_out<VEC, ACC>(ddl, wrow0, wrows, L, t0, nt0, sT, lane, dr);
  if (valid) {
#pragma unroll
    for (int n = 0; n < N; ++n) dA_part[((b * nc + c) * D + d) * NT + n0 + n] = dA[n];
  }
}

// 4. the sums: dA over batch rows and chunks; dB, dC over channel blocks
// dA: each workgroup takes 64 consecutive (d, n) columns; its 16 waves sum
// every 16th row (batch row, chunk) each, and wave 0 adds the 16 partial
// sums in wave order.
constexpr int kRedWaves = 16;
__global__ __launch_bounds__(64 * kRedWaves) void s6_bwd_reduce_dA(const float* __restrict__ part,
                                                                   float* __restrict__ dA, int64_t rows,
                                                                   int64_t DN) {
  __shared__ float red[kRedWaves][64];
  const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
  const int64_t i = blockIdx.x * (int64_t)64 + lane;
  float s = 0.f;
  if (i < DN) {
#pragma unroll 8
    for (int64_t r = w; r < rows; r += kRedWaves) s += part[r * DN + i];
  }
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && i < DN) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < kRedWaves; ++k) t += red[k][lane];
    dA[i] = t;
  }
}
unsigned dA_grid(int64_t DN) { return (unsigned)(DN > 0 ? (DN + 63) / 64 : 1); }
// dB, dC: the channel blocks' parts summed in block order; V4: four
// consecutive tokens per thread (N L a multiple of 4, dB and dC 16-byte
// aligned)
template <bool V4>
__global__ void s6_bwd_reduce_bc(const float* __restrict__ pb, const float* __restrict__ pc, float* __restrict__ dB,
                                 float* __restrict__ dC, int64_t bt, int ncb, int64_t NL) {
  constexpr int W = V4 ? 4 : 1;
  const int64_t nl = NL / W;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < bt * nl; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / nl, e = (i % nl) * W;
    if constexpr (V4) {
      float4 sb = make_float4(0.f, 0.f, 0.f, 0.f), sc = sb;
      // eight blocks' loads issued before their sums (left to itself the
      // compiler waits for each load in turn)
      int k = 0;
      for (; k + 8 <= ncb; k += 8) {
        float4 vb[8], vc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t o = (b * ncb + k + j) * NL + e;
          vb[j] = *reinterpret_cast<const float4*>(pb + o);
          vc[j] = *reinterpret_cast<const float4*>(pc + o);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          sb.x += vb[j].x; sb.y += vb[j].y; sb.z += vb[j].z; sb.w += vb[j].w;
          sc.x += vc[j].x; sc.y += vc[j].y; sc.z += vc[j].z; sc.w += vc[j].w;
        }
      }
      for (; k < ncb; ++k) {
        const float4 vb = *reinterpret_cast<const float4*>(pb + (b * ncb + k) * NL + e);
        const float4 vc = *reinterpret_cast<const float4*>(pc + (b * ncb + k) * NL + e);
        sb.x += vb.x; sb.y += vb.y; sb.z += vb.z; sb.w += vb.w;
        sc.x += vc.x; sc.y += vc.y; sc.z += vc.z; sc.w += vc.w;
      }
      *reinterpret_cast<float4*>(dB + b * NL + e) = sb;
      *reinterpret_cast<float4*>(dC + b * NL + e) = sc;
    } else {
      float sb = 0.f, sc = 0.f;
#pragma unroll 8
      for (int k = 0; k < ncb; ++k) {
        sb += pb[(b * ncb + k) * NL + e];
        sc += pc[(b * ncb + k) * NL + e];
      }
      dB[b * NL + e] = sb;
      dC[b * NL + e] = sc;
    }
  }
}

unsigned grid_of(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (unsigned)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

template <int N>
hipError_t launch_bwd_n(const S6BwdProblem& p, hipStream_t s) {
  const int64_t nc = (p.L + kChunk - 1) / kChunk;
  const int64_t ncb = (p.D + kBwdLanes - 1) / kBwdLanes;
  const int vec = (p.L % 4 == 0 && p.L <= ((int64_t)1 << 22) && (reinterpret_cast<uintptr_t>(p.x) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.delta) & 15) == 0 && (reinterpret_cast<uintptr_t>(p.dy) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.dx) & 15) == 0 && (reinterpret_cast<uintptr_t>(p.ddelta) & 15) == 0)
                      ? 1 : 0;
  const dim3 grid((unsigned)(p.bt * ncb), (unsigned)nc);
  if (p.bt == 0 || nc == 0) {
    // no token: dA is zero, dh0 the upstream dhT (or zero); nothing else
    hipLaunchKernelGGL(s6_bwd_reduce_dA, dim3(dA_grid(p.D * N)), dim3(64 * kRedWaves), 0, s, p.dA_part, p.dA, (int64_t)0,
                       p.D * N);
    if (p.bt > 0)
      hipLaunchKernelGGL(s6_bwd_carry<N>, dim3(grid_of(p.bt * p.D * N)), dim3(256), 0, s, p.A, p.O, p.SD, p.dhT,
                         p.R, p.dh0, p.bt, (int)p.D, (int64_t)0);
    return hipGetLastError();
  }
  // (O and SD come from the forward sweep, s6_onepass)
  hipLaunchKernelGGL(s6_bwd_carry<N>, dim3(grid_of(p.bt * p.D * N)), dim3(256), 0, s, p.A, p.O, p.SD, p.dhT, p.R,
                     p.dh0, p.bt, (int)p.D, nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one pass per group of (up to) 4 states; passes after the first add to dx, ddelta
  constexpr int NG = N < 4 ? N : 4;
  for (int n0 = 0; n0 < N; n0 += NG) {
    const auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, grid, dim3(kBwdLanes), 0, s, p.x, p.delta, p.A, p.B, p.C, p.dy, p.h0, p.incl, p.R,
                         p.dx, p.ddelta, p.dA_part, p.dB_part, p.dC_part, p.L, (int)p.D, nc, n0);
    };
    if (n0 == 0) {
      if (vec)
        go(s6_bwd_chunk<NG, N, true, false>);
      else
        go(s6_bwd_chunk<NG, N, false, false>);
    } else if constexpr (N > NG) {
      if (vec)
        go(s6_bwd_chunk<NG, N, true, true>);
      else
        go(s6_bwd_chunk<NG, N, false, true>);
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(s6_bwd_reduce_dA, dim3(dA_grid(p.D * N)), dim3(64 * kRedWaves), 0, s, p.dA_part, p.dA, p.bt * nc, p.D * N);
  const int ncbp = (int)ncb;
  if ((N * p.L) % 4 == 0 && (reinterpret_cast<uintptr_t>(p.dB) & 15) == 0 && (reinterpret_cast<uintptr_t>(p.dC) & 15) == 0)
    hipLaunchKernelGGL(s6_bwd_reduce_bc<true>, dim3(grid_of(p.bt * N * p.L / 4)), dim3(256), 0, s, p.dB_part,
                       p.dC_part, p.dB, p.dC, p.bt, ncbp, (int64_t)N * p.L);
  else
    hipLaunchKernelGGL(s6_bwd_reduce_bc<false>, dim3(grid_of(p.bt * N * p.L)), dim3(256), 0, s, p.dB_part, p.dC_part,
                       p.dB, p.dC, p.bt, ncbp, (int64_t)N * p.L);
  return hipGetLastError();
}

}  // namespace

bool s6_bwd_has(int64_t N) { return N == 1 || N == 2 || N == 4 || N == 8 || N == 16; }
int64_t s6_bwd_channel_block() { return kBwdLanes; }

hipError_t launch_s6_bwd(const S6BwdProblem& p, hipStream_t s) {
  switch (p.N) {
    case 1: return launch_bwd_n<1>(p, s);
    case 2: return launch_bwd_n<2>(p, s);
    case 4: return launch_bwd_n<4>(p, s);
    case 8: return launch_bwd_n<8>(p, s);
    case 16: return launch_bwd_n<16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd

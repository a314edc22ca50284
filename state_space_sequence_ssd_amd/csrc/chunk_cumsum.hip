// ssd_chunk_cumsum: chunk-local inclusive cumulative sum of a_t = A[h]*dt_t,
// scaled by log2(e) so that the later kernels evaluate decays with the
// hardware's base-2 exponential (CUDA Tile Mamba-2 blog, section "Kernel 1":
// the sum restarts at every chunk and is stored pre-multiplied by log2 e).
//
// One workgroup per (chunk, block of 32 heads, batch row). The dt tile
// [chunk tokens][32 heads] is read with whole 128-byte rows, scanned per
// head through LDS, and written transposed, [batch][head][token], so the
// consumers read each head's decays contiguously (the blog's "GMEM layout"
// point, done here once for both consumers). Three arrays come out, all
// head-major: dt itself, G' (the scaled cumsum) and the chunk-state weight
// w_t = dt_t * 2^(G'_last - G'_t) <= dt_t that ssd_chunk_state multiplies into
// x (G'_last is the chunk's last G', known here once the scan is done).
//
// Monotonicity. Each head's chunk is split into 8 segments of Q/8 tokens.
// A thread sums its segment sequentially; segment prefixes are then chained
// sequentially, P_{s+1} = P_s + L_s, and element i of segment s becomes
// P_s + local_i. Since local_i only decreases (a_t <= 0), rounding is
// monotone, and the last element of segment s is exactly P_{s+1}, the stored
// sequence never increases along the chunk. So every exponent the causal
// mask keeps later, G'_i - G'_j with i >= j, is <= 0 exactly, as the blog's
// stability argument requires.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kHB = 32;    // heads per workgroup
constexpr int kSeg = 8;    // segments per head (threads per head)

template <int Q>
__global__ __launch_bounds__(256) void ssd_chunk_cumsum(const float* __restrict__ dt,
                                                        const float* __restrict__ A,
                                                        float* __restrict__ gcum,
                                                        float* __restrict__ dtt,
                                                        float* __restrict__ wst,
                                                        int64_t T, int H, int64_t Tp) {
  constexpr int SL = Q / kSeg;
  __shared__ float s_t[Q][kHB + 1];   // dt tile, then the scaled cumsum in place
  __shared__ float s_w[Q][kHB + 1];   // state weights
  __shared__ float s_pre[kSeg][kHB];
  __shared__ float s_lastloc[kHB];

  const int k = blockIdx.x;
  const int h0 = blockIdx.y * kHB;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)k * Q;

  // token-major tile, 32 heads per row: lanes 0..31 read one 128-byte row
  for (int idx = tid; idx < Q * kHB; idx += 256) {
    const int t = idx / kHB, hh = idx % kHB;
    float v = 0.f;
    if (t0 + t < T && h0 + hh < H) v = dt[(b * T + t0 + t) * H + h0 + hh];
    s_t[t][hh] = v;
  }
  __syncthreads();

  // dt, head-major: consecutive lanes write consecutive tokens
  for (int idx = tid; idx < Q * kHB; idx += 256) {
    const int hl = idx / Q, t = idx % Q;
    if (h0 + hl < H) dtt[(b * H + h0 + hl) * Tp + t0 + t] = s_t[t][hl];
  }

  const int hh = tid % kHB, seg = tid / kHB;
  const float a = (h0 + hh < H) ? A[h0 + hh] : 0.f;
  float loc[SL];
  float run = 0.f;
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    run += a * s_t[seg * SL + i][hh];
    loc[i] = run;
  }
  s_pre[seg][hh] = run;
  if (seg == kSeg - 1) s_lastloc[hh] = run;
  __syncthreads();   // also orders the dtt reads of s_t before it is overwritten
  if (seg == 0) {
    float p = 0.f;
#pragma unroll
    for (int s = 0; s < kSeg; ++s) {
      const float tot = s_pre[s][hh];
      s_pre[s][hh] = p;
      p = p + tot;
    }
  }
  __syncthreads();
  const float pre = s_pre[seg][hh];
  // G'_last: the last segment's prefix plus its last local sum, times log2 e
  const float glast = (s_pre[kSeg - 1][hh] + s_lastloc[hh]) * kLog2e;
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    const int t = seg * SL + i;
    const float gv = (pre + loc[i]) * kLog2e;
    s_w[t][hh] = s_t[t][hh] * exp2_hw(glast - gv);
    s_t[t][hh] = gv;
  }
  __syncthreads();

  for (int idx = tid; idx < Q * kHB; idx += 256) {
    const int hl = idx / Q, t = idx % Q;
    if (h0 + hl < H) {
      const int64_t o = (b * H + h0 + hl) * Tp + t0 + t;
      gcum[o] = s_t[t][hl];
      wst[o] = s_w[t][hl];
    }
  }
}

}  // namespace

hipError_t launch_chunk_cumsum(const Problem& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.nc, (unsigned)((p.H + kHB - 1) / kHB), (unsigned)p.bt);
  const dim3 block(256);
  switch (p.Q) {
    case 64:
      hipLaunchKernelGGL(ssd_chunk_cumsum<64>, grid, block, 0, stream, p.dt, p.A, p.gcum, p.dtt, p.wst, p.T, (int)p.H, p.Tp);
      break;
    case 128:
      hipLaunchKernelGGL(ssd_chunk_cumsum<128>, grid, block, 0, stream, p.dt, p.A, p.gcum, p.dtt, p.wst, p.T, (int)p.H, p.Tp);
      break;
    case 256:
      hipLaunchKernelGGL(ssd_chunk_cumsum<256>, grid, block, 0, stream, p.dt, p.A, p.gcum, p.dtt, p.wst, p.T, (int)p.H, p.Tp);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ssd

// ssd_chunk_cumsum: chunk-local inclusive cumulative sum of a_t = A[h]*dt_t,
// scaled by log2(e) so that the later kernels evaluate decays with the
// hardware's base-2 exponential (CUDA Tile Mamba-2 blog, section "Kernel 1":
// the sum restarts at every chunk and is stored pre-multiplied by log2 e).
//
// One workgroup per (block of 16 heads, chunk, batch row). The dt tile
// [chunk tokens][16 heads] is read as whole 64-byte rows (or, for dt given
// head-major, as each head's contiguous run of the chunk's tokens), scanned
// per head through LDS, and written transposed, [batch][head][token], so the
// consumers read each head's decays contiguously (the blog's "GMEM layout"
// point, done here once for both consumers). Three arrays come out, all
// head-major: dt itself, G' (the scaled cumsum) and the chunk-state weight
// w_t = dt_t * 2^(G'_last - G'_t) <= dt_t that ssd_chunk_state multiplies into
// x (G'_last is the chunk's last G', known here once the scan is done).
//
// Monotonicity. Each head's chunk is split into 16 segments of Q/16 tokens.
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

constexpr int kHB = 16;    // heads per workgroup
constexpr int kSeg = 16;   // segments per head (threads per head)

template <int Q>
__global__ __launch_bounds__(256) void ssd_chunk_cumsum(const float* __restrict__ dt,
                                                        const float* __restrict__ A,
                                                        float* __restrict__ gcum,
                                                        float* __restrict__ dtt,
                                                        float* __restrict__ wst,
                                                        int64_t T, int H, int64_t Tp, int dt_hm,
                                                        int* __restrict__ sync, int nsync) {
  constexpr int SL = Q / kSeg;
  __shared__ float s_t[Q][kHB + 1];   // dt tile, then the scaled cumsum in place
  __shared__ float s_w[Q][kHB + 1];   // state weights
  __shared__ float s_pre[kSeg][kHB];
  __shared__ float s_lastloc[kHB];

  const int h0 = blockIdx.x * kHB;
  const int k = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)k * Q;
  // the chained path's counters start at zero (its kernel runs next on the stream)
  if (sync) {
    const int64_t gid = ((int64_t)(blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * 256 + tid;
    const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * gridDim.z * 256;
    for (int64_t i = gid; i < nsync; i += nthreads) sync[i] = 0;
  }
  const int nh = H - h0 < kHB ? H - h0 : kHB;          // heads of this block
  const int nt = T - t0 < Q ? (int)(T - t0) : Q;       // tokens of this chunk
  if (dt_hm) {
    // head-major dt: each head's tokens of the chunk are contiguous; 16-byte
    // pieces when every head row is 16-byte aligned and the chunk is full
    const float* srch = dt + (b * H + h0) * T + t0;
    if (nt == Q && T % 4 == 0 && (reinterpret_cast<uintptr_t>(dt) & 15) == 0) {
      for (int idx = tid; idx < kHB * (Q / 4); idx += 256) {
        const int hh = idx / (Q / 4), t = 4 * (idx % (Q / 4));
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (hh < nh) v = *reinterpret_cast<const float4*>(srch + (int64_t)hh * T + t);
        s_t[t][hh] = v.x; s_t[t + 1][hh] = v.y; s_t[t + 2][hh] = v.z; s_t[t + 3][hh] = v.w;
      }
    } else {
      for (int idx = tid; idx < kHB * Q; idx += 256) {
        const int hh = idx / Q, t = idx % Q;
        s_t[t][hh] = (t < nt && hh < nh) ? srch[(int64_t)hh * T + t] : 0.f;
      }
    }
    __syncthreads();
  } else {
    const float* src = dt + (b * T + t0) * H + h0;

    // token-major tile, kHB heads per row (64 bytes); whole rows as 16-byte
    // pieces when every row of the block is full and 16-byte aligned
    if (nh == kHB && H % 4 == 0 && (reinterpret_cast<uintptr_t>(dt) & 15) == 0) {
      for (int idx = tid; idx < Q * (kHB / 4); idx += 256) {
        const int t = idx / (kHB / 4), c = idx % (kHB / 4);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < nt) v = *reinterpret_cast<const float4*>(src + (int64_t)t * H + 4 * c);
        s_t[t][4 * c] = v.x; s_t[t][4 * c + 1] = v.y; s_t[t][4 * c + 2] = v.z; s_t[t][4 * c + 3] = v.w;
      }
    } else {
      for (int idx = tid; idx < Q * kHB; idx += 256) {
        const int t = idx / kHB, hh = idx % kHB;
        s_t[t][hh] = (t < nt && hh < nh) ? src[(int64_t)t * H + hh] : 0.f;
      }
    }
    __syncthreads();
  }

  // dt, head-major: each thread writes 4 consecutive tokens of one head
  for (int idx = tid; idx < (Q / 4) * kHB; idx += 256) {
    const int hl = idx / (Q / 4), t = 4 * (idx % (Q / 4));
    if (hl < nh)
      *reinterpret_cast<float4*>(dtt + (b * H + h0 + hl) * Tp + t0 + t) =
          make_float4(s_t[t][hl], s_t[t + 1][hl], s_t[t + 2][hl], s_t[t + 3][hl]);
  }

  const int hh = tid % kHB, seg = tid / kHB;
  const float a = hh < nh ? A[h0 + hh] : 0.f;
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

  for (int idx = tid; idx < (Q / 4) * kHB; idx += 256) {
    const int hl = idx / (Q / 4), t = 4 * (idx % (Q / 4));
    if (hl < nh) {
      const int64_t o = (b * H + h0 + hl) * Tp + t0 + t;
      *reinterpret_cast<float4*>(gcum + o) = make_float4(s_t[t][hl], s_t[t + 1][hl], s_t[t + 2][hl], s_t[t + 3][hl]);
      if (wst)
        *reinterpret_cast<float4*>(wst + o) = make_float4(s_w[t][hl], s_w[t + 1][hl], s_w[t + 2][hl], s_w[t + 3][hl]);
    }
  }
}

}  // namespace

hipError_t launch_chunk_cumsum(const Problem& p, hipStream_t stream) {
  // head blocks fastest, so neighbouring workgroups read the same dt rows
  const dim3 grid((unsigned)((p.H + kHB - 1) / kHB), (unsigned)p.nc, (unsigned)p.bt);
  const dim3 block(256);
  switch (p.Q) {
    case 64:
      hipLaunchKernelGGL(ssd_chunk_cumsum<64>, grid, block, 0, stream, p.dt, p.A, p.gcum, p.dtt, p.wst, p.T, (int)p.H, p.Tp, p.dt_head_major, p.sync, p.nsync);
      break;
    case 128:
      hipLaunchKernelGGL(ssd_chunk_cumsum<128>, grid, block, 0, stream, p.dt, p.A, p.gcum, p.dtt, p.wst, p.T, (int)p.H, p.Tp, p.dt_head_major, p.sync, p.nsync);
      break;
    case 256:
      hipLaunchKernelGGL(ssd_chunk_cumsum<256>, grid, block, 0, stream, p.dt, p.A, p.gcum, p.dtt, p.wst, p.T, (int)p.H, p.Tp, p.dt_head_major, p.sync, p.nsync);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ssd

// The Mamba-1 selective scan (S6): one scalar state per (batch row, channel
// d, state n), discretized per step ("Mamba: The Hard Way", Part 5):
//
//   h[n] <- exp(delta_t A[d, n]) h[n] + delta_t B[n, t] x_t,   y_t = sum_n C[n, t] h[n]
//
// Layouts: x, delta, y [batch][channels][seqlen]; B, C [batch][dstate][seqlen];
// A [channels][dstate]; states [batch][channels][dstate]; all fp32.
//
// The sequence is cut into chunks of kChunk tokens, scanned in parallel:
//   s6_chunk<N, false>  each (b, d, chunk) scans its tokens from a zero state:
//                       the chunk's end state S and its sum of delta;
//   s6_carry<N>         per (b, d, n), the chunks in order: the state entering
//                       each chunk, h <- 2^(log2e A sum(delta)) h + S (the
//                       chunk's decays multiply to exp(A sum(delta))), and
//                       the final state;
//   s6_chunk<N, true>   each (b, d, chunk) scans again from its entering
//                       state and writes y.
// The "Part 2/3" view of the page is the same: a scan splits into blocks
// whose summaries combine associatively. A thread owns one channel of one
// chunk, its N states in registers; a workgroup takes 256 channels of one
// chunk, so the chunk's B and C rows are staged once in LDS, and each wave
// stages its 64 channels' x and delta in 16-token column blocks (64-byte row
// pieces, then each lane walks its own row) and y the same way back, in
// the x tile (a lane overwrites the x values of its own row it has read).
// Two column blocks are loaded ahead: the scan itself is short, and one
// memory round trip per block would set the time; at about 100 registers
// per lane four waves fit per SIMD, so a 1024-channel, 2048-token, 8-row
// call runs all its waves at once.
#include "ssd_device.h"
#include "s6_launch.h"

namespace ssd {

namespace {

constexpr int kChunk = 64;    // tokens per chunk
constexpr int kSub = 16;      // tokens per staged column block
constexpr int kWaves = 4;     // waves per workgroup, 64 channels each

// A lane's share of one wave's 64 rows x kSub tokens of a [rows][L] array:
// rows 16 i + lane / 4, tokens t + 4 (lane % 4) .. + 3 (zeros past the
// sequence or the channels).
__device__ __forceinline__ void load_rows(float4 (&v)[4], const float* src, int64_t row0, int rows_valid,
                                          int64_t L, int64_t t, int lane, bool vec) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = i * 16 + lane / 4, piece = lane % 4;
    const int64_t tk = t + piece * 4;
    float e[4] = {0.f, 0.f, 0.f, 0.f};
    if (r < rows_valid) {
      const float* p = src + (row0 + r) * L + tk;
      if (vec && tk + 3 < L) {
        const float4 q = *reinterpret_cast<const float4*>(p);
        e[0] = q.x; e[1] = q.y; e[2] = q.z; e[3] = q.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (tk + j < L) e[j] = p[j];
      }
    }
    v[i] = make_float4(e[0], e[1], e[2], e[3]);
  }
}
// ... and those values into the wave's LDS tile [64 rows][kSub + 1]
__device__ __forceinline__ void store_rows(float (*dst)[kSub + 1], const float4 (&v)[4], int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = i * 16 + lane / 4, piece = lane % 4;
    dst[r][piece * 4 + 0] = v[i].x;
    dst[r][piece * 4 + 1] = v[i].y;
    dst[r][piece * 4 + 2] = v[i].z;
    dst[r][piece * 4 + 3] = v[i].w;
  }
}

template <int N, bool FINAL>
__global__ __launch_bounds__(256) void s6_chunk(const float* __restrict__ x, const float* __restrict__ dl,
                                                const float* __restrict__ A, const float* __restrict__ Bm,
                                                const float* __restrict__ Cm, const float* __restrict__ hin,
                                                float* __restrict__ y, float* __restrict__ S,
                                                float* __restrict__ sumd, int64_t L, int D, int64_t nc, int vec) {
  __shared__ __attribute__((aligned(16))) float sB[N][kChunk];
  __shared__ __attribute__((aligned(16))) float sC[FINAL ? N : 1][kChunk];
  __shared__ float sx[kWaves][64][kSub + 1];
  __shared__ float sd[kWaves][64][kSub + 1];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int64_t b = blockIdx.z, c = blockIdx.y;
  const int dw = blockIdx.x * 256 + wave * 64;          // the wave's first channel
  const int d = dw + lane;
  const bool valid = d < D;
  const int rows_valid = D - dw;                         // channels of this wave (may be <= 0)
  const int64_t t0 = c * kChunk;
  const int nt = L - t0 < kChunk ? (int)(L - t0) : kChunk;
  const int64_t row0 = b * D + dw;
  constexpr int NB = kChunk / kSub;
  // two column blocks in flight: blocks 0 and 1 now, block kb + 2 into the
  // registers block kb has just left
  float4 xr[2][4], dr[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    load_rows(xr[kb], x, row0, rows_valid, L, t0 + kb * kSub, lane, vec);
    load_rows(dr[kb], dl, row0, rows_valid, L, t0 + kb * kSub, lane, vec);
  }

  for (int idx = tid; idx < N * kChunk; idx += 256) {
    const int n = idx / kChunk, k = idx % kChunk;
    const int64_t o = (b * N + n) * L + t0 + k;
    sB[n][k] = k < nt ? Bm[o] : 0.f;
    if (FINAL) sC[n][k] = k < nt ? Cm[o] : 0.f;
  }
  float a2[N], h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    a2[n] = valid ? A[(int64_t)d * N + n] * kLog2e : 0.f;
    h[n] = (FINAL && valid) ? hin[(((int64_t)b * D + d) * nc + c) * N + n] : 0.f;
  }
  float dsum = 0.f;
  __syncthreads();   // B and C staged
  // From here each wave touches only its own tiles, and one wave's LDS
  // operations complete in program order: no workgroup barrier is needed.
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {
    const int ks = kb * kSub;
    if (ks >= nt) break;
    store_rows(sx[wave], xr[kb & 1], lane);
    store_rows(sd[wave], dr[kb & 1], lane);
    if (kb + 2 < NB) {
      load_rows(xr[kb & 1], x, row0, rows_valid, L, t0 + (kb + 2) * kSub, lane, vec);
      load_rows(dr[kb & 1], dl, row0, rows_valid, L, t0 + (kb + 2) * kSub, lane, vec);
    }
    const int kn = nt - ks < kSub ? nt - ks : kSub;
    // four tokens at a time: B and C of a state for 4 tokens in one 16-byte
    // read. Past the sequence x, delta, B and C are zero, so the padded
    // tokens of the last group leave h unchanged (exp2(0) = 1, no input).
    for (int k4 = 0; k4 < kn; k4 += 4) {
      float dv[4], u[4], yv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dv[j] = sd[wave][lane][k4 + j];
        u[j] = dv[j] * sx[wave][lane][k4 + j];
        dsum += dv[j];
      }
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const float4 b4 = *reinterpret_cast<const float4*>(&sB[n][ks + k4]);
        const float bj[4] = {b4.x, b4.y, b4.z, b4.w};
        float cj[4] = {0.f, 0.f, 0.f, 0.f};
        if (FINAL) {
          const float4 c4 = *reinterpret_cast<const float4*>(&sC[n][ks + k4]);
          cj[0] = c4.x; cj[1] = c4.y; cj[2] = c4.z; cj[3] = c4.w;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h[n] = fmaf(exp2_hw(dv[j] * a2[n]), h[n], u[j] * bj[j]);
          if (FINAL) yv[j] = fmaf(cj[j], h[n], yv[j]);
        }
      }
      if (FINAL) {
        // y replaces x in the lane's own row: those x values are read above
#pragma unroll
        for (int j = 0; j < 4; ++j) sx[wave][lane][k4 + j] = yv[j];
      }
    }
    if (FINAL) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i * 16 + lane / 4, piece = lane % 4;
        if (r >= rows_valid) continue;
        float* p = y + (row0 + r) * L + t0 + ks + piece * 4;
        if (vec && piece * 4 + 3 < kn) {
          *reinterpret_cast<float4*>(p) = make_float4(sx[wave][r][piece * 4], sx[wave][r][piece * 4 + 1],
                                                      sx[wave][r][piece * 4 + 2], sx[wave][r][piece * 4 + 3]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (piece * 4 + j < kn) p[j] = sx[wave][r][piece * 4 + j];
        }
      }
    }
  }
  if (!FINAL && valid) {
    const int64_t o = ((int64_t)b * D + d) * nc + c;
#pragma unroll
    for (int n = 0; n < N; ++n) S[o * N + n] = h[n];
    sumd[o] = dsum;
  }
}

// per (b, d, n): the state entering every chunk, and the final state
template <int N>
__global__ void s6_carry(const float* __restrict__ A, const float* __restrict__ S, const float* __restrict__ sumd,
                         const float* __restrict__ h0, float* __restrict__ hin, float* __restrict__ hT, int64_t rows,
                         int D, int64_t nc) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;   // (b * D + d) * N + n
  if (i >= rows * N) return;
  const int64_t bd = i / N;
  const int n = (int)(i % N), d = (int)(bd % D);
  const float a2 = A[(int64_t)d * N + n] * kLog2e;
  float h = h0 ? h0[i] : 0.f;
  for (int64_t c = 0; c < nc; ++c) {
    const int64_t o = bd * nc + c;
    hin[o * N + n] = h;
    h = fmaf(exp2_hw(a2 * sumd[o]), h, S[o * N + n]);
  }
  if (hT) hT[i] = h;
}

template <int N>
hipError_t launch_n(const S6Problem& p, hipStream_t s) {
  const int64_t nc = (p.L + kChunk - 1) / kChunk;
  const int64_t rows = p.bt * p.D;
  // 16-byte row pieces of x, delta and y when every row starts 16-byte aligned
  const int vec = (p.L % 4 == 0 && (reinterpret_cast<uintptr_t>(p.x) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.delta) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.y) & 15) == 0) ? 1 : 0;
  const dim3 grid((unsigned)((p.D + 255) / 256), (unsigned)nc, (unsigned)p.bt);
  if (nc > 0 && rows > 0) {
    hipLaunchKernelGGL((s6_chunk<N, false>), grid, dim3(256), 0, s, p.x, p.delta, p.A, p.B, p.C,
                       (const float*)nullptr, (float*)nullptr, p.S, p.sumd, p.L, (int)p.D, nc, vec);
  }
  if (rows > 0) {
    const int64_t threads = rows * N;
    hipLaunchKernelGGL((s6_carry<N>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p.A, p.S, p.sumd,
                       p.h0, p.hin, p.hT, rows, (int)p.D, nc);
  }
  if (nc > 0 && rows > 0) {
    hipLaunchKernelGGL((s6_chunk<N, true>), grid, dim3(256), 0, s, p.x, p.delta, p.A, p.B, p.C, p.hin, p.y,
                       (float*)nullptr, (float*)nullptr, p.L, (int)p.D, nc, vec);
  }
  return hipGetLastError();
}

}  // namespace

int64_t s6_chunk_tokens() { return kChunk; }

bool s6_has(int64_t N) { return N == 1 || N == 2 || N == 4 || N == 8 || N == 16; }

hipError_t launch_s6(const S6Problem& p, hipStream_t s) {
  switch (p.N) {
    case 1: return launch_n<1>(p, s);
    case 2: return launch_n<2>(p, s);
    case 4: return launch_n<4>(p, s);
    case 8: return launch_n<8>(p, s);
    case 16: return launch_n<16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd

// The backward pass of the SSD layer: every input's gradient from the
// upstream gradients dy (like y) and dfinal (like the final state).
//
// Source of the method: the chunked "jump" form of the forward pass (NVIDIA
// developer blog "Accelerating Mamba-2 with high-performance forward-pass
// kernels in NVIDIA CUDA Tile", section "Mamba-2 architecture") differentiated
// block by block, and the observation of "Part 3" of Sasha Rush's "Mamba: The
// Hard Way" that the state's adjoint runs the same scan backwards in time.
// Per chunk of Q tokens, with G' the chunk-local cumsum of A dt times log2 e,
// E_i = 2^(G'_i), L_ij = 2^(G'_i - G'_j) (i >= j, else 0), w_j = dt_j
// 2^(G'_last - G'_j), Hprev the state entering the chunk and dHn the adjoint
// of the state leaving it:
//
//   dHprev = 2^(G'_last) dHn + dY^T diag(E) C            (reverse chunk pass)
//   dx     = (L o CB o dt_j)^T dY + diag(w) B dHn^T + D dY
//   dB_h   = (L o DX o dt_j)^T C  + diag(w) X dHn         (summed over a group)
//   dC_h   = (L o DX o dt_j) B    + diag(E) dY Hprev      (summed over a group)
//
// with CB = C B^T and DX = dY X^T, and the gradient with respect to the
// natural-log cumsum G (rows minus columns of Z = L o CB o DX o dt_j, the
// carried-state and chunk-end terms) passed to dt and A through
// G_i = A sum_{s <= i} dt_s.
//
// This first form favours clarity over speed: fp32 throughout (bf16 inputs
// are exact in fp32), the contractions as one batched fp32 GEMM kernel with
// LDS tiles, and small elementwise kernels between them, all through a
// caller-provided workspace.
#include "ssd_bwd.h"
#include "ssd_device.h"

namespace ssd {

namespace {

// ---------------------------------------------------------------- GEMM
// C[z] = beta C[z] + diag(rs[z]) (A[z] diag(ks[z]) B[z]), fp32. Every operand
// is addressed by a base pointer, element strides (row, col) and a batch
// offset z0 s0 + z1 s1 + (z2 / d2) s2 for z = (z0 Z1 + z1) Z2 + z2; the
// divisor d2 maps a head index to its group for operands shared by a group.
// Scale vectors may be null (ones).
constexpr int GT = 64, GK = 16;   // output tile GT x GT, k-step GK; 256 threads, a 32 x 32 quarter per wave

struct Operand {
  const float* p;
  int64_t rs, cs;        // element strides of rows and columns
  int64_t s0, s1, s2;    // batch strides
  int d2;                // z2 divisor
  __device__ int64_t base(int z0, int z1, int z2) const { return z0 * s0 + z1 * s1 + (int64_t)(z2 / d2) * s2; }
};

// Causal shapes. The Q x Q blocks are used on and below the diagonal only:
// kLowerOut computes only output tiles that reach it (the others are never
// read), kKFromRow / kKToRow limit the contraction to k >= m (A upper
// triangular, a transposed lower block) or k <= m (A lower triangular).
enum : int { kFull = 0, kLowerOut = 1, kKFromRow = 2, kKToRow = 3 };

struct GemmArgs {
  Operand a, b, c, rsc, ksc;   // rsc / ksc: only p, s0..s2, d2 used (unit stride vectors)
  int M, N, K, Z1, Z2;
  float beta;
  int shape;
  int vec;                     // operands staged as 16-byte pieces (see gemm())
  // optional second product added to the first: the sum over hsum heads of
  // (diag(rsc2_head) A2_head) B2_head, contraction length K2 over the full
  // range (no causal shape); only without an output row scale
  Operand a2, b2, rsc2;
  int K2;
  int hsum;                    // heads the second product sums (>= 1 when a2 is set)
  int cvec;                    // output rows contiguous and 16-byte aligned (see gemm())
};

// Stage one GK-deep slice of A (GT rows from m0) and B (GT columns from n0)
// into LDS as [k][m] and [k][n]; rows, columns and k past the operands are
// zero.
__device__ __forceinline__ void stage_k(float (*sa)[GT + 4], float (*sb)[GT + 4], const Operand& ao,
                                        const Operand& bo, const float* A, const float* B, const float* ks,
                                        const float* ra, int m0, int n0, int k0, int M, int N, int kend, int vec,
                                        int tid) {
  // consecutive threads walk whichever index is contiguous in memory
  const bool a_k_unit = ao.cs == 1, b_n_unit = bo.cs == 1;
  if (vec) {
    // one 16-byte piece per thread and operand, along the contiguous index
    if (a_k_unit) {
      const int mm = tid / 4, kq = (tid % 4) * 4, m = m0 + mm;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m < M) {
        v = *reinterpret_cast<const float4*>(A + m * ao.rs + k0 + kq);
        if (ks) {
          const float4 s4 = *reinterpret_cast<const float4*>(ks + k0 + kq);
          v.x *= s4.x; v.y *= s4.y; v.z *= s4.z; v.w *= s4.w;
        }
        if (ra) {
          const float r = ra[m];
          v.x *= r; v.y *= r; v.z *= r; v.w *= r;
        }
      }
      sa[kq][mm] = v.x; sa[kq + 1][mm] = v.y; sa[kq + 2][mm] = v.z; sa[kq + 3][mm] = v.w;
    } else {
      const int kk = tid / 16, mq = (tid % 16) * 4, k = k0 + kk;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m0 + mq < M) {
        v = *reinterpret_cast<const float4*>(A + (m0 + mq) + k * ao.cs);
        if (ks) {
          const float sk = ks[k];
          v.x *= sk; v.y *= sk; v.z *= sk; v.w *= sk;
        }
        if (ra) {
          v.x *= ra[m0 + mq]; v.y *= ra[m0 + mq + 1]; v.z *= ra[m0 + mq + 2]; v.w *= ra[m0 + mq + 3];
        }
      }
      *reinterpret_cast<float4*>(&sa[kk][mq]) = v;
    }
    if (b_n_unit) {
      const int kb = tid / 16, nq = (tid % 16) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (n0 + nq < N) v = *reinterpret_cast<const float4*>(B + (k0 + kb) * bo.rs + n0 + nq);
      *reinterpret_cast<float4*>(&sb[kb][nq]) = v;
    } else {
      const int nn = tid / 4, kq = (tid % 4) * 4, n = n0 + nn;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (n < N) v = *reinterpret_cast<const float4*>(B + (k0 + kq) + n * bo.cs);
      sb[kq][nn] = v.x; sb[kq + 1][nn] = v.y; sb[kq + 2][nn] = v.z; sb[kq + 3][nn] = v.w;
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = tid + 256 * e;          // 0 .. 1023
    const int kk = a_k_unit ? idx % GK : idx / GT, mm = a_k_unit ? idx / GK : idx % GT;
    const int m = m0 + mm, k = k0 + kk;
    float v = 0.f;
    if (m < M && k < kend) {
      v = A[m * ao.rs + k * ao.cs];
      if (ks) v *= ks[k];
      if (ra) v *= ra[m];
    }
    sa[kk][mm] = v;
    const int nn = b_n_unit ? idx % GT : idx / GK, kb = b_n_unit ? idx / GT : idx % GK;
    const int n = n0 + nn, kq = k0 + kb;
    sb[kb][nn] = (n < N && kq < kend) ? B[kq * bo.rs + n * bo.cs] : 0.f;
  }
}

// The 16-byte path of stage_k in two halves, so the loads of the next slice
// can be in flight while this slice's MFMAs run: kload reads a thread's
// pieces of A and B (and the scale factors) into registers, kstore applies
// the scales and writes them into LDS.
struct KSlice {
  float4 a, b, sa4;   // A piece, B piece, A scales (k scales or row scales)
  float sa1;          // the other A scale (a row scale or a k scale)
};
__device__ __forceinline__ void kload(KSlice& v, const Operand& ao, const Operand& bo, const float* A,
                                      const float* B, const float* ks, const float* ra, int m0, int n0, int k0,
                                      int M, int N, int tid) {
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f), o4 = make_float4(1.f, 1.f, 1.f, 1.f);
  v.a = z4;
  v.sa4 = o4;
  v.sa1 = 1.f;
  if (ao.cs == 1) {
    const int mm = tid / 4, kq = (tid % 4) * 4, m = m0 + mm;
    if (m < M) {
      v.a = *reinterpret_cast<const float4*>(A + m * ao.rs + k0 + kq);
      if (ks) v.sa4 = *reinterpret_cast<const float4*>(ks + k0 + kq);
      if (ra) v.sa1 = ra[m];
    }
  } else {
    const int kk = tid / 16, mq = (tid % 16) * 4, k = k0 + kk;
    if (m0 + mq < M) {
      v.a = *reinterpret_cast<const float4*>(A + (m0 + mq) + k * ao.cs);
      if (ks) v.sa1 = ks[k];
      if (ra) v.sa4 = make_float4(ra[m0 + mq], ra[m0 + mq + 1], ra[m0 + mq + 2], ra[m0 + mq + 3]);
    }
  }
  v.b = z4;
  if (bo.cs == 1) {
    const int kb = tid / 16, nq = (tid % 16) * 4;
    if (n0 + nq < N) v.b = *reinterpret_cast<const float4*>(B + (k0 + kb) * bo.rs + n0 + nq);
  } else {
    const int nn = tid / 4, kq = (tid % 4) * 4, n = n0 + nn;
    if (n < N) v.b = *reinterpret_cast<const float4*>(B + (k0 + kq) + n * bo.cs);
  }
}
__device__ __forceinline__ void kstore(float (*sa)[GT + 4], float (*sb)[GT + 4], const KSlice& v, const Operand& ao,
                                       const Operand& bo, int tid) {
  // (x k scale) then (x row scale), as stage_k multiplies
  const bool kfirst = ao.cs == 1;   // sa4 holds the k scales
  const float4 a = kfirst ? make_float4(v.a.x * v.sa4.x * v.sa1, v.a.y * v.sa4.y * v.sa1, v.a.z * v.sa4.z * v.sa1,
                                        v.a.w * v.sa4.w * v.sa1)
                          : make_float4(v.a.x * v.sa1 * v.sa4.x, v.a.y * v.sa1 * v.sa4.y, v.a.z * v.sa1 * v.sa4.z,
                                        v.a.w * v.sa1 * v.sa4.w);
  if (ao.cs == 1) {
    const int mm = tid / 4, kq = (tid % 4) * 4;
    sa[kq][mm] = a.x; sa[kq + 1][mm] = a.y; sa[kq + 2][mm] = a.z; sa[kq + 3][mm] = a.w;
  } else {
    const int kk = tid / 16, mq = (tid % 16) * 4;
    *reinterpret_cast<float4*>(&sa[kk][mq]) = a;
  }
  if (bo.cs == 1) {
    const int kb = tid / 16, nq = (tid % 16) * 4;
    *reinterpret_cast<float4*>(&sb[kb][nq]) = v.b;
  } else {
    const int nn = tid / 4, kq = (tid % 4) * 4;
    sb[kq][nn] = v.b.x; sb[kq + 1][nn] = v.b.y; sb[kq + 2][nn] = v.b.z; sb[kq + 3][nn] = v.b.w;
  }
}

// HAS2: the optional second product (only the dB and dC products have it);
// without it the kernel needs fewer registers
template <bool HAS2>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HAS2 ? 3 : 4))) void bwd_gemm(GemmArgs g) {
  // one LDS block: the A and B slices while the products run, then the
  // output staging (every wave has passed the last slice's barrier by then)
  constexpr int kSlice = GK * (GT + 4), kStage = 4 * 32 * 40;
  __shared__ __attribute__((aligned(16))) float lds[2 * kSlice > kStage ? 2 * kSlice : kStage];
  float (*sa)[GT + 4] = reinterpret_cast<float (*)[GT + 4]>(lds);
  float (*sb)[GT + 4] = reinterpret_cast<float (*)[GT + 4]>(lds + kSlice);
  const int tiles_n = (g.N + GT - 1) / GT;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int z = blockIdx.y;
  const int z2 = z % g.Z2, z1 = (z / g.Z2) % g.Z1, z0 = z / (g.Z2 * g.Z1);
  const int tid = threadIdx.x;
  const int m0 = tm * GT, n0 = tn * GT;
  if (g.shape == kLowerOut && n0 > m0 + GT - 1) return;   // wholly above the diagonal
  const int kbeg = g.shape == kKFromRow ? m0 : 0;
  const int kend = g.shape == kKToRow ? min(g.K, m0 + GT) : g.K;
  // each wave computes one 32 x 32 quarter of the tile with the fp32 MFMA
  // (32x32x2): lane l supplies A[row l%32][k l/32] and B[k l/32][col l%32]
  const int wave = tid / 64, lane = tid % 64, lm = lane % 32, lg = lane / 32;
  const int wm = 32 * (wave / 2), wn = 32 * (wave % 2);
  f32x16 acc = f32x16{};
  {
    const float* A = g.a.p + g.a.base(z0, z1, z2);
    const float* B = g.b.p + g.b.base(z0, z1, z2);
    const float* ks = g.ksc.p ? g.ksc.p + g.ksc.base(z0, z1, z2) : nullptr;
    if (g.vec) {
      // the next slice's loads are issued before this slice's MFMAs
      KSlice v;
      if (kbeg < kend) kload(v, g.a, g.b, A, B, ks, nullptr, m0, n0, kbeg, g.M, g.N, tid);
      for (int k0 = kbeg; k0 < kend; k0 += GK) {
        kstore(sa, sb, v, g.a, g.b, tid);
        __syncthreads();
        if (k0 + GK < kend) kload(v, g.a, g.b, A, B, ks, nullptr, m0, n0, k0 + GK, g.M, g.N, tid);
#pragma unroll
        for (int kk = 0; kk < GK; kk += 2)
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sa[kk + lg][wm + lm], sb[kk + lg][wn + lm], acc, 0, 0, 0);
        __syncthreads();
      }
    } else {
      for (int k0 = kbeg; k0 < kend; k0 += GK) {
        stage_k(sa, sb, g.a, g.b, A, B, ks, nullptr, m0, n0, k0, g.M, g.N, kend, g.vec, tid);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < GK; kk += 2)
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sa[kk + lg][wm + lm], sb[kk + lg][wn + lm], acc, 0, 0, 0);
        __syncthreads();
      }
    }
  }
  if (HAS2 && g.a2.p) {
    // the second product, summed over hsum consecutive heads of the batch
    // index (head z2 * hsum + hl), each A2 row scaled by its head's rsc2 row
    // before the sum, into the same accumulators (the host allows a second
    // product only with hsum > 0 and no output row scale)
    for (int hl = 0; hl < g.hsum; ++hl) {
      const int zh = z2 * g.hsum + hl;
      const float* A = g.a2.p + g.a2.base(z0, z1, zh);
      const float* B = g.b2.p + g.b2.base(z0, z1, zh);
      const float* ra = g.rsc2.p ? g.rsc2.p + g.rsc2.base(z0, z1, zh) : nullptr;
      if (g.vec) {
        KSlice v;
        if (g.K2 > 0) kload(v, g.a2, g.b2, A, B, nullptr, ra, m0, n0, 0, g.M, g.N, tid);
        for (int k0 = 0; k0 < g.K2; k0 += GK) {
          kstore(sa, sb, v, g.a2, g.b2, tid);
          __syncthreads();
          if (k0 + GK < g.K2) kload(v, g.a2, g.b2, A, B, nullptr, ra, m0, n0, k0 + GK, g.M, g.N, tid);
#pragma unroll
          for (int kk = 0; kk < GK; kk += 2)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sa[kk + lg][wm + lm], sb[kk + lg][wn + lm], acc, 0, 0, 0);
          __syncthreads();
        }
      } else {
        for (int k0 = 0; k0 < g.K2; k0 += GK) {
          stage_k(sa, sb, g.a2, g.b2, A, B, nullptr, ra, m0, n0, k0, g.M, g.N, g.K2, g.vec, tid);
          __syncthreads();
#pragma unroll
          for (int kk = 0; kk < GK; kk += 2)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sa[kk + lg][wm + lm], sb[kk + lg][wn + lm], acc, 0, 0, 0);
          __syncthreads();
        }
      }
    }
  }
  float* Cp = const_cast<float*>(g.c.p) + g.c.base(z0, z1, z2);
  const float* rs = g.rsc.p ? g.rsc.p + g.rsc.base(z0, z1, z2) : nullptr;
  if (g.cvec && g.beta == 0.f && m0 + GT <= g.M && n0 + GT <= g.N) {
    // whole tile, row-major output: each wave's 32 x 32 quarter goes out
    // through LDS as 16-byte row pieces, 4 stores per lane instead of 16
    // (rows of 32 values plus 8 of padding: the two half-waves write rows 4
    // apart, 32 banks apart)
    float (*q)[40] = reinterpret_cast<float (*)[40]>(lds + wave * 32 * 40);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int mr = drow(r, lg);
      float v = (rs ? rs[m0 + wm + mr] : 1.f) * acc[r];
      q[mr][lm] = v;
    }
    // a wave's own LDS operations complete in order: no barrier
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 8 * i + lane / 8, c4 = (lane % 8) * 4;
      const float4 v = *reinterpret_cast<const float4*>(&q[row][c4]);
      *reinterpret_cast<float4*>(Cp + (int64_t)(m0 + wm + row) * g.c.rs + n0 + wn + c4) = v;
    }
    return;
  }
  const int n = n0 + wn + lm;
  if (n >= g.N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + wm + drow(r, lg);   // the accumulator's row for this lane and register
    if (m >= g.M) continue;
    float* cp = Cp + m * g.c.rs + n * g.c.cs;
    float v = (rs ? rs[m] : 1.f) * acc[r];
    *cp = g.beta == 0.f ? v : fmaf(g.beta, *cp, v);
  }
}

Operand op(const float* p, int64_t rs, int64_t cs, int64_t s0, int64_t s1, int64_t s2, int d2 = 1) {
  return Operand{p, rs, cs, s0, s1, s2, d2};
}
Operand none() { return Operand{nullptr, 0, 0, 0, 0, 0, 1}; }

hipError_t gemm(const Operand& a, const Operand& b, const Operand& c, const Operand& rsc, const Operand& ksc,
                int M, int N, int K, int Z0, int Z1, int Z2, float beta, hipStream_t s, int shape = kFull,
                const Operand* a2 = nullptr, const Operand* b2 = nullptr, const Operand* rsc2 = nullptr,
                int K2 = 0, int hsum = 0) {
  // 16-byte staging needs every 4-element piece along the contiguous index
  // aligned and wholly inside or outside the operand: bases 16-byte aligned,
  // all other strides multiples of 4, and K, M, N multiples of 4
  auto al4 = [](const Operand& o) {
    return (reinterpret_cast<uintptr_t>(o.p) & 15) == 0 && o.s0 % 4 == 0 && o.s1 % 4 == 0 && o.s2 % 4 == 0 &&
           (o.rs == 1 || o.rs % 4 == 0) && (o.cs == 1 || o.cs % 4 == 0) && (o.rs == 1 || o.cs == 1);
  };
  const Operand no{nullptr, 0, 0, 0, 0, 0, 1};
  const int vec = al4(a) && al4(b) && (!ksc.p || al4(Operand{ksc.p, 1, 1, ksc.s0, ksc.s1, ksc.s2, ksc.d2})) &&
                  K % 16 == 0 && M % 4 == 0 && N % 4 == 0 && (!a2 || (al4(*a2) && al4(*b2) && K2 % 16 == 0));
  // 16-byte output pieces: unit column stride, row and batch strides
  // multiples of 4, base 16-byte aligned
  const int cvec = c.cs == 1 && (reinterpret_cast<uintptr_t>(c.p) & 15) == 0 && c.rs % 4 == 0 && c.s0 % 4 == 0 &&
                   c.s1 % 4 == 0 && c.s2 % 4 == 0;
  GemmArgs g{a, b, c, rsc, ksc, M, N, K, Z1, Z2, beta, shape, vec, a2 ? *a2 : no, b2 ? *b2 : no,
             rsc2 ? *rsc2 : no, K2, hsum, cvec};
  const int64_t tiles = (int64_t)((M + GT - 1) / GT) * ((N + GT - 1) / GT);
  const int64_t Z = (int64_t)Z0 * Z1 * Z2;
  if (Z == 0 || tiles == 0) return hipSuccess;
  if (Z > kMaxGridYZ) return hipErrorInvalidValue;
  if (a2 && (hsum <= 0 || rsc.p)) return hipErrorInvalidValue;   // see bwd_gemm
  if (a2)
    hipLaunchKernelGGL(bwd_gemm<true>, dim3((unsigned)tiles, (unsigned)Z), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(bwd_gemm<false>, dim3((unsigned)tiles, (unsigned)Z), dim3(256), 0, s, g);
  return hipGetLastError();
}

// ---------------------------------------------------------- elementwise
template <typename T> __device__ __forceinline__ float ld(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<bf16>(const bf16* p, int64_t i) {
  return __uint_as_float((uint32_t)(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
}

// rows [bt][T][W] of the io type -> fp32 [bt][Tp][W], zero rows past T
template <typename T>
__global__ void pad_rows(const T* __restrict__ src, float* __restrict__ dst, int64_t T_, int64_t Tp, int64_t W,
                         int64_t total) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t w = i % W, t = (i / W) % Tp, b = i / (W * Tp);
    dst[i] = t < T_ ? ld(src, (b * T_ + t) * W + w) : 0.f;
  }
}

// The same, 8 values per thread (W a multiple of 8, both arrays 16-byte
// aligned): one 16-byte (bf16) or two (fp32) loads and two 16-byte stores,
// so a thread's loads are not each issued behind its previous store.
template <typename T> __device__ __forceinline__ void ld8(const T* p, float* v);
template <> __device__ __forceinline__ void ld8<float>(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <> __device__ __forceinline__ void ld8<bf16>(const bf16* p, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <typename T>
__global__ void pad_rows8(const T* __restrict__ src, float* __restrict__ dst, int64_t T_, int64_t Tp, int64_t W,
                          int64_t total8) {
  const int64_t W8 = W / 8;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total8; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t w8 = i % W8, t = (i / W8) % Tp, b = i / (W8 * Tp);
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (t < T_) ld8(src + (b * T_ + t) * W + 8 * w8, v);
    float4* d = reinterpret_cast<float4*>(dst + 8 * i);
    d[0] = make_float4(v[0], v[1], v[2], v[3]);
    d[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

__global__ void exp2_all(const float* __restrict__ g, float* __restrict__ e, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    e[i] = exp2_hw(g[i]);
}

// The chunk recursion over one (b, h) state, one thread per state element:
// forward (rev = 0): out[k] = h; h = 2^(G'_last,k) h + S[k], from init (or 0);
// reverse (rev = 1): out[k] = h; h = 2^(G'_last,k) h + S[k] for k from the
// last chunk down, from dfinal (or 0), and the end value goes to `last`.
__global__ void chunk_recursion(const float* __restrict__ S, const float* __restrict__ gcum,
                                const float* __restrict__ h0, float* __restrict__ out, float* __restrict__ last,
                                int64_t nc, int64_t Tp, int64_t Q, int64_t PN, int64_t total, int rev) {
  // chunks are taken CR at a time with their loads issued first: a load
  // issued after the previous chunk's store would wait for it
  constexpr int CR = 16;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bh = i / PN, e = i % PN;
    float h = h0 ? h0[i] : 0.f;
    for (int64_t s0 = 0; s0 < nc; s0 += CR) {
      float sv[CR], gv[CR];
#pragma unroll
      for (int c = 0; c < CR; ++c) {
        const int64_t s = s0 + c;
        const int64_t k = rev ? nc - 1 - s : s;
        sv[c] = s < nc ? S[(bh * nc + k) * PN + e] : 0.f;
        gv[c] = s < nc ? gcum[bh * Tp + k * Q + Q - 1] : 0.f;
      }
#pragma unroll
      for (int c = 0; c < CR; ++c) {
        const int64_t s = s0 + c;
        if (s >= nc) break;
        const int64_t k = rev ? nc - 1 - s : s;
        out[(bh * nc + k) * PN + e] = h;
        h = fmaf(exp2_hw(gv[c]), h, sv[c]);
      }
    }
    if (last) last[i] = h;
  }
}

// Per (b, k, h): the masked, decayed blocks W1s = L o CB o dt_j (in its own
// array) and W2s = L o DX o dt_j (over DX, in place), zero above the
// diagonal where they are read, and the sums the time gradient needs: rows
// and columns of Z = L o CB o DX o dt_j, and the columns of L o CB o DX.
// One thread per column walks the rows once: it writes the blocks, keeps
// its column sums, and leaves its Z entries of MD_ROWS rows in LDS, where
// one wave per row adds them up (lane l takes columns l, l + 64, ...; then
// a butterfly over the lanes). Fixed summation orders: the result does not
// depend on scheduling.
constexpr int MD_ROWS = 16;
__global__ __launch_bounds__(256) void mask_decay(const float* __restrict__ CB, float* __restrict__ DXW2,
                                                  float* __restrict__ W1, const float* __restrict__ gcum,
                                                  const float* __restrict__ dtt, float* __restrict__ rowZ,
                                                  float* __restrict__ colZ, float* __restrict__ colW,
                                                  int Q, int H, int hpg, int64_t nc, int64_t Tp) {
  __shared__ float sg[256], sd[256];
  __shared__ float sz[MD_ROWS][256 + 4];
  const int h = blockIdx.x % H;
  const int64_t k = (blockIdx.x / H) % nc, b = blockIdx.x / (H * nc);
  const int64_t QQ = (int64_t)Q * Q;
  const float* cb = CB + ((b * nc + k) * (H / hpg) + h / hpg) * QQ;
  float* dx = DXW2 + ((b * nc + k) * H + h) * QQ;
  float* w1 = W1 + ((b * nc + k) * H + h) * QQ;
  const int64_t tb = (b * H + h) * Tp + k * Q;
  for (int i = threadIdx.x; i < Q; i += blockDim.x) {
    sg[i] = gcum[tb + i];
    sd[i] = dtt[tb + i];
  }
  __syncthreads();
  // Q <= 256 = blockDim.x: thread j owns column j. Entries above the
  // diagonal are read only inside the GT x GT blocks on it (the causal
  // products run their contraction from the first row of an output tile, or
  // to its last): only those are cleared.
  const int j = threadIdx.x, wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const bool col = j < Q;
  const float gj = col ? sg[j] : 0.f, dj = col ? sd[j] : 0.f;
  const int ifirst = (j / GT) * GT;
  float cz = 0.f, cw = 0.f;
  for (int i0 = 0; i0 < Q; i0 += MD_ROWS) {
    // the block's loads first, so they are in flight together (issued after
    // the previous block's stores, a load would wait for them)
    float cbv[MD_ROWS], dxv[MD_ROWS];
#pragma unroll
    for (int r = 0; r < MD_ROWS; ++r) {
      const int i = i0 + r;
      const int64_t o = (int64_t)i * Q + j;
      const bool lower = col && i >= j;
      cbv[r] = lower ? cb[o] : 0.f;
      dxv[r] = lower ? dx[o] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < MD_ROWS; ++r) {
      const int i = i0 + r;
      float z = 0.f;
      if (col && i >= ifirst) {
        const int64_t o = (int64_t)i * Q + j;
        if (i < j) {
          w1[o] = 0.f;
          dx[o] = 0.f;
        } else {
          const float L = exp2_hw(sg[i] - gj);
          const float lcb = L * cbv[r], d = dxv[r];
          w1[o] = lcb * dj;
          dx[o] = L * d * dj;
          z = lcb * d * dj;
          cz += z;
          cw += lcb * d;
        }
      }
      sz[r][j] = z;
    }
    __syncthreads();
    for (int rr = 0; rr < MD_ROWS / 4; ++rr) {
      const int r = wave * (MD_ROWS / 4) + rr;
      float v = 0.f;
      for (int jj = lane; jj < Q; jj += 64) v += sz[r][jj];
#pragma unroll
      for (int off = 32; off >= 1; off /= 2) v += __shfl_xor(v, off, 64);
      if (lane == 0) rowZ[tb + i0 + r] = v;
    }
    __syncthreads();   // the rows are summed before the next block overwrites them
  }
  if (col) {
    colZ[tb + j] = cz;
    colW[tb + j] = cw;
  }
}

// Per (b, h, k), Q threads: dx (output), ddt (output), and this chunk's
// parts of dA and dD. U = B dHn^T and V = C Hprev^T rows, dXp = W1s^T dY.
__global__ __launch_bounds__(256) void finish_chunk(const BwdProblem p) {
  __shared__ float s_dg[256], s_dt[256], s_red[256], s_avec[256], s_bvec[256], s_ddx[256];
  __shared__ float s_scal[2];
  const int Q = (int)p.Q, P = (int)p.P, H = (int)p.H;
  const int h = blockIdx.x % H;
  const int64_t k = (blockIdx.x / H) % p.nc, b = blockIdx.x / (H * p.nc);
  const int i = threadIdx.x;
  const int64_t tb = (b * H + h) * p.Tp + k * Q;
  const int64_t t = k * Q + i;   // this thread's token in the per-token steps
  const int64_t PN = p.P * p.N;
  const float* Hp = p.hprev + ((b * H + h) * p.nc + k) * PN;
  const float* dHn = p.dhn + ((b * H + h) * p.nc + k) * PN;
  // <dHn, Hprev> over the block
  float part = 0.f;
  for (int64_t e = i; e < PN; e += blockDim.x) part += dHn[e] * Hp[e];
  s_red[i] = part;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s /= 2) {
    if (i < s) s_red[i] += s_red[i + s];
    __syncthreads();
  }
  if (i == 0) s_scal[0] = s_red[0];
  __syncthreads();

  // per-row dot products over headdim, one wave per row at a time with its
  // lanes across the row (whole-row reads), and dx written on the way
  {
    const int wave = i / 64, lane = i % 64;
    const float D = p.D[h];
    for (int r = wave; r < Q; r += blockDim.x / 64) {
      const int64_t tr = k * Q + r;
      const int64_t row = ((b * p.Tp + tr) * H + h) * P;           // [bt][Tp][H][P] rows
      const int64_t urow = (((b * p.nc + k) * H + h) * Q + r) * P;  // [bt][nc][H][Q][P] rows
      const float wr = p.wst[tb + r];
      float a = 0.f, bb = 0.f, dd = 0.f;
      for (int q = lane; q < P; q += 64) {
        const float xv = p.Xp[row + q], dyv = p.dYp[row + q], u = p.U[urow + q];
        a += dyv * p.V[urow + q];
        bb += xv * u;
        dd += dyv * xv;
        if (tr < p.T) p.dx[((b * p.T + tr) * H + h) * P + q] = p.dXp[row + q] + wr * u + D * dyv;
      }
#pragma unroll
      for (int off = 32; off >= 1; off /= 2) {
        a += __shfl_xor(a, off, 64);
        bb += __shfl_xor(bb, off, 64);
        dd += __shfl_xor(dd, off, 64);
      }
      if (lane == 0) {
        s_avec[r] = a;
        s_bvec[r] = bb;
        s_ddx[r] = dd;
      }
    }
  }
  __syncthreads();
  float bvec = 0.f, dterm = 0.f, gi = 0.f, wi = 0.f;
  if (i < Q) {
    const float E = p.E[tb + i];
    wi = p.wst[tb + i];
    gi = p.gcum[tb + i];
    const float avec = s_avec[i];
    bvec = s_bvec[i];
    dterm = s_ddx[i];
    s_dg[i] = E * avec + p.rowZ[tb + i] - p.colZ[tb + i] - wi * bvec;
    s_dt[i] = p.dtt[tb + i];
  }
  __syncthreads();
  // the chunk-end term: 2^(G'_last) <dHn, Hprev> + sum_j w_j bvec_j
  s_red[i] = (i < Q) ? wi * bvec : 0.f;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s /= 2) {
    if (i < s) s_red[i] += s_red[i + s];
    __syncthreads();
  }
  if (i == 0) {
    const float glast = p.gcum[tb + Q - 1];
    s_dg[Q - 1] += exp2_hw(glast) * s_scal[0] + s_red[0];
  }
  __syncthreads();
  if (i == 0) {
    // sequential scans over the chunk (Q <= 256): reverse cumsum of dG into
    // s_red, and the chunk's dA part sum_i dG_i * cumdt_i
    float acc = 0.f;
    for (int j = Q - 1; j >= 0; --j) {
      acc += s_dg[j];
      s_red[j] = acc;
    }
    float cum = 0.f, da = 0.f;
    for (int j = 0; j < Q; ++j) {
      cum += s_dt[j];
      da += s_dg[j] * cum;
    }
    p.dA_part[(b * H + h) * p.nc + k] = da;
  }
  __syncthreads();
  if (i < Q && t < p.T) {
    const float glast = p.gcum[tb + Q - 1];
    p.ddt[(b * p.T + t) * H + h] = p.colW[tb + i] + exp2_hw(glast - gi) * bvec + p.A[h] * s_red[i];
  }
  // dD part: sum over the chunk of dy . x
  __syncthreads();
  s_red[i] = (i < Q) ? dterm : 0.f;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s /= 2) {
    if (i < s) s_red[i] += s_red[i + s];
    __syncthreads();
  }
  if (i == 0) p.dD_part[(b * H + h) * p.nc + k] = s_red[0];
}

// sum over the heads of each group of the Q x Q blocks [bt][nc][H][Q][Q]
// -> [bt][nc][G][Q][Q]
__global__ void sum_heads(const float* __restrict__ in, float* __restrict__ out, int hpg, int Q, int64_t QQ,
                          int64_t total4) {
  // four adjacent values of a row per thread (Q a multiple of 4): 16-byte
  // loads, one per head, and one 16-byte store
  for (int64_t i4 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i4 < total4;
       i4 += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = 4 * i4;
    const int64_t o = i % QQ, bkg = i / QQ;   // (b * nc + k) * G + g
    if ((o % Q) / GT > (o / Q) / GT) continue;   // a GT x GT block above the diagonal: never read
    const float* src = in + bkg * hpg * QQ + o;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < hpg; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(src + j * QQ);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    *reinterpret_cast<float4*>(out + i) = acc;
  }
}

// [bt][Tp][H][N] -> [bt][T][G][N]: the sum over each group's heads of the
// padded rows (with H = G: the unpadding copy)
__global__ void group_sum(const float* __restrict__ part, float* __restrict__ out, int64_t T_, int64_t Tp, int H,
                          int G, int64_t N, int64_t total) {
  const int hpg = H / G;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = i % N, g = (i / N) % G, t = (i / (N * G)) % T_, b = i / (N * G * T_);
    const float* src = part + ((b * Tp + t) * H + g * hpg) * N + n;
    float s = 0.f;
    for (int j = 0; j < hpg; ++j) s += src[j * N];
    out[i] = s;
  }
}

// dA, dD: sums over batch rows and chunks of the per-(b, h, k) parts
__global__ void head_sums(const float* __restrict__ dA_part, const float* __restrict__ dD_part, float* __restrict__ dA,
                          float* __restrict__ dD, int64_t bt, int H, int64_t nc) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  float sa = 0.f, sd = 0.f;
  for (int64_t b = 0; b < bt; ++b)
    for (int64_t k = 0; k < nc; ++k) {
      sa += dA_part[(b * H + h) * nc + k];
      sd += dD_part[(b * H + h) * nc + k];
    }
  dA[h] = sa;
  dD[h] = sd;
}

unsigned grid_for(int64_t total) {
  const int64_t g = (total + 255) / 256;
  return (unsigned)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

}  // namespace

BwdLayout bwd_layout(int64_t bt, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q, int64_t nc, int io) {
  BwdLayout L{};
  // the fused kernels need no padded x or dy and no per-head Q x Q blocks:
  // DX holds the per-segment W2 sums, U and V the transposed states
  const bool fused = bwd_fused_supported(io, P, N, Q);
  const int64_t nseg = fused ? bwd_fused_segments(bt, nc, H, G) : 0;
  const int64_t Tp = nc * Q;
  size_t off = 0;
  auto take = [&](size_t floats) {
    const size_t o = off;
    off = (off + floats * 4 + 255) / 256 * 256;
    return o;
  };
  L.gcum = take(bt * H * Tp);
  L.dtt = take(bt * H * Tp);
  L.wst = take(bt * H * Tp);
  L.E = take(bt * H * Tp);
  L.Xp = take(fused ? 0 : bt * Tp * H * P);
  L.dYp = take(fused ? 0 : bt * Tp * H * P);
  L.Bp = take(bt * Tp * G * N);
  L.Cp = take(bt * Tp * G * N);
  L.S = take(bt * H * nc * P * N);
  L.hprev = take(bt * H * nc * P * N);
  L.dhn = take(bt * H * nc * P * N);
  L.CB = take(bt * nc * G * Q * Q);
  L.DX = take(fused ? bt * nc * G * nseg * Q * Q : bt * nc * H * Q * Q);
  L.W1 = take(fused ? 0 : bt * nc * H * Q * Q);
  L.U = take(fused ? bt * H * nc * P * N : bt * nc * H * Q * P);
  L.V = take(fused ? bt * H * nc * P * N : bt * nc * H * Q * P);
  L.dXp = take(bt * Tp * H * P);
  L.dBh = take(bt * Tp * G * N);
  L.dCh = take(bt * Tp * G * N);
  L.rowZ = take(bt * H * Tp);
  L.colZ = take(bt * H * Tp);
  L.colW = take(bt * H * Tp);
  L.dA_part = take(bt * H * nc);
  L.dD_part = take(bt * H * nc);
  L.total = off;
  return L;
}

hipError_t launch_ssd_bwd(BwdProblem p, hipStream_t s) {
  const int64_t bt = p.bt, T = p.T, H = p.H, P = p.P, N = p.N, G = p.G, Q = p.Q, nc = p.nc, Tp = p.Tp;
  const int hpg = (int)(H / G);
  const int64_t PN = P * N, QQ = Q * Q;
  hipError_t e = hipSuccess;
  auto ok = [&](hipError_t r) {
    if (e == hipSuccess) e = r;
    return e == hipSuccess;
  };
  // 1. inputs to padded fp32, and 2^(G')
  const int64_t nx = bt * Tp * H * P, nb = bt * Tp * G * N;
  // inputs to padded fp32 rows, 8 values per thread where the rows allow
  auto pad = [&](const void* src, float* dst, int64_t W, int64_t n) {
    const bool v8 = W % 8 == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
    if (p.io == 1) {
      if (v8)
        hipLaunchKernelGGL(pad_rows8<bf16>, dim3(grid_for(n / 8)), dim3(256), 0, s, (const bf16*)src, dst, T, Tp, W, n / 8);
      else
        hipLaunchKernelGGL(pad_rows<bf16>, dim3(grid_for(n)), dim3(256), 0, s, (const bf16*)src, dst, T, Tp, W, n);
    } else {
      if (v8)
        hipLaunchKernelGGL(pad_rows8<float>, dim3(grid_for(n / 8)), dim3(256), 0, s, (const float*)src, dst, T, Tp, W,
                           n / 8);
      else
        hipLaunchKernelGGL(pad_rows<float>, dim3(grid_for(n)), dim3(256), 0, s, (const float*)src, dst, T, Tp, W, n);
    }
  };
  const bool fused = bwd_fused_supported(p.io, P, N, Q);
  if (!fused) {   // (the fused kernels read x and dy as they are)
    pad(p.x, p.Xp, H * P, nx);
    pad(p.dy, p.dYp, H * P, nx);
  }
  pad(p.B, p.Bp, G * N, nb);
  pad(p.C, p.Cp, G * N, nb);
  const int64_t ng = bt * H * Tp;
  hipLaunchKernelGGL(exp2_all, dim3(grid_for(ng)), dim3(256), 0, s, p.gcum, p.E, ng);
  if (!ok(hipGetLastError())) return e;

  // batch order of the chunk GEMMs: z = (b, k, h); tile bases
  const int Bi = (int)bt, Ki = (int)nc, Hi = (int)H, Qi = (int)Q, Pi = (int)P, Ni = (int)N;
  // x / dy tile (b, k, h): rows i at stride H P
  const Operand X = op(p.Xp, H * P, 1, Tp * H * P, Q * H * P, P);
  const Operand dY = op(p.dYp, H * P, 1, Tp * H * P, Q * H * P, P);
  const Operand Bt = op(p.Bp, G * N, 1, Tp * G * N, Q * G * N, N, hpg);
  const Operand Ct = op(p.Cp, G * N, 1, Tp * G * N, Q * G * N, N, hpg);
  // per-(b, h, k) vectors over the chunk's tokens, [bt][H][Tp]
  auto vec = [&](const float* v) { return op(v, 0, 0, H * Tp, Q, Tp); };
  // per-(b, h, k) P x N blocks, [bt][H][nc][P][N], for the (b, k, h) batch order
  auto blk = [&](const float* v, bool transposed) {
    return transposed ? op(v, 1, N, H * nc * PN, PN, nc * PN) : op(v, N, 1, H * nc * PN, PN, nc * PN);
  };

  // chunk-state products on the forward pass's own kernel where it has the
  // shape (bf16 operands on the bf16 MFMA, read from the unpadded inputs)
  const bool cs_kernel = chunk_state_has(p.io, P, N, Q);
  auto chunk_states = [&](const void* xin, const void* bin, float* weights) {
    if (bt * nc * H == 0) return hipSuccess;   // no chunk: nothing to launch
    Problem f{};
    f.bt = bt; f.T = T; f.H = H; f.P = P; f.N = N; f.G = G; f.Q = Q; f.nc = nc; f.Tp = Tp; f.io = p.io;
    f.x = xin; f.B = bin; f.wst = weights; f.states = p.S;
    return launch_chunk_state(f, s);
  };
  // 2. forward chunk states S = X^T diag(wst) B, then Hprev
  if (cs_kernel)
    ok(chunk_states(p.x, p.B, p.wst));
  else
    ok(gemm(op(p.Xp, 1, H * P, Tp * H * P, Q * H * P, P), Bt, blk(p.S, false), none(), vec(p.wst), Pi, Ni, Qi, Bi, Ki,
            Hi, 0.f, s));
  const int64_t nst = bt * H * PN;
  if (e == hipSuccess) {
    hipLaunchKernelGGL(chunk_recursion, dim3(grid_for(nst)), dim3(256), 0, s, p.S, p.gcum, p.init, p.hprev,
                       (float*)nullptr, nc, Tp, Q, PN, nst, 0);
    ok(hipGetLastError());
  }
  // 3. dS = dY^T diag(E) C, then the reverse pass: dHn per chunk, dinit
  if (cs_kernel)
    ok(chunk_states(p.dy, p.C, p.E));
  else
    ok(gemm(op(p.dYp, 1, H * P, Tp * H * P, Q * H * P, P), Ct, blk(p.S, false), none(), vec(p.E), Pi, Ni, Qi, Bi, Ki,
            Hi, 0.f, s));
  if (e == hipSuccess) {
    hipLaunchKernelGGL(chunk_recursion, dim3(grid_for(nst)), dim3(256), 0, s, p.S, p.gcum, p.dfinal, p.dhn, p.dinit,
                       nc, Tp, Q, PN, nst, 1);
    ok(hipGetLastError());
  }
  if (!fused) {
    // 6. U = B dHn^T, V = C Hprev^T (rows j: dHn B_j, Hprev C_j)
    const Operand Uo = op(p.U, P, 1, nc * H * Q * P, H * Q * P, Q * P);
    const Operand Vo = op(p.V, P, 1, nc * H * Q * P, H * Q * P, Q * P);
    ok(gemm(Bt, blk(p.dhn, true), Uo, none(), none(), Qi, Pi, Ni, Bi, Ki, Hi, 0.f, s));
    ok(gemm(Ct, blk(p.hprev, true), Vo, none(), none(), Qi, Pi, Ni, Bi, Ki, Hi, 0.f, s));
  }
  if (fused) {
    // 4, 5, 7 and the group sums of W2 in one pass over each chunk's heads
    ok(launch_bwd_fused_qq(p, p.DX, bwd_fused_segments(bt, nc, H, G), s));
  } else {
    // 4. CB = C B^T per (b, k, g) and DX = dY X^T per (b, k, h)
    ok(gemm(op(p.Cp, G * N, 1, Tp * G * N, Q * G * N, N), op(p.Bp, 1, G * N, Tp * G * N, Q * G * N, N),
            op(p.CB, Q, 1, nc * G * QQ, G * QQ, QQ), none(), none(), Qi, Qi, Ni, Bi, Ki, (int)G, 0.f, s, kLowerOut));
    ok(gemm(dY, op(p.Xp, 1, H * P, Tp * H * P, Q * H * P, P), op(p.DX, Q, 1, nc * H * QQ, H * QQ, QQ), none(), none(),
            Qi, Qi, Pi, Bi, Ki, Hi, 0.f, s, kLowerOut));
    // 5. masks, decays, and the sums for the time gradient
    if (e == hipSuccess && bt * nc * H > 0) {
      hipLaunchKernelGGL(mask_decay, dim3((unsigned)(bt * nc * H)), dim3(256), 0, s, p.CB, p.DX, p.W1, p.gcum, p.dtt,
                         p.rowZ, p.colZ, p.colW, Qi, Hi, hpg, nc, Tp);
      ok(hipGetLastError());
    }
    // 7. dXp = W1s^T dY
    const Operand Wqq1T = op(p.W1, 1, Q, nc * H * QQ, H * QQ, QQ);
    ok(gemm(Wqq1T, dY, op(p.dXp, H * P, 1, Tp * H * P, Q * H * P, P), none(), none(), Qi, Pi, Qi, Bi, Ki, Hi, 0.f, s,
            kKFromRow));
    // the group's sum of the heads' W2s blocks (over CB, no longer needed)
    const int64_t nsum = bt * nc * G * QQ;
    if (e == hipSuccess && nsum > 0) {
      hipLaunchKernelGGL(sum_heads, dim3(grid_for(nsum / 4)), dim3(256), 0, s, p.DX, p.CB, hpg, Qi, QQ, nsum / 4);
      ok(hipGetLastError());
    }
  }
  // 8. dB_h = W2s^T C + diag(w) X dHn;  dC_h = W2s B + diag(E) dY Hprev
  // per (b, k, group): B and C are shared by the group's heads, so the
  // causal products take the sum of the heads' W2s blocks, and the state
  // products sum the heads' parts
  // 9. dx, ddt and the dA / dD parts; then the group and head sums
  const Operand W2g = op(p.CB, Q, 1, nc * G * QQ, G * QQ, QQ), W2gT = op(p.CB, 1, Q, nc * G * QQ, G * QQ, QQ);
  const Operand Bg = op(p.Bp, G * N, 1, Tp * G * N, Q * G * N, N), Cg = op(p.Cp, G * N, 1, Tp * G * N, Q * G * N, N);
  const Operand dBg = op(p.dBh, G * N, 1, Tp * G * N, Q * G * N, N), dCg = op(p.dCh, G * N, 1, Tp * G * N, Q * G * N, N);
  if (fused) {
    // the finishing kernel (U and V formed on the fly) also leaves the states
    // transposed for the head-summed state products; the causal products are
    // added on top
    ok(launch_bwd_fused_finish(p, s));
    ok(launch_bwd_fused_headsum(p, p.x, p.wst, p.U, p.dBh, s));
    ok(launch_bwd_fused_headsum(p, p.dy, p.E, p.V, p.dCh, s));
    ok(gemm(W2gT, Cg, dBg, none(), none(), Qi, Ni, Qi, Bi, Ki, (int)G, 1.f, s, kKFromRow));
    ok(gemm(W2g, Bg, dCg, none(), none(), Qi, Ni, Qi, Bi, Ki, (int)G, 1.f, s, kKToRow));
  } else {
    const Operand dhn = blk(p.dhn, false), hpv = blk(p.hprev, false), w = vec(p.wst), ev = vec(p.E);
    ok(gemm(W2gT, Cg, dBg, none(), none(), Qi, Ni, Qi, Bi, Ki, (int)G, 0.f, s, kKFromRow, &X, &dhn, &w, Pi, hpg));
    ok(gemm(W2g, Bg, dCg, none(), none(), Qi, Ni, Qi, Bi, Ki, (int)G, 0.f, s, kKToRow, &dY, &hpv, &ev, Pi, hpg));
    if (e == hipSuccess && bt * nc * H > 0) {
      hipLaunchKernelGGL(finish_chunk, dim3((unsigned)(bt * nc * H)), dim3(256), 0, s, p);
      ok(hipGetLastError());
    }
  }
  const int64_t nbo = bt * T * G * N;
  if (e == hipSuccess && nbo > 0) {
    hipLaunchKernelGGL(group_sum, dim3(grid_for(nbo)), dim3(256), 0, s, p.dBh, p.dB, T, Tp, (int)G, (int)G, N, nbo);
    hipLaunchKernelGGL(group_sum, dim3(grid_for(nbo)), dim3(256), 0, s, p.dCh, p.dC, T, Tp, (int)G, (int)G, N, nbo);
    ok(hipGetLastError());
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(head_sums, dim3((unsigned)((H + 255) / 256)), dim3(256), 0, s, p.dA_part, p.dD_part, p.dA,
                       p.dD, bt, Hi, nc);
    ok(hipGetLastError());
  }
  return e;
}

}  // namespace ssd

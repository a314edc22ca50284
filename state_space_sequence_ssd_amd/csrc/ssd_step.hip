// ssd_step: one token of the SSD recurrence for every (batch row, head), the
// recurrent ("decode") form of the same layer:
//
//   state[p, n] <- exp(A * dt) * state[p, n] + dt * x[p] * B[n]
//   y[p]         = sum_n C[n] * state[p, n] + D * x[p]
//
// (CUDA Tile Mamba-2 blog, section "Mamba-2 architecture": the core
// recurrence h_t = exp(A dt_t) h_{t-1} + dt_t B_t x_t^T, y_t = c_t^T h_t +
// D x_t, which the blog notes suits token-by-token inference; the final
// state of a chunked forward call is this recurrence's state.)
//
// The step reads and writes the whole fp32 state once, so it is bound by HBM
// bandwidth: per (batch row, head) 8 P N bytes of state traffic against
// 3 P N flops. Work split: a state row (b, h, p) of N floats is covered by
// L = N/4 consecutive lanes, 16 bytes each (whole 16-byte pieces; one
// wave-instruction reads 64/L whole rows). A thread walks R rows that lie
// 256/L rows apart, so each thread has R independent 16-byte loads in flight
// before it computes. y[p] is a sum over the row's L lanes (xor shuffles).
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kStepThreads = 256;
constexpr int kStepRows = 4;   // rows per thread (loads in flight)

template <typename T> struct StepIo;
template <> struct StepIo<float> {
  // 4 consecutive elements
  __device__ static __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
  __device__ static __forceinline__ void store1(float* p, float v) { *p = v; }
};
template <> struct StepIo<bf16> {
  __device__ static __forceinline__ float4 load4(const bf16* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y));
  }
  __device__ static __forceinline__ float load1(const bf16* p) {
    return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
  }
  __device__ static __forceinline__ void store1(bf16* p, float v) {
    *reinterpret_cast<uint16_t*>(p) = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
  }
};

template <typename T, int N>
__global__ __launch_bounds__(kStepThreads) void ssd_step_kernel(
    const T* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dp,
    float* __restrict__ state, T* __restrict__ y, uint32_t rows, uint32_t P, uint32_t H, uint32_t hpg,
    uint32_t G) {
  using S = StepIo<T>;
  constexpr int L = N / 4;                       // lanes per state row
  constexpr int RPP = kStepThreads / L;          // rows per pass of the block
  const int lane_in_row = threadIdx.x % L;
  const uint32_t row0 = blockIdx.x * (uint32_t)(RPP * kStepRows) + threadIdx.x / L;
  const int n0 = lane_in_row * 4;

  float4 s[kStepRows];
  // issue every state load first
#pragma unroll
  for (int i = 0; i < kStepRows; ++i) {
    const uint32_t r = row0 + i * RPP;
    if (r < rows) s[i] = *reinterpret_cast<const float4*>(state + (size_t)r * N + n0);
  }
#pragma unroll
  for (int i = 0; i < kStepRows; ++i) {
    const uint32_t r = row0 + i * RPP;
    if (r >= rows) continue;                     // whole row groups of L lanes skip together
    const uint32_t bh = r / P;                   // b * H + h
    const uint32_t b = bh / H, h = bh - b * H;
    const uint32_t bc = (b * G + h / hpg) * (uint32_t)N + (uint32_t)n0;
    const float d = dt[bh];
    const float alpha = exp2_hw(A[h] * d * kLog2e);   // exp(A dt) <= 1
    const float xv = S::load1(x + r);
    const float xd = xv * d;
    const float4 bv = S::load4(Bm + bc);
    const float4 cv = S::load4(Cm + bc);
    float4 o;
    o.x = fmaf(alpha, s[i].x, xd * bv.x);
    o.y = fmaf(alpha, s[i].y, xd * bv.y);
    o.z = fmaf(alpha, s[i].z, xd * bv.z);
    o.w = fmaf(alpha, s[i].w, xd * bv.w);
    *reinterpret_cast<float4*>(state + (size_t)r * N + n0) = o;
    float acc = cv.x * o.x + cv.y * o.y + cv.z * o.z + cv.w * o.w;
#pragma unroll
    for (int off = L / 2; off >= 1; off /= 2) acc += __shfl_xor(acc, off, L);
    if (lane_in_row == 0) S::store1(y + r, acc + Dp[h] * xv);
  }
}

template <typename T, int N>
hipError_t launch_n(const StepProblem& p, hipStream_t stream) {
  const uint64_t rows = (uint64_t)p.bt * p.H * p.P;
  constexpr int RPB = (kStepThreads / (N / 4)) * kStepRows;
  const uint64_t blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((ssd_step_kernel<T, N>), dim3((uint32_t)blocks), dim3(kStepThreads), 0, stream,
                     static_cast<const T*>(p.x), p.dt, p.A, static_cast<const T*>(p.B),
                     static_cast<const T*>(p.C), p.D, p.state, static_cast<T*>(p.y), (uint32_t)rows,
                     (uint32_t)p.P, (uint32_t)p.H, (uint32_t)(p.H / p.G), (uint32_t)p.G);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const StepProblem& p, hipStream_t stream) {
  switch (p.N) {
    case 64: return launch_n<T, 64>(p, stream);
    case 128: return launch_n<T, 128>(p, stream);
    case 256: return launch_n<T, 256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool step_has(int io, int64_t N) { return (io == 0 || io == 1) && (N == 64 || N == 128 || N == 256); }

hipError_t launch_ssd_step(const StepProblem& p, hipStream_t stream) {
  if (p.bt * p.H * p.P == 0) return hipSuccess;
  return p.io == 1 ? launch_t<bf16>(p, stream) : launch_t<float>(p, stream);
}

}  // namespace ssd

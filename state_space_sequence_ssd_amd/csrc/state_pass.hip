// ssd_state_pass: the sequential recurrence across chunk checkpoints
// (CUDA Tile Mamba-2 blog, section "Kernel 2: fwd_pass_state": for each
// chunk in order, record the state entering it, then jump over it with
// h <- exp(G_last) * h + S_k; the last state is the final state).
//
//   h = init (or 0)
//   for k in 0 .. nchunks-1:  hprev[k] = h;  h = 2^(G'_last,k) * h + S[k]
//   final = h
//
// Every (batch, head, element of the headdim x dstate state) is an
// independent chain, so the grid is (batch*head, state/1024) and each thread
// carries 4 consecutive state elements through all chunks in fp32
// registers. The kernel is pure streaming: S is read once and hprev written
// once; loads for later chunks are issued ahead of the dependent FMAs so each
// thread keeps several 16-byte reads in flight.
//
// hprev format. With fp32 io, hprev is the fp32 state. With bf16 io it is
// stored as ready-made MFMA operand pairs: the fp32 state h is split as
// hi = bf16(h), lo = bf16(h - hi), and for every row p and every aligned
// group of 8 dstate columns the 8 hi values are followed by the 8 lo values
// (32 bytes, the same size as the fp32 values). The output kernel then loads
// a lane's hi and lo fragments with two 16-byte reads and no conversion.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kDepth = 4;   // chunks whose S loads are in flight per thread

template <typename T>
__device__ __forceinline__ void store_hprev(void* hp, int64_t chunk_off, int e, const float4& h);

template <>
__device__ __forceinline__ void store_hprev<float>(void* hp, int64_t chunk_off, int e, const float4& h) {
  *reinterpret_cast<float4*>(static_cast<float*>(hp) + chunk_off + e) = h;
}

template <>
__device__ __forceinline__ void store_hprev<bf16>(void* hp, int64_t chunk_off, int e, const float4& h) {
  // element e (a multiple of 4) sits in group e/8 at position e%8 (0 or 4)
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const uint32_t h01 = pack_bf16x2(h.x, h.y), h23 = pack_bf16x2(h.z, h.w);
  u32x2 hi, lo;
  hi[0] = h01;
  hi[1] = h23;
  lo[0] = pack_bf16x2(h.x - bf16lo(h01), h.y - bf16hi(h01));
  lo[1] = pack_bf16x2(h.z - bf16lo(h23), h.w - bf16hi(h23));
  bf16* base = static_cast<bf16*>(hp) + 2 * chunk_off + (e / 8) * 16 + (e % 8);
  *reinterpret_cast<u32x2*>(base) = hi;
  *reinterpret_cast<u32x2*>(base + 8) = lo;
}

template <typename T>
__global__ __launch_bounds__(256) void ssd_state_pass(const float* __restrict__ states,
                                                      const float* __restrict__ gcum,
                                                      const float* init,            // may equal final_state
                                                      void* __restrict__ hprev,
                                                      float* final_state,
                                                      int nc, int Q, int64_t Tp, int PN) {
  const int64_t bh = blockIdx.x;
  const int e = (blockIdx.y * 256 + threadIdx.x) * 4;   // PN is a multiple of 1024

  float4 h = make_float4(0.f, 0.f, 0.f, 0.f);
  if (init) h = *reinterpret_cast<const float4*>(init + bh * PN + e);

  const float* sp = states + bh * (int64_t)nc * PN + e;
  const int64_t hbase = bh * (int64_t)nc * PN;
  const float* glast = gcum + bh * Tp + (Q - 1);

  float4 buf[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth; ++i)
    if (i < nc) buf[i] = *reinterpret_cast<const float4*>(sp + (int64_t)i * PN);

  for (int k0 = 0; k0 < nc; k0 += kDepth) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      const int k = k0 + i;
      if (k < nc) {
        const float4 s = buf[i];
        if (k + kDepth < nc) buf[i] = *reinterpret_cast<const float4*>(sp + (int64_t)(k + kDepth) * PN);
        store_hprev<T>(hprev, hbase + (int64_t)k * PN, e, h);
        const float sc = exp2_hw(glast[(int64_t)k * Q]);
        h.x = fmaf(sc, h.x, s.x);
        h.y = fmaf(sc, h.y, s.y);
        h.z = fmaf(sc, h.z, s.z);
        h.w = fmaf(sc, h.w, s.w);
      }
    }
  }
  if (final_state) *reinterpret_cast<float4*>(final_state + bh * PN + e) = h;
}

}  // namespace

hipError_t launch_state_pass(const Problem& p, hipStream_t stream) {
  const int PN = (int)(p.P * p.N);
  const dim3 grid((unsigned)(p.bt * p.H), (unsigned)(PN / 1024));
  const dim3 block(256);
  if (p.io == 1)
    hipLaunchKernelGGL(ssd_state_pass<bf16>, grid, block, 0, stream, p.states, p.gcum, p.init, p.hprev,
                       p.final_state, (int)p.nc, (int)p.Q, p.Tp, PN);
  else
    hipLaunchKernelGGL(ssd_state_pass<float>, grid, block, 0, stream, p.states, p.gcum, p.init, p.hprev,
                       p.final_state, (int)p.nc, (int)p.Q, p.Tp, PN);
  return hipGetLastError();
}

}  // namespace ssd

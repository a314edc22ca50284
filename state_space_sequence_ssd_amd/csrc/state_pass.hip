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
// independent chain, so the grid is (batch*head, state/(256*EPT)) and each
// thread carries EPT consecutive state elements through all chunks in fp32
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

// Each thread carries EPT consecutive state elements (EPT = 4 or 8, so one or
// two 16-byte pieces per chunk) and keeps the S loads of the next DEPTH
// chunks in flight. The host picks EPT = 8 (half the waves, each walking the
// chunks with twice the bytes per load) for large problems, EPT = 4 for more
// parallelism on small ones.
template <typename T, int EPT>
__device__ __forceinline__ void store_hprev(void* hp, int64_t chunk_off, int e, const float* h);

template <>
__device__ __forceinline__ void store_hprev<float, 4>(void* hp, int64_t chunk_off, int e, const float* h) {
  *reinterpret_cast<float4*>(static_cast<float*>(hp) + chunk_off + e) = make_float4(h[0], h[1], h[2], h[3]);
}

template <>
__device__ __forceinline__ void store_hprev<float, 8>(void* hp, int64_t chunk_off, int e, const float* h) {
  float4* d = reinterpret_cast<float4*>(static_cast<float*>(hp) + chunk_off + e);
  d[0] = make_float4(h[0], h[1], h[2], h[3]);
  d[1] = make_float4(h[4], h[5], h[6], h[7]);
}

// bf16 pairs: element e sits in the aligned group of 8 columns e/8, at
// position e%8; the group holds 8 hi values then 8 lo values.
template <>
__device__ __forceinline__ void store_hprev<bf16, 4>(void* hp, int64_t chunk_off, int e, const float* h) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 hi, lo;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t d = pack_bf16x2(h[2 * i], h[2 * i + 1]);
    hi[i] = d;
    lo[i] = pack_bf16x2(h[2 * i] - bf16lo(d), h[2 * i + 1] - bf16hi(d));
  }
  bf16* base = static_cast<bf16*>(hp) + 2 * chunk_off + (e / 8) * 16 + (e % 8);
  *reinterpret_cast<u32x2*>(base) = hi;
  *reinterpret_cast<u32x2*>(base + 8) = lo;
}

template <>
__device__ __forceinline__ void store_hprev<bf16, 8>(void* hp, int64_t chunk_off, int e, const float* h) {
  u32x4 hi, lo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t d = pack_bf16x2(h[2 * i], h[2 * i + 1]);
    hi[i] = d;
    lo[i] = pack_bf16x2(h[2 * i] - bf16lo(d), h[2 * i + 1] - bf16hi(d));
  }
  u32x4* base = reinterpret_cast<u32x4*>(static_cast<bf16*>(hp) + 2 * chunk_off + 2 * e);
  base[0] = hi;
  base[1] = lo;
}

template <int EPT>
struct Piece {
  float v[EPT];
};

template <int EPT>
__device__ __forceinline__ Piece<EPT> load_piece(const float* p) {
  Piece<EPT> r;
#pragma unroll
  for (int i = 0; i < EPT; i += 4) {
    const float4 a = *reinterpret_cast<const float4*>(p + i);
    r.v[i] = a.x; r.v[i + 1] = a.y; r.v[i + 2] = a.z; r.v[i + 3] = a.w;
  }
  return r;
}

// The jump's decays 2^(G'_last,k) of the (batch, head) go to LDS first (nc
// floats, one load each by the workgroup's threads), so the walk itself
// waits only on S. Its steady state is straight-line code with the S loads of
// chunk k + DEPTH issued unconditionally as chunk k is consumed: with a
// guarded prefetch the compiler has to assume any load may still be
// outstanding at the loop head and waits for all of them.
constexpr int kMaxLdsChunks = 8192;   // chunks per (batch, head) whose decays fit the LDS table

template <typename T, int EPT, bool TABLE>
__global__ __launch_bounds__(256) void ssd_state_pass(const float* __restrict__ states,
                                                      const float* __restrict__ gcum,
                                                      const float* init,            // may equal final_state
                                                      void* __restrict__ hprev,
                                                      float* final_state,
                                                      int nc, int Q, int64_t Tp, int PN) {
  constexpr int DEPTH = 32 / EPT;
  extern __shared__ float sdec[];   // nc decays
  const int64_t bh = blockIdx.x;
  const int e = (blockIdx.y * 256 + threadIdx.x) * EPT;   // PN is a multiple of 256 * EPT

  const float* glast = gcum + bh * Tp + (Q - 1);
  if (TABLE)
    for (int k = threadIdx.x; k < nc; k += 256) sdec[k] = exp2_hw(glast[(int64_t)k * Q]);

  Piece<EPT> h;
  if (init) {
    h = load_piece<EPT>(init + bh * PN + e);
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i) h.v[i] = 0.f;
  }

  const float* sp = states + bh * (int64_t)nc * PN + e;
  const int64_t hbase = bh * (int64_t)nc * PN;

  Piece<EPT> buf[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i)
    if (i < nc) buf[i] = load_piece<EPT>(sp + (int64_t)i * PN);
  __syncthreads();   // the decay table

  auto jump = [&](int k, const Piece<EPT>& s) {
    store_hprev<T, EPT>(hprev, hbase + (int64_t)k * PN, e, h.v);
    const float sc = TABLE ? sdec[k] : exp2_hw(glast[(int64_t)k * Q]);
#pragma unroll
    for (int j = 0; j < EPT; ++j) h.v[j] = fmaf(sc, h.v[j], s.v[j]);
  };
  int k0 = 0;
  for (; k0 + 2 * DEPTH <= nc; k0 += DEPTH) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      const Piece<EPT> s = buf[i];
      buf[i] = load_piece<EPT>(sp + (int64_t)(k0 + i + DEPTH) * PN);
      jump(k0 + i, s);
    }
  }
  // the last DEPTH .. 2 DEPTH - 1 chunks
  for (; k0 < nc; k0 += DEPTH) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      const int k = k0 + i;
      if (k < nc) {
        const Piece<EPT> s = buf[i];
        if (k + DEPTH < nc) buf[i] = load_piece<EPT>(sp + (int64_t)(k + DEPTH) * PN);
        jump(k, s);
      }
    }
  }
  if (final_state) {
    float* f = final_state + bh * PN + e;
#pragma unroll
    for (int i = 0; i < EPT; i += 4)
      *reinterpret_cast<float4*>(f + i) = make_float4(h.v[i], h.v[i + 1], h.v[i + 2], h.v[i + 3]);
  }
}

template <typename T, int EPT>
hipError_t launch(const Problem& p, hipStream_t stream) {
  const int PN = (int)(p.P * p.N);
  const dim3 grid((unsigned)(p.bt * p.H), (unsigned)(PN / (256 * EPT)));
  if (p.nc <= kMaxLdsChunks)
    hipLaunchKernelGGL((ssd_state_pass<T, EPT, true>), grid, dim3(256), (size_t)p.nc * 4, stream, p.states, p.gcum,
                       p.init, p.hprev, p.final_state, (int)p.nc, (int)p.Q, p.Tp, PN);
  else
    hipLaunchKernelGGL((ssd_state_pass<T, EPT, false>), grid, dim3(256), 0, stream, p.states, p.gcum, p.init,
                       p.hprev, p.final_state, (int)p.nc, (int)p.Q, p.Tp, PN);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state_pass(const Problem& p, hipStream_t stream) {
  // waves with 8 elements per thread: bt*H*P*N / 512; 256 CUs x 16 waves
  const bool wide = p.bt * p.H * p.P * p.N / 512 >= 256 * 16;
  if (p.io == 1) return wide ? launch<bf16, 8>(p, stream) : launch<bf16, 4>(p, stream);
  return wide ? launch<float, 8>(p, stream) : launch<float, 4>(p, stream);
}

}  // namespace ssd

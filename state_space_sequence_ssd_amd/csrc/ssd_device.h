// Device-side building blocks shared by the four SSD kernels (gfx950 only).
//
// MFMA fragments. Every contraction here uses the 32x32 MFMA shapes:
//   bf16: v_mfma_f32_32x32x16_bf16   (K = 16, 8 bf16 per lane per operand)
//   f32 : v_mfma_f32_32x32x2_f32     (K = 2,  1 fp32 per lane per operand)
// Both share one lane layout (checked on gfx950):
//   A (M x K): lane l holds row l%32, k = KPL*(l/32) + i, i < KPL
//   B (K x N): lane l holds col l%32, k = KPL*(l/32) + i
//   D (M x N): lane l holds col l%32 and 16 rows 8*(r/4) + 4*(l/32) + r%4
// so one kernel body serves both io types through Io<T>.
//
// "Column groups". Operand tiles whose contraction index is the slow
// (token) dimension in memory are loaded one dword per lane per token row:
// lane m (= l%32) loads the dword holding columns E*m .. E*m+E-1 of a
// 32*E-wide column group (E = 4 / sizeof(T)). Element e of that dword feeds
// the MFMA block of parity e, whose column c stands for column E*c + e. A
// wave-wide load thus reads whole 128-byte rows, and no transpose through
// LDS is needed: the token index lands in the MFMA K slot directly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;   // 1 / ln 2

// 2^x on the hardware exponential unit (v_exp_f32 is base 2 natively).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16hi(uint32_t d) { return __uint_as_float(d & 0xffff0000u); }

// Round two floats to bf16 (nearest even, v_cvt_pk_bf16_f32); a -> low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct Io;

template <> struct Io<bf16> {
  static constexpr int E = 2;     // elements per dword
  static constexpr int KPL = 8;   // contraction elements per lane per MFMA
  using Frag = bf16x8;
  __device__ static __forceinline__ void mma(f32x16& c, const Frag& a, const Frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float elem(uint32_t d, int e) { return e ? bf16hi(d) : bf16lo(d); }
  // Fragment from KPL floats, rounded to bf16.
  __device__ static __forceinline__ Frag from_f32(const float* v) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    return __builtin_bit_cast(Frag, u);
  }
  // Split KPL floats into a bf16 pair: hi = bf16(v), lo = bf16(v - hi). v - hi
  // is exact in fp32, and hi + lo carries 16 significant bits, so a product
  // with an exact bf16 operand issued as two MFMAs (hi, then lo) keeps the
  // operand to about 2^-17 relative instead of 2^-9.
  static constexpr bool SPLIT = true;
  __device__ static __forceinline__ void split(const float* v, Frag& hi, Frag& lo) {
    u32x4 uh, ul;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t h = pack_bf16x2(v[2 * i], v[2 * i + 1]);
      uh[i] = h;
      ul[i] = pack_bf16x2(v[2 * i] - bf16lo(h), v[2 * i + 1] - bf16hi(h));
    }
    hi = __builtin_bit_cast(Frag, uh);
    lo = __builtin_bit_cast(Frag, ul);
  }
  // KPL contiguous floats (32 bytes) at p, split as above.
  __device__ static __forceinline__ void load_split(const float* p, Frag& hi, Frag& lo) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    split(v, hi, lo);
  }
  // Fragment of parity e taken from KPL dwords without rounding.
  __device__ static __forceinline__ Frag from_dwords(const uint32_t* d, int e) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a = d[2 * i], b = d[2 * i + 1];
      u[i] = e ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    return __builtin_bit_cast(Frag, u);
  }
  // KPL contiguous elements (16 bytes) at p; zeros when !valid.
  __device__ static __forceinline__ Frag load_row(const bf16* p, bool valid) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (valid) u = *reinterpret_cast<const u32x4*>(p);
    return __builtin_bit_cast(Frag, u);
  }
  __device__ static __forceinline__ void store_pair(bf16* p, float a, float b) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
  }
  // the dword store_pair writes
  __device__ static __forceinline__ uint32_t pack_pair(float a, float b) { return pack_bf16x2(a, b); }
  __device__ static __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 v;
    v[0] = pack_bf16x2(a, b);
    v[1] = pack_bf16x2(c, d);
    *reinterpret_cast<u32x2*>(p) = v;
  }
};

template <> struct Io<float> {
  static constexpr int E = 1;
  static constexpr int KPL = 1;
  using Frag = float;
  __device__ static __forceinline__ void mma(f32x16& c, const Frag& a, const Frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float elem(uint32_t d, int) { return __uint_as_float(d); }
  __device__ static __forceinline__ Frag from_f32(const float* v) { return v[0]; }
  // fp32 operands go to the fp32 MFMA whole: no split, lo is never used.
  static constexpr bool SPLIT = false;
  __device__ static __forceinline__ void split(const float* v, Frag& hi, Frag& lo) { hi = v[0]; lo = 0.f; }
  __device__ static __forceinline__ void load_split(const float* p, Frag& hi, Frag& lo) { hi = *p; lo = 0.f; }
  __device__ static __forceinline__ Frag from_dwords(const uint32_t* d, int) { return __uint_as_float(d[0]); }
  __device__ static __forceinline__ Frag load_row(const float* p, bool valid) { return valid ? *p : 0.f; }
  __device__ static __forceinline__ void store_pair(float* p, float a, float) { *p = a; }
  __device__ static __forceinline__ uint32_t pack_pair(float a, float) { return __float_as_uint(a); }
  __device__ static __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
};

// Raw buffer resource over `bytes` bytes at `base` (gfx9 word 3). Loads
// through it return 0 for any byte offset >= bytes instead of touching
// memory, and their scalar offset operand carries wave-uniform address
// terms with no vector arithmetic. Range checks here always put the whole
// offset in the vector operand (scalar offset 0) where they matter.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buf_load_dword(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
// Store through a buffer resource; with the whole offset in the vector
// operand, bytes at or past the resource's size are dropped.
__device__ __forceinline__ void buf_store_dword(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, 0, 0);
}

// Direct global->LDS load of 16 bytes per lane: lane i's 16 bytes at gptr
// land at LDS address lds + 16 i (lds wave-uniform; it goes in M0). Written
// as inline assembly so the compiler does not treat the asynchronous LDS
// write as aliasing every later LDS read and wait for the whole vector
// memory queue before each of them: the kernels order these loads
// themselves, with explicit vmcnt waits and barriers. The compiler still
// counts them nowhere, which keeps its own waits conservative (they can
// only see more operations outstanding than they assume).
__device__ __forceinline__ void lds_dma16(const void* gptr, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(gptr) : "memory", "m0");
}

// Row of the 32x32 D block held in register r of a lane in half g = l/32.
__device__ __forceinline__ constexpr int drow(int r, int g) { return 8 * (r / 4) + 4 * g + (r % 4); }

}  // namespace ssd

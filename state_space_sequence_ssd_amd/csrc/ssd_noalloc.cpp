// mamba2_ssd_fwd_noalloc: the forward pass with its workspace in a
// file-scope device array instead of caller memory, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation). Declared in include/mamba2_ssd.h.
//
// The array `scratch` exists once per GPU the library's code object is loaded
// on, at its own address there. Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): the device
// address is looked up once per device, with that device current, through
// hipGetSymbolAddress, and kept in g_ptr; every later use goes through it.
#include "mamba2_ssd.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // MAMBA2_SSD_NOALLOC_MAX_WORKSPACE
static_assert(kScratchBytes == MAMBA2_SSD_NOALLOC_MAX_WORKSPACE, "header and library agree");
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on `dev`, looked up on first use with that
// device current (the caller's current device is restored afterwards).
hipError_t scratch_on(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int mamba2_ssd_fwd_noalloc(const mamba2_ssd_dims* dims, int io_dtype, const void* x, const float* dt,
                                      const float* A, const void* B, const void* C, const float* D,
                                      const float* init_state, void* y, float* final_state, void* stream) {
  // sizes first: a call whose workspace exceeds the array is rejected
  // before anything touches the GPU
  mamba2_ssd_workspace_layout L;
  const int st = mamba2_ssd_workspace_layout_query(dims, io_dtype, &L);
  if (st != MAMBA2_SSD_OK) return st;
  if (L.total_bytes > kScratchBytes) return MAMBA2_SSD_ERR_WORKSPACE;
  if (dims->batch == 0 || L.total_bytes == 0)
    return mamba2_ssd_fwd(dims, io_dtype, x, dt, A, B, C, D, init_state, y, final_state, nullptr, 0, stream);
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return MAMBA2_SSD_ERR_HIP;
  }
  void* ws = nullptr;
  if (scratch_on(dev, &ws) != hipSuccess) {
    (void)hipGetLastError();
    return MAMBA2_SSD_ERR_HIP;
  }
  return mamba2_ssd_fwd(dims, io_dtype, x, dt, A, B, C, D, init_state, y, final_state, ws, kScratchBytes, stream);
}

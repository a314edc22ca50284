// C ABI of the selective scan (include/mamba1_s6.h): host-side validation,
// workspace carve-up and launch.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>

#include "mamba1_s6.h"
#include "mamba2_ssd.h"

#include "s6_launch.h"

namespace {

constexpr int64_t kMaxDimS6 = (int64_t)1 << 40;

struct S6Sizes {
  int64_t nc = 0, n_x = 0, n_bc = 0, n_state = 0;
  size_t off_sumd = 0, off_incl = 0, off_sync = 0, total = 0;
};

size_t align_up(size_t v) { return (v + 255) / 256 * 256; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

int s6_sizes(const mamba1_s6_dims* d, S6Sizes* s) {
  if (!d) return MAMBA2_SSD_ERR_NULL_POINTER;
  if (d->batch < 0 || d->seqlen < 0 || d->channels <= 0 || d->dstate <= 0) return MAMBA2_SSD_ERR_BAD_DIM;
  if (d->batch > kMaxDimS6 || d->seqlen > kMaxDimS6 || d->channels > kMaxDimS6) return MAMBA2_SSD_ERR_BAD_DIM;
  if (!ssd::s6_has(d->dstate)) return MAMBA2_SSD_ERR_UNSUPPORTED;
  S6Sizes r;
  const int64_t q = ssd::s6_chunk_tokens();
  r.nc = (d->seqlen + q - 1) / q;
  if (d->batch > 65535 || r.nc > 65535 || d->channels > INT32_MAX - 256) return MAMBA2_SSD_ERR_BAD_DIM;
  int64_t bd, t;
  if (!mul_ok(d->batch, d->channels, &bd) || !mul_ok(bd, d->seqlen, &r.n_x)) return MAMBA2_SSD_ERR_BAD_DIM;
  if (!mul_ok(d->batch, d->dstate, &t) || !mul_ok(t, d->seqlen, &r.n_bc)) return MAMBA2_SSD_ERR_BAD_DIM;
  if (!mul_ok(bd, d->dstate, &r.n_state)) return MAMBA2_SSD_ERR_BAD_DIM;
  int64_t ns, nsum;
  if (!mul_ok(r.n_state, r.nc, &ns) || !mul_ok(bd, r.nc, &nsum) || !mul_ok(ns, 8, &t)) return MAMBA2_SSD_ERR_BAD_DIM;
  const int64_t nsync = ssd::s6_sync_words(d->batch, d->channels, d->seqlen, d->dstate);
  r.off_sumd = align_up((size_t)ns * 4);
  r.off_incl = r.off_sumd + align_up((size_t)nsum * 4);
  r.off_sync = r.off_incl + align_up((size_t)ns * 4);
  r.total = r.off_sync + align_up((size_t)nsync * 4);
  *s = r;
  return MAMBA2_SSD_OK;
}

// The backward workspace: the forward's (its scan leaves the chunks' end
// states in incl), then O, SD, R, the dA parts and the dB, dC parts.
struct S6BwdSizes {
  S6Sizes f;
  int64_t ncb = 0;
  size_t off_O = 0, off_SD = 0, off_R = 0, off_dA = 0, off_dB = 0, off_dC = 0, total = 0;
};

int s6_bwd_sizes(const mamba1_s6_dims* d, S6BwdSizes* s) {
  S6BwdSizes r;
  const int st = s6_sizes(d, &r.f);
  if (st != MAMBA2_SSD_OK) return st;
  if (!ssd::s6_bwd_has(d->dstate)) return MAMBA2_SSD_ERR_UNSUPPORTED;
  const int64_t cbk = ssd::s6_bwd_channel_block();
  r.ncb = (d->channels + cbk - 1) / cbk;
  int64_t ns, bd, nsum, bcb, t, nbc;
  if (!mul_ok(r.f.n_state, r.f.nc, &ns) || !mul_ok(d->batch, d->channels, &bd) || !mul_ok(bd, r.f.nc, &nsum))
    return MAMBA2_SSD_ERR_BAD_DIM;
  // (grid x of the chunk kernels: batch rows times channel blocks)
  if (!mul_ok(d->batch, r.ncb, &bcb) || bcb > INT32_MAX || !mul_ok(bcb, d->dstate, &t) || !mul_ok(t, d->seqlen, &nbc))
    return MAMBA2_SSD_ERR_BAD_DIM;
  r.off_O = r.f.total;
  r.off_SD = r.off_O + align_up((size_t)ns * 4);
  r.off_R = r.off_SD + align_up((size_t)nsum * 4);
  r.off_dA = r.off_R + align_up((size_t)ns * 4);
  r.off_dB = r.off_dA + align_up((size_t)ns * 4);
  r.off_dC = r.off_dB + align_up((size_t)nbc * 4);
  r.total = r.off_dC + align_up((size_t)nbc * 4);
  *s = r;
  return MAMBA2_SSD_OK;
}

struct Range {
  uintptr_t lo, hi;
};
Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, p ? a + bytes : a};
}
bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

// float arrays at their natural 4 bytes; the workspace at 256 bytes (its
// records are moved in 16-byte pieces and its ticket counter is a 64-bit
// atomic)
bool floats_aligned(std::initializer_list<const float*> ps) {
  for (const float* q : ps)
    if (reinterpret_cast<uintptr_t>(q) % 4) return false;
  return true;
}
bool workspace_aligned(const void* w) { return reinterpret_cast<uintptr_t>(w) % 256 == 0; }

}  // namespace

extern "C" {

int mamba1_s6_supported(int64_t dstate) { return ssd::s6_has(dstate) ? 1 : 0; }

size_t mamba1_s6_workspace_bytes(const mamba1_s6_dims* dims) {
  S6Sizes s;
  return s6_sizes(dims, &s) == MAMBA2_SSD_OK ? s.total : 0;
}

int mamba1_s6_check_args(const mamba1_s6_dims* d, const float* x, const float* delta, const float* A,
                         const float* B, const float* C, const float* h0, const float* y, const float* hT,
                         const void* workspace, size_t workspace_bytes) {
  S6Sizes s;
  const int st = s6_sizes(d, &s);
  if (st != MAMBA2_SSD_OK) return st;
  if (!A) return MAMBA2_SSD_ERR_NULL_POINTER;
  if (s.n_x > 0 && (!x || !delta || !B || !C || !y)) return MAMBA2_SSD_ERR_NULL_POINTER;
  const bool work = d->batch > 0;
  if (work && s.total > 0 && (!workspace || workspace_bytes < s.total)) return MAMBA2_SSD_ERR_WORKSPACE;
  if (!floats_aligned({x, delta, A, B, C, h0, y, hT}) || (work && !workspace_aligned(workspace)))
    return MAMBA2_SSD_ERR_ALIGN;
  const Range rx = range_of(x, (size_t)s.n_x * 4), rd = range_of(delta, (size_t)s.n_x * 4);
  const Range rA = range_of(A, (size_t)(d->channels * d->dstate) * 4);
  const Range rB = range_of(B, (size_t)s.n_bc * 4), rC = range_of(C, (size_t)s.n_bc * 4);
  const Range rh0 = range_of(h0, (size_t)s.n_state * 4), ry = range_of(y, (size_t)s.n_x * 4);
  const Range rhT = range_of(hT, (size_t)s.n_state * 4), rws = range_of(workspace, work ? s.total : 0);
  for (const Range& r : {rx, rd, rA, rB, rC}) {
    if (overlap(ry, r) || overlap(rhT, r) || overlap(rws, r)) return MAMBA2_SSD_ERR_ALIAS;
  }
  if (overlap(ry, rh0) || overlap(rws, rh0) || overlap(ry, rhT) || overlap(ry, rws) || overlap(rhT, rws))
    return MAMBA2_SSD_ERR_ALIAS;
  // hT may be exactly h0 (an in-place state update), never a partial overlap
  if (overlap(rhT, rh0) && !(rhT.lo == rh0.lo && rhT.hi == rh0.hi)) return MAMBA2_SSD_ERR_ALIAS;
  return MAMBA2_SSD_OK;
}

int mamba1_s6_fwd(const mamba1_s6_dims* d, const float* x, const float* delta, const float* A, const float* B,
                  const float* C, const float* h0, float* y, float* hT, void* workspace, size_t workspace_bytes,
                  void* stream) {
  const int st = mamba1_s6_check_args(d, x, delta, A, B, C, h0, y, hT, workspace, workspace_bytes);
  if (st != MAMBA2_SSD_OK) return st;
  if (d->batch == 0) return MAMBA2_SSD_OK;
  S6Sizes s;
  s6_sizes(d, &s);
  char* ws = static_cast<char*>(workspace);
  ssd::S6Problem p{};
  p.bt = d->batch; p.L = d->seqlen; p.D = d->channels; p.N = d->dstate;
  p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.h0 = h0; p.y = y; p.hT = hT;
  p.aggS = ws ? reinterpret_cast<float*>(ws) : nullptr;
  p.aggD = ws ? reinterpret_cast<float*>(ws + s.off_sumd) : nullptr;
  p.incl = ws ? reinterpret_cast<float*>(ws + s.off_incl) : nullptr;
  p.sync = ws ? reinterpret_cast<int*>(ws + s.off_sync) : nullptr;
  const hipError_t err = ssd::launch_s6(p, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? MAMBA2_SSD_OK : MAMBA2_SSD_ERR_HIP;
}

size_t mamba1_s6_bwd_workspace_bytes(const mamba1_s6_dims* dims) {
  S6BwdSizes s;
  return s6_bwd_sizes(dims, &s) == MAMBA2_SSD_OK ? s.total : 0;
}

int mamba1_s6_bwd_check_args(const mamba1_s6_dims* d, const float* x, const float* delta, const float* A,
                             const float* B, const float* C, const float* h0, const float* dy, const float* dhT,
                             const float* dx, const float* ddelta, const float* dA, const float* dB, const float* dC,
                             const float* dh0, const void* workspace, size_t workspace_bytes) {
  S6BwdSizes s;
  const int st = s6_bwd_sizes(d, &s);
  if (st != MAMBA2_SSD_OK) return st;
  if (!A || !dA) return MAMBA2_SSD_ERR_NULL_POINTER;
  if (s.f.n_x > 0 && (!x || !delta || !B || !C || !dy || !dx || !ddelta || !dB || !dC))
    return MAMBA2_SSD_ERR_NULL_POINTER;
  const bool work = d->batch > 0;
  if (work && (!workspace || workspace_bytes < s.total)) return MAMBA2_SSD_ERR_WORKSPACE;
  if (!floats_aligned({x, delta, A, B, C, h0, dy, dhT, dx, ddelta, dA, dB, dC, dh0}) ||
      (work && !workspace_aligned(workspace)))
    return MAMBA2_SSD_ERR_ALIGN;
  const size_t nx = (size_t)s.f.n_x * 4, nbc = (size_t)s.f.n_bc * 4, nst = (size_t)s.f.n_state * 4;
  const size_t nA = (size_t)(d->channels * d->dstate) * 4;
  const Range ins[] = {range_of(x, nx), range_of(delta, nx), range_of(A, nA), range_of(B, nbc), range_of(C, nbc),
                       range_of(h0, nst), range_of(dy, nx), range_of(dhT, nst)};
  const Range outs[] = {range_of(dx, nx), range_of(ddelta, nx), range_of(dA, nA), range_of(dB, nbc),
                        range_of(dC, nbc), range_of(dh0, nst), range_of(workspace, work ? s.total : 0)};
  const int no = sizeof(outs) / sizeof(outs[0]);
  for (int i = 0; i < no; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return MAMBA2_SSD_ERR_ALIAS;
    for (int j = i + 1; j < no; ++j)
      if (overlap(outs[i], outs[j])) return MAMBA2_SSD_ERR_ALIAS;
  }
  return MAMBA2_SSD_OK;
}

int mamba1_s6_bwd(const mamba1_s6_dims* d, const float* x, const float* delta, const float* A, const float* B,
                  const float* C, const float* h0, const float* dy, const float* dhT, float* dx, float* ddelta,
                  float* dA, float* dB, float* dC, float* dh0, void* workspace, size_t workspace_bytes,
                  void* stream) {
  const int st = mamba1_s6_bwd_check_args(d, x, delta, A, B, C, h0, dy, dhT, dx, ddelta, dA, dB, dC, dh0, workspace,
                                          workspace_bytes);
  if (st != MAMBA2_SSD_OK) return st;
  S6BwdSizes s;
  s6_bwd_sizes(d, &s);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  auto f = [&](size_t off) { return ws ? reinterpret_cast<float*>(ws + off) : nullptr; };
  hipError_t err = hipSuccess;
  if (d->batch > 0 && s.f.nc > 0) {
    // the forward sweep: the chunks' end states (no y) and, from dy, each
    // chunk's own adjoint record O and delta sum SD
    ssd::S6Problem p{};
    p.bt = d->batch; p.L = d->seqlen; p.D = d->channels; p.N = d->dstate;
    p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.h0 = h0; p.y = nullptr; p.hT = nullptr;
    p.aggS = f(0); p.aggD = f(s.f.off_sumd); p.incl = f(s.f.off_incl);
    p.sync = ws ? reinterpret_cast<int*>(ws + s.f.off_sync) : nullptr;
    p.dy = dy; p.O = f(s.off_O); p.SD = f(s.off_SD);
    err = ssd::launch_s6(p, hs);
  }
  if (err == hipSuccess) {
    ssd::S6BwdProblem q{};
    q.bt = d->batch; q.L = d->seqlen; q.D = d->channels; q.N = d->dstate;
    q.x = x; q.delta = delta; q.A = A; q.B = B; q.C = C; q.h0 = h0; q.dy = dy; q.dhT = dhT;
    q.dx = dx; q.ddelta = ddelta; q.dA = dA; q.dB = dB; q.dC = dC; q.dh0 = dh0;
    q.incl = f(s.f.off_incl); q.O = f(s.off_O); q.SD = f(s.off_SD); q.R = f(s.off_R);
    q.dA_part = f(s.off_dA); q.dB_part = f(s.off_dB); q.dC_part = f(s.off_dC);
    err = ssd::launch_s6_bwd(q, hs);
  }
  return err == hipSuccess ? MAMBA2_SSD_OK : MAMBA2_SSD_ERR_HIP;
}

}  // extern "C"

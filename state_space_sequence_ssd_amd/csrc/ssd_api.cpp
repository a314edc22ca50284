// C ABI of the Mamba-2 chunked SSD forward pass and its one-token decode step
// (declared in include/mamba2_ssd.h). Host code only: argument validation,
// workspace layout, and the launches in dependency order on the caller's
// stream (the kernel order of the CUDA Tile Mamba-2 blog: cumulative sum,
// state pass, then the outputs, with the state contraction split out of the
// pass).
#include "mamba2_ssd.h"

#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <string>

#include "ssd_launch.h"
#include "ssd_bwd.h"

namespace {

thread_local std::string g_last_hip_error;

constexpr size_t kAlign = 256;
constexpr int64_t kMaxDim = int64_t(1) << 40;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

bool valid_io(int io) { return io == MAMBA2_SSD_F32 || io == MAMBA2_SSD_BF16; }
// The io argument of the forward entry points: the dtype in the low byte,
// layout flags above it.
int io_type(int io_arg) { return io_arg & 0xff; }
bool valid_io_arg(int io_arg) {
  return valid_io(io_type(io_arg)) && (io_arg & ~(0xff | MAMBA2_SSD_DT_HEAD_MAJOR | MAMBA2_SSD_PATH_MASK)) == 0;
}
int path_field(int io_arg) { return io_arg & MAMBA2_SSD_PATH_MASK; }
size_t io_size(int io_arg) { return io_type(io_arg) == MAMBA2_SSD_BF16 ? 2 : 4; }

struct Sizes {
  int path = 0;                  // MAMBA2_SSD_PATH_FOUR, _THREE or _CHAINED
  int64_t nc = 0, Tp = 0;
  int64_t n_x = 0, n_dt = 0, n_bc = 0, n_state = 0, n_chunkstates = 0;
};

// The kernel sequence a forward call takes (MAMBA2_SSD_PATH_FOUR, _THREE or
// _CHAINED), or 0 when the path field of io_arg asks for one that does not
// support the shape. Automatic choice: the chained kernel wherever it
// supports the shape; otherwise the chunk states inside the state pass when
// the (batch, head, dstate group) walks alone fill the GPU
// (chunk_state_pass_pays); otherwise the four kernels.
constexpr bool kAutoChained = false;
int choose_path(const ssd::Problem& p, int io_arg) {
  switch (path_field(io_arg)) {
    case MAMBA2_SSD_PATH_FOUR: return MAMBA2_SSD_PATH_FOUR;
    case MAMBA2_SSD_PATH_THREE: return ssd::chunk_state_pass_fits(p) ? MAMBA2_SSD_PATH_THREE : 0;
    case MAMBA2_SSD_PATH_CHAINED: return ssd::chunk_chained_fits(p) ? MAMBA2_SSD_PATH_CHAINED : 0;
    default: break;
  }
  if (kAutoChained && ssd::chunk_chained_fits(p)) return MAMBA2_SSD_PATH_CHAINED;
  if (ssd::chunk_state_pass_fits(p) && ssd::chunk_state_pass_pays(p)) return MAMBA2_SSD_PATH_THREE;
  return MAMBA2_SSD_PATH_FOUR;
}

// Dimension checks shared by every entry point.
int check_dims(const mamba2_ssd_dims* d, int io_arg, Sizes* s) {
  if (!d) return MAMBA2_SSD_ERR_NULL_POINTER;
  if (!valid_io_arg(io_arg)) return MAMBA2_SSD_ERR_UNSUPPORTED;
  const int io = io_type(io_arg);
  if (d->batch < 0 || d->seqlen < 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 ||
      d->ngroups <= 0 || d->chunk <= 0)
    return MAMBA2_SSD_ERR_BAD_DIM;
  if (d->batch > kMaxDim || d->seqlen > kMaxDim || d->nheads > kMaxDim || d->ngroups > kMaxDim)
    return MAMBA2_SSD_ERR_BAD_DIM;
  if (d->nheads % d->ngroups) return MAMBA2_SSD_ERR_GROUPS;
  if (d->chunk != 64 && d->chunk != 128 && d->chunk != 256) return MAMBA2_SSD_ERR_CHUNK;
  if (!ssd::chunk_state_has(io, d->headdim, d->dstate, d->chunk) ||
      !ssd::chunk_scan_has(io, d->headdim, d->dstate, d->chunk))
    return MAMBA2_SSD_ERR_UNSUPPORTED;
  Sizes r;
  r.nc = (d->seqlen + d->chunk - 1) / d->chunk;
  r.Tp = r.nc * d->chunk;
  int64_t bt, bth, pn;
  if (!mul_ok(d->batch, d->seqlen, &bt)) return MAMBA2_SSD_ERR_BAD_DIM;
  if (!mul_ok(bt, d->nheads, &bth)) return MAMBA2_SSD_ERR_BAD_DIM;
  if (!mul_ok(bth, d->headdim, &r.n_x)) return MAMBA2_SSD_ERR_BAD_DIM;
  r.n_dt = bth;
  int64_t btg;
  if (!mul_ok(bt, d->ngroups, &btg) || !mul_ok(btg, d->dstate, &r.n_bc)) return MAMBA2_SSD_ERR_BAD_DIM;
  pn = d->headdim * d->dstate;
  int64_t bh;
  if (!mul_ok(d->batch, d->nheads, &bh) || !mul_ok(bh, pn, &r.n_state)) return MAMBA2_SSD_ERR_BAD_DIM;
  if (!mul_ok(r.n_state, r.nc, &r.n_chunkstates)) return MAMBA2_SSD_ERR_BAD_DIM;
  int64_t bytes;
  if (!mul_ok(r.n_chunkstates, 8, &bytes) || !mul_ok(r.n_x, 8, &bytes)) return MAMBA2_SSD_ERR_BAD_DIM;
  // grid limits of the launchers: y = nchunks (chunk-parallel kernels), z = batch
  if (r.nc > ssd::kMaxGridYZ || d->batch > ssd::kMaxGridYZ) return MAMBA2_SSD_ERR_BAD_DIM;
  if (bh > INT32_MAX) return MAMBA2_SSD_ERR_BAD_DIM;
  // the kernels address one chunk of x (or of B, C) with 32-bit byte offsets
  const int64_t esz = io == MAMBA2_SSD_BF16 ? 2 : 4;
  if (d->chunk * d->nheads * d->headdim * esz >= (int64_t)1 << 31 ||
      d->chunk * d->ngroups * d->dstate * esz >= (int64_t)1 << 31)
    return MAMBA2_SSD_ERR_BAD_DIM;
  ssd::Problem p{};
  p.bt = d->batch; p.T = d->seqlen; p.H = d->nheads; p.P = d->headdim; p.N = d->dstate;
  p.G = d->ngroups; p.Q = d->chunk; p.nc = r.nc; p.Tp = r.Tp; p.io = io;
  r.path = choose_path(p, io_arg);
  if (!r.path) return MAMBA2_SSD_ERR_UNSUPPORTED;
  *s = r;
  return MAMBA2_SSD_OK;
}

// Regions a path does not use take no bytes (their offset is that of the
// next region).
void layout_of(const mamba2_ssd_dims* d, const Sizes& s, mamba2_ssd_workspace_layout* L) {
  const size_t bh = (size_t)d->batch * (size_t)d->nheads;
  const bool four = s.path == MAMBA2_SSD_PATH_FOUR, chained = s.path == MAMBA2_SSD_PATH_CHAINED;
  size_t off = 0;
  L->gcum_offset = off;
  off = align_up(off + bh * (size_t)s.Tp * 4);
  L->dtt_offset = off;
  off = align_up(off + bh * (size_t)s.Tp * 4);
  L->wst_offset = off;
  if (!chained) off = align_up(off + bh * (size_t)s.Tp * 4);   // the chained kernel forms w itself
  L->states_offset = off;
  if (four) off = align_up(off + (size_t)s.n_chunkstates * 4);
  L->hprev_offset = off;
  if (!chained) off = align_up(off + (size_t)s.n_chunkstates * 4);
  L->chain_offset = off;
  if (chained) off = align_up(off + (size_t)s.n_state * 4);
  L->sync_offset = off;
  if (chained) off = align_up(off + (bh + 64) * 4);
  L->total_bytes = off;
  L->nchunks = s.nc;
  L->path = s.path;
}

ssd::Problem problem_of(const mamba2_ssd_dims* d, int io_arg, const Sizes& s) {
  ssd::Problem p{};
  p.bt = d->batch; p.T = d->seqlen; p.H = d->nheads; p.P = d->headdim; p.N = d->dstate;
  p.G = d->ngroups; p.Q = d->chunk; p.nc = s.nc; p.Tp = s.Tp; p.io = io_type(io_arg);
  p.dt_head_major = (io_arg & MAMBA2_SSD_DT_HEAD_MAJOR) ? 1 : 0;
  return p;
}

struct Range {
  uintptr_t lo, hi;   // [lo, hi); empty when lo == hi
};
Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, p ? a + bytes : a};
}
bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

}  // namespace

extern "C" {

int mamba2_ssd_supported(int64_t headdim, int64_t dstate, int64_t chunk, int io_dtype) {
  const int io = io_type(io_dtype);
  return valid_io_arg(io_dtype) && ssd::chunk_state_has(io, headdim, dstate, chunk) &&
         ssd::chunk_scan_has(io, headdim, dstate, chunk);
}

int mamba2_ssd_workspace_layout_query(const mamba2_ssd_dims* dims, int io_dtype,
                                      mamba2_ssd_workspace_layout* out) {
  Sizes s;
  const int st = check_dims(dims, io_dtype, &s);
  if (st != MAMBA2_SSD_OK) return st;
  if (!out) return MAMBA2_SSD_ERR_NULL_POINTER;
  layout_of(dims, s, out);
  return MAMBA2_SSD_OK;
}

size_t mamba2_ssd_fwd_workspace_bytes(const mamba2_ssd_dims* dims, int io_dtype) {
  mamba2_ssd_workspace_layout L;
  if (mamba2_ssd_workspace_layout_query(dims, io_dtype, &L) != MAMBA2_SSD_OK) return 0;
  return L.total_bytes;
}

int mamba2_ssd_check_args(const mamba2_ssd_dims* d, int io, const void* x, const float* dt,
                          const float* A, const void* B, const void* C, const float* D,
                          const float* init_state, const void* y, const float* final_state,
                          const void* workspace, size_t workspace_bytes) {
  Sizes s;
  int st = check_dims(d, io, &s);
  if (st != MAMBA2_SSD_OK) return st;
  const bool tokens = s.n_x > 0;
  if (!A || !D) return MAMBA2_SSD_ERR_NULL_POINTER;
  if (tokens && (!x || !dt || !B || !C || !y)) return MAMBA2_SSD_ERR_NULL_POINTER;
  // the kernels move x, B, C, y and the states in 16-byte pieces and address
  // the workspace regions at 256-byte offsets
  auto mis = [](const void* q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) & (a - 1)) != 0; };
  if (mis(x, 16) || mis(B, 16) || mis(C, 16) || mis(y, 16) || mis(init_state, 16) || mis(final_state, 16) ||
      mis(dt, 4) || mis(A, 4) || mis(D, 4) || mis(workspace, kAlign))
    return MAMBA2_SSD_ERR_ALIGN;
  mamba2_ssd_workspace_layout L;
  layout_of(d, s, &L);
  if (d->batch > 0 && L.total_bytes > 0 && (!workspace || workspace_bytes < L.total_bytes))
    return MAMBA2_SSD_ERR_WORKSPACE;

  const size_t e = io_size(io);
  const Range rx = range_of(x, (size_t)s.n_x * e), rdt = range_of(dt, (size_t)s.n_dt * 4);
  const Range rA = range_of(A, (size_t)d->nheads * 4), rD = range_of(D, (size_t)d->nheads * 4);
  const Range rB = range_of(B, (size_t)s.n_bc * e), rC = range_of(C, (size_t)s.n_bc * e);
  const Range rinit = range_of(init_state, (size_t)s.n_state * 4);
  const Range ry = range_of(y, (size_t)s.n_x * e), rfin = range_of(final_state, (size_t)s.n_state * 4);
  const Range rws = range_of(workspace, d->batch > 0 ? L.total_bytes : 0);

  const Range others[] = {rx, rdt, rA, rD, rB, rC};
  for (const Range& r : others) {
    if (overlap(ry, r) || overlap(rws, r) || overlap(rfin, r)) return MAMBA2_SSD_ERR_ALIAS;
  }
  if (overlap(ry, rinit) || overlap(rws, rinit)) return MAMBA2_SSD_ERR_ALIAS;
  // final_state may be exactly init_state (an in-place update), never a partial overlap
  if (overlap(rfin, rinit) && !(rfin.lo == rinit.lo && rfin.hi == rinit.hi)) return MAMBA2_SSD_ERR_ALIAS;
  if (overlap(ry, rfin) || overlap(ry, rws) || overlap(rfin, rws)) return MAMBA2_SSD_ERR_ALIAS;
  return MAMBA2_SSD_OK;
}

int mamba2_ssd_fwd(const mamba2_ssd_dims* d, int io, const void* x, const float* dt, const float* A,
                   const void* B, const void* C, const float* D, const float* init_state, void* y,
                   float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
  return mamba2_ssd_fwd_timed(d, io, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                              workspace_bytes, stream, nullptr);
}

int mamba2_ssd_fwd_timed(const mamba2_ssd_dims* d, int io, const void* x, const float* dt,
                         const float* A, const void* B, const void* C, const float* D,
                         const float* init_state, void* y, float* final_state, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* events) {
  g_last_hip_error.clear();
  int st = mamba2_ssd_check_args(d, io, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                                 workspace_bytes);
  if (st != MAMBA2_SSD_OK) return st;
  if (d->batch == 0) return MAMBA2_SSD_OK;

  Sizes s;
  check_dims(d, io, &s);
  mamba2_ssd_workspace_layout L;
  layout_of(d, s, &L);
  char* ws = static_cast<char*>(workspace);

  ssd::Problem p = problem_of(d, io, s);
  p.x = x; p.dt = dt; p.A = A; p.B = B; p.C = C; p.D = D;
  p.init = init_state; p.y = y; p.final_state = final_state;
  p.gcum = reinterpret_cast<float*>(ws + L.gcum_offset);
  p.dtt = reinterpret_cast<float*>(ws + L.dtt_offset);
  p.wst = reinterpret_cast<float*>(ws + L.wst_offset);
  p.states = reinterpret_cast<float*>(ws + L.states_offset);
  p.hprev = ws + L.hprev_offset;
  const bool chained = s.path == MAMBA2_SSD_PATH_CHAINED;
  if (chained) p.wst = nullptr;
  p.chain = chained ? reinterpret_cast<float*>(ws + L.chain_offset) : nullptr;
  p.sync = chained ? reinterpret_cast<int*>(ws + L.sync_offset) : nullptr;
  p.nsync = chained ? (int)(d->batch * d->nheads + 64) : 0;
  hipStream_t hs = static_cast<hipStream_t>(stream);

  hipError_t err = hipSuccess;
  auto mark = [&](int i) {
    if (events && err == hipSuccess) err = hipEventRecord(static_cast<hipEvent_t>(events[i]), hs);
  };
  mark(0);
  if (err == hipSuccess && s.nc > 0) err = ssd::launch_chunk_cumsum(p, hs);
  mark(1);
  switch (s.path) {
    case MAMBA2_SSD_PATH_CHAINED:
      // states, pass and outputs in one kernel: events 1..2 enclose it
      if (err == hipSuccess) err = ssd::launch_chunk_chained(p, hs);
      mark(2);
      mark(3);
      break;
    case MAMBA2_SSD_PATH_THREE:
      // chunk states and the pass in one kernel: events 1..2 enclose it
      if (err == hipSuccess) err = ssd::launch_chunk_state_pass(p, hs);
      mark(2);
      mark(3);
      if (err == hipSuccess && s.nc > 0) err = ssd::launch_chunk_scan(p, hs);
      break;
    default:
      if (err == hipSuccess && s.nc > 0) err = ssd::launch_chunk_state(p, hs);
      mark(2);
      // with seqlen == 0 the pass runs zero chunks: final_state = init_state (or 0)
      if (err == hipSuccess && (s.nc > 0 || final_state)) err = ssd::launch_state_pass(p, hs);
      mark(3);
      if (err == hipSuccess && s.nc > 0) err = ssd::launch_chunk_scan(p, hs);
      break;
  }
  mark(4);
  if (err != hipSuccess) {
    g_last_hip_error = hipGetErrorString(err);
    return MAMBA2_SSD_ERR_HIP;
  }
  return MAMBA2_SSD_OK;
}

int mamba2_ssd_fwd_path(const mamba2_ssd_dims* dims, int io_dtype) {
  Sizes s;
  const int st = check_dims(dims, io_dtype, &s);
  return st != MAMBA2_SSD_OK ? st : s.path;
}

int mamba2_ssd_fused_state_pass(const mamba2_ssd_dims* dims, int io_dtype) {
  Sizes s;
  if (check_dims(dims, io_dtype, &s) != MAMBA2_SSD_OK) return 0;
  return s.path != MAMBA2_SSD_PATH_FOUR ? 1 : 0;
}

int mamba2_ssd_step_supported(int64_t dstate, int io_dtype) {
  return valid_io(io_dtype) && ssd::step_has(io_dtype, dstate);
}

int mamba2_ssd_step_check_args(const mamba2_ssd_step_dims* d, int io, const void* x, const float* dt,
                               const float* A, const void* B, const void* C, const float* D,
                               const float* state, const void* y) {
  if (!d) return MAMBA2_SSD_ERR_NULL_POINTER;
  if (!valid_io(io)) return MAMBA2_SSD_ERR_UNSUPPORTED;
  if (d->batch < 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 || d->ngroups <= 0)
    return MAMBA2_SSD_ERR_BAD_DIM;
  if (d->batch > kMaxDim || d->nheads > kMaxDim || d->headdim > kMaxDim || d->ngroups > kMaxDim)
    return MAMBA2_SSD_ERR_BAD_DIM;
  if (d->nheads % d->ngroups) return MAMBA2_SSD_ERR_GROUPS;
  if (!ssd::step_has(io, d->dstate)) return MAMBA2_SSD_ERR_UNSUPPORTED;
  int64_t bh, rows, bg, nbc, nstate;
  if (!mul_ok(d->batch, d->nheads, &bh) || !mul_ok(bh, d->headdim, &rows) ||
      !mul_ok(d->batch, d->ngroups, &bg) || !mul_ok(bg, d->dstate, &nbc) || !mul_ok(rows, d->dstate, &nstate))
    return MAMBA2_SSD_ERR_BAD_DIM;
  // the kernel indexes rows and B/C elements with 32-bit integers
  if (rows >= INT32_MAX || nbc >= INT32_MAX) return MAMBA2_SSD_ERR_BAD_DIM;
  if (rows == 0) return MAMBA2_SSD_OK;
  if (!x || !dt || !A || !B || !C || !D || !state || !y) return MAMBA2_SSD_ERR_NULL_POINTER;
  const size_t e = io_size(io);
  const uintptr_t bc_align = io == MAMBA2_SSD_BF16 ? 8 : 16;
  if (reinterpret_cast<uintptr_t>(state) % 16 || reinterpret_cast<uintptr_t>(B) % bc_align ||
      reinterpret_cast<uintptr_t>(C) % bc_align || reinterpret_cast<uintptr_t>(x) % e ||
      reinterpret_cast<uintptr_t>(y) % e || reinterpret_cast<uintptr_t>(dt) % 4 ||
      reinterpret_cast<uintptr_t>(A) % 4 || reinterpret_cast<uintptr_t>(D) % 4)
    return MAMBA2_SSD_ERR_ALIGN;
  const Range rx = range_of(x, (size_t)rows * e), rdt = range_of(dt, (size_t)bh * 4);
  const Range rA = range_of(A, (size_t)d->nheads * 4), rD = range_of(D, (size_t)d->nheads * 4);
  const Range rB = range_of(B, (size_t)nbc * e), rC = range_of(C, (size_t)nbc * e);
  const Range rs = range_of(state, (size_t)nstate * 4), ry = range_of(y, (size_t)rows * e);
  const Range inputs[] = {rx, rdt, rA, rD, rB, rC};
  for (const Range& r : inputs)
    if (overlap(rs, r) || overlap(ry, r)) return MAMBA2_SSD_ERR_ALIAS;
  if (overlap(rs, ry)) return MAMBA2_SSD_ERR_ALIAS;
  return MAMBA2_SSD_OK;
}

int mamba2_ssd_step(const mamba2_ssd_step_dims* d, int io, const void* x, const float* dt, const float* A,
                    const void* B, const void* C, const float* D, float* state, void* y, void* stream) {
  g_last_hip_error.clear();
  const int st = mamba2_ssd_step_check_args(d, io, x, dt, A, B, C, D, state, y);
  if (st != MAMBA2_SSD_OK) return st;
  if (d->batch == 0) return MAMBA2_SSD_OK;
  ssd::StepProblem p;
  p.bt = d->batch; p.H = d->nheads; p.P = d->headdim; p.N = d->dstate; p.G = d->ngroups; p.io = io;
  p.x = x; p.dt = dt; p.A = A; p.B = B; p.C = C; p.D = D; p.state = state; p.y = y;
  const hipError_t err = ssd::launch_ssd_step(p, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    g_last_hip_error = hipGetErrorString(err);
    return MAMBA2_SSD_ERR_HIP;
  }
  return MAMBA2_SSD_OK;
}

const char* mamba2_ssd_status_string(int status) {
  switch (status) {
    case MAMBA2_SSD_OK: return "ok";
    case MAMBA2_SSD_ERR_NULL_POINTER: return "a required pointer is NULL";
    case MAMBA2_SSD_ERR_BAD_DIM: return "invalid or too large dimension";
    case MAMBA2_SSD_ERR_GROUPS: return "nheads is not a multiple of ngroups";
    case MAMBA2_SSD_ERR_CHUNK: return "chunk must be 64, 128 or 256";
    case MAMBA2_SSD_ERR_UNSUPPORTED: return "unsupported (headdim, dstate, chunk, io dtype)";
    case MAMBA2_SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case MAMBA2_SSD_ERR_ALIAS: return "an output overlaps another array";
    case MAMBA2_SSD_ERR_HIP: return "HIP launch failure";
    case MAMBA2_SSD_ERR_ALIGN: return "a pointer is not aligned as required";
    default: return "unknown status";
  }
}

const char* mamba2_ssd_last_hip_error(void) { return g_last_hip_error.c_str(); }


// ---- backward pass ---------------------------------------------------------

static int bwd_sizes(const mamba2_ssd_dims* d, int io_dtype, Sizes* s, ssd::BwdLayout* L) {
  if (io_dtype & ~0xff) return MAMBA2_SSD_ERR_UNSUPPORTED;   // no layout flags here
  const int st = check_dims(d, io_dtype, s);
  if (st != MAMBA2_SSD_OK) return st;
  // the GEMM batches (batch, chunk, head) go in grid dimension y
  int64_t z;
  if (!mul_ok(d->batch, s->nc, &z) || !mul_ok(z, d->nheads, &z) || z > ssd::kMaxGridYZ) return MAMBA2_SSD_ERR_BAD_DIM;
  *L = ssd::bwd_layout(d->batch, d->nheads, d->headdim, d->dstate, d->ngroups, d->chunk, s->nc, io_dtype);
  return MAMBA2_SSD_OK;
}

size_t mamba2_ssd_bwd_workspace_bytes(const mamba2_ssd_dims* dims, int io_dtype) {
  Sizes s;
  ssd::BwdLayout L;
  if (bwd_sizes(dims, io_dtype, &s, &L) != MAMBA2_SSD_OK) return 0;
  return L.total;
}

int mamba2_ssd_bwd_check_args(const mamba2_ssd_dims* d, int io, const void* x, const float* dt, const float* A,
                              const void* B, const void* C, const float* D, const float* init_state, const void* dy,
                              const float* dfinal, const float* dx, const float* ddt, const float* dA,
                              const float* dB, const float* dC, const float* dD, const float* dinit,
                              const void* workspace, size_t workspace_bytes) {
  Sizes s;
  ssd::BwdLayout L;
  const int st = bwd_sizes(d, io, &s, &L);
  if (st != MAMBA2_SSD_OK) return st;
  const bool tokens = s.n_x > 0;
  if (!A || !D || !dA || !dD) return MAMBA2_SSD_ERR_NULL_POINTER;
  if (tokens && (!x || !dt || !B || !C || !dy || !dx || !ddt || !dB || !dC)) return MAMBA2_SSD_ERR_NULL_POINTER;
  if (d->batch > 0 && (!workspace || workspace_bytes < L.total)) return MAMBA2_SSD_ERR_WORKSPACE;
  // its regions start at 256-byte offsets and are read in 16-byte pieces
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return MAMBA2_SSD_ERR_ALIGN;
  const size_t e = io_size(io);
  const Range ins[] = {range_of(x, (size_t)s.n_x * e), range_of(dt, (size_t)s.n_dt * 4),
                       range_of(A, (size_t)d->nheads * 4), range_of(B, (size_t)s.n_bc * e),
                       range_of(C, (size_t)s.n_bc * e), range_of(D, (size_t)d->nheads * 4),
                       range_of(init_state, (size_t)s.n_state * 4), range_of(dy, (size_t)s.n_x * e),
                       range_of(dfinal, (size_t)s.n_state * 4)};
  const Range outs[] = {range_of(dx, (size_t)s.n_x * 4), range_of(ddt, (size_t)s.n_dt * 4),
                        range_of(dA, (size_t)d->nheads * 4), range_of(dB, (size_t)s.n_bc * 4),
                        range_of(dC, (size_t)s.n_bc * 4), range_of(dD, (size_t)d->nheads * 4),
                        range_of(dinit, (size_t)s.n_state * 4),
                        range_of(workspace, d->batch > 0 ? L.total : 0)};
  const int no = sizeof(outs) / sizeof(outs[0]);
  for (int i = 0; i < no; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return MAMBA2_SSD_ERR_ALIAS;
    for (int j = i + 1; j < no; ++j)
      if (overlap(outs[i], outs[j])) return MAMBA2_SSD_ERR_ALIAS;
  }
  return MAMBA2_SSD_OK;
}

int mamba2_ssd_bwd(const mamba2_ssd_dims* d, int io, const void* x, const float* dt, const float* A, const void* B,
                   const void* C, const float* D, const float* init_state, const void* dy, const float* dfinal,
                   float* dx, float* ddt, float* dA, float* dB, float* dC, float* dD, float* dinit, void* workspace,
                   size_t workspace_bytes, void* stream) {
  g_last_hip_error.clear();
  const int st = mamba2_ssd_bwd_check_args(d, io, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA, dB, dC, dD,
                                           dinit, workspace, workspace_bytes);
  if (st != MAMBA2_SSD_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  {
    // (with batch 0 the workspace may be null: no kernel then touches it, and
    // dA, dD receive zeros)
    Sizes s;
    ssd::BwdLayout L;
    bwd_sizes(d, io, &s, &L);
    char* ws = static_cast<char*>(workspace);
    auto f = [&](size_t off) { return ws ? reinterpret_cast<float*>(ws + off) : nullptr; };
    ssd::BwdProblem p{};
    p.bt = d->batch; p.T = d->seqlen; p.H = d->nheads; p.P = d->headdim; p.N = d->dstate; p.G = d->ngroups;
    p.Q = d->chunk; p.nc = s.nc; p.Tp = s.Tp; p.io = io;
    p.x = x; p.dt = dt; p.A = A; p.B = B; p.C = C; p.D = D; p.init = init_state; p.dy = dy; p.dfinal = dfinal;
    p.dx = dx; p.ddt = ddt; p.dA = dA; p.dB = dB; p.dC = dC; p.dD = dD; p.dinit = dinit;
    p.gcum = f(L.gcum); p.dtt = f(L.dtt); p.wst = f(L.wst); p.E = f(L.E); p.Xp = f(L.Xp); p.dYp = f(L.dYp);
    p.Bp = f(L.Bp); p.Cp = f(L.Cp); p.S = f(L.S); p.hprev = f(L.hprev); p.dhn = f(L.dhn); p.CB = f(L.CB);
    p.DX = f(L.DX); p.W1 = f(L.W1); p.U = f(L.U); p.V = f(L.V); p.dXp = f(L.dXp); p.dBh = f(L.dBh);
    p.dCh = f(L.dCh); p.rowZ = f(L.rowZ); p.colZ = f(L.colZ); p.colW = f(L.colW); p.dA_part = f(L.dA_part);
    p.dD_part = f(L.dD_part);
    // the chunk-local cumsum, dt and the state weights, as the forward pass computes them
    ssd::Problem fp = problem_of(d, io, s);
    fp.dt = dt; fp.A = A; fp.gcum = p.gcum; fp.dtt = p.dtt; fp.wst = p.wst;
    if (s.nc > 0 && d->batch > 0) err = ssd::launch_chunk_cumsum(fp, hs);
    if (err == hipSuccess) err = ssd::launch_ssd_bwd(p, hs);
  }
  if (err != hipSuccess) {
    g_last_hip_error = hipGetErrorString(err);
    return MAMBA2_SSD_ERR_HIP;
  }
  return MAMBA2_SSD_OK;
}

}  // extern "C"

// ssd_state_lookback: the chunk states and the pass over them (bf16 io,
// headdim 64, chunk 256, dstate 64 or 128) with every chunk's tile on
// whichever workgroup claims it, the carried state handed from the tile of
// chunk k-1 to the tile of chunk k of the same head through memory. For each
// (batch, chunk k, head), with G' the chunk-local cumsum of A*dt times log2 e
// (from ssd_chunk_cumsum) and h_k the state entering chunk k:
//
//   S_k      = sum_t w_t x_t (x) B_t,   w_t = dt_t 2^(G'_last - G'_t)
//   h_{k+1}  = 2^(G'_last) h_k + S_k
//   hprev[k] = h_k, as bf16 (hi, lo) pairs (the format ssd_chunk_scan reads)
//
// (CUDA Tile Mamba-2 blog, section "Mamba-2 architecture": the jump formula;
// "Kernel 2: fwd_pass_state": the chunk loop, here spread over tiles.)
//
// Why. A walk of a head's chunks inside one workgroup (ssd_chunk_state_pass)
// puts at most (batch x heads x dstate groups) walks on the GPU, each with
// its chunks in series, although the chunk products, most of the work, do not
// depend on one another. Here the products of all chunks run in parallel on
// persistent workgroups, and only the jump of chunk k waits for that of chunk
// k-1 (the hand-off protocol is described in lookback_device.h).
//
// A workgroup has 8 waves in two halves of 4. A ticket is (chunk k, batch b,
// block of HB heads of one group, HB even): the workgroup loads the B tile of
// (b, k, group) once into LDS, and half f takes heads 2 r + f of the block in
// rounds r, so two heads are computed at a time (two waves per SIMD). Per head
// and half:
//   tables   w_t from the head's G' and dt rows (in LDS), alpha = 2^(G'_last)
//   product  S_k^T = B^T (w o X): wave w of the half takes headdim half w & 1
//            and dstate blocks NBW (w >> 1) + i, i < NBW = N / 64; B^T and X^T
//            fragments come from LDS by gfx950's transposing reads; w o X
//            enters as a bf16 (hi, lo) pair, two MFMAs against the exact B
//   jump     each wave on its own quarter of the state, with no barrier:
//            h_k by device-coherent loads straight into the accumulator layout
//            of S_k^T (the initial state or zeros at chunk 0), h_{k+1} =
//            alpha h_k + S_k by fmaf, stored device-coherent to the head's
//            slot (to final_state after the last chunk); once those stores
//            have completed the wave adds 1 to the head's flag (chunk k reads
//            h_k once the flag reaches 4 k). Then hprev[k] is stored as
//            (hi, lo) pairs, off the hand-off's path.
// The next round's x tiles and G', dt rows (and, before a new ticket, its B
// tile) are issued after the jump.
#include "lookback_device.h"
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

using namespace lookback;

template <int N>
struct LbCfg {
  static constexpr int P = 64, Q = 256, WAVES = 8, THREADS = 512;
  static constexpr int NBW = N / 64;            // dstate blocks per wave
  static constexpr int XBYTES = Q * P * 2;      // x tile, 128-byte rows
  static constexpr int GBYTES = 2 * Q * 4;      // G' row, then dt row
  static constexpr int SLOT = XBYTES + GBYTES;  // one half's head
  static constexpr int BRB = N * 2;             // B row, unpadded, pieces swizzled
  static constexpr int BBYTES = Q * BRB;
  static constexpr int IX = XBYTES / 1024, IB = BBYTES / 1024;
  static constexpr int LX = IX / 4;             // x loads per wave of a half
  static constexpr int LB = IB / WAVES;         // B loads per wave
  static_assert(IX % 4 == 0 && IB % WAVES == 0, "whole direct-load instructions");
  static_assert(BBYTES + 2 * SLOT + 2 * Q * 4 + 64 <= 160 * 1024, "LDS");
};

template <int N>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void ssd_state_lookback(const bf16* __restrict__ x, const bf16* __restrict__ Bm, const float* __restrict__ gcum,
                        const float* __restrict__ dtt, const float* init, void* __restrict__ hprev,
                        float* final_state, float* chain, int* sync, int64_t Tlen, int H, int G, int64_t nc,
                        int64_t Tp, int HB, int64_t ntickets) {
  using Cf = LbCfg<N>;
  using I = Io<bf16>;
  using Frag = bf16x8;
  constexpr int P = 64, Q = 256, BRB = Cf::BRB, NBW = Cf::NBW;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

  __shared__ __attribute__((aligned(1024))) unsigned char sB[Cf::BBYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char sX[2][Cf::SLOT];
  __shared__ __attribute__((aligned(16))) float sWs[2][Q];   // dt_t 2^(G'_last - G'_t) <= dt_t
  __shared__ int64_t sTicket;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  __builtin_assume(wave >= 0 && wave < 8);
  const int lane = tid % 64;
  const int hf = wave >> 2, hw = wave & 3;   // half, wave within the half
  const int NHB = H / HB, R = HB / 2;
  const uint32_t xrb = (uint32_t)H * P * 2;       // x row stride in bytes
  const uint32_t bstride = (uint32_t)G * N * 2;   // B row stride in bytes
  unsigned char* const sXh = sX[hf];
  const float* const sG = reinterpret_cast<const float*>(sXh + Cf::XBYTES);
  const float* const sDt = sG + Q;
  float* const sW = sWs[hf];

  // Direct loads. x tile of a half: instruction kk (8 rows) puts lane l at
  // row 8 kk + l / 8, 16-byte piece l % 8 with the 64-byte halves swapped in
  // rows with bit 1 set; wave w of the half issues kk = w + 4 i. B tile:
  // instruction kk puts lane l at row RPI kk + t_l, stored piece c = l % PPR,
  // which holds logical piece c ^ bswz(row); wave issues kk = wave + 8 i, and
  // the swizzle of row RPI (wave + 8 i) + t_l is that of RPI wave + t_l (bswz
  // has period N / 8 rows), so a lane's source offset is one constant. The
  // per-lane offsets are formed where the loads are issued, from a laundered
  // lane id, so they do not stay live across the head.
  constexpr int PPR = BRB / 16, RPI = 1024 / BRB;
  auto issue_x = [&](int b, int k, int h, int nvalid) {
    int ll = lane, w = hw;
    asm volatile("" : "+v"(ll), "+s"(w));
    const uint32_t jl = (uint32_t)ll >> 3;
    const uint32_t xl = jl * xrb + ((((uint32_t)ll & 7) ^ ((jl & 2) << 1)) * 16);
    const bf16* xs = x + (((int64_t)b * Tlen + (int64_t)k * Q) * H + h) * P;
    const __amdgpu_buffer_rsrc_t rx = urs(xs, (uint32_t)(nvalid - 1) * xrb + P * 2);
#pragma unroll
    for (int i = 0; i < Cf::LX; ++i) {
      const int kk = w + 4 * i;
      bdma16<false>(rx, xl, (uint32_t)(kk * 8) * xrb, sXh + kk * 1024);
    }
    // the G' row (wave 0 of the half) and the dt row (wave 1)
    if (w < 2) {
      const float* src = (w == 0 ? gcum : dtt) + ((int64_t)b * H + h) * Tp + (int64_t)k * Q;
      bdma16<false>(urs(src, Q * 4), (uint32_t)ll * 16, 0, sXh + Cf::XBYTES + w * 1024);
    }
  };
  auto issue_B = [&](const bf16* bt, int nvalid) {
    int ll = lane, w = wave;
    asm volatile("" : "+v"(ll), "+s"(w));
    const uint32_t tl = (uint32_t)ll / PPR, cs = (uint32_t)ll % PPR;
    const uint32_t bl = tl * bstride + ((cs ^ bswz<N>((uint32_t)(RPI * w) + tl)) * 16);
    const __amdgpu_buffer_rsrc_t rb = urs(bt, (uint32_t)(nvalid - 1) * bstride + N * 2);
#pragma unroll
    for (int i = 0; i < Cf::LB; ++i) {
      const int kk = w + 8 * i;
      bdma16<false>(rb, bl, (uint32_t)(RPI * kk) * bstride, sB + kk * 1024);
    }
  };

  const int64_t per = ntickets / nc;   // tickets per chunk = batch * NHB
  struct Tk {
    int k, b, h0, nvalid;
    const bf16* bt;
  };
  auto decode = [&](int64_t t) {
    Tk d;
    d.k = (int)(t / per);
    const int u = (int)(t % per);
    d.b = u / NHB;
    d.h0 = (u % NHB) * HB;
    const int64_t t0 = (int64_t)d.k * Q;
    d.nvalid = (int)(Tlen - t0 < Q ? Tlen - t0 : Q);
    d.bt = Bm + (((int64_t)d.b * Tlen + t0) * G + d.h0 / (H / G)) * N;
    return d;
  };

  if (tid == 0) sTicket = claim_ticket(sync);
  lds_barrier();
  int64_t ticket = uniform64(sTicket);
  if (ticket < ntickets) {
    const Tk d = decode(ticket);
    issue_B(d.bt, d.nvalid);
    issue_x(d.b, d.k, d.h0 + hf, d.nvalid);
  }
  vm_lds_barrier();

  while (ticket < ntickets) {
    const Tk cur = decode(ticket);
    const int k = cur.k, b = cur.b;
    int64_t next_ticket = ntickets;
    for (int r = 0; r < R; ++r) {
      const int h = cur.h0 + 2 * r + hf;
      const int64_t bh = (int64_t)b * H + h;
      int lt = lane;
      asm volatile("" : "+v"(lt));
      const int m = lt & 31, g = lt >> 5;

      // ---- tables, once this round's x, G' and dt have landed (and the
      // previous round's hprev stores have completed)
      vm_lds_barrier();
      if (r == 0 && tid == 0) sTicket = claim_ticket(sync);
      sW[tid & 255] = sDt[tid & 255] * exp2_hw(sG[Q - 1] - sG[tid & 255]);
      const float alpha = exp2_hw(sG[Q - 1]);
      lds_barrier();
      if (r == 0) next_ticket = uniform64(sTicket);   // claimed above, visible after the barrier

      // ---- product: S_k^T[n][p] = sum_t B[t][n] (w_t x[t][p]); rows n of
      // dstate blocks NBW (hw >> 1) + i, columns p of headdim block hw & 1
      const int pe_a = hw & 1, nb0 = NBW * (hw >> 1);
      f32x16 sacc[NBW];
#pragma unroll
      for (int i = 0; i < NBW; ++i) sacc[i] = f32x16{};
      {
        // transposing x reads: lane s supplies row 4 (s / 32) + (s % 16) / 4
        // of a 16-row step, headdim columns 16 ((s / 16) % 2) + 4 (s % 4) +
        // 32 pe (the 64-byte half flipped in rows with bit 1 set)
        const uint32_t xtr = (uint32_t)(4 * g + ((lt & 15) >> 2)) * 128 +
                             ((((uint32_t)(32 * ((lt >> 4) & 1) + 8 * (lt & 3))) ^ (uint32_t)(64 * ((lt & 15) >> 3))) ^
                              (pe_a ? 64u : 0u));
        // B^T fragment reads: lane supplies row 16 s + 8 hh + 4 g + (l % 16) / 4,
        // the 8 bytes of dstate columns 32 nb + 16 ((l / 16) % 2) + 4 (l % 4) ..
        // (row 16 s + t_r has the swizzle of row t_r: bswz has period 16 or 8)
        const uint32_t a_ = (uint32_t)((lt & 15) >> 2);
        const uint32_t piece0 = (uint32_t)(2 * ((lt >> 4) & 1) + ((lt & 3) >> 1));
        const uint32_t half = (uint32_t)(lt & 1) * 8;
        uint32_t btoff[2][NBW];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < NBW; ++i) {
            const uint32_t tr = (uint32_t)(8 * hh + 4 * g) + a_;
            btoff[hh][i] = tr * BRB + (((uint32_t)(4 * (nb0 + i)) + piece0) ^ bswz<N>(tr)) * 16 + half;
          }
        auto tr_read = [](const unsigned char* a0, const unsigned char* a1) -> Frag {
          const uint64_t h0 = __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                               (__attribute__((address_space(3))) s16x4*)(a0)));
          const uint64_t h1 = __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                               (__attribute__((address_space(3))) s16x4*)(a1)));
          const u32x4 w4 = {(uint32_t)h0, (uint32_t)(h0 >> 32), (uint32_t)h1, (uint32_t)(h1 >> 32)};
          return __builtin_bit_cast(Frag, w4);
        };
        // software pipeline over the 16 steps: at step s the fragments of step
        // s + 2 are read, the (hi, lo) split of step s + 1 is formed, and the
        // MFMAs of step s run (their split was formed one step earlier)
        Frag xf[3], bfr[3][NBW];
        float4 wq[3][2];
        Frag shi[2], slo[2];
        auto ldA = [&](int s, int sl) {
          const unsigned char* xa = sXh + xtr + 16 * s * 128;
          xf[sl] = tr_read(xa, xa + 8 * 128);
#pragma unroll
          for (int i = 0; i < NBW; ++i)
            bfr[sl][i] = tr_read(sB + btoff[0][i] + 16 * s * BRB, sB + btoff[1][i] + 16 * s * BRB);
          wq[sl][0] = *reinterpret_cast<const float4*>(&sW[16 * s + 4 * g]);
          wq[sl][1] = *reinterpret_cast<const float4*>(&sW[16 * s + 8 + 4 * g]);
        };
        // w o x of one step as a bf16 (hi, lo) pair
        auto splitA = [&](int sl, Frag& hi, Frag& lo) {
          const float wv[8] = {wq[sl][0].x, wq[sl][0].y, wq[sl][0].z, wq[sl][0].w,
                               wq[sl][1].x, wq[sl][1].y, wq[sl][1].z, wq[sl][1].w};
          const u32x4 xd = __builtin_bit_cast(u32x4, xf[sl]);
          u32x4 uh, ul;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v0 = wv[2 * i] * bf16lo(xd[i]), v1 = wv[2 * i + 1] * bf16hi(xd[i]);
            uint32_t hh = pack_bf16x2(v0, v1);
            asm volatile("" : "+v"(hh));
            uh[i] = hh;
            ul[i] = pack_bf16x2(v0 - __uint_as_float(hh << 16), v1 - __uint_as_float(hh & 0xffff0000u));
          }
          hi = __builtin_bit_cast(Frag, uh);
          lo = __builtin_bit_cast(Frag, ul);
        };
        ldA(0, 0);
        ldA(1, 1);
        splitA(0, shi[0], slo[0]);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          if (s + 2 < 16) ldA(s + 2, (s + 2) % 3);
#pragma unroll
          for (int i = 0; i < NBW; ++i) I::mma(sacc[i], bfr[s % 3][i], shi[s & 1]);
#pragma unroll
          for (int i = 0; i < NBW; ++i) I::mma(sacc[i], bfr[s % 3][i], slo[s & 1]);
          if (s + 1 < 16) splitA((s + 1) % 3, shi[(s + 1) & 1], slo[(s + 1) & 1]);
#pragma unroll
          for (int q = 0; q < 2 * NBW; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 40 / (2 * NBW), 0);   // then VALU
          }
        }
      }
      // every wave is done with this round's x (and, in the last round, with B)
      lds_barrier();

      // ---- jump, each wave on its own quarter of the state (rows n =
      // 32 (nb0 + i) + 8 q + 4 g + e, columns p = 32 pe_a + m, the
      // accumulator layout): the head's flag counts the quarters published,
      // so chunk k may read h_k once it reaches 4 k.
      // h_{k+1} = alpha h_k + S_k
      const int p = 32 * pe_a + m;
      float4 hk[NBW][4];
      if (k > 0) {
        wait_flag(sync + kSyncFlags + bh, 4 * k, sync);
        const __amdgpu_buffer_rsrc_t rh = urs(chain + bh * (int64_t)(P * N), (uint32_t)(P * N * 4));
#pragma unroll
        for (int i = 0; i < NBW; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            hk[i][q] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rh, (uint32_t)(p * N + 32 * (nb0 + i) + 8 * q + 4 * g) * 4, 0, 16));
      } else if (init) {
        const __amdgpu_buffer_rsrc_t rh = urs(init + bh * (int64_t)(P * N), (uint32_t)(P * N * 4));
#pragma unroll
        for (int i = 0; i < NBW; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            hk[i][q] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rh, (uint32_t)(p * N + 32 * (nb0 + i) + 8 * q + 4 * g) * 4, 0, 0));
      } else {
#pragma unroll
        for (int i = 0; i < NBW; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) hk[i][q] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      vm_wait0();   // h_k has landed
      // h_{k+1}: to the head's slot (device-coherent), or after the last
      // chunk to final_state (if wanted); once the stores have completed, the
      // quarter is published
      const bool last_chunk = k + 1 == nc;
      float* hdst = last_chunk ? final_state : chain;
      if (hdst) {
        const __amdgpu_buffer_rsrc_t rs = urs(hdst + bh * (int64_t)(P * N), (uint32_t)(P * N * 4));
#pragma unroll
        for (int i = 0; i < NBW; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 a = hk[i][q];
            const u32x4 v = {__float_as_uint(fmaf(alpha, a.x, sacc[i][4 * q])),
                             __float_as_uint(fmaf(alpha, a.y, sacc[i][4 * q + 1])),
                             __float_as_uint(fmaf(alpha, a.z, sacc[i][4 * q + 2])),
                             __float_as_uint(fmaf(alpha, a.w, sacc[i][4 * q + 3]))};
            const uint32_t off = (uint32_t)(p * N + 32 * (nb0 + i) + 8 * q + 4 * g) * 4;
            if (last_chunk) __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 0);
            else __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 16);   // sc1
          }
      }
      vm_wait0();
      if (lane == 0) __hip_atomic_fetch_add(sync + kSyncFlags + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

      // hprev[k] = h_k: row p holds 4 N bytes; dstate group n / 8 takes 32
      // bytes, its 8 hi values then its 8 lo values
      {
        unsigned char* hp = static_cast<unsigned char*>(hprev) + ((bh * nc + k) * (int64_t)(P * N) + p * N) * 4;
#pragma unroll
        for (int i = 0; i < NBW; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 a = hk[i][q];
            const uint32_t h01 = pack_bf16x2(a.x, a.y), h23 = pack_bf16x2(a.z, a.w);
            const uint32_t l01 = pack_bf16x2(a.x - bf16lo(h01), a.y - bf16hi(h01));
            const uint32_t l23 = pack_bf16x2(a.z - bf16lo(h23), a.w - bf16hi(h23));
            unsigned char* grp8 = hp + (4 * (nb0 + i) + q) * 32 + 8 * g;
            __builtin_nontemporal_store(u32x2{h01, h23}, reinterpret_cast<u32x2*>(grp8));
            __builtin_nontemporal_store(u32x2{l01, l23}, reinterpret_cast<u32x2*>(grp8 + 16));
          }
      }

      // ---- the next round's loads (every wave is past this round's product,
      // so x and B may be overwritten): the next heads of this ticket, or the
      // first heads and the B tile of the next ticket
      if (r + 1 < R) {
        issue_x(b, k, cur.h0 + 2 * (r + 1) + hf, cur.nvalid);
      } else if (next_ticket < ntickets) {
        const Tk d = decode(next_ticket);
        issue_B(d.bt, d.nvalid);
        issue_x(d.b, d.k, d.h0 + hf, d.nvalid);
      }
    }
    ticket = next_ticket;
  }
}

template <int N>
int lookback_grid() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    dev = 0;
  }
  if (!cached[dev]) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ssd_state_lookback<N>, LbCfg<N>::THREADS, 0) !=
            hipSuccess ||
        cus <= 0 || per_cu <= 0) {
      (void)hipGetLastError();
      cus = 256;
      per_cu = 1;
    }
    cached[dev] = cus * per_cu;
  }
  return cached[dev];
}

// Heads per ticket: 4 (the B tile serves two rounds) where that still gives
// every workgroup a few tickets, else 2.
int lookback_heads_per_ticket(const Problem& p, int slots) {
  const int64_t hpg = p.H / p.G;
  if (hpg % 4 == 0 && p.bt * p.nc * (p.H / 4) >= 3 * (int64_t)slots) return 4;
  return 2;
}

template <int N>
hipError_t launch_lookback(const Problem& p, hipStream_t stream) {
  const int slots = lookback_grid<N>();
  const int HB = lookback_heads_per_ticket(p, slots);
  const int64_t ntickets = p.bt * p.nc * (p.H / HB);
  const int64_t grid = ntickets < slots ? ntickets : slots;
  hipLaunchKernelGGL((ssd_state_lookback<N>), dim3((unsigned)grid), dim3(LbCfg<N>::THREADS), 0, stream,
                     (const bf16*)p.x, (const bf16*)p.B, p.gcum, p.dtt, p.init, p.hprev, p.final_state, p.chain,
                     p.sync, p.T, (int)p.H, (int)p.G, p.nc, p.Tp, HB, ntickets);
  return hipGetLastError();
}

}  // namespace

bool state_lookback_fits(const Problem& p) {
  return p.io == 1 && p.P == 64 && p.Q == 256 && (p.N == 64 || p.N == 128) && p.nc > 0 && (p.H / p.G) % 2 == 0;
}

hipError_t launch_state_lookback(const Problem& p, hipStream_t stream) {
  if (p.bt == 0 || p.nc == 0) return hipSuccess;
  return p.N == 64 ? launch_lookback<64>(p, stream) : launch_lookback<128>(p, stream);
}

}  // namespace ssd

// gfx950 kernels of libssmscan: the scan's backward (recompute-and-reverse
// gradients) and its fixed-order reductions.
#include "device.h"

namespace ssm {
namespace {

// ---------------------------------------------------------- backward kernel
//
// Reverse-mode gradients of the scan (the chain rule applied to the
// recurrence; the pages give the forward only).  With dt2 = dt log2(e) as in
// the forward kernel, a_t = exp2(dt2_t A), u2_t = dt2_t x_t and B' = B ln 2:
//   dy_t   = dout_t SiLU(z_t)                   dz_t = dout_t y_t SiLU'(z_t)
//   dh_t   = dy_t C_t + a_{t+1} dh_{t+1}        (carry from dlast)
//   dx_t   = dy_t D + dt2_t (dh_t . B'_t)
//   ddt_t  = sum_n dh_t A a_t h_{t-1} + x_t log2(e) (dh_t . B'_t)
//   ddelta = ddt sigmoid(delta + bias) (softplus) or ddt
//   dB_t  += ln 2 dh_t u2_t,   dC_t += dy_t h_t   (over channels)
//   dA    += ln 2 dh_t a_t h_{t-1} dt2_t          (over steps and rows)
// A workgroup owns 64 channels of one batch row (4 wavefronts x 4 states per
// lane, as in the forward).  Phase 1 runs the forward and stores the state
// entering every tile of kBwdTile steps.  Phase 2 walks the tiles backwards:
// it recomputes the tile's forward from its checkpoint (keeping each step's
// incoming state, and with two-channel items each transition, in registers),
// then runs the reverse recurrence on those values.  Sums over a
// channel's 16 states go through LDS partials, summed in a fixed order; dB and
// dC are reduced over the wavefront's 64 channels in registers (lane swaps and
// DPP, lane_sum8), and stored per channel block for a second, fixed-order
// reduction kernel: the result does not depend on timing.
//
// A long sequence with few channel blocks is cut into time chunks, one
// workgroup per (chunk, batch row, block).  Chunk k then starts its forward
// from the state entering it (slot k - 1 of ws_hin, from the forward's pass A
// and carry; the caller's initial state for k = 0) and its reverse walk from
// the gradient arriving at its end (slot k of ws_dl, from the reverse pass A
// and carry below; the caller's dlast for the last chunk).  The chunk length
// is a multiple of the tile, so the chunk's tiles are tiles of the whole
// sequence and share its checkpoint layout.

// Totals over the 64 lanes of a wavefront of eight values per lane, in
// registers: gfx950's lane-swap instructions pair lanes l and l ^ 32 (then
// l ^ 16) while halving the values each lane carries, a rotation by 8 within
// each 16-lane row pairs l and l ^ 8 for the last two, and three DPP steps sum
// each 8-lane group.  Every lane of 8-lane group l >> 3 returns the total of
// value sum8_index(l).
__device__ __forceinline__ float2 swap_lanes32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));  // {a[0..31], b[0..31]}, {a[32..], b[32..]}
}
__device__ __forceinline__ float2 swap_rows16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));  // rows {a0, b0, a2, b2}, {a1, b1, a3, b3}
}
__device__ __forceinline__ int sum8_index(int lane) {
  const int r = (lane >> 4) & 3;
  return ((r & 1) << 1) + (r >> 1) + 4 * ((lane >> 3) & 1);
}
__device__ __forceinline__ float lane_sum8(const float (&v)[8], int lane) {
  float S[4], T[2];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float2 r = swap_lanes32(v[2 * p], v[2 * p + 1]);
    S[p] = r.x + r.y;   // lanes 0..31: value 2p over l, l + 32; lanes 32..63: value 2p + 1
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float2 r = swap_rows16(S[2 * p], S[2 * p + 1]);
    T[p] = r.x + r.y;   // row 0: value 4p, row 1: 4p + 2, row 2: 4p + 1, row 3: 4p + 3 (over 4 lanes)
  }
  const bool hi = (lane >> 3) & 1;
  const float keep = hi ? T[1] : T[0], give = hi ? T[0] : T[1];
  float u = keep + SSM_DPP(0.0f, give, 0x128, 0xf);   // row_ror:8 brings lane l ^ 8
  u += SSM_DPP(0.0f, u, 0xb1, 0xf);                   // quad_perm [1,0,3,2]
  u += SSM_DPP(0.0f, u, 0x4e, 0xf);                   // quad_perm [2,3,0,1]
  u += SSM_DPP(0.0f, u, 0x141, 0xf);                  // row_half_mirror
  return u;
}

template <typename Tin, typename Tg, bool HAS_Z, int CW>
__global__ void __launch_bounds__(256, 3) scan_bwd_kernel(BwdArgs a) {
  constexpr int NS = 4, G = 4, T = kBwdTile, NTHR = 256;
  constexpr int CPR = kWave / CW;
  constexpr int IPT = T * CPR / NTHR;
  static_assert(IPT >= 1 && IPT * NTHR == T * CPR, "tile does not split evenly");
  using R = Raw<Tin, CW>;
  using RG = Raw<Tg, CW>;
  // B and C staging: one value per thread and tile (256 threads = T rows x 16
  // states x {B, C} for 8-step tiles; both per thread for 16-step tiles)
  constexpr bool kSplitBC = T * kDState * 2 <= NTHR;
  static_assert(T * kDState * (kSplitBC ? 2 : 1) == NTHR, "B/C staging does not cover the tile");

  __shared__ float2 sh_dtu[T][kWave + 1];      // (dt2, u2)
  __shared__ float sh_dy[T][kWave + 1];
  __shared__ float sh_B[T][kDState];           // B ln 2
  __shared__ float sh_C[T][kDState];
  __shared__ float sh_y[T][G * kWave + 1];     // forward readout partials
  __shared__ float sh_s1[T][G * kWave + 1];    // partial dh . B'
  __shared__ float sh_s2[T][G * kWave + 1];    // partial sum dh A a h_{t-1}
  __shared__ float sh_bc[T][2][kDState];       // the tile's dB', dC of this block

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int g = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int64_t b = blockIdx.z;
  const int kc = blockIdx.y;   // time chunk
  const int K = a.n_chunks;
  const int blk = blockIdx.x;
  const int64_t Dn = a.d_inner, L = a.seqlen;
  const int64_t d0 = (int64_t)blk * kWave;
  const int nvalid = (int)min((int64_t)kWave, Dn - d0);
  const int loff = min(lane, nvalid - 1);
  const int64_t dl = d0 + loff;
  const bool softplus = a.softplus != 0;
  const int64_t t_begin = (int64_t)kc * a.chunk_len;
  const int64_t Lc = min(a.chunk_len, L - t_begin);   // steps of this chunk
  const int64_t ntiles = (Lc + T - 1) / T;
  const int64_t row = b * K + kc;                      // per-(row, chunk) partial sums

  float Ad[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) Ad[i] = a.A[dl * kDState + g * NS + i];

  int irow[IPT], icol[IPT];
  float ibias[IPT][CW], iD[IPT][CW];
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int idx = tid + it * NTHR;
    irow[it] = idx / CPR;
    icol[it] = min(idx % CPR, (nvalid + CW - 1) / CW - 1) * CW;
#pragma unroll
    for (int q = 0; q < CW; ++q) {
      const int64_t dq = d0 + min(icol[it] + q, nvalid - 1);
      ibias[it][q] = a.bias != nullptr ? a.bias[dq] : 0.0f;
      iD[it][q] = a.D != nullptr ? a.D[dq] : 0.0f;
    }
  }
  const int64_t row0 = (b * L + t_begin) * Dn + d0;
  const Tin* xb = static_cast<const Tin*>(a.x) + row0;
  const Tin* db = static_cast<const Tin*>(a.delta) + row0;
  const Tin* zb = HAS_Z ? static_cast<const Tin*>(a.z) + row0 : nullptr;
  const Tg* gb = static_cast<const Tg*>(a.dout) + row0;
  const Tin* Bb = static_cast<const Tin*>(a.B) + (b * L + t_begin) * kDState;
  const Tin* Cb = static_cast<const Tin*>(a.C) + (b * L + t_begin) * kDState;
  const int64_t ntiles_all = (L + T - 1) / T;
  float* ck = a.ws_ckpt + ((b * a.nblk + blk) * ntiles_all + t_begin / T) * (int64_t)(kWave * kDState);

  // Raw inputs of one tile, loaded one tile ahead of their use (rows past
  // the tile's end repeat its last row, so every load is unconditional).
  struct Bank {
    R rx[IPT], rd[IPT], rz[IPT];
    RG rg[IPT];
    float bv, cv;   // this thread's staged B or C element (cv only when one thread stages both)
  };
  auto tile_rows = [&](int64_t k) SSM_INLINE { return (int)min((int64_t)T, Lc - k * T); };
  auto load = [&](Bank& bk, int64_t k, bool full) SSM_INLINE {
    const int64_t t0 = k * T;
    const int nt = tile_rows(k);
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int64_t off = (t0 + min(irow[it], nt - 1)) * Dn + icol[it];
      bk.rx[it].load(xb + off);
      bk.rd[it].load(db + off);
      if (full) {
        bk.rg[it].load(gb + off);
        if (HAS_Z) bk.rz[it].load(zb + off);
      }
    }
    if constexpr (kSplitBC) {
      // waves 0..1 take B, waves 2..3 take C (uniform per wave)
      const int64_t t = t0 + min((tid / kDState) % T, nt - 1);
      if (tid < T * kDState) bk.bv = ld_in(Bb + t * kDState + tid % kDState);
      else if (full) bk.bv = ld_in(Cb + t * kDState + tid % kDState);
    } else {
      const int64_t t = t0 + min(tid / kDState, nt - 1);
      bk.bv = ld_in(Bb + t * kDState + tid % kDState);
      if (full) bk.cv = ld_in(Cb + t * kDState + tid % kDState);
    }
  };
  auto stage_bc = [&](const Bank& bk, bool with_c) SSM_INLINE {
    const int n = tid % kDState;
    if constexpr (kSplitBC) {
      const int r = (tid / kDState) % T;
      if (tid < T * kDState) sh_B[r][n] = bk.bv * kLn2;
      else if (with_c) sh_C[r][n] = bk.bv;
    } else {
      const int r = tid / kDState;
      sh_B[r][n] = bk.bv * kLn2;
      if (with_c) sh_C[r][n] = bk.cv;
    }
  };

  // The state entering every tile comes from the forward scan kernel's
  // checkpoint pass (ScanArgs::ckpt), run before this kernel: slot 4 j + i of
  // a lane's 16 holds state j + 4 i, so this wave's states 4 g .. 4 g + 3 are
  // slots g, g + 4, g + 8, g + 12.
  auto ld_ckpt = [&](int64_t k) SSM_INLINE {
    const float* p = ck + (k * kWave + lane) * kDState + g;
    return make_float4(p[0], p[4], p[8], p[12]);
  };
  float h[NS];
  const ProgressPriority prio(ntiles);
  Bank cur, nxt;

  // ---- phase 2: the tiles in reverse
  float carry[NS], dAacc[NS];
  const float* gsrc = kc + 1 < K ? a.ws_dl + (row * Dn + dl) * kDState
                      : a.dlast != nullptr ? a.dlast + (b * Dn + dl) * kDState : nullptr;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    carry[i] = gsrc != nullptr ? gsrc[g * NS + i] : 0.0f;
    dAacc[i] = 0.0f;
  }
  float dDacc[IPT][CW], dBacc[IPT][CW];
#pragma unroll
  for (int it = 0; it < IPT; ++it)
#pragma unroll
    for (int q = 0; q < CW; ++q) dDacc[it][q] = dBacc[it][q] = 0.0f;

  load(cur, ntiles - 1, true);
  float4 hc = ld_ckpt(ntiles - 1);
  for (int64_t k = ntiles - 1; k >= 0; --k) {
    if (a.fair) prio.at(ntiles - 1 - k);
    const int64_t t0 = k * T;
    const int nt = tile_rows(k);
    // the tile's per-element values, from the raw inputs (which stay live for
    // the tile; the finish below derives them again instead of keeping them)
    auto elem = [&](int it, int q, float& x, float& dt2, float& dy) SSM_INLINE {
      x = cur.rx[it].get(q);
      const float u2 = (cur.rd[it].get(q) + ibias[it][q]) * kLog2e;
      dt2 = softplus ? softplus2_f(u2) : u2;
      dy = cur.rg[it].get(q);
      if (HAS_Z) dy = dy * silu_f(cur.rz[it].get(q));
    };
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
#pragma unroll
      for (int q = 0; q < CW; ++q) {
        float x, dt2, dy;
        elem(it, q, x, dt2, dy);
        sh_dtu[irow[it]][icol[it] + q] = make_float2(dt2, dt2 * x);
        sh_dy[irow[it]][icol[it] + q] = dy;
      }
    }
    stage_bc(cur, true);
    h[0] = hc.x; h[1] = hc.y; h[2] = hc.z; h[3] = hc.w;
    if (k > 0) {
      load(nxt, k - 1, true);
      hc = ld_ckpt(k - 1);
    }
    block_sync();

    // forward within the tile: each step's incoming state, and readout
    // partials; steps past a ragged tile's end keep the final state, so
    // hp[s + 1] (or h after the last step) is the state after step s
    // With two channels per item the transitions a of the tile also stay in
    // registers for the reverse walk (32 VGPRs, 163 in all: still three
    // workgroups per CU); the one-channel variant recomputes them, which
    // keeps it from spilling.
    constexpr bool kKeepA = CW == 2;
    float hp[T][NS], ap[T][NS];
#pragma unroll
    for (int s = 0; s < T; ++s) {
#pragma unroll
      for (int i = 0; i < NS; ++i) hp[s][i] = h[i];
      if (s < nt) {
        const float2 v = sh_dtu[s][loff];
        float y = 0.0f;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          ap[s][i] = __builtin_amdgcn_exp2f(v.x * Ad[i]);
          h[i] = __builtin_fmaf(ap[s][i], h[i], v.y * sh_B[s][g * NS + i]);
          y = __builtin_fmaf(sh_C[s][g * NS + i], h[i], y);
        }
        sh_y[s][g * kWave + lane] = y;
      }
    }

    // reverse within the tile.  With bf16 inputs each step's LDS operands are
    // read one step ahead, before the later step's guard (rows past a ragged
    // tile's end are in bounds and unused), so their latency hides behind that
    // step's arithmetic; fp32 inputs' wider register banks leave no room for
    // the prefetch (it would spill), so they read each step's operands there.
    constexpr bool kPrefetch = sizeof(Tin) == 2;
    float2 fv;
    float fdy;
    float4 fb, fc;
    auto fetch = [&](int r) SSM_INLINE {
      fv = sh_dtu[r][loff];
      fdy = sh_dy[r][loff];
      fb = *reinterpret_cast<const float4*>(&sh_B[r][g * NS]);
      fc = *reinterpret_cast<const float4*>(&sh_C[r][g * NS]);
    };
    if (kPrefetch) fetch(T - 1);
#pragma unroll
    for (int s = T - 1; s >= 0; --s) {
      if (!kPrefetch) fetch(s);
      const float2 v = fv;
      const float dy = fdy;
      const float bq[4] = {fb.x, fb.y, fb.z, fb.w}, cq[4] = {fc.x, fc.y, fc.z, fc.w};
      if (kPrefetch && s > 0) fetch(s - 1);
      if (s < nt) {
        float s1 = 0.0f, s2 = 0.0f, cb[NS], cc[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const float aa = kKeepA ? ap[s][i] : __builtin_amdgcn_exp2f(v.x * Ad[i]);
          const float Bs = bq[i];
          const float dh = __builtin_fmaf(dy, cq[i], carry[i]);
          const float hs = s + 1 < T ? hp[s + 1][i] : h[i];  // the state after step s
          cc[i] = dy * hs;
          cb[i] = dh * v.y;
          s1 = __builtin_fmaf(dh, Bs, s1);
          const float qv = dh * aa * hp[s][i];
          s2 = __builtin_fmaf(qv, Ad[i], s2);
          dAacc[i] = __builtin_fmaf(qv, v.x, dAacc[i]);
          carry[i] = aa * dh;
        }
        sh_s1[s][g * kWave + lane] = s1;
        sh_s2[s][g * kWave + lane] = s2;
        // dB', dC of this step over the wavefront's 64 channels (lanes),
        // in registers; lanes past the last channel hold duplicates and
        // contribute zero
        float v8[8];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          v8[i] = cb[i];
          v8[NS + i] = cc[i];
        }
        if (nvalid != kWave) {
#pragma unroll
          for (int i = 0; i < 8; ++i) v8[i] = lane < nvalid ? v8[i] : 0.0f;
        }
        const float tot = lane_sum8(v8, lane);
        if ((lane & 7) == 0) {
          const int j = sum8_index(lane);
          sh_bc[s][j >> 2][g * NS + (j & 3)] = tot;
        }
      }
    }
    block_sync();

    // per element: dz, dx, ddelta; per channel: dD, dbias
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int r = irow[it];
      if (r < nt) {
        float ox[CW], od[CW], oz[CW];
#pragma unroll
        for (int q = 0; q < CW; ++q) {
          const int col = icol[it] + q;
          float S1 = 0.0f, S2 = 0.0f, y = 0.0f;
#pragma unroll
          for (int gg = 0; gg < G; ++gg) {
            S1 += sh_s1[r][gg * kWave + col];
            S2 += sh_s2[r][gg * kWave + col];
            if (HAS_Z) y += sh_y[r][gg * kWave + col];
          }
          float xq, dt2q, dyq;
          elem(it, q, xq, dt2q, dyq);
          if (HAS_Z) {
            y = __builtin_fmaf(iD[it][q], xq, y);
            const float z = cur.rz[it].get(q);
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
            oz[q] = cur.rg[it].get(q) * y * (sg * __builtin_fmaf(z, 1.0f - sg, 1.0f));
          }
          ox[q] = __builtin_fmaf(dyq, iD[it][q], dt2q * S1);
          const float ddt = __builtin_fmaf(xq * kLog2e, S1, S2);
          const float u = cur.rd[it].get(q) + ibias[it][q];
          od[q] = softplus ? ddt * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u * kLog2e)) : ddt;
          dDacc[it][q] = __builtin_fmaf(dyq, xq, dDacc[it][q]);
          dBacc[it][q] += od[q];
        }
        const int64_t off = (t0 + r) * Dn + icol[it];
        store_row<Tg, CW>(static_cast<Tg*>(a.dx) + row0 + off, ox);
        store_row<Tg, CW>(static_cast<Tg*>(a.ddelta) + row0 + off, od);
        if (HAS_Z) store_row<Tg, CW>(static_cast<Tg*>(a.dz) + row0 + off, oz);
      }
    }
    // this tile's dB', dC of the block
    for (int i = tid; i < nt * 2 * kDState; i += NTHR) {
      const int s = i / (2 * kDState), w = i % (2 * kDState);
      a.ws_bc[((b * L + t_begin + t0 + s) * a.nblk + blk) * (2 * kDState) + w] = (&sh_bc[s][0][0])[w];
    }
    block_sync();
    cur = nxt;
  }

  // per-(row, chunk) parameter gradients and the initial state's gradient
  if (lane < nvalid) {
    *reinterpret_cast<float4*>(a.ws_a + (row * Dn + dl) * kDState + g * NS) =
        make_float4(dAacc[0] * kLn2, dAacc[1] * kLn2, dAacc[2] * kLn2, dAacc[3] * kLn2);
    if (kc == 0 && a.dh0 != nullptr)
      *reinterpret_cast<float4*>(a.dh0 + (b * Dn + dl) * kDState + g * NS) =
          make_float4(carry[0], carry[1], carry[2], carry[3]);
  }
  // dD and dbias: the items of one channel are summed over rows in row order
  float* sred = &sh_s1[0][0];  // free after the last tile: [T][64] x 2
#pragma unroll
  for (int it = 0; it < IPT; ++it)
#pragma unroll
    for (int q = 0; q < CW; ++q) {
      sred[irow[it] * kWave + icol[it] + q] = dDacc[it][q];
      sred[T * kWave + irow[it] * kWave + icol[it] + q] = dBacc[it][q];
    }
  block_sync();
  if (tid < kWave && tid < nvalid) {
    float sD = 0.0f, sB = 0.0f;
    for (int r = 0; r < T; ++r) {
      sD += sred[r * kWave + tid];
      sB += sred[T * kWave + r * kWave + tid];
    }
    a.ws_dd[(row * Dn + d0 + tid) * 2] = sD;
    a.ws_dd[(row * Dn + d0 + tid) * 2 + 1] = sB;
  }
}

// ------------------------------------------------- chunked backward carries
//
// The gradient arriving at the end of chunk k depends on chunks k+1 .. K-1
// only through an affine map: with g the gradient with respect to the state
// after chunk k+1's last step, the reverse recurrence over chunk k+1 yields
//   dL/d(state entering chunk k+1) = r_{k+1} + exp2(A S_{k+1}) g,
// where r_{k+1} is that walk started from g = 0 and S_{k+1} the chunk's
// step-size sum (log2 units).  That is the pair operator of the forward's
// chunk carry, applied in reverse time order.
//
// bwd_rev_kernel: r_k and S_k for chunks k = 1 .. K-1, one workgroup per
// (chunk, batch row, 64-channel block), lane = channel and 4 states per lane
// as in the backward kernel.  Tiles of 32 steps are walked from the chunk's
// end (its ragged tile first); each stages (dt2, dy) and C in LDS and runs
//   g <- exp2(dt2 A) (dy C + g)
// over its steps in reverse.  As in the forward scan, a thread item is 8
// consecutive channels of one step (16-byte loads) when d_inner is a multiple
// of 8, else one channel; the next tile's raw inputs load behind the current
// tile's arithmetic.
template <typename Tin, typename Tg, bool HAS_Z, bool WIDE>
__global__ void __launch_bounds__(256) bwd_rev_kernel(BwdArgs a) {
  constexpr int NS = 4, T = 32, NTHR = 256;
  constexpr int CW = WIDE ? 8 : 1;
  constexpr int CPR = kWave / CW;
  constexpr int IPT = T * CPR / NTHR;
  static_assert(IPT >= 1 && IPT * NTHR == T * CPR, "tile does not split evenly");
  constexpr int EPV = Vec16<Tin>::kElems;   // C elements per 16-byte vector
  constexpr int CVECS = T * kDState / EPV;  // 16-byte vectors of a tile's C rows
  static_assert(CVECS <= NTHR, "C staging takes at most one vector per thread");
  using R = Raw<Tin, CW>;
  using RG = Raw<Tg, CW>;
  __shared__ float2 sh_dty[T][kWave + 1];   // (dt2, dy)
  __shared__ float sh_C[T][kDState];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int g = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int64_t b = blockIdx.z;
  const int kc = blockIdx.y + 1;
  const int blk = blockIdx.x;
  const int64_t Dn = a.d_inner, L = a.seqlen;
  const int64_t d0 = (int64_t)blk * kWave;
  const int nvalid = (int)min((int64_t)kWave, Dn - d0);
  const int loff = min(lane, nvalid - 1);
  const int64_t dl = d0 + loff;
  const bool softplus = a.softplus != 0;
  const int64_t t_begin = (int64_t)kc * a.chunk_len;
  const int64_t Lc = min(a.chunk_len, L - t_begin);
  const int64_t ntiles = (Lc + T - 1) / T;

  float Ad[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) Ad[i] = a.A[dl * kDState + g * NS + i];
  int irow[IPT], icol[IPT];
  float ibias[IPT][CW];
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int idx = tid + it * NTHR;
    irow[it] = idx / CPR;
    icol[it] = min(idx % CPR, (nvalid + CW - 1) / CW - 1) * CW;
#pragma unroll
    for (int q = 0; q < CW; ++q) {
      const int64_t dq = d0 + min(icol[it] + q, nvalid - 1);
      ibias[it][q] = a.bias != nullptr ? a.bias[dq] : 0.0f;
    }
  }
  const int64_t row0 = (b * L + t_begin) * Dn + d0;
  const Tin* db = static_cast<const Tin*>(a.delta) + row0;
  const Tin* zb = HAS_Z ? static_cast<const Tin*>(a.z) + row0 : nullptr;
  const Tg* gb = static_cast<const Tg*>(a.dout) + row0;
  const Tin* Cb = static_cast<const Tin*>(a.C) + (b * L + t_begin) * kDState;

  struct Bank {
    R rd[IPT], rz[IPT];
    RG rg[IPT];
    uint4 cv;
  };
  // rows past the tile's end repeat its last row, so every load is unconditional
  auto load = [&](Bank& bk, int64_t k) SSM_INLINE {
    const int64_t t0 = k * T;
    const int nt = (int)min((int64_t)T, Lc - t0);
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int64_t off = (t0 + min(irow[it], nt - 1)) * Dn + icol[it];
      bk.rd[it].load(db + off);
      bk.rg[it].load(gb + off);
      if (HAS_Z) bk.rz[it].load(zb + off);
    }
    const int v = tid % CVECS;
    const int64_t t = t0 + min(v / (kDState / EPV), nt - 1);
    bk.cv = *reinterpret_cast<const uint4*>(Cb + t * kDState + (v % (kDState / EPV)) * EPV);
  };
  auto stage = [&](const Bank& bk) SSM_INLINE {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
#pragma unroll
      for (int q = 0; q < CW; ++q) {
        const float u2 = (bk.rd[it].get(q) + ibias[it][q]) * kLog2e;
        const float dt2 = softplus ? softplus2_f(u2) : u2;
        float dy = bk.rg[it].get(q);
        if (HAS_Z) dy = dy * silu_f(bk.rz[it].get(q));
        sh_dty[irow[it]][icol[it] + q] = make_float2(dt2, dy);
      }
    }
    if (tid < CVECS) {
      float f[EPV];
      Vec16<Tin>::unpack(bk.cv, f);
      float* dst = &sh_C[tid / (kDState / EPV)][(tid % (kDState / EPV)) * EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) dst[e] = f[e];
    }
  };

  float gacc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) gacc[i] = 0.0f;
  float dtsum = 0.0f;
  auto step = [&](int s) SSM_INLINE {
    const float2 v = sh_dty[s][loff];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const float dh = __builtin_fmaf(v.y, sh_C[s][g * NS + i], gacc[i]);
      gacc[i] = __builtin_amdgcn_exp2f(v.x * Ad[i]) * dh;
    }
    dtsum += v.x;
  };
  Bank cur, nxt;
  load(cur, ntiles - 1);
  for (int64_t k = ntiles - 1; k >= 0; --k) {
    const int nt = (int)min((int64_t)T, Lc - k * T);
    stage(cur);
    if (k > 0) load(nxt, k - 1);
    block_sync();
    if (nt == T) {   // every tile but possibly the chunk's last, which is walked first
#pragma unroll
      for (int s = T - 1; s >= 0; --s) step(s);
    } else {
      for (int s = nt - 1; s >= 0; --s) step(s);
    }
    block_sync();
    cur = nxt;
  }
  if (lane < nvalid) {
    const int64_t slot = (b * a.n_chunks + kc) * Dn + dl;
    *reinterpret_cast<float4*>(a.ws_rev + slot * kDState + g * NS) = make_float4(gacc[0], gacc[1], gacc[2], gacc[3]);
    if (g == 0) a.ws_rsum[slot] = dtsum;
  }
}

// bwd_rev_carry_kernel: the gradient arriving at the end of every chunk but
// the last, composing the chunks' pairs from the sequence's end (where the
// caller's dlast, or zero, arrives) in reverse order.  One thread per
// (batch row, channel, state), sequential over chunks.
__global__ void __launch_bounds__(256) bwd_rev_carry_kernel(BwdArgs a) {
  const int64_t ncol = a.d_inner * kDState;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = blockIdx.y;
  if (i >= ncol) return;
  const int K = a.n_chunks;
  const float a2 = a.A[i];
  float gv = a.dlast != nullptr ? a.dlast[b * ncol + i] : 0.0f;
  for (int k = K - 1; k >= 1; --k) {
    const int64_t p = b * K + k;
    gv = __builtin_fmaf(__builtin_amdgcn_exp2f(a2 * a.ws_rsum[p * a.d_inner + (i >> 4)]), gv,
                        a.ws_rev[p * ncol + i]);
    a.ws_dl[(p - 1) * ncol + i] = gv;
  }
}

// dB, dC: sum the per-block partials (dB also takes the ln 2).  One wavefront
// per (batch row, step): that row's nblk x 32 partials are contiguous, so the
// wavefront reads them with 16-byte loads, lane l taking float4s l, l + 64, ...
// Every such float4 holds values 4(l % 8) .. 4(l % 8) + 3 of one block, so
// each lane sums its blocks in order and the 8 lanes with equal l % 8 then
// combine theirs (xor 8, 16, 32): a fixed order, the same on every call.
template <typename Tg>
__global__ void __launch_bounds__(256) bwd_reduce_bc_kernel(const float* ws_bc, Tg* dB, Tg* dC, int64_t rows,
                                                            int nblk) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float4* src = reinterpret_cast<const float4*>(ws_bc + row * nblk * (2 * kDState));
  const int n4 = nblk * (2 * kDState / 4);
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 4
  for (int q = lane; q < n4; q += kWave) {
    const float4 v = src[q];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
#pragma unroll
  for (int m = 8; m < kWave; m <<= 1) {
    acc.x += __shfl_xor(acc.x, m);
    acc.y += __shfl_xor(acc.y, m);
    acc.z += __shfl_xor(acc.z, m);
    acc.w += __shfl_xor(acc.w, m);
  }
  if (lane >= 8) return;
  const bool isB = lane < 4;
  Tg* dst = (isB ? dB : dC) + row * kDState + 4 * (lane & 3);
  const float f = isB ? kLn2 : 1.0f;
  const float v[4] = {acc.x * f, acc.y * f, acc.z * f, acc.w * f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (sizeof(Tg) == 4) dst[j] = v[j];
    else dst[j] = f32_to_bf16_rne(v[j]);
  }
}

// dA, dD, dbias: sum the per-(row, chunk) partials in order (`batch` counts
// rows times chunks).
__global__ void __launch_bounds__(256) bwd_reduce_params_kernel(const float* ws_a, const float* ws_dd, float* dA,
                                                                float* dD, float* dbias, int64_t batch,
                                                                int64_t Dn) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < Dn * kDState) {
    float acc = 0.0f;
    for (int64_t b = 0; b < batch; ++b) acc += ws_a[b * Dn * kDState + i];
    dA[i] = acc;
  }
  if (i < Dn) {
    float sD = 0.0f, sB = 0.0f;
    for (int64_t b = 0; b < batch; ++b) {
      sD += ws_dd[(b * Dn + i) * 2];
      sB += ws_dd[(b * Dn + i) * 2 + 1];
    }
    if (dD != nullptr) dD[i] = sD;
    if (dbias != nullptr) dbias[i] = sB;
  }
}

}  // namespace

namespace {

// One launch of a backward kernel instance, with the progress-priority scheme
// (ProgressPriority) on when the device holds the whole grid at once.
template <typename K>
void launch_bwd_pass(K kern, dim3 grid, const BwdArgs& a, hipStream_t s) {
  BwdArgs b = a;
  b.fair = grid_coresident(resident_per_cu(kern, 256), a.cus, grid) ? 1 : 0;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, b);
}

// The forward scan's arguments for the backward's forward work: the chunk
// carry (states_only) and the checkpoint pass (ckpt).
ScanArgs forward_args(const BwdArgs& a) {
  ScanArgs f{};
  f.x = a.x;
  f.delta = a.delta;
  f.B = a.B;
  f.C = a.C;
  f.A = a.A;
  f.bias = a.bias;
  f.h0 = a.h0;
  f.ws_state = a.ws_hin;
  f.ws_dtsum = a.ws_fsum;
  f.seqlen = a.seqlen;
  f.d_inner = a.d_inner;
  f.chunk_len = a.chunk_len;
  f.n_chunks = a.n_chunks;
  f.softplus = a.softplus;
  f.batch = a.batch;
  f.cus = a.cus;
  return f;
}

// The chunked backward's carries: each chunk's entering state (the forward's
// pass A and carry, run by the forward scan's own launcher; only to start the
// checkpoint pass, so not when the checkpoints are given), then each chunk's
// arriving gradient (reverse pass A, reverse carry).
template <typename Tin, typename Tg>
hipError_t launch_bwd_carries(const BwdArgs& a, DT in, hipStream_t s) {
  if (!a.ckpt_given) {
    ScanArgs f = forward_args(a);
    f.states_only = 1;
    const hipError_t e = launch_scan(f, in, DT::F32, 4, s);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)a.nblk, (unsigned)(a.n_chunks - 1), (unsigned)a.batch);
  // the wide items need rows that split into aligned groups of 8
  const bool wide = a.d_inner % 8 == 0;
  if (a.z != nullptr) {
    if (wide) hipLaunchKernelGGL((bwd_rev_kernel<Tin, Tg, true, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((bwd_rev_kernel<Tin, Tg, true, false>), grid, dim3(256), 0, s, a);
  } else {
    if (wide) hipLaunchKernelGGL((bwd_rev_kernel<Tin, Tg, false, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((bwd_rev_kernel<Tin, Tg, false, false>), grid, dim3(256), 0, s, a);
  }
  const unsigned ncolblk = (unsigned)((a.d_inner * kDState + 255) / 256);
  hipLaunchKernelGGL(bwd_rev_carry_kernel, dim3(ncolblk, (unsigned)a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename Tin, typename Tg>
hipError_t launch_scan_bwd_t(const BwdArgs& a, DT in, float* dA, void* dB, void* dC, float* dD, float* dbias,
                             hipStream_t s) {
  const dim3 grid((unsigned)a.nblk, (unsigned)a.n_chunks, (unsigned)a.batch);
  // the state entering every 8-step tile, from the forward scan kernel's
  // checkpoint pass (after the chunk carry, whose states it starts from)
  auto checkpoints = [&]() {
    if (a.ckpt_given) return hipSuccess;
    ScanArgs f = forward_args(a);
    f.ckpt = a.ws_ckpt;
    f.ckpt_only = 1;
    f.ckpt_nblk = a.nblk;
    f.ckpt_tiles = (a.seqlen + kBwdTile - 1) / kBwdTile;
    return launch_scan(f, in, DT::F32, 4, s);
  };
  if (a.seqlen > 0) {
    // channels per element item: 8-step tiles x 64 channels = 256 threads x 2
    if (a.d_inner % 2 == 0) {
      if (a.n_chunks > 1) {
        const hipError_t e = launch_bwd_carries<Tin, Tg>(a, in, s);
        if (e != hipSuccess) return e;
      }
      if (const hipError_t e = checkpoints(); e != hipSuccess) return e;
      if (a.z != nullptr) launch_bwd_pass(scan_bwd_kernel<Tin, Tg, true, 2>, grid, a, s);
      else launch_bwd_pass(scan_bwd_kernel<Tin, Tg, false, 2>, grid, a, s);
    } else {
      if (a.n_chunks > 1) {
        const hipError_t e = launch_bwd_carries<Tin, Tg>(a, in, s);
        if (e != hipSuccess) return e;
      }
      if (const hipError_t e = checkpoints(); e != hipSuccess) return e;
      if (a.z != nullptr) launch_bwd_pass(scan_bwd_kernel<Tin, Tg, true, 1>, grid, a, s);
      else launch_bwd_pass(scan_bwd_kernel<Tin, Tg, false, 1>, grid, a, s);
    }
    const int64_t rows = (int64_t)a.batch * a.seqlen;
    hipLaunchKernelGGL((bwd_reduce_bc_kernel<Tg>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a.ws_bc,
                       static_cast<Tg*>(dB), static_cast<Tg*>(dC), rows, a.nblk);
  }
  const int64_t np = a.d_inner * kDState;
  hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, s, a.ws_a, a.ws_dd,
                     dA, dD, dbias, (int64_t)a.batch * a.n_chunks, a.d_inner);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_bwd(const BwdArgs& a, DT in, DT grad, float* dA, void* dB, void* dC, float* dD,
                           float* dbias, hipStream_t s) {
  if (in == DT::F32 && grad == DT::F32) return launch_scan_bwd_t<float, float>(a, in, dA, dB, dC, dD, dbias, s);
  if (in == DT::F32 && grad == DT::BF16) return launch_scan_bwd_t<float, uint16_t>(a, in, dA, dB, dC, dD, dbias, s);
  if (in == DT::BF16 && grad == DT::F32) return launch_scan_bwd_t<uint16_t, float>(a, in, dA, dB, dC, dD, dbias, s);
  return launch_scan_bwd_t<uint16_t, uint16_t>(a, in, dA, dB, dC, dD, dbias, s);
}

}  // namespace ssm

// The chunked selective-scan kernel of libssmscan (template) and its launch
// templates, included by scan_inst.hip, which the build compiles once per
// (input dtype, output dtype, input coefficient).
#ifndef SSMSCAN_SCAN_KERNEL_H
#define SSMSCAN_SCAN_KERNEL_H

#include "device.h"

namespace ssm {
namespace {

// The main loop is straight-line code: loads, LDS staging and stores are all
// unconditional, so the compiler can count outstanding memory operations
// exactly and wait only for the tile it needs.  (Any conditional load or
// store inside the loop makes it fall back to draining the whole memory
// pipeline at every tile.)  To get there:
//  * the ragged part of the chunk (nsteps % T steps) is peeled off and run
//    first as one short tile; every later tile is full;
//  * lanes past the last channel compute the last channel's values, which
//    are bit-identical, and items past it repeat the last item's work, so
//    their duplicate stores are benign;
//  * threads past the B/C staging work stage a duplicate of another thread's
//    vector (same value, same LDS address);
//  * two register banks hold the raw inputs of the next two tiles, so each
//    thread keeps two tiles of HBM reads in flight behind its arithmetic; the
//    prefetch index is clamped to the last tile, so it always reads valid rows.
//
// Phases 1 and 3 are elementwise over (step, channel), so they use their own
// thread mapping: with WIDE, thread item (row r, chunk c) covers CW
// consecutive channels of one step, read and written with 16-byte accesses
// (1 KiB per wavefront instruction); without WIDE (d_inner not a multiple of
// 8), CW = 1 and an item is one channel.  Phase 2 keeps lane = channel.
//
// ZOH selects the exact zero-order-hold input coefficient: per state the
// update adds zoh_ratio(a) * (dt2 x) * B with a = exp2(dt2 A), which is
// (e^{dt A} - 1) / A * x * B (B is then staged without the ln 2 factor).
//
// Transitions from powers (NS == 4, dt coefficient).  Where every channel of
// the block has A[d, n] = (n + 1) * A[d, 0] -- the standard initialisation
// A = -exp(log(n + 1)) -- the transitions of one step are powers of one
// number: exp(dt A[d, n]) = e^(n + 1) with e = exp2(dt2 A[d, 0]).  Phase 1
// then stages e in place of dt2 (one exponential per (step, channel)), and
// the recurrence forms e^(n + 1) by multiplication: its instruction stream
// holds no transcendental, so gfx950 issues its fp32 VALU work at about twice
// the rate it manages beside v_exp_f32 (about 2.2 against 4 SIMD-cycles per
// wave64 instruction, measured).  A workgroup checks this structure of A
// exactly, once, and otherwise runs the exponentials.  With NS == 4, wave g
// carries the states n = g + 4 i (i < 4), so its transitions are
// e^(g+1) * (e^4)^i; B and C rows are staged in that order.
template <typename Tin, typename Tout, int NS, bool PASS_A, bool HAS_Z, bool WIDE, bool ZOH, bool CKPT = false>
__global__ void __launch_bounds__(kWave * (kDState / NS))
scan_chunk_kernel(ScanArgs a) {
  constexpr int G = kDState / NS;         // wavefronts per workgroup (state groups)
  constexpr int T = Tile<G>::T;           // time steps per tile
  constexpr int NTHR = kWave * G;
  constexpr int CW = WIDE ? Tile<G>::CW : 1;   // channels per item
  constexpr int CPR = kWave / CW;         // items per row
  constexpr int IPT = T * CPR / NTHR;     // items per thread
  static_assert(IPT >= 1 && IPT * NTHR == T * CPR, "tile does not split evenly");
  constexpr int EPV = Vec16<Tin>::kElems; // B/C elements per 16-byte vector
  constexpr int VPR = kDState / EPV;      // 16-byte vectors per B or C row
  constexpr int BC_VECS = (PASS_A ? 1 : 2) * T * VPR;
  constexpr int BC_R = (BC_VECS + NTHR - 1) / NTHR;
  constexpr bool kZ = HAS_Z && !PASS_A;
  // states of wave g: g + 4 i (interleaved) with NS == 4, else g * NS + i
  constexpr bool kPerm = NS == 4;
  constexpr bool kPow = kPerm && !ZOH;
  using R = Raw<Tin, CW>;

  // Rows are padded by one element: the prologue/epilogue items (CW
  // consecutive channels per thread, 64 / CW threads per row) then spread
  // over all LDS banks, while lane = channel accesses stay consecutive.
  __shared__ float2 sh_dtv[T][kWave + 1];             // (dt, dt * x)
  __shared__ float sh_B[T][kDState];
  __shared__ float sh_C[PASS_A ? 1 : T][kDState];
  __shared__ float sh_y[PASS_A ? 1 : T][G * kWave + 1];  // partial readouts, [row][wave][channel]

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // the wave index is uniform across the wave: keep it in a scalar register
  const int g = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int b = blockIdx.z;
  const int k = blockIdx.y;
  const int K = a.n_chunks;
  const int64_t Dn = a.d_inner;
  const int64_t L = a.seqlen;
  const int64_t d0 = (int64_t)blockIdx.x * kWave;
  const int nvalid = (int)min((int64_t)kWave, Dn - d0);   // channels of this block
  // phase 2: lanes past the last channel take the last channel's place
  const int loff = min(lane, nvalid - 1);
  const int64_t dl = d0 + loff;
  const int64_t t_begin = (int64_t)k * a.chunk_len;
  const int64_t t_end = min(t_begin + a.chunk_len, L);
  const bool softplus = a.softplus != 0;
  const bool has_D = a.D != nullptr;

  // the state held in slot i of this wave
  auto st_of = [&](int i) SSM_INLINE { return kPerm ? g + 4 * i : g * NS + i; };
  float Ad[NS];  // this lane's A[d, n]; step sizes are in log2 units (dt2)
#pragma unroll
  for (int i = 0; i < NS; ++i) Ad[i] = a.A[dl * kDState + st_of(i)];
  // Transitions from powers when every channel's A row is (n + 1) * A[d, 0]
  // (the check is exact; every wave covers the same channels, so all waves of
  // the workgroup reach the same answer).
  bool pow_mode = false;
  float pf1 = 0.0f, pn1 = 1.0f, pf2 = 0.0f, pn2 = 1.0f;  // selects e^(g+1) = e * e^(g&1) * (e^2)^(g>>1)
  if constexpr (kPow) {
    const float* Ar = a.A + dl * kDState;
    bool ok = true;
#pragma unroll
    for (int n = 1; n < kDState; ++n) ok = ok && (Ar[n] == (float)(n + 1) * Ar[0]);
    pow_mode = __all(ok);
    // per-wave constants, kept in VGPRs (computed from the thread index): an SGPR
    // operand would slow the VALU instructions that read it
    const int gv = (int)(threadIdx.x >> 6);
    pf1 = (float)(gv & 1);
    pn1 = 1.0f - pf1;
    pf2 = (float)((gv >> 1) & 1);
    pn2 = 1.0f - pf2;
  }

  // phases 1 and 3: this thread's items (row, first channel), fixed for the kernel.
  // (Their per-channel parameters stay in registers: LDS tables for them would
  // take the workgroup past the LDS share that lets three share a CU.)
  int irow[IPT], icol[IPT];
  float ibias[IPT][CW], iD[IPT][CW];  // bias in log2 units, D
  float iA0[kPow ? IPT : 1][kPow ? CW : 1];  // A[d, 0] of the items (transitions from powers)
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int idx = tid + it * NTHR;
    irow[it] = idx / CPR;
    icol[it] = min(idx % CPR, (nvalid + CW - 1) / CW - 1) * CW;  // clamp to the last valid item
#pragma unroll
    for (int q = 0; q < CW; ++q) {
      const int64_t dq = d0 + min(icol[it] + q, nvalid - 1);
      ibias[it][q] = a.bias != nullptr ? a.bias[dq] * kLog2e : 0.0f;
      iD[it][q] = has_D ? a.D[dq] : 0.0f;
      if constexpr (kPow) iA0[it][q] = a.A[dq * kDState];
    }
  }

  // checkpoints (see ScanArgs::ckpt), a separate instance: stored by pass B,
  // or by pass A's instance run from each chunk's entering state (ckpt_only).
  // (A runtime switch in the ordinary instances cost 10 % on the layer.)
  constexpr bool ckpt_mode = CKPT && NS == 4;
  float h[NS];
  if ((!PASS_A || ckpt_mode) && k > 0) {
    const float* src = a.ws_state + (((int64_t)b * K + (k - 1)) * Dn + dl) * kDState;
#pragma unroll
    for (int i = 0; i < NS; ++i) h[i] = src[st_of(i)];
  } else if (k == 0 && a.h0 != nullptr) {  // continuing from a stored state
    const float* src = a.h0 + ((int64_t)b * Dn + dl) * kDState;
#pragma unroll
    for (int i = 0; i < NS; ++i) h[i] = src[st_of(i)];
  } else {
#pragma unroll
    for (int i = 0; i < NS; ++i) h[i] = 0.0f;
  }
  float dtsum = 0.0f;
  // pass A with powers: the step sizes of this thread's items, summed over the
  // chunk's steps in the staging phase (reduced over threads at the end)
  constexpr bool kItemSum = PASS_A && kPow && !CKPT;  // the checkpoint pass writes no sums
  float isum[kItemSum ? IPT : 1][kItemSum ? CW : 1];
#pragma unroll
  for (int it = 0; it < (kItemSum ? IPT : 1); ++it)
#pragma unroll
    for (int q = 0; q < (kItemSum ? CW : 1); ++q) isum[it][q] = 0.0f;
  float* const ckb = ckpt_mode ? a.ckpt + (((int64_t)b * a.ckpt_nblk + blockIdx.x) * a.ckpt_tiles) * (kWave * kDState) +
                                     lane * kDState + g * 4
                               : nullptr;
  // the state entering chunk-relative step tt (t_begin + tt a multiple of 8)
  auto store_ckpt = [&](int64_t tt) SSM_INLINE {
    if constexpr (NS == 4)
      *reinterpret_cast<float4*>(ckb + ((t_begin + tt) >> 3) * (kWave * kDState)) = make_float4(h[0], h[1], h[2], h[3]);
  };

  // Row pointers of this chunk: element (t_begin + tt, d0) of batch row b.
  const int64_t base_e = ((int64_t)b * L + t_begin) * Dn + d0;
  const Tin* xb = static_cast<const Tin*>(a.x) + base_e;
  const Tin* db = static_cast<const Tin*>(a.delta) + base_e;
  const Tin* zb = kZ ? static_cast<const Tin*>(a.z) + base_e : nullptr;
  Tout* ob = PASS_A ? nullptr : static_cast<Tout*>(a.out) + base_e;
  const Tin* Bb = static_cast<const Tin*>(a.B) + ((int64_t)b * L + t_begin) * kDState;
  const Tin* Cb = static_cast<const Tin*>(a.C) + ((int64_t)b * L + t_begin) * kDState;

  struct Bank {
    R rx[IPT], rdt[IPT], rz[IPT];
    uint4 rbc[BC_R];
  };
  Bank bk0, bk1;
  float xs[IPT][CW];    // x of the tile being finished
  R zs[IPT];            // raw z of the tile being finished

  // Issue the loads of the tile at chunk-relative step tt0 with nt valid steps
  // (rows past nt re-read the last valid row).
  auto issue = [&](Bank& bk, int64_t tt0, int nt) SSM_INLINE {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int64_t off = (tt0 + min(irow[it], nt - 1)) * Dn + icol[it];
      bk.rx[it].load(xb + off);
      bk.rdt[it].load(db + off);
      if (kZ) bk.rz[it].load(zb + off);
    }
#pragma unroll
    for (int r = 0; r < BC_R; ++r) {
      const int v = (tid + r * NTHR) % BC_VECS;
      const int which = v / (T * VPR);
      const int w = v - which * (T * VPR);
      const int row = min(w / VPR, nt - 1);
      const int part = w % VPR;
      const Tin* src = (which ? Cb : Bb) + (tt0 + row) * kDState + part * EPV;
      bk.rbc[r] = *reinterpret_cast<const uint4*>(src);
    }
  };

  // Phase 1: discretise this thread's items into LDS as (dt2, dt2 * x), the
  // step size in log2 units and the input term's factor (the ln 2 that
  // dt2 * x carries is folded into the staged B rows); stage B/C rows as
  // fp32.  The softplus switch is taken once per tile (a uniform branch
  // around the whole item loop), never per element.
  // With transitions from powers, (e, dt2 * x) is staged, e = exp2(dt2 A[d, 0]).
  auto discretise = [&](Bank& bk, int nt, auto sp_c, auto pow_c) SSM_INLINE {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
#pragma unroll
      for (int q = 0; q < CW; ++q) {
        const float x = bk.rx[it].get(q);
        const float u2 = __builtin_fmaf(bk.rdt[it].get(q), kLog2e, ibias[it][q]);
        const float dt2 = decltype(sp_c)::value ? softplus2_f(u2) : u2;
        if constexpr (decltype(pow_c)::value) {
          sh_dtv[irow[it]][icol[it] + q] = make_float2(__builtin_amdgcn_exp2f(dt2 * iA0[it][q]), dt2 * x);
          // rows past a ragged tile's end repeat its last row: not summed
          if constexpr (kItemSum) isum[it][q] += irow[it] < nt ? dt2 : 0.0f;
        } else {
          sh_dtv[irow[it]][icol[it] + q] = make_float2(dt2, dt2 * x);
        }
        xs[it][q] = x;
      }
    }
  };
  auto commit = [&](Bank& bk, int nt) SSM_INLINE {
    if constexpr (kPow) {
      if (pow_mode) {
        if (softplus) discretise(bk, nt, std::true_type(), std::true_type());
        else discretise(bk, nt, std::false_type(), std::true_type());
      } else {
        if (softplus) discretise(bk, nt, std::true_type(), std::false_type());
        else discretise(bk, nt, std::false_type(), std::false_type());
      }
    } else {
      if (softplus) discretise(bk, nt, std::true_type(), std::false_type());
      else discretise(bk, nt, std::false_type(), std::false_type());
    }
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      if (kZ) zs[it] = bk.rz[it];
    }
#pragma unroll
    for (int r = 0; r < BC_R; ++r) {
      const int v = (tid + r * NTHR) % BC_VECS;
      const int which = v / (T * VPR);
      const int w = v - which * (T * VPR);
      const int row = w / VPR;
      const int part = w % VPR;
      float f[EPV];
      Vec16<Tin>::unpack(bk.rbc[r], f);
      float* dst = which ? &sh_C[PASS_A ? 0 : row][0] : &sh_B[row][0];
      // B carries the ln 2 of dt2 * x; with ZOH, zoh_ratio carries it
      const float scale = (which || ZOH) ? 1.0f : kLn2;
#pragma unroll
      for (int i = 0; i < EPV; ++i) {
        // state n goes to the slot that the wave holding it reads: slot g * NS + i
        // holds state g + 4 i when the states are interleaved
        const int n = part * EPV + i;
        dst[kPerm ? (n & 3) * 4 + (n >> 2) : n] = f[i] * scale;
      }
    }
  };

  // Phase 2: the recurrence for this wave's NS states over steps [0, n).
  // Software-pipelined by one step: the transitions exp(dt * A) of step s + 1
  // (and with ZOH their input ratios) do not depend on the state, so they are
  // computed while step s updates it, which keeps each exp's latency off the
  // h dependency chain.
  constexpr int NR = ZOH ? NS : 1;
  // The recurrence with transitions from powers: slot i holds state g + 4 i,
  // whose transition is e^(g+1) * (e^4)^i; e^(g+1) = e * e^(g&1) * (e^2)^(g>>1)
  // is selected by per-wave 0/1 constants (fma(f, v, 1 - f) is v or exactly 1)
  // in the peeled ragged tile; full tiles run a copy of the loop per wave with
  // the base formed directly.  No transcendental: at most eight multiplies,
  // two selects and the update's three instructions per state.
  auto run_steps_pow_plain = [&](int n, int64_t tt0) SSM_INLINE {  // the peeled ragged tile
    const int ph = (int)((t_begin + tt0) & 7);
    for (int s = 0; s < n; ++s) {
      if (ckpt_mode && ((ph + s) & 7) == 0) store_ckpt(tt0 + s);
      const float2 v = sh_dtv[s][loff];
      const float e = v.x;
      const float e2 = e * e;
      const float e4 = e2 * e2;
      float ap = (e * __builtin_fmaf(pf1, e, pn1)) * __builtin_fmaf(pf2, e2, pn2);
      float y = 0.0f;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (i > 0) ap = ap * e4;
        h[i] = __builtin_fmaf(ap, h[i], v.y * sh_B[s][g * NS + i]);
        if (!PASS_A) y = __builtin_fmaf(sh_C[PASS_A ? 0 : s][g * NS + i], h[i], y);
      }
      if (!PASS_A) sh_y[PASS_A ? 0 : s][(PASS_A ? 0 : g) * kWave + lane] = y;
    }
  };
  // Full tiles (n is a constant), instantiated once per wave: GB is the wave
  // index g, so the base e^(g+1) is e, e^2, e * e^2 or e^4, the same products
  // the selects form, with no select.
  auto run_steps_pow_piped = [&](auto n_c, auto gb_c, int64_t tt0) SSM_INLINE {
    constexpr int n = decltype(n_c)::value;
    constexpr int GB = decltype(gb_c)::value;
    // Keeps the compiler from hoisting the four copies' common LDS reads above
    // the switch on g, which held them live across it (187 VGPRs against 149).
    __asm__ volatile("" ::: "memory");
    const int ph = (int)((t_begin + tt0) & 7);
    // Software-pipelined by two steps: a step's LDS operands -- (e, dt2 x) of the
    // lane's channel and the wave's four B and C values -- are read two steps
    // before they are used.  Without the exponentials a step is only about
    // twenty VALU instructions, too short to cover an LDS read's latency.
    constexpr int PD = 2;
    float2 rv[PD + 1];
    float4 rb[PD + 1], rc[PD + 1];
    auto fetch = [&](int s, int slot) SSM_INLINE {
      rv[slot] = sh_dtv[s][loff];
      rb[slot] = *reinterpret_cast<const float4*>(&sh_B[s][g * NS]);
      if (!PASS_A) rc[slot] = *reinterpret_cast<const float4*>(&sh_C[PASS_A ? 0 : s][g * NS]);
    };
#pragma unroll
    for (int p = 0; p < PD; ++p)
      if (p < n) fetch(p, p);
#pragma unroll
    for (int s = 0; s < n; ++s) {
      if (s + PD < n) fetch(s + PD, (s + PD) % (PD + 1));
      if (ckpt_mode && ((ph + s) & 7) == 0) store_ckpt(tt0 + s);
      const int cur = s % (PD + 1);
      const float2 v = rv[cur];
      const float bv[4] = {rb[cur].x, rb[cur].y, rb[cur].z, rb[cur].w};
      const float cv[4] = {rc[cur].x, rc[cur].y, rc[cur].z, rc[cur].w};
      const float e = v.x;
      const float e2 = e * e;
      const float e4 = e2 * e2;
      float ap;
      if constexpr (GB == 0) ap = e;
      else if constexpr (GB == 1) ap = e2;
      else if constexpr (GB == 2) ap = e * e2;
      else ap = e4;
      float y = 0.0f;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (i > 0) ap = ap * e4;
        h[i] = __builtin_fmaf(ap, h[i], v.y * bv[i]);
        if (!PASS_A) y = __builtin_fmaf(cv[i], h[i], y);
      }
      if (!PASS_A) sh_y[PASS_A ? 0 : s][(PASS_A ? 0 : g) * kWave + lane] = y;
      // keep the prefetch distance: the scheduler would otherwise sink the
      // reads of step s + PD next to their use
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto run_steps_pow = [&](auto n_c, int64_t tt0) SSM_INLINE {
    if constexpr (std::is_same_v<decltype(n_c), int>) {
      run_steps_pow_plain(n_c, tt0);
    } else {
      switch (g) {   // wave-uniform
        case 0: run_steps_pow_piped(n_c, std::integral_constant<int, 0>(), tt0); break;
        case 1: run_steps_pow_piped(n_c, std::integral_constant<int, 1>(), tt0); break;
        case 2: run_steps_pow_piped(n_c, std::integral_constant<int, 2>(), tt0); break;
        default: run_steps_pow_piped(n_c, std::integral_constant<int, 3>(), tt0); break;
      }
    }
  };
  auto run_steps = [&](auto n_c, int64_t tt0) SSM_INLINE {
    if constexpr (kPow) {
      if (pow_mode) {
        run_steps_pow(n_c, tt0);
        return;
      }
    }
    const int n = n_c;
    const int ph = (int)((t_begin + tt0) & 7);
    float2 v = sh_dtv[0][loff];
    float ar[NS], rr[NR];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const float u2 = v.x * Ad[i];
      ar[i] = __builtin_amdgcn_exp2f(u2);
      if constexpr (ZOH) rr[i] = zoh_ratio(ar[i], u2);
    }
#pragma unroll
    for (int s = 0; s < n; ++s) {
      float2 vn = v;
      float an[NS], rn[NR];
      if (s + 1 < n) {
        vn = sh_dtv[s + 1][loff];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const float u2 = vn.x * Ad[i];
          an[i] = __builtin_amdgcn_exp2f(u2);
          if constexpr (ZOH) rn[i] = zoh_ratio(an[i], u2);
        }
      }
      if (ckpt_mode && ((ph + s) & 7) == 0) store_ckpt(tt0 + s);
      float y = 0.0f;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const float in = v.y * sh_B[s][g * NS + i];
        if constexpr (ZOH) h[i] = __builtin_fmaf(ar[i], h[i], rr[i] * in);
        else h[i] = __builtin_fmaf(ar[i], h[i], in);
        if (!PASS_A) y = __builtin_fmaf(sh_C[PASS_A ? 0 : s][g * NS + i], h[i], y);
      }
      if (PASS_A) {
        dtsum += v.x;
      } else {
        sh_y[PASS_A ? 0 : s][(PASS_A ? 0 : g) * kWave + lane] = y;
      }
      if (s + 1 < n) {
        v = vn;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          ar[i] = an[i];
          if constexpr (ZOH) rr[i] = rn[i];
        }
      }
    }
  };

  // Phase 3: finish this thread's items into registers: sum the partials in
  // a fixed order, D skip, gate.  The D switch is taken once per tile.
  float yv[IPT][CW];
  auto finish_items = [&](auto d_c) SSM_INLINE {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int r = irow[it];
#pragma unroll
      for (int q = 0; q < CW; ++q) {
        const int col = icol[it] + q;
        float acc = sh_y[PASS_A ? 0 : r][col];
#pragma unroll
        for (int gg = 1; gg < G; ++gg) acc += sh_y[PASS_A ? 0 : r][(PASS_A ? 0 : gg) * kWave + col];
        if (decltype(d_c)::value) acc = __builtin_fmaf(iD[it][q], xs[it][q], acc);
        if (kZ) acc = acc * silu_f(zs[it].get(q));
        yv[it][q] = acc;
      }
    }
  };
  auto finish = [&]() SSM_INLINE {
    if (has_D) finish_items(std::true_type());
    else finish_items(std::false_type());
  };
  // Store the finished tile that starts at chunk-relative step tt0.  Full
  // tiles store unconditionally; the peeled ragged tile (full == false)
  // skips rows past nt.
  auto store = [&](int64_t tt0, int nt, bool full) SSM_INLINE {
#pragma unroll
    for (int it = 0; it < IPT; ++it)
      if (full || irow[it] < nt) store_row<Tout, CW>(ob + (tt0 + irow[it]) * Dn + icol[it], yv[it]);
  };

  // A full tile, straight-line.  The outputs of the previous full tile
  // (at step prev0, when has_prev) are stored only after this tile's inputs
  // have been committed: the wait for those inputs then never includes the
  // acknowledgement of stores issued just before it.
  auto full_tile = [&](Bank& bk, int64_t tt0, int64_t pf0, auto has_prev_c, int64_t prev0) SSM_INLINE {
    commit(bk, T);
    if (!PASS_A && decltype(has_prev_c)::value) store(prev0, T, true);
    issue(bk, pf0, T);
    block_sync();
    run_steps(std::integral_constant<int, T>(), tt0);
    block_sync();
    if (!PASS_A) finish();
  };

  const int64_t nsteps = t_end - t_begin;
  const int tail = (int)(nsteps % T);          // the peeled ragged tile
  const int64_t nfull = nsteps / T;
  const int64_t last_full = tail + (nfull - 1) * T;   // start of the last full tile
  if (tail > 0) {
    issue(bk0, 0, tail);
    if (nfull > 0) issue(bk1, tail, T);
    commit(bk0, tail);
    if (nfull > 1) issue(bk0, tail + T, T);
    block_sync();
    run_steps(tail, 0);
    block_sync();
    if (!PASS_A) {
      finish();
      store(0, tail, false);
    }
  } else {
    if (nfull > 0) issue(bk1, 0, T);
    if (nfull > 1) issue(bk0, T, T);
  }
  // full tiles f = 0, 1, ...: tile f's inputs are in bk1 for even f and bk0
  // for odd f; each tile prefetches tile f + 2 into the bank it just used and
  // stores the outputs of tile f - 1
  if (nfull > 0) {
    full_tile(bk1, tail, min(tail + 2 * T, last_full), std::false_type(), 0);
    const ProgressPriority prio(nfull);
    int64_t f = 1;
    for (; f + 1 < nfull; f += 2) {
      const int64_t t0 = tail + f * T;
      if (a.fair) prio.at(f);
      full_tile(bk0, t0, min(t0 + 2 * T, last_full), std::true_type(), t0 - T);
      full_tile(bk1, t0 + T, min(t0 + 3 * T, last_full), std::true_type(), t0);
    }
    if (f < nfull) full_tile(bk0, tail + f * T, last_full, std::true_type(), tail + (f - 1) * T);
    if (!PASS_A) store(last_full, T, true);
  }

  if (PASS_A && !ckpt_mode) {
    float* dst = a.ws_state + (((int64_t)b * K + k) * Dn + dl) * kDState;
#pragma unroll
    for (int i = 0; i < NS; ++i) dst[st_of(i)] = h[i];
    if (kItemSum && pow_mode) {
      // the items' sums, one row of the tile's channels per thread row, in the
      // LDS of the last tile's (e, dt2 x), which the barrier after that tile's
      // recurrence has freed; each channel then sums its T rows in order
      float* red = reinterpret_cast<float*>(&sh_dtv[0][0]);  // [T][kWave]
#pragma unroll
      for (int it = 0; it < (kItemSum ? IPT : 1); ++it)
#pragma unroll
        for (int q = 0; q < (kItemSum ? CW : 1); ++q) red[irow[it] * kWave + icol[it] + q] = isum[it][q];
      block_sync();
      if (g == 0) {
        float sum = 0.0f;
        for (int r = 0; r < T; ++r) sum += red[r * kWave + loff];
        dtsum = sum;
      }
    }
    if (g == 0) a.ws_dtsum[((int64_t)b * K + k) * Dn + dl] = dtsum;
  } else if (!PASS_A && k == K - 1 && a.last_state != nullptr) {
    float* dst = a.last_state + ((int64_t)b * Dn + dl) * kDState;
#pragma unroll
    for (int i = 0; i < NS; ++i) dst[st_of(i)] = h[i];
  }
}


// Launch one pass; the progress-priority scheme (ProgressPriority) is turned
// on when the device holds the whole grid at once.
template <typename K>
void launch_pass(K kern, int per_cu, dim3 grid, int threads, const ScanArgs& a, hipStream_t s) {
  ScanArgs b = a;
  b.fair = grid_coresident(per_cu, a.cus, grid) ? 1 : 0;
  hipLaunchKernelGGL(kern, grid, dim3(threads), 0, s, b);
}

template <typename Tin, typename Tout, int NS, bool WIDE, bool ZOH>
hipError_t launch_scan_w(const ScanArgs& a, hipStream_t s) {
  constexpr int G = kDState / NS;
  constexpr int NTHR = kWave * G;
  const auto kA = scan_chunk_kernel<Tin, Tout, NS, true, false, WIDE, ZOH>;
  const auto kBz = scan_chunk_kernel<Tin, Tout, NS, false, true, WIDE, ZOH>;
  const auto kB = scan_chunk_kernel<Tin, Tout, NS, false, false, WIDE, ZOH>;
  static const int occA = resident_per_cu(kA, NTHR);
  static const int occBz = resident_per_cu(kBz, NTHR);
  static const int occB = resident_per_cu(kB, NTHR);
  const unsigned nblk = (unsigned)((a.d_inner + kWave - 1) / kWave);
  if (a.ckpt != nullptr) {
    if constexpr (NS == 4 && !ZOH) {
      if (a.ckpt_only) {  // the checkpoint pass over every chunk
        const auto kC = scan_chunk_kernel<Tin, Tout, NS, true, false, WIDE, ZOH, true>;
        static const int occC = resident_per_cu(kC, NTHR);
        launch_pass(kC, occC, dim3(nblk, (unsigned)a.n_chunks, (unsigned)a.batch), NTHR, a, s);
        return hipGetLastError();
      }
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (a.n_chunks > 1) {
    launch_pass(kA, occA, dim3(nblk, (unsigned)(a.n_chunks - 1), (unsigned)a.batch), NTHR, a, s);
    const hipError_t e = launch_carry(a, s);
    if (e != hipSuccess) return e;
  }
  if (a.states_only) return hipGetLastError();
  const dim3 gridB(nblk, (unsigned)a.n_chunks, (unsigned)a.batch);
  if constexpr (NS == 4 && !ZOH) {
    if (a.ckpt != nullptr) {  // pass B that also stores the checkpoints
      const auto kBzC = scan_chunk_kernel<Tin, Tout, NS, false, true, WIDE, ZOH, true>;
      const auto kBC = scan_chunk_kernel<Tin, Tout, NS, false, false, WIDE, ZOH, true>;
      static const int occBzC = resident_per_cu(kBzC, NTHR);
      static const int occBC = resident_per_cu(kBC, NTHR);
      if (a.z != nullptr) launch_pass(kBzC, occBzC, gridB, NTHR, a, s);
      else launch_pass(kBC, occBC, gridB, NTHR, a, s);
      return hipGetLastError();
    }
  }
  if (a.z != nullptr) launch_pass(kBz, occBz, gridB, NTHR, a, s);
  else launch_pass(kB, occB, gridB, NTHR, a, s);
  return hipGetLastError();
}

// The wide prologue/epilogue needs rows that split into aligned groups of 8.
template <typename Tin, typename Tout, int NS, bool ZOH>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s) {
  if (a.d_inner % 8 == 0) return launch_scan_w<Tin, Tout, NS, true, ZOH>(a, s);
  return launch_scan_w<Tin, Tout, NS, false, ZOH>(a, s);
}

template <typename Tin, typename Tout, bool ZOH>
hipError_t launch_scan_ns(const ScanArgs& a, int ns, hipStream_t s) {
  switch (ns) {
    case 1: return launch_scan_t<Tin, Tout, 1, ZOH>(a, s);
    case 2: return launch_scan_t<Tin, Tout, 2, ZOH>(a, s);
    case 4: return launch_scan_t<Tin, Tout, 4, ZOH>(a, s);
    case 8: return launch_scan_t<Tin, Tout, 8, ZOH>(a, s);
    case 16: return launch_scan_t<Tin, Tout, 16, ZOH>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace ssm

#endif  // SSMSCAN_SCAN_KERNEL_H

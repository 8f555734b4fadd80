// gfx950 kernels of libssmscan: chunked selective scan, affine-pair carry
// pass, decode state update.
//
// What is computed (pages: "Mamba и State Space Models", nareshka.ru,
// "Ключевая инновация" and "Selective Scan (core algorithm)"; "State Space
// Models: Mamba и альтернатива Transformer", johe.ru, "_scan" for the D skip
// and "Параллельная форма" for the prefix form; "Модуль 8. Альтернативы
// Transformer", vladkulikov.com, section 7 for the affine-pair operator):
//   dt = softplus(delta + bias);  h[n] <- exp(dt A[d,n]) h[n] + dt B_t[n] x
//   out = (sum_n C_t[n] h[n] + D x) * silu(z)
//
// Work decomposition (MI355X-first; see the design notes in the repository):
//  * A workgroup owns 64 consecutive channels of one batch row and one time
//    chunk.  Its G = 16 / NS wavefronts each carry NS of the 16 states of all
//    64 channels (lane = channel), so B_t[n] and C_t[n] are the same for every
//    lane of a wave and are read as LDS broadcasts; the fp32 state lives in
//    VGPRs for the whole chunk and never touches HBM mid-sequence.
//  * Time is processed in tiles of T steps.  Phase 1: each wave converts and
//    discretises T/G of the tile's steps (softplus, dt*x) into LDS, and the
//    workgroup stages the tile's B/C rows in LDS as fp32.  Phase 2: every wave
//    runs the recurrence over the whole tile for its states and leaves a
//    partial readout per step in LDS.  Phase 3: each wave finishes T/G steps
//    (sum of the partials in a fixed order, D skip, SiLU gate, store).  The
//    HBM loads of the tile after next are issued before phase 2, so two tiles
//    of reads are in flight behind the arithmetic.
//  * Long sequences are cut into chunks.  Pass A reduces every chunk but the
//    last to its affine pair per state coordinate: the end state from zero and
//    the step-size sum S (the chunk's decay is exp(A S)).  The carry kernel
//    scans the pairs in time order with a wavefront DPP scan (lane = chunk).
//    Pass B re-runs each chunk from its incoming state with the full readout.
#include <type_traits>

#include "internal.h"

namespace ssm {
namespace {

// Every lambda of a kernel body must be inlined: an outlined call would pass
// the state and the register banks through scratch memory.
#define SSM_INLINE __attribute__((always_inline))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// ---------------------------------------------------------------- element io

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// fp32 -> bfloat16, round to nearest even: gfx950's v_cvt_pk_bf16_f32, which
// converts two values per instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two values rounded and packed, the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T>
struct Io;

template <>
struct Io<float> {
  using raw = float;
  static __device__ __forceinline__ raw load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ float cvt(raw r) { return r; }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};

template <>
struct Io<uint16_t> {  // bfloat16 bit patterns
  using raw = uint16_t;
  static __device__ __forceinline__ raw load(const void* p, int64_t i) {
    return static_cast<const uint16_t*>(p)[i];
  }
  static __device__ __forceinline__ float cvt(raw r) { return bf16_to_f32(r); }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16_rne(v);
  }
};

// Unpack a 16-byte vector of B/C elements into fp32.
template <typename T>
struct Vec16;

template <>
struct Vec16<float> {
  static constexpr int kElems = 4;
  static __device__ __forceinline__ void unpack(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
  }
};

template <>
struct Vec16<uint16_t> {
  static constexpr int kElems = 8;
  static __device__ __forceinline__ void unpack(const uint4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// ------------------------------------------------------- pointwise functions

// softplus(u) = log(1 + e^u) = max(u, 0) + log1p(e), e = exp(-|u|) in (0, 1].
// log1p(e) is log(w) plus the rounding error c of w = 1 + e (c is exact,
// |c| <= 2^-24), which keeps the result accurate to a few ulp also when e is
// tiny and w rounds to 1.
__device__ __forceinline__ float softplus_f(float u) {
  const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(u) * kLog2e);
  const float w = 1.0f + e;
  const float c = e - (w - 1.0f);
  const float l = __builtin_amdgcn_logf(w);  // log2(w)
  return __builtin_fmaxf(u, 0.0f) + __builtin_fmaf(l, kLn2, c);
}

// The same in log2 units: softplus(u) * log2(e) from a = u * log2(e),
// = max(a, 0) + log2(1 + 2^-|a|), with the rounding error c of w = 1 + 2^-|a|
// added back as c * log2(e).  The scan works with step sizes in these units:
// exp(dt A) = exp2(dt2 A) with dt2 = dt log2(e).
__device__ __forceinline__ float softplus2_f(float a) {
  const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(a));
  const float w = 1.0f + e;
  const float c = e - (w - 1.0f);
  const float l = __builtin_amdgcn_logf(w);  // log2(w)
  return __builtin_fmaxf(a, 0.0f) + __builtin_fmaf(c, kLog2e, l);
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^{-z}).
__device__ __forceinline__ float silu_f(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * kLog2e);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// ------------------------------------------------ wavefront affine-pair scan

#define SSM_DPP(old, src, ctrl, rmask)                                                    \
  __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), \
                                             (ctrl), (rmask), 0xf, false))

// Inclusive scan over the 64 lanes of a wavefront of affine pairs (a, b),
// lane order = time order: lane i ends with pair_i o pair_{i-1} o ... o pair_0,
// where (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2).  Hillis-Steele within each
// 16-lane row (row_shr 1, 2, 4, 8), then row_bcast:15 and row_bcast:31 join
// the rows.  Lanes without a predecessor receive the identity (1, 0).  All 64
// lanes must be active.
__device__ __forceinline__ void affine_wave_scan(float& a, float& b) {
#define SSM_SCAN_STEP(ctrl, rmask)                 \
  {                                                \
    const float pa = SSM_DPP(1.0f, a, ctrl, rmask); \
    const float pb = SSM_DPP(0.0f, b, ctrl, rmask); \
    b = __builtin_fmaf(a, pb, b);                  \
    a = a * pa;                                    \
  }
  SSM_SCAN_STEP(0x111, 0xf)  // row_shr:1
  SSM_SCAN_STEP(0x112, 0xf)  // row_shr:2
  SSM_SCAN_STEP(0x114, 0xf)  // row_shr:4
  SSM_SCAN_STEP(0x118, 0xf)  // row_shr:8
  SSM_SCAN_STEP(0x142, 0xa)  // row_bcast:15 into rows 1 and 3
  SSM_SCAN_STEP(0x143, 0xc)  // row_bcast:31 into rows 2 and 3
#undef SSM_SCAN_STEP
}

// Workgroup barrier pinned in the instruction schedule.  __syncthreads()
// alone has been seen to let the machine scheduler hoist the s_barrier above
// the LDS reads that precede it (the IR order was correct), which let fast
// waves overwrite tile inputs that slower waves were still reading; the
// scheduling fences on both sides keep every LDS access on its side.
__device__ __forceinline__ void block_sync() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// ------------------------------------------------------------- scan kernel

template <int G>
struct Tile {
  static constexpr int T = (G == 1 || G >= 8) ? 16 : 32;  // steps per tile
  // channels per prologue/epilogue item on the wide path (8 x bf16 = 16 B)
  static constexpr int CW = (T / G) < 8 ? (T / G) : 8;
};

// CW contiguous input elements of one row, as raw 32-bit words.
template <typename Tin, int CW>
struct Raw {
  static constexpr int kBytes = CW * (int)sizeof(Tin);
  static constexpr int kWords = kBytes >= 4 ? kBytes / 4 : 1;
  uint32_t w[kWords];
  __device__ __forceinline__ void load(const Tin* p) {
    if constexpr (kBytes == 2) {
      w[0] = *reinterpret_cast<const uint16_t*>(p);
    } else if constexpr (kBytes == 4) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else if constexpr (kBytes == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x;
      w[1] = v.y;
    } else {
#pragma unroll
      for (int q = 0; q < kBytes / 16; ++q) {
        const uint4 v = reinterpret_cast<const uint4*>(p)[q];
        w[4 * q] = v.x;
        w[4 * q + 1] = v.y;
        w[4 * q + 2] = v.z;
        w[4 * q + 3] = v.w;
      }
    }
  }
  __device__ __forceinline__ float get(int k) const {
    if constexpr (sizeof(Tin) == 4) {
      return __uint_as_float(w[k]);
    } else {
      const uint32_t word = w[k >> 1];
      return (k & 1) ? __uint_as_float(word & 0xffff0000u) : __uint_as_float(word << 16);
    }
  }
};

// Store CW contiguous outputs of one row.
template <typename Tout, int CW>
__device__ __forceinline__ void store_row(Tout* p, const float* v) {
  if constexpr (sizeof(Tout) == 4) {
    if constexpr (CW % 4 == 0) {
#pragma unroll
      for (int q = 0; q < CW / 4; ++q)
        reinterpret_cast<float4*>(p)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    } else if constexpr (CW == 2) {
      *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    } else {
      p[0] = v[0];
    }
  } else {
    if constexpr (CW == 1) {
      p[0] = f32_to_bf16_rne(v[0]);
    } else {
      uint32_t w[CW / 2];
#pragma unroll
      for (int q = 0; q < CW / 2; ++q)
        w[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
      if constexpr (CW % 8 == 0) {
#pragma unroll
        for (int q = 0; q < CW / 8; ++q)
          reinterpret_cast<uint4*>(p)[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
      } else if constexpr (CW == 4) {
        *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
      } else {
        *reinterpret_cast<uint32_t*>(p) = w[0];
      }
    }
  }
}

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
template <typename Tin, typename Tout, int NS, bool PASS_A, bool HAS_Z, bool WIDE>
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

  float Ad[NS];  // this lane's A[d, n]; step sizes are in log2 units (dt2)
#pragma unroll
  for (int i = 0; i < NS; ++i) Ad[i] = a.A[dl * kDState + g * NS + i];

  // phases 1 and 3: this thread's items (row, first channel), fixed for the kernel
  int irow[IPT], icol[IPT];
  float ibias[IPT][CW], iD[IPT][CW];  // bias in log2 units, D
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
    }
  }

  float h[NS];
  if (!PASS_A && k > 0) {
    const float* src = a.ws_state + (((int64_t)b * K + (k - 1)) * Dn + dl) * kDState + g * NS;
#pragma unroll
    for (int i = 0; i < NS; ++i) h[i] = src[i];
  } else if (k == 0 && a.h0 != nullptr) {  // continuing from a stored state
    const float* src = a.h0 + ((int64_t)b * Dn + dl) * kDState + g * NS;
#pragma unroll
    for (int i = 0; i < NS; ++i) h[i] = src[i];
  } else {
#pragma unroll
    for (int i = 0; i < NS; ++i) h[i] = 0.0f;
  }
  float dtsum = 0.0f;

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
  auto discretise = [&](Bank& bk, auto sp_c) SSM_INLINE {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
#pragma unroll
      for (int q = 0; q < CW; ++q) {
        const float x = bk.rx[it].get(q);
        const float u2 = __builtin_fmaf(bk.rdt[it].get(q), kLog2e, ibias[it][q]);
        const float dt2 = decltype(sp_c)::value ? softplus2_f(u2) : u2;
        sh_dtv[irow[it]][icol[it] + q] = make_float2(dt2, dt2 * x);
        xs[it][q] = x;
      }
    }
  };
  auto commit = [&](Bank& bk) SSM_INLINE {
    if (softplus) discretise(bk, std::true_type());
    else discretise(bk, std::false_type());
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
      float* dst = which ? &sh_C[PASS_A ? 0 : row][part * EPV] : &sh_B[row][part * EPV];
      const float scale = which ? 1.0f : kLn2;  // B carries the ln 2 of dt2 * x
#pragma unroll
      for (int i = 0; i < EPV; ++i) dst[i] = f[i] * scale;
    }
  };

  // Phase 2: the recurrence for this wave's NS states over steps [0, n).
  // Software-pipelined by one step: the transitions exp(dt * A) of step s + 1
  // do not depend on the state, so they are computed while step s updates it,
  // which keeps each exp's latency off the h dependency chain.
  auto run_steps = [&](auto n_c) SSM_INLINE {
    const int n = n_c;
    float2 v = sh_dtv[0][loff];
    float ar[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) ar[i] = __builtin_amdgcn_exp2f(v.x * Ad[i]);
#pragma unroll
    for (int s = 0; s < n; ++s) {
      float2 vn = v;
      float an[NS];
      if (s + 1 < n) {
        vn = sh_dtv[s + 1][loff];
#pragma unroll
        for (int i = 0; i < NS; ++i) an[i] = __builtin_amdgcn_exp2f(vn.x * Ad[i]);
      }
      float y = 0.0f;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        h[i] = __builtin_fmaf(ar[i], h[i], v.y * sh_B[s][g * NS + i]);
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
        for (int i = 0; i < NS; ++i) ar[i] = an[i];
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
    commit(bk);
    if (!PASS_A && decltype(has_prev_c)::value) store(prev0, T, true);
    issue(bk, pf0, T);
    block_sync();
    run_steps(std::integral_constant<int, T>());
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
    commit(bk0);
    if (nfull > 1) issue(bk0, tail + T, T);
    block_sync();
    run_steps(tail);
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
    int64_t f = 1;
    for (; f + 1 < nfull; f += 2) {
      const int64_t t0 = tail + f * T;
      full_tile(bk0, t0, min(t0 + 2 * T, last_full), std::true_type(), t0 - T);
      full_tile(bk1, t0 + T, min(t0 + 3 * T, last_full), std::true_type(), t0);
    }
    if (f < nfull) full_tile(bk0, tail + f * T, last_full, std::true_type(), tail + (f - 1) * T);
    if (!PASS_A) store(last_full, T, true);
  }

  if (PASS_A) {
    float* dst = a.ws_state + (((int64_t)b * K + k) * Dn + dl) * kDState + g * NS;
#pragma unroll
    for (int i = 0; i < NS; ++i) dst[i] = h[i];
    if (g == 0) a.ws_dtsum[((int64_t)b * K + k) * Dn + dl] = dtsum;
  } else if (k == K - 1 && a.last_state != nullptr) {
    float* dst = a.last_state + ((int64_t)b * Dn + dl) * kDState + g * NS;
#pragma unroll
    for (int i = 0; i < NS; ++i) dst[i] = h[i];
  }
}

// ------------------------------------------------------------ carry kernel
//
// On entry, slot p < K-1 of ws_state holds chunk p's end state from zero
// and ws_dtsum its step-size sum S_p in log2 units (the scan kernel's dt2);
// the pair of chunk p for coordinate (d, n) is (exp2(A[d,n] S_p), end state).  On exit slot p holds the state
// entering chunk p + 1: the inclusive composition of pairs 0..p applied to
// h = 0.  A workgroup takes 64 consecutive (d, n) columns; pairs are loaded
// 64 at a time (coalesced along columns) into LDS, each wave scans 16
// columns with lane = chunk, and a per-column carry joins the segments.
__global__ void __launch_bounds__(256) carry_kernel(float* ws_state, const float* ws_dtsum,
                                                    const float* A, int64_t Dn, int K) {
  __shared__ float sa[64][65];
  __shared__ float sb[64][65];
  __shared__ float ca[64];
  __shared__ float cb[64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int b = blockIdx.y;
  const int64_t ncol = Dn * kDState;
  const int64_t col = (int64_t)blockIdx.x * 64 + lane;
  const int npairs = K - 1;
  const float a2 = col < ncol ? A[col] : 0.0f;  // S is a sum of log2-unit step sizes
  if (tid < 64) {
    ca[tid] = 1.0f;
    cb[tid] = 0.0f;
  }
  for (int p0 = 0; p0 < npairs; p0 += 64) {
    const int np = min(64, npairs - p0);
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int r = w + 4 * i;
      float av = 1.0f, bv = 0.0f;
      if (r < np && col < ncol) {
        const int64_t p = (int64_t)b * K + p0 + r;
        bv = ws_state[p * ncol + col];
        const float S = ws_dtsum[p * Dn + (col >> 4)];
        av = __builtin_amdgcn_exp2f(S * a2);
      }
      sa[r][lane] = av;
      sb[r][lane] = bv;
    }
    block_sync();
    for (int j = 0; j < 16; ++j) {
      const int c = w + 4 * j;
      float av = sa[lane][c];
      float bv = sb[lane][c];
      affine_wave_scan(av, bv);
      const float cav = ca[c];
      const float cbv = cb[c];
      const float rb = __builtin_fmaf(av, cbv, bv);  // (av, bv) o carry
      const float ra = av * cav;
      sb[lane][c] = rb;
      const float na = readlane_f(ra, 63);
      const float nb = readlane_f(rb, 63);
      if (lane == 0) {
        ca[c] = na;
        cb[c] = nb;
      }
    }
    block_sync();
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int r = w + 4 * i;
      if (r < np && col < ncol) ws_state[((int64_t)b * K + p0 + r) * ncol + col] = sb[r][lane];
    }
    block_sync();
  }
}

// Exclusive affine-pair scan of one array (one wavefront; the combine of the
// carry kernel, exposed for tests).
__global__ void __launch_bounds__(64) affine_exclusive_scan_kernel(const float* a, const float* b,
                                                                   float* oa, float* ob, int64_t n) {
  const int lane = threadIdx.x;
  float ca = 1.0f, cb = 0.0f;
  for (int64_t s0 = 0; s0 < n; s0 += 64) {
    const int64_t i = s0 + lane;
    float av = i < n ? a[i] : 1.0f;
    float bv = i < n ? b[i] : 0.0f;
    affine_wave_scan(av, bv);
    const float ia = av * ca;
    const float ib = __builtin_fmaf(av, cb, bv);
    const float ea = SSM_DPP(ca, ia, 0x138, 0xf);  // wave_shr:1, lane 0 keeps the carry
    const float eb = SSM_DPP(cb, ib, 0x138, 0xf);
    if (i < n) {
      oa[i] = ea;
      ob[i] = eb;
    }
    ca = readlane_f(ia, 63);
    cb = readlane_f(ib, 63);
  }
}

// ----------------------------------------------------------- decode kernel
//
// One (b, d) pair per quad of lanes; lane q of the quad owns states 4q..4q+3
// (one 16-byte load and store of the fp32 state).  The readout is reduced
// over the quad with two DPP quad permutes; lane 0 of the quad applies the
// D skip and the gate and stores out.  The per-step inputs are read with
// non-temporal loads and out is stored non-temporally: they are touched once,
// and keeping them out of the caches leaves room for the state, which every
// step reads and writes again.
template <typename Tin>
__device__ __forceinline__ float nt_load(const void* p, int64_t i) {
  if constexpr (sizeof(Tin) == 4) {
    return __builtin_nontemporal_load(static_cast<const float*>(p) + i);
  } else {
    return bf16_to_f32(__builtin_nontemporal_load(static_cast<const uint16_t*>(p) + i));
  }
}

template <typename Tin>
__device__ __forceinline__ void load4(const void* p, int64_t i, float* o) {
  if constexpr (sizeof(Tin) == 4) {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xffff0000u);
  }
}

template <typename Tin, typename Tout>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e = gid >> 2;
  const int q = threadIdx.x & 3;
  if (e >= a.pairs) return;  // whole quads leave together
  const int64_t d = e % a.d_inner;
  const int64_t b = e / a.d_inner;

  float4 hs = *reinterpret_cast<const float4*>(a.state + e * kDState + 4 * q);
  const float4 av = *reinterpret_cast<const float4*>(a.A + d * kDState + 4 * q);
  float Bv[4], Cv[4];
  load4<Tin>(a.B, b * kDState + 4 * q, Bv);
  load4<Tin>(a.C, b * kDState + 4 * q, Cv);
  const float x = nt_load<Tin>(a.x, e);
  const float dl = nt_load<Tin>(a.delta, e);
  const float u = dl + (a.bias != nullptr ? a.bias[d] : 0.0f);
  const float dt = a.softplus ? softplus_f(u) : u;
  const float dtx = dt * x;
  float h[4] = {hs.x, hs.y, hs.z, hs.w};
  const float A2[4] = {av.x * kLog2e, av.y * kLog2e, av.z * kLog2e, av.w * kLog2e};
  float y = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float ar = __builtin_amdgcn_exp2f(dt * A2[i]);
    h[i] = __builtin_fmaf(ar, h[i], dtx * Bv[i]);
    y = __builtin_fmaf(Cv[i], h[i], y);
  }
  *reinterpret_cast<float4*>(a.state + e * kDState + 4 * q) = make_float4(h[0], h[1], h[2], h[3]);
  // quad sum in a fixed order: (q0 + q1) + (q2 + q3) on every lane
  y = y + SSM_DPP(0.0f, y, 0xB1, 0xf);  // quad_perm [1,0,3,2]
  y = y + SSM_DPP(0.0f, y, 0x4E, 0xf);  // quad_perm [2,3,0,1]
  if (q == 0) {
    if (a.D != nullptr) y = __builtin_fmaf(a.D[d], x, y);
    if (a.z != nullptr) y = y * silu_f(nt_load<Tin>(a.z, e));
    if constexpr (sizeof(Tout) == 4) {
      __builtin_nontemporal_store(y, static_cast<float*>(a.out) + e);
    } else {
      __builtin_nontemporal_store(f32_to_bf16_rne(y), static_cast<uint16_t*>(a.out) + e);
    }
  }
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

__global__ void copy_f32_kernel(float* dst, const float* src, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// ----------------------------------------------------------- conv1d kernels
//
// The block's causal depthwise convolution ("Mamba и State Space Models",
// nareshka.ru, "Реализация MambaBlock": Conv1d with one width-K filter per
// channel, padding K - 1, cut to the sequence; johe.ru's MambaBlock applies
// SiLU after it):
//   out[b,t,d] = act(bias[d] + sum_{k<K} w[d,k] * x[b, t-K+1+k, d])
// Inputs before t = 0 come from the cache [batch, d_inner, K] (the K most
// recent earlier inputs, oldest first; "Модуль 8", vladkulikov.com, sections
// 6 and 14), or are zero.
//
// Bandwidth-bound: each thread keeps a K-deep window of CW consecutive
// channels in registers and slides it over a run of steps, so every input is
// read once (plus K - 1 steps of overlap per run) and every output written
// once, with 16-byte accesses when d_inner allows.

template <typename Tin>
__device__ __forceinline__ float ld_in(const Tin* p) {
  if constexpr (sizeof(Tin) == 4) return *reinterpret_cast<const float*>(p);
  else return bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
}

template <typename Tin>
__device__ __forceinline__ void st_in(Tin* p, float v) {
  if constexpr (sizeof(Tin) == 4) *reinterpret_cast<float*>(p) = v;
  else *reinterpret_cast<uint16_t*>(p) = f32_to_bf16_rne(v);  // exact: v came from a Tin
}

// Steps per thread: a multiple of 8, chosen on the host (conv_run_len).

// Grid: x = blocks of 64 channel groups (one wavefront), y = runs (strided),
// z = batch row, so the run (and with it every load and store condition) is
// uniform across the wavefront.
template <typename Tin, typename Tout, int K, int CW, bool SILU>
__global__ void __launch_bounds__(64) conv1d_kernel(ConvArgs a, int64_t groups, int64_t runs, int run_len) {
  using R = Raw<Tin, CW>;
  const int64_t cg = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (cg >= groups) return;
  const int64_t b = blockIdx.z;
  const int64_t Dn = a.d_inner, L = a.seqlen;
  const int64_t d0 = cg * CW;
  const Tin* xb = static_cast<const Tin*>(a.x) + b * L * Dn + d0;
  Tout* ob = static_cast<Tout*>(a.out) + b * L * Dn + d0;

  float w[CW][K], bias[CW];
#pragma unroll
  for (int q = 0; q < CW; ++q) {
#pragma unroll
    for (int k = 0; k < K; ++k) w[q][k] = a.w[(d0 + q) * K + k];
    bias[q] = a.bias != nullptr ? a.bias[d0 + q] : 0.0f;
  }
  // one output step: shift x in, filter, activation
  auto step = [&](float (&win)[K][CW], const R& xr, float* y) SSM_INLINE {
#pragma unroll
    for (int q = 0; q < CW; ++q) {
#pragma unroll
      for (int k = 0; k + 1 < K; ++k) win[k][q] = win[k + 1][q];
      win[K - 1][q] = xr.get(q);
      float acc = bias[q];
#pragma unroll
      for (int k = 0; k < K; ++k) acc = __builtin_fmaf(w[q][k], win[k][q], acc);
      y[q] = SILU ? acc * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-acc * kLog2e)) : acc;
    }
  };

  for (int64_t r = blockIdx.y; r < runs; r += gridDim.y) {
    const int64_t t0 = r * run_len;
    const int nt = (int)min((int64_t)run_len, L - t0);
    // win[k] holds the input at time t - K + 1 + k once step t is shifted in;
    // before the first step, win[1..K-1] hold times t0 - K + 1 .. t0 - 1
    float win[K][CW];
#pragma unroll
    for (int k = 1; k < K; ++k) {
      const int64_t tau = t0 - K + k;
      if (tau >= 0) {
        R v;
        v.load(xb + tau * Dn);
#pragma unroll
        for (int q = 0; q < CW; ++q) win[k][q] = v.get(q);
      } else {
#pragma unroll
        for (int q = 0; q < CW; ++q)
          win[k][q] = a.state_in != nullptr
                          ? ld_in(static_cast<const Tin*>(a.state_in) + ((b * Dn + d0 + q) * K + (tau + K)))
                          : 0.0f;
      }
    }
    if (nt == run_len) {
      // full run: blocks of 8 steps, all loads unconditional; the loads of the
      // next block are issued before the current block is computed (the last
      // block re-reads its own rows instead of reading past the run)
      R xa[8], xn[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xa[j].load(xb + (t0 + j) * Dn);
#pragma unroll 1
      for (int j0 = 0; j0 < run_len; j0 += 8) {
        const int64_t tn = t0 + min(j0 + 8, run_len - 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) xn[j].load(xb + (tn + j) * Dn);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float y[CW];
          step(win, xa[j], y);
          store_row<Tout, CW>(ob + (t0 + j0 + j) * Dn, y);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) xa[j] = xn[j];
      }
    } else {
      for (int j = 0; j < nt; ++j) {
        R xr;
        xr.load(xb + (t0 + j) * Dn);
        float y[CW];
        step(win, xr, y);
        store_row<Tout, CW>(ob + (t0 + j) * Dn, y);
      }
    }
  }
}

// The cache after a prefill: the K most recent inputs of each (b, d), taken
// from x, or from the incoming cache for steps before the sequence.  One
// thread per (b, d) reads all K values before writing any, so the outgoing
// cache may be the incoming one.
template <typename Tin, int K>
__global__ void __launch_bounds__(256) conv1d_state_kernel(ConvArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t Dn = a.d_inner, L = a.seqlen;
  if (i >= (int64_t)a.batch * Dn) return;
  const int64_t b = i / Dn, d = i % Dn;
  const Tin* xs = static_cast<const Tin*>(a.x);
  const Tin* si = static_cast<const Tin*>(a.state_in);
  float v[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t tau = L - K + k;
    v[k] = tau >= 0 ? ld_in(xs + (b * L + tau) * Dn + d) : (si != nullptr ? ld_in(si + i * K + (tau + K)) : 0.0f);
  }
  Tin* so = static_cast<Tin*>(a.state_out) + i * K;
#pragma unroll
  for (int k = 0; k < K; ++k) st_in(so + k, v[k]);
}

// One decode step: the cache [batch, d_inner, K] drops its oldest input and
// appends x [batch, d_inner]; out is the filter applied to the new cache.  A
// thread takes CW consecutive channels: their caches are one contiguous run
// of CW * K inputs, read and written with 16-byte accesses when CW > 1.
template <typename Tin, typename Tout, int K, int CW, bool SILU>
__global__ void __launch_bounds__(256) conv1d_update_kernel(ConvArgs a, int64_t nthreads) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= nthreads) return;
  const int64_t i0 = gid * CW;  // flat (b, d) of the first channel
  const int64_t d0 = i0 % a.d_inner;
  Tin* cache = static_cast<Tin*>(a.state_out) + i0 * K;
  const Tin* xp = static_cast<const Tin*>(a.x) + i0;
  constexpr int kCacheBytes = CW * K * (int)sizeof(Tin);
  constexpr bool kVec = kCacheBytes == 4 || kCacheBytes == 8 || kCacheBytes % 16 == 0;
  float sv[CW * K], xv[CW];
  if constexpr (!kVec) {  // element-wise: the cache run is not a vector width
#pragma unroll
    for (int k = 0; k < K; ++k) sv[k] = ld_in(cache + k);
    xv[0] = ld_in(xp);
  } else {
    Raw<Tin, CW * K> st;
    st.load(cache);
    Raw<Tin, CW> xr;
    xr.load(xp);
#pragma unroll
    for (int j = 0; j < CW * K; ++j) sv[j] = st.get(j);
#pragma unroll
    for (int q = 0; q < CW; ++q) xv[q] = xr.get(q);
  }
  float nv[CW * K], y[CW];
#pragma unroll
  for (int q = 0; q < CW; ++q) {
#pragma unroll
    for (int k = 0; k + 1 < K; ++k) nv[q * K + k] = sv[q * K + k + 1];
    nv[q * K + K - 1] = xv[q];
    float acc = a.bias != nullptr ? a.bias[d0 + q] : 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) acc = __builtin_fmaf(a.w[(d0 + q) * K + k], nv[q * K + k], acc);
    y[q] = SILU ? acc * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-acc * kLog2e)) : acc;
  }
  // exact: every cached value came from a Tin
  if constexpr (!kVec) {
#pragma unroll
    for (int k = 0; k < K; ++k) st_in(cache + k, nv[k]);
  } else {
    store_row<Tin, CW * K>(cache, nv);
  }
  store_row<Tout, CW>(static_cast<Tout*>(a.out) + i0, y);
}

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
// incoming state in registers), then runs the reverse recurrence.  Sums over a
// channel's 16 states go through LDS partials, summed in a fixed order; dB and
// dC are reduced over the wavefront's 64 channels through a wave-local LDS
// transpose and 3 DPP steps, and stored per channel block for a second,
// fixed-order reduction kernel: the result does not depend on timing.

template <typename Tin, typename Tg, bool HAS_Z, int CW>
__global__ void __launch_bounds__(256) scan_bwd_kernel(BwdArgs a) {
  constexpr int NS = 4, G = 4, T = kBwdTile, NTHR = 256;
  constexpr int CPR = kWave / CW;
  constexpr int IPT = T * CPR / NTHR;
  static_assert(IPT >= 1 && IPT * NTHR == T * CPR, "tile does not split evenly");
  using R = Raw<Tin, CW>;
  using RG = Raw<Tg, CW>;
  constexpr int RS = kWave + 4;  // staging row stride (16-byte aligned rows)

  __shared__ float2 sh_dtu[T][kWave + 1];      // (dt2, u2)
  __shared__ float sh_dy[T][kWave + 1];
  __shared__ float sh_B[T][kDState];           // B ln 2
  __shared__ float sh_C[T][kDState];
  __shared__ float sh_y[T][G * kWave + 1];     // forward readout partials
  __shared__ float sh_s1[T][G * kWave + 1];    // partial dh . B'
  __shared__ float sh_s2[T][G * kWave + 1];    // partial sum dh A a h_{t-1}
  __shared__ float sh_red[G][kWave * 9];        // per-lane dB', dC contributions, stride 9
  __shared__ float sh_bc[T][2][kDState];       // the tile's dB', dC of this block

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int g = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int64_t b = blockIdx.y;
  const int blk = blockIdx.x;
  const int64_t Dn = a.d_inner, L = a.seqlen;
  const int64_t d0 = (int64_t)blk * kWave;
  const int nvalid = (int)min((int64_t)kWave, Dn - d0);
  const int loff = min(lane, nvalid - 1);
  const int64_t dl = d0 + loff;
  const bool softplus = a.softplus != 0;
  const int64_t ntiles = (L + T - 1) / T;

  float Ad[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) Ad[i] = a.A[dl * kDState + g * NS + i];

  int irow[IPT], icol[IPT];
  float ibias[IPT][CW], ibias2[IPT][CW], iD[IPT][CW];
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int idx = tid + it * NTHR;
    irow[it] = idx / CPR;
    icol[it] = min(idx % CPR, (nvalid + CW - 1) / CW - 1) * CW;
#pragma unroll
    for (int q = 0; q < CW; ++q) {
      const int64_t dq = d0 + min(icol[it] + q, nvalid - 1);
      ibias[it][q] = a.bias != nullptr ? a.bias[dq] : 0.0f;
      ibias2[it][q] = ibias[it][q] * kLog2e;
      iD[it][q] = a.D != nullptr ? a.D[dq] : 0.0f;
    }
  }
  const int64_t row0 = b * L * Dn + d0;
  const Tin* xb = static_cast<const Tin*>(a.x) + row0;
  const Tin* db = static_cast<const Tin*>(a.delta) + row0;
  const Tin* zb = HAS_Z ? static_cast<const Tin*>(a.z) + row0 : nullptr;
  const Tg* gb = static_cast<const Tg*>(a.dout) + row0;
  const Tin* Bb = static_cast<const Tin*>(a.B) + b * L * kDState;
  const Tin* Cb = static_cast<const Tin*>(a.C) + b * L * kDState;
  float* ck = a.ws_ckpt + ((b * a.nblk + blk) * ntiles) * (int64_t)(kWave * kDState);

  // Raw inputs of one tile, loaded one tile ahead of their use (rows past
  // the tile's end repeat its last row, so every load is unconditional).
  struct Bank {
    R rx[IPT], rd[IPT], rz[IPT];
    RG rg[IPT];
    float bv, cv;   // this thread's B, C element (256 threads = 16 rows x 16 states)
  };
  auto tile_rows = [&](int64_t k) SSM_INLINE { return (int)min((int64_t)T, L - k * T); };
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
    const int64_t t = t0 + min(tid / kDState, nt - 1);
    bk.bv = ld_in(Bb + t * kDState + tid % kDState);
    if (full) bk.cv = ld_in(Cb + t * kDState + tid % kDState);
  };
  auto stage_bc = [&](const Bank& bk, bool with_c) SSM_INLINE {
    const int r = tid / kDState, n = tid % kDState;
    sh_B[r][n] = bk.bv * kLn2;
    if (with_c) sh_C[r][n] = bk.cv;
  };

  // ---- phase 1: forward, storing the state entering each tile
  float h[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) h[i] = a.h0 != nullptr ? a.h0[(b * Dn + dl) * kDState + g * NS + i] : 0.0f;
  Bank cur, nxt;
  load(cur, 0, false);
  for (int64_t k = 0; k < ntiles; ++k) {
    const int nt = tile_rows(k);
    *reinterpret_cast<float4*>(ck + (k * kWave + lane) * kDState + g * NS) = make_float4(h[0], h[1], h[2], h[3]);
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
#pragma unroll
      for (int q = 0; q < CW; ++q) {
        const float u2 = __builtin_fmaf(cur.rd[it].get(q), kLog2e, ibias2[it][q]);
        const float dt2 = softplus ? softplus2_f(u2) : u2;
        sh_dtu[irow[it]][icol[it] + q] = make_float2(dt2, dt2 * cur.rx[it].get(q));
      }
    }
    stage_bc(cur, false);
    if (k + 1 < ntiles) load(nxt, k + 1, false);
    block_sync();
    for (int s = 0; s < nt; ++s) {
      const float2 v = sh_dtu[s][loff];
#pragma unroll
      for (int i = 0; i < NS; ++i)
        h[i] = __builtin_fmaf(__builtin_amdgcn_exp2f(v.x * Ad[i]), h[i], v.y * sh_B[s][g * NS + i]);
    }
    block_sync();
    cur = nxt;
  }

  // ---- phase 2: the tiles in reverse
  float carry[NS], dAacc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    carry[i] = a.dlast != nullptr ? a.dlast[(b * Dn + dl) * kDState + g * NS + i] : 0.0f;
    dAacc[i] = 0.0f;
  }
  float dDacc[IPT][CW], dBacc[IPT][CW];
#pragma unroll
  for (int it = 0; it < IPT; ++it)
#pragma unroll
    for (int q = 0; q < CW; ++q) dDacc[it][q] = dBacc[it][q] = 0.0f;

  load(cur, ntiles - 1, true);
  float4 hc = *reinterpret_cast<const float4*>(ck + ((ntiles - 1) * kWave + lane) * kDState + g * NS);
  for (int64_t k = ntiles - 1; k >= 0; --k) {
    const int64_t t0 = k * T;
    const int nt = tile_rows(k);
    float xv[IPT][CW], dyv[IPT][CW], dt2v[IPT][CW], sgv[IPT][CW], gv[IPT][CW], zv[IPT][CW];
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
#pragma unroll
      for (int q = 0; q < CW; ++q) {
        const float x = cur.rx[it].get(q);
        const float u = cur.rd[it].get(q) + ibias[it][q];
        const float u2 = __builtin_fmaf(cur.rd[it].get(q), kLog2e, ibias2[it][q]);
        const float dt2 = softplus ? softplus2_f(u2) : u2;
        const float gg = cur.rg[it].get(q);
        float dy = gg;
        if (HAS_Z) {
          const float z = cur.rz[it].get(q);
          zv[it][q] = z;
          dy = gg * silu_f(z);
        }
        xv[it][q] = x;
        gv[it][q] = gg;
        dyv[it][q] = dy;
        dt2v[it][q] = dt2;
        sgv[it][q] = softplus ? __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u * kLog2e)) : 1.0f;
        sh_dtu[irow[it]][icol[it] + q] = make_float2(dt2, dt2 * x);
        sh_dy[irow[it]][icol[it] + q] = dy;
      }
    }
    stage_bc(cur, true);
    h[0] = hc.x; h[1] = hc.y; h[2] = hc.z; h[3] = hc.w;
    if (k > 0) {
      load(nxt, k - 1, true);
      hc = *reinterpret_cast<const float4*>(ck + ((k - 1) * kWave + lane) * kDState + g * NS);
    }
    block_sync();

    // forward within the tile: each step's incoming state, and readout partials
    float hp[T][NS];
#pragma unroll
    for (int s = 0; s < T; ++s) {
      if (s < nt) {
        const float2 v = sh_dtu[s][loff];
        float y = 0.0f;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          hp[s][i] = h[i];
          h[i] = __builtin_fmaf(__builtin_amdgcn_exp2f(v.x * Ad[i]), h[i], v.y * sh_B[s][g * NS + i]);
          y = __builtin_fmaf(sh_C[s][g * NS + i], h[i], y);
        }
        sh_y[s][g * kWave + lane] = y;
      }
    }

    // reverse within the tile
#pragma unroll
    for (int s = T - 1; s >= 0; --s) {
      if (s < nt) {
        const float2 v = sh_dtu[s][loff];
        const float dy = sh_dy[s][loff];
        float s1 = 0.0f, s2 = 0.0f, cb[NS], cc[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const float aa = __builtin_amdgcn_exp2f(v.x * Ad[i]);
          const float Bs = sh_B[s][g * NS + i];
          const float dh = __builtin_fmaf(dy, sh_C[s][g * NS + i], carry[i]);
          const float hs = __builtin_fmaf(aa, hp[s][i], v.y * Bs);
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
        // dB', dC of this step over the wavefront's 64 channels: every lane
        // stages its 8 contributions; lane 8j + p sums contribution j of
        // lanes 8p .. 8p + 7; three DPP steps (two within the quad, then
        // row_half_mirror, which swaps the two quads of each 8-lane half)
        // leave the total in all 8 lanes of group j.
        // (a lane's 8 values sit at stride 9: 9 is odd, so both the writes
        // and the column reads below touch 64 distinct banks)
        float* red = &sh_red[g][0];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          red[lane * 9 + i] = cb[i];
          red[lane * 9 + NS + i] = cc[i];
        }
        __builtin_amdgcn_wave_barrier();
        const int j = lane >> 3, p = lane & 7;
        float acc = 0.0f;
        if (nvalid == kWave) {
#pragma unroll
          for (int m = 0; m < 8; ++m) acc += red[(p * 8 + m) * 9 + j];
        } else {  // lanes past the last channel hold duplicates: leave them out
#pragma unroll
          for (int m = 0; m < 8; ++m) acc += (p * 8 + m < nvalid) ? red[(p * 8 + m) * 9 + j] : 0.0f;
        }
        acc += SSM_DPP(0.0f, acc, 0xb1, 0xf);   // quad_perm [1,0,3,2]
        acc += SSM_DPP(0.0f, acc, 0x4e, 0xf);   // quad_perm [2,3,0,1]
        acc += SSM_DPP(0.0f, acc, 0x141, 0xf);  // row_half_mirror
        if (p == 0) sh_bc[s][j >> 2][g * NS + (j & 3)] = acc;
        __builtin_amdgcn_wave_barrier();
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
          if (HAS_Z) {
            y = __builtin_fmaf(iD[it][q], xv[it][q], y);
            const float z = zv[it][q];
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
            oz[q] = gv[it][q] * y * (sg * __builtin_fmaf(z, 1.0f - sg, 1.0f));
          }
          ox[q] = __builtin_fmaf(dyv[it][q], iD[it][q], dt2v[it][q] * S1);
          const float ddt = __builtin_fmaf(xv[it][q] * kLog2e, S1, S2);
          od[q] = ddt * sgv[it][q];
          dDacc[it][q] = __builtin_fmaf(dyv[it][q], xv[it][q], dDacc[it][q]);
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
      a.ws_bc[((b * L + t0 + s) * a.nblk + blk) * (2 * kDState) + w] = (&sh_bc[s][0][0])[w];
    }
    block_sync();
    cur = nxt;
  }

  // per-row parameter gradients and the initial state's gradient
  if (lane < nvalid) {
    *reinterpret_cast<float4*>(a.ws_a + (b * Dn + dl) * kDState + g * NS) =
        make_float4(dAacc[0] * kLn2, dAacc[1] * kLn2, dAacc[2] * kLn2, dAacc[3] * kLn2);
    if (a.dh0 != nullptr)
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
    a.ws_dd[(b * Dn + d0 + tid) * 2] = sD;
    a.ws_dd[(b * Dn + d0 + tid) * 2 + 1] = sB;
  }
}

// dB, dC: sum the per-block partials in block order (dB also takes the ln 2).
template <typename Tg>
__global__ void __launch_bounds__(256) bwd_reduce_bc_kernel(const float* ws_bc, Tg* dB, Tg* dC, int64_t rows,
                                                            int nblk) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * 2 * kDState) return;
  const int64_t row = i / (2 * kDState);
  const int w = (int)(i % (2 * kDState));
  float acc = 0.0f;
  for (int k = 0; k < nblk; ++k) acc += ws_bc[(row * nblk + k) * (2 * kDState) + w];
  Tg* dst = w < kDState ? dB : dC;
  const float v = w < kDState ? acc * kLn2 : acc;
  const int64_t o = row * kDState + (w % kDState);
  if constexpr (sizeof(Tg) == 4) dst[o] = v;
  else dst[o] = f32_to_bf16_rne(v);
}

// dA, dD, dbias: sum the per-row partials over the batch in row order.
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

// --------------------------------------------------------------- launchers

template <typename Tin, typename Tout, int NS, bool WIDE>
hipError_t launch_scan_w(const ScanArgs& a, hipStream_t s) {
  constexpr int G = kDState / NS;
  const unsigned nblk = (unsigned)((a.d_inner + kWave - 1) / kWave);
  if (a.n_chunks > 1) {
    dim3 gridA(nblk, (unsigned)(a.n_chunks - 1), (unsigned)a.batch);
    hipLaunchKernelGGL((scan_chunk_kernel<Tin, Tout, NS, true, false, WIDE>), gridA, dim3(kWave * G), 0, s, a);
    const unsigned ncolblk = (unsigned)((a.d_inner * kDState + 63) / 64);
    hipLaunchKernelGGL(carry_kernel, dim3(ncolblk, (unsigned)a.batch), dim3(256), 0, s, a.ws_state,
                       (const float*)a.ws_dtsum, a.A, a.d_inner, a.n_chunks);
  }
  dim3 gridB(nblk, (unsigned)a.n_chunks, (unsigned)a.batch);
  if (a.z != nullptr)
    hipLaunchKernelGGL((scan_chunk_kernel<Tin, Tout, NS, false, true, WIDE>), gridB, dim3(kWave * G), 0, s, a);
  else
    hipLaunchKernelGGL((scan_chunk_kernel<Tin, Tout, NS, false, false, WIDE>), gridB, dim3(kWave * G), 0, s, a);
  return hipGetLastError();
}

// The wide prologue/epilogue needs rows that split into aligned groups of 8.
template <typename Tin, typename Tout, int NS>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s) {
  if (a.d_inner % 8 == 0) return launch_scan_w<Tin, Tout, NS, true>(a, s);
  return launch_scan_w<Tin, Tout, NS, false>(a, s);
}

template <typename Tin, typename Tout>
hipError_t launch_scan_ns(const ScanArgs& a, int ns, hipStream_t s) {
  switch (ns) {
    case 1: return launch_scan_t<Tin, Tout, 1>(a, s);
    case 2: return launch_scan_t<Tin, Tout, 2>(a, s);
    case 4: return launch_scan_t<Tin, Tout, 4>(a, s);
    case 8: return launch_scan_t<Tin, Tout, 8>(a, s);
    case 16: return launch_scan_t<Tin, Tout, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, DT in, DT out, int ns, hipStream_t s) {
  if (in == DT::F32 && out == DT::F32) return launch_scan_ns<float, float>(a, ns, s);
  if (in == DT::F32 && out == DT::BF16) return launch_scan_ns<float, uint16_t>(a, ns, s);
  if (in == DT::BF16 && out == DT::F32) return launch_scan_ns<uint16_t, float>(a, ns, s);
  return launch_scan_ns<uint16_t, uint16_t>(a, ns, s);
}

hipError_t launch_decode(const DecodeArgs& a, DT in, DT out, hipStream_t s) {
  const int64_t threads = a.pairs * 4;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (in == DT::F32 && out == DT::F32)
    hipLaunchKernelGGL((decode_kernel<float, float>), dim3(grid), dim3(256), 0, s, a);
  else if (in == DT::F32 && out == DT::BF16)
    hipLaunchKernelGGL((decode_kernel<float, uint16_t>), dim3(grid), dim3(256), 0, s, a);
  else if (in == DT::BF16 && out == DT::F32)
    hipLaunchKernelGGL((decode_kernel<uint16_t, float>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<uint16_t, uint16_t>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = min((int64_t)4096, (n + 255) / 256);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = min((int64_t)4096, (n + 255) / 256);
  hipLaunchKernelGGL(copy_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

namespace {

// Run length: 32 steps, doubled while the grid would need more than about
// three wavefronts per SIMD (the kernel's occupancy), so that one round of
// resident wavefronts covers the whole sequence.
int conv_run_len(int64_t waves_per_step_row, int64_t batch, int64_t seqlen) {
  int run = 32;
  while (run < 256 && waves_per_step_row * batch * ((seqlen + run - 1) / run) > 3 * 1024) run *= 2;
  return run;
}

template <typename Tin, typename Tout, int K, int CW>
void launch_conv1d_cw(const ConvArgs& a, hipStream_t s) {
  const int64_t groups = a.d_inner / CW;
  const int64_t gblocks = (groups + 63) / 64;
  const int run = conv_run_len(gblocks, a.batch, a.seqlen);
  const int64_t runs = (a.seqlen + run - 1) / run;
  const dim3 grid((unsigned)gblocks, (unsigned)min(runs, (int64_t)65535), (unsigned)a.batch);
  if (a.silu)
    hipLaunchKernelGGL((conv1d_kernel<Tin, Tout, K, CW, true>), grid, dim3(64), 0, s, a, groups, runs, run);
  else
    hipLaunchKernelGGL((conv1d_kernel<Tin, Tout, K, CW, false>), grid, dim3(64), 0, s, a, groups, runs, run);
}

template <typename Tin, typename Tout, int K>
hipError_t launch_conv1d_k(const ConvArgs& a, hipStream_t s) {
  if (a.seqlen > 0 && a.batch > 0 && a.d_inner > 0) {
    constexpr int CWV = 16 / (int)sizeof(Tin);  // channels per 16-byte access
    if (a.d_inner % CWV == 0) launch_conv1d_cw<Tin, Tout, K, CWV>(a, s);
    else launch_conv1d_cw<Tin, Tout, K, 1>(a, s);
  }
  if (a.state_out != nullptr && a.batch > 0 && a.d_inner > 0) {
    const int64_t blocks = ((int64_t)a.batch * a.d_inner + 255) / 256;
    hipLaunchKernelGGL((conv1d_state_kernel<Tin, K>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_conv1d_t(const ConvArgs& a, int K, hipStream_t s) {
  switch (K) {
    case 2: return launch_conv1d_k<Tin, Tout, 2>(a, s);
    case 3: return launch_conv1d_k<Tin, Tout, 3>(a, s);
    case 4: return launch_conv1d_k<Tin, Tout, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename Tin, typename Tout, int K, int CW>
void launch_conv1d_update_cw(const ConvArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.batch * a.d_inner / CW;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (a.silu)
    hipLaunchKernelGGL((conv1d_update_kernel<Tin, Tout, K, CW, true>), grid, dim3(256), 0, s, a, n);
  else
    hipLaunchKernelGGL((conv1d_update_kernel<Tin, Tout, K, CW, false>), grid, dim3(256), 0, s, a, n);
}

// Channels per thread: enough that a thread's cache run (CW * K inputs) is
// one or three 16-byte vectors.
template <typename Tin, typename Tout, int K>
void launch_conv1d_update_k(const ConvArgs& a, hipStream_t s) {
  constexpr int kBytes = K * (int)sizeof(Tin);
  constexpr int CW = (16 % kBytes == 0) ? 16 / kBytes : 48 / kBytes;
  if (a.d_inner % CW == 0) launch_conv1d_update_cw<Tin, Tout, K, CW>(a, s);
  else launch_conv1d_update_cw<Tin, Tout, K, 1>(a, s);
}

template <typename Tin, typename Tout>
hipError_t launch_conv1d_update_t(const ConvArgs& a, int K, hipStream_t s) {
  if ((int64_t)a.batch * a.d_inner <= 0) return hipSuccess;
  switch (K) {
    case 2: launch_conv1d_update_k<Tin, Tout, 2>(a, s); break;
    case 3: launch_conv1d_update_k<Tin, Tout, 3>(a, s); break;
    case 4: launch_conv1d_update_k<Tin, Tout, 4>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv1d(const ConvArgs& a, DT in, DT out, int K, hipStream_t s) {
  if (in == DT::F32 && out == DT::F32) return launch_conv1d_t<float, float>(a, K, s);
  if (in == DT::F32 && out == DT::BF16) return launch_conv1d_t<float, uint16_t>(a, K, s);
  if (in == DT::BF16 && out == DT::F32) return launch_conv1d_t<uint16_t, float>(a, K, s);
  return launch_conv1d_t<uint16_t, uint16_t>(a, K, s);
}

hipError_t launch_conv1d_update(const ConvArgs& a, DT in, DT out, int K, hipStream_t s) {
  if (in == DT::F32 && out == DT::F32) return launch_conv1d_update_t<float, float>(a, K, s);
  if (in == DT::F32 && out == DT::BF16) return launch_conv1d_update_t<float, uint16_t>(a, K, s);
  if (in == DT::BF16 && out == DT::F32) return launch_conv1d_update_t<uint16_t, float>(a, K, s);
  return launch_conv1d_update_t<uint16_t, uint16_t>(a, K, s);
}

namespace {

template <typename Tin, typename Tg>
void launch_scan_bwd_t(const BwdArgs& a, float* dA, void* dB, void* dC, float* dD, float* dbias, hipStream_t s) {
  const dim3 grid((unsigned)a.nblk, (unsigned)a.batch);
  if (a.seqlen > 0) {
    if (a.d_inner % 4 == 0) {
      if (a.z != nullptr) hipLaunchKernelGGL((scan_bwd_kernel<Tin, Tg, true, 4>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((scan_bwd_kernel<Tin, Tg, false, 4>), grid, dim3(256), 0, s, a);
    } else {
      if (a.z != nullptr) hipLaunchKernelGGL((scan_bwd_kernel<Tin, Tg, true, 1>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((scan_bwd_kernel<Tin, Tg, false, 1>), grid, dim3(256), 0, s, a);
    }
    const int64_t rows = (int64_t)a.batch * a.seqlen;
    const int64_t n = rows * 2 * kDState;
    hipLaunchKernelGGL((bwd_reduce_bc_kernel<Tg>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.ws_bc,
                       static_cast<Tg*>(dB), static_cast<Tg*>(dC), rows, a.nblk);
  }
  const int64_t np = a.d_inner * kDState;
  hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, s, a.ws_a, a.ws_dd,
                     dA, dD, dbias, (int64_t)a.batch, a.d_inner);
}

}  // namespace

hipError_t launch_scan_bwd(const BwdArgs& a, DT in, DT grad, float* dA, void* dB, void* dC, float* dD,
                           float* dbias, hipStream_t s) {
  if (in == DT::F32 && grad == DT::F32) launch_scan_bwd_t<float, float>(a, dA, dB, dC, dD, dbias, s);
  else if (in == DT::F32 && grad == DT::BF16) launch_scan_bwd_t<float, uint16_t>(a, dA, dB, dC, dD, dbias, s);
  else if (in == DT::BF16 && grad == DT::F32) launch_scan_bwd_t<uint16_t, float>(a, dA, dB, dC, dD, dbias, s);
  else launch_scan_bwd_t<uint16_t, uint16_t>(a, dA, dB, dC, dD, dbias, s);
  return hipGetLastError();
}

hipError_t launch_affine_exclusive_scan(const float* a, const float* b, float* oa, float* ob,
                                        int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(affine_exclusive_scan_kernel, dim3(1), dim3(64), 0, s, a, b, oa, ob, n);
  return hipGetLastError();
}

}  // namespace ssm

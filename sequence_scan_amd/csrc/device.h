// Device-side helpers shared by the gfx950 kernels of libssmscan: element
// loads and conversions (bf16 <-> fp32), pointwise functions (softplus, SiLU),
// the wavefront affine-pair scan, the pinned workgroup barrier and the
// vector load/store shapes of the tiled kernels.  Everything here is inlined
// into the kernels of each translation unit.
#ifndef SSMSCAN_DEVICE_H
#define SSMSCAN_DEVICE_H

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

// Streaming (non-temporal) 16-byte access to four floats, for data that a
// kernel touches once: the decode kernels' states, which one step reads and
// writes and the next step reads again after every other state has passed
// through the caches.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_stream4(const float* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream4(float* p, float4 v) {
  const f32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4_t*>(p));
}

// Four consecutive input elements (fp32, or bf16 bit patterns) as floats; the
// address is 16-byte (fp32) or 8-byte (bf16) aligned.
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

// One element of the input dtype, as fp32 (and back: exact for a value that
// came from that dtype).
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

// The exact zero-order-hold input coefficient in the scan's log2 units.  For
// a diagonal entry A and step dt the coefficient is (e^{dt A} - 1) / A (the
// integral of e^{sA} over the step), = zoh_ratio(a) * dt2 with a = exp2(u2),
// u2 = dt2 A, dt2 = dt log2(e), and zoh_ratio(a) = (a - 1) / log2(a).  Forming
// a - 1 directly cancels when dt A is small; taking the logarithm of the same
// rounded a (W. Kahan's device for expm1) makes the two errors cancel in the
// ratio, which is a smooth function of a (about ln 2 * (1 + (a - 1) / 2) near
// 1).  The ratio is ln 2 at a = 1 (its limit), and below the smallest normal
// a, where the logarithm is not usable, u2 stands in for log2(a) (there a - 1
// is -1 to fp32 precision).
__device__ __forceinline__ float zoh_ratio(float a, float u2) {
  const float l = a >= 1.17549435e-38f ? __builtin_amdgcn_logf(a) : u2;  // log2(a)
  const float r = (a - 1.0f) * __builtin_amdgcn_rcpf(l);
  return a == 1.0f ? kLn2 : r;
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^{-z}).
__device__ __forceinline__ float silu_f(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * kLog2e);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// The wavefronts that share a SIMD are issued oldest first.  When every
// workgroup of a grid is resident at once, the workgroups placed last on a CU
// therefore fall behind and finish alone, with one wavefront per SIMD.
// Lowering a wavefront's issue priority as it progresses (four levels, one per
// quarter of its work) hands issue slots to the wavefronts that lag, so the
// workgroups of a CU finish together.  Work counts are uniform in the wave.
struct ProgressPriority {
  int64_t q1, q2, q3;  // first item of the second, third and fourth quarter
  __device__ explicit ProgressPriority(int64_t total)
      : q1((total + 3) / 4), q2((2 * total + 3) / 4), q3((3 * total + 3) / 4) {}
  __device__ __forceinline__ void at(int64_t done) const {
    if (done < q1) __builtin_amdgcn_s_setprio(3);
    else if (done < q2) __builtin_amdgcn_s_setprio(2);
    else if (done < q3) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  }
};

// Host side: workgroups of `kern` that one CU holds at once (0 if the query
// fails), and whether a grid of that kernel is resident all at once on a
// device of `cus` CUs.
template <typename K>
inline int resident_per_cu(K kern, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, 0) != hipSuccess) n = 0;
  return n;
}

inline bool grid_coresident(int per_cu, int cus, dim3 grid) {
  const int64_t wgs = (int64_t)grid.x * grid.y * grid.z;
  return per_cu > 0 && cus > 0 && wgs <= (int64_t)per_cu * cus;
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

// Store CW contiguous outputs of one row.  Groups of four fp32 values go out as
// non-temporal stores: outputs are written once and not read again by the
// kernel, so they need not displace cached inputs (about 1 % on the scan).
template <typename Tout, int CW>
__device__ __forceinline__ void store_row(Tout* p, const float* v) {
  if constexpr (sizeof(Tout) == 4) {
    if constexpr (CW % 4 == 0) {
#pragma unroll
      for (int q = 0; q < CW / 4; ++q)
        __builtin_nontemporal_store(f32x4_t{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]},
                                    reinterpret_cast<f32x4_t*>(p) + q);
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


}  // namespace
}  // namespace ssm

#endif  // SSMSCAN_DEVICE_H

// Issue-rate probe of gfx950's vector ALU for the scan's instruction mix.
// Built as its own library (libssmprobe.so) for the benchmark's ceiling leg;
// the scan library does not contain or call it.
//
// Each kernel runs a fixed number of iterations of straight-line fp32 work on
// independent registers, so that with several wavefronts per SIMD the SIMD's
// issue rate, not latency, sets the time.  Every wavefront records its shader
// clock counter (s_memtime) and the 100 MHz real-time counter (s_memrealtime)
// at start and end, which gives the clock the work ran at.  The host derives
// SIMD-cycles per instruction from the launch's duration, that clock and the
// instruction count.
//
// Kinds:
//   0  v_mul_f32 on 8 independent chains
//   1  v_fma_f32 on 8 independent chains
//   2  v_exp_f32 on 8 independent chains
//   3  the scan's state update for 4 states per lane, as its kernel issues it:
//      a = exp2(w * A_n); h_n = fma(a, h_n, u * B_n); y = fma(C_n, h_n, y)
//      (four VALU instructions and one v_exp_f32 per update)
//   4  v_log_f32, 5  v_rcp_f32 on 8 independent chains
//   6  the state update of kind 3 without the exponential (a = w * A_n):
//      four VALU instructions per update, no transcendental in the stream
//   7  v_mul_f32 with a wave-uniform operand read from an SGPR, 8 chains
//   9  the scan's state update with transitions as powers of one number e
//      (per step and 4 states: e^2, e^4, two selects, the base, three chain
//      multiplies, then per state u * B, fma(a, h, .), fma(C, h, y)): 21 fp32
//      VALU instructions per 4 updates, no transcendental
//   8  even wavefronts run v_exp_f32 only (2 chains), odd wavefronts
//      v_fma_f32 only (8 chains): the count is of instructions issued per
//      pair of wavefronts, 2 exps + 8 FMAs per step
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// keeps the compiler from treating v as loop-invariant (emits no instruction)
#define PROBE_OPAQUE(v) asm volatile("" : "+v"(v))

template <int KIND>
__global__ void __launch_bounds__(256) probe_kernel(int iters, float seed, float uniform, float* sink,
                                                    int64_t* stamps) {
  const int tid = threadIdx.x;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + tid) >> 6;
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = seed * (float)(i + 1) + (float)tid * 1e-3f;
  const float c = 0.999f, d = 1e-3f;
  // per-lane operands in VGPRs, as in the scan kernel (A per channel; B and C
  // there come from LDS into VGPRs)
  float A[4], Bv[4], Cv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    A[i] = -1.13f * (float)(i + 1) - (float)tid * 1e-6f;
    Bv[i] = 0.53f - 0.27f * (float)i + (float)tid * 1e-6f;
    Cv[i] = 1.03f - 0.51f * (float)i - (float)tid * 1e-6f;
  }
  float w = seed * 1e-2f, u = seed;
  float ys[8];  // one readout chain per unrolled step, as the kernel restarts it every step
#pragma unroll
  for (int i = 0; i < 8; ++i) ys[i] = 0.0f;
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = 0.9f + (float)tid * 1e-5f * (float)(i + 1);
  const int64_t t0 = (int64_t)__builtin_amdgcn_s_memtime();
  const int64_t r0 = (int64_t)__builtin_amdgcn_s_memrealtime();
  if constexpr (KIND == 8) {
    // specialised wavefronts: the branch is uniform per wavefront and taken once
    if (((__builtin_amdgcn_readfirstlane(tid) >> 6) & 1) == 0) {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
          for (int i = 0; i < 2; ++i) r[i] = __builtin_amdgcn_exp2f(r[i]);
        }
      }
    } else {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
          for (int i = 0; i < 8; ++i) r[i] = __builtin_fmaf(r[i], q[i], d);
        }
      }
    }
  }
  if constexpr (KIND != 8)
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if constexpr (KIND == 9) {
        PROBE_OPAQUE(w);
        PROBE_OPAQUE(u);
        const float e = w, e2 = e * e, e4 = e2 * e2;
        float ap = (e * __builtin_fmaf(q[0], e, q[1])) * __builtin_fmaf(q[2], e2, q[3]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i > 0) ap = ap * e4;
          r[i] = __builtin_fmaf(ap, r[i], u * Bv[i]);
          ys[s] = __builtin_fmaf(Cv[i], r[i], ys[s]);
        }
      } else if constexpr (KIND == 3 || KIND == 6) {
        PROBE_OPAQUE(w);
        PROBE_OPAQUE(u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = KIND == 3 ? __builtin_amdgcn_exp2f(w * A[i]) : w * A[i];
          r[i] = __builtin_fmaf(a, r[i], u * Bv[i]);
          ys[s] = __builtin_fmaf(Cv[i], r[i], ys[s]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if constexpr (KIND == 0) r[i] = r[i] * c;
          if constexpr (KIND == 1) r[i] = __builtin_fmaf(r[i], c, d);
          if constexpr (KIND == 2) r[i] = __builtin_amdgcn_exp2f(r[i]);
          if constexpr (KIND == 4) r[i] = __builtin_amdgcn_logf(r[i]);
          if constexpr (KIND == 5) r[i] = __builtin_amdgcn_rcpf(r[i]);
          if constexpr (KIND == 7) r[i] = r[i] * uniform;
        }
      }
    }
  }
  const int64_t t1 = (int64_t)__builtin_amdgcn_s_memtime();
  const int64_t r1 = (int64_t)__builtin_amdgcn_s_memrealtime();
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc += r[i] + ys[i];
  sink[(int64_t)blockIdx.x * blockDim.x + tid] = acc;
  if ((tid & 63) == 0) {
    stamps[wave * 4 + 0] = t0;
    stamps[wave * 4 + 1] = t1;
    stamps[wave * 4 + 2] = r0;
    stamps[wave * 4 + 3] = r1;
  }
}

}  // namespace

extern "C" {

// Instructions of the measured kind per wavefront and iteration (kinds 3, 6
// and 9 count state updates: five, four and 5.25 instructions each; kind 8
// counts the average over its two kinds of wavefront).
int ssm_probe_ops_per_iter(int kind) { return (kind == 3 || kind == 6 || kind == 9) ? 32 : (kind == 8 ? 40 : 64); }

// Launch `blocks` workgroups of 256 threads (4 wavefronts) running `iters`
// iterations of kind `kind`.  sink: blocks * 256 floats; stamps: blocks * 4 * 4
// int64 (per wavefront: memtime start, end, realtime start, end).  Returns a
// hipError_t code (0 on success).
int ssm_probe_launch(int kind, int blocks, int iters, float seed, float* sink, int64_t* stamps, void* stream) {
  if (blocks < 1 || iters < 1 || !sink || !stamps) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)blocks), block(256);
  const float u = 0.9993f;
  switch (kind) {
    case 0: hipLaunchKernelGGL(probe_kernel<0>, grid, block, 0, s, iters, seed, u, sink, stamps); break;
    case 1: hipLaunchKernelGGL(probe_kernel<1>, grid, block, 0, s, iters, seed, u, sink, stamps); break;
    case 2: hipLaunchKernelGGL(probe_kernel<2>, grid, block, 0, s, iters, seed, u, sink, stamps); break;
    case 3: hipLaunchKernelGGL(probe_kernel<3>, grid, block, 0, s, iters, seed, u, sink, stamps); break;
    case 4: hipLaunchKernelGGL(probe_kernel<4>, grid, block, 0, s, iters, seed, u, sink, stamps); break;
    case 5: hipLaunchKernelGGL(probe_kernel<5>, grid, block, 0, s, iters, seed, u, sink, stamps); break;
    case 6: hipLaunchKernelGGL(probe_kernel<6>, grid, block, 0, s, iters, seed, u, sink, stamps); break;
    case 7: hipLaunchKernelGGL(probe_kernel<7>, grid, block, 0, s, iters, seed, u, sink, stamps); break;
    case 8: hipLaunchKernelGGL(probe_kernel<8>, grid, block, 0, s, iters, seed, u, sink, stamps); break;
    case 9: hipLaunchKernelGGL(probe_kernel<9>, grid, block, 0, s, iters, seed, u, sink, stamps); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // extern "C"

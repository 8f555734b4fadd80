// gfx950 kernels of libssmscan: the block's causal depthwise conv1d (prefill
// and decode step).
#include "device.h"

namespace ssm {
namespace {

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

// Steps per thread: a multiple of 8, chosen on the host (conv_run_len).

// Grid: x = blocks of 64 channel groups (one wavefront), y = runs (strided),
// z = batch row, so the run (and with it every load and store condition) is
// uniform across the wavefront.
// With write_cache, the thread that runs a channel group's last run also
// stores the outgoing cache from its final window (the last K inputs, oldest
// first); the host asks for this only when the outgoing cache is not the
// incoming one, which other runs may still be reading.
template <typename Tin, typename Tout, int K, int CW, bool SILU>
__global__ void __launch_bounds__(64) conv1d_kernel(ConvArgs a, int64_t groups, int64_t runs, int run_len,
                                                    int write_cache) {
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
    if (write_cache && r == runs - 1) {
      // exact: every window value came from a Tin
      Tin* cache = static_cast<Tin*>(a.state_out) + (b * Dn + d0) * K;
      constexpr int kCacheBytes = CW * K * (int)sizeof(Tin);
      float cv[CW * K];
#pragma unroll
      for (int q = 0; q < CW; ++q)
#pragma unroll
        for (int k = 0; k < K; ++k) cv[q * K + k] = win[k][q];
      if constexpr (kCacheBytes == 4 || kCacheBytes == 8 || kCacheBytes % 16 == 0) {
        store_row<Tin, CW * K>(cache, cv);
      } else {
#pragma unroll
        for (int j = 0; j < CW * K; ++j) st_in(cache + j, cv[j]);
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

}  // namespace

namespace {

// Run length: 32 steps, doubled while the grid would need more than about
// six wavefronts per SIMD, so that few rounds of wavefronts cover the whole
// sequence and each run's K - 1 re-read steps stay a small share.  (On
// MI355X: 32 steps for the Mamba-2.8B-like layer ran 80.5 us against 84.5 us
// at 64; 16 steps slowed narrow layers; the 2^18-step sequence runs 256 at
// copy speed.)
// The prefill kernel stores the outgoing cache itself unless it is the
// incoming one (updated in place): then a separate kernel, launched after the
// prefill, reads each channel's inputs before writing them.
bool conv_cache_fused(const ConvArgs& a) {
  return a.state_out != nullptr && a.state_out != a.state_in && a.seqlen > 0;
}

int conv_run_len(int64_t waves_per_step_row, int64_t batch, int64_t seqlen) {
  int run = 32;
  while (run < 256 && waves_per_step_row * batch * ((seqlen + run - 1) / run) > 6 * 1024) run *= 2;
  return run;
}

template <typename Tin, typename Tout, int K, int CW>
void launch_conv1d_cw(const ConvArgs& a, hipStream_t s) {
  const int64_t groups = a.d_inner / CW;
  const int64_t gblocks = (groups + 63) / 64;
  const int run = conv_run_len(gblocks, a.batch, a.seqlen);
  const int64_t runs = (a.seqlen + run - 1) / run;
  const dim3 grid((unsigned)gblocks, (unsigned)min(runs, (int64_t)65535), (unsigned)a.batch);
  const int wc = conv_cache_fused(a) ? 1 : 0;
  if (a.silu)
    hipLaunchKernelGGL((conv1d_kernel<Tin, Tout, K, CW, true>), grid, dim3(64), 0, s, a, groups, runs, run, wc);
  else
    hipLaunchKernelGGL((conv1d_kernel<Tin, Tout, K, CW, false>), grid, dim3(64), 0, s, a, groups, runs, run, wc);
}

template <typename Tin, typename Tout, int K>
hipError_t launch_conv1d_k(const ConvArgs& a, hipStream_t s) {
  if (a.seqlen > 0 && a.batch > 0 && a.d_inner > 0) {
    constexpr int CWV = 16 / (int)sizeof(Tin);  // channels per 16-byte access
    if (a.d_inner % CWV == 0) launch_conv1d_cw<Tin, Tout, K, CWV>(a, s);
    else launch_conv1d_cw<Tin, Tout, K, 1>(a, s);
  }
  if (a.state_out != nullptr && a.batch > 0 && a.d_inner > 0 && !conv_cache_fused(a)) {
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

}  // namespace ssm

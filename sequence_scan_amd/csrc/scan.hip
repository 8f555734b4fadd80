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
//    scans the pairs in time order with a wavefront DPP scan (lane = chunk);
//    with at most 16 chunks one thread per coordinate applies them in order.
//    Pass B re-runs each chunk from its incoming state with the full readout.
#include <mutex>

#include "device.h"

namespace ssm {
namespace {

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

// The carry for a sequence cut into few chunks (at most kFewPairs pairs): one
// thread per (batch row, coordinate) applies its pairs in time order,
// h <- exp2(A[d,n] S_p) h + end_p from h = 0, and stores each h in slot p.
// The loads of every pair are independent of h, so they are all in flight at
// once; the wavefront scan above would spend a whole DPP scan on each column
// for a handful of lanes.
constexpr int kFewPairs = 15;
__global__ void __launch_bounds__(256) carry_few_kernel(float* ws_state, const float* ws_dtsum, const float* A,
                                                        int64_t Dn, int K) {
  const int64_t ncol = Dn * kDState;
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = blockIdx.y;
  if (col >= ncol) return;
  const float a2 = A[col];  // S is a sum of log2-unit step sizes
  const int np = K - 1;
  float e[kFewPairs], S[kFewPairs];
#pragma unroll
  for (int p = 0; p < kFewPairs; ++p) {
    if (p < np) {
      const int64_t slot = b * K + p;
      e[p] = ws_state[slot * ncol + col];
      S[p] = ws_dtsum[slot * Dn + (col >> 4)];
    }
  }
  float h = 0.0f;
#pragma unroll
  for (int p = 0; p < kFewPairs; ++p) {
    if (p < np) {
      h = __builtin_fmaf(__builtin_amdgcn_exp2f(S[p] * a2), h, e[p]);
      ws_state[(b * K + p) * ncol + col] = h;
    }
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
// (one 16-byte load and store of the fp32 state).  Each thread takes the same
// channel in kDecodeRows consecutive batch rows: it issues every row's loads
// before the first row's arithmetic, and the rows share the channel's A, D
// and bias.  The readout is reduced over the quad with two DPP quad permutes;
// lane 0 of the quad applies the D skip and the gate and stores out.  The
// state and the per-step x, delta, z and out stream (non-temporal loads and
// stores): one step touches them once, and the 128 MiB state of a batch-256
// step does not survive in the caches until the next step anyway.  Streaming
// the state too took that step from 63.9 to 57.7 us on MI355X (4.5 -> 5.0
// TB/s), and two rows per thread from 58.3 to 50.7 us (5.7 TB/s; four rows:
// 52.2 us; two lanes of eight states per channel: 60.8 us).  A, B, C, D and
// the bias, which many rows share, are ordinary cached loads.
constexpr int kDecodeRows = 2;

template <typename Tin>
__device__ __forceinline__ float nt_load(const void* p, int64_t i) {
  if constexpr (sizeof(Tin) == 4) {
    return __builtin_nontemporal_load(static_cast<const float*>(p) + i);
  } else {
    return bf16_to_f32(__builtin_nontemporal_load(static_cast<const uint16_t*>(p) + i));
  }
}


template <typename Tin, typename Tout, bool ZOH>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a) {
  // grid: x = blocks of 64 channels, y = groups of kDecodeRows batch rows
  const int64_t d = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int q = threadIdx.x & 3;
  if (d >= a.d_inner) return;  // whole quads leave together
  const int64_t nb = a.pairs / a.d_inner;
  const float4 av = *reinterpret_cast<const float4*>(a.A + d * kDState + 4 * q);
  const float A2[4] = {av.x * kLog2e, av.y * kLog2e, av.z * kLog2e, av.w * kLog2e};
  const float bias = a.bias != nullptr ? a.bias[d] : 0.0f;
  const float Dd = a.D != nullptr ? a.D[d] : 0.0f;
  // every row's loads first; a row past the batch (odd batch) re-reads the
  // last row and stores nothing
  float4 hs[kDecodeRows];
  float Bv[kDecodeRows][4], Cv[kDecodeRows][4], x[kDecodeRows], dl[kDecodeRows], zv[kDecodeRows];
  int64_t e[kDecodeRows];
  bool live[kDecodeRows];
#pragma unroll
  for (int r = 0; r < kDecodeRows; ++r) {
    const int64_t br = (int64_t)blockIdx.y * kDecodeRows + r;
    live[r] = br < nb;
    const int64_t b = live[r] ? br : nb - 1;
    e[r] = b * a.d_inner + d;
    hs[r] = load_stream4(a.state + e[r] * kDState + 4 * q);
    load4<Tin>(a.B, b * kDState + 4 * q, Bv[r]);
    load4<Tin>(a.C, b * kDState + 4 * q, Cv[r]);
    x[r] = nt_load<Tin>(a.x, e[r]);
    dl[r] = nt_load<Tin>(a.delta, e[r]);
    zv[r] = a.z != nullptr ? nt_load<Tin>(a.z, e[r]) : 0.0f;
  }
#pragma unroll
  for (int r = 0; r < kDecodeRows; ++r) {
    const float u = dl[r] + bias;
    const float dt = a.softplus ? softplus_f(u) : u;
    const float dtx = dt * x[r];
    float h[4] = {hs[r].x, hs[r].y, hs[r].z, hs[r].w};
    float y = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float u2 = dt * A2[i];
      const float ar = __builtin_amdgcn_exp2f(u2);
      // ZOH: (e^{dt A} - 1) / A = zoh_ratio(ar) * dt * log2(e)
      if constexpr (ZOH) h[i] = __builtin_fmaf(ar, h[i], (zoh_ratio(ar, u2) * kLog2e) * (dtx * Bv[r][i]));
      else h[i] = __builtin_fmaf(ar, h[i], dtx * Bv[r][i]);
      y = __builtin_fmaf(Cv[r][i], h[i], y);
    }
    if (live[r]) store_stream4(a.state + e[r] * kDState + 4 * q, make_float4(h[0], h[1], h[2], h[3]));
    // quad sum in a fixed order: (q0 + q1) + (q2 + q3) on every lane
    y = y + SSM_DPP(0.0f, y, 0xB1, 0xf);  // quad_perm [1,0,3,2]
    y = y + SSM_DPP(0.0f, y, 0x4E, 0xf);  // quad_perm [2,3,0,1]
    if (q == 0 && live[r]) {
      if (a.D != nullptr) y = __builtin_fmaf(Dd, x[r], y);
      if (a.z != nullptr) y = y * silu_f(zv[r]);
      if constexpr (sizeof(Tout) == 4) {
        __builtin_nontemporal_store(y, static_cast<float*>(a.out) + e[r]);
      } else {
        __builtin_nontemporal_store(f32_to_bf16_rne(y), static_cast<uint16_t*>(a.out) + e[r]);
      }
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

}  // namespace

hipError_t launch_scan(const ScanArgs& a, DT in, DT out, int ns, hipStream_t s) {
  using Fn = hipError_t (*)(const ScanArgs&, int, hipStream_t);
  // [zoh][input bf16][output bf16]
  static const Fn table[2][2][2] = {
      {{launch_scan_f32_f32, launch_scan_f32_bf16}, {launch_scan_bf16_f32, launch_scan_bf16_bf16}},
      {{launch_scan_f32_f32_zoh, launch_scan_f32_bf16_zoh}, {launch_scan_bf16_f32_zoh, launch_scan_bf16_bf16_zoh}}};
  return table[a.zoh ? 1 : 0][in == DT::BF16 ? 1 : 0][out == DT::BF16 ? 1 : 0](a, ns, s);
}

hipError_t launch_carry(const ScanArgs& a, hipStream_t s) {
  if (a.n_chunks - 1 <= kFewPairs) {
    const unsigned nblk = (unsigned)((a.d_inner * kDState + 255) / 256);
    hipLaunchKernelGGL(carry_few_kernel, dim3(nblk, (unsigned)a.batch), dim3(256), 0, s, a.ws_state,
                       (const float*)a.ws_dtsum, a.A, a.d_inner, a.n_chunks);
    return hipGetLastError();
  }
  const unsigned ncolblk = (unsigned)((a.d_inner * kDState + 63) / 64);
  hipLaunchKernelGGL(carry_kernel, dim3(ncolblk, (unsigned)a.batch), dim3(256), 0, s, a.ws_state,
                     (const float*)a.ws_dtsum, a.A, a.d_inner, a.n_chunks);
  return hipGetLastError();
}

namespace {

template <bool ZOH>
void launch_decode_z(const DecodeArgs& a, DT in, DT out, hipStream_t s) {
  const dim3 grid((unsigned)((a.d_inner + 63) / 64),
                  (unsigned)((a.pairs / a.d_inner + kDecodeRows - 1) / kDecodeRows));
  if (in == DT::F32 && out == DT::F32)
    hipLaunchKernelGGL((decode_kernel<float, float, ZOH>), dim3(grid), dim3(256), 0, s, a);
  else if (in == DT::F32 && out == DT::BF16)
    hipLaunchKernelGGL((decode_kernel<float, uint16_t, ZOH>), dim3(grid), dim3(256), 0, s, a);
  else if (in == DT::BF16 && out == DT::F32)
    hipLaunchKernelGGL((decode_kernel<uint16_t, float, ZOH>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<uint16_t, uint16_t, ZOH>), dim3(grid), dim3(256), 0, s, a);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, DT in, DT out, hipStream_t s) {
  if (a.zoh) launch_decode_z<true>(a, in, out, s);
  else launch_decode_z<false>(a, in, out, s);
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

hipError_t launch_affine_exclusive_scan(const float* a, const float* b, float* oa, float* ob,
                                        int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(affine_exclusive_scan_kernel, dim3(1), dim3(64), 0, s, a, b, oa, ob, n);
  return hipGetLastError();
}

// ------------------------------------------------------------ fixed scratch
//
// The carry workspace of ssm_scan_fwd_noalloc, for callers that cannot
// allocate device memory.  Every GPU the library runs on holds its own copy of
// this array until the process ends.  In host code the name `scratch` is a
// host-side stand-in, not a device address: each device's address is looked
// up once with hipGetSymbolAddress while that device is current, and only that
// address is ever handed to kernels.
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

hipError_t scratch_address(float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace ssm

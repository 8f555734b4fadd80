// Internal interface between the C-ABI host layer (api.cpp) and the gfx950
// kernel units (scan_inst.hip, scan.hip, conv.hip, bwd.hip, ssd.hip).  Not
// installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr int kDState = 16;   // the Mamba-1 scan's d_state (the SSD kernels take 64 or 128)
constexpr int kWave = 64;     // gfx950 wavefront size

enum class DT : int { F32 = 0, BF16 = 1 };

struct ScanArgs {
  const void* x;
  const void* delta;
  const void* z;          // nullable
  const void* B;
  const void* C;
  const float* A;         // [d_inner, 16]
  const float* D;         // nullable
  const float* bias;      // nullable
  void* out;
  float* last_state;      // nullable
  const float* h0;        // nullable: initial state [batch, d_inner, 16]
  float* ws_state;        // [batch, n_chunks, d_inner, 16]; chunked runs only
  float* ws_dtsum;        // [batch, n_chunks, d_inner];    chunked runs only
  int64_t seqlen;
  int64_t d_inner;
  int64_t chunk_len;
  int32_t n_chunks;
  int32_t softplus;
  int32_t batch;
  int32_t zoh;            // exact zero-order-hold input coefficient
  int32_t cus;            // compute units of the device
  int32_t fair;           // set by the launcher: the whole grid is co-resident
  int32_t states_only;    // chunked runs: stop after the carry pass (ws_state then holds
                          // the state entering chunk k + 1 in slot k); no out is written
  // Checkpoints (ckpt != nullptr; 4 states per wavefront; chunk lengths
  // multiples of 8): the state entering every global step t with t % 8 == 0 is
  // stored at ckpt[((b * ckpt_nblk + block) * ckpt_tiles + t / 8) * 1024 +
  // lane * 16 + 4 g + i], which holds state g + 4 i of channel d0 + lane (lanes
  // past d_inner repeat the last channel).  With ckpt_only the launch is only
  // that: every chunk runs from its entering state (chunk 0: h0; chunk k > 0:
  // slot k - 1 of ws_state, left by a states_only run) without readout or
  // output.  Without it the scan runs as usual and its pass B stores them.
  float* ckpt;
  int64_t ckpt_tiles;
  int32_t ckpt_nblk;
  int32_t ckpt_only;
};

struct DecodeArgs {
  float* state;
  const void* x;
  const void* delta;
  const void* z;
  const void* B;
  const void* C;
  const float* A;
  const float* D;
  const float* bias;
  void* out;
  int64_t d_inner;
  int64_t pairs;          // batch * d_inner
  int32_t softplus;
  int32_t zoh;            // exact zero-order-hold input coefficient
};

// Causal depthwise conv1d (+ bias, + SiLU) over [batch, seqlen, d_inner].
struct ConvArgs {
  const void* x;
  const float* w;         // [d_inner, K]
  const float* bias;      // nullable
  const void* state_in;   // nullable: [batch, d_inner, K] in the input dtype
  void* out;
  void* state_out;        // nullable: [batch, d_inner, K] in the input dtype
  int64_t seqlen;
  int64_t d_inner;
  int32_t batch;
  int32_t silu;
};

// The Mamba-2 (SSD) scan and its decode step.  x, z, out: [batch, L, nheads,
// headdim]; dt: [batch, L, nheads]; B, C: [batch, L, ngroups, d_state]; A,
// dt_bias: [nheads]; D: [nheads * headdim]; states [batch, nheads, headdim,
// d_state] fp32.  The decode step uses the same struct with seqlen 1.
struct SsdArgs {
  const void* x;
  const void* dt;
  const void* z;          // nullable
  const void* B;
  const void* C;
  const float* A;
  const float* D;         // nullable
  const float* bias;      // nullable
  const float* h0;        // nullable (scan only)
  void* out;
  float* state;           // scan: last_state (nullable); decode: the state, in place
  // Scans cut into time chunks (n_chunks > 1) only:
  float* ws_state;        // [batch, n_chunks, nheads, headdim, d_state]: pass A's end states; after the
                          // carry, slot k holds the state entering chunk k + 1
  float* ws_decay;        // [batch, n_chunks, nheads]: a chunk's summed log2 decay, sum of dt A log2(e)
  int64_t seqlen;
  int64_t chunk_len;      // steps per time chunk: a multiple of 32 unless n_chunks == 1
  int32_t n_chunks;
  int32_t batch;
  int32_t nheads;
  int32_t headdim;
  int32_t ngroups;
  int32_t d_state;
  int32_t softplus;
  int32_t cus;            // compute units of the device
  int32_t fair;           // set by the launcher: the whole grid is co-resident
};

// Backward of the scan.  Elementwise gradients and dout share one dtype.
struct BwdArgs {
  const void* x;
  const void* delta;
  const void* z;          // nullable
  const void* B;
  const void* C;
  const float* A;
  const float* D;         // nullable
  const float* bias;      // nullable
  const float* h0;        // nullable
  const void* dout;
  const float* dlast;     // nullable
  void* dx;
  void* ddelta;
  void* dz;               // non-null iff z is
  float* ws_ckpt;         // [batch, nblk, ntiles, 64, 16] states entering each tile
  float* ws_bc;           // [batch, seqlen, nblk, 2, 16] per-block dB (before the ln 2), dC
  float* ws_a;            // [batch, d_inner, 16] per-row dA
  float* ws_dd;           // [batch, d_inner, 2] per-row dD, dbias
  float* dh0;             // nullable: [batch, d_inner, 16]
  // Chunked runs (n_chunks > 1) only, each [batch, n_chunks, d_inner, ...]:
  float* ws_hin;          // [.., 16] slot k: the state entering chunk k + 1 (forward pass A + carry)
  float* ws_fsum;         // [..] forward pass A's step-size sums
  float* ws_rev;          // [.., 16] slot k: dL/d(state entering chunk k) when none arrives at its end
  float* ws_rsum;         // [..] slot k: chunk k's step-size sum (log2 units)
  float* ws_dl;           // [.., 16] slot k: dL/d(state after chunk k), k < n_chunks - 1
  int32_t ckpt_given;     // ws_ckpt holds the forward's checkpoints already (ssm_scan_fwd_ckpt)
  int64_t seqlen;
  int64_t d_inner;
  int64_t chunk_len;      // steps per chunk: a multiple of kBwdTile unless n_chunks == 1
  int32_t n_chunks;
  int32_t batch;
  int32_t softplus;
  int32_t nblk;           // ceil(d_inner / 64)
  int32_t cus;            // compute units of the device
  int32_t fair;           // set by the launcher: the whole grid is co-resident
};

constexpr int kBwdTile = 8;  // steps per backward tile (and per checkpoint)

// Size of the fixed per-device scratch array that ssm_scan_fwd_noalloc uses
// in place of a stream-ordered workspace (scan.hip).
constexpr int64_t kScratchBytes = 32ll << 20;

// Launchers; each returns the hipGetLastError() of its launches.
hipError_t launch_scan(const ScanArgs& a, DT in, DT out, int states_per_wave, hipStream_t s);
// What launch_scan dispatches to: the kernel instances of one (input dtype,
// output dtype, input coefficient) each (scan_inst.hip), and the chunk carry
// pass they share.
hipError_t launch_scan_f32_f32(const ScanArgs& a, int states_per_wave, hipStream_t s);
hipError_t launch_scan_f32_bf16(const ScanArgs& a, int states_per_wave, hipStream_t s);
hipError_t launch_scan_bf16_f32(const ScanArgs& a, int states_per_wave, hipStream_t s);
hipError_t launch_scan_bf16_bf16(const ScanArgs& a, int states_per_wave, hipStream_t s);
hipError_t launch_scan_f32_f32_zoh(const ScanArgs& a, int states_per_wave, hipStream_t s);
hipError_t launch_scan_f32_bf16_zoh(const ScanArgs& a, int states_per_wave, hipStream_t s);
hipError_t launch_scan_bf16_f32_zoh(const ScanArgs& a, int states_per_wave, hipStream_t s);
hipError_t launch_scan_bf16_bf16_zoh(const ScanArgs& a, int states_per_wave, hipStream_t s);
hipError_t launch_carry(const ScanArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, DT in, DT out, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t s);
// The device address of the current device's copy of the fixed scratch array
// (kScratchBytes), looked up once per device.
hipError_t scratch_address(float** out);
// K is the filter width (2, 3 or 4).  The forward launch writes out, then
// (stream-ordered) the new cache; the update reads and rewrites the cache.
hipError_t launch_conv1d(const ConvArgs& a, DT in, DT out, int K, hipStream_t s);
hipError_t launch_conv1d_update(const ConvArgs& a, DT in, DT out, int K, hipStream_t s);
// Backward: the per-block kernel, then the fixed-order reductions into dA, dB,
// dC, dD and dbias (dD / dbias may be NULL when the forward had none).  With
// n_chunks > 1 it first runs the forward's pass A and carry (launch_scan with
// states_only) for each chunk's entering state, and the reverse pass A and
// reverse carry for the gradient arriving at each chunk's end.
hipError_t launch_scan_bwd(const BwdArgs& a, DT in, DT grad, float* dA, void* dB, void* dC, float* dD,
                           float* dbias, hipStream_t s);
// The SSD scan (bf16 inputs, headdim 64, d_state 64 or 128) and decode step.
hipError_t launch_ssd(const SsdArgs& a, DT out, hipStream_t s);
hipError_t launch_ssd_update(const SsdArgs& a, DT in, DT out, hipStream_t s);
hipError_t launch_affine_exclusive_scan(const float* a, const float* b, float* oa, float* ob,
                                        int64_t n, hipStream_t s);

}  // namespace ssm

// A host-only stand-in for the HIP runtime and for the kernel launchers of
// libssmscan, so that the C-ABI host layer (api.cpp) can be built with
// AddressSanitizer and UndefinedBehaviorSanitizer and run on a machine with no
// GPU.  Device memory is host memory here: hipMallocAsync is malloc.  Each
// launcher stub reads the first and the last byte of every buffer the host
// layer hands to that kernel, at the extent the kernel indexes (the layouts of
// internal.h), so a buffer or workspace the host layer sized too small is an
// out-of-bounds read that the sanitizer reports.  Nothing is computed.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "../../sequence_scan_amd/csrc/internal.h"

namespace {
int g_fail_alloc = 0;     // the next allocation fails (test of the error path)
long g_launches = 0;
long g_allocs = 0;
long g_frees = 0;

void touch(const char* what, const void* p, int64_t n, int64_t esize) {
  if (n <= 0) return;
  if (!p) {
    std::fprintf(stderr, "launcher got NULL %s for %lld elements\n", what, (long long)n);
    std::abort();
  }
  const volatile unsigned char* c = static_cast<const volatile unsigned char*>(p);
  (void)c[0];
  (void)c[n * esize - 1];
}
int64_t es(ssm::DT t) { return t == ssm::DT::F32 ? 4 : 2; }
}  // namespace

extern "C" {
void fake_fail_next_alloc(void) { g_fail_alloc = 1; }
long fake_launches(void) { return g_launches; }
long fake_live_allocs(void) { return g_allocs - g_frees; }

hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}
hipError_t hipMallocAsync(void** p, size_t bytes, hipStream_t) {
  if (g_fail_alloc) {
    g_fail_alloc = 0;
    *p = nullptr;
    return hipErrorOutOfMemory;
  }
  *p = std::malloc(bytes ? bytes : 1);
  if (!*p) return hipErrorOutOfMemory;
  ++g_allocs;
  return hipSuccess;
}
int g_pools = 0;
hipError_t hipMemPoolCreate(hipMemPool_t* pool, const hipMemPoolProps* props) {
  if (props->location.type != hipMemLocationTypeDevice || props->allocType != hipMemAllocationTypePinned)
    std::abort();
  static int dummy;
  *pool = reinterpret_cast<hipMemPool_t>(&dummy);
  ++g_pools;
  return hipSuccess;
}
hipError_t hipMemPoolSetAttribute(hipMemPool_t, hipMemPoolAttr, void*) { return hipSuccess; }
hipError_t hipMemPoolDestroy(hipMemPool_t) { return hipSuccess; }
hipError_t hipMemPoolTrimTo(hipMemPool_t, size_t) { return hipSuccess; }
hipError_t hipMallocFromPoolAsync(void** p, size_t bytes, hipMemPool_t, hipStream_t s) {
  return hipMallocAsync(p, bytes, s);
}
int hipGetStreamDeviceId(hipStream_t) { return 0; }
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* st) {
  *st = hipStreamCaptureStatusNone;
  return hipSuccess;
}
int fake_pools(void) { return g_pools; }
hipError_t hipFreeAsync(void* p, hipStream_t) {
  std::free(p);
  ++g_frees;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "fake runtime error"; }
}

namespace ssm {

hipError_t scratch_address(float** out) {
  static float* scratch = static_cast<float*>(std::malloc(kScratchBytes));
  *out = scratch;
  return hipSuccess;
}

hipError_t launch_scan(const ScanArgs& a, DT in, DT out, int states_per_wave, hipStream_t) {
  if (states_per_wave < 1 || states_per_wave > kDState || kDState % states_per_wave) std::abort();
  const int64_t rows = (int64_t)a.batch * a.seqlen, elems = rows * a.d_inner;
  if (a.n_chunks < 1 || a.chunk_len < 1 || (int64_t)a.n_chunks * a.chunk_len < a.seqlen ||
      (int64_t)(a.n_chunks - 1) * a.chunk_len >= a.seqlen) {
    std::fprintf(stderr, "inconsistent plan: %d chunks of %lld for %lld steps\n", a.n_chunks,
                 (long long)a.chunk_len, (long long)a.seqlen);
    std::abort();
  }
  touch("x", a.x, elems, es(in));
  touch("delta", a.delta, elems, es(in));
  touch("z", a.z, a.z ? elems : 0, es(in));
  touch("B", a.B, rows * kDState, es(in));
  touch("C", a.C, rows * kDState, es(in));
  touch("A", a.A, a.d_inner * kDState, 4);
  touch("D", a.D, a.D ? a.d_inner : 0, 4);
  touch("bias", a.bias, a.bias ? a.d_inner : 0, 4);
  if (!a.states_only) touch("out", a.out, elems, es(out));
  const int64_t states = (int64_t)a.batch * a.d_inner * kDState;
  touch("last_state", a.last_state, a.last_state ? states : 0, 4);
  touch("h0", a.h0, a.h0 ? states : 0, 4);
  if (a.n_chunks > 1) {
    touch("ws_state", a.ws_state, states * a.n_chunks, 4);
    touch("ws_dtsum", a.ws_dtsum, (int64_t)a.batch * a.n_chunks * a.d_inner, 4);
  }
  if (a.ckpt) {
    if (states_per_wave != 4 || a.ckpt_nblk != (a.d_inner + 63) / 64 || a.ckpt_tiles != (a.seqlen + 7) / 8 ||
        (a.n_chunks > 1 && a.chunk_len % 8 != 0))
      std::abort();
    touch("ckpt", a.ckpt, (int64_t)a.batch * a.ckpt_nblk * a.ckpt_tiles * 1024, 4);
  }
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, DT in, DT out, hipStream_t) {
  const int64_t batch = a.d_inner ? a.pairs / a.d_inner : 0;
  touch("state", a.state, a.pairs * kDState, 4);
  touch("x", a.x, a.pairs, es(in));
  touch("delta", a.delta, a.pairs, es(in));
  touch("z", a.z, a.z ? a.pairs : 0, es(in));
  touch("B", a.B, batch * kDState, es(in));
  touch("C", a.C, batch * kDState, es(in));
  touch("A", a.A, a.d_inner * kDState, 4);
  touch("D", a.D, a.D ? a.d_inner : 0, 4);
  touch("bias", a.bias, a.bias ? a.d_inner : 0, 4);
  touch("out", a.out, a.pairs, es(out));
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t) {
  touch("fill", p, n, 4);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t) {
  touch("copy dst", dst, n, 4);
  touch("copy src", src, n, 4);
  ++g_launches;
  return hipSuccess;
}

static void touch_conv(const ConvArgs& a, DT in, DT out, int K) {
  const int64_t elems = (int64_t)a.batch * a.seqlen * a.d_inner, st = (int64_t)a.batch * a.d_inner * K;
  touch("x", a.x, elems, es(in));
  touch("w", a.w, a.d_inner * K, 4);
  touch("bias", a.bias, a.bias ? a.d_inner : 0, 4);
  touch("state_in", a.state_in, a.state_in ? st : 0, es(in));
  touch("out", a.out, elems, es(out));
  touch("state_out", a.state_out, a.state_out ? st : 0, es(in));
}

hipError_t launch_conv1d(const ConvArgs& a, DT in, DT out, int K, hipStream_t) {
  touch_conv(a, in, out, K);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_conv1d_update(const ConvArgs& a, DT in, DT out, int K, hipStream_t) {
  if (a.seqlen != 1) std::abort();
  touch_conv(a, in, out, K);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_scan_bwd(const BwdArgs& a, DT in, DT grad, float* dA, void* dB, void* dC, float* dD,
                           float* dbias, hipStream_t) {
  const int64_t rows = (int64_t)a.batch * a.seqlen, elems = rows * a.d_inner;
  const int64_t states = (int64_t)a.batch * a.d_inner * kDState;
  const int64_t ntiles = (a.seqlen + kBwdTile - 1) / kBwdTile;
  if (a.nblk != (a.d_inner + 63) / 64) std::abort();
  touch("x", a.x, elems, es(in));
  touch("delta", a.delta, elems, es(in));
  touch("z", a.z, a.z ? elems : 0, es(in));
  touch("B", a.B, rows * kDState, es(in));
  touch("C", a.C, rows * kDState, es(in));
  touch("A", a.A, a.d_inner * kDState, 4);
  touch("D", a.D, a.D ? a.d_inner : 0, 4);
  touch("bias", a.bias, a.bias ? a.d_inner : 0, 4);
  touch("h0", a.h0, a.h0 ? states : 0, 4);
  touch("dout", a.dout, elems, es(grad));
  touch("dlast", a.dlast, a.dlast ? states : 0, 4);
  touch("dx", a.dx, elems, es(grad));
  touch("ddelta", a.ddelta, elems, es(grad));
  touch("dz", a.dz, a.z ? elems : 0, es(grad));
  touch("ws_ckpt", a.ws_ckpt, (int64_t)a.batch * a.nblk * ntiles * 64 * kDState, 4);
  touch("ws_bc", a.ws_bc, rows * a.nblk * 2 * kDState, 4);
  touch("ws_a", a.ws_a, states, 4);
  touch("ws_dd", a.ws_dd, (int64_t)a.batch * a.d_inner * 2, 4);
  touch("dh0", a.dh0, a.dh0 ? states : 0, 4);
  if (a.n_chunks > 1) {
    const int64_t cs = states * a.n_chunks, cd = (int64_t)a.batch * a.n_chunks * a.d_inner;
    touch("ws_hin", a.ws_hin, cs, 4);
    touch("ws_fsum", a.ws_fsum, cd, 4);
    touch("ws_rev", a.ws_rev, cs, 4);
    touch("ws_rsum", a.ws_rsum, cd, 4);
    touch("ws_dl", a.ws_dl, cs, 4);
  }
  touch("dA", dA, a.d_inner * kDState, 4);
  touch("dB", dB, rows * kDState, es(grad));
  touch("dC", dC, rows * kDState, es(grad));
  touch("dD", dD, a.D ? a.d_inner : 0, 4);
  touch("dbias", dbias, a.bias ? a.d_inner : 0, 4);
  ++g_launches;
  return hipSuccess;
}

static void touch_ssd(const SsdArgs& a, DT in, DT out, bool decode) {
  const int64_t L = decode ? 1 : a.seqlen;
  const int64_t tok = (int64_t)a.batch * L, ch = (int64_t)a.nheads * a.headdim;
  const int64_t states = (int64_t)a.batch * ch * a.d_state;
  touch("x", a.x, tok * ch, es(in));
  touch("dt", a.dt, tok * a.nheads, es(in));
  touch("z", a.z, a.z ? tok * ch : 0, es(in));
  touch("B", a.B, tok * a.ngroups * a.d_state, es(in));
  touch("C", a.C, tok * a.ngroups * a.d_state, es(in));
  touch("A", a.A, a.nheads, 4);
  touch("D", a.D, a.D ? ch : 0, 4);
  touch("bias", a.bias, a.bias ? a.nheads : 0, 4);
  touch("h0", a.h0, a.h0 ? states : 0, 4);
  touch("out", a.out, tok * ch, es(out));
  touch("state", a.state, a.state ? states : 0, 4);
  if (!decode && a.n_chunks > 1) {
    if (a.chunk_len % 32) std::abort();
    touch("ws_state", a.ws_state, states * a.n_chunks, 4);
    touch("ws_decay", a.ws_decay, (int64_t)a.batch * a.n_chunks * a.nheads, 4);
  }
}

hipError_t launch_ssd(const SsdArgs& a, DT out, hipStream_t) {
  touch_ssd(a, DT::BF16, out, false);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_ssd_update(const SsdArgs& a, DT in, DT out, hipStream_t) {
  touch_ssd(a, in, out, true);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_affine_exclusive_scan(const float* a, const float* b, float* oa, float* ob, int64_t n,
                                        hipStream_t) {
  touch("a", a, n, 4);
  touch("b", b, n, 4);
  touch("out_a", oa, n, 4);
  touch("out_b", ob, n, 4);
  ++g_launches;
  return hipSuccess;
}

}  // namespace ssm

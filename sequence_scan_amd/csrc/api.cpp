// C-ABI host layer of libssmscan: argument checks, plan choice, workspace,
// launches.  Every check runs before anything is enqueued; on any non-OK
// status nothing has been enqueued and no output has been written.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/ssmscan.h"
#include "internal.h"

namespace {

thread_local std::string g_last_error;

ssm_status fail(ssm_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

ssm_status ok() {
  return SSM_OK;
}

// A failed HIP runtime call also records its error as the calling thread's
// last error, which the launchers read back after their launches.  Once a
// call has reported such a failure itself, it clears that record, so the
// failure is not reported a second time by a later, valid call.
ssm_status fail_hip(const char* what, long long bytes, hipError_t e) {
  (void)hipGetLastError();
  if (bytes >= 0) return fail(SSM_ERR_HIP, "%s(%lld bytes) failed: %s", what, bytes, hipGetErrorString(e));
  return fail(SSM_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

// Workspace memory.  A stream-ordered allocation from a device's default pool
// goes back to the system at the next synchronisation (that pool's release
// threshold is 0), so every call that follows one maps its workspace again:
// measured on MI355X, 21 ms for the 840 MB of the Mamba-2.8B-like layer's
// backward, ten times the kernels.  The library therefore allocates from a
// pool of its own per device whose freed memory stays reserved for the next
// call (ssm_trim_workspace hands it back).  Under stream capture the
// allocation is the stream's own (hipMallocAsync): the graph then owns it.
constexpr int kMaxDevices = 64;
std::mutex g_pool_mu;
hipMemPool_t g_pool[kMaxDevices] = {};
bool g_pool_tried[kMaxDevices] = {};

int stream_device(hipStream_t s) {
  if (s != nullptr) {
    const int d = hipGetStreamDeviceId(s);
    if (d >= 0) return d;
    (void)hipGetLastError();
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return dev;
}

// The library's pool on `dev` (created on first use), or nullptr where the
// device offers none; then workspaces come from the default pool.
hipMemPool_t workspace_pool(int dev, bool create) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_pool_mu);
  if (create && !g_pool_tried[dev]) {
    g_pool_tried[dev] = true;
    hipMemPoolProps props{};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    if (hipMemPoolCreate(&pool, &props) == hipSuccess && pool != nullptr) {
      uint64_t keep = UINT64_MAX;
      if (hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep) == hipSuccess) g_pool[dev] = pool;
      else (void)hipMemPoolDestroy(pool);
    }
    (void)hipGetLastError();
  }
  return g_pool[dev];
}

hipError_t ws_alloc(void** p, int64_t bytes, hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    cs = hipStreamCaptureStatusNone;
  }
  if (cs == hipStreamCaptureStatusNone) {
    if (hipMemPool_t pool = workspace_pool(stream_device(s), true))
      return hipMallocFromPoolAsync(p, (size_t)bytes, pool, s);
  }
  return hipMallocAsync(p, (size_t)bytes, s);
}

struct Range {
  const char* name;
  uintptr_t lo;
  uintptr_t hi;  // exclusive
};

Range range(const char* name, const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, p ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool overlaps(const Range& a, const Range& b) {
  if (a.lo == 0 || b.lo == 0 || a.hi == a.lo || b.hi == b.lo) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool mul_ok(int64_t a, int64_t b, int64_t* r) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *r = a * b;
  return true;
}

int64_t esize(ssm_dtype t) { return t == SSM_BF16 ? 2 : 4; }

bool valid_dtype(ssm_dtype t) { return t == SSM_F32 || t == SSM_BF16; }

ssm::DT to_dt(ssm_dtype t) { return t == SSM_BF16 ? ssm::DT::BF16 : ssm::DT::F32; }

ssm_status check_align(const char* name, const void* p, uintptr_t bytes = 16) {
  if (p != nullptr && (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) != 0)
    return fail(SSM_ERR_UNSUPPORTED, "%s is not %d-byte aligned", name, (int)bytes);
  return SSM_OK;
}

int device_simds() {
  int dev = 0;
  int cus = 0;
  // without a device the planner assumes MI355X's 256 CUs; the failed query's
  // error record is cleared (see fail_hip)
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return 1024;
  }
  return cus * 4;
}

// The plan (from measurements on MI355X): 4 states per wave (a workgroup of
// 4 wavefronts per 64 channels) is the fastest split on every workload
// measured.  When the channel blocks give fewer than half a wavefront per
// SIMD, the sequence is also cut into chunks until there are about 12
// wavefronts per SIMD, with chunks of at least 1024 steps: the extra
// reduction pass costs less than idle SIMDs.  With more blocks than that but
// fewer than one per CU, some CUs would idle: the sequence is cut so that the
// grid holds about three workgroups per CU (the kernel's occupancy), with
// chunks of at least 512 steps.  Chunk lengths are rounded up to the 32-step
// tile.  (The Mamba-130M-like layer, 192 blocks: 4 chunks of 512 steps, 179 us
// against 196 us in one chunk and 189-230 us for chunks of 192 to 1024 steps;
// the long single row: 96 chunks of 2752 steps, 3.26 ms, with chunks of 1024
// to 8192 steps within 3 %.)
void choose_plan(int64_t batch, int64_t seqlen, int64_t d_inner, int simds, ssm_plan* p) {
  const int64_t blocks = batch * ((d_inner + 63) / 64);
  const int64_t waves = std::max<int64_t>(1, blocks * 4);
  const int64_t cus = std::max(1, simds / 4);
  int64_t chunks = 1;
  if (waves < simds / 2) {
    chunks = (12 * (int64_t)simds + waves - 1) / waves;
    chunks = std::min(chunks, std::max<int64_t>(1, seqlen / 1024));
  } else if (blocks < cus) {
    chunks = (3 * cus + blocks - 1) / blocks;
    chunks = std::min(chunks, std::max<int64_t>(1, seqlen / 512));
  }
  int64_t chunk_len = seqlen > 0 ? (seqlen + chunks - 1) / chunks : 1;
  // a cut sequence is cut at multiples of the kernel's 32-step tile, so that
  // only the last chunk can have a ragged tile
  if (chunks > 1) chunk_len = (chunk_len + 31) / 32 * 32;
  if (chunk_len < 1) chunk_len = 1;
  p->states_per_wave = 4;
  p->reserved0 = 0;
  p->chunk_len = chunk_len;
  p->n_chunks = seqlen > 0 ? (seqlen + chunk_len - 1) / chunk_len : 0;
  for (auto& r : p->reserved) r = 0;
}

// The backward's plan (from measurements on MI355X).  Its workgroup holds 64
// channels of one batch row for a whole chunk, three workgroups per CU.  With
// at most 1.75 channel blocks per CU the sequence is cut into chunks (a
// multiple of the 8-step tile, at least 512 steps) until there are about 24
// workgroups per CU.  Cutting at all costs a forward pass A and a reverse pass
// A over the sequence, about 45 % of the backward's own work, whatever the
// number of chunks; more, shorter chunks then only balance the CUs better.
// Measured against one chunk: 448 blocks 1.67 against 1.74 ms, 320 blocks
// 1.22 against 1.70 ms, the Mamba-130M-like layer (192 blocks) 0.75 against
// 1.51 ms, the long single-row sequence (32 blocks, 262144 steps) 13.5 ms in
// chunks of 1024 steps against 14.6 ms in chunks of 10928 and 184 ms in one.
// At 512 blocks two chunks were slower (2.00 against 1.77 ms).
// Bytes of the backward's checkpoints: the state entering every 8-step tile,
// [batch, ceil(d_inner / 64), ceil(seqlen / 8), 64, 16] fp32.
ssm_status ckpt_size(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t* bytes) {
  const int64_t nblk = (d_inner + 63) / 64, ntiles = (seqlen + ssm::kBwdTile - 1) / ssm::kBwdTile;
  int64_t n;
  if (!mul_ok(batch * nblk, ntiles * 64 * ssm::kDState, &n) || !mul_ok(n, 4, bytes))
    return fail(SSM_ERR_BAD_SHAPE, "checkpoint size overflows int64");
  return SSM_OK;
}

void choose_bwd_plan(int64_t batch, int64_t seqlen, int64_t d_inner, int simds, ssm_plan* p) {
  const int64_t blocks = std::max<int64_t>(1, batch * ((d_inner + 63) / 64));
  const int64_t cus = std::max(1, simds / 4);
  int64_t chunks = 1;
  if (4 * blocks <= 7 * cus) {
    chunks = (24 * cus + blocks - 1) / blocks;
    chunks = std::min(chunks, std::max<int64_t>(1, seqlen / 512));
  }
  int64_t chunk_len = seqlen > 0 ? (seqlen + chunks - 1) / chunks : 1;
  if (chunks > 1) chunk_len = (chunk_len + ssm::kBwdTile - 1) / ssm::kBwdTile * ssm::kBwdTile;
  if (chunk_len < 1) chunk_len = 1;
  p->states_per_wave = 4;
  p->reserved0 = 0;
  p->chunk_len = chunk_len;
  p->n_chunks = seqlen > 0 ? (seqlen + chunk_len - 1) / chunk_len : 0;
  for (auto& r : p->reserved) r = 0;
}

// The Mamba-2 scan's plan.  Its workgroup walks one (batch row, head) through
// the sequence; with at most 1.75 such workgroups per CU the sequence is cut
// into time chunks (a multiple of the 32-step matrix chunk, at least 1024
// steps) until there are about 12 workgroups per CU.  Each cut costs a pass A
// (the chunk's state update alone, about half the scan's work per step) and
// a carry over the chunks.
void choose_ssd_plan(int64_t batch, int64_t seqlen, int64_t nheads, int simds, ssm_plan* p) {
  const int64_t wgs = std::max<int64_t>(1, batch * nheads);
  const int64_t cus = std::max(1, simds / 4);
  int64_t chunks = 1;
  if (4 * wgs <= 7 * cus) {
    chunks = (12 * cus + wgs - 1) / wgs;
    chunks = std::min(chunks, std::max<int64_t>(1, seqlen / 1024));
  }
  int64_t chunk_len = seqlen > 0 ? (seqlen + chunks - 1) / chunks : 1;
  if (chunks > 1) chunk_len = (chunk_len + 31) / 32 * 32;
  if (chunk_len < 1) chunk_len = 1;
  p->states_per_wave = 0;
  p->reserved0 = 0;
  p->chunk_len = chunk_len;
  p->n_chunks = seqlen > 0 ? (seqlen + chunk_len - 1) / chunk_len : 0;
  for (auto& r : p->reserved) r = 0;
}

struct Sizes {
  int64_t elems;      // batch * seqlen * d_inner
  int64_t bc;         // batch * seqlen * d_state
  int64_t state;      // batch * d_inner * d_state
};

ssm_status check_common(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                        ssm_dtype in_dtype, ssm_dtype out_dtype, Sizes* sz) {
  if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state < 0)
    return fail(SSM_ERR_BAD_SHAPE, "negative size (batch=%lld seqlen=%lld d_inner=%lld d_state=%lld)",
                (long long)batch, (long long)seqlen, (long long)d_inner, (long long)d_state);
  if (d_state != ssm::kDState)
    return fail(SSM_ERR_UNSUPPORTED, "d_state=%lld is not supported (this build supports 16)", (long long)d_state);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(SSM_ERR_UNSUPPORTED, "unknown dtype (in=%d out=%d)", (int)in_dtype, (int)out_dtype);
  int64_t t1, t2;
  if (!mul_ok(batch, seqlen, &t1) || !mul_ok(t1, d_inner, &sz->elems) || !mul_ok(sz->elems, 8, &t2) ||
      !mul_ok(t1, d_state, &sz->bc) || !mul_ok(batch, d_inner, &t2) || !mul_ok(t2, d_state, &sz->state) ||
      !mul_ok(sz->state, 8, &t1))
    return fail(SSM_ERR_BAD_SHAPE, "element count overflows int64");
  if (batch > 65535) return fail(SSM_ERR_UNSUPPORTED, "batch=%lld exceeds 65535", (long long)batch);
  return SSM_OK;
}

ssm_status conv_check(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_conv, ssm_dtype in_dtype,
                      ssm_dtype out_dtype) {
  if (batch < 0 || seqlen < 0 || d_inner < 0 || d_conv < 0)
    return fail(SSM_ERR_BAD_SHAPE, "negative size (batch=%lld seqlen=%lld d_inner=%lld d_conv=%lld)",
                (long long)batch, (long long)seqlen, (long long)d_inner, (long long)d_conv);
  if (d_conv < 2 || d_conv > 4)
    return fail(SSM_ERR_UNSUPPORTED, "d_conv=%lld is not supported (2, 3 or 4)", (long long)d_conv);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(SSM_ERR_UNSUPPORTED, "unknown dtype (in=%d out=%d)", (int)in_dtype, (int)out_dtype);
  int64_t t1, t2;
  if (!mul_ok(batch, seqlen, &t1) || !mul_ok(t1, d_inner, &t2) || !mul_ok(t2, 8, &t1) ||
      !mul_ok(batch, d_inner, &t1) || !mul_ok(t1, d_conv * 8, &t2))
    return fail(SSM_ERR_BAD_SHAPE, "element count overflows int64");
  if (batch > 65535) return fail(SSM_ERR_UNSUPPORTED, "batch=%lld exceeds 65535", (long long)batch);
  return SSM_OK;
}

// The step flags word: SSM_SOFTPLUS and SSM_ZOH are its only bits.
ssm_status check_flags(int flags, bool allow_zoh) {
  if ((flags & ~(SSM_SOFTPLUS | SSM_ZOH)) != 0)
    return fail(SSM_ERR_UNSUPPORTED, "step flags %d: only SSM_SOFTPLUS (1) and SSM_ZOH (2) are defined", flags);
  if (!allow_zoh && (flags & SSM_ZOH) != 0)
    return fail(SSM_ERR_UNSUPPORTED, "the backward is defined for the dt input coefficient only, not SSM_ZOH");
  return SSM_OK;
}

ssm_status scan_impl(const void* x, const void* delta, const float* A, const void* B, const void* C,
                     const float* D, const void* z, const float* delta_bias, int softplus, const float* h0,
                     void* out, float* last_state, int64_t batch, int64_t seqlen, int64_t d_inner,
                     int64_t d_state, ssm_dtype in_dtype, ssm_dtype out_dtype, void* stream,
                     const ssm_plan* plan_in, bool fixed_scratch = false, float* ckpt = nullptr) {
  Sizes sz;
  ssm_status st = check_common(batch, seqlen, d_inner, d_state, in_dtype, out_dtype, &sz);
  if (st != SSM_OK) return st;
  if ((st = check_flags(softplus, true)) != SSM_OK) return st;
  int64_t ckpt_bytes = 0;
  if (ckpt != nullptr) {
    if (softplus & SSM_ZOH) return fail(SSM_ERR_UNSUPPORTED, "checkpoints are for the backward, which rejects SSM_ZOH");
    if ((st = ckpt_size(batch, seqlen, d_inner, &ckpt_bytes)) != SSM_OK) return st;
  }
  // a required pointer may be NULL only when its tensor is empty
  const bool need_e = sz.elems > 0, need_bc = sz.bc > 0, need_a = d_inner > 0;
  if ((need_e && (!x || !delta || !out)) || (need_a && !A) || (need_bc && (!B || !C))) {
    const char* which = (need_e && !x) ? "x" : (need_e && !delta) ? "delta" : (need_a && !A) ? "A"
                      : (need_bc && !B) ? "B" : (need_bc && !C) ? "C" : "out";
    return fail(SSM_ERR_NULL_ARG, "required pointer %s is NULL", which);
  }
  const void* ptrs[] = {x, delta, A, B, C, D, z, delta_bias, out, last_state, h0, ckpt};
  const char* names[] = {"x", "delta", "A", "B", "C", "D", "z", "delta_bias", "out", "last_state",
                         "initial_state", "ckpt"};
  for (int i = 0; i < 12; ++i)
    if ((st = check_align(names[i], ptrs[i])) != SSM_OK) return st;
  const int64_t si = esize(in_dtype), so = esize(out_dtype);
  const Range ins[] = {
      range("x", x, sz.elems * si),          range("delta", delta, sz.elems * si),
      range("z", z, sz.elems * si),          range("B", B, sz.bc * si),
      range("C", C, sz.bc * si),             range("A", A, d_inner * d_state * 4),
      range("D", D, d_inner * 4),            range("delta_bias", delta_bias, d_inner * 4),
  };
  const Range ro = range("out", out, sz.elems * so);
  const Range rl = range("last_state", last_state, sz.state * 4);
  const Range rh = range("initial_state", h0, sz.state * 4);
  for (const Range& r : ins) {
    if (overlaps(ro, r)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps input %s", r.name);
    if (overlaps(rl, r)) return fail(SSM_ERR_UNSUPPORTED, "last_state overlaps input %s", r.name);
  }
  if (overlaps(ro, rl)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps last_state");
  if (overlaps(ro, rh)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps initial_state");
  // the final state may replace the initial one in place, but not overlap it otherwise
  const bool h0_in_place = h0 != nullptr && static_cast<const void*>(h0) == static_cast<const void*>(last_state);
  if (!h0_in_place && overlaps(rl, rh)) return fail(SSM_ERR_UNSUPPORTED, "last_state partly overlaps initial_state");
  const Range rc = range("ckpt", ckpt, ckpt_bytes);
  for (const Range& r : ins)
    if (overlaps(rc, r)) return fail(SSM_ERR_UNSUPPORTED, "ckpt overlaps input %s", r.name);
  if (overlaps(rc, ro) || overlaps(rc, rl) || overlaps(rc, rh))
    return fail(SSM_ERR_UNSUPPORTED, "ckpt overlaps out, last_state or initial_state");

  ssm_plan plan;
  if (plan_in) {
    plan = *plan_in;
    const int ns = plan.states_per_wave;
    if (ns != 1 && ns != 2 && ns != 4 && ns != 8 && ns != 16)
      return fail(SSM_ERR_UNSUPPORTED, "plan.states_per_wave=%d not in {1,2,4,8,16}", ns);
    if (plan.chunk_len < 1) return fail(SSM_ERR_UNSUPPORTED, "plan.chunk_len must be >= 1");
    plan.n_chunks = seqlen > 0 ? (seqlen + plan.chunk_len - 1) / plan.chunk_len : 0;
    if (plan.n_chunks > 65535) return fail(SSM_ERR_UNSUPPORTED, "plan gives more than 65535 chunks");
  } else {
    choose_plan(batch, seqlen, d_inner, device_simds(), &plan);
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (batch == 0 || d_inner == 0) return ok();
  if (seqlen == 0) {
    if (last_state && !h0_in_place) {
      hipError_t e = h0 ? ssm::launch_copy_f32(last_state, h0, sz.state, s)
                        : ssm::launch_fill_zero(last_state, sz.state, s);
      if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    }
    return ok();
  }

  ssm::ScanArgs a{};
  a.x = x;
  a.delta = delta;
  a.z = z;
  a.B = B;
  a.C = C;
  a.A = A;
  a.D = D;
  a.bias = delta_bias;
  a.out = out;
  a.last_state = last_state;
  a.h0 = h0;
  a.seqlen = seqlen;
  a.d_inner = d_inner;
  a.chunk_len = plan.chunk_len;
  a.n_chunks = (int32_t)plan.n_chunks;
  a.softplus = (softplus & SSM_SOFTPLUS) ? 1 : 0;
  a.zoh = (softplus & SSM_ZOH) ? 1 : 0;
  a.batch = (int32_t)batch;
  a.cus = device_simds() / 4;
  if (ckpt != nullptr) {  // the default plan: 4 states per wavefront, chunks of a multiple of 32 steps
    a.ckpt = ckpt;
    a.ckpt_nblk = (int32_t)((d_inner + 63) / 64);
    a.ckpt_tiles = (seqlen + ssm::kBwdTile - 1) / ssm::kBwdTile;
  }

  void* ws = nullptr;       // a stream-ordered allocation, freed below
  hipError_t e = hipSuccess;
  if (plan.n_chunks > 1) {
    // With several chunks, the workgroups that read the initial state are not
    // the ones that write the final state: an in-place initial state is read
    // from a copy in the workspace.
    const int64_t n_h0 = h0_in_place ? sz.state : 0;
    int64_t n_state, n_sum, bytes;
    if (!mul_ok(batch * plan.n_chunks, d_inner * d_state, &n_state) ||
        !mul_ok(batch * plan.n_chunks, d_inner, &n_sum) || !mul_ok(n_state + n_sum + n_h0, 4, &bytes))
      return fail(SSM_ERR_BAD_SHAPE, "workspace size overflows int64");
    float* base = nullptr;
    if (fixed_scratch) {
      // Every slot the passes read is written first in stream order (pass A,
      // the carry, the initial-state copy), so the array needs no clearing.
      if (bytes > ssm::kScratchBytes)
        return fail(SSM_ERR_UNSUPPORTED, "the plan's carry workspace needs %lld bytes; the fixed scratch holds %lld",
                    (long long)bytes, (long long)ssm::kScratchBytes);
      e = ssm::scratch_address(&base);
      if (e != hipSuccess) return fail_hip("looking up the fixed scratch", -1, e);
    } else {
      e = ws_alloc(&ws, bytes, s);
      if (e != hipSuccess || ws == nullptr)
        return fail_hip("workspace allocation", (long long)bytes, e);
      base = static_cast<float*>(ws);
    }
    a.ws_state = base;
    a.ws_dtsum = a.ws_state + n_state;
    if (n_h0 > 0) {
      float* copy = a.ws_dtsum + n_sum;
      e = ssm::launch_copy_f32(copy, h0, n_h0, s);
      a.h0 = copy;
    }
  }
  if (e == hipSuccess) e = ssm::launch_scan(a, to_dt(in_dtype), to_dt(out_dtype), plan.states_per_wave, s);
  if (ws) {
    hipError_t e2 = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Sizes of the Mamba-2 (SSD) calls.
struct SsdSizes {
  int64_t elems;   // batch * seqlen * nheads * headdim
  int64_t steps;   // batch * seqlen * nheads (dt)
  int64_t bc;      // batch * seqlen * ngroups * d_state
  int64_t state;   // batch * nheads * headdim * d_state
};

ssm_status ssd_check(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                     int64_t d_state, ssm_dtype in_dtype, ssm_dtype out_dtype, int flags, bool scan, SsdSizes* sz) {
  if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 0 || ngroups < 0 || d_state < 0)
    return fail(SSM_ERR_BAD_SHAPE, "negative size (batch=%lld seqlen=%lld nheads=%lld headdim=%lld ngroups=%lld "
                "d_state=%lld)", (long long)batch, (long long)seqlen, (long long)nheads, (long long)headdim,
                (long long)ngroups, (long long)d_state);
  if (ngroups < 1 || nheads < 1 || nheads % ngroups != 0)
    return fail(SSM_ERR_UNSUPPORTED, "nheads=%lld must be a positive multiple of ngroups=%lld", (long long)nheads,
                (long long)ngroups);
  if (d_state != 64 && d_state != 128)
    return fail(SSM_ERR_UNSUPPORTED, "d_state=%lld is not supported (64 or 128)", (long long)d_state);
  if (scan && headdim != 64) return fail(SSM_ERR_UNSUPPORTED, "headdim=%lld is not supported (64)", (long long)headdim);
  if (!scan && headdim < 1) return fail(SSM_ERR_UNSUPPORTED, "headdim=%lld must be positive", (long long)headdim);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(SSM_ERR_UNSUPPORTED, "unknown dtype (in=%d out=%d)", (int)in_dtype, (int)out_dtype);
  if (scan && in_dtype != SSM_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "the SSD scan takes bf16 inputs (its products run on bf16 matrix cores)");
  if ((flags & ~SSM_SOFTPLUS) != 0)
    return fail(SSM_ERR_UNSUPPORTED, "step flags %d: the SSD calls take SSM_SOFTPLUS only", flags);
  int64_t t1, t2, t3;
  if (!mul_ok(batch, seqlen, &t1) || !mul_ok(t1, nheads, &sz->steps) || !mul_ok(sz->steps, headdim, &sz->elems) ||
      !mul_ok(sz->elems, 8, &t2) || !mul_ok(t1, ngroups * d_state, &sz->bc) || !mul_ok(batch, nheads, &t2) ||
      !mul_ok(t2, headdim * d_state, &sz->state) || !mul_ok(sz->state, 8, &t3))
    return fail(SSM_ERR_BAD_SHAPE, "element count overflows int64");
  if (batch > 65535) return fail(SSM_ERR_UNSUPPORTED, "batch=%lld exceeds 65535", (long long)batch);
  // the decode grid and the carry of a chunked scan have one workgroup row per
  // head, and the scan kernel addresses one 32-step chunk of a tensor with
  // 32-bit byte offsets, which at most 65535 heads keep below 2^31
  if (nheads > 65535) return fail(SSM_ERR_UNSUPPORTED, "nheads=%lld exceeds 65535", (long long)nheads);
  if (nheads > INT32_MAX || headdim > INT32_MAX || ngroups > INT32_MAX)
    return fail(SSM_ERR_UNSUPPORTED, "nheads, headdim and ngroups must fit in 32 bits");
  return SSM_OK;
}

}  // namespace

extern "C" {

ssm_status ssm_scan_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                        const float* D, const void* z, const float* delta_bias, int softplus, void* out,
                        float* last_state, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                        ssm_dtype in_dtype, ssm_dtype out_dtype, void* stream) {
  return scan_impl(x, delta, A, B, C, D, z, delta_bias, softplus, nullptr, out, last_state, batch, seqlen,
                   d_inner, d_state, in_dtype, out_dtype, stream, nullptr);
}

ssm_status ssm_scan_fwd_plan(const void* x, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, int softplus, void* out,
                             float* last_state, int64_t batch, int64_t seqlen, int64_t d_inner,
                             int64_t d_state, ssm_dtype in_dtype, ssm_dtype out_dtype, void* stream,
                             const ssm_plan* plan) {
  if (!plan) return fail(SSM_ERR_NULL_ARG, "plan is NULL");
  return scan_impl(x, delta, A, B, C, D, z, delta_bias, softplus, nullptr, out, last_state, batch, seqlen,
                   d_inner, d_state, in_dtype, out_dtype, stream, plan);
}

ssm_status ssm_scan_fwd_from(const void* x, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, int softplus,
                             const float* initial_state, void* out, float* last_state, int64_t batch,
                             int64_t seqlen, int64_t d_inner, int64_t d_state, ssm_dtype in_dtype,
                             ssm_dtype out_dtype, void* stream, const ssm_plan* plan) {
  return scan_impl(x, delta, A, B, C, D, z, delta_bias, softplus, initial_state, out, last_state, batch, seqlen,
                   d_inner, d_state, in_dtype, out_dtype, stream, plan);
}

static_assert(ssm::kScratchBytes == SSM_NOALLOC_SCRATCH_BYTES, "the header states the fixed scratch size");

ssm_status ssm_scan_fwd_noalloc(const void* x, const void* delta, const float* A, const void* B, const void* C,
                                const float* D, const void* z, const float* delta_bias, int softplus,
                                const float* initial_state, void* out, float* last_state, int64_t batch,
                                int64_t seqlen, int64_t d_inner, int64_t d_state, ssm_dtype in_dtype,
                                ssm_dtype out_dtype, void* stream, const ssm_plan* plan) {
  return scan_impl(x, delta, A, B, C, D, z, delta_bias, softplus, initial_state, out, last_state, batch, seqlen,
                   d_inner, d_state, in_dtype, out_dtype, stream, plan, true);
}

ssm_status ssm_scan_plan(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state, ssm_plan* plan) {
  if (!plan) return fail(SSM_ERR_NULL_ARG, "plan is NULL");
  Sizes sz;
  ssm_status st = check_common(batch, seqlen, d_inner, d_state, SSM_F32, SSM_F32, &sz);
  if (st != SSM_OK) return st;
  choose_plan(batch, seqlen, d_inner, device_simds(), plan);
  return SSM_OK;
}

ssm_status ssm_state_update(float* state, const void* x, const void* delta, const float* A, const void* B,
                            const void* C, const float* D, const void* z, const float* delta_bias, int softplus,
                            void* out, int64_t batch, int64_t d_inner, int64_t d_state, ssm_dtype in_dtype,
                            ssm_dtype out_dtype, void* stream) {
  Sizes sz;
  ssm_status st = check_common(batch, 1, d_inner, d_state, in_dtype, out_dtype, &sz);
  if (st != SSM_OK) return st;
  if ((st = check_flags(softplus, true)) != SSM_OK) return st;
  const bool need_e = sz.elems > 0, need_bc = sz.bc > 0, need_a = d_inner > 0;
  if ((need_e && (!state || !x || !delta || !out)) || (need_a && !A) || (need_bc && (!B || !C))) {
    const char* which = (need_e && !state) ? "state" : (need_e && !x) ? "x" : (need_e && !delta) ? "delta"
                      : (need_a && !A) ? "A" : (need_bc && !B) ? "B" : (need_bc && !C) ? "C" : "out";
    return fail(SSM_ERR_NULL_ARG, "required pointer %s is NULL", which);
  }
  const void* ptrs[] = {state, x, delta, A, B, C, D, z, delta_bias, out};
  const char* names[] = {"state", "x", "delta", "A", "B", "C", "D", "z", "delta_bias", "out"};
  for (int i = 0; i < 10; ++i)
    if ((st = check_align(names[i], ptrs[i])) != SSM_OK) return st;
  const int64_t si = esize(in_dtype), so = esize(out_dtype);
  const Range ins[] = {
      range("x", x, sz.elems * si),       range("delta", delta, sz.elems * si),
      range("z", z, sz.elems * si),       range("B", B, sz.bc * si),
      range("C", C, sz.bc * si),          range("A", A, d_inner * d_state * 4),
      range("D", D, d_inner * 4),         range("delta_bias", delta_bias, d_inner * 4),
  };
  const Range rs = range("state", state, sz.state * 4);
  const Range ro = range("out", out, sz.elems * so);
  for (const Range& r : ins) {
    if (overlaps(ro, r)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps input %s", r.name);
    if (overlaps(rs, r)) return fail(SSM_ERR_UNSUPPORTED, "state overlaps input %s", r.name);
  }
  if (overlaps(ro, rs)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps state");
  if (batch == 0 || d_inner == 0) return ok();
  ssm::DecodeArgs a{};
  a.state = state;
  a.x = x;
  a.delta = delta;
  a.z = z;
  a.B = B;
  a.C = C;
  a.A = A;
  a.D = D;
  a.bias = delta_bias;
  a.out = out;
  a.d_inner = d_inner;
  a.pairs = batch * d_inner;
  a.softplus = (softplus & SSM_SOFTPLUS) ? 1 : 0;
  a.zoh = (softplus & SSM_ZOH) ? 1 : 0;
  hipError_t e = ssm::launch_decode(a, to_dt(in_dtype), to_dt(out_dtype), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

static ssm_status bwd_impl(const void* x, const void* delta, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* delta_bias, int softplus,
                           const float* initial_state, const void* dout, const float* dlast_state, void* dx,
                           void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                           float* dinitial_state, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                           ssm_dtype in_dtype, ssm_dtype grad_dtype, void* stream, const ssm_plan* plan_in,
                           const float* ckpt_in = nullptr) {
  Sizes sz;
  ssm_status st = check_common(batch, seqlen, d_inner, d_state, in_dtype, grad_dtype, &sz);
  if (st != SSM_OK) return st;
  if ((st = check_flags(softplus, false)) != SSM_OK) return st;
  const bool need_e = sz.elems > 0, need_bc = sz.bc > 0, need_a = d_inner > 0;
  struct Req { const char* name; const void* p; bool need; };
  const Req req[] = {{"x", x, need_e}, {"delta", delta, need_e}, {"dout", dout, need_e}, {"dx", dx, need_e},
                     {"ddelta", ddelta, need_e}, {"A", A, need_a}, {"dA", dA, need_a}, {"B", B, need_bc},
                     {"C", C, need_bc}, {"dB", dB, need_bc}, {"dC", dC, need_bc},
                     {"dD", dD, need_a && D != nullptr}, {"dz", dz, need_e && z != nullptr},
                     {"ddelta_bias", ddelta_bias, need_a && delta_bias != nullptr}};
  for (const Req& r : req)
    if (r.need && r.p == nullptr) return fail(SSM_ERR_NULL_ARG, "required pointer %s is NULL", r.name);
  if ((dD != nullptr && D == nullptr) || (dz != nullptr && z == nullptr) ||
      (ddelta_bias != nullptr && delta_bias == nullptr))
    return fail(SSM_ERR_UNSUPPORTED, "a gradient was requested for an input the forward did not have");
  const void* ptrs[] = {x, delta, A, B, C, D, z, delta_bias, initial_state, dout, dlast_state, dx, ddelta, dA,
                        dB, dC, dD, dz, ddelta_bias, dinitial_state};
  const char* names[] = {"x", "delta", "A", "B", "C", "D", "z", "delta_bias", "initial_state", "dout",
                         "dlast_state", "dx", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias",
                         "dinitial_state"};
  for (int i = 0; i < 20; ++i)
    if ((st = check_align(names[i], ptrs[i])) != SSM_OK) return st;
  if ((st = check_align("ckpt", ckpt_in)) != SSM_OK) return st;
  int64_t ckpt_bytes = 0;
  if (ckpt_in != nullptr && (st = ckpt_size(batch, seqlen, d_inner, &ckpt_bytes)) != SSM_OK) return st;
  const Range rck = range("ckpt", ckpt_in, ckpt_bytes);
  const int64_t si = esize(in_dtype), sg = esize(grad_dtype);
  const Range ins[] = {
      range("x", x, sz.elems * si),          range("delta", delta, sz.elems * si),
      range("z", z, sz.elems * si),          range("B", B, sz.bc * si),
      range("C", C, sz.bc * si),             range("A", A, d_inner * d_state * 4),
      range("D", D, d_inner * 4),            range("delta_bias", delta_bias, d_inner * 4),
      range("initial_state", initial_state, sz.state * 4), range("dout", dout, sz.elems * sg),
      range("dlast_state", dlast_state, sz.state * 4),
  };
  const Range outs[] = {
      range("dx", dx, sz.elems * sg),        range("ddelta", ddelta, sz.elems * sg),
      range("dz", dz, sz.elems * sg),        range("dB", dB, sz.bc * sg),
      range("dC", dC, sz.bc * sg),           range("dA", dA, d_inner * d_state * 4),
      range("dD", dD, d_inner * 4),          range("ddelta_bias", ddelta_bias, d_inner * 4),
      range("dinitial_state", dinitial_state, sz.state * 4),
  };
  for (int i = 0; i < 9; ++i) {
    if (overlaps(outs[i], rck)) return fail(SSM_ERR_UNSUPPORTED, "%s overlaps input ckpt", outs[i].name);
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return fail(SSM_ERR_UNSUPPORTED, "%s overlaps input %s", outs[i].name, r.name);
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outs[j]))
        return fail(SSM_ERR_UNSUPPORTED, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  ssm_plan plan;
  if (plan_in) {
    plan = *plan_in;
    if (plan.states_per_wave != 4)
      return fail(SSM_ERR_UNSUPPORTED, "plan.states_per_wave=%d: the backward carries 4 states per wavefront",
                  plan.states_per_wave);
    if (plan.chunk_len < 1) return fail(SSM_ERR_UNSUPPORTED, "plan.chunk_len must be >= 1");
    plan.n_chunks = seqlen > 0 ? (seqlen + plan.chunk_len - 1) / plan.chunk_len : 0;
    if (plan.n_chunks > 1 && plan.chunk_len % ssm::kBwdTile != 0)
      return fail(SSM_ERR_UNSUPPORTED, "plan.chunk_len=%lld must be a multiple of %d when it cuts the sequence",
                  (long long)plan.chunk_len, ssm::kBwdTile);
    if (plan.n_chunks > 65535) return fail(SSM_ERR_UNSUPPORTED, "plan gives more than 65535 chunks");
  } else {
    choose_bwd_plan(batch, seqlen, d_inner, device_simds(), &plan);
  }
  const int64_t K = std::max<int64_t>(1, plan.n_chunks);

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (d_inner == 0) return ok();
  if (batch == 0 || seqlen == 0) {
    // no steps: the parameter gradients are zero and the state's gradient
    // passes through unchanged
    e = ssm::launch_fill_zero(dA, d_inner * d_state, s);
    if (e == hipSuccess && dD) e = ssm::launch_fill_zero(dD, d_inner, s);
    if (e == hipSuccess && ddelta_bias) e = ssm::launch_fill_zero(ddelta_bias, d_inner, s);
    if (e == hipSuccess && dinitial_state && sz.state > 0)
      e = dlast_state ? ssm::launch_copy_f32(dinitial_state, dlast_state, sz.state, s)
                      : ssm::launch_fill_zero(dinitial_state, sz.state, s);
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  const int64_t nblk = (d_inner + 63) / 64;
  const int64_t ntiles = (seqlen + ssm::kBwdTile - 1) / ssm::kBwdTile;
  // per (row, chunk): dA partials, dD / dbias partials; chunked runs also
  // keep each chunk's entering state, arriving gradient and reverse pair
  int64_t n_ck, n_bc, n_a, n_dd, n_cs, n_cd, bytes;
  // (the checkpoints live in the workspace unless the caller hands them in)
  if (!mul_ok(batch * nblk, ckpt_in ? 0 : ntiles * 64 * d_state, &n_ck) ||
      !mul_ok(sz.bc / d_state, nblk * 2 * d_state, &n_bc) ||
      !mul_ok(sz.state, K, &n_a) || !mul_ok(batch * d_inner, 2 * K, &n_dd) ||
      !mul_ok(sz.state, K > 1 ? K : 0, &n_cs) || !mul_ok(batch * d_inner, K > 1 ? K : 0, &n_cd) ||
      !mul_ok(n_ck + n_bc + n_a + n_dd + 3 * n_cs + 2 * n_cd, 4, &bytes))
    return fail(SSM_ERR_BAD_SHAPE, "workspace size overflows int64");
  void* ws = nullptr;
  e = ws_alloc(&ws, bytes, s);
  if (e != hipSuccess || ws == nullptr)
    return fail_hip("workspace allocation", (long long)bytes, e);
  ssm::BwdArgs a{};
  a.x = x;
  a.delta = delta;
  a.z = z;
  a.B = B;
  a.C = C;
  a.A = A;
  a.D = D;
  a.bias = delta_bias;
  a.h0 = initial_state;
  a.dout = dout;
  a.dlast = dlast_state;
  a.dx = dx;
  a.ddelta = ddelta;
  a.dz = dz;
  a.ws_ckpt = ckpt_in ? const_cast<float*>(ckpt_in) : static_cast<float*>(ws);  // read only when given
  a.ckpt_given = ckpt_in ? 1 : 0;
  a.ws_bc = static_cast<float*>(ws) + n_ck;
  a.ws_a = a.ws_bc + n_bc;
  a.ws_dd = a.ws_a + n_a;
  if (K > 1) {
    a.ws_hin = a.ws_dd + n_dd;
    a.ws_rev = a.ws_hin + n_cs;
    a.ws_dl = a.ws_rev + n_cs;
    a.ws_fsum = a.ws_dl + n_cs;
    a.ws_rsum = a.ws_fsum + n_cd;
  }
  a.dh0 = dinitial_state;
  a.seqlen = seqlen;
  a.d_inner = d_inner;
  a.chunk_len = K > 1 ? plan.chunk_len : seqlen;
  a.n_chunks = (int32_t)K;
  a.batch = (int32_t)batch;
  a.softplus = (softplus & SSM_SOFTPLUS) ? 1 : 0;
  a.nblk = (int32_t)nblk;
  a.cus = device_simds() / 4;
  e = ssm::launch_scan_bwd(a, to_dt(in_dtype), to_dt(grad_dtype), dA, dB, dC, dD, ddelta_bias, s);
  hipError_t e2 = hipFreeAsync(ws, s);
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

ssm_status ssm_scan_bwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                        const float* D, const void* z, const float* delta_bias, int softplus,
                        const float* initial_state, const void* dout, const float* dlast_state, void* dx,
                        void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                        float* dinitial_state, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                        ssm_dtype in_dtype, ssm_dtype grad_dtype, void* stream) {
  return bwd_impl(x, delta, A, B, C, D, z, delta_bias, softplus, initial_state, dout, dlast_state, dx, ddelta, dA,
                  dB, dC, dD, dz, ddelta_bias, dinitial_state, batch, seqlen, d_inner, d_state, in_dtype, grad_dtype,
                  stream, nullptr);
}

ssm_status ssm_scan_ckpt_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state, int64_t* bytes) {
  if (!bytes) return fail(SSM_ERR_NULL_ARG, "bytes is NULL");
  if (batch < 0 || seqlen < 0 || d_inner < 0)
    return fail(SSM_ERR_BAD_SHAPE, "negative size (batch=%lld seqlen=%lld d_inner=%lld)", (long long)batch,
                (long long)seqlen, (long long)d_inner);
  if (d_state != ssm::kDState)
    return fail(SSM_ERR_UNSUPPORTED, "d_state=%lld is not supported (16)", (long long)d_state);
  return ckpt_size(batch, seqlen, d_inner, bytes);
}

ssm_status ssm_scan_fwd_ckpt(const void* x, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, int softplus,
                             const float* initial_state, void* out, float* last_state, float* ckpt, int64_t batch,
                             int64_t seqlen, int64_t d_inner, int64_t d_state, ssm_dtype in_dtype,
                             ssm_dtype out_dtype, void* stream) {
  if (!ckpt && batch > 0 && seqlen > 0 && d_inner > 0) return fail(SSM_ERR_NULL_ARG, "required pointer ckpt is NULL");
  return scan_impl(x, delta, A, B, C, D, z, delta_bias, softplus, initial_state, out, last_state, batch, seqlen,
                   d_inner, d_state, in_dtype, out_dtype, stream, nullptr, false, ckpt);
}

ssm_status ssm_scan_bwd_ckpt(const void* x, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, int softplus,
                             const float* initial_state, const void* dout, const float* dlast_state,
                             const float* ckpt, void* dx, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                             void* dz, float* ddelta_bias, float* dinitial_state, int64_t batch, int64_t seqlen,
                             int64_t d_inner, int64_t d_state, ssm_dtype in_dtype, ssm_dtype grad_dtype,
                             void* stream) {
  if (!ckpt && batch > 0 && seqlen > 0 && d_inner > 0) return fail(SSM_ERR_NULL_ARG, "required pointer ckpt is NULL");
  return bwd_impl(x, delta, A, B, C, D, z, delta_bias, softplus, initial_state, dout, dlast_state, dx, ddelta, dA,
                  dB, dC, dD, dz, ddelta_bias, dinitial_state, batch, seqlen, d_inner, d_state, in_dtype, grad_dtype,
                  stream, nullptr, ckpt);
}

ssm_status ssm_scan_bwd_plan(const void* x, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, int softplus,
                             const float* initial_state, const void* dout, const float* dlast_state, void* dx,
                             void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                             float* ddelta_bias, float* dinitial_state, int64_t batch, int64_t seqlen,
                             int64_t d_inner, int64_t d_state, ssm_dtype in_dtype, ssm_dtype grad_dtype,
                             void* stream, const ssm_plan* plan) {
  if (!plan) return fail(SSM_ERR_NULL_ARG, "plan is NULL");
  return bwd_impl(x, delta, A, B, C, D, z, delta_bias, softplus, initial_state, dout, dlast_state, dx, ddelta, dA,
                  dB, dC, dD, dz, ddelta_bias, dinitial_state, batch, seqlen, d_inner, d_state, in_dtype, grad_dtype,
                  stream, plan);
}

ssm_status ssm_scan_bwd_plan_query(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                                   ssm_plan* plan) {
  if (!plan) return fail(SSM_ERR_NULL_ARG, "plan is NULL");
  Sizes sz;
  ssm_status st = check_common(batch, seqlen, d_inner, d_state, SSM_F32, SSM_F32, &sz);
  if (st != SSM_OK) return st;
  choose_bwd_plan(batch, seqlen, d_inner, device_simds(), plan);
  return SSM_OK;
}

ssm_status ssm_conv1d_fwd(const void* x, const float* weight, const float* bias, int silu,
                          const void* conv_state_in, void* out, void* conv_state_out, int64_t batch,
                          int64_t seqlen, int64_t d_inner, int64_t d_conv, ssm_dtype in_dtype,
                          ssm_dtype out_dtype, void* stream) {
  ssm_status st = conv_check(batch, seqlen, d_inner, d_conv, in_dtype, out_dtype);
  if (st != SSM_OK) return st;
  const int64_t elems = batch * seqlen * d_inner, cache = batch * d_inner * d_conv;
  if ((elems > 0 && (!x || !out)) || (d_inner > 0 && !weight))
    return fail(SSM_ERR_NULL_ARG, "required pointer %s is NULL", (elems > 0 && !x) ? "x" : !weight ? "weight" : "out");
  const void* ptrs[] = {x, weight, bias, conv_state_in, out, conv_state_out};
  const char* names[] = {"x", "weight", "bias", "conv_state_in", "out", "conv_state_out"};
  for (int i = 0; i < 6; ++i)
    if ((st = check_align(names[i], ptrs[i])) != SSM_OK) return st;
  const int64_t si = esize(in_dtype), so = esize(out_dtype);
  const Range ins[] = {range("x", x, elems * si), range("weight", weight, d_inner * d_conv * 4),
                       range("bias", bias, d_inner * 4), range("conv_state_in", conv_state_in, cache * si)};
  const Range ro = range("out", out, elems * so);
  const Range rs = range("conv_state_out", conv_state_out, cache * si);
  const bool in_place = conv_state_out != nullptr && conv_state_out == conv_state_in;
  for (int i = 0; i < 4; ++i) {
    if (overlaps(ro, ins[i])) return fail(SSM_ERR_UNSUPPORTED, "out overlaps input %s", ins[i].name);
    // the outgoing cache may replace the incoming one in place (i == 3)
    if (overlaps(rs, ins[i]) && !(in_place && i == 3))
      return fail(SSM_ERR_UNSUPPORTED, "conv_state_out overlaps input %s", ins[i].name);
  }
  if (overlaps(ro, rs)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps conv_state_out");
  if (batch == 0 || d_inner == 0) return ok();
  ssm::ConvArgs a{};
  a.x = x;
  a.w = weight;
  a.bias = bias;
  a.state_in = conv_state_in;
  a.out = out;
  a.state_out = conv_state_out;
  a.seqlen = seqlen;
  a.d_inner = d_inner;
  a.batch = (int32_t)batch;
  a.silu = silu ? 1 : 0;
  hipError_t e = ssm::launch_conv1d(a, to_dt(in_dtype), to_dt(out_dtype), (int)d_conv, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

ssm_status ssm_conv1d_update(void* conv_state, const void* x, const float* weight, const float* bias, int silu,
                             void* out, int64_t batch, int64_t d_inner, int64_t d_conv, ssm_dtype in_dtype,
                             ssm_dtype out_dtype, void* stream) {
  ssm_status st = conv_check(batch, 1, d_inner, d_conv, in_dtype, out_dtype);
  if (st != SSM_OK) return st;
  const int64_t elems = batch * d_inner, cache = batch * d_inner * d_conv;
  if (elems > 0 && (!conv_state || !x || !out || !weight))
    return fail(SSM_ERR_NULL_ARG, "required pointer %s is NULL",
                !conv_state ? "conv_state" : !x ? "x" : !weight ? "weight" : "out");
  const void* ptrs[] = {conv_state, x, weight, bias, out};
  const char* names[] = {"conv_state", "x", "weight", "bias", "out"};
  for (int i = 0; i < 5; ++i)
    if ((st = check_align(names[i], ptrs[i])) != SSM_OK) return st;
  const int64_t si = esize(in_dtype), so = esize(out_dtype);
  const Range ins[] = {range("x", x, elems * si), range("weight", weight, d_inner * d_conv * 4),
                       range("bias", bias, d_inner * 4)};
  const Range ro = range("out", out, elems * so);
  const Range rs = range("conv_state", conv_state, cache * si);
  for (const Range& r : ins) {
    if (overlaps(ro, r)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps input %s", r.name);
    if (overlaps(rs, r)) return fail(SSM_ERR_UNSUPPORTED, "conv_state overlaps input %s", r.name);
  }
  if (overlaps(ro, rs)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps conv_state");
  if (elems == 0) return ok();
  ssm::ConvArgs a{};
  a.x = x;
  a.w = weight;
  a.bias = bias;
  a.state_in = conv_state;
  a.out = out;
  a.state_out = conv_state;
  a.seqlen = 1;
  a.d_inner = d_inner;
  a.batch = (int32_t)batch;
  a.silu = silu ? 1 : 0;
  hipError_t e =
      ssm::launch_conv1d_update(a, to_dt(in_dtype), to_dt(out_dtype), (int)d_conv, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

ssm_status ssm_affine_exclusive_scan(const float* a, const float* b, float* out_a, float* out_b, int64_t n,
                                     void* stream) {
  if (n < 0) return fail(SSM_ERR_BAD_SHAPE, "n=%lld is negative", (long long)n);
  if (n > 0 && (!a || !b || !out_a || !out_b)) return fail(SSM_ERR_NULL_ARG, "required pointer is NULL");
  hipError_t e = ssm::launch_affine_exclusive_scan(a, b, out_a, out_b, n, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

static ssm_status ssd_impl(const void* x, const void* dt, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* dt_bias, int softplus,
                           const float* initial_state, void* out, float* last_state, int64_t batch,
                           int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups, int64_t d_state,
                           ssm_dtype in_dtype, ssm_dtype out_dtype, void* stream, const ssm_plan* plan_in) {
  SsdSizes sz;
  ssm_status st = ssd_check(batch, seqlen, nheads, headdim, ngroups, d_state, in_dtype, out_dtype, softplus, true,
                            &sz);
  if (st != SSM_OK) return st;
  const bool need_e = sz.elems > 0, need_bc = sz.bc > 0;
  struct Req { const char* name; const void* p; bool need; };
  const Req req[] = {{"x", x, need_e}, {"dt", dt, need_e}, {"out", out, need_e}, {"A", A, need_e},
                     {"B", B, need_bc}, {"C", C, need_bc}};
  for (const Req& r : req)
    if (r.need && r.p == nullptr) return fail(SSM_ERR_NULL_ARG, "required pointer %s is NULL", r.name);
  const void* ptrs[] = {x, A, B, C, D, z, dt_bias, out, last_state, initial_state};
  const char* names[] = {"x", "A", "B", "C", "D", "z", "dt_bias", "out", "last_state", "initial_state"};
  for (int i = 0; i < 10; ++i)
    if ((st = check_align(names[i], ptrs[i])) != SSM_OK) return st;
  // dt is read one element at a time: element alignment suffices
  if ((st = check_align("dt", dt, (uintptr_t)esize(in_dtype))) != SSM_OK) return st;
  const int64_t si = esize(in_dtype), so = esize(out_dtype);
  const Range ins[] = {
      range("x", x, sz.elems * si),     range("dt", dt, sz.steps * si),     range("z", z, sz.elems * si),
      range("B", B, sz.bc * si),        range("C", C, sz.bc * si),          range("A", A, nheads * 4),
      range("D", D, nheads * headdim * 4), range("dt_bias", dt_bias, nheads * 4),
  };
  const Range ro = range("out", out, sz.elems * so);
  const Range rl = range("last_state", last_state, sz.state * 4);
  const Range rh = range("initial_state", initial_state, sz.state * 4);
  for (const Range& r : ins) {
    if (overlaps(ro, r)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps input %s", r.name);
    if (overlaps(rl, r)) return fail(SSM_ERR_UNSUPPORTED, "last_state overlaps input %s", r.name);
  }
  if (overlaps(ro, rl)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps last_state");
  if (overlaps(ro, rh)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps initial_state");
  // each workgroup reads its own slice of the initial state before it writes
  // the same slice of the final state, so the two may be one buffer
  const bool in_place = initial_state != nullptr &&
                        static_cast<const void*>(initial_state) == static_cast<const void*>(last_state);
  if (!in_place && overlaps(rl, rh)) return fail(SSM_ERR_UNSUPPORTED, "last_state partly overlaps initial_state");
  ssm_plan plan;
  if (plan_in) {
    plan = *plan_in;
    if (plan.chunk_len < 1) return fail(SSM_ERR_UNSUPPORTED, "plan.chunk_len must be >= 1");
    plan.n_chunks = seqlen > 0 ? (seqlen + plan.chunk_len - 1) / plan.chunk_len : 0;
    if (plan.n_chunks > 1 && plan.chunk_len % 32 != 0)
      return fail(SSM_ERR_UNSUPPORTED, "plan.chunk_len=%lld must be a multiple of 32 when it cuts the sequence",
                  (long long)plan.chunk_len);
    if (plan.n_chunks > 65535) return fail(SSM_ERR_UNSUPPORTED, "plan gives more than 65535 chunks");
  } else {
    choose_ssd_plan(batch, seqlen, nheads, device_simds(), &plan);
  }
  const int64_t K = std::max<int64_t>(1, plan.n_chunks);

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (batch == 0) return ok();
  if (seqlen == 0) {
    if (last_state && !in_place) {
      hipError_t e = initial_state ? ssm::launch_copy_f32(last_state, initial_state, sz.state, s)
                                   : ssm::launch_fill_zero(last_state, sz.state, s);
      if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    }
    return ok();
  }
  ssm::SsdArgs a{};
  a.x = x;
  a.dt = dt;
  a.z = z;
  a.B = B;
  a.C = C;
  a.A = A;
  a.D = D;
  a.bias = dt_bias;
  a.h0 = initial_state;
  a.out = out;
  a.state = last_state;
  a.seqlen = seqlen;
  a.chunk_len = K > 1 ? plan.chunk_len : seqlen;
  a.n_chunks = (int32_t)K;
  a.batch = (int32_t)batch;
  a.nheads = (int32_t)nheads;
  a.headdim = (int32_t)headdim;
  a.ngroups = (int32_t)ngroups;
  a.d_state = (int32_t)d_state;
  a.softplus = (softplus & SSM_SOFTPLUS) ? 1 : 0;
  a.cus = device_simds() / 4;
  void* ws = nullptr;
  hipError_t e = hipSuccess;
  if (K > 1) {
    // With several chunks, the workgroups that read the initial state are not
    // the ones that write the final state: an in-place initial state is read
    // from a copy in the workspace.
    const int64_t n_h0 = in_place ? sz.state : 0;
    int64_t n_state, n_decay, bytes;
    if (!mul_ok(sz.state, K, &n_state) || !mul_ok(batch * nheads, K, &n_decay) ||
        !mul_ok(n_state + n_decay + n_h0, 4, &bytes))
      return fail(SSM_ERR_BAD_SHAPE, "workspace size overflows int64");
    e = ws_alloc(&ws, bytes, s);
    if (e != hipSuccess || ws == nullptr)
      return fail_hip("workspace allocation", (long long)bytes, e);
    a.ws_state = static_cast<float*>(ws);
    a.ws_decay = a.ws_state + n_state;
    if (n_h0 > 0) {
      float* copy = a.ws_decay + n_decay;
      e = ssm::launch_copy_f32(copy, initial_state, n_h0, s);
      a.h0 = copy;
    }
  }
  if (e == hipSuccess) e = ssm::launch_ssd(a, to_dt(out_dtype), s);
  if (ws) {
    hipError_t e2 = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

ssm_status ssm_ssd_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                       const float* D, const void* z, const float* dt_bias, int softplus,
                       const float* initial_state, void* out, float* last_state, int64_t batch, int64_t seqlen,
                       int64_t nheads, int64_t headdim, int64_t ngroups, int64_t d_state, ssm_dtype in_dtype,
                       ssm_dtype out_dtype, void* stream) {
  return ssd_impl(x, dt, A, B, C, D, z, dt_bias, softplus, initial_state, out, last_state, batch, seqlen, nheads,
                  headdim, ngroups, d_state, in_dtype, out_dtype, stream, nullptr);
}

ssm_status ssm_ssd_fwd_plan(const void* x, const void* dt, const float* A, const void* B, const void* C,
                            const float* D, const void* z, const float* dt_bias, int softplus,
                            const float* initial_state, void* out, float* last_state, int64_t batch,
                            int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups, int64_t d_state,
                            ssm_dtype in_dtype, ssm_dtype out_dtype, void* stream, const ssm_plan* plan) {
  if (!plan) return fail(SSM_ERR_NULL_ARG, "plan is NULL");
  return ssd_impl(x, dt, A, B, C, D, z, dt_bias, softplus, initial_state, out, last_state, batch, seqlen, nheads,
                  headdim, ngroups, d_state, in_dtype, out_dtype, stream, plan);
}

ssm_status ssm_ssd_plan_query(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                              int64_t d_state, ssm_plan* plan) {
  if (!plan) return fail(SSM_ERR_NULL_ARG, "plan is NULL");
  SsdSizes sz;
  ssm_status st = ssd_check(batch, seqlen, nheads, headdim, ngroups, d_state, SSM_BF16, SSM_F32, 0, true, &sz);
  if (st != SSM_OK) return st;
  choose_ssd_plan(batch, seqlen, nheads, device_simds(), plan);
  return SSM_OK;
}

ssm_status ssm_ssd_state_update(float* state, const void* x, const void* dt, const float* A, const void* B,
                                const void* C, const float* D, const void* z, const float* dt_bias, int softplus,
                                void* out, int64_t batch, int64_t nheads, int64_t headdim, int64_t ngroups,
                                int64_t d_state, ssm_dtype in_dtype, ssm_dtype out_dtype, void* stream) {
  SsdSizes sz;
  ssm_status st = ssd_check(batch, 1, nheads, headdim, ngroups, d_state, in_dtype, out_dtype, softplus, false, &sz);
  if (st != SSM_OK) return st;
  const bool need_e = sz.elems > 0;
  struct Req { const char* name; const void* p; bool need; };
  const Req req[] = {{"state", state, need_e}, {"x", x, need_e}, {"dt", dt, need_e}, {"out", out, need_e},
                     {"A", A, need_e}, {"B", B, need_e}, {"C", C, need_e}};
  for (const Req& r : req)
    if (r.need && r.p == nullptr) return fail(SSM_ERR_NULL_ARG, "required pointer %s is NULL", r.name);
  const void* ptrs[] = {state, x, A, B, C, D, z, dt_bias, out};
  const char* names[] = {"state", "x", "A", "B", "C", "D", "z", "dt_bias", "out"};
  for (int i = 0; i < 9; ++i)
    if ((st = check_align(names[i], ptrs[i])) != SSM_OK) return st;
  if ((st = check_align("dt", dt, (uintptr_t)esize(in_dtype))) != SSM_OK) return st;
  const int64_t si = esize(in_dtype), so = esize(out_dtype);
  const Range ins[] = {
      range("x", x, sz.elems * si),     range("dt", dt, sz.steps * si),     range("z", z, sz.elems * si),
      range("B", B, sz.bc * si),        range("C", C, sz.bc * si),          range("A", A, nheads * 4),
      range("D", D, nheads * headdim * 4), range("dt_bias", dt_bias, nheads * 4),
  };
  const Range rs = range("state", state, sz.state * 4);
  const Range ro = range("out", out, sz.elems * so);
  for (const Range& r : ins) {
    if (overlaps(ro, r)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps input %s", r.name);
    if (overlaps(rs, r)) return fail(SSM_ERR_UNSUPPORTED, "state overlaps input %s", r.name);
  }
  if (overlaps(ro, rs)) return fail(SSM_ERR_UNSUPPORTED, "out overlaps state");
  if (batch == 0) return ok();
  ssm::SsdArgs a{};
  a.x = x;
  a.dt = dt;
  a.z = z;
  a.B = B;
  a.C = C;
  a.A = A;
  a.D = D;
  a.bias = dt_bias;
  a.out = out;
  a.state = state;
  a.seqlen = 1;
  a.batch = (int32_t)batch;
  a.nheads = (int32_t)nheads;
  a.headdim = (int32_t)headdim;
  a.ngroups = (int32_t)ngroups;
  a.d_state = (int32_t)d_state;
  a.softplus = (softplus & SSM_SOFTPLUS) ? 1 : 0;
  hipError_t e = ssm::launch_ssd_update(a, to_dt(in_dtype), to_dt(out_dtype), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

ssm_status ssm_trim_workspace(void) {
  const int dev = stream_device(nullptr);
  if (hipMemPool_t pool = workspace_pool(dev, false)) {
    const hipError_t e = hipMemPoolTrimTo(pool, 0);
    if (e != hipSuccess) return fail_hip("hipMemPoolTrimTo", -1, e);
  }
  return ok();
}

const char* ssm_status_string(ssm_status s) {
  switch (s) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_NULL_ARG: return "SSM_ERR_NULL_ARG: a required pointer is NULL";
    case SSM_ERR_BAD_SHAPE: return "SSM_ERR_BAD_SHAPE: a size is negative or overflows";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED: dtype, d_state, alignment, aliasing or plan";
    case SSM_ERR_HIP: return "SSM_ERR_HIP: the HIP runtime refused an allocation or launch";
    default: return "unknown ssm_status";
  }
}

const char* ssm_last_error(void) { return g_last_error.c_str(); }

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

}  // extern "C"

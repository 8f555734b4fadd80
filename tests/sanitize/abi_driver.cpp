// Drives every entry point of the C ABI through the host layer built with
// AddressSanitizer and UndefinedBehaviorSanitizer over the fake runtime of
// fake_runtime.cpp: valid calls (every plan kind, empty sizes, in-place
// states), rejected calls (each status code), and a workspace allocation that
// fails.  Buffers are allocated at their exact sizes, so any read past one in
// the launcher stubs is reported.  Prints "abi driver ok" and exits 0 when
// every expectation holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/ssmscan.h"

extern "C" void fake_fail_next_alloc(void);
extern "C" long fake_launches(void);
extern "C" long fake_live_allocs(void);
extern "C" int fake_pools(void);

namespace {
int g_failures = 0;
std::vector<void*> g_bufs;

void* buf(int64_t elems, int64_t esize) {
  if (elems <= 0) return nullptr;
  void* p = nullptr;
  if (posix_memalign(&p, 16, (size_t)(elems * esize)) != 0) std::abort();
  std::memset(p, 0, (size_t)(elems * esize));
  g_bufs.push_back(p);
  return p;
}

void expect(const char* what, ssm_status got, ssm_status want) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d (%s), expected %d; last error: %s\n", what, (int)got,
                 ssm_status_string(got), (int)want, ssm_last_error());
    ++g_failures;
  }
}

int64_t es(ssm_dtype t) { return t == SSM_F32 ? 4 : 2; }

struct Scan {
  int64_t b, L, d;
  ssm_dtype in, out;
  void *x, *dl, *z, *B, *C, *y;
  float *A, *D, *bias, *last, *h0;
  Scan(int64_t b_, int64_t L_, int64_t d_, ssm_dtype i, ssm_dtype o) : b(b_), L(L_), d(d_), in(i), out(o) {
    const int64_t n = b * L * d, r = b * L;
    x = buf(n, es(in));
    dl = buf(n, es(in));
    z = buf(n, es(in));
    B = buf(r * 16, es(in));
    C = buf(r * 16, es(in));
    y = buf(n, es(out));
    A = static_cast<float*>(buf(d * 16, 4));
    D = static_cast<float*>(buf(d, 4));
    bias = static_cast<float*>(buf(d, 4));
    last = static_cast<float*>(buf(b * d * 16, 4));
    h0 = static_cast<float*>(buf(b * d * 16, 4));
  }
  ssm_status fwd() {
    return ssm_scan_fwd(x, dl, A, B, C, D, z, bias, SSM_SOFTPLUS, y, last, b, L, d, 16, in, out, nullptr);
  }
  ssm_status plan(int spw, int64_t chunk, int flags = SSM_SOFTPLUS) {
    ssm_plan p{};
    p.states_per_wave = spw;
    p.chunk_len = chunk;
    return ssm_scan_fwd_plan(x, dl, A, B, C, D, z, bias, flags, y, last, b, L, d, 16, in, out, nullptr, &p);
  }
  ssm_status from(const float* init, float* last_out, const ssm_plan* p, bool noalloc) {
    auto f = noalloc ? ssm_scan_fwd_noalloc : ssm_scan_fwd_from;
    return f(x, dl, A, B, C, D, z, bias, SSM_SOFTPLUS, init, y, last_out, b, L, d, 16, in, out, nullptr, p);
  }
};

void scan_calls() {
  for (ssm_dtype in : {SSM_F32, SSM_BF16})
    for (ssm_dtype out : {SSM_F32, SSM_BF16}) {
      Scan s(2, 37, 70, in, out);
      expect("scan_fwd", s.fwd(), SSM_OK);
      for (int spw : {1, 2, 4, 8, 16})
        for (int64_t chunk : {1, 8, 36, 37, 100}) expect("scan_fwd_plan", s.plan(spw, chunk), SSM_OK);
      expect("scan_fwd_plan zoh", s.plan(4, 8, SSM_SOFTPLUS | SSM_ZOH), SSM_OK);
      ssm_plan p{};
      p.states_per_wave = 4;
      p.chunk_len = 8;
      expect("scan_fwd_from", s.from(s.h0, s.last, &p, false), SSM_OK);
      expect("scan_fwd_from in place", s.from(s.last, s.last, &p, false), SSM_OK);
      expect("scan_fwd_from default plan", s.from(s.h0, s.last, nullptr, false), SSM_OK);
      expect("scan_fwd_noalloc", s.from(s.h0, s.last, &p, true), SSM_OK);
      expect("scan_fwd_noalloc in place", s.from(s.last, s.last, &p, true), SSM_OK);
      expect("scan_fwd_noalloc default plan", s.from(nullptr, s.last, nullptr, true), SSM_OK);
    }
  // empty sizes
  Scan e0(0, 5, 3, SSM_BF16, SSM_F32), e1(2, 0, 3, SSM_BF16, SSM_F32), e2(2, 5, 0, SSM_F32, SSM_F32);
  expect("scan batch 0", e0.fwd(), SSM_OK);
  expect("scan seqlen 0", e1.fwd(), SSM_OK);
  expect("scan seqlen 0 from state", e1.from(e1.h0, e1.last, nullptr, false), SSM_OK);
  expect("scan d_inner 0", e2.fwd(), SSM_OK);
  // the planner over a range of shapes
  for (int64_t b : {1, 3, 8})
    for (int64_t L : {1, 31, 2048, 262144})
      for (int64_t d : {1, 64, 1536, 5120}) {
        ssm_plan p{};
        expect("scan_plan", ssm_scan_plan(b, L, d, 16, &p), SSM_OK);
        expect("bwd_plan_query", ssm_scan_bwd_plan_query(b, L, d, 16, &p), SSM_OK);
      }
}

void scan_rejections() {
  Scan s(2, 37, 70, SSM_BF16, SSM_F32);
  const long before = fake_launches();
  expect("NULL x", ssm_scan_fwd(nullptr, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, 1, s.y, s.last, 2, 37, 70, 16,
                                SSM_BF16, SSM_F32, nullptr), SSM_ERR_NULL_ARG);
  expect("negative seqlen", ssm_scan_fwd(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, 1, s.y, s.last, 2, -1, 70, 16,
                                         SSM_BF16, SSM_F32, nullptr), SSM_ERR_BAD_SHAPE);
  expect("element count overflow",
         ssm_scan_fwd(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, 1, s.y, s.last, INT64_MAX / 4, 37, 70, 16,
                      SSM_BF16, SSM_F32, nullptr), SSM_ERR_BAD_SHAPE);
  expect("d_state 8", ssm_scan_fwd(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, 1, s.y, s.last, 2, 37, 70, 8,
                                   SSM_BF16, SSM_F32, nullptr), SSM_ERR_UNSUPPORTED);
  expect("misaligned x", ssm_scan_fwd(static_cast<char*>(s.x) + 2, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, 1, s.y,
                                      s.last, 2, 37, 70, 16, SSM_BF16, SSM_F32, nullptr), SSM_ERR_UNSUPPORTED);
  expect("out aliases x", ssm_scan_fwd(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, 1, const_cast<void*>(s.x), s.last,
                                       2, 37, 70, 16, SSM_BF16, SSM_BF16, nullptr), SSM_ERR_UNSUPPORTED);
  expect("unknown flag", ssm_scan_fwd(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, 8, s.y, s.last, 2, 37, 70, 16,
                                      SSM_BF16, SSM_F32, nullptr), SSM_ERR_UNSUPPORTED);
  expect("bad dtype", ssm_scan_fwd(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, 1, s.y, s.last, 2, 37, 70, 16,
                                   (ssm_dtype)7, SSM_F32, nullptr), SSM_ERR_UNSUPPORTED);
  expect("plan 3 states per wave", s.plan(3, 8), SSM_ERR_UNSUPPORTED);
  expect("plan chunk 0", s.plan(4, 0), SSM_ERR_UNSUPPORTED);
  expect("last_state overlaps initial_state",
         ssm_scan_fwd_from(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, 1, s.h0, s.y, s.h0 + 16, 2, 37, 70, 16,
                           SSM_BF16, SSM_F32, nullptr, nullptr), SSM_ERR_UNSUPPORTED);
  Scan big(1, 65536, 4096, SSM_BF16, SSM_F32);
  ssm_plan p{};
  p.states_per_wave = 4;
  p.chunk_len = 32;   // 2048 chunks: a carry workspace larger than the fixed array
  expect("noalloc beyond the fixed array", big.from(nullptr, big.last, &p, true), SSM_ERR_UNSUPPORTED);
  if (fake_launches() != before) {
    std::fprintf(stderr, "a rejected call launched work\n");
    ++g_failures;
  }
  // a workspace that cannot be allocated: SSM_ERR_HIP before any launch
  fake_fail_next_alloc();
  p.chunk_len = 8;
  expect("failed workspace allocation", s.from(s.h0, s.last, &p, false), SSM_ERR_HIP);
  if (fake_launches() != before) {
    std::fprintf(stderr, "a call whose allocation failed launched work\n");
    ++g_failures;
  }
  if (std::strlen(ssm_last_error()) == 0) {
    std::fprintf(stderr, "no message after a failed call\n");
    ++g_failures;
  }
  expect("a valid call after the failure", s.from(s.h0, s.last, &p, false), SSM_OK);
}

void checkpoint_calls() {
  for (ssm_dtype in : {SSM_F32, SSM_BF16})
    for (int64_t L : {37, 3000}) {   // one chunk; chunks (3000 steps, 2 x 70 channels: the planner cuts it)
      Scan s(2, L, 70, in, SSM_F32);
      int64_t bytes = 0;
      expect("scan_ckpt_bytes", ssm_scan_ckpt_bytes(2, L, 70, 16, &bytes), SSM_OK);
      float* ck = static_cast<float*>(buf(bytes / 4, 4));
      expect("scan_fwd_ckpt", ssm_scan_fwd_ckpt(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, SSM_SOFTPLUS, s.h0, s.y,
                                                s.last, ck, 2, L, 70, 16, in, SSM_F32, nullptr), SSM_OK);
      const int64_t n = 2 * L * 70, r = 2 * L;
      void *dout = buf(n, es(in)), *dx = buf(n, es(in)), *ddl = buf(n, es(in)), *dz = buf(n, es(in));
      void *dB = buf(r * 16, es(in)), *dC = buf(r * 16, es(in));
      float *dA = static_cast<float*>(buf(70 * 16, 4)), *dD = static_cast<float*>(buf(70, 4));
      float* dbias = static_cast<float*>(buf(70, 4));
      expect("scan_bwd_ckpt", ssm_scan_bwd_ckpt(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, SSM_SOFTPLUS, s.h0, dout,
                                                nullptr, ck, dx, ddl, dA, dB, dC, dD, dz, dbias, nullptr, 2, L, 70, 16,
                                                in, in, nullptr), SSM_OK);
    }
}

void decode_calls() {
  for (ssm_dtype in : {SSM_F32, SSM_BF16}) {
    const int64_t b = 3, d = 70;
    float* st = static_cast<float*>(buf(b * d * 16, 4));
    void *x = buf(b * d, es(in)), *dl = buf(b * d, es(in)), *z = buf(b * d, es(in));
    void *B = buf(b * 16, es(in)), *C = buf(b * 16, es(in)), *y = buf(b * d, 4);
    float *A = static_cast<float*>(buf(d * 16, 4)), *D = static_cast<float*>(buf(d, 4));
    float* bias = static_cast<float*>(buf(d, 4));
    expect("state_update", ssm_state_update(st, x, dl, A, B, C, D, z, bias, SSM_SOFTPLUS, y, b, d, 16, in, SSM_F32,
                                            nullptr), SSM_OK);
    expect("state_update zoh, no options",
           ssm_state_update(st, x, dl, A, B, C, nullptr, nullptr, nullptr, SSM_ZOH, y, b, d, 16, in, SSM_F32, nullptr),
           SSM_OK);
    expect("state_update out aliases state",
           ssm_state_update(st, x, dl, A, B, C, D, z, bias, 1, st, b, d, 16, in, SSM_F32, nullptr),
           SSM_ERR_UNSUPPORTED);
  }
}

void bwd_calls() {
  for (ssm_dtype in : {SSM_F32, SSM_BF16}) {
    Scan s(2, 37, 70, in, in);
    const int64_t n = 2 * 37 * 70, r = 2 * 37, st = 2 * 70 * 16;
    void *dout = buf(n, es(in)), *dx = buf(n, es(in)), *ddl = buf(n, es(in)), *dz = buf(n, es(in));
    void *dB = buf(r * 16, es(in)), *dC = buf(r * 16, es(in));
    float *dA = static_cast<float*>(buf(70 * 16, 4)), *dD = static_cast<float*>(buf(70, 4));
    float *dbias = static_cast<float*>(buf(70, 4)), *dlast = static_cast<float*>(buf(st, 4));
    float* dh0 = static_cast<float*>(buf(st, 4));
    expect("scan_bwd", ssm_scan_bwd(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, SSM_SOFTPLUS, s.h0, dout, dlast, dx,
                                    ddl, dA, dB, dC, dD, dz, dbias, dh0, 2, 37, 70, 16, in, in, nullptr), SSM_OK);
    for (int64_t chunk : {8, 16, 40}) {
      ssm_plan p{};
      p.states_per_wave = 4;
      p.chunk_len = chunk;
      expect("scan_bwd_plan", ssm_scan_bwd_plan(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, SSM_SOFTPLUS, s.h0, dout,
                                                dlast, dx, ddl, dA, dB, dC, dD, dz, dbias, dh0, 2, 37, 70, 16, in, in,
                                                nullptr, &p), SSM_OK);
    }
    ssm_plan bad{};
    bad.states_per_wave = 4;
    bad.chunk_len = 12;   // below seqlen and not a multiple of 8
    expect("scan_bwd_plan chunk 12", ssm_scan_bwd_plan(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, SSM_SOFTPLUS, s.h0,
                                                       dout, dlast, dx, ddl, dA, dB, dC, dD, dz, dbias, dh0, 2, 37, 70,
                                                       16, in, in, nullptr, &bad), SSM_ERR_UNSUPPORTED);
    expect("scan_bwd zoh", ssm_scan_bwd(s.x, s.dl, s.A, s.B, s.C, s.D, s.z, s.bias, SSM_ZOH, s.h0, dout, dlast, dx,
                                        ddl, dA, dB, dC, dD, dz, dbias, dh0, 2, 37, 70, 16, in, in, nullptr),
           SSM_ERR_UNSUPPORTED);
    expect("scan_bwd without options", ssm_scan_bwd(s.x, s.dl, s.A, s.B, s.C, nullptr, nullptr, nullptr, 0, nullptr,
                                                    dout, nullptr, dx, ddl, dA, dB, dC, nullptr, nullptr, nullptr,
                                                    nullptr, 2, 37, 70, 16, in, in, nullptr), SSM_OK);
  }
}

void conv_calls() {
  for (ssm_dtype in : {SSM_F32, SSM_BF16})
    for (int64_t K : {2, 3, 4}) {
      const int64_t b = 2, L = 37, d = 70;
      void *x = buf(b * L * d, es(in)), *y = buf(b * L * d, es(in));
      void *si = buf(b * d * K, es(in)), *so = buf(b * d * K, es(in));
      float *w = static_cast<float*>(buf(d * K, 4)), *bias = static_cast<float*>(buf(d, 4));
      expect("conv1d_fwd", ssm_conv1d_fwd(x, w, bias, 1, si, y, so, b, L, d, K, in, in, nullptr), SSM_OK);
      expect("conv1d_fwd no cache", ssm_conv1d_fwd(x, w, nullptr, 0, nullptr, y, nullptr, b, L, d, K, in, in, nullptr),
             SSM_OK);
      void *xs = buf(b * d, es(in)), *ys = buf(b * d, es(in));
      expect("conv1d_update", ssm_conv1d_update(si, xs, w, bias, 1, ys, b, d, K, in, in, nullptr), SSM_OK);
    }
}

void ssd_calls() {
  const int64_t b = 2, L = 70, H = 4, P = 64, G = 2;
  for (int64_t N : {64, 128}) {
    void *x = buf(b * L * H * P, 2), *dt = buf(b * L * H, 2), *z = buf(b * L * H * P, 2);
    void *B = buf(b * L * G * N, 2), *C = buf(b * L * G * N, 2), *y = buf(b * L * H * P, 4);
    float *A = static_cast<float*>(buf(H, 4)), *D = static_cast<float*>(buf(H * P, 4));
    float *bias = static_cast<float*>(buf(H, 4)), *h0 = static_cast<float*>(buf(b * H * P * N, 4));
    float* last = static_cast<float*>(buf(b * H * P * N, 4));
    expect("ssd_fwd", ssm_ssd_fwd(x, dt, A, B, C, D, z, bias, SSM_SOFTPLUS, h0, y, last, b, L, H, P, G, N, SSM_BF16,
                                  SSM_F32, nullptr), SSM_OK);
    for (int64_t chunk : {32, 64, 70}) {
      ssm_plan p{};
      p.states_per_wave = 4;
      p.chunk_len = chunk;
      expect("ssd_fwd_plan", ssm_ssd_fwd_plan(x, dt, A, B, C, D, z, bias, SSM_SOFTPLUS, h0, y, last, b, L, H, P, G, N,
                                              SSM_BF16, SSM_F32, nullptr, &p), SSM_OK);
      expect("ssd_fwd_plan in place", ssm_ssd_fwd_plan(x, dt, A, B, C, D, z, bias, SSM_SOFTPLUS, last, y, last, b, L,
                                                       H, P, G, N, SSM_BF16, SSM_F32, nullptr, &p), SSM_OK);
    }
    ssm_plan p{};
    expect("ssd_plan_query", ssm_ssd_plan_query(b, 262144, 32, P, 1, N, &p), SSM_OK);
    void *xs = buf(b * H * P, 2), *dts = buf(b * H, 2), *Bs = buf(b * G * N, 2), *Cs = buf(b * G * N, 2);
    void* ys = buf(b * H * P, 2);
    expect("ssd_state_update", ssm_ssd_state_update(last, xs, dts, A, Bs, Cs, D, nullptr, bias, SSM_SOFTPLUS, ys, b,
                                                    H, P, G, N, SSM_BF16, SSM_BF16, nullptr), SSM_OK);
    expect("ssd headdim 48", ssm_ssd_fwd(x, dt, A, B, C, D, z, bias, 1, h0, y, last, b, L, H, 48, G, N, SSM_BF16,
                                         SSM_F32, nullptr), SSM_ERR_UNSUPPORTED);
  }
  float *a = static_cast<float*>(buf(100, 4)), *bb = static_cast<float*>(buf(100, 4));
  float *oa = static_cast<float*>(buf(100, 4)), *ob = static_cast<float*>(buf(100, 4));
  expect("affine_exclusive_scan", ssm_affine_exclusive_scan(a, bb, oa, ob, 100, nullptr), SSM_OK);
  expect("affine_exclusive_scan negative", ssm_affine_exclusive_scan(a, bb, oa, ob, -1, nullptr), SSM_ERR_BAD_SHAPE);
}
}  // namespace

int main() {
  if (ssm_abi_version() != SSM_ABI_VERSION) {
    std::fprintf(stderr, "ABI version mismatch\n");
    return 1;
  }
  scan_calls();
  scan_rejections();
  decode_calls();
  bwd_calls();
  checkpoint_calls();
  conv_calls();
  ssd_calls();
  if (fake_live_allocs() != 0) {
    std::fprintf(stderr, "%ld workspace allocations not freed\n", fake_live_allocs());
    ++g_failures;
  }
  if (fake_pools() != 1) {
    std::fprintf(stderr, "%d workspace pools created, expected one\n", fake_pools());
    ++g_failures;
  }
  expect("trim_workspace", ssm_trim_workspace(), SSM_OK);
  for (void* p : g_bufs) std::free(p);
  if (g_failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_failures);
    return 1;
  }
  std::printf("abi driver ok: %ld launches\n", fake_launches());
  return 0;
}

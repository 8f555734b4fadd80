// Streaming-bandwidth probe of MI355X's HBM: a copy and a read of a large
// buffer, shaped for bandwidth (16-byte non-temporal accesses, enough
// workgroups to keep every CU's memory pipeline full).  Built into the probe
// library (libssmprobe.so) beside the VALU probe, for the benchmark's
// measured streaming ceilings; the scan library does not contain or call it.
//
// Shapes (chosen by a sweep on one MI355X over 1 GiB: one, two or four
// vectors per thread, plain or non-temporal, 1024 workgroups to one per
// 256 vectors):
//   copy: one 16-byte vector per thread, one workgroup per 256 vectors;
//   read: two 16-byte vectors per thread and iteration, grid-stride over
//         one workgroup per 512 vectors, summed into a register that is
//         stored only if it takes a sentinel value (so no write traffic).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) stream_copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                          int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ void __launch_bounds__(256) stream_read_kernel(const f32x4* __restrict__ src, float* __restrict__ sink,
                                                          int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 512;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t base = (int64_t)blockIdx.x * 512 + threadIdx.x; base < n; base += stride) {
    if (base < n) acc += __builtin_nontemporal_load(src + base);
    if (base + 256 < n) acc += __builtin_nontemporal_load(src + base + 256);
  }
  if (acc.x == -1.5e38f) sink[0] = acc.y + acc.z + acc.w;  // never true for the probe's data
}

}  // namespace

// kind 0: copy n16 16-byte vectors from src to dst; kind 1: read them.
// src and dst are 16-byte aligned device buffers; sink is one float.
extern "C" int ssm_stream_probe_launch(int kind, const void* src, void* dst, int64_t n16, void* stream) {
  if (n16 <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0) {
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                       static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), n16);
  } else if (kind == 1) {
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)((n16 + 511) / 512)), dim3(256), 0, s,
                       static_cast<const f32x4*>(src), static_cast<float*>(dst), n16);
  } else {
    return -1;
  }
  return (int)hipGetLastError();
}

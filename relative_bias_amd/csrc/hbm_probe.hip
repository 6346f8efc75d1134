// Streaming-read ceiling of the device's HBM, for the benchmark's report:
// one pass of 16-byte loads over a buffer, with the data folded into one
// value per workgroup so the loads are not removed.  Not part of the
// attention path; built as its own library (libhbmprobe.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *src, int64_t n16, uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < kThreads; ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

extern "C" {

// Reads `bytes` bytes (a multiple of 16, 16-byte aligned device memory) once;
// `sink` receives `blocks` words.  Returns 0, or -1 for bad arguments, -5 for
// a failed launch.
int hbm_stream_read(const void *src, int64_t bytes, uint32_t *sink, int32_t blocks, void *stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || blocks <= 0) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"

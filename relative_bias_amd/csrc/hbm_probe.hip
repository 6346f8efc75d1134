// Streaming-read ceiling of the device's HBM, for the benchmark's report:
// one pass of 16-byte nontemporal loads over a buffer, each workgroup reading
// one contiguous chunk of it (eight loads per thread in flight), with the data
// folded into one value per workgroup so the loads are not removed.  Of the
// patterns measured this one reads fastest (about 7.0 TB/s on MI355X, against
// about 6.4 TB/s for a grid-stride pass and 10 % less again without the
// nontemporal hint).  Not part of the attention path; built as its own
// library (libhbmprobe.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *src, int64_t n16, uint32_t *sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t begin = (int64_t)blockIdx.x * per;
  const int64_t end = begin + per < n16 ? begin + per : n16;
  uint32_t acc = 0;
  int64_t i = begin + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < end; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < end; i += kThreads) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
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

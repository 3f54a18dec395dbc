// Streaming-read kernel: the measured HBM read ceiling that the attend
// kernels' throughput is compared with (every KV byte is read exactly once,
// so a plain read of the same number of bytes bounds the fused path).
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr unsigned kReadGrid = 1024;  // 4 workgroups per CU

// Each thread reads 16-byte words grid-stride, four in flight, and folds them
// into one XOR; the fold is stored only if it equals an arbitrary constant, so
// no load can be dropped and nothing is written in practice.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ p,
                                                                   long long n,
                                                                   unsigned* __restrict__ sink) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  unsigned acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    const u32x4 x = (a ^ b) ^ (c ^ d);
    acc ^= (x.x ^ x.y) ^ (x.z ^ x.w);
  }
  for (; i < n; i += stride) {
    const u32x4 a = p[i];
    acc ^= (a.x ^ a.y) ^ (a.z ^ a.w);
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* data, long long bytes, unsigned* sink,
                              hipStream_t stream) {
  const long long n = bytes / 16;
  const long long want = (n + kReadThreads - 1) / kReadThreads;
  const unsigned grid = static_cast<unsigned>(want < kReadGrid ? want : kReadGrid);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kReadThreads), 0, stream,
                     static_cast<const u32x4*>(data), n, sink);
  return hipGetLastError();
}

}  // namespace kvq

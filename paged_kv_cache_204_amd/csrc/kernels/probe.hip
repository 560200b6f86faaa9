// Streaming-read probe: the HBM read ceiling the attention kernels are
// compared with.  Every thread reads 16-byte chunks, four in flight per
// iteration, over a grid-strided range, and folds them into one word that
// is stored only if it equals a value passed at launch: the compiler cannot
// drop the loads, and for real data a thread stores (into the caller's sink
// word) with probability 2^-32.
#include "../kernels.hpp"

namespace pkv {
namespace {

__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, int64_t n,
                                                         uint32_t* __restrict__ sink, uint32_t magic) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == magic) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                             hipStream_t s) {
  const int64_t n = static_cast<int64_t>(bytes / 16);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(read_probe_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s,
                     static_cast<const uint4*>(src), n, sink, 0x9E3779B9u);
  return hipGetLastError();
}

}  // namespace pkv

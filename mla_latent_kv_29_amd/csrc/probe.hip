// Achievable HBM read bandwidth, the measured ceiling that the decode
// kernels' byte roofline is read against beside the 8 TB/s of the data
// sheet: a plain stream of 16-byte loads over a buffer, 2048 blocks of 256
// threads in a grid-stride loop, nothing written.
#include "internal.hpp"

namespace mla {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_read_probe(const i32x4* __restrict__ p, size_t n, int* __restrict__ sink) {
  i32x4 acc = {0, 0, 0, 0};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    acc ^= __builtin_nontemporal_load(p + i);
  const int r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (r == 0x5bd1e995) sink[0] = r;  // keeps the loads; practically never stores
}

}  // namespace

hipError_t read_probe(const void* src, size_t bytes, int* sink, hipStream_t st) {
  return launch(&k_read_probe, dim3(2048), dim3(256), 0, st, (const i32x4*)src, bytes / 16, sink);
}

}  // namespace mla

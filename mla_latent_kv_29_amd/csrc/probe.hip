// Measurement probes, no part of the MLA maths.
//  * Achievable HBM read bandwidth, the measured ceiling that the decode
//    kernels' byte roofline is read against beside the 8 TB/s of the data
//    sheet: a plain stream of 16-byte loads over a buffer, 2048 blocks of 256
//    threads in a grid-stride loop, nothing written.
//  * Achievable bf16 MFMA rate: every wave runs eight independent chains of
//    v_mfma_f32_32x32x16_bf16 on operands held in registers (eight A and
//    four B fragments of random values, so that the inputs change from one
//    MFMA to the next as in a real kernel), with no memory traffic at all.
//    It is the ceiling that an MFMA-bound kernel can reach at the clock the
//    part holds under dense MFMA work.  (Four chains at four waves a SIMD
//    ran about 15% slower than this form; eight chains, or one wave a SIMD,
//    reach the same rate.)
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

constexpr int MP_BLOCKS = 1024, MP_A = 8, MP_B = 4, MP_C = 8;  // 4096 waves, eight accumulator chains

__global__ __launch_bounds__(256) void k_mfma_probe(const bf16x8* __restrict__ ops, int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[MP_A], b[MP_B];
#pragma unroll
  for (int k = 0; k < MP_A; ++k) a[k] = ops[64 * k + lane];
#pragma unroll
  for (int j = 0; j < MP_B; ++j) b[j] = ops[64 * (MP_A + j) + lane];
  f32x16 c[MP_C];
#pragma unroll
  for (int j = 0; j < MP_C; ++j) c[j] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < MP_A; ++k)
#pragma unroll
      for (int j = 0; j < MP_B; ++j) {
        c[(MP_B * k + j) % MP_C] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[j], c[(MP_B * k + j) % MP_C], 0, 0, 0);
      }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < MP_C; ++j) s += c[j][lane & 15];
  if (s == 1234.5f) sink[0] = s;  // keeps the products; practically never stores
}

}  // namespace

hipError_t mfma_probe(const void* ops, int iters, float* sink, hipStream_t st) {
  return launch(&k_mfma_probe, dim3(MP_BLOCKS), dim3(256), 0, st, (const bf16x8*)ops, iters, sink);
}

double mfma_probe_flops(int iters) {
  return (double)MP_BLOCKS * 4 * iters * MP_A * MP_B * (32.0 * 32 * 16 * 2);
}

hipError_t read_probe(const void* src, size_t bytes, int* sink, hipStream_t st) {
  return launch(&k_read_probe, dim3(2048), dim3(256), 0, st, (const i32x4*)src, bytes / 16, sink);
}

}  // namespace mla

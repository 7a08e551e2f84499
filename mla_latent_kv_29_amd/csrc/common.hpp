// Device-side helpers shared by the MLA kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <tuple>
#include <utility>
#include "../../include/mla.h"

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

namespace mla {

// Kernel launch that returns this launch's own status (no dependence on the
// thread's sticky last-error state).
template <typename K, typename Tup, size_t... I>
inline hipError_t launch_impl(K kern, dim3 grid, dim3 block, size_t shmem, hipStream_t st, Tup& a,
                              std::index_sequence<I...>) {
  void* p[] = {(void*)&std::get<I>(a)..., nullptr};
  return hipLaunchKernel((const void*)kern, grid, block, p, shmem, st);
}
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t st,
                         Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> a(std::forward<Args>(args)...);
  return launch_impl(kern, grid, block, shmem, st, a, std::index_sequence_for<KArgs...>{});
}

#define MLA_TRY(x)                            \
  do {                                        \
    hipError_t e_ = (x);                      \
    if (e_ != hipSuccess) return e_;          \
  } while (0)

// ---------------------------------------------------------------- scalars
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }  // RNE

// OCP E4M3FN (bias 7, max 448) -- the gfx950 fp8 conversion instructions use
// this format.  Hardware conversion rounds to nearest even but turns values
// beyond the largest finite one into NaN, so the input is clamped first.
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
  x = fminf(fmaxf(x, -448.0f), 448.0f);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false);
  return (uint8_t)(r & 0xff);
}
__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false)[0];
}

// ---------------------------------------------------------------- cache layout
// The two FP8 cache formats share the page layout and the codes; they differ
// only in how a tile's scale is chosen (see tile_scale).
__host__ __device__ inline bool is_fp8_cache(int t) { return t == MLA_FP8_E4M3 || t == MLA_FP8_E4M3_E8; }

// Scale of a 1x128 tile with largest magnitude amax: amax/448, or for the
// power-of-two (UE8M0) format the smallest power of two >= amax/448 and at
// least 2^-126 (adding a full mantissa and clearing it rounds a positive
// float up to its binade's power of two; a subnormal quotient gives 2^-126).
// 1 for an all-zero tile.
__device__ inline float tile_scale(float amax, int dtype) {
  if (!(amax > 0.0f)) return 1.0f;
  const float s = amax / 448.0f;
  if (dtype != MLA_FP8_E4M3_E8) return s;
  return __uint_as_float((__float_as_uint(s) + 0x007FFFFFu) & 0x7F800000u);
}

struct CacheGeom {
  int d_c, d_rope, page_size, dtype;
  size_t page_bytes;
  // byte offsets inside an FP8 page
  size_t fp8_scale_off, fp8_rope_off;
};

__host__ __device__ inline size_t page_bytes_of(int d_c, int d_rope, int page_size, int dtype) {
  if (dtype == MLA_F32) return (size_t)page_size * (d_c + d_rope) * 4;
  if (dtype == MLA_BF16) return (size_t)page_size * (d_c + d_rope) * 2;
  return (size_t)page_size * ((size_t)d_c + 4 * (size_t)(d_c / 128) + 2 * (size_t)d_rope);
}

inline CacheGeom make_geom(const mla_dims& d, int dtype) {
  CacheGeom g;
  g.d_c = d.d_c; g.d_rope = d.d_rope; g.page_size = d.page_size; g.dtype = dtype;
  g.page_bytes = page_bytes_of(d.d_c, d.d_rope, d.page_size, dtype);
  g.fp8_scale_off = (size_t)d.page_size * d.d_c;
  g.fp8_rope_off = g.fp8_scale_off + (size_t)d.page_size * (d.d_c / 128) * 4;
  return g;
}

// Frequency of RoPE pair m: theta^(-2m/d_rope), in double so that angles at
// positions up to 2^17 keep full single-precision accuracy after sincos.
__device__ __forceinline__ void rope_cs(int pos, int m, int d_rope, float theta, float* c, float* s) {
  double w = pow((double)theta, -2.0 * (double)m / (double)d_rope);
  double sn, cs;
  sincos((double)pos * w, &sn, &cs);
  *c = (float)cs; *s = (float)sn;
}

// The same rotation from a precomputed frequency w = theta^(-2m/d_rope)
// (double): the angle pos*w is reduced modulo 2 pi in double, so that the
// single-precision sincos of the remainder keeps full accuracy at any
// position, at a fraction of the cost of the double-precision functions.
__device__ __forceinline__ void rope_cs_w(int pos, double w, float* c, float* s) {
  const double x = (double)pos * w;
  const double k = rint(x * 0.15915494309189535);           // 1 / (2 pi)
  const double r = fma(-k, 2.4492935982947064e-16, fma(-k, 6.283185307179586, x));  // 2 pi = hi + lo
  sincosf((float)r, s, c);
}

// Workgroup barrier for LDS rings filled by global_load_lds.  The caller has
// already waited (vmcnt) for the loads that must have landed; __syncthreads()
// would also drain the loads still in flight for later stages, which empties
// the ring every step.  LDS reads and writes issued before it are complete
// when any wave passes it.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace mla

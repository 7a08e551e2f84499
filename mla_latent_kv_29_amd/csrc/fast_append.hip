// Latent-cache append on MFMA for the DeepSeek-V3 shape (gfx950).
//
// DeepSeek-V3 reading lesson, §2.1.1 (and the summary "Báo cáo Kỹ thuật
// DeepSeek-V3", Phương pháp item 1): c^KV_t = W^DKV h_t, k^R_t =
// RoPE(W^KR h_t); only these 576 numbers per token are cached.
//
// A block computes 64 tokens x all 576 outputs ([W^DKV; W^KR] rows) with
// v_mfma_f32_16x16x32_bf16 (each of the 4 waves owns 144 columns), the k loop
// staged through a 3-deep LDS ring filled by global_load_lds_dwordx4.  The fp32
// result tile then goes through LDS so that each token row is finished in one
// place: RoPE on the last 64 channels (angles in double precision), then bf16
// conversion or E4M3 quantisation with one fp32 scale per 1x128 tile (lesson
// §3.3, item 2), and a scatter into the token's page slot.
#include "internal.hpp"
#include "layout.hpp"

namespace mla {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

constexpr int DC = 512, DR = 64, D = 576, TOK = 64;
constexpr int NSA = 3;
constexpr int XT_BYTES = TOK * 32 * 2;          // 4 KiB
constexpr int WT_BYTES = D * 32 * 2;            // 36 KiB
constexpr int STA_BYTES = XT_BYTES + WT_BYTES;  // 40 KiB
constexpr int OUT_BYTES = TOK * D * 4;          // 147 456: fp32 result tile
constexpr int APPEND_LDS = OUT_BYTES > NSA * STA_BYTES ? OUT_BYTES : NSA * STA_BYTES;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// rows x 32 k tile, row r chunk q at r*4 + (q ^ ((r>>2)&3))
__device__ __forceinline__ int tpos(int r, int q) { return r * 4 + (q ^ ((r >> 2) & 3)); }

__device__ __forceinline__ void load_tile_instr(const bf16_t* base, long ld, int r0, int rows_valid, int k0,
                                                uint8_t* dst, int i, int lane) {
  const int pos = 64 * i + lane;
  const int r = pos >> 2, q = (pos & 3) ^ ((r >> 2) & 3);
  int row = r0 + r;
  row = row < rows_valid ? row : rows_valid - 1;
  __builtin_amdgcn_global_load_lds((gbl_void*)(base + (long)row * ld + k0 + 8 * q), (lds_void*)(dst + i * 1024), 16,
                                   0, 0);
}

__global__ __launch_bounds__(256) void k_append_v3(int n_tok, int d_model, float theta, const bf16_t* __restrict__ h,
                                                   const int32_t* __restrict__ seq_id, const int32_t* __restrict__ pos,
                                                   const bf16_t* __restrict__ W_DKV, const bf16_t* __restrict__ W_KR,
                                                   uint8_t* __restrict__ pages, CacheGeom g,
                                                   const int32_t* __restrict__ bt, int max_pages) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TOK;
  const int nsteps = d_model / 32;
  const int g16 = lane >> 4, i16 = lane & 15;

  // 40 instructions per stage: 4 for the h tile, 32 for W^DKV rows, 4 for W^KR rows
  auto issue = [&](int step) {
    uint8_t* st = lds + (step % NSA) * STA_BYTES;
    const int k0 = step * 32;
#pragma unroll
    for (int n = 0; n < 10; ++n) {
      const int i = wave + 4 * n;
      if (i < 4) load_tile_instr(h, d_model, t0, n_tok, k0, st, i, lane);
      else if (i < 36) load_tile_instr(W_DKV, d_model, 0, DC, k0, st + XT_BYTES, i - 4, lane);
      else load_tile_instr(W_KR, d_model, 0, DR, k0, st + XT_BYTES + 32 * 1024, i - 36, lane);
    }
  };

  f32x4 acc[4][9];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 9; ++b) acc[a][b] = f32x4{};

  for (int s = 0; s < NSA - 1 && s < nsteps; ++s) issue(s);
  for (int step = 0; step < nsteps; ++step) {
    if (step + 1 < nsteps) wait_vmcnt<10>();
    else wait_vmcnt<0>();
    ring_barrier();
    if (step + NSA - 1 < nsteps) issue(step + NSA - 1);
    const uint8_t* st = lds + (step % NSA) * STA_BYTES;
    bf16x8 a[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) a[mi] = *(const bf16x8*)(st + tpos(16 * mi + i16, g16) * 16);
#pragma unroll
    for (int ni = 0; ni < 9; ++ni) {
      const int col = 144 * wave + 16 * ni + i16;  // W row
      const bf16x8 b = *(const bf16x8*)(st + XT_BYTES + tpos(col, g16) * 16);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b, acc[mi][ni], 0, 0, 0);
    }
  }
  __syncthreads();  // ring no longer read: reuse LDS for the result tile

  float* tile = (float*)lds;  // [TOK][D]
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 9; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) tile[(16 * mi + 4 * g16 + r) * D + 144 * wave + 16 * ni + i16] = acc[mi][ni][r];
  __syncthreads();

  for (int tl = wave; tl < TOK; tl += 4) {
    const int t = t0 + tl;
    if (t >= n_tok) break;
    const int p = pos[t];
    const int page = bt[(long)seq_id[t] * max_pages + p / g.page_size];
    const int slot = p % g.page_size;
    uint8_t* pg = pages + (size_t)page * g.page_bytes;
    const float* row = tile + tl * D;
    if (g.dtype == MLA_BF16) {
      for (int C = lane; C < D / 8; C += 64) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = row[8 * C + e];
        if (C >= DC / 8) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float cs, sn;
            rope_cs(p, (8 * C - DC + e) >> 1, DR, theta, &cs, &sn);
            const float x0 = v[e], x1 = v[e + 1];
            v[e] = x0 * cs - x1 * sn;
            v[e + 1] = x0 * sn + x1 * cs;
          }
        }
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16_t)v[e];
        *(bf16x8*)(pg + bf16_page_off(slot, 8 * C, g.page_size)) = o;
      }
    } else {
      // latent: lane covers channels 8*lane .. +7; a 1x128 tile is 16 lanes
      float v[8];
      float am = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = row[8 * lane + e];
        am = fmaxf(am, fabsf(v[e]));
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
      const float s = am > 0.0f ? am / 448.0f : 1.0f;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) lo |= (uint32_t)f32_to_e4m3(v[e] / s) << (8 * e);
#pragma unroll
      for (int e = 0; e < 4; ++e) hi |= (uint32_t)f32_to_e4m3(v[4 + e] / s) << (8 * e);
      *(uint2*)(pg + fp8_code_off(slot, 8 * lane, g.page_size)) = make_uint2(lo, hi);
      if ((lane & 15) == 0) ((float*)(pg + g.fp8_scale_off))[slot * (DC / 128) + (lane >> 4)] = s;
      if (lane < DR / 8) {
        float r8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) r8[e] = row[DC + 8 * lane + e];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float cs, sn;
          rope_cs(p, (8 * lane + e) >> 1, DR, theta, &cs, &sn);
          const float x0 = r8[e], x1 = r8[e + 1];
          r8[e] = x0 * cs - x1 * sn;
          r8[e + 1] = x0 * sn + x1 * cs;
        }
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16_t)r8[e];
        *(bf16x8*)(pg + g.fp8_rope_off + fp8_rope_elem_off(slot, 8 * lane, g.page_size)) = o;
      }
    }
  }
}

}  // namespace

bool fast_append_shape(const mla_dims& d) { return d.d_c == DC && d.d_rope == DR && d.d_model % 32 == 0; }

hipError_t fast_append(const AppendArgs& a) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_append_v3, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       APPEND_LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int blocks = (a.n_tok + TOK - 1) / TOK;
  MLA_TRY(launch(&k_append_v3, dim3(blocks), dim3(256), APPEND_LDS, a.stream, a.n_tok, a.d.d_model,
                     a.d.rope_theta, (const bf16_t*)a.h, a.seq_id, a.pos, (const bf16_t*)a.W_DKV,
                     (const bf16_t*)a.W_KR, a.pages, a.g, a.block_table, a.max_pages));
  return hipSuccess;
}

}  // namespace mla

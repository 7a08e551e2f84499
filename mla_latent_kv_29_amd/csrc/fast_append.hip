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
// place: RoPE on the last 64 channels (angles reduced in double precision), then bf16
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

// RoPE rotation of pair m at position p: the frequency theta^(-2m/d_rope)
// in double (through exp2), the angle reduced modulo 2 pi in double, then a
// single-precision sincos of the remainder (full accuracy at any position,
// far cheaper than double-precision sincos).  All three append kernels use
// it, so a token's k^R does not depend on which of them wrote it.
__device__ __forceinline__ void rope_rot(int p, int m, float theta, float* cs, float* sn) {
  rope_cs_w(p, exp2(-2.0 * (double)m / DR * log2((double)theta)), cs, sn);
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
            rope_rot(p, (8 * C - DC + e) >> 1, theta, &cs, &sn);
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
      const float s = tile_scale(am, g.dtype);
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
          rope_rot(p, (8 * lane + e) >> 1, theta, &cs, &sn);
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

// ------------------------------------------------------------ few tokens
// The append of a decode step (one or a few new tokens per sequence): a block
// of k_append_v3 covers 64 tokens and streams the whole 8.26 MB of
// [W^DKV; W^KR], so a batch of 64 new tokens would be one block on one CU
// (372 us for 64 tokens, against 70 us here with 20 blocks; a CU streams
// these weight rows at about 30 GB/s, so the time is the bytes per block).
// Here a block takes one 128-channel tile of the outputs (four latent tiles,
// then the 64 RoPE channels) for 16 tokens, and its eight waves split
// d_model, each streaming its share of the tile's weight rows straight into
// MFMA operands (v_mfma_f32_16x16x32_bf16, A = h rows, B^T = weight rows,
// several k-steps of loads in flight); the eight partial tiles meet in LDS
// (summed in a fixed order) and the same epilogue arithmetic as above
// finishes each token row: RoPE on the RoPE tile, bf16 or E4M3 with the
// tile's scale, the scatter into the token's page slot.
constexpr int AR_TOK = 16, AR_COLS = 128, AR_NW = 8, AR_PD = 4;
constexpr int AR_TILES = DC / AR_COLS + 1;                    // 4 latent tiles + the RoPE tile
constexpr int AR_LDS = AR_NW * AR_TOK * AR_COLS * 4;          // 64 KiB of partial tiles
constexpr int APPEND_ROWS_MAX = 4096;                         // tokens a call up to which this path is taken

template <int NSUB>  // 16-column sub-tiles: 8 (latent tile) or 4 (RoPE tile)
__device__ __forceinline__ void ar_tile(int n_tok, int d_model, int tg, const bf16_t* __restrict__ h,
                                        const bf16_t* __restrict__ W, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int tok = min(tg * AR_TOK + r16, n_tok - 1);  // rows past the last token: computed, never stored
  const int kw = d_model / AR_NW, nks = kw / 32;
  const bf16_t* hp = h + (size_t)tok * d_model + wave * kw + 8 * kq;
  const bf16_t* wp = W + (size_t)r16 * d_model + wave * kw + 8 * kq;
  f32x4 acc[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) acc[s] = f32x4{};
  bf16x8 fa[AR_PD], fb[AR_PD][NSUB];
  // nks is a multiple of AR_PD (the launcher checks d_model).  The loads of a
  // k-step go out in one fixed order (its weight rows s = 0.., then its h
  // rows), in the prologue as in the loop, each pinned by a scheduling
  // barrier: the compiler's wait counts then see the same order on both
  // edges into the loop and wait, before each MFMA, only for the loads of
  // its own k-step (mismatched orders made it wait for nearly every load in
  // flight).  The steady state has no branch, for the same reason.
#pragma unroll
  for (int i = 0; i < AR_PD; ++i) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      fb[i][s] = *(const bf16x8*)(wp + (size_t)16 * s * d_model + 32 * i);
      __builtin_amdgcn_sched_barrier(0);
    }
    fa[i] = *(const bf16x8*)(hp + 32 * i);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int ks = 0; ks < nks - AR_PD; ks += AR_PD) {
#pragma unroll
    for (int i = 0; i < AR_PD; ++i) {
      const int kn = ks + i + AR_PD;  // the k-step that takes this slot next
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[i][s], acc[s], 0, 0, 0);
        fb[i][s] = *(const bf16x8*)(wp + (size_t)16 * s * d_model + 32 * kn);
        __builtin_amdgcn_sched_barrier(0);
      }
      fa[i] = *(const bf16x8*)(hp + 32 * kn);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < AR_PD; ++i)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[i][s], acc[s], 0, 0, 0);
  // C lane layout: tokens 4 kq + r of column 16 s + r16
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * AR_TOK + 4 * kq + r) * AR_COLS + 16 * s + r16] = acc[s][r];
}

__global__ __launch_bounds__(AR_NW * 64) void k_append_rows(int n_tok, int d_model, float theta,
                                                           const bf16_t* __restrict__ h,
                                                           const int32_t* __restrict__ seq_id,
                                                           const int32_t* __restrict__ pos,
                                                           const bf16_t* __restrict__ W_DKV,
                                                           const bf16_t* __restrict__ W_KR, uint8_t* __restrict__ pages,
                                                           CacheGeom g, const int32_t* __restrict__ bt, int max_pages) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  float* red = (float*)lds;  // [AR_NW][AR_TOK][AR_COLS]
  const int ct = blockIdx.x % AR_TILES, tg = blockIdx.x / AR_TILES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncols = ct < AR_TILES - 1 ? AR_COLS : DR;
  if (ct < AR_TILES - 1) ar_tile<AR_COLS / 16>(n_tok, d_model, tg, h, W_DKV + (size_t)AR_COLS * ct * d_model, red);
  else ar_tile<DR / 16>(n_tok, d_model, tg, h, W_KR, red);
  __syncthreads();
  // the tile: the eight partials summed in wave order into red[0]
  for (int i = tid; i < AR_TOK * ncols; i += AR_NW * 64) {
    const int t = i / ncols, c = i % ncols;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < AR_NW; ++w) v += red[(w * AR_TOK + t) * AR_COLS + c];
    red[t * AR_COLS + c] = v;
  }
  __syncthreads();
  // lane: token 4 wave + lane / 16 (waves 0-3), eight channels 8 (lane % 16)
  if (wave >= 4) return;
  const int tl = 4 * wave + (lane >> 4), c8 = lane & 15;
  const int t = tg * AR_TOK + tl;
  const bool live = t < n_tok && 8 * c8 < ncols;
  int p = 0;
  uint8_t* pg = pages;
  int slot = 0;
  if (t < n_tok) {
    p = pos[t];
    pg = pages + (size_t)bt[(long)seq_id[t] * max_pages + p / g.page_size] * g.page_bytes;
    slot = p % g.page_size;
  }
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = red[tl * AR_COLS + 8 * c8 + e];
  if (ct == AR_TILES - 1) {
    if (!live) return;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float cs, sn;
      rope_rot(p, (8 * c8 + e) >> 1, theta, &cs, &sn);
      const float x0 = v[e], x1 = v[e + 1];
      v[e] = x0 * cs - x1 * sn;
      v[e + 1] = x0 * sn + x1 * cs;
    }
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16_t)v[e];
    if (g.dtype == MLA_BF16) *(bf16x8*)(pg + bf16_page_off(slot, DC + 8 * c8, g.page_size)) = o;
    else *(bf16x8*)(pg + g.fp8_rope_off + fp8_rope_elem_off(slot, 8 * c8, g.page_size)) = o;
    return;
  }
  const int ch = AR_COLS * ct + 8 * c8;
  if (g.dtype == MLA_BF16) {
    if (!live) return;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16_t)v[e];
    *(bf16x8*)(pg + bf16_page_off(slot, ch, g.page_size)) = o;
    return;
  }
  // E4M3: the 16 lanes of a token hold its 1 x 128 tile
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[e]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
  if (!live) return;
  const float sc = tile_scale(am, g.dtype);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) lo |= (uint32_t)f32_to_e4m3(v[e] / sc) << (8 * e);
#pragma unroll
  for (int e = 0; e < 4; ++e) hi |= (uint32_t)f32_to_e4m3(v[4 + e] / sc) << (8 * e);
  *(uint2*)(pg + fp8_code_off(slot, ch, g.page_size)) = make_uint2(lo, hi);
  if (c8 == 0) ((float*)(pg + g.fp8_scale_off))[slot * (DC / 128) + ct] = sc;
}

// The second half of the workspace append: token blockIdx.x's row is the sum
// of the k-group partials (in k-group order), then the same epilogue as
// above.  Threads 0-63: latent channels 8 t .. +7 (a 1 x 128 tile is 16
// threads); threads 64-71: the RoPE channels 8 (t - 64) .. +7.
__global__ __launch_bounds__(128) void k_append_reduce(int n_tok, int kgroups, const float* __restrict__ part,
                                                       float theta, const int32_t* __restrict__ seq_id,
                                                       const int32_t* __restrict__ pos, uint8_t* __restrict__ pages,
                                                       CacheGeom g, const int32_t* __restrict__ bt, int max_pages) {
  const int t = blockIdx.x, tid = threadIdx.x;
  const bool rope = tid >= DC / 8;
  const int c8 = rope ? tid - DC / 8 : tid;
  if (rope && c8 >= DR / 8) return;
  const int ch = rope ? DC + 8 * c8 : 8 * c8;
  float v[8] = {};
  for (int k = 0; k < kgroups; ++k) {
    const float* src = part + ((long)k * n_tok + t) * D + ch;
    const float4 a0 = *(const float4*)src, a1 = *(const float4*)(src + 4);
    v[0] += a0.x; v[1] += a0.y; v[2] += a0.z; v[3] += a0.w;
    v[4] += a1.x; v[5] += a1.y; v[6] += a1.z; v[7] += a1.w;
  }
  const int p = pos[t];
  uint8_t* pg = pages + (size_t)bt[(long)seq_id[t] * max_pages + p / g.page_size] * g.page_bytes;
  const int slot = p % g.page_size;
  if (rope) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float cs, sn;
      rope_rot(p, (8 * c8 + e) >> 1, theta, &cs, &sn);
      const float x0 = v[e], x1 = v[e + 1];
      v[e] = x0 * cs - x1 * sn;
      v[e + 1] = x0 * sn + x1 * cs;
    }
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16_t)v[e];
    if (g.dtype == MLA_BF16) *(bf16x8*)(pg + bf16_page_off(slot, ch, g.page_size)) = o;
    else *(bf16x8*)(pg + g.fp8_rope_off + fp8_rope_elem_off(slot, 8 * c8, g.page_size)) = o;
    return;
  }
  if (g.dtype == MLA_BF16) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16_t)v[e];
    *(bf16x8*)(pg + bf16_page_off(slot, ch, g.page_size)) = o;
    return;
  }
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[e]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
  const float sc = tile_scale(am, g.dtype);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) lo |= (uint32_t)f32_to_e4m3(v[e] / sc) << (8 * e);
#pragma unroll
  for (int e = 0; e < 4; ++e) hi |= (uint32_t)f32_to_e4m3(v[4 + e] / sc) << (8 * e);
  *(uint2*)(pg + fp8_code_off(slot, ch, g.page_size)) = make_uint2(lo, hi);
  if ((c8 & 15) == 0) ((float*)(pg + g.fp8_scale_off))[slot * (DC / 128) + (c8 >> 4)] = sc;
}

}  // namespace

hipError_t append_reduce(const AppendArgs& a, const float* part, int kgroups) {
  return launch(&k_append_reduce, dim3(a.n_tok), dim3(128), 0, a.stream, a.n_tok, kgroups, part, a.d.rope_theta,
                a.seq_id, a.pos, a.pages, a.g, a.block_table, a.max_pages);
}

bool fast_append_shape(const mla_dims& d) { return d.d_c == DC && d.d_rope == DR && d.d_model % 32 == 0; }

hipError_t fast_append(const AppendArgs& a) {
  if (a.n_tok <= APPEND_ROWS_MAX && a.d.d_model % (32 * AR_NW * AR_PD) == 0) {
    MLA_TRY(lds_limit((const void*)k_append_rows, AR_LDS));
    const int blocks = AR_TILES * ((a.n_tok + AR_TOK - 1) / AR_TOK);
    return launch(&k_append_rows, dim3(blocks), dim3(AR_NW * 64), AR_LDS, a.stream, a.n_tok, a.d.d_model,
                  a.d.rope_theta, (const bf16_t*)a.h, a.seq_id, a.pos, (const bf16_t*)a.W_DKV,
                  (const bf16_t*)a.W_KR, a.pages, a.g, a.block_table, a.max_pages);
  }
  MLA_TRY(lds_limit((const void*)k_append_v3, APPEND_LDS));
  const int blocks = (a.n_tok + TOK - 1) / TOK;
  MLA_TRY(launch(&k_append_v3, dim3(blocks), dim3(256), APPEND_LDS, a.stream, a.n_tok, a.d.d_model,
                     a.d.rope_theta, (const bf16_t*)a.h, a.seq_id, a.pos, (const bf16_t*)a.W_DKV,
                     (const bf16_t*)a.W_KR, a.pages, a.g, a.block_table, a.max_pages));
  return hipSuccess;
}

}  // namespace mla

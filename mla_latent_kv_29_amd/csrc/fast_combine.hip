// Combine for up to 64 query rows, or up to 512 rows of at most 4 splits
// (gfx950): the merge of the attention's per-split partials and the W^UV
// projection in one kernel.
//
// What it computes: the softmax over all visible tokens from the softmaxes
// the attention took over disjoint token ranges (split s: normalised
// latent output O_s and log2-sum-exp2 lse_s of its scores), and then W^UV
// after the weighted latent sum, which the linearity of v^C = W^UV c^KV
// permits (DeepSeek-V3 reading lesson, §2.1.1).  For query row r and head i,
//     O_lat = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M),  M = max_s lse_s
// over the splits s that saw at least one token (lse_s = -inf marks an empty
// split, whose rows are never read), rounded to bf16, and then
//     out[r][i] = W^UV_i O_lat        (W^UV_i: [d_head][d_c], d_c contiguous)
// plus the row's natural-log LSE when asked for.
//
// One block per (head i, group of 32-row blocks taken in turn), eight
// waves; at most two groups a head, so that the grid stays at one block per
// CU and W^UV_i (128 KiB) streams HBM -> LDS with global_load_lds once a
// block, while the waves merge the first block's rows (wave w: rows w, w+8,
// w+16, w+24; lane l: channels 8l .. 8l+7, so each partial-row load is one
// contiguous 1 KiB wave access, and the rows of up to eight splits of all
// four rows are in flight together).  The merged rows land in LDS as bf16,
// and the 32 x 128 output tile is one MFMA pass over d_c.  The groups of a
// head run on one XCD, so W^UV_i comes from HBM once.  O_lat never leaves
// the CU, and the merge and the projection are one launch instead of two.
//
// LDS: O_lat tile [32 rows][512] then W^UV_i [128 n][512 k], bf16 rows of
// 1 KiB whose 16-byte chunk q sits at slot q ^ (row & 15): the MFMA operand
// reads (16 rows, one chunk each) hit 16 distinct bank groups.
#include <algorithm>

#include "internal.hpp"

namespace mla {
namespace {

constexpr int CB_DC = 512, CB_DV = 128, CB_ROWS = 32, CB_WAVES = 8;
constexpr int CB_W_OFF = CB_ROWS * CB_DC * 2;          // 32 KiB
constexpr int CB_LDS = CB_W_OFF + CB_DV * CB_DC * 2;   // 160 KiB
static_assert(CB_LDS <= 160 * 1024, "LDS");
// E4M3 weights: O_lat codes [32 rows][512], W^UV_i codes [128 n][512 k], the
// O_lat tile scales [32][4]; rows of 512 bytes, chunk q at slot q ^ (row & 15)
constexpr int CB8_W_OFF = CB_ROWS * CB_DC;                // 16 KiB
constexpr int CB8_S_OFF = CB8_W_OFF + CB_DV * CB_DC;      // 80 KiB
constexpr int CB8_LDS = CB8_S_OFF + CB_ROWS * (CB_DC / 128) * 4;

typedef __attribute__((address_space(3))) uint8_t lu8;
typedef __attribute__((address_space(3))) bf16x8 lbf16x8;

// One 1 KiB wave-instruction of a global -> LDS copy (16 bytes a lane at
// gbase + voff to LDS lds_addr + 16 lane), from asm so that the compiler's
// wait accounting leaves it alone; the kernel waits for it explicitly.
// Nothing else in k_merge_uv uses M0.
__device__ __forceinline__ void cb_dma(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds_addr)
               : "memory");
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x4 li32x4;

// 32 E4M3 bytes of an MFMA operand: 16-byte slots s0 and s1 of an LDS row
__device__ __forceinline__ i32x8 frag8(const lu8* row, int s0, int s1) {
  const i32x4 lo = *(const li32x4*)(row + 16 * s0);
  const i32x4 hi = *(const li32x4*)(row + 16 * s1);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

struct CbArgs {
  int batch, s_q, H, R;
  int S;              // splits (the host's count, checked against the workspace size)
  const uint8_t* ws;
  size_t lpart_off;
  const bf16_t* Wuv;  // [H][d_head][d_c]
  bf16_t* out;        // [R][H][d_head]
  float* lse_out;     // [R][H] or null
  const uint8_t* Wc;  // E4M3 form: codes [H][d_head][d_c], scales [H][d_c / 128]
  const float* Ws;
  int passes;         // 32-row blocks a workgroup takes in turn (W^UV_i loaded once)
};

template <bool F8>
__global__ __launch_bounds__(CB_WAVES * 64) void k_merge_uv(CbArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lu8* lds = (lu8*)lds_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, i16 = lane & 15;
  // blocks are dealt to the 8 XCDs round-robin; the row blocks of a head are
  // consecutive blocks of one XCD
  const int nrb = (a.R + CB_ROWS - 1) / CB_ROWS;
  const int nrg = (nrb + a.passes - 1) / a.passes;  // groups of `passes` row blocks
  const int lin = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);  // each XCD: a contiguous run
  const int head = lin / nrg, rg = lin % nrg;

  // W^UV_i rows to LDS first: the split weights below are one latency-bound
  // round trip (header, then the lse values), which the copy overlaps (the
  // compiler's wait for those loads covers the copy too, as loads complete
  // in order).  Row n = instruction n (16 per wave), chunk q of the row at
  // slot q ^ (n & 15), i.e. lane l reads chunk l ^ (n & 15).
  // E4M3: rows n = 2t (lanes 0..31) and 2t + 1 (lanes 32..63) in instruction
  // t (8 per wave), chunk q of row n at slot q ^ (n & 15).
  if constexpr (F8) {
    const uint8_t* W = a.Wc + (size_t)head * CB_DV * CB_DC;
    const uint32_t wt = (uint32_t)(uintptr_t)(lds + CB8_W_OFF);
#pragma unroll
    for (int jj = 0; jj < CB_DV / 2 / CB_WAVES; ++jj) {
      const int t = wave + CB_WAVES * jj, n = 2 * t + (lane >> 5);
      cb_dma(W, (uint32_t)(n * CB_DC + 16 * ((lane & 31) ^ (n & 15))), wt + 1024 * t);
    }
  } else {
    const bf16_t* W = a.Wuv + (size_t)head * CB_DV * CB_DC;
    const uint32_t wt = (uint32_t)(uintptr_t)(lds + CB_W_OFF);
#pragma unroll
    for (int jj = 0; jj < CB_DV / CB_WAVES; ++jj) {
      const int n = wave + CB_WAVES * jj;
      cb_dma(W, (uint32_t)((n * CB_DC + 8 * (lane ^ (n & 15))) * 2), wt + 1024 * n);
    }
  }

  const int32_t* hdr = (const int32_t*)a.ws;
  const int S = a.S;
  const bool pbf16 = hdr[HDR_PDT] == MLA_BF16;
  const float* lpart = (const float*)(a.ws + a.lpart_off);
  const uint8_t* opart = a.ws + opart_offset(a.lpart_off, a.batch, S, a.s_q, a.H);
  const size_t pstep = (size_t)a.s_q * a.H;  // partial row stride between splits

  // With several row blocks and at most 4 splits, the next block's lse values
  // and partial rows are loaded as soon as this block's are consumed, so that
  // they arrive while this block's projection runs (rows of empty splits
  // are loaded too and selected away, the sums stay as without prefetch).
  const bool pf = pbf16 && a.passes > 1 && S <= 4;
  float pre_lt[4];
  bf16x8 pre_v[4][4];
  bool have_pre = false;
  auto prefetch = [&](int rbn) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = CB_ROWS * rbn + wave + CB_WAVES * i;
      const bool lv = row < a.R;
      const int b = lv ? row / a.s_q : 0, j = lv ? row % a.s_q : 0;
      const size_t q0 = (((size_t)b * S) * a.s_q + j) * a.H + head;
      pre_lt[i] = lv && lane < S ? lpart[q0 + (size_t)lane * pstep] : -INFINITY;
#pragma unroll
      for (int uu = 0; uu < 4; ++uu)
        pre_v[i][uu] = lv && uu < S ? *(const bf16x8*)((const bf16_t*)opart + (q0 + (size_t)uu * pstep) * CB_DC + 8 * lane)
                                    : bf16x8{};
    }
  };

  // Row blocks rg * passes + p, one after the other: W^UV_i stays in LDS.
  for (int pass = 0; pass < a.passes; ++pass) {
    const int rb = rg * a.passes + pass;
    if (rb >= nrb) break;
    // 1. merge: wave w, rows w + 8i of the block; lane l, channels 8l .. +7
    size_t p0[4];
    float M[4], invW[4], wt0[4];
    bool live[4];
    // lse of split `lane` for the four rows at once (one round trip), then the
    // maxima and sums (splits 64.. only when there are more than 64)
    float lt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = CB_ROWS * rb + wave + CB_WAVES * i;
      live[i] = row < a.R;
      const int b = live[i] ? row / a.s_q : 0, j = live[i] ? row % a.s_q : 0;
      p0[i] = (((size_t)b * S) * a.s_q + j) * a.H + head;
      if (have_pre)
        lt[i] = pre_lt[i];
      else
        lt[i] = live[i] && lane < S ? lpart[p0[i] + (size_t)lane * pstep] : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = lt[i];
      if (live[i])
        for (int s = 64 + lane; s < S; s += 64) m = fmaxf(m, lpart[p0[i] + s * pstep]);
      M[i] = wmax(m);
      // lane t's weight of split t (0 for empty splits, whose rows are never read)
      wt0[i] = lt[i] == -INFINITY ? 0.0f : exp2f(lt[i] - M[i]);
      float w = wt0[i];
      if (live[i])
        for (int s = 64 + lane; s < S; s += 64) {
          const float l = lpart[p0[i] + s * pstep];
          w += l == -INFINITY ? 0.0f : exp2f(l - M[i]);
        }
      const float W = wsum(w);
      invW[i] = W > 0.0f ? 1.0f / W : 0.0f;
      if (a.lse_out && live[i] && lane == 0) {
        const int row = CB_ROWS * rb + wave + CB_WAVES * i;
        a.lse_out[(size_t)row * a.H + head] = W > 0.0f ? (M[i] + log2f(W)) * 0.6931471805599453f : -INFINITY;
      }
    }
    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
    if (have_pre) {
      // the prefetched rows: the sums of the four-row path below, in its order
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
          const float w = __shfl(wt0[i], uu, 64);  // 0 past the splits (lanes >= S hold 0)
          const bf16x8 v = w != 0.0f ? pre_v[i][uu] : bf16x8{};
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][e] += w * (float)v[e];
        }
    } else if (pbf16 && !live[1]) {
      // One row on this wave (at most 8 rows per block): sixteen splits in
      // flight at a time instead of four, so that a long split list costs a
      // quarter of the memory round trips.
      for (int s0 = 0; s0 < S; s0 += 64) {
        const int n = min(64, S - s0);
        float wt = wt0[0];
        if (s0 > 0) {  // more than 64 splits
          const float l = live[0] && lane < n ? lpart[p0[0] + (size_t)(s0 + lane) * pstep] : -INFINITY;
          wt = l == -INFINITY ? 0.0f : exp2f(l - M[0]);
        }
        for (int u0 = 0; u0 < n; u0 += 16) {
          float w[16];
          bf16x8 v[16];
#pragma unroll
          for (int uu = 0; uu < 16; ++uu) {
            w[uu] = __shfl(wt, u0 + uu, 64);  // 0 past the group (lanes >= n hold 0)
            v[uu] = bf16x8{};
            if (w[uu] != 0.0f)
              v[uu] = *(const bf16x8*)((const bf16_t*)opart + (p0[0] + (size_t)(s0 + u0 + uu) * pstep) * CB_DC + 8 * lane);
          }
#pragma unroll
          for (int uu = 0; uu < 16; ++uu)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[0][e] += w[uu] * (float)v[uu][e];
        }
      }
    } else if (pbf16) {
      // Splits four at a time, the loads of all four rows together; lane t of
      // a 64-split group holds split t's weight.
      for (int s0 = 0; s0 < S; s0 += 64) {
        const int n = min(64, S - s0);
        float wt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (s0 == 0) {
            wt[i] = wt0[i];
          } else {  // more than 64 splits
            const float l = live[i] && lane < n ? lpart[p0[i] + (size_t)(s0 + lane) * pstep] : -INFINITY;
            wt[i] = l == -INFINITY ? 0.0f : exp2f(l - M[i]);
          }
        }
        for (int u0 = 0; u0 < n; u0 += 4) {
          float w[4][4];
          bf16x8 v[4][4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int uu = 0; uu < 4; ++uu) {
              w[i][uu] = __shfl(wt[i], u0 + uu, 64);  // 0 past the group (lanes >= n hold 0)
              v[i][uu] = bf16x8{};
              if (w[i][uu] != 0.0f)
                v[i][uu] = *(const bf16x8*)((const bf16_t*)opart + (p0[i] + (size_t)(s0 + u0 + uu) * pstep) * CB_DC + 8 * lane);
            }
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int uu = 0; uu < 4; ++uu)
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[i][e] += w[i][uu] * (float)v[i][uu][e];
        }
      }
    } else {
      // fp32 partials (written by the portable attention)
      for (int i = 0; i < 4; ++i) {
        if (!live[i]) continue;
        for (int s = 0; s < S; ++s) {
          const float l = lpart[p0[i] + s * pstep];
          if (l == -INFINITY) continue;
          const float w = exp2f(l - M[i]);
          const float* src = (const float*)opart + (p0[i] + s * pstep) * CB_DC + 8 * lane;
          const f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[i][e] += w * x0[e];
            acc[i][4 + e] += w * x1[e];
          }
        }
      }
    }
    // merged rows (bf16) to the O_lat tile; rows past R are zero
    if constexpr (F8) {
      // the bf16 rows quantised in 1 x 128 tiles (16 lanes a tile): scale
      // s = amax / 448 (1 for an all-zero tile), code = E4M3 of x / s
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wave + CB_WAVES * i;
        float x[8], am = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = (float)(bf16_t)(acc[i][e] * invW[i]);
          am = fmaxf(am, fabsf(x[e]));
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
        const float sc = am > 0.0f ? am / 448.0f : 1.0f;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) lo |= (uint32_t)f32_to_e4m3(x[e] / sc) << (8 * e);
#pragma unroll
        for (int e = 0; e < 4; ++e) hi |= (uint32_t)f32_to_e4m3(x[4 + e] / sc) << (8 * e);
        *(__attribute__((address_space(3))) i32x2*)(lds + 512 * m + 16 * ((lane >> 1) ^ (m & 15)) + 8 * (lane & 1)) =
            i32x2{(int)lo, (int)hi};
        if ((lane & 15) == 0) *(__attribute__((address_space(3))) float*)(lds + CB8_S_OFF + 4 * (4 * m + (lane >> 4))) = sc;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wave + CB_WAVES * i;
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16_t)(acc[i][e] * invW[i]);
        *(lbf16x8*)(lds + 1024 * m + 16 * (lane ^ (m & 15))) = o;
      }
    }
    // this wave's W^UV copies (issued first; the merge's loads, already
    // consumed, waited for them in practice), before any prefetch goes out
    if (pass == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    have_pre = false;
    if (pf && pass + 1 < a.passes && rb + 1 < nrb) {
      prefetch(rb + 1);
      have_pre = true;
    }
    __syncthreads();

    // 2. out tile [32 m][128 n] = O_lat W^UV_i^T: wave w, row block w&1,
    // column blocks 2(w>>1), 2(w>>1)+1; K = d_c in 16 k-steps.
    const int mb = wave & 1, nb0 = 2 * (wave >> 1);
    f32x4 c[2] = {f32x4{}, f32x4{}};
    if constexpr (F8) {
      // per k-block j: the integer-grid partial of one 16 x 16 x 128 product,
      // promoted by the weight block's scale times the row tile's scale
      const int ma = 16 * mb + i16;
      const lu8* arow = lds + 512 * ma;
      const lu8* brow0 = lds + CB8_W_OFF + 512 * (16 * nb0 + i16);
      const lu8* brow1 = brow0 + 512 * 16;
      const float* sw = a.Ws + (size_t)head * (CB_DC / 128);
#pragma unroll
      for (int j = 0; j < CB_DC / 128; ++j) {
        const int s0 = (8 * j + g) ^ i16, s1 = (8 * j + 4 + g) ^ i16;  // k = 128 j + 16 g .., 128 j + 64 + 16 g ..
        const i32x8 xq = frag8(arow, s0, s1), w0 = frag8(brow0, s0, s1), w1 = frag8(brow1, s0, s1);
        const float xs = *(const __attribute__((address_space(3))) float*)(lds + CB8_S_OFF + 4 * (4 * ma + j));
        const f32x4 p0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w0, xq, f32x4{}, 0, 0, 0, 0, 0, 0);
        const f32x4 p1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w1, xq, f32x4{}, 0, 0, 0, 0, 0, 0);
        c[0] += (sw[j] * xs) * p0;
        c[1] += (sw[j] * xs) * p1;
      }
    } else {
      const int ma = 16 * mb + i16;
      const lu8* arow = lds + 1024 * ma;
      const lu8* brow0 = lds + CB_W_OFF + 1024 * (16 * nb0 + i16);
      const lu8* brow1 = brow0 + 1024 * 16;
      // (rows 16nb + i16 all have (row & 15) == i16)
#pragma unroll
      for (int ks = 0; ks < CB_DC / 32; ++ks) {
        const int slot = (4 * ks + g) ^ i16;
        const bf16x8 av = *(const lbf16x8*)(arow + 16 * slot);
        const bf16x8 b0 = *(const lbf16x8*)(brow0 + 16 * slot);
        const bf16x8 b1 = *(const lbf16x8*)(brow1 + 16 * slot);
        c[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0, av, c[0], 0, 0, 0);
        c[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1, av, c[1], 0, 0, 0);
      }
    }
    // C = out^T tile: lane holds columns n = 16 nb + 4g + r (r = 0..3) of row
    // m = 16 mb + i16.  Staged in the (dead) O_lat tile as [32 m][128 n] bf16,
    // then one 16-byte store per thread.
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = (bf16_t)c[t][r];
      const int m = 16 * mb + i16, n = 16 * (nb0 + t) + 4 * g;
      *(__attribute__((address_space(3))) bf16x4*)(lds + (m * CB_DV + n) * 2) = o;
    }
    __syncthreads();
    {
      const int m = threadIdx.x >> 4, q = threadIdx.x & 15;  // 32 rows x 16 chunks
      const int row = CB_ROWS * rb + m;
      if (row < a.R)
        *(bf16x8*)(a.out + ((size_t)row * a.H + head) * CB_DV + 8 * q) = *(const lbf16x8*)(lds + (m * CB_DV + 8 * q) * 2);
    }
    __syncthreads();  // the staged rows are out before the next pass writes its tile
  }
}

}  // namespace

// Up to 64 rows always; up to 512 rows while there are at most 4 splits to
// merge (each wave merges four rows, four splits at a time: with more splits
// the one-wave-per-row merge of the general path keeps more loads in flight).
// Measured at 256 rows: 2 splits 60 -> 49 us of combine, 4 splits 65.7 ->
// 64.9 us; at 128 rows of 16 splits 47.2 -> 48.4 us, so that case stays on
// the general path.
bool merge_uv_supported(const mla_dims& d, int R, int S) {
  return R >= 1 && (R <= 2 * CB_ROWS || (R <= 16 * CB_ROWS && S <= 4)) && d.d_c == CB_DC && d.d_head == CB_DV;
}

// 32-row blocks a workgroup takes in turn: as many as keep the grid at one
// workgroup per CU (at 256 rows, 1024 workgroups of one row block each
// streamed W^UV_i into LDS eight times a head).
int merge_uv_passes(int H, int nrb) {
  const int nrg = std::min(nrb, std::max(1, 256 / H));  // row groups a head
  return (nrb + nrg - 1) / nrg;
}

// Merge + W^UV: grid H x ceil(R / (32 passes)).
hipError_t merge_uv(const CombineArgs& a) {
  const int R = a.batch * a.s_q, H = a.d.n_heads;
  const int nrb = (R + CB_ROWS - 1) / CB_ROWS, passes = merge_uv_passes(H, nrb), nrg = (nrb + passes - 1) / passes;
  if ((H * nrg) % 8 != 0) return hipErrorInvalidValue;
  CbArgs cb{a.batch, a.s_q, H, R, a.S, a.ws, a.L.lpart, (const bf16_t*)a.W_UV, (bf16_t*)a.out, a.lse_out,
            nullptr, nullptr, passes};
  MLA_TRY(lds_limit((const void*)&k_merge_uv<false>, CB_LDS));
  return launch(&k_merge_uv<false>, dim3(H * nrg), dim3(CB_WAVES * 64), CB_LDS, a.stream, cb);
}

// The same on E4M3 W^UV (codes [H][d_head][d_c], one scale per 128 x 128
// block, so [H][d_c / 128]): the merged rows are quantised in 1 x 128 tiles
// in LDS and each k-block's product is promoted by its two scales.
hipError_t merge_uv_f8(const CombineArgs& a, const uint8_t* uv_c, const float* uv_s) {
  const int R = a.batch * a.s_q, H = a.d.n_heads;
  const int nrb = (R + CB_ROWS - 1) / CB_ROWS, passes = merge_uv_passes(H, nrb), nrg = (nrb + passes - 1) / passes;
  if ((H * nrg) % 8 != 0) return hipErrorInvalidValue;
  CbArgs cb{a.batch, a.s_q, H, R, a.S, a.ws, a.L.lpart, nullptr, (bf16_t*)a.out, a.lse_out, uv_c, uv_s, passes};
  MLA_TRY(lds_limit((const void*)&k_merge_uv<true>, CB8_LDS));
  return launch(&k_merge_uv<true>, dim3(H * nrg), dim3(CB_WAVES * 64), CB8_LDS, a.stream, cb);
}

}  // namespace mla

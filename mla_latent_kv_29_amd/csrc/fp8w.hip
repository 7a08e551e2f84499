// Decode step with FP8 block-scaled projection weights (gfx950).
//
// The pages' FP8 GEMM scheme ("Читаем техотчёт DeepSeek-V3 вместе", §3.3
// "Обучение в FP8", items 2-4; the same in the "Báo cáo Kỹ thuật
// DeepSeek-V3" summary): E4M3 codes, weights in 128 x 128 blocks and
// activations in 1 x 128 tiles, each group with its own fp32 scale
// s = amax / 448, and each 128-wide partial product promoted into an fp32
// sum with its two scales.  Here it is applied to the four projections of
// the absorbed decode step (lesson §2.1.1 and its Question 2):
//
//   c^Q = W^DQ h                    fp8_gemm (one GEMM over all rows)
//   u   = W^UQ c^Q = [q^C_i ; q^R_i]                 k_skinny_f8 (fp8w_uq), whose
//   qt_i[d_c:]  = tau log2(e) RoPE(q^R_i)            epilogue rotates the RoPE pairs
//   qt_i[:d_c]  = tau log2(e) W^UK_i^T q^C_i         k_f8_heads (per head)
//   ... the attention of the bf16 step, unchanged, on qt and the cache ...
//   out_i = W^UV_i O_lat_i                           k_merge_uv<true> (merge +
//                                                    W^UV), or k_merge, k_f8_heads
//
// k_f8_heads is the per-head form of the block-scaled GEMM for at most 64
// rows a block: Y[m][i][n] = alpha sum_kb sx[m][i][kb] sw[i][n/128][kb]
// (Xq[m][i][kb] . Wq[i][n][kb]) with the activations X[m][i][:] quantised in
// 1 x 128 tiles inside the kernel (s = amax / 448 in fp32, code = RNE of
// x / s saturated, exactly as k_quant_x does).  One
// v_mfma_scale_f32_16x16x128_f8f6f4 per (16 columns, 16 rows, k-block)
// gives the integer-grid partial of a whole block, which the two scales
// promote into the fp32 sum.
#include "internal.hpp"

namespace mla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct F8HeadsArgs {
  int M;                  // rows
  const bf16_t* X;        // X[m][i][k] at X + m ldx + i hx + k
  long ldx, hx;
  const uint8_t* Wc;      // [H][N][K] E4M3 codes
  const float* Ws;        // [H][N / 128][K / 128] scales
  bf16_t* Y;              // Y[m][i][n] at Y + m ldy + i hy + n
  long ldy, hy;
  float alpha;
};

constexpr int FH_SPLIT = 2;  // column halves per head (blocks per head and row group)

// Grid (H, FH_SPLIT, ceil(M / 64)), 4 waves.  K = 128 KB; N = 128 NBW: each
// block owns N / 2 columns, each wave NBW column blocks of 16 of them.  The
// weight fragments of the wave go out first; then the block quantises its
// 64 rows of X into LDS (16 lanes a tile, 8 values a lane), and every wave
// reads its operand fragments from there.
template <int KB, int NBW>
__global__ __launch_bounds__(256) void k_f8_heads(F8HeadsArgs a) {
  constexpr int K = 128 * KB, N = 128 * NBW, LD = K + 16;  // LDS row pitch: 16-byte reads of 16 rows hit 16 bank groups
  __shared__ __attribute__((aligned(16))) uint8_t xc[64 * LD];
  __shared__ float xs[64][KB];
  const int head = blockIdx.x, half = blockIdx.y, m0 = blockIdx.z * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, i16 = lane & 15;

  // weight rows n = 16 nb + i16 of the wave's column blocks; a lane's 32 bytes
  // of k-block j are k = 128 j + 16 g .. +15 and 128 j + 64 + 16 g .. +15
  const uint8_t* wh = a.Wc + (long)head * N * K;
  const float* sh = a.Ws + (long)head * NBW * KB;
  i32x8 wf[NBW][KB];
  int nbs[NBW];
#pragma unroll
  for (int c = 0; c < NBW; ++c) {
    const int nb = (half * 4 + wave) * NBW + c;  // column block of 16 within the head
    nbs[c] = nb;
    const uint8_t* wp = wh + (long)(16 * nb + i16) * K + 16 * g;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const uint4 lo = *(const uint4*)(wp + 128 * j);
      const uint4 hi = *(const uint4*)(wp + 128 * j + 64);
      wf[c][j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }

  // quantise rows m0 .. m0 + 63 (clamped to M - 1: rows past M are computed
  // and never stored) of this head, tile (row r, k-block j) by 16 lanes;
  // a thread's 4 KB tiles t = tid/16 + 16 n, all loads issued before the first use
  {
    constexpr int NT = 4 * KB;
    const int q = threadIdx.x & 15;
    bf16x8 xv[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int t = (threadIdx.x >> 4) + 16 * n, r = t / KB, j = t % KB;
      const int m = min(m0 + r, a.M - 1);
      xv[n] = *(const bf16x8*)(a.X + (long)m * a.ldx + (long)head * a.hx + 128 * j + 8 * q);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int t = (threadIdx.x >> 4) + 16 * n, r = t / KB, j = t % KB;
      const bf16x8 x = xv[n];
      float am = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf((float)x[e]));
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
      const float sc = am > 0.0f ? am / 448.0f : 1.0f;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) lo |= (uint32_t)f32_to_e4m3((float)x[e] / sc) << (8 * e);
#pragma unroll
      for (int e = 0; e < 4; ++e) hi |= (uint32_t)f32_to_e4m3((float)x[4 + e] / sc) << (8 * e);
      *(uint2*)(xc + r * LD + 128 * j + 8 * q) = make_uint2(lo, hi);
      if (q == 0) xs[r][j] = sc;
    }
  }
  __syncthreads();

  i32x8 xq[4][KB];
  float xsv[4][KB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int r = 16 * mb + i16;
      const uint4 lo = *(const uint4*)(xc + r * LD + 128 * j + 16 * g);
      const uint4 hi = *(const uint4*)(xc + r * LD + 128 * j + 64 + 16 * g);
      xq[mb][j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      xsv[mb][j] = xs[r][j];
    }

#pragma unroll
  for (int c = 0; c < NBW; ++c) {
    const int nb = nbs[c];
    f32x4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{};
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const float sw = sh[(nb >> 3) * KB + j];  // 128-row block nb / 8 of the head
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[c][j], xq[mb][j], f32x4{}, 0, 0, 0, 0, 0, 0);
        acc[mb] += (sw * xsv[mb][j]) * p;
      }
    }
    // C = Y^T: lane holds n = 16 nb + 4 g + r (r = 0..3), row 16 mb + i16
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + 16 * mb + i16;
      if (m < a.M) {
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = (bf16_t)(a.alpha * acc[mb][r]);
        *(bf16x4*)(a.Y + (long)m * a.ldy + (long)head * a.hy + 16 * nb + 4 * g) = o;
      }
    }
  }
}

// E4M3 quantisation of the transposes of `batch` matrices W[b][R][C] (bf16)
// in 128 x 128 blocks: codes [b][C][R], scales [b][C / 128][R / 128], i.e.
// k_quant_w applied to each W[b]^T (a block of W^T is the transpose of a
// block of W, with the same amax).  One 256-thread block per 128 x 128
// block, staged through LDS: thread t reads row t/2, half t&1 of the source
// block and writes row t/2, half t&1 of the transposed codes.
__global__ __launch_bounds__(256) void k_quant_wt(int R, int C, const bf16_t* __restrict__ W,
                                                  uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ bf16_t blk[128][136];  // the source block (bf16 is exact; 272-byte rows spread the column reads)
  __shared__ float red[4];
  const int c0 = blockIdx.x * 128, r0 = blockIdx.y * 128, b = blockIdx.z;
  const int row = threadIdx.x >> 1, h = 64 * (threadIdx.x & 1);
  const bf16_t* src = W + ((long)b * R + r0 + row) * C + c0 + h;
  float am = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const bf16x8 x = *(const bf16x8*)(src + 8 * q);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      blk[row][h + 8 * q + e] = x[e];
      am = fmaxf(am, fabsf((float)x[e]));
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = am > 0.0f ? am / 448.0f : 1.0f;
  // transposed row `row` = source column c0 + row, codes for source rows r0 + h ..
  uint8_t* dst = codes + ((long)b * C + c0 + row) * R + r0 + h;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t u = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) u |= (uint32_t)f32_to_e4m3((float)blk[h + 16 * q + 4 * i + e][row] / sc) << (8 * e);
      w4[i] = u;
    }
    *(uint4*)(dst + 16 * q) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
  if (threadIdx.x == 0) scales[((long)b * (C / 128) + blockIdx.x) * (R / 128) + blockIdx.y] = sc;
}

template <int KB, int NBW>
hipError_t launch_heads(const F8HeadsArgs& f, int H, hipStream_t st) {
  return launch(&k_f8_heads<KB, NBW>, dim3(H, FH_SPLIT, (f.M + 63) / 64), dim3(256), 0, st, f);
}

}  // namespace

hipError_t fp8_quantize_weight_t(int batch, int R, int C, const bf16_t* W, uint8_t* codes, float* scales,
                                 hipStream_t st) {
  return launch(&k_quant_wt, dim3(C / 128, R / 128, batch), dim3(256), 0, st, R, C, W, codes, scales);
}

bool fp8w_supported(const mla_dims& d) {
  return d.d_head == 128 && d.d_c == 512 && d.d_rope == 64 && fp8_gemm_supported(d.d_cq, d.d_model) &&
         fp8_gemm_supported(d.n_heads * (d.d_head + d.d_rope), d.d_cq);
}

// The workspace of the bf16 step (the attention and the combine use its
// regions unchanged) followed by the FP8 GEMMs' scratch.
size_t fp8w_scratch_offset(const WsLayout& L) { return align256(L.total); }
size_t fp8w_scratch_bytes(const mla_dims& d, int R) {
  const F8Plan a = fp8_plan(R, d.d_cq, d.d_model), b = fp8_plan(R, d.n_heads * (d.d_head + d.d_rope), d.d_cq);
  return align256(a.ws_bytes > b.ws_bytes ? a.ws_bytes : b.ws_bytes);
}

// c^Q, u with its RoPE tail, and the absorption: qt of the bf16 step.
hipError_t fp8w_query(const DecodeArgs& a, const Fp8Weights& w) {
  const mla_dims& d = a.d;
  const int R = a.batch * a.s_q, H = d.n_heads;
  uint8_t* f8ws = a.ws + fp8w_scratch_offset(a.L);
  bf16_t* cq = (bf16_t*)(a.ws + a.L.cq);
  bf16_t* qc = (bf16_t*)(a.ws + a.L.u);  // q^C [R][H][d_head] in the (fp32-sized) u region
  bf16_t* qt = (bf16_t*)(a.ws + a.L.qt);
  MLA_TRY(fp8_gemm(R, d.d_cq, d.d_model, (const bf16_t*)a.hq, w.dq_c, w.dq_s, cq, f8ws, a.stream));
  MLA_TRY(fp8w_uq(a, w.uq_c, w.uq_s, cq, qc, f8ws));
  // absorption: X = q^C_i, W = (W^UK_i)^T [d_c][d_head]
  const F8HeadsArgs f{R, qc, (long)H * d.d_head, d.d_head, w.ukt_c, w.ukt_s, qt, (long)H * (d.d_c + d.d_rope),
                      d.d_c + d.d_rope, a.scale * 1.4426950408889634f};
  return launch_heads<1, 4>(f, H, a.stream);
}

// The merge of the split partials (O_lat and the lse) as in the bf16 step,
// then out_i = W^UV_i O_lat_i on the FP8 weight: in one kernel where the
// bf16 step fuses the two, else k_merge into O_lat and k_f8_heads.
hipError_t fp8w_combine(const CombineArgs& a, const uint8_t* uv_c, const float* uv_s) {
  const mla_dims& d = a.d;
  const int R = a.batch * a.s_q, H = d.n_heads;
  if (merge_uv_supported(d, R, a.S)) return merge_uv_f8(a, uv_c, uv_s);
  MLA_TRY(merge_partials(a));
  const F8HeadsArgs f{R, (const bf16_t*)(a.ws + a.L.olat), (long)H * d.d_c, d.d_c, uv_c, uv_s, (bf16_t*)a.out,
                      (long)H * d.d_head, d.d_head, 1.0f};
  return launch_heads<4, 1>(f, H, a.stream);
}

}  // namespace mla

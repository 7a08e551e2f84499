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
//   u   = W^UQ c^Q = [q^C_i ; q^R_i]                 k_uqa_f8 (at most 64 rows), or
//   qt_i[d_c:]  = tau log2(e) RoPE(q^R_i)            k_skinny_f8 with a RoPE epilogue
//   qt_i[:d_c]  = tau log2(e) W^UK_i^T q^C_i         and k_f8_heads (per head)
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

// ------------------------------------------------------------ W^UQ + RoPE + absorption
// For at most 64 rows, one block per (head i, half e of d_c), 8 waves: the
// FP8 form of the bf16 step's fused W^UQ kernel.
//   1. u_i = Q(c^Q) . Q(W^UQ_i)^T for the head's 128 content rows and the 32
//      RoPE rows of half e.  The c^Q codes and tile scales come from the
//      W^DQ GEMM's k-group sum (k_reduce_quant), straight into the registers
//      that feed the MFMA (quantising c^Q here would repeat it in every
//      block: 256 times the conversions, which measured slower than the
//      whole step it replaces).  The W^UQ codes
//      stream HBM -> LDS in 24 KiB units (16 rows x d_cq) through a 5-slot
//      ring with global_load_lds.  Content sums, rounded to bf16, stay in LDS
//      as the q^C_i tile; the RoPE pairs are rotated at the row's position,
//      scaled by tau log2 e and written to the tail of qt.
//   2. The q^C_i rows are quantised (one 1 x 128 tile each) and
//      qt_i[256 e ..] = tau log2 e Q(q^C_i) . Q(W^UK_i^T)^T over the half's 256
//      rows of W^UK_i^T, whose codes (two 16 KiB units) ride the same ring.
// Waves are 4 row blocks x 2 halves of the 12 k-blocks; the pair sums
// through a 1 KiB slab.  Every 128-wide product is one
// v_mfma_scale_f32_16x16x128_f8f6f4 from zero, promoted by the weight
// block's and the activation tile's scales into the fp32 sum.
constexpr int QA_DCQ = 1536, QA_KB = QA_DCQ / 128, QA_KBW = QA_KB / 2;
constexpr int QA_DH = 128, QA_NCOL = 256;
constexpr int QA_UNIT = 16 * QA_DCQ;                  // 24 KiB: 16 W^UQ rows
constexpr int QA_NB = QA_DH / 16 + 2;                 // W^UQ units: 8 content + 2 RoPE
constexpr int QA_UNITS = QA_NB + 2;                   // + two W^UK^T units of 128 rows x 128 B
constexpr int QA_SLOTS = 5;
constexpr int QA_QC_LD = QA_DH + 8;                   // q^C tile row, bf16
constexpr int QA_QC_OFF = QA_SLOTS * QA_UNIT;
constexpr int QA_SLAB_OFF = QA_QC_OFF + 64 * QA_QC_LD * 2;
constexpr int QA_LDS = QA_SLAB_OFF + 2 * 4 * 1024;
constexpr int QA_STAGE_OFF = 2 * QA_UNIT;             // output [64][256] bf16: slots 2-3
constexpr int QA_CODE_OFF = 4 * QA_UNIT;              // q^C codes [64][128]: slot 4
constexpr int QA_SC_OFF = QA_CODE_OFF + 64 * 128;     // q^C tile scales [64]
static_assert(QA_LDS <= 160 * 1024, "LDS");
static_assert(QA_STAGE_OFF + 64 * QA_NCOL * 2 <= QA_CODE_OFF && QA_SC_OFF + 256 <= QA_QC_OFF, "slots 2-4");
static_assert(QA_NB % QA_SLOTS == 0, "the W^UK^T units land in slots 0 and 1");

typedef __attribute__((address_space(3))) uint8_t lu8;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x4 li32x4;

template <int N>
__device__ __forceinline__ void qa_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One 1 KiB wave-instruction of a global -> LDS copy (16 bytes a lane at
// gbase + voff, to LDS lds_addr + 16 lane), from asm so that the compiler's
// wait accounting leaves it alone (it would otherwise wait for every copy in
// flight before each LDS read); the kernel waits (vmcnt) explicitly.
// Nothing else in k_uqa_f8 uses M0.
__device__ __forceinline__ void qa_dma(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds_addr)
               : "memory");
}

// 32 code bytes of an MFMA operand from two 16-byte LDS chunks
__device__ __forceinline__ i32x8 qa_frag(const lu8* base, uint32_t o0, uint32_t o1) {
  const i32x4 lo = *(const li32x4*)(base + o0), hi = *(const li32x4*)(base + o1);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Rows of 128 code bytes (W^UK^T units, the q^C codes): chunk c of row r at
// slot c ^ ((r >> 1) & 7), so that the 16 rows of an operand read fill all
// 64 banks.
__device__ __forceinline__ uint32_t qa_row128(int r, int c) { return 128 * r + 16 * (c ^ ((r >> 1) & 7)); }

struct QaArgs {
  int M, H, d_c, d_rope, s_q;
  const uint8_t* Xc;       // c^Q codes [M][d_cq]
  const float* Xs;         // c^Q tile scales [M][d_cq / 128]
  const uint8_t* Wuq;      // W^UQ codes [H (d_head + d_rope)][d_cq]
  const float* Suq;        // [H (d_head + d_rope) / 128][d_cq / 128]
  const uint8_t* Wukt;     // W^UK_i^T codes [H][d_c][d_head]
  const float* Sukt;       // [H][d_c / 128]
  bf16_t* qt;              // [M][H][d_c + d_rope]
  const int32_t* seqlens;  // position of row m = b s_q + j: seqlens[b] - s_q + j
  float scale2;            // tau log2 e
  double freq[32];         // theta^(-2p/d_rope) of RoPE pair p
};

struct QaCtx {
  const uint8_t *wq, *wk;  // W^UQ_i rows, W^UK_i^T rows of half e
  uint32_t ring;
  int wave, lane, e;
};

// Unit u into slot u % 5: W^UQ units as 24 wave-instructions (rows 2(j/3),
// 2(j/3)+1, chunks 32(j%3) .. +31 of the row's 96; chunk c of row r at slot
// c ^ (r & 15) of its run), W^UK^T units as 16 (8 rows each).
__device__ __forceinline__ void qa_issue(const QaCtx& c, int u) {
  if (u >= QA_UNITS) return;
  const uint32_t dst = c.ring + (u % QA_SLOTS) * QA_UNIT;
  if (u < QA_NB) {
    const int row0 = u < QA_DH / 16 ? 16 * u : QA_DH + 32 * c.e + 16 * (u - QA_DH / 16);
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) {
      const int j = c.wave + 8 * jj;
      const int r = 2 * (j / 3) + (c.lane >> 5), s = 32 * (j % 3) + (c.lane & 31);
      qa_dma(c.wq, (uint32_t)((row0 + r) * QA_DCQ + 16 * (s ^ (r & 15))), dst + 1024 * j);
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int t = c.wave + 8 * jj, r = 8 * t + (c.lane >> 3), sl = c.lane & 7;
      const int ch = sl ^ ((r >> 1) & 7);
      qa_dma(c.wk, (uint32_t)((128 * (u - QA_NB) + r) * QA_DH + 16 * ch), dst + 1024 * t);
    }
  }
}

__global__ __launch_bounds__(512) void k_uqa_f8(QaArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lu8* lds = (lu8*)lds_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, i16 = lane & 15;
  const int rb = wave >> 1, kq = wave & 1;
  // blocks are dealt to the 8 XCDs round-robin: the two halves of a head are
  // consecutive blocks of one XCD (the second reads the content rows from L2)
  const int xcd = blockIdx.x & 7, ub = blockIdx.x >> 3;
  const int head = xcd * (gridDim.x >> 4) + (ub >> 1), e = ub & 1;
  const int wrow0 = head * (QA_DH + a.d_rope);  // first W^UQ row of the head

  // The row's position and the lane's four RoPE frequencies (pairs of
  // columns 32 e + 16 j + 4 g, +2); the first four units; the c^Q rows
  // 16 rb + i16 (clamped: rows past M are computed, never stored), the lane's
  // 32 codes of each of k-blocks 6 kq .. 6 kq + 5 and their scales.  All of
  // it is waited for at once, so that no wait of the compiler's later drains
  // the ring.
  const int m = 16 * rb + i16;
  const int sl = m < a.M ? a.seqlens[m / a.s_q] : 0;
  double fr[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) fr[j][h] = a.freq[16 * e + 8 * j + 2 * g + h];
  QaCtx c;
  c.wq = a.Wuq + (long)wrow0 * QA_DCQ;
  c.wk = a.Wukt + ((long)head * a.d_c + QA_NCOL * e) * QA_DH;
  c.ring = (uint32_t)(uintptr_t)lds;
  c.wave = wave;
  c.lane = lane;
  c.e = e;
#pragma unroll
  for (int u = 0; u < QA_SLOTS - 1; ++u) qa_issue(c, u);
  // weight scales, one a lane: lane 6 u + jj holds unit u's scale of k-block
  // 6 kq + jj, lanes 60 and 61 the two W^UK^T block scales of the half (read
  // back with readlane: loads in the loop would make the compiler wait for
  // every copy in flight)
  float swl = 1.0f;
  if (lane < 6 * QA_NB) {
    const int u = lane / 6, row0 = u < QA_DH / 16 ? 16 * u : QA_DH + 32 * e + 16 * (u - QA_DH / 16);
    swl = a.Suq[(long)((wrow0 + row0) >> 7) * QA_KB + QA_KBW * kq + lane % 6];
  } else if (lane < 6 * QA_NB + 2) {
    swl = a.Sukt[(long)head * (a.d_c / 128) + 2 * e + lane - 6 * QA_NB];
  }
  i32x8 xq[QA_KBW];
  float xs[QA_KBW];
  {
    const long row = min(m, a.M - 1);
    const uint8_t* x = a.Xc + row * QA_DCQ + 128 * QA_KBW * kq + 16 * g;
#pragma unroll
    for (int jj = 0; jj < QA_KBW; ++jj) {
      const i32x4 lo = *(const i32x4*)(x + 128 * jj), hi = *(const i32x4*)(x + 128 * jj + 64);
      xq[jj] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      xs[jj] = a.Xs[row * QA_KB + QA_KBW * kq + jj];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  qa_wait_vmcnt<0>();

  // LDS offsets of the lane's weight fragments in a unit: row i16, chunks
  // 8 j + g and 8 j + 4 + g of k-block j = 6 kq + jj
  uint32_t ao[QA_KBW][2];
#pragma unroll
  for (int jj = 0; jj < QA_KBW; ++jj)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = 8 * (QA_KBW * kq + jj) + 4 * h + g, s = ch ^ i16;
      ao[jj][h] = (uint32_t)(1024 * (3 * (i16 >> 1) + (s >> 5)) + 512 * (i16 & 1) + 16 * (s & 31));
    }
  int ps = m < a.M ? sl - a.s_q + m % a.s_q : 0;
  ps = ps < 0 ? 0 : ps;
  lu8* slab = lds + QA_SLAB_OFF;
  lu8* qct = lds + QA_QC_OFF;

  // unit nb's epilogue (waves kq = 0): the pair's sum, then the q^C tile or
  // the rotated RoPE pairs; lane holds columns 16 nb + 4 g + r of row m
  auto epilogue = [&](int nb, const f32x4& acc) {
    const f32x4 v = acc + *(const __attribute__((address_space(3))) f32x4*)(slab + ((nb & 1) * 4 + rb) * 1024 + 16 * lane);
    if (nb < QA_DH / 16) {
      bf16x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = (bf16_t)v[r];
      *(__attribute__((address_space(3))) bf16x4*)(qct + (m * QA_QC_LD + 16 * nb + 4 * g) * 2) = o;
    } else if (m < a.M) {
      const int j = nb - QA_DH / 16;
      bf16x4 o;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float cs, sn;
        rope_cs_w(ps, fr[j][h], &cs, &sn);
        o[2 * h] = (bf16_t)(a.scale2 * (v[2 * h] * cs - v[2 * h + 1] * sn));
        o[2 * h + 1] = (bf16_t)(a.scale2 * (v[2 * h] * sn + v[2 * h + 1] * cs));
      }
      *(bf16x4*)(a.qt + ((long)m * a.H + head) * (a.d_c + a.d_rope) + a.d_c + 32 * e + 16 * j + 4 * g) = o;
    }
  };

  f32x4 acc = f32x4{};
#pragma unroll 1
  for (int u = 0; u < QA_NB; ++u) {
    // this wave's copies of unit u have landed; younger in flight: units
    // u+1 .. u+3, 3 instructions a W^UQ unit, 2 a W^UK^T unit
    if (u < 7) qa_wait_vmcnt<9>();
    else if (u == 7) qa_wait_vmcnt<8>();
    else if (u == 8) qa_wait_vmcnt<7>();
    else qa_wait_vmcnt<4>();
    ring_barrier();  // everyone's copies of unit u are in; everyone is done with unit u-1 and the slab
    qa_issue(c, u + QA_SLOTS - 1);  // into unit u-1's slot (slot 4 at u = 0)
    if (u > 0 && kq == 0) epilogue(u - 1, acc);
    acc = f32x4{};
    const lu8* sb = lds + (u % QA_SLOTS) * QA_UNIT;
#pragma unroll
    for (int jj = 0; jj < QA_KBW; ++jj) {
      const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa_frag(sb, ao[jj][0], ao[jj][1]), xq[jj],
                                                                      f32x4{}, 0, 0, 0, 0, 0, 0);
      const float sw = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, swl), 6 * u + jj));
      acc += (sw * xs[jj]) * p;
    }
    if (kq == 1) *(__attribute__((address_space(3))) f32x4*)(slab + ((u & 1) * 4 + rb) * 1024 + 16 * lane) = acc;
  }
  qa_wait_vmcnt<0>();  // the W^UK^T units
  ring_barrier();
  if (kq == 0) epilogue(QA_NB - 1, acc);
  ring_barrier();  // the q^C tile is complete

  // 2a. q^C rows to E4M3: thread t, row t / 8, values 16 (t % 8) .. +15
  {
    const int r = threadIdx.x >> 3, q = threadIdx.x & 7;
    const bf16x8 v0 = *(const __attribute__((address_space(3))) bf16x8*)(qct + (r * QA_QC_LD + 16 * q) * 2);
    const bf16x8 v1 = *(const __attribute__((address_space(3))) bf16x8*)(qct + (r * QA_QC_LD + 16 * q + 8) * 2);
    float am = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) am = fmaxf(am, fmaxf(fabsf((float)v0[t]), fabsf((float)v1[t])));
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    const float sc = am > 0.0f ? am / 448.0f : 1.0f;
    uint32_t w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t uu = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int k = 4 * i + t;
        uu |= (uint32_t)f32_to_e4m3((float)(k < 8 ? v0[k] : v1[k - 8]) / sc) << (8 * t);
      }
      w4[i] = uu;
    }
    *(__attribute__((address_space(3))) i32x4*)(lds + QA_CODE_OFF + qa_row128(r, q)) =
        i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
    if (q == 0) *(__attribute__((address_space(3))) float*)(lds + QA_SC_OFF + 4 * r) = sc;
  }
  __syncthreads();

  // 2b. wave w: columns 32 w .. 32 w + 31 of the half's 256 (W^UK^T rows),
  // all 64 rows; K = d_head, one k-block
  f32x4 ab[2][4];
  {
    i32x8 qf[4];
    float qs[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int r = 16 * mb + i16;
      qf[mb] = qa_frag(lds + QA_CODE_OFF, qa_row128(r, g), qa_row128(r, g + 4));
      qs[mb] = *(const __attribute__((address_space(3))) float*)(lds + QA_SC_OFF + 4 * r);
    }
#pragma unroll
    for (int nbi = 0; nbi < 2; ++nbi) {
      const int n = 32 * wave + 16 * nbi + i16;  // W^UK^T row within the half
      const lu8* ub = lds + (n >> 7) * QA_UNIT;   // units 10, 11: slots 0, 1
      const i32x8 wf = qa_frag(ub, qa_row128(n & 127, g), qa_row128(n & 127, g + 4));
      // the 128-row block of the column block
      const float sw = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, swl), 6 * QA_NB + (wave >> 2)));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, qf[mb], f32x4{}, 0, 0, 0, 0, 0, 0);
        ab[nbi][mb] = f32x4{} + (sw * qs[mb]) * p;
      }
    }
  }
  // output rows staged in slots 2-3 as [64 m][256 n] bf16, 16-byte chunk j of
  // row m at j ^ (m & 31); lane holds n = 32 w + 16 nbi + 4 g + r of row
  // m = 16 mb + i16
  {
    lu8* st = lds + QA_STAGE_OFF;
#pragma unroll
    for (int nbi = 0; nbi < 2; ++nbi)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int mm = 16 * mb + i16, n = 32 * wave + 16 * nbi + 4 * g;
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = (bf16_t)(a.scale2 * ab[nbi][mb][r]);
        *(__attribute__((address_space(3))) bf16x4*)(st + mm * QA_NCOL * 2 + 16 * ((n >> 3) ^ (mm & 31)) + 2 * (n & 7)) = o;
      }
  }
  __syncthreads();
  for (int p = threadIdx.x; p < 64 * 32; p += 512) {
    const int mm = p >> 5, j = p & 31;
    if (mm < a.M)
      *(bf16x8*)(a.qt + ((long)mm * a.H + head) * (a.d_c + a.d_rope) + QA_NCOL * e + 8 * j) =
          *(const __attribute__((address_space(3))) bf16x8*)(lds + QA_STAGE_OFF + mm * QA_NCOL * 2 + 16 * (j ^ (mm & 31)));
  }
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
  const float scale2 = a.scale * 1.4426950408889634f;
  if (R <= 64 && d.d_cq == QA_DCQ && H % 8 == 0) {
    // c^Q with its codes (in the u region), then W^UQ, RoPE and the
    // absorption in one kernel
    uint8_t* cqc = a.ws + a.L.u;
    float* cqs = (float*)(cqc + align256((size_t)R * QA_DCQ));
    MLA_TRY(fp8_gemm(R, d.d_cq, d.d_model, (const bf16_t*)a.hq, w.dq_c, w.dq_s, cq, f8ws, a.stream, cqc, cqs));
    QaArgs q{R, H, d.d_c, d.d_rope, a.s_q, cqc, cqs, w.uq_c, w.uq_s, w.ukt_c, w.ukt_s, qt, a.seqlens, scale2, {}};
    for (int p = 0; p < d.d_rope / 2; ++p) q.freq[p] = pow((double)d.rope_theta, -2.0 * p / d.d_rope);
    MLA_TRY(lds_limit((const void*)&k_uqa_f8, QA_LDS));
    return launch(&k_uqa_f8, dim3(2 * H), dim3(512), QA_LDS, a.stream, q);
  }
  MLA_TRY(fp8_gemm(R, d.d_cq, d.d_model, (const bf16_t*)a.hq, w.dq_c, w.dq_s, cq, f8ws, a.stream));
  MLA_TRY(fp8w_uq(a, w.uq_c, w.uq_s, cq, qc, f8ws));
  // absorption: X = q^C_i, W = (W^UK_i)^T [d_c][d_head]
  const F8HeadsArgs f{R, qc, (long)H * d.d_head, d.d_head, w.ukt_c, w.ukt_s, qt, (long)H * (d.d_c + d.d_rope),
                      d.d_c + d.d_rope, scale2};
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

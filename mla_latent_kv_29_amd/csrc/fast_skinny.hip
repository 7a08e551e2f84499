// Weight-streaming GEMMs of the decode projections for at most 64
// activation rows (gfx950).
//
// With M <= 64 rows the projections are reads of the weights and little
// else: every weight byte is used once per decode step.  These kernels keep
// as many weight bytes in flight per CU as the register file allows and
// read each weight byte straight from HBM into the registers that feed the
// MFMA (no LDS staging), while the activations, which every block needs,
// are held in registers too:
//
//   k_skinny   Y = X . W^T with W[N][K] (k contiguous): W^DQ.
//              The waves of a block split K; each wave loads its K-slice of
//              all M rows of X once, then streams W for the block's columns
//              with several column blocks of loads outstanding.  The waves'
//              partial sums meet in LDS (one slab per wave, summed by the
//              epilogue threads).  A grid dimension over K (k-groups) writes
//              fp32 partials that k_reduce_rows sums.
//   k_uq_absorb  q_i = W^UQ_i c^Q for one head (the same split of K over
//              the waves), then qt_i = tau log2(e) q^C_i . W^UK_i with
//              W^UK_i[d_head][d_c] (n contiguous) in LDS, read by the
//              transposing LDS read; q^C_i stays in LDS between the two.
//
// MFMA v_mfma_f32_16x16x32_bf16, C[16][16] += A[16][32] B[32][16]: lane l
// holds row l%16, k 8(l/16)..+7 of A, the same of B^T, and rows 4(l/16)..+3
// of column l%16 of C.  With A = W (rows n) and B = X (rows m), C = Y^T.
#include <math.h>
#include "internal.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct SkArgs {
  int M;              // activation rows (<= 64)
  int kg_len;         // k per k-group = waves * KS * 32
  const bf16_t* W;    // W[batch][N][ldw]
  long ldw, bsw;
};

// Sources of the activation fragments: lane (i16, g) of a wave gets, for
// rows m = 16 mb + i16 (clamped to M-1: rows past M are computed and never
// stored) and k-steps ks, the 8 values at k = k0 + 32 ks (k0 includes 8 g).
struct XPlain {  // X[batch][M][ldx] (bf16)
  const bf16_t* X;
  long ldx, bsx;
  template <int KS>
  __device__ void load(int batch, long k0, int i16, int g, int wave, int M, bf16x8 (&xf)[4][KS]) const {
    const bf16_t* x = X + (long)batch * bsx + k0;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = min(16 * mb + i16, M - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) xf[mb][ks] = *(const bf16x8*)(x + (long)m * ldx + 32 * ks);
    }
  }
};

// Cross-wave reduction: each wave stores its partial C tiles for NBR column
// blocks at a time in its own LDS slab [64 m][NBR*16 n + 4] fp32 (the pad
// spreads the 16-byte stores over the banks); then every thread sums the
// waves for its column pairs and hands them to the epilogue.
template <int WPB, int NB>
struct SkPlan {
  static constexpr int bytes(int nbr) { return (WPB * 64 * (nbr * 16 + 4) + (nbr == NB ? 0 : 64 * (NB * 16 + 2))) * 4; }
  static constexpr int pick() {
    for (int nbr = NB; nbr > 1; --nbr)
      if (NB % nbr == 0 && bytes(nbr) <= 160 * 1024) return nbr;
    return 1;
  }
  static constexpr int NBR = pick();  // column blocks per reduction round
  static constexpr int LDN = NBR * 16 + 4;
  static constexpr int SLAB = 64 * LDN;  // floats per wave
  // with several rounds the sums wait in a final tile [64 m][NB*16 + 2] for
  // the epilogue, which then runs once the registers of the main loop are free
  static constexpr int LDF = NB * 16 + 2;
  static constexpr int FINAL = NBR == NB ? 0 : 64 * LDF;
  static constexpr int LDS_BYTES = (WPB * SLAB + FINAL) * 4;
  static_assert(NB % NBR == 0, "reduction rounds");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Grid (column groups, k-groups, batch); WPB waves of KS k-steps each; NB
// column blocks of 16 per block, DEPTH of them loading ahead.
template <int WPB, int KS, int NB, int DEPTH, class XSrc, class Epi>
__global__ __launch_bounds__(WPB * 64) void k_skinny(SkArgs a, XSrc xs, Epi epi) {
  using P = SkPlan<WPB, NB>;
  extern __shared__ __attribute__((aligned(16))) float slab[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int n0 = blockIdx.x * NB * 16;
  const int kg = blockIdx.y, batch = blockIdx.z;
  const long k0 = (long)kg * a.kg_len + wave * KS * 32 + 8 * g;
  const bf16_t* W = a.W + (long)batch * a.bsw + (long)(n0 + i16) * a.ldw + k0;

  // W rows n0 + 16 nb + i16 of this wave's K-slice, DEPTH column blocks ahead
  bf16x8 wf[DEPTH][KS];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      if (d < NB) wf[d][ks] = *(const bf16x8*)(W + (long)(16 * d) * a.ldw + 32 * ks);
  bf16x8 xf[4][KS];
  xs.template load<KS>(batch, k0, i16, g, wave, a.M, xf);

  float* mine = slab + wave * P::SLAB;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 w = wf[nb % DEPTH][ks];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, xf[mb][ks], acc[mb], 0, 0, 0);
    }
    if (nb + DEPTH < NB) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        wf[nb % DEPTH][ks] = *(const bf16x8*)(W + (long)(16 * (nb + DEPTH)) * a.ldw + 32 * ks);
    }
    // C = Y^T: lane holds n = 16 nb + 4g + r (r = 0..3), m = 16 mb + i16
    const int nr = nb % P::NBR;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) *(f32x4*)(mine + (16 * mb + i16) * P::LDN + 16 * nr + 4 * g) = acc[mb];
    if (nr == P::NBR - 1) {
      ring_barrier();  // every wave's slab holds this round (the weight loads stay in flight)
      constexpr int PAIRS = P::NBR * 8;
      const int c_base = n0 + 16 * (nb + 1 - P::NBR);
      for (int p = threadIdx.x; p < PAIRS * 64; p += WPB * 64) {
        const int m = p / PAIRS, c = 2 * (p % PAIRS);
        float2 v = *(const float2*)(slab + m * P::LDN + c);
#pragma unroll
        for (int w = 1; w < WPB; ++w) {
          const float2 u = *(const float2*)(slab + w * P::SLAB + m * P::LDN + c);
          v.x += u.x;
          v.y += u.y;
        }
        if constexpr (P::FINAL == 0) {
          if (m < a.M) epi(batch, kg, m, c_base + c, v.x, v.y);
        } else {
          *(float2*)(slab + WPB * P::SLAB + m * P::LDF + (c_base - n0) + c) = v;
        }
      }
      ring_barrier();  // the slabs (and final tile) are complete before reuse
    }
  }
  if constexpr (P::FINAL != 0) {
    constexpr int PAIRS = NB * 8;
    const float* fin = slab + WPB * P::SLAB;
    for (int p = threadIdx.x; p < PAIRS * 64; p += WPB * 64) {
      const int m = p / PAIRS, c = 2 * (p % PAIRS);
      const float2 v = *(const float2*)(fin + m * P::LDF + c);
      if (m < a.M) epi(batch, kg, m, n0 + c, v.x, v.y);
    }
  }
}

// ------------------------------------------------------------ epilogues
// fp32 partial of k-group kg: part[kg][m][n]
struct EpiKPart {
  float* part;
  int M, N;
  __device__ void operator()(int, int kg, int m, int n, float v0, float v1) const {
    float2 v = {v0, v1};
    *(float2*)(part + ((long)kg * M + m) * N + n) = v;
  }
};

// Y[m][n] = sum over the k-groups of part[kg][m][n] in k-group order, rounded
// to bf16 (a separate launch: summing inside the GEMM would need device-wide
// fences, which write back and invalidate the L2 of every XCD).
__global__ __launch_bounds__(256) void k_reduce_rows(int MN, int KG, const float* __restrict__ part,
                                                     bf16_t* __restrict__ y) {
  const int i = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (i >= MN) return;
  f32x4 s = *(const f32x4*)(part + i);
  for (int k = 1; k < KG; ++k) s += *(const f32x4*)(part + (long)k * MN + i);
  bf16x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = (bf16_t)s[e];
  *(bf16x4*)(y + i) = o;
}

// ------------------------------------------------------------ W^UQ + absorption
// One block per (head i, half e of d_c), 8 waves:
//   1. u_i = W^UQ_i c^Q for the head's 128 content rows and the 32 RoPE rows
//      of half e (16 pairs), K = d_cq split over the waves as in k_skinny;
//      the content sums, rounded to bf16, stay in LDS as the q^C_i tile, the
//      RoPE pairs are rotated at the row's position, scaled by tau log2 e and
//      written to the tail of qt.
//   2. qt_i[:, 256e .. 256e+255] = tau log2 e q^C_i W^UK_i[:, 256e ..], with
//      the W^UK tile copied to LDS (global_load_lds) while phase 1 streams.
// Both halves of a head read the same content rows of W^UQ; the two blocks
// are placed on one XCD, so the second read is served by that XCD's L2.
// Per block: 491 KiB of W^UQ (393 KiB shared with the partner), 64 KiB of
// W^UK and c^Q (64 x 1536 bf16) from L2.  One launch instead of a W^UQ GEMM
// plus an absorption kernel, and q^C never leaves the CU.
//
// W^UK_i[128 k][512 n] in LDS as 64-column tiles [128 k][64 n]: row k chunk
// q (8 n) at k*8 + (q ^ swz(k)) -- the layout whose transposing reads are
// bank-conflict free.
__device__ __forceinline__ int ab_pos(int k, int q) { return k * 8 + (q ^ (4 * ((k >> 1) & 1)) ^ (2 * ((k >> 3) & 1))); }

constexpr int AB_DH = 128;                     // d_head (k of the absorption)
constexpr int AB_NCOL = 256;                   // absorbed columns per block (half of d_c)
constexpr int AB_TILE = AB_DH * 64 * 2;        // one 64-column W^UK tile, bytes
constexpr int UA_WAVES = 8, UA_KS = 6;         // K = 8 waves x 6 k-steps x 32 = d_cq
constexpr int UA_DCQ = UA_WAVES * UA_KS * 32;  // 1536
constexpr int UA_NOPE_NB = AB_DH / 16;         // content column blocks (8)
constexpr int UA_NB = UA_NOPE_NB + 2;          // + two RoPE column blocks (32 columns)
constexpr int UA_DEPTH = 4;                    // column blocks of W^UQ loads in flight
constexpr int UA_LDN = 2 * 16 + 4;             // slab row, floats (two column blocks per round)
constexpr int UA_SLAB = 64 * UA_LDN;           // floats per wave
constexpr int UA_QC_LD = AB_DH + 8;            // q^C tile row, bf16 (rows 16 bytes apart in the banks)
constexpr int UA_QC_OFF = UA_WAVES * UA_SLAB * 4;
constexpr int UA_W_OFF = UA_QC_OFF + 64 * UA_QC_LD * 2;
constexpr int UA_LDS = UA_W_OFF + 4 * AB_TILE;
static_assert(UA_LDS <= 160 * 1024, "LDS");
static_assert(UA_W_OFF % 1024 == 0, "W^UK tile alignment");
static_assert(64 * AB_NCOL * 2 <= UA_QC_OFF, "output staging fits in the slabs");

typedef __attribute__((address_space(3))) uint8_t lu8;

// One 1 KiB wave-instruction of a global -> LDS copy (16 bytes a lane at
// gbase + voff, to LDS lds_addr + 16 lane).  Issued from asm: the compiler
// cannot tell where such a copy lands, so for the builtin it waits for every
// outstanding load before any later LDS access, which would drain the weight
// stream at each reduction round.  The caller waits (vmcnt) before reading
// the copy.  Nothing else in k_uq_absorb uses M0.
__device__ __forceinline__ void ua_dma(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds_addr)
               : "memory");
}

constexpr int MAX_ROPE_PAIRS = 32;
struct UaArgs {
  int M, H, d_c, d_rope, s_q;
  const bf16_t* X;         // c^Q [M][d_cq]
  const bf16_t* Wuq;       // [H][d_head + d_rope][d_cq], RoPE rows as interleaved pairs
  const bf16_t* Wuk;       // [H][d_head][d_c]
  bf16_t* qt;              // [M][H][d_c + d_rope]
  const int32_t* seqlens;  // position of row m = b s_q + j: seqlens[b] - s_q + j
  float scale2;            // tau log2 e
  double freq[MAX_ROPE_PAIRS];  // theta^(-2p/d_rope) of RoPE pair p
};

__global__ __launch_bounds__(UA_WAVES * 64) void k_uq_absorb(UaArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  float* slab = (float*)lds;
  bf16_t* qct = (bf16_t*)(lds + UA_QC_OFF);
  uint8_t* wt = lds + UA_W_OFF;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, in an SGPR
  const int g = lane >> 4, i16 = lane & 15;
  // Blocks are dealt to the 8 XCDs round-robin: XCD x runs blocks x, x + 8,
  // ...; its consecutive pairs of those are the two halves of one head.
  const int xcd = blockIdx.x & 7, u = blockIdx.x >> 3;
  const int head = xcd * (gridDim.x >> 4) + (u >> 1), e = u & 1;
  const int wd = AB_DH + a.d_rope;

  // Issue order: the W^UK copy, then the c^Q rows, then the first UA_DEPTH
  // column blocks of W^UQ.  Loads complete in issue order, so the wait for
  // any weight block also covers everything issued before it.
  {
    const bf16_t* Wk = a.Wuk + (long)head * AB_DH * a.d_c + AB_NCOL * e;
    const uint32_t wt_addr = (uint32_t)(uintptr_t)(lu8*)wt;
#pragma unroll
    for (int n = 0; n < 8; ++n) {  // 64 KiB as 64 wave-instructions of 1 KiB (8 k-rows x 128 B of a tile)
      const int ii = wave + 8 * n;
      const int t = ii >> 4, i = ii & 15;
      const int pos = 64 * i + lane, k = pos >> 3, phys = pos & 7;
      const int q = phys ^ (4 * ((k >> 1) & 1)) ^ (2 * ((k >> 3) & 1));
      ua_dma(Wk, (uint32_t)((k * a.d_c + 64 * t + 8 * q) * 2), wt_addr + t * AB_TILE + i * 1024);
    }
  }
  bf16x8 xf[4][UA_KS];
  XPlain{a.X, UA_DCQ, 0}.load<UA_KS>(0, wave * UA_KS * 32 + 8 * g, i16, g, wave, a.M, xf);
  __builtin_amdgcn_sched_barrier(0);
  // W^UQ rows of column block nb (lane row i16) from this wave's K-slice
  const bf16_t* Wq = a.Wuq + (long)head * wd * UA_DCQ + wave * UA_KS * 32 + 8 * g;
  auto wrow = [&](int nb) -> const bf16_t* {
    const int r = nb < UA_NOPE_NB ? 16 * nb : AB_DH + 32 * e + 16 * (nb - UA_NOPE_NB);
    return Wq + (long)(r + i16) * UA_DCQ;
  };
  bf16x8 wf[UA_DEPTH][UA_KS];
#pragma unroll
  for (int d = 0; d < UA_DEPTH; ++d)
#pragma unroll
    for (int ks = 0; ks < UA_KS; ++ks) wf[d][ks] = *(const bf16x8*)(wrow(d) + 32 * ks);

  float* mine = slab + wave * UA_SLAB;
#pragma unroll
  for (int nb = 0; nb < UA_NB; ++nb) {
    // the MFMAs of block nb, then the loads of block nb + UA_DEPTH, kept in
    // this order so that UA_DEPTH - 1 blocks stay in flight meanwhile
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < UA_KS; ++ks) {
      const bf16x8 w = wf[nb % UA_DEPTH][ks];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, xf[mb][ks], acc[mb], 0, 0, 0);
    }
    if (nb + UA_DEPTH < UA_NB) {
#pragma unroll
      for (int ks = 0; ks < UA_KS; ++ks) wf[nb % UA_DEPTH][ks] = *(const bf16x8*)(wrow(nb + UA_DEPTH) + 32 * ks);
    }
    __builtin_amdgcn_sched_barrier(0);
    // C = u^T: lane holds column 16 nb + 4g + r (r = 0..3) of row m = 16 mb + i16
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) *(f32x4*)(mine + (16 * mb + i16) * UA_LDN + 16 * (nb & 1) + 4 * g) = acc[mb];
    if (nb & 1) {
      ring_barrier();  // every wave's slab holds column blocks nb-1, nb
      const int cb = nb - 1;
      for (int p = threadIdx.x; p < 16 * 64; p += UA_WAVES * 64) {
        const int m = p >> 4, c = 2 * (p & 15);
        float2 v = *(const float2*)(slab + m * UA_LDN + c);
#pragma unroll
        for (int w = 1; w < UA_WAVES; ++w) {
          const float2 t = *(const float2*)(slab + w * UA_SLAB + m * UA_LDN + c);
          v.x += t.x;
          v.y += t.y;
        }
        if (cb < UA_NOPE_NB) {
          *(bf16x2*)(qct + m * UA_QC_LD + 16 * cb + c) = bf16x2{(bf16_t)v.x, (bf16_t)v.y};
        } else if (m < a.M) {
          const int d = 32 * e + 16 * (cb - UA_NOPE_NB) + c;  // RoPE column (pair d/2)
          const int b = m / a.s_q, j = m % a.s_q;
          int ps = a.seqlens[b] - a.s_q + j;
          ps = ps < 0 ? 0 : ps;
          float cs, sn;
          rope_cs_w(ps, a.freq[d >> 1], &cs, &sn);
          *(bf16x2*)(a.qt + ((long)m * a.H + head) * (a.d_c + a.d_rope) + a.d_c + d) =
              bf16x2{(bf16_t)(a.scale2 * (v.x * cs - v.y * sn)), (bf16_t)(a.scale2 * (v.x * sn + v.y * cs))};
        }
      }
      ring_barrier();  // the slabs are free again; the q^C columns are in LDS
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the W^UK copy (issued first) has landed
  __syncthreads();

  // 2. absorption, K = d_head: wave w computes columns 32w .. 32w+31 of the
  // block's 256 for all 64 rows.  A = q^C rows from the tile; B[k][n] from two
  // transposing reads of 4 k-rows each.
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      xf[mb][ks] = *(const __attribute__((address_space(3))) bf16x8*)((const __attribute__((address_space(3))) uint8_t*)qct +
                                                                      ((16 * mb + i16) * UA_QC_LD + 32 * ks + 8 * g) * 2);
  f32x4 acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb][0] = acc[mb][1] = f32x4{};
  const int e4 = i16 >> 2, qq = i16 & 3;
#pragma unroll
  for (int nbi = 0; nbi < 2; ++nbi) {
    const int nloc = 32 * wave + 16 * nbi;
    const int t = nloc >> 6, nq = (nloc & 63) + 4 * qq;
    const int c = nq >> 3, half = (nq >> 2) & 1;
    const uint8_t* tb = wt + t * AB_TILE + half * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k1 = 32 * ks + 8 * g + e4, k2 = k1 + 4;
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(tb + ab_pos(k1, c) * 16));
      const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(tb + ab_pos(k2, c) * 16));
      const short s8 __attribute__((ext_vector_type(8))) = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
      const bf16x8 bw = __builtin_bit_cast(bf16x8, s8);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb][nbi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[mb][ks], bw, acc[mb][nbi], 0, 0, 0);
    }
  }
  // Output rows staged in the (free) slab area as [64 m][256 n] bf16, 16-byte
  // chunk j of row m at j ^ (m & 31); C lane layout: rows m = 16 mb + 4 g + r,
  // column n = 32 w + 16 nbi + i16.
  bf16_t* st = (bf16_t*)lds;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nbi = 0; nbi < 2; ++nbi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * mb + 4 * g + r, n = 32 * wave + 16 * nbi + i16;
        st[m * AB_NCOL + 8 * ((n >> 3) ^ (m & 31)) + (n & 7)] = (bf16_t)(a.scale2 * acc[mb][nbi][r]);
      }
  __syncthreads();
  for (int p = threadIdx.x; p < 64 * 32; p += UA_WAVES * 64) {
    const int m = p >> 5, j = p & 31;
    if (m < a.M)
      *(bf16x8*)(a.qt + ((long)m * a.H + head) * (a.d_c + a.d_rope) + AB_NCOL * e + 8 * j) =
          *(const bf16x8*)(st + m * AB_NCOL + 8 * (j ^ (m & 31)));
  }
}

template <int WPB, int KS, int NB, int DEPTH, class XSrc, class Epi>
hipError_t launch_skinny(const SkArgs& a, const XSrc& xs, int n_groups, int k_groups, int batch, const Epi& epi,
                         hipStream_t st) {
  constexpr int lds = SkPlan<WPB, NB>::LDS_BYTES;
  auto kern = &k_skinny<WPB, KS, NB, DEPTH, XSrc, Epi>;
  static bool attr_set = false;  // one flag per instantiation
  if (!attr_set) {
    MLA_TRY(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    attr_set = true;
  }
  return launch(kern, dim3(n_groups, k_groups, batch), dim3(WPB * 64), lds, st, a, xs, epi);
}

}  // namespace

// Plans for the DeepSeek-V3 shapes; anything else returns false and the
// caller uses the general GEMM.
bool skinny_query_supported(const mla_dims& d, int R) {
  return R >= 1 && R <= 64 && d.d_model % 896 == 0 && d.d_model / 896 <= KSPLIT_MAX && d.d_cq == UA_DCQ &&
         d.d_head == AB_DH && d.d_c == 2 * AB_NCOL && d.d_rope == 64 && d.n_heads % 4 == 0;
}

// c^Q = W^DQ h (k-groups + reduction), then W^UQ with RoPE and the
// absorption in one kernel.
hipError_t skinny_query(const DecodeArgs& a) {
  const mla_dims& d = a.d;
  const int R = a.batch * a.s_q, H = d.n_heads;
  const float scale2 = a.scale * 1.4426950408889634f;
  bf16_t* qt = (bf16_t*)(a.ws + a.L.qt);
  const bf16_t* cq = (const bf16_t*)a.hq;
  if (a.W_DQ) {
    // 7 waves x 4 k-steps = 896 k per k-group; 3 column blocks per block
    const int kgroups = d.d_model / 896;
    SkArgs s{R, 896, (const bf16_t*)a.W_DQ, d.d_model, 0};
    XPlain xs{(const bf16_t*)a.hq, d.d_model, 0};
    float* part = (float*)(a.ws + a.L.cq_part);
    MLA_TRY((launch_skinny<7, 4, 3, 3>(s, xs, d.d_cq / 48, kgroups, 1, EpiKPart{part, R, d.d_cq}, a.stream)));
    bf16_t* cqb = (bf16_t*)(a.ws + a.L.cq);
    const int MN = R * d.d_cq;
    MLA_TRY(launch(&k_reduce_rows, dim3((MN / 4 + 255) / 256), dim3(256), 0, a.stream, MN, kgroups,
                   (const float*)part, cqb));
    cq = cqb;
  }
  UaArgs ua{R, H, d.d_c, d.d_rope, a.s_q, cq, (const bf16_t*)a.W_UQ, (const bf16_t*)a.W_UK, qt, a.seqlens, scale2, {}};
  for (int m = 0; m < d.d_rope / 2; ++m) ua.freq[m] = pow((double)d.rope_theta, -2.0 * m / d.d_rope);
  static bool attr_set = false;
  if (!attr_set) {
    MLA_TRY(hipFuncSetAttribute((const void*)&k_uq_absorb, hipFuncAttributeMaxDynamicSharedMemorySize, UA_LDS));
    attr_set = true;
  }
  return launch(&k_uq_absorb, dim3(2 * H), dim3(UA_WAVES * 64), UA_LDS, a.stream, ua);
}

}  // namespace mla

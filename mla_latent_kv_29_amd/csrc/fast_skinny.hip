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
//              The same kernel streams W^O (y = W^O o, K = H d_head).
//   k_uq_absorb  q_i = W^UQ_i c^Q for one head (the same split of K over
//              the waves), then qt_i = tau log2(e) q^C_i . W^UK_i with
//              W^UK_i[d_head][d_c] (n contiguous) in LDS, read by the
//              transposing LDS read; q^C_i stays in LDS between the two.
//
// MFMA v_mfma_f32_16x16x32_bf16, C[16][16] += A[16][32] B[32][16]: lane l
// holds row l%16, k 8(l/16)..+7 of A, the same of B^T, and rows 4(l/16)..+3
// of column l%16 of C.  With A = W (rows n) and B = X (rows m), C = Y^T.
#include <algorithm>
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
  // columns from n_split on are rows n - n_split of W2 (two weights in one
  // launch; n_split a multiple of the block's columns)
  int n_split = 1 << 30;
  const bf16_t* W2 = nullptr;
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

// One reduction round, after column block nb: every wave has stored its C
// tiles of the round's NBR column blocks in its slab; all threads sum the
// waves for their column pairs and hand them to the epilogue (or park them
// in the final tile when there are several rounds).
template <int WPB, int NB, class Epi>
__device__ __forceinline__ void sk_round(float* slab, int nb, int n0, int batch, int kg, int M, const Epi& epi) {
  using P = SkPlan<WPB, NB>;
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
      if (m < M) epi(batch, kg, m, c_base + c, v.x, v.y);
    } else {
      *(float2*)(slab + WPB * P::SLAB + m * P::LDF + (c_base - n0) + c) = v;
    }
  }
  ring_barrier();  // the slabs (and final tile) are complete before reuse
}

// With several rounds: the parked sums go to the epilogue once all are in.
template <int WPB, int NB, class Epi>
__device__ __forceinline__ void sk_final(const float* slab, int n0, int batch, int kg, int M, const Epi& epi) {
  using P = SkPlan<WPB, NB>;
  if constexpr (P::FINAL != 0) {
    constexpr int PAIRS = NB * 8;
    const float* fin = slab + WPB * P::SLAB;
    for (int p = threadIdx.x; p < PAIRS * 64; p += WPB * 64) {
      const int m = p / PAIRS, c = 2 * (p % PAIRS);
      const float2 v = *(const float2*)(fin + m * P::LDF + c);
      if (m < M) epi(batch, kg, m, n0 + c, v.x, v.y);
    }
  }
}

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
  const bf16_t* W = n0 < a.n_split ? a.W + (long)batch * a.bsw + (long)(n0 + i16) * a.ldw + k0
                                   : a.W2 + (long)(n0 - a.n_split + i16) * a.ldw + k0;

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
    if (nr == P::NBR - 1) sk_round<WPB, NB>(slab, nb, n0, batch, kg, a.M, epi);
  }
  sk_final<WPB, NB>(slab, n0, batch, kg, a.M, epi);
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

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_vmcnt0() { wait_vmcnt<0>(); }

// ------------------------------------------------------------ W^UQ + absorption
// One block per (head i, half e of d_c), 8 waves:
//   1. u_i = W^UQ_i c^Q for the head's 128 content rows and the 32 RoPE rows
//      of half e (16 pairs).  The content sums, rounded to bf16, stay in LDS
//      as the q^C_i tile; the RoPE pairs are rotated at the row's position,
//      scaled by tau log2 e and written to the tail of qt.
//   2. qt_i[:, 256e .. 256e+255] = tau log2 e q^C_i W^UK_i[:, 256e ..].
// Both halves of a head read the same content rows of W^UQ; the two blocks
// are placed on one XCD, so the second read is served by that XCD's L2.
//
// Weights reach LDS through global_load_lds in units of 24 KiB (16 weight
// rows x half of d_cq), every wave-instruction reading whole 512-byte runs
// of two rows: a CU keeps more bytes in flight this way than with loads of
// 16 rows x 64 bytes straight into MFMA operands.  A ring of five unit
// slots holds four units in flight while one is multiplied.  The 23 units
// are the 20 of W^UQ (column block nb = u/2, K half u%2) and then W^UK_i's
// half-e tile (64 KiB), which so lands in slots 0-2, i.e. in one piece at the
// ring's start.  Wave w = 2 rb + kq multiplies rows 16 rb .. +15 of c^Q (held
// in registers) with k-quarter kq of each unit; the two k-quarters of a row
// block meet through a 1 KiB slab.
//
// W^UQ unit layout: wave-instruction j (0..23) covers rows 2(j/3), 2(j/3)+1
// and 16-byte chunks 32(j%3) .. +31 of the unit's 96; chunk c of row r sits
// at slot c ^ (r & 15) of its run (conflict-free MFMA operand reads).
// W^UK tile: 64-column tiles [128 k][64 n], row k chunk q (8 n) at
// k*8 + (q ^ swz(k)), the layout whose transposing reads are conflict free.
__device__ __forceinline__ int ab_pos(int k, int q) { return k * 8 + (q ^ (4 * ((k >> 1) & 1)) ^ (2 * ((k >> 3) & 1))); }

constexpr int AB_DH = 128;                     // d_head (k of the absorption)
constexpr int AB_NCOL = 256;                   // absorbed columns per block (half of d_c)
constexpr int AB_TILE = AB_DH * 64 * 2;        // one 64-column W^UK tile, bytes
constexpr int UA_WAVES = 8;
constexpr int UA_DCQ = 1536;                   // d_cq
constexpr int UA_NOPE_NB = AB_DH / 16;         // content column blocks (8)
constexpr int UA_NB = UA_NOPE_NB + 2;          // + two RoPE column blocks (32 columns)
constexpr int UA_UNIT = 16 * UA_DCQ;           // bytes of a unit: 16 rows x half of d_cq
constexpr int UA_QUNITS = 2 * UA_NB;           // W^UQ units
constexpr int UA_UNITS = UA_QUNITS + 3;        // + the W^UK tile (24 + 24 + 16 KiB)
constexpr int UA_SLOTS = 5;
constexpr int UA_KS = UA_DCQ / 2 / 2 / 32;     // k-steps of a wave per unit (12)
constexpr int UA_QC_LD = AB_DH + 8;            // q^C tile row, bf16 (rows 16 bytes apart in the banks)
constexpr int UA_QC_OFF = UA_SLOTS * UA_UNIT;
constexpr int UA_SLAB_OFF = UA_QC_OFF + 64 * UA_QC_LD * 2;
constexpr int UA_LDS = UA_SLAB_OFF + 2 * 4 * 1024;
constexpr int UA_STAGE_OFF = 3 * UA_UNIT;      // output staging: slots 3-4, free once W^UQ is done
static_assert(UA_LDS <= 160 * 1024, "LDS");
static_assert(4 * AB_TILE <= UA_STAGE_OFF && 3 * UA_UNIT == 72 * 1024, "W^UK tile in slots 0-2");
static_assert(UA_STAGE_OFF + 64 * AB_NCOL * 2 <= UA_QC_OFF, "output staging in slots 3-4");
static_assert((UA_QUNITS + 0) % UA_SLOTS == 0, "the W^UK units start at slot 0");

typedef __attribute__((address_space(3))) uint8_t lu8;
typedef __attribute__((address_space(3))) bf16x8 lbf16x8;

// One 1 KiB wave-instruction of a global -> LDS copy (16 bytes a lane at
// gbase + voff, to LDS lds_addr + 16 lane).  Issued from asm: the compiler
// cannot tell where such a copy lands, so for the builtin it waits for every
// outstanding load before any later LDS access, which would drain the weight
// stream at each step.  The caller waits (vmcnt) before reading the copy.
// Nothing else in k_uq_absorb uses M0.
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

struct UaCtx {
  const bf16_t *wq, *wk;  // W^UQ_i, W^UK_i half e
  uint32_t ring;          // LDS address of the ring
  int wave, lane, e;
};

// Unit u into its ring slot: this wave's 3 (the last W^UK unit: 2) of the
// unit's wave-instructions.
__device__ __forceinline__ void ua_issue(const UaCtx& c, int u) {
  if (u >= UA_UNITS) return;
  if (u < UA_QUNITS) {
    const int nb = u >> 1, kh = u & 1;
    const int row0 = nb < UA_NOPE_NB ? 16 * nb : AB_DH + 32 * c.e + 16 * (nb - UA_NOPE_NB);
    const uint32_t dst = c.ring + (u % UA_SLOTS) * UA_UNIT;
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) {
      const int j = c.wave + 8 * jj;
      const int r = 2 * (j / 3) + (c.lane >> 5), s = 32 * (j % 3) + (c.lane & 31);
      const int ch = s ^ (r & 15);
      ua_dma(c.wq, (uint32_t)(((row0 + r) * UA_DCQ + kh * (UA_DCQ / 2) + 8 * ch) * 2), dst + 1024 * j);
    }
  } else {
    // W^UK instruction ii (0..63): tile t = ii/16, k-rows 8(ii%16) .. +7
    const int n = u == UA_UNITS - 1 ? 2 : 3;
    for (int jj = 0; jj < n; ++jj) {
      const int ii = 24 * (u - UA_QUNITS) + c.wave + 8 * jj;
      const int t = ii >> 4, i = ii & 15;
      const int pos = 64 * i + c.lane, k = pos >> 3, phys = pos & 7;
      const int q = phys ^ (4 * ((k >> 1) & 1)) ^ (2 * ((k >> 3) & 1));
      ua_dma(c.wk, (uint32_t)((k * 2 * AB_NCOL + 64 * t + 8 * q) * 2), c.ring + 1024 * ii);
    }
  }
}

__global__ __launch_bounds__(UA_WAVES * 64) void k_uq_absorb(UaArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lu8* lds = (lu8*)lds_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, in an SGPR
  const int g = lane >> 4, i16 = lane & 15;
  const int rb = wave >> 1, kq = wave & 1;
  // Blocks are dealt to the 8 XCDs round-robin: XCD x runs blocks x, x + 8,
  // ...; its consecutive pairs of those are the two halves of one head.
  const int xcd = blockIdx.x & 7, ub = blockIdx.x >> 3;
  const int head = xcd * (gridDim.x >> 4) + (ub >> 1), e = ub & 1;

  // The row's position and its lane's four RoPE frequencies (pairs of
  // columns 32e + 16j + 4g, +2 for j = 0, 1), for the RoPE epilogue; then
  // the first four units, then the c^Q rows 16 rb + i16 (clamped: rows past
  // M are computed, never stored), k = 768 kh + 384 kq + 32 ks + 8 g .. +7.
  const int m = 16 * rb + i16;
  const int sl = m < a.M ? a.seqlens[m / a.s_q] : 0;
  double fr[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) fr[j][h] = a.freq[16 * e + 8 * j + 2 * g + h];
  UaCtx c;
  c.wq = a.Wuq + (long)head * (AB_DH + a.d_rope) * UA_DCQ;
  c.wk = a.Wuk + (long)head * AB_DH * a.d_c + AB_NCOL * e;
  c.ring = (uint32_t)(uintptr_t)lds;
  c.wave = wave;
  c.lane = lane;
  c.e = e;
  for (int u = 0; u < UA_SLOTS - 1; ++u) ua_issue(c, u);

  bf16x8 xf[2][UA_KS];
  {
    const bf16_t* x = a.X + (long)min(m, a.M - 1) * UA_DCQ + 384 * kq + 8 * g;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int ks = 0; ks < UA_KS; ++ks) xf[kh][ks] = *(const bf16x8*)(x + 768 * kh + 32 * ks);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load of the prologue is out before anything waits
  wait_vmcnt0();  // all of the above (and units 0-3) have landed: no later wait of the compiler's drains the ring

  // LDS offsets of this lane's A fragments (row i16, chunk 48 kq + 4 ks + g)
  uint32_t aoff[UA_KS];
#pragma unroll
  for (int ks = 0; ks < UA_KS; ++ks) {
    const int ch = 48 * kq + 4 * ks + g, s = ch ^ i16;
    aoff[ks] = (uint32_t)(1024 * (3 * (i16 >> 1) + (s >> 5)) + 512 * (i16 & 1) + 16 * (s & 31));
  }
  int ps = m < a.M ? sl - a.s_q + m % a.s_q : 0;
  ps = ps < 0 ? 0 : ps;
  lu8* slab = lds + UA_SLAB_OFF;
  lu8* qct = lds + UA_QC_OFF;  // q^C tile [64 m][UA_QC_LD] bf16

  // Column block nb's epilogue (waves kq = 0): the pair's sum, then the q^C
  // tile (content) or the rotated RoPE pairs (qt tail).  Lane holds columns
  // 16 nb + 4g + r (r = 0..3) of row m.
  auto epilogue = [&](int nb, const f32x4& acc) {
    const f32x4 v = acc + *(const __attribute__((address_space(3))) f32x4*)(slab + ((nb & 1) * 4 + rb) * 1024 + 16 * lane);
    if (nb < UA_NOPE_NB) {
      bf16x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = (bf16_t)v[r];
      *(__attribute__((address_space(3))) bf16x4*)(qct + (m * UA_QC_LD + 16 * nb + 4 * g) * 2) = o;
    } else if (m < a.M) {
      const int j = nb - UA_NOPE_NB;
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
  for (int nb = 0; nb < UA_NB; ++nb) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int u = 2 * nb + kh;
      // this wave's copies of unit u have landed (younger: units u+1 .. u+3,
      // three instructions each but for the last W^UK unit's two)
      if (u == UA_QUNITS - 1) wait_vmcnt<8>(); else wait_vmcnt<9>();
      ring_barrier();  // everyone's copies of unit u are in; everyone is done with unit u-1 and the slab
      ua_issue(c, u + UA_SLOTS - 1);  // into unit u-1's slot
      if (kh == 0) {
        if (nb > 0 && kq == 0) epilogue(nb - 1, acc);
        acc = f32x4{};
      }
      const lu8* sb = lds + (u % UA_SLOTS) * UA_UNIT;
#pragma unroll
      for (int ks = 0; ks < UA_KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const lbf16x8*)(sb + aoff[ks]), xf[kh][ks], acc, 0, 0, 0);
      if (kh == 1 && kq == 1) *(__attribute__((address_space(3))) f32x4*)(slab + ((nb & 1) * 4 + rb) * 1024 + 16 * lane) = acc;
    }
  }
  wait_vmcnt0();  // the W^UK units
  ring_barrier();
  if (kq == 0) epilogue(UA_NB - 1, acc);
  ring_barrier();  // the q^C tile is complete

  // 2. absorption, K = d_head: wave w computes columns 32w .. 32w+31 of the
  // block's 256 for all 64 rows.  A = q^C rows from the tile; B[k][n] from two
  // transposing reads of 4 k-rows each.
  bf16x8 qf[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[mb][ks] = *(const lbf16x8*)(qct + ((16 * mb + i16) * UA_QC_LD + 32 * ks + 8 * g) * 2);
  f32x4 ab[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) ab[mb][0] = ab[mb][1] = f32x4{};
  const int e4 = i16 >> 2, qq = i16 & 3;
#pragma unroll
  for (int nbi = 0; nbi < 2; ++nbi) {
    const int nloc = 32 * wave + 16 * nbi;
    const int t = nloc >> 6, nq = (nloc & 63) + 4 * qq;
    const int cc = nq >> 3, half = (nq >> 2) & 1;
    const lu8* tb = lds + t * AB_TILE + half * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k1 = 32 * ks + 8 * g + e4, k2 = k1 + 4;
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(tb + ab_pos(k1, cc) * 16));
      const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(tb + ab_pos(k2, cc) * 16));
      const short s8 __attribute__((ext_vector_type(8))) = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
      const bf16x8 bw = __builtin_bit_cast(bf16x8, s8);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) ab[mb][nbi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[mb][ks], bw, ab[mb][nbi], 0, 0, 0);
    }
  }
  // Output rows staged (slots 3-4) as [64 m][256 n] bf16, 16-byte chunk j of
  // row m at j ^ (m & 31); C lane layout: rows m = 16 mb + 4 g + r, column
  // n = 32 w + 16 nbi + i16.
  __attribute__((address_space(3))) bf16_t* st = (__attribute__((address_space(3))) bf16_t*)(lds + UA_STAGE_OFF);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nbi = 0; nbi < 2; ++nbi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mm = 16 * mb + 4 * g + r, n = 32 * wave + 16 * nbi + i16;
        st[mm * AB_NCOL + 8 * ((n >> 3) ^ (mm & 31)) + (n & 7)] = (bf16_t)(a.scale2 * ab[mb][nbi][r]);
      }
  __syncthreads();
  for (int p = threadIdx.x; p < 64 * 32; p += UA_WAVES * 64) {
    const int mm = p >> 5, j = p & 31;
    if (mm < a.M)
      *(bf16x8*)(a.qt + ((long)mm * a.H + head) * (a.d_c + a.d_rope) + AB_NCOL * e + 8 * j) =
          *(const __attribute__((address_space(3))) bf16x8*)(st + mm * AB_NCOL + 8 * (j ^ (mm & 31)));
  }
}

// ------------------------------------------------------------ FP8 block-scaled weights
// E4M3 quantisation of a weight W[N][K] in 128 x 128 blocks (the last
// row-block may be shorter): scale s = amax / 448 in fp32 (1 for an all-zero
// block), code = RNE(x / s) saturated.  One 256-thread block per weight
// block; thread t owns row t/2, columns 64 (t & 1) .. +63.
__global__ __launch_bounds__(256) void k_quant_w(int N, int K, const bf16_t* __restrict__ W,
                                                 uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float red[4];
  const int r0 = blockIdx.x * 128, kb = blockIdx.y;
  const int r = threadIdx.x >> 1, c0 = kb * 128 + 64 * (threadIdx.x & 1);
  const bool live = r0 + r < N;
  float v[64];
  float am = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    bf16x8 x = live ? *(const bf16x8*)(W + (long)(r0 + r) * K + c0 + 8 * q) : bf16x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[8 * q + e] = (float)x[e];
      am = fmaxf(am, fabsf(v[8 * q + e]));
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = am > 0.0f ? am / 448.0f : 1.0f;
  if (live) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t w4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t u = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) u |= (uint32_t)f32_to_e4m3(v[16 * q + 4 * i + e] / sc) << (8 * e);
        w4[i] = u;
      }
      *(uint4*)(codes + (long)(r0 + r) * K + c0 + 16 * q) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
  }
  if (threadIdx.x == 0) scales[(long)blockIdx.x * (K / 128) + kb] = sc;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// E4M3 quantisation of activations X[M][K] in 1 x 128 tiles: codes [M][K],
// scales [M][K / 128].  16 lanes per tile, 8 values a lane; the tile's amax
// meets by four lane swaps.
__global__ __launch_bounds__(256) void k_quant_x(int tiles, int K, const bf16_t* __restrict__ X,
                                                 uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4), j = threadIdx.x & 15;
  const bool live = t < tiles;
  const int kt = K / 128, row = live ? t / kt : 0, c0 = live ? (t % kt) * 128 + 8 * j : 0;
  const bf16x8 x = live ? *(const bf16x8*)(X + (long)row * K + c0) : bf16x8{};
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf((float)x[e]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
  const float sc = am > 0.0f ? am / 448.0f : 1.0f;
  if (!live) return;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) lo |= (uint32_t)f32_to_e4m3((float)x[e] / sc) << (8 * e);
#pragma unroll
  for (int e = 0; e < 4; ++e) hi |= (uint32_t)f32_to_e4m3((float)x[4 + e] / sc) << (8 * e);
  *(uint2*)(codes + (long)row * K + c0) = make_uint2(lo, hi);
  if (j == 0) scales[t] = sc;
}

// The k-group sums of k_reduce_rows for Y[M][N] (N a multiple of 128), also
// quantised in 1 x 128 tiles from the bf16 sums, exactly as k_quant_x would
// quantise Y: codes [M][N], scales [M][N / 128].  16 lanes per tile.
__global__ __launch_bounds__(256) void k_reduce_quant(int M, int N, int KG, const float* __restrict__ part,
                                                      bf16_t* __restrict__ y, uint8_t* __restrict__ codes,
                                                      float* __restrict__ scales) {
  const int nt = N / 128, t = blockIdx.x * 16 + (threadIdx.x >> 4), j = threadIdx.x & 15;
  const bool live = t < M * nt;
  const long i = live ? (long)(t / nt) * N + (t % nt) * 128 + 8 * j : 0;
  const long MN = (long)M * N;
  f32x4 s0 = f32x4{}, s1 = f32x4{};
  if (live) {
    s0 = *(const f32x4*)(part + i);
    s1 = *(const f32x4*)(part + i + 4);
    for (int k = 1; k < KG; ++k) {
      s0 += *(const f32x4*)(part + k * MN + i);
      s1 += *(const f32x4*)(part + k * MN + i + 4);
    }
  }
  bf16x8 x;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = (bf16_t)s0[e];
    x[4 + e] = (bf16_t)s1[e];
  }
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf((float)x[e]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
  const float sc = am > 0.0f ? am / 448.0f : 1.0f;
  if (!live) return;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) lo |= (uint32_t)f32_to_e4m3((float)x[e] / sc) << (8 * e);
#pragma unroll
  for (int e = 0; e < 4; ++e) hi |= (uint32_t)f32_to_e4m3((float)x[4 + e] / sc) << (8 * e);
  *(bf16x8*)(y + i) = x;
  *(uint2*)(codes + i) = make_uint2(lo, hi);
  if (j == 0) scales[t] = sc;
}

struct F8Args {
  int M, K;             // activation rows (<= 64), reduction length (multiple of 512)
  const uint8_t* Xc;    // activation codes [M][K]
  const float* Xs;      // activation scales [M][K / 128]
  const uint8_t* Wc;    // weight codes [N][K]
  const float* Ws;      // weight scales [ceil(N / 128)][K / 128]
};

// Y[m][n] = sum over 128-wide k-blocks kb of sx[m][kb] sw[n / 128][kb]
// (Xc[m][kb] . Wc[n][kb]) for at most 64 rows: four waves, wave w of k-group
// kg owns k-blocks (4 kg + w) KB .. +KB-1; NB column blocks of 16 per block,
// all of whose weight loads go out at once.  One
// v_mfma_f32_16x16x128_f8f6f4 per (column block, k-block, row block) gives
// the integer-grid partial, which the two scales promote into the fp32 sum.
// A lane's 32 operand bytes of a k-block are k = 16 g .. +15 and
// 64 + 16 g .. +15 (g = lane / 16), the same order for W and X, so that
// every 16-byte weight load covers 16 rows x 64 contiguous bytes.
template <int KB, int NB, int DEPTH, class Epi>
__global__ __launch_bounds__(256) void k_skinny_f8(F8Args a, Epi epi) {
  constexpr int WPB = 4;
  using P = SkPlan<WPB, NB>;
  extern __shared__ __attribute__((aligned(16))) float slab[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int n0 = blockIdx.x * NB * 16, kg = blockIdx.y;
  const int kb0 = (kg * WPB + wave) * KB;
  const int kbs = a.K / 128;

  // activation codes and scales of rows 16 mb + i16 (clamped), k-blocks kb0 ..
  i32x8 xq[4][KB];
  float xs[4][KB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int row = min(16 * mb + i16, a.M - 1);
    const uint8_t* xp = a.Xc + (long)row * a.K + 16 * g;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const uint4 lo = *(const uint4*)(xp + (kb0 + j) * 128);
      const uint4 hi = *(const uint4*)(xp + (kb0 + j) * 128 + 64);
      xq[mb][j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      xs[mb][j] = a.Xs[(long)row * kbs + kb0 + j];
    }
  }
  // weight rows n0 + 16 nb + i16, DEPTH column blocks loading ahead (DEPTH =
  // NB: all of them at once)
  i32x8 wf[DEPTH][KB];
  auto load_w = [&](int nb, int slot) {
    const uint8_t* wp = a.Wc + (long)(n0 + 16 * nb + i16) * a.K + 16 * g;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const uint4 lo = *(const uint4*)(wp + (kb0 + j) * 128);
      const uint4 hi = *(const uint4*)(wp + (kb0 + j) * 128 + 64);
      wf[slot][j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  };
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load_w(d, d);

  float* mine = slab + wave * P::SLAB;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{};
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const float sw = a.Ws[(long)((n0 + 16 * nb) >> 7) * kbs + kb0 + j];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[nb % DEPTH][j], xq[mb][j], f32x4{}, 0,
                                                                        0, 0, 0, 0, 0);
        acc[mb] += (sw * xs[mb][j]) * p;
      }
    }
    if (nb + DEPTH < NB) load_w(nb + DEPTH, nb % DEPTH);
    // C = Y^T: lane holds n = 16 nb + 4g + r (r = 0..3), m = 16 mb + i16
    const int nr = nb % P::NBR;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) *(f32x4*)(mine + (16 * mb + i16) * P::LDN + 16 * nr + 4 * g) = acc[mb];
    if (nr == P::NBR - 1) sk_round<WPB, NB>(slab, nb, n0, 0, kg, a.M, epi);
  }
  sk_final<WPB, NB>(slab, n0, 0, kg, a.M, epi);
}

// Y[m][n] (bf16) directly, when one k-group covers K
struct EpiRowsBf16 {
  bf16_t* y;
  int N;
  __device__ void operator()(int, int, int m, int n, float v0, float v1) const {
    bf16x2 v = {(bf16_t)v0, (bf16_t)v1};
    *(bf16x2*)(y + (long)m * N + n) = v;
  }
};

// u = Q(c^Q) . Q(W^UQ)^T of the FP8-weight decode with its RoPE epilogue:
// the content part q^C_i goes to qc [R][H][d_head] (bf16), the RoPE pairs
// (adjacent columns 2p, 2p + 1 of the head's d_rope) are rotated at the
// row's position, scaled by tau log2 e and written to the tail of qt.
struct EpiUQF8 {
  bf16_t* qc;
  bf16_t* qt;
  const int32_t* seqlens;
  int H, d_head, d_rope, d_c, s_q, m0;  // m0: first row of this 64-row chunk
  float scale2;
  double freq[32];  // theta^(-2p/d_rope) of RoPE pair p
  __device__ void operator()(int, int, int m, int n, float v0, float v1) const {
    const int w = d_head + d_rope, i = n / w, d = n % w;
    const int rr = m0 + m;
    if (d < d_head) {
      bf16x2 o = {(bf16_t)v0, (bf16_t)v1};
      *(bf16x2*)(qc + ((long)rr * H + i) * d_head + d) = o;
      return;
    }
    const int b = rr / s_q, j = rr % s_q;
    int pos = seqlens[b] - s_q + j;
    pos = pos < 0 ? 0 : pos;
    float cs, sn;
    rope_cs_w(pos, freq[(d - d_head) >> 1], &cs, &sn);
    bf16x2 o = {(bf16_t)(scale2 * (v0 * cs - v1 * sn)), (bf16_t)(scale2 * (v0 * sn + v1 * cs))};
    *(bf16x2*)(qt + ((long)rr * H + i) * (d_c + d_rope) + d_c + (d - d_head)) = o;
  }
};

template <int KB, int NB, class Epi, int DEPTH = NB>
hipError_t launch_f8(const F8Args& a, int n_groups, int k_groups, const Epi& epi, hipStream_t st) {
  constexpr int lds = SkPlan<4, NB>::LDS_BYTES;
  auto kern = &k_skinny_f8<KB, NB, DEPTH, Epi>;
  MLA_TRY(lds_limit((const void*)kern, lds));
  return launch(kern, dim3(n_groups, k_groups), dim3(256), lds, st, a, epi);
}

template <int KB, class Epi>
hipError_t launch_f8_nb(const F8Args& a, int nb, int N, int k_groups, const Epi& epi, hipStream_t st) {
  switch (nb) {
    case 28:  // 448 columns a block, streamed four column blocks ahead
      if constexpr (KB <= 2) return launch_f8<KB, 28, Epi, 4>(a, N / 448, k_groups, epi, st);
      [[fallthrough]];
    case 4:
      if constexpr (KB * 4 <= 12) return launch_f8<KB, 4>(a, N / 64, k_groups, epi, st);
      [[fallthrough]];
    case 2: return launch_f8<KB, 2>(a, N / 32, k_groups, epi, st);
    default: return launch_f8<KB, 1>(a, N / 16, k_groups, epi, st);
  }
}

template <class Epi>
hipError_t launch_f8_kb(const F8Args& a, const F8Plan& p, int N, const Epi& epi, hipStream_t st) {
  switch (p.kb) {
    case 3: return launch_f8_nb<3>(a, p.nb, N, p.kgroups, epi, st);
    case 2: return launch_f8_nb<2>(a, p.nb, N, p.kgroups, epi, st);
    default: return launch_f8_nb<1>(a, p.nb, N, p.kgroups, epi, st);
  }
}

template <int WPB, int KS, int NB, int DEPTH, class XSrc, class Epi>
hipError_t launch_skinny(const SkArgs& a, const XSrc& xs, int n_groups, int k_groups, int batch, const Epi& epi,
                         hipStream_t st) {
  constexpr int lds = SkPlan<WPB, NB>::LDS_BYTES;
  auto kern = &k_skinny<WPB, KS, NB, DEPTH, XSrc, Epi>;
  MLA_TRY(lds_limit((const void*)kern, lds));
  return launch(kern, dim3(n_groups, k_groups, batch), dim3(WPB * 64), lds, st, a, xs, epi);
}

}  // namespace

// Plans for the DeepSeek-V3 shapes; anything else returns false and the
// caller uses the general GEMM.
bool skinny_query_supported(const mla_dims& d, int R) {
  return R >= 1 && R <= 64 && d.d_model % 896 == 0 && d.d_model / 896 <= KSPLIT_MAX && d.d_cq == UA_DCQ &&
         d.d_head == AB_DH && d.d_c == 2 * AB_NCOL && d.d_rope == 64 && d.n_heads % 4 == 0;
}

// W^O: 1024 k per k-group.  With N a multiple of 448 (d_model 7168): 8 waves
// x 4 k-steps and 28 column blocks of 16 per block, four loading ahead, so
// that each block streams 0.9 MB of the weight without a break (one block
// per CU); measured 57 us at 64 rows against 84 us for blocks of 64 columns
// (4 waves x 8 k-steps, three ahead), which serve other N.
bool skinny_out_supported(int rows, int N, int K) {
  return rows >= 1 && rows <= 64 && N % 64 == 0 && K % 1024 == 0 && K / 1024 <= 64;
}

hipError_t skinny_out(const OutProjArgs& a, int kgroups) {
  SkArgs s{a.rows, 1024, (const bf16_t*)a.W_O, a.K, 0};
  XPlain xs{(const bf16_t*)a.o, a.K, 0};
  float* part = (float*)a.ws;
  const EpiKPart epi{part, a.rows, a.N};
  if (a.N % 448 == 0)  // 8 waves x 4 k-steps, 28 column blocks streamed four ahead: 256 blocks at V3
    MLA_TRY((launch_skinny<8, 4, 28, 4>(s, xs, a.N / 448, kgroups, 1, epi, a.stream)));
  else
    MLA_TRY((launch_skinny<4, 8, 4, 3>(s, xs, a.N / 64, kgroups, 1, epi, a.stream)));
  const int MN = a.rows * a.N;
  return launch(&k_reduce_rows, dim3((MN / 4 + 255) / 256), dim3(256), 0, a.stream, MN, kgroups, (const float*)part,
                (bf16_t*)a.y);
}

// The GEMM half of the decode-step append with a workspace: the latent rows
// [c^KV | k^R before RoPE] = h [W^DKV; W^KR]^T of at most 64 tokens as fp32
// partials per k-group of 896, part[kg][m][d_c + d_rope], W^DKV's columns
// first.  Blocks of 32 columns and 7 waves x 4 k-steps, both weights in one
// launch: with 8 k-groups at d_model 7168, 144 blocks stream the 8.26 MB.
struct EpiKPartOff {
  float* part;
  int M, ldp, off;
  __device__ void operator()(int, int kg, int m, int n, float v0, float v1) const {
    float2 v = {v0, v1};
    *(float2*)(part + ((long)kg * M + m) * ldp + off + n) = v;
  }
};

bool skinny_append_supported(const mla_dims& d, int n_tok) {
  return n_tok >= 1 && n_tok <= 64 && d.d_model % 896 == 0 && d.d_c % 32 == 0 && d.d_rope % 32 == 0;
}

int skinny_append_kgroups(const mla_dims& d) { return d.d_model / 896; }

hipError_t skinny_append_partials(const AppendArgs& a, float* part) {
  const mla_dims& d = a.d;
  const int kg = skinny_append_kgroups(d), ld = d.d_c + d.d_rope;
  XPlain xs{(const bf16_t*)a.h, d.d_model, 0};
  SkArgs sa{a.n_tok, 896, (const bf16_t*)a.W_DKV, d.d_model, 0, d.d_c, (const bf16_t*)a.W_KR};
  return launch_skinny<7, 4, 2, 2>(sa, xs, ld / 32, kg, 1, EpiKPartOff{part, a.n_tok, ld, 0}, a.stream);
}

// ------------------------------------------------------------ FP8 host side
bool fp8_gemm_supported(int N, int K) { return N >= 16 && N % 16 == 0 && K >= 512 && K % 512 == 0; }

F8Plan fp8_plan(int M, int N, int K) {
  F8Plan p{};
  if (!fp8_gemm_supported(N, K) || M < 1) return p;
  // the most k-blocks per wave, up to 3 (fewest k-groups, so the fewest
  // fp32 partials; 4 measured slower for W^O), that divide K; then the
  // widest column group that still gives a block per CU, within the
  // registers (NB x KB operand tiles of 8 VGPRs)
  for (int kb : {3, 2, 1})
    if ((K / 512) % kb == 0) {
      p.kb = kb;
      break;
    }
  p.kgroups = K / (512 * p.kb);
  p.nb = 1;
  for (int nb : {28, 4, 2})
    if ((nb == 28 ? p.kb <= 2 : nb * p.kb <= 12) && (N / 16) % nb == 0 && (long)(N / (16 * nb)) * p.kgroups >= 256) {
      p.nb = nb;
      break;
    }
  const size_t rows = std::min(M, 64);
  p.xc_off = 0;
  p.xs_off = (rows * K + 255) / 256 * 256;
  p.part_off = p.xs_off + (rows * (K / 128) * 4 + 255) / 256 * 256;
  p.ws_bytes = p.part_off + (p.kgroups > 1 ? (size_t)p.kgroups * rows * N * 4 : 0);
  return p;
}

hipError_t fp8_quantize_weight(int N, int K, const bf16_t* W, uint8_t* codes, float* scales, hipStream_t st) {
  return launch(&k_quant_w, dim3((N + 127) / 128, K / 128), dim3(256), 0, st, N, K, W, codes, scales);
}

// Y = Q(X) . Q(W)^T in chunks of 64 rows (each chunk streams the weight).
// With yc (at most 64 rows, N a multiple of 128), Y is also quantised in
// 1 x 128 tiles into yc [M][N] and ys [M][N / 128].
hipError_t fp8_gemm(int M, int N, int K, const bf16_t* X, const uint8_t* Wc, const float* Ws, bf16_t* Y, uint8_t* ws,
                    hipStream_t st, uint8_t* yc, float* ys) {
  if (yc && (M > 64 || N % 128 != 0)) return hipErrorInvalidValue;
  const F8Plan p = fp8_plan(M, N, K);
  uint8_t* xc = ws + p.xc_off;
  float* xs = (float*)(ws + p.xs_off);
  for (int m0 = 0; m0 < M; m0 += 64) {
    const int rows = std::min(64, M - m0);
    const int tiles = rows * (K / 128);
    MLA_TRY(launch(&k_quant_x, dim3((tiles + 15) / 16), dim3(256), 0, st, tiles, K, X + (long)m0 * K, xc, xs));
    F8Args a{rows, K, xc, xs, Wc, Ws};
    bf16_t* y = Y + (long)m0 * N;
    if (p.kgroups == 1) {
      MLA_TRY(launch_f8_kb(a, p, N, EpiRowsBf16{y, N}, st));
      if (yc) {
        const int yt = rows * (N / 128);
        MLA_TRY(launch(&k_quant_x, dim3((yt + 15) / 16), dim3(256), 0, st, yt, N, (const bf16_t*)y, yc, ys));
      }
      continue;
    }
    float* part = (float*)(ws + p.part_off);
    MLA_TRY(launch_f8_kb(a, p, N, EpiKPart{part, rows, N}, st));
    const int MN = rows * N;
    if (yc) {
      const int yt = rows * (N / 128);
      MLA_TRY(launch(&k_reduce_quant, dim3((yt + 15) / 16), dim3(256), 0, st, rows, N, p.kgroups, (const float*)part,
                     y, yc, ys));
      continue;
    }
    MLA_TRY(launch(&k_reduce_rows, dim3((MN / 4 + 255) / 256), dim3(256), 0, st, MN, p.kgroups, (const float*)part, y));
  }
  return hipSuccess;
}

// W^UQ of the FP8-weight decode (one k-group: K = d_cq = 1536 is three
// k-blocks a wave): the activations quantised per 64-row chunk, then one
// GEMM launch whose epilogue splits q^C from the rotated RoPE pairs.  Six
// column blocks of 96 columns a block give 256 blocks at V3 (one per CU),
// streamed three ahead.
hipError_t fp8w_uq(const DecodeArgs& a, const uint8_t* Wc, const float* Ws, const bf16_t* cq, bf16_t* qc,
                   uint8_t* ws) {
  const mla_dims& d = a.d;
  const int R = a.batch * a.s_q, H = d.n_heads, N = H * (d.d_head + d.d_rope), K = d.d_cq;
  const F8Plan p = fp8_plan(R, N, K);
  if (p.kgroups != 1 || d.d_rope / 2 > 32) return hipErrorInvalidValue;
  EpiUQF8 epi{qc, (bf16_t*)(a.ws + a.L.qt), a.seqlens, H, d.d_head, d.d_rope, d.d_c, a.s_q, 0,
              a.scale * 1.4426950408889634f, {}};
  for (int m = 0; m < d.d_rope / 2; ++m) epi.freq[m] = pow((double)d.rope_theta, -2.0 * m / d.d_rope);
  uint8_t* xc = ws + p.xc_off;
  float* xs = (float*)(ws + p.xs_off);
  for (int m0 = 0; m0 < R; m0 += 64) {
    const int rows = std::min(64, R - m0);
    const int tiles = rows * (K / 128);
    MLA_TRY(launch(&k_quant_x, dim3((tiles + 15) / 16), dim3(256), 0, a.stream, tiles, K, cq + (long)m0 * K, xc, xs));
    F8Args f{rows, K, xc, xs, Wc, Ws};
    epi.m0 = m0;
    if (p.kb == 3 && (N / 16) % 6 == 0)
      MLA_TRY((launch_f8<3, 6, EpiUQF8, 3>(f, N / 96, 1, epi, a.stream)));
    else
      MLA_TRY(launch_f8_kb(f, p, N, epi, a.stream));
  }
  return hipSuccess;
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
  MLA_TRY(lds_limit((const void*)&k_uq_absorb, UA_LDS));
  return launch(&k_uq_absorb, dim3(2 * H), dim3(UA_WAVES * 64), UA_LDS, a.stream, ua);
}

}  // namespace mla

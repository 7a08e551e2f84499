// W^UQ, RoPE and the W^UK absorption for more than 64 query rows (gfx950).
//
// What it computes (DeepSeek-V3 reading lesson, §2.1.1: the query
// up-projection from the compressed query c^Q into a content part q^C and a
// RoPE part q^R per head; its Question 2: W^UK folded into the query): for
// query row m and head i,
//   u = W^UQ_i c^Q_m                      (d_head + d_rope = 192 values)
//   qt[m][i][d_c:] = tau log2(e) RoPE(q^R) at the row's position
//   qt[m][i][:d_c] = tau log2(e) W^UK_i^T q^C   (q^C rounded to bf16 first)
//
// One block per (head i, 128 rows), four waves.  Up to 64 rows the
// activations fit in the registers and only the weights stream
// (k_uq_absorb); beyond that both operands stream:
//   1. u for the block's 128 rows and the head's 192 W^UQ rows: 64-deep
//      k-steps of the c^Q rows (16 KiB) and the W^UQ rows (24 KiB) HBM/L2 ->
//      LDS with global_load_lds through a 3-stage ring, each copy
//      instruction reading whole 128-byte lines of 8 rows; each wave owns 64
//      rows x 96 columns (2 x 3 v_mfma_f32_32x32x16_bf16 accumulators) and
//      reads the fragments of the next k-step while the MFMAs of this one
//      run.  The c^Q tiles are shared by all heads and the W^UQ tiles by the
//      head's row blocks, which run on one XCD, so many copies come from L2;
//      each head starts the k-steps at its own offset, so that the blocks of
//      an XCD do not all read one c^Q tile at once.
//   2. The content sums, rounded to bf16, go to an LDS tile of q^C (in the
//      ring, free by then); the RoPE pairs (adjacent columns, held by one
//      lane) are rotated at the row's position, scaled and written to the
//      tail of qt.
//   3. The absorption over the head's W^UK (8 tiles of [128 k][64 n], two
//      loaded at the start into LDS beside the ring, five into the ring once
//      it is free, the last into the first one's place) with
//      v_mfma_f32_16x16x32_bf16: each wave holds the q^C fragments of all
//      128 rows and computes 16 columns of each tile, W^UK^T as the A
//      operand from transposing LDS reads, so that a lane ends with four
//      adjacent output columns of one row.
#include "internal.hpp"

namespace mla {
namespace {

constexpr int QR_ROWS = 128;                        // rows per block
constexpr int QR_DCQ = 1536, QR_DH = 128, QR_DR = 64, QR_W = QR_DH + QR_DR, QR_DC = 512, QR_H = 128;
constexpr int QR_BK = 64;                           // k per step: 128-byte rows
constexpr int QR_XT = QR_ROWS * 128;                // 16 KiB of c^Q rows
constexpr int QR_WT = QR_W * 128;                   // 24 KiB of W^UQ rows
constexpr int QR_STAGE = QR_XT + QR_WT;             // 40 KiB
constexpr int QR_NS = 3;
constexpr int QR_RING = QR_NS * QR_STAGE;           // 120 KiB
constexpr int QR_QC_LD = QR_DH + 8;                 // q^C tile row, bf16
constexpr int QR_QC_OFF = 0;                        // in the ring, once phase 1 is done
constexpr int QR_QC_BYTES = QR_ROWS * QR_QC_LD * 2; // 34 KiB
constexpr int QR_UK_TILE = QR_DH * 64 * 2;          // 16 KiB: [128 k][64 n]
constexpr int QR_SPARE_OFF = QR_RING;               // W^UK tiles 0 (then 7) and 1
constexpr int QR_LDS = QR_SPARE_OFF + 2 * QR_UK_TILE;
constexpr int QR_NK = QR_DCQ / QR_BK;               // 24 k-steps
static_assert(QR_LDS <= 160 * 1024, "LDS");
static_assert(QR_QC_BYTES % 1024 == 0 && QR_NK % (2 * QR_NS) == 0, "layout");
static_assert(QR_QC_BYTES + 5 * QR_UK_TILE <= QR_RING, "q^C and W^UK tiles 2-6 in the ring");

typedef __attribute__((address_space(3))) uint8_t lu8;
typedef __attribute__((address_space(3))) bf16x8 lbf16x8;
typedef __attribute__((address_space(3))) i16x4 li16x4;

template <int N>
__device__ __forceinline__ void qr_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One 1 KiB wave-instruction of a global -> LDS copy (16 bytes a lane at
// gbase + voff, to LDS lds_addr + 16 lane), from asm so that the compiler's
// wait accounting leaves it alone; the kernel waits (vmcnt) explicitly.
// Nothing else in k_uq_rows uses M0.
__device__ __forceinline__ void qr_dma(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds_addr)
               : "memory");
}

// W^UK tile: row k (128 bytes, 8 chunks of 8 columns) chunk q at slot
// k * 8 + (q ^ swz(k)): the layout whose transposing reads are conflict free
__device__ __forceinline__ int qr_uk_pos(int k, int q) { return k * 8 + (q ^ (4 * ((k >> 1) & 1)) ^ (2 * ((k >> 3) & 1))); }

struct QrArgs {
  int R, s_q, nrb;
  const bf16_t* X;         // c^Q [R][d_cq]
  const bf16_t* Wuq;       // [H][d_head + d_rope][d_cq], RoPE rows as interleaved pairs
  const bf16_t* Wuk;       // [H][d_head][d_c]
  bf16_t* qt;              // [R][H][d_c + d_rope]
  const int32_t* seqlens;  // position of row m = b s_q + j: seqlens[b] - s_q + j
  float scale2;            // tau log2 e
  double freq[QR_DR / 2];  // theta^(-2p/d_rope) of RoPE pair p
};

__global__ __launch_bounds__(256, 1) void k_uq_rows(QrArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lu8* lds = (lu8*)lds_raw;
  const uint32_t lbase = (uint32_t)(uintptr_t)lds_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hw = lane >> 5;       // 32x32 MFMA lane layout
  const int g = lane >> 4, i16 = lane & 15;        // 16x16 MFMA lane layout
  // blocks reach the XCDs round-robin: the row blocks of a head are
  // consecutive items of one XCD
  const int per = (int)gridDim.x >> 3;
  const int w = ((int)blockIdx.x & 7) * per + ((int)blockIdx.x >> 3);
  const int head = w / a.nrb, m0 = (w % a.nrb) * QR_ROWS;
  const uint8_t* wuk = (const uint8_t*)(a.Wuk + (long)head * QR_DH * QR_DC);

  // W^UK tile t (LDS offset): 16 wave-instructions of 8 k-rows; wave w
  // issues w, w+4, w+8, w+12
  auto uk_tile = [&](int t) -> int {
    return t == 0 || t == 7 ? QR_SPARE_OFF : t == 1 ? QR_SPARE_OFF + QR_UK_TILE : QR_QC_BYTES + (t - 2) * QR_UK_TILE;
  };
  auto issue_uk = [&](int t) {
    const uint32_t dst = lbase + uk_tile(t);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int i = wave + 4 * jj, pos = 64 * i + lane, k = pos >> 3, phys = pos & 7;
      const int q = phys ^ (4 * ((k >> 1) & 1)) ^ (2 * ((k >> 3) & 1));
      qr_dma(wuk, (uint32_t)((k * QR_DC + 64 * t + 8 * q) * 2), dst + 1024 * i);
    }
  };

  // phase-1 copies: instruction n covers tile rows 8 n .. 8 n + 7 (wave w
  // issues n = w, w + 4, ...), lane: row 8 n + lane / 8, chunk slot lane % 8
  // holding chunk slot ^ ((row >> 1) & 7), so that the 16 rows of a fragment
  // read (16 lanes a cycle) fill all 64 banks; the k position goes into the
  // scalar base.  c^Q rows past R are clamped (computed, never stored).
  uint32_t xo[4], wo[6];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row = 8 * (wave + 4 * n) + (lane >> 3), c = (lane & 7) ^ ((row >> 1) & 7);
    xo[n] = (uint32_t)(min(row, a.R - 1 - m0) * QR_DCQ * 2 + 16 * c);
  }
#pragma unroll
  for (int n = 0; n < 6; ++n) {
    const int row = 8 * (wave + 4 * n) + (lane >> 3), c = (lane & 7) ^ ((row >> 1) & 7);
    wo[n] = (uint32_t)(row * QR_DCQ * 2 + 16 * c);
  }
  const uint8_t* xb = (const uint8_t*)(a.X + (long)m0 * QR_DCQ);
  const uint8_t* wb = (const uint8_t*)(a.Wuq + (long)head * QR_W * QR_DCQ);
  // each head walks the k-steps from its own starting point, so that the
  // blocks of an XCD do not all read the same c^Q tile at once
  const int kofs = (head * 7) % QR_NK;
  auto issue = [&](int ks, int stg) {
    int kk = ks + kofs;
    kk = kk >= QR_NK ? kk - QR_NK : kk;
    const uint8_t* xk = xb + kk * 128;
    const uint8_t* wk = wb + kk * 128;
    const uint32_t d = lbase + stg * QR_STAGE;
#pragma unroll
    for (int n = 0; n < 4; ++n) qr_dma(xk, xo[n], d + 1024 * (wave + 4 * n));
#pragma unroll
    for (int n = 0; n < 6; ++n) qr_dma(wk, wo[n], d + QR_XT + 1024 * (wave + 4 * n));
  };

  issue_uk(0);
  issue_uk(1);
#pragma unroll
  for (int ks = 0; ks < QR_NS; ++ks) issue(ks, ks);
  // the sequence lengths of the lane's two rows (m = 64 wm + 32 ib + l32),
  // first used after phase 1, where nothing else is in flight
  const int wm = wave >> 1, wn = wave & 1;
  int slv[2];
#pragma unroll
  for (int ib = 0; ib < 2; ++ib) {
    const int m = m0 + 64 * wm + 32 * ib + l32;
    slv[ib] = m < a.R ? a.seqlens[m / a.s_q] : 0;
  }

  // fragment read addresses in stage 0 (the stage adds an offset): c^Q
  // row 64 wm + 32 ib + l32, W^UQ row 96 wn + 32 jb + l32, chunk
  // 2 k16 + hw at slot chunk ^ ((row >> 1) & 7)
  uint32_t fx[4], fw[4];
#pragma unroll
  for (int k16 = 0; k16 < 4; ++k16) {
    const uint32_t o = lbase + l32 * 128 + 16 * ((2 * k16 + hw) ^ ((l32 >> 1) & 7));
    fx[k16] = o + 64 * wm * 128;
    fw[k16] = o + QR_XT + 96 * wn * 128;
  }
  f32x16 acc[3][2];
#pragma unroll
  for (int jb = 0; jb < 3; ++jb)
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) acc[jb][ib] = f32x16{};

  // The fragments of a k-step are read one step ahead, while the MFMAs of
  // the step before run (reading them at the top of their own step left the
  // MFMA pipe idle for the LDS latency and bandwidth of all four waves).
  struct Frags {
    bf16x8 x[4][2], w[4][3];
  };
  auto read_frags = [&](Frags& f, uint32_t so) {
#pragma unroll
    for (int k16 = 0; k16 < 4; ++k16) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) f.x[k16][ib] = *(const lbf16x8*)(fx[k16] + so + 4096 * ib);
#pragma unroll
      for (int jb = 0; jb < 3; ++jb) f.w[k16][jb] = *(const lbf16x8*)(fw[k16] + so + 4096 * jb);
    }
  };
  // k-step ks: its fragments are in `cur`; k-step ks + 1 is read into `nxt`
  auto step = [&](auto stg_c, Frags& cur, Frags& nxt, int ks) {
    constexpr int STG = decltype(stg_c)::value;
    qr_wait_vmcnt<10>();  // this wave's copies of k-step ks + 1 landed (ks + 2 may be in flight)
    ring_barrier();       // every wave's copies of ks + 1 landed; every wave's reads of ks are done
    // k-step ks + 3 into the stage of ks; past the last k-step a repeat of
    // it (never used), so that the loop body has no branch
    issue(min(ks + QR_NS, QR_NK - 1), STG);
    read_frags(nxt, ((STG + 1) % QR_NS) * QR_STAGE);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k16 = 0; k16 < 4; ++k16)
#pragma unroll
      for (int jb = 0; jb < 3; ++jb)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
          acc[jb][ib] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.w[k16][jb], cur.x[k16][ib], acc[jb][ib], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  Frags fa, fb;
  qr_wait_vmcnt<20>();  // k-step 0 landed (1 and 2 may be in flight)
  ring_barrier();
  read_frags(fa, 0);
  for (int ks = 0; ks < QR_NK; ks += 2 * QR_NS) {
    step(std::integral_constant<int, 0>{}, fa, fb, ks);
    step(std::integral_constant<int, 1>{}, fb, fa, ks + 1);
    step(std::integral_constant<int, 2>{}, fa, fb, ks + 2);
    step(std::integral_constant<int, 0>{}, fb, fa, ks + 3);
    step(std::integral_constant<int, 1>{}, fa, fb, ks + 4);
    step(std::integral_constant<int, 2>{}, fb, fa, ks + 5);
  }
  qr_wait_vmcnt<0>();  // the repeat copies too
  // the compiler's own wait for the sequence lengths goes here, where
  // nothing else is in flight
  asm volatile("" ::"v"(slv[0]), "v"(slv[1]));
  ring_barrier();      // every wave is done with the ring
#pragma unroll 1
  for (int t = 2; t < 7; ++t) issue_uk(t);

  // 2. lane holds u for c^Q row m = 64 wm + 32 ib + l32 and W^UQ rows
  // n = 96 wn + 32 jb + 8 jj + 4 hw + r (r = 0..3)
  lu8* qct = lds + QR_QC_OFF;
#pragma unroll
  for (int ib = 0; ib < 2; ++ib) {
    const int m = 64 * wm + 32 * ib + l32;
    int ps = m0 + m < a.R ? slv[ib] - a.s_q + (m0 + m) % a.s_q : 0;
    ps = ps < 0 ? 0 : ps;
#pragma unroll
    for (int jb = 0; jb < 3; ++jb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int n0 = 96 * wn + 32 * jb + 8 * jj + 4 * hw;
        const f32x16& v = acc[jb][ib];
        if (wn == 0 || jb == 0) {  // content columns (n0 < d_head)
          bf16x4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = (bf16_t)v[4 * jj + r];
          *(__attribute__((address_space(3))) bf16x4*)(qct + (m * QR_QC_LD + n0) * 2) = o;
        } else if (m0 + m < a.R) {
          // RoPE pairs p0 = (n0 - d_head) / 2 and p0 + 1
          const int pb = 16 * (jb - 1) + 4 * jj;  // p0 for hw = 0; hw = 1 adds 2
          bf16x4 o;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            // both candidates as uniform loads, then a per-lane select (an
            // indexed load here would make the compiler wait for the W^UK copies)
            const double f0 = a.freq[pb + h], f1 = a.freq[pb + 2 + h];
            const double f = hw ? f1 : f0;
            // the angle in turns, reduced in double to [-1/2, 1/2], then the
            // hardware sine and cosine of a turn fraction
            const double tr = (double)ps * f * 0.15915494309189535;
            const float rf = (float)(tr - rint(tr));
            const float cs = __builtin_amdgcn_cosf(rf), sn = __builtin_amdgcn_sinf(rf);
            const float x0 = v[4 * jj + 2 * h], x1 = v[4 * jj + 2 * h + 1];
            o[2 * h] = (bf16_t)(a.scale2 * (x0 * cs - x1 * sn));
            o[2 * h + 1] = (bf16_t)(a.scale2 * (x0 * sn + x1 * cs));
          }
          *(bf16x4*)(a.qt + ((long)(m0 + m) * QR_H + head) * (QR_DC + QR_DR) + QR_DC + n0 - QR_DH) = o;
        }
      }
  }
  ring_barrier();  // the q^C tile is complete

  // 3. absorption.  q^C fragments of all 128 rows (B operand: column m =
  // 16 mb + i16, k = 32 ks + 8 g .. +7)
  bf16x8 qf[8][4];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[mb][ks] = *(const lbf16x8*)(qct + ((16 * mb + i16) * QR_QC_LD + 32 * ks + 8 * g) * 2);
  // this wave's 16 columns of a tile, read transposed: lane (e4, qq) reads
  // four columns at k-rows k1 and k1 + 4 (A operand: row n = 16 wave + i16)
  const int e4 = i16 >> 2, qq = i16 & 3;
  const int nq = 16 * wave + 4 * qq, cc = nq >> 3, half = (nq >> 2) & 1;
  auto absorb = [&](int t) {
    const lu8* tb = lds + uk_tile(t) + half * 8;
    f32x4 c[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) c[mb] = f32x4{};
    bf16x8 bw[4];  // all of the tile's reads first
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k1 = 32 * ks + 8 * g + e4, k2 = k1 + 4;
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)(tb + qr_uk_pos(k1, cc) * 16));
      const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)(tb + qr_uk_pos(k2, cc) * 16));
      const short s8 __attribute__((ext_vector_type(8))) = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
      bw[ks] = __builtin_bit_cast(bf16x8, s8);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) c[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[ks], qf[mb][ks], c[mb], 0, 0, 0);
    // C: rows n = 16 wave + 4 g + r of the tile, column m = 16 mb + i16
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int m = m0 + 16 * mb + i16;
      if (m < a.R) {
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = (bf16_t)(a.scale2 * c[mb][r]);
        *(bf16x4*)(a.qt + ((long)m * QR_H + head) * (QR_DC + QR_DR) + 64 * t + 16 * wave + 4 * g) = o;
      }
    }
  };
  absorb(0);
  absorb(1);
  ring_barrier();  // every wave is done with tile 0, whose place takes tile 7
  issue_uk(7);
  qr_wait_vmcnt<4>();  // tiles 2-6 (and every store before tile 7's copies) have landed
  ring_barrier();
#pragma unroll 1
  for (int t = 2; t < 7; ++t) absorb(t);
  qr_wait_vmcnt<0>();
  ring_barrier();
  absorb(7);
}

}  // namespace

bool rows_query_supported(const mla_dims& d, int R) {
  return R > 64 && d.n_heads == QR_H && d.d_cq == QR_DCQ && d.d_head == QR_DH && d.d_rope == QR_DR &&
         d.d_c == QR_DC;
}

// W^UQ + RoPE + absorption for R > 64 rows from c^Q (bf16 [R][d_cq]).
hipError_t rows_query(const DecodeArgs& a, const bf16_t* cq) {
  const mla_dims& d = a.d;
  const int R = a.batch * a.s_q;
  const int nrb = (R + QR_ROWS - 1) / QR_ROWS;
  QrArgs q{R, a.s_q, nrb, cq, (const bf16_t*)a.W_UQ, (const bf16_t*)a.W_UK, (bf16_t*)(a.ws + a.L.qt), a.seqlens,
           a.scale * 1.4426950408889634f, {}};
  for (int p = 0; p < QR_DR / 2; ++p) q.freq[p] = pow((double)d.rope_theta, -2.0 * p / QR_DR);
  MLA_TRY(lds_limit((const void*)&k_uq_rows, QR_LDS));
  return launch(&k_uq_rows, dim3(QR_H * nrb), dim3(256), QR_LDS, a.stream, q);
}

}  // namespace mla

// Causal MLA prefill attention on MFMA for the DeepSeek-V3 shape (gfx950).
//
// What it computes (DeepSeek-V3 reading lesson, §2.1.1, in the non-absorbed
// form: per head i an explicit key k_{t,i} = [k^C_{t,i} ; k^R_t] with
// k^C = W^UK c^KV and the shared RoPE key k^R, value v^C = W^UV c^KV; the
// scaled softmax of q_{j,i} . k_{t,i} over the tokens t <= j of the same
// sequence): for every token j of every packed sequence and every head i,
//     o_{j,i} = sum_{t<=j} p_t v^C_{t,i},  p = softmax_t(tau q_{j,i} . k_{t,i}),
// and lse_{j,i} (natural log).  q arrives pre-scaled by tau log2(e), so the
// softmax runs in the exp2 domain, and without its RoPE: each wave rotates
// the q^R part of its query fragments as it loads them, from a per-token
// (cos, sin) table.
//
// Work item = (sequence, head, tile of 128 query rows); four waves of 32 rows.
// All query tiles of one (sequence, head) run on one XCD together, so the K
// and V tiles that they all stream come from that XCD's L2.
// Per 64-key tile (keys up to the tile's last query):
//   S^T[32 keys][32 queries] blocks = K . Q^T with v_mfma_f32_32x32x16_bf16:
//     K fragments from LDS (192-wide rows: k^C of the head, then k^R), the
//     wave's Q^T fragments in 48 VGPRs for the whole kernel.  A 1 KiB K
//     fragment feeds 16384 multiply-adds (32 queries), which keeps the LDS
//     reads of four waves within what the LDS delivers.
//   Online softmax (running row maximum m and sum l): a lane holds sixteen
//     keys of one query per 32-key block, so the row maximum needs one lane
//     swap; O is rescaled by 2^(m_old - m_new) only when some row's maximum
//     moved.
//   O^T[32 channels][32 queries] += V^T . P^T: P^T is the S^T register layout
//     itself (keys 4h..4h+3 and 8+4h..8+4h+3 of a 16-key step make the eight
//     k-slots of half-wave h), and two transposing LDS reads deliver V^T in
//     the same key order, so P never leaves the registers.
// The tiles are software-pipelined within each wave: step i computes the
// scores of tile i+1 with the exponentials of tile i slotted between those
// MFMAs, then tile i's P.V with tile i+1's row maximum between those.  The
// vector work of the softmax thus issues while the matrix unit runs the
// other product, instead of after it.
// K and V tiles stream HBM/L2 -> LDS with global_load_lds into two K slots
// (24 KiB) and two V slots (16 KiB): step i reads K tile i+1 and V tile i
// while K tile i+2 and V tile i+1 are in flight.  At 80 KiB a block, two
// blocks share a CU, i.e. two waves per SIMD.  The LDS layouts (16-byte chunk
// q of row r at slot q ^ f(r)) spread the K fragment reads and the
// transposing V reads over the banks.
#include <algorithm>
#include <type_traits>

#include "internal.hpp"

namespace mla {
namespace {

constexpr int PH = 128, PDH = 128, PDR = 64, PDQK = PDH + PDR;  // heads, d_head (= d_v), d_rope, q.k width
constexpr int BQ = 128, BKT = 64;                                // query rows per block, keys per tile
constexpr int KC_BYTES = BKT * PDH * 2;                          // 16 KiB
constexpr int KR_BYTES = BKT * PDR * 2;                          // 8 KiB
constexpr int K_BYTES = KC_BYTES + KR_BYTES;                     // 24 KiB: a K slot (k^C rows, then k^R rows)
constexpr int V_BYTES = BKT * PDH * 2;                           // 16 KiB
constexpr int V_OFF = 2 * K_BYTES;                               // the two V slots follow the two K slots
constexpr int PA_LDS = 2 * K_BYTES + 2 * V_BYTES;                // 80 KiB
static_assert(K_BYTES == 24 * 1024 && V_BYTES == 16 * 1024, "six K and four V copies per wave and tile");

typedef __attribute__((address_space(3))) uint8_t lu8;
typedef __attribute__((address_space(3))) bf16x8 lbf16x8;
typedef __attribute__((address_space(3))) i16x4 li16x4;

// One 1 KiB wave-instruction of a global -> LDS copy (16 bytes a lane at
// gbase + voff to LDS lds_addr + 16 lane), issued from asm so that the
// compiler's wait accounting leaves it alone: the kernel waits for the tile
// explicitly (wait_vmcnt) before the barrier that publishes it.  Nothing else
// in k_prefill_attn uses M0.
__device__ __forceinline__ void pa_dma(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds_addr)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Slot of 16-byte chunk c of tile row r: k^C rows (256 B), k^R rows (128 B),
// V rows (256 B).  The V swizzle gives the four key rows that one
// transposing read of 32 lanes touches four disjoint groups of four slots.
__device__ __forceinline__ int kc_slot(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int kr_slot(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ int v_swz(int r) { return 4 * (r & 3); }

struct PaArgs {
  const bf16_t* q;   // [H][n_tok][192], pre-scaled by tau log2(e), RoPE not yet applied
  const bf16_t* kc;  // [H][n_tok][128]
  const bf16_t* vc;  // [H][n_tok][128]
  const bf16_t* kr;  // [n_tok][64]
  const int32_t* cu; // [n_seq + 1]
  const float2* cs_tab;  // [n_tok][32] (cos, sin) of the tokens' RoPE angles
  int n_tok, qtiles, n_seq;
  bf16_t* out;       // [n_tok][H][128]
  float* lse;        // [n_tok][H] or null
};

// Per-lane byte offsets of this wave's tile copies, the same for every tile
// and every copy of a kind (the swizzle depends on row bits that the copy
// index does not change): k^C copy j (rows 4j + lane/16), k^R copy j (rows
// 8j + lane/8), V copy j (rows 4j + lane/16).
struct TileOffsets {
  uint32_t kc, kr, v;
};
__device__ __forceinline__ TileOffsets tile_offsets(int wave, int lane) {
  TileOffsets t;
  t.kc = (uint32_t)(((lane >> 4) * PDH + 8 * ((lane & 15) ^ ((4 * wave + (lane >> 4)) & 15))) * 2);
  t.kr = (uint32_t)(((lane >> 3) * PDR + 8 * ((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7))) * 2);
  t.v = (uint32_t)(((lane >> 4) * PDH + 8 * ((lane & 15) ^ v_swz(lane >> 4))) * 2);
  return t;
}

// Key tile kt (keys 64 kt .. +63 of the sequence, clamped to its last token):
// its k^C and k^R rows into the K slot at kbuf, its V rows into the V slot at
// vbuf.  Of a K tile's 24 copies (0-15 k^C rows, 16-23 k^R rows) wave w issues
// w, w+4, ..., w+20: copies n = 0-3 of the wave are k^C, 4-5 k^R; of a V
// tile's 16, w, w+4, w+8, w+12.  A tile inside the sequence needs no clamping:
// its copies take the per-lane offsets above and the tile's position in the
// scalar base; the sequence's last tile clamps rows.
__device__ __forceinline__ void issue_k(const bf16_t* kc_h, const bf16_t* kr, int start, int len, int kt,
                                        uint32_t kbuf, int wave, int lane, const TileOffsets& to) {
  const int k0 = kt * BKT;
  const uint32_t lb = kbuf + 1024 * wave;
  if (k0 + BKT <= len) {
    const uint8_t* kcb = (const uint8_t*)kc_h + (size_t)(start + k0 + 4 * wave) * PDH * 2;
    const uint8_t* krb = (const uint8_t*)kr + (size_t)(start + k0 + 8 * wave) * PDR * 2;
#pragma unroll
    for (int n = 0; n < 4; ++n) pa_dma(kcb + 16 * n * PDH * 2, to.kc, lb + 4096 * n);
#pragma unroll
    for (int n = 0; n < 2; ++n) pa_dma(krb + 32 * n * PDR * 2, to.kr, lb + KC_BYTES + 4096 * n);
    return;
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int r = 4 * (wave + 4 * n) + (lane >> 4), c = kc_slot(r, lane & 15);
    const int key = min(k0 + r, len - 1);
    pa_dma(kc_h, (uint32_t)(((start + key) * PDH + 8 * c) * 2), lb + 4096 * n);
  }
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int r = 8 * (wave + 4 * n) + (lane >> 3), c = kr_slot(r, lane & 7);
    const int key = min(k0 + r, len - 1);
    pa_dma(kr, (uint32_t)(((start + key) * PDR + 8 * c) * 2), lb + KC_BYTES + 4096 * n);
  }
}
__device__ __forceinline__ void issue_v(const bf16_t* vc_h, int start, int len, int kt, uint32_t vbuf, int wave,
                                        int lane, const TileOffsets& to) {
  const int k0 = kt * BKT;
  const uint32_t lb = vbuf + 1024 * wave;
  if (k0 + BKT <= len) {
    const uint8_t* vb = (const uint8_t*)vc_h + (size_t)(start + k0 + 4 * wave) * PDH * 2;
#pragma unroll
    for (int n = 0; n < 4; ++n) pa_dma(vb + 16 * n * PDH * 2, to.v, lb + 4096 * n);
    return;
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int r = 4 * (wave + 4 * n) + (lane >> 4), c = (lane & 15) ^ v_swz(r);
    const int key = min(k0 + r, len - 1);
    pa_dma(vc_h, (uint32_t)(((start + key) * PDH + 8 * c) * 2), lb + 4096 * n);
  }
}

__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// maximum over the lanes l and l ^ 32
__device__ __forceinline__ float max_x32(float m) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int N>
using IC = std::integral_constant<int, N>;

__global__ __launch_bounds__(256, 2) void k_prefill_attn(PaArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lu8* lds = (lu8*)lds_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hw = lane >> 5;  // 32x32 MFMA lane layout: row/column l32, k-half hw
  // Work item w = (pair (head, sequence), query tile): workgroups reach the
  // eight XCDs round-robin, so item w runs on XCD w / (G / 8) when block
  // L = 8 (w mod G/8) + XCD.  All query tiles of a (head, sequence) then run
  // on one XCD at about the same time and re-read its K and V tiles from
  // that XCD's L2.  Within a pair the longest (last) query tiles go first.
  const int G = (int)gridDim.x, per = G >> 3;  // G = qtiles * n_seq * 128, a multiple of 8
  const int w = ((int)blockIdx.x & 7) * per + ((int)blockIdx.x >> 3);
  const int pair = w / a.qtiles, b = pair % a.n_seq, h = pair / a.n_seq;
  const int start = a.cu[b], len = a.cu[b + 1] - start;
  const int qt = a.qtiles - 1 - (w - pair * a.qtiles);
  const int q0 = qt * BQ;
  if (q0 >= len) return;
  const int ntiles = (min(len, q0 + BQ) - 1) / BKT + 1;  // causal: keys up to the block's last query
  const bf16_t* kc_h = a.kc + (size_t)h * a.n_tok * PDH;
  const bf16_t* vc_h = a.vc + (size_t)h * a.n_tok * PDH;
  const uint32_t ring = (uint32_t)(uintptr_t)lds;

  // Q^T fragments (B operand): query row q0 + 32 wave + l32 (clamped: rows
  // past the sequence are computed and never stored), k = 16 ks + 8 hw.
  const int wq0 = q0 + 32 * wave;  // this wave's first query
  const int qrow = wq0 + l32;
  bf16x8 qf[12];
  {
    const int tok = start + min(qrow, len - 1);
    const bf16_t* qp = a.q + ((size_t)h * a.n_tok + tok) * PDQK + 8 * hw;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) qf[ks] = *(const bf16x8*)(qp + 16 * ks);
    // RoPE of q^R (dims 128..191, pairs (2m, 2m+1) within the lane's eight
    // values) at the token's position, from the (cos, sin) table
    const float2* cs = a.cs_tab + (size_t)tok * (PDR / 2) + 4 * hw;
    float2 t[4][4];
#pragma unroll
    for (int ks = 8; ks < 12; ++ks)
#pragma unroll
      for (int p = 0; p < 4; ++p) t[ks - 8][p] = cs[8 * (ks - 8) + p];
#pragma unroll
    for (int ks = 8; ks < 12; ++ks)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = (float)qf[ks][2 * p], x1 = (float)qf[ks][2 * p + 1];
        const float c = t[ks - 8][p].x, sn = t[ks - 8][p].y;
        qf[ks][2 * p] = (bf16_t)(x0 * c - x1 * sn);
        qf[ks][2 * p + 1] = (bf16_t)(x0 * sn + x1 * c);
      }
  }
  wait_vmcnt<0>();  // the compiler's loads are done before the copies go out
  const TileOffsets to = tile_offsets(wave, lane);
  // K tile t lives in K slot t & 1, V tile t in V slot t & 1
  issue_k(kc_h, a.kr, start, len, 0, ring, wave, lane, to);
  if (ntiles > 1) issue_k(kc_h, a.kr, start, len, 1, ring + K_BYTES, wave, lane, to);
  issue_v(vc_h, start, len, 0, ring + V_OFF, wave, lane, to);

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.0f;  // row maximum in use (log2 domain) and this lane's partial sum

  // LDS byte addresses of the lane's reads in slot 0 (the slot, the key
  // block and the key step become instruction offsets):
  //  K: k-step ks (16-wide slice 16 ks .. of the 192-wide key row, this
  //     lane's half 8 hw ..) of key row l32;
  //  V^T: 16-lane group G = lane/16 covers channels 32 db + 16 (G & 1) ..
  //     +15 for k-half G/2 (= hw); lane (e, qq) of the group addresses key
  //     row 4 hw + e (+ 16 kk, + 8), channels +4 qq .. +3.
  uint32_t ka[12], va[4];
  {
    const uint32_t base = (uint32_t)(uintptr_t)lds;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ka[ks] = base + l32 * 256 + 16 * kc_slot(l32, 2 * ks + hw);
#pragma unroll
    for (int ks = 8; ks < 12; ++ks) ka[ks] = base + KC_BYTES + l32 * 128 + 16 * kr_slot(l32, 2 * (ks - 8) + hw);
    const int e = (lane & 15) >> 2, qq = lane & 3, gsub = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < 4; ++db)
      va[db] = base + V_OFF + (4 * hw + e) * 256 + 16 * ((4 * db + 2 * gsub + (qq >> 1)) ^ v_swz(e)) + 8 * (qq & 1);
  }

  // K fragment t of the score chain (k-step t/2, key block t&1) in K slot KSL
  auto kread = [&](auto ksl, int t) -> bf16x8 {
    constexpr int KSL = decltype(ksl)::value;
    const int ks = t >> 1, kb = t & 1;
    return *(const lbf16x8*)(ka[ks] + KSL * K_BYTES + (ks < 8 ? kb * 8192 : kb * 4096));
  };
  // V^T fragment of P.V MFMA u (key step u/4, channel block u%4) in V slot VSL
  auto vread = [&](auto vsl, int u) -> bf16x8 {
    constexpr int VSL = decltype(vsl)::value;
    const uint32_t adr = va[u & 3] + VSL * V_BYTES + (u >> 2) * 4096;
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)adr);
    const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)(adr + 2048));
    const short s8 __attribute__((ext_vector_type(8))) = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
    return __builtin_bit_cast(bf16x8, s8);
  };
  // Scores S^T of a key tile: lane holds keys 32 kb + 8 j + 4 hw + i (VGPR
  // 4j + i of sc[kb]) of query l32.  The two key blocks alternate (two
  // independent chains); K fragments are read D MFMAs ahead.
  constexpr int D = 3;
  // keys after the lane's query get -inf (only tiles that reach past the
  // wave's first query have any)
  auto mask = [&](int kt, f32x16(&sc)[2]) {
    const int k0 = kt * BKT;
    if (k0 + BKT - 1 > wq0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (k0 + 32 * kb + 8 * (v >> 2) + 4 * hw + (v & 3) > qrow) sc[kb][v] = -INFINITY;
    }
  };
  // part j (0..7) of the row maximum: keys 4 (j & 3) .. +3 of key block j/2
  auto max_part = [&](const f32x16(&sc)[2], int j, float mx) -> float {
    const int kb = j >> 2, v = 4 * (j & 3);
    return vmax3(mx, vmax3(sc[kb][v], sc[kb][v + 1], sc[kb][v + 2]), sc[kb][v + 3]);
  };
  // Online softmax with a lazily raised maximum: p = 2^(s - m) with the m in
  // use, which moves (and O and the sum are rescaled) only when some score
  // exceeds it by more than 2^8; every p stays below 256, and the result
  // o / l is the same for any m.
  auto rescale = [&](float mt) {
    if (__any(mt > m + 8.0f)) {  // tile 0 always: m is -inf and every query sees key 0
      const float mn = mt > m + 8.0f ? mt : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      m = mn;
    }
  };
  // Weights of scores v, v+1 (v even): p = 2^(s - m), summed into ls.  The
  // empty asm statements pin each result where it is computed: without them
  // the compiler sinks these pure instructions past the score MFMAs they are
  // meant to overlap, to the block after the mask's branch.
  auto exp2v = [&](f32x16(&sc)[2], int v, float& ls) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float p = __builtin_amdgcn_exp2f(sc[(v + e) >> 4][(v + e) & 15] - m);
      asm volatile("" : "+v"(p));
      sc[(v + e) >> 4][(v + e) & 15] = p;
      ls += p;
    }
    asm volatile("" : "+v"(ls));
  };
  // P^T fragment of key step g: keys 16g + 4hw + 0..3 and 16g + 8 + 4hw + 0..3,
  // which are values 8 (g & 1) .. +7 of sc[g / 2]: the S^T layout itself
  auto pack = [&](const f32x16(&sc)[2], int g) -> bf16x8 {
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[i] = (bf16_t)sc[g >> 1][8 * (g & 1) + i];
    return pb;
  };

  f32x16 s[2][2];  // scores of the tiles in the two K slots
  float mt;        // row maximum of the scores that the next step turns into weights

  // Tile 0's scores on their own.
  if (ntiles > 1) wait_vmcnt<10>();  // K tile 1 and V tile 0 may stay in flight
  else wait_vmcnt<4>();
  ring_barrier();
  {
    s[0][0] = f32x16{};
    s[0][1] = f32x16{};
    bf16x8 kf[D];
#pragma unroll
    for (int t = 0; t < D; ++t) kf[t] = kread(IC<0>{}, t);
#pragma unroll
    for (int t = 0; t < 24; ++t) {
      s[0][t & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % D], qf[t >> 1], s[0][t & 1], 0, 0, 0);
      if (t + D < 24) kf[t % D] = kread(IC<0>{}, t + D);
      __builtin_amdgcn_sched_barrier(0);
    }
    mask(0, s[0]);
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = max_part(s[0], j, mx);
    mt = max_x32(mx);
  }

  // Step i (P = i & 1): the weights of tile i and its P.V, overlapped with
  // the scores of tile i+1.  Part (a): the 24 score MFMAs of tile i+1 (K slot
  // 1-P), the exponentials and bf16 packing of tile i's weights slotted
  // between them; part (b): tile i's 16 P.V MFMAs (V slot P), the mask and
  // row maximum of tile i+1 between them.  So the matrix unit has
  // independent work queued while the vector unit computes the softmax.
  // After the barrier every wave is done with step i-1, i.e. with K tile i
  // and V tile i-1, whose slots take K tile i+2 and V tile i+1.
  auto step = [&](auto par, int i) {
    constexpr int P = decltype(par)::value;
    wait_vmcnt<0>();  // K tile i+1 and V tile i (issued one step earlier)
    ring_barrier();
    const uint32_t kbuf = ring + P * K_BYTES, vbuf = ring + V_OFF + (1 - P) * V_BYTES;
    const bool act = i * BKT <= wq0 + 31;  // some key of tile i is visible to some query of this wave
    // K tile i+2 and V tile i+1: a tile inside the sequence is copied between
    // the score MFMAs below (a wave whose copy waits for the address unit
    // issues nothing else, so copies issued back to back here would leave the
    // matrix unit idle); a clamped last tile, or a wave with no tile i, copies
    // here.
    const bool kin = i + 2 < ntiles && (i + 3) * BKT <= len, vin = i + 1 < ntiles && (i + 2) * BKT <= len;
    if (i + 2 < ntiles && (!kin || !act)) issue_k(kc_h, a.kr, start, len, i + 2, kbuf, wave, lane, to);
    if (i + 1 < ntiles && (!vin || !act)) issue_v(vc_h, start, len, i + 1, vbuf, wave, lane, to);
    if (!act) return;  // every key of tile i is after every query of this wave
    const uint8_t* kcb = (const uint8_t*)kc_h + (size_t)(start + (i + 2) * BKT + 4 * wave) * PDH * 2;
    const uint8_t* krb = (const uint8_t*)a.kr + (size_t)(start + (i + 2) * BKT + 8 * wave) * PDR * 2;
    const uint8_t* vcb = (const uint8_t*)vc_h + (size_t)(start + (i + 1) * BKT + 4 * wave) * PDH * 2;
    // copy c (0-5: K tile, 6-9: V tile) of this wave, the offsets of issue_k / issue_v's
    // in-sequence case
    auto copy = [&](int c) {
      if (c < 4) {
        if (kin) pa_dma(kcb + 16 * c * PDH * 2, to.kc, kbuf + 1024 * wave + 4096 * c);
      } else if (c < 6) {
        if (kin) pa_dma(krb + 32 * (c - 4) * PDR * 2, to.kr, kbuf + KC_BYTES + 1024 * wave + 4096 * (c - 4));
      } else {
        if (vin) pa_dma(vcb + 16 * (c - 6) * PDH * 2, to.v, vbuf + 1024 * wave + 4096 * (c - 6));
      }
    };
    // One code path for every step: when the wave has no tile i+1 (its keys
    // are all after the wave's queries, or past the block's last tile), the
    // score MFMAs still run on whatever K slot 1-P holds and their results
    // are never used.
    f32x16(&sc)[2] = s[P];
    f32x16(&sn)[2] = s[1 - P];
    rescale(mt);
    float ls = 0.0f;
    bf16x8 pb[4];
    sn[0] = f32x16{};
    sn[1] = f32x16{};
    {
      bf16x8 kf[D];
#pragma unroll
      for (int t = 0; t < D; ++t) kf[t] = kread(IC<1 - P>{}, t);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 24; ++t) {
        sn[t & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % D], qf[t >> 1], sn[t & 1], 0, 0, 0);
        if (t + D < 24) kf[t % D] = kread(IC<1 - P>{}, t + D);
        const int g = t / 6, r = t % 6;
        if (r < 4) exp2v(sc, 8 * g + 2 * r, ls);
        else if (r == 4) {
          pb[g] = pack(sc, g);
          asm volatile("" : "+v"(pb[g]));
        }
        if ((t & 1) && t < 20) copy(t >> 1);  // copies 0-9 after MFMAs 1, 3, .., 19
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mask(i + 1, sn);
    l += ls;
    // (b) O^T += V^T P^T; V^T fragments read two MFMAs ahead
    constexpr int DV = 2;
    bf16x8 vf[DV + 1];
#pragma unroll
    for (int u = 0; u < DV; ++u) vf[u] = vread(IC<P>{}, u);
    float mx = -INFINITY;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      o[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u % (DV + 1)], pb[u >> 2], o[u & 3], 0, 0, 0);
      if (u + DV < 16) vf[(u + DV) % (DV + 1)] = vread(IC<P>{}, u + DV);
      // tile i+1's row maximum (unused when this wave has no tile i+1)
      if (u >= 2 && u < 10) mx = max_part(sn, u - 2, mx);
      if (u == 10) mt = max_x32(mx);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = 0; kt < ntiles; kt += 2) {
    step(IC<0>{}, kt);
    if (kt + 1 < ntiles) step(IC<1>{}, kt + 1);
  }
  wait_vmcnt<0>();  // nothing in flight into LDS when the block leaves

  // O^T lane layout: channels 32 db + 8 j + 4 hw + i (VGPR 4j + i) of query
  // l32; the row's sum is split over the lanes l32 and l32 + 32
  const float lt = l + __shfl_xor(l, 32, 64);
  if (qrow < len) {
    const float inv = 1.0f / lt;
    bf16_t* op = a.out + ((size_t)(start + qrow) * PH + h) * PDH + 4 * hw;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (bf16_t)(o[db][4 * j + i] * inv);
        *(bf16x4*)(op + 32 * db + 8 * j) = v;
      }
    if (a.lse && hw == 0) a.lse[(size_t)(start + qrow) * PH + h] = (m + __log2f(lt)) * 0.6931471805599453f;
  }
}

}  // namespace

bool prefill_supported(const mla_dims& d, int act) {
  return act == MLA_BF16 && d.n_heads == PH && d.d_head == PDH && d.d_rope == PDR && d.d_c == 512 &&
         d.d_model % 64 == 0 && d.d_cq % 64 == 0;
}

hipError_t prefill_attention(const PrefillArgs& a) {
  const int qtiles = (a.max_seqlen + BQ - 1) / BQ;
  PaArgs pa{(const bf16_t*)(a.ws + a.L.q), (const bf16_t*)(a.ws + a.L.kc), (const bf16_t*)(a.ws + a.L.vc),
            (const bf16_t*)(a.ws + a.L.kr), a.cu_seqlens, (const float2*)(a.ws + a.L.rope), a.n_tok, qtiles,
            a.n_seq, a.out, a.lse_out};
  MLA_TRY(lds_limit((const void*)&k_prefill_attn, PA_LDS));
  // at most 2^30 workgroups a launch: sequences in chunks
  const int chunk = std::max(1, (1 << 30) / (qtiles * PH));
  for (int s0 = 0; s0 < a.n_seq; s0 += chunk) {
    pa.cu = a.cu_seqlens + s0;
    pa.n_seq = std::min(chunk, a.n_seq - s0);
    MLA_TRY(launch(&k_prefill_attn, dim3(qtiles * pa.n_seq * PH), dim3(256), PA_LDS, a.stream, pa));
  }
  return hipSuccess;
}

hipError_t fast_prefill(const PrefillArgs& a) {
  MLA_TRY(prefill_projections(a));
  return prefill_attention(a);
}

}  // namespace mla

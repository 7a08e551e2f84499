// Split-KV MLA decode attention on MFMA for the DeepSeek-V3 shape
// (d_c 512, d_rope 64, 128 heads, 64-token bf16 or fp8 pages), gfx950.
//
// What it computes (absorbed form; DeepSeek-V3 reading lesson, §2.1.1 and
// Question 2): for every query row (head i, query j) of sequence b and every
// cached token t visible to it inside this split,
//     s_t = qt_i . [c_t ; k^R_t]      (qt = tau*log2(e)*[W^UK_i^T q^C_i ; q^R_i])
// an online softmax in the exp2 domain, and O_i = sum_t p_t c_t / sum_t p_t
// (the attention-weighted latent; W^UV is applied later by the combine).
//
// Work item = (sequence b, split s, row block of 128 rows = one query j and
// all 128 heads).  Four waves, one per SIMD, each owns 32 heads:
//   * its 32 rows of qt stay in VGPRs for the whole split (36 MFMA B operands)
//   * S^T[32 tokens x 32 heads] = K . Q^T with v_mfma_f32_32x32x16_bf16,
//     K read from LDS row-wise (one 16-byte chunk per lane)
//   * softmax per lane (one head, 16 tokens; the other 16 sit in lane ^ 32)
//   * O^T[512 x 32 heads] += V^T . P^T, V^T read from LDS with the gfx950
//     transposing ds_read_b64_tr_b16; P^T comes straight from the S^T
//     accumulator registers (no lane exchange); O^T lives in 256 AGPRs.
// Cache tokens stream HBM -> LDS with global_load_lds_dwordx4 (no VGPR
// staging) through a 3-deep ring of 32-token stages (110 592 B of LDS); the
// 64-wide RoPE part of the queries sits in LDS beside it (16 KiB) so that the
// 512-wide absorbed part (128 VGPRs) and O (256 AGPRs) fit one wave per SIMD.
// The chunk-major swizzled page layout (layout.hpp) makes that copy verbatim
// and both LDS access patterns bank-conflict free.
//
// FP8 cache (E4M3 codes with one fp32 scale per token and 1x128 channel tile,
// lesson §3.3; bf16 k^R): a 4-deep ring of fp8 half-page stages (20 992 B
// each) is filled the same way; each stage is then widened in LDS, by the
// whole block, to the bf16 stage image (code * scale, rounded once to bf16),
// and the bf16 compute above runs on it.  Products stay bf16 x bf16 with fp32
// accumulation.
#include "internal.hpp"
#include "layout.hpp"

namespace mla {
namespace {

constexpr int H = 128, DC = 512, DKV = 576, PAGE = 64;
constexpr int NCH = DKV / 8;               // 72 sixteen-byte chunks per token
constexpr int ST_T = 32;                   // tokens per pipeline stage
constexpr int NST = 3;                     // stages in the LDS ring
constexpr int ST_BYTES = NCH * ST_T * 16;  // 36 864
constexpr int QR_OFF = NST * ST_BYTES;     // q^R rows of the 128 heads: 128 x 64 bf16
constexpr int LDS_BYTES = QR_OFF + H * 64 * 2;  // 126 976
// FP8 layout: q^R at 0, the bf16 work stage, then the fp8 ring
constexpr int F8_CODES = 32 * ST_T * 16;   // 16 384: 32 sixteen-channel chunks x 32 tokens
constexpr int F8_SCALES = ST_T * 16;       // 512: 4 fp32 scales per token
constexpr int F8_ROPE = 8 * ST_T * 16;     // 4 096: 8 chunks x 32 tokens
constexpr int F8_BYTES = F8_CODES + F8_SCALES + F8_ROPE;  // 20 992
constexpr int NST8 = 4;
constexpr int F8_QR_OFF = 0;
constexpr int F8_WORK_OFF = H * 64 * 2;
constexpr int F8_RING_OFF = F8_WORK_OFF + ST_BYTES;
constexpr int LDS_BYTES_FP8 = F8_RING_OFF + NST8 * F8_BYTES;  // 137 216

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;
// LDS-typed pointers keep address arithmetic in 32 bits with constant offsets
// folded into the ds_read immediate field.
typedef __attribute__((address_space(3))) uint8_t lu8;
typedef __attribute__((address_space(3))) const bf16x8 lbf16x8;
typedef __attribute__((address_space(3))) i16x4 li16x4;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One 32-token half of a page into one LDS stage: 36 wave-instructions of
// 1 KiB (chunks 2q and 2q+1), nine per wave.
__device__ __forceinline__ void issue_stage(const uint8_t* page, int half, lu8* dst, int wave, int lane) {
  const uint8_t* src = page + (size_t)(lane >> 5) * (PAGE * 16) + half * (ST_T * 16) + (lane & 31) * 16;
#pragma unroll
  for (int n = 0; n < 9; ++n) {
    const int q = wave + 4 * n;
    __builtin_amdgcn_global_load_lds((gbl_void*)(src + (size_t)(2 * q) * (PAGE * 16)), (lds_void*)(dst + q * 1024),
                                     16, 0, 0);
  }
}


// Everything a pass over the split needs.
struct SplitCtx {
  const uint8_t* pages;
  size_t page_bytes;
  const int32_t* bt_row;
  int p0;       // first page index (in the block-table row) of the split
  int bt_lane;  // lane l holds bt_row[p0 + l] (first 64 pages of the split)
  int t_begin, ntok, nst;
  lu8* lds;
  int wave, lane, cg;
  int kofs_even, kofs_odd, vofs1, vofs2, qr_x;
  const lu8* qr_lds;
  // fp8 pages: offsets of the scale and rope blocks inside a page, and the
  // 1 KiB load instructions this wave issues per stage (6 or 5)
  size_t f8_scale_off, f8_rope_off;
  int f8_issue;
};

// S^T[32 tokens][32 heads] of one stage: 36 MFMAs, K fragments prefetched two
// k-steps ahead, the absorbed query part from VGPRs, the RoPE part from LDS.
__device__ __forceinline__ f32x16 stage_scores(const SplitCtx& c, const lu8* st, const bf16x8 (&qf)[32]) {
  // two independent accumulation chains (even / odd k-steps)
  f32x16 s0 = {}, s1 = {};
  const lu8* ke = st + c.kofs_even;
  const lu8* ko = st + c.kofs_odd;
  bf16x8 k0 = *(lbf16x8*)(ke);
  bf16x8 k1 = *(lbf16x8*)(ko + 1024);
  bf16x8 k2 = *(lbf16x8*)(ke + 2048);
  bf16x8 k3 = *(lbf16x8*)(ko + 3072);
#pragma unroll
  for (int kk = 0; kk < 36; kk += 2) {
    bf16x8 n0 = k0, n1 = k1;
    if (kk + 4 < 36) {
      n0 = *(lbf16x8*)(ke + 1024 * (kk + 4));
      n1 = *(lbf16x8*)(ko + 1024 * (kk + 5));
    }
    bf16x8 q0, q1;
    if (kk < 32) {
      q0 = qf[kk];
      q1 = qf[kk + 1];
    } else {
      q0 = *(lbf16x8*)(c.qr_lds + (((2 * (kk - 32) + c.cg) ^ c.qr_x) * 16));
      q1 = *(lbf16x8*)(c.qr_lds + (((2 * (kk + 1 - 32) + c.cg) ^ c.qr_x) * 16));
    }
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, q0, s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, q1, s1, 0, 0, 0);
    k0 = k2;
    k1 = k3;
    k2 = n0;
    k3 = n1;
  }
  return s0 + s1;
}

// Page holding token t0 (block-table entries of the split are held in lanes).
__device__ __forceinline__ const uint8_t* stage_page(const SplitCtx& c, int t0) {
  const int idx = t0 / PAGE - c.p0;
  const int page = idx < 64 ? __builtin_amdgcn_readlane(c.bt_lane, idx) : c.bt_row[t0 / PAGE];
  return c.pages + (size_t)page * c.page_bytes;
}

// Issues the first two stages of a pass into the ring.
__device__ __forceinline__ void prologue_bf16(const SplitCtx& c) {
  for (int k = 0; k < 2 && k < c.nst; ++k) {
    const int t0 = c.t_begin + k * ST_T;
    issue_stage(stage_page(c, t0), (t0 / ST_T) & 1, c.lds + k * ST_BYTES, c.wave,
                c.lane);
  }
}

// Waits for stage k, then refills the ring slot that stage k-1 used.
__device__ __forceinline__ const lu8* advance_bf16(const SplitCtx& c, int k) {
  if (k + 1 < c.nst) wait_vmcnt<9>();
  else wait_vmcnt<0>();
  ring_barrier();
  if (k + 2 < c.nst) {
    const int t0 = c.t_begin + (k + 2) * ST_T;
    issue_stage(stage_page(c, t0), (t0 / ST_T) & 1, c.lds + ((k + 2) % NST) * ST_BYTES,
                c.wave, c.lane);
  }
  return c.lds + (k % NST) * ST_BYTES;
}

// fp8 half-page stage k: 21 instructions of 1 KiB -- 16 for the codes (chunks
// 2q, 2q+1), one for the 32 tokens' scales (lanes 0..31), four for the rope
// chunks -- instruction i issued by wave i % 4.
__device__ __forceinline__ void issue_fp8(const SplitCtx& c, int k) {
  const int t0 = c.t_begin + k * ST_T;
  const int half = (t0 / ST_T) & 1;
  const uint8_t* page = stage_page(c, t0);
  lu8* dst = c.lds + F8_RING_OFF + (k % NST8) * F8_BYTES;
  const int lofs = (c.lane >> 5) * (PAGE * 16) + half * (ST_T * 16) + (c.lane & 31) * 16;
#pragma unroll
  for (int n = 0; n < 6; ++n) {
    const int i = c.wave + 4 * n;
    if (i < 16) {
      __builtin_amdgcn_global_load_lds((gbl_void*)(page + (size_t)(2 * i) * (PAGE * 16) + lofs),
                                       (lds_void*)(dst + i * 1024), 16, 0, 0);
    } else if (i == 16) {
      if (c.lane < 32)
        __builtin_amdgcn_global_load_lds((gbl_void*)(page + c.f8_scale_off + (size_t)(half * ST_T + c.lane) * 16),
                                         (lds_void*)(dst + F8_CODES), 16, 0, 0);
    } else if (i < 21) {
      __builtin_amdgcn_global_load_lds((gbl_void*)(page + c.f8_rope_off + (size_t)(2 * (i - 17)) * (PAGE * 16) + lofs),
                                       (lds_void*)(dst + F8_CODES + F8_SCALES + (i - 17) * 1024), 16, 0, 0);
    }
  }
}

__device__ __forceinline__ void prologue_fp8(const SplitCtx& c) {
  for (int k = 0; k < NST8 - 1 && k < c.nst; ++k) issue_fp8(c, k);
}

// Widens fp8 stage k into the bf16 stage image: thread handles token tid%32,
// bf16 chunks tid/32 + 8n (n < 8) and rope chunk tid/32.
__device__ __forceinline__ void widen_fp8(const lu8* src, lu8* dst, int tid) {
  const int t = tid & 31, c0 = tid >> 5;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int c = c0 + 8 * n;  // 8-channel chunk, 0..63
    const int C8 = c >> 1;     // 16-channel fp8 chunk
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 code =
        *(__attribute__((address_space(3))) const u32x2*)(src + 16 * (C8 * ST_T + (t ^ slot_x(C8))) + 8 * (c & 1));
    const float sc = *(__attribute__((address_space(3))) const float*)(src + F8_CODES + 16 * t + 4 * (c >> 4));
    bf16x8 v;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t word = code[w];
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
      v[4 * w + 0] = (bf16_t)(lo[0] * sc);
      v[4 * w + 1] = (bf16_t)(lo[1] * sc);
      v[4 * w + 2] = (bf16_t)(hi[0] * sc);
      v[4 * w + 3] = (bf16_t)(hi[1] * sc);
    }
    *(__attribute__((address_space(3))) bf16x8*)(dst + 16 * (c * ST_T + (t ^ slot_x(c)))) = v;
  }
  {
    const int m = c0;  // rope chunk 0..7, same swizzle in source and destination
    const bf16x8 r = *(lbf16x8*)(src + F8_CODES + F8_SCALES + 16 * (m * ST_T + (t ^ slot_x(m))));
    *(__attribute__((address_space(3))) bf16x8*)(dst + 16 * ((64 + m) * ST_T + (t ^ slot_x(m)))) = r;
  }
}

// Waits for fp8 stage k, refills the ring slot of stage k-1, widens stage k
// into the work image (once every wave is done with the previous one).
__device__ __forceinline__ const lu8* advance_fp8(const SplitCtx& c, int k) {
  const int after = min(NST8 - 2, c.nst - 1 - k);
  if (c.f8_issue == 6) {
    if (after >= 2) wait_vmcnt<12>();
    else if (after == 1) wait_vmcnt<6>();
    else wait_vmcnt<0>();
  } else {
    if (after >= 2) wait_vmcnt<10>();
    else if (after == 1) wait_vmcnt<5>();
    else wait_vmcnt<0>();
  }
  ring_barrier();
  if (k + NST8 - 1 < c.nst) issue_fp8(c, k + NST8 - 1);
  lu8* work = c.lds + F8_WORK_OFF;
  widen_fp8(c.lds + F8_RING_OFF + (k % NST8) * F8_BYTES, work, c.wave * 64 + c.lane);
  ring_barrier();
  return work;
}

template <bool FP8>
__device__ __forceinline__ void prologue(const SplitCtx& c) {
  if (FP8) prologue_fp8(c);
  else prologue_bf16(c);
}
template <bool FP8>
__device__ __forceinline__ const lu8* advance(const SplitCtx& c, int k) {
  return FP8 ? advance_fp8(c, k) : advance_bf16(c, k);
}

// Masks the scores of tokens past the end of the split (only the last stage
// can be partial), returns the row max over this lane's 16 tokens.
__device__ __forceinline__ float mask_max(const SplitCtx& c, f32x16& sc, int k) {
  const int nvalid = c.ntok - k * ST_T;
  if (nvalid < ST_T) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 8 * (r >> 2) + 4 * c.cg + (r & 3);
      if (t >= nvalid) sc[r] = -INFINITY;
    }
  }
  float mloc = sc[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, sc[r]);
  return mloc;
}

constexpr float HEADROOM = 96.0f;

// The pass over the split.  O and l accumulate exp2(s - m_ref) weights and O
// is never rescaled, so its 256 accumulators stay in AGPRs.  With fixed ==
// false, m_ref is set to the first stage's maximum and the return value says
// whether a later score rose more than HEADROOM above it in some row of the
// wave; with fixed == true m_ref is the exact maximum of the split.
template <bool FP8>
__device__ __forceinline__ bool attend_pass(const SplitCtx& c, const bf16x8 (&qf)[32], bool fixed, float& m_ref,
                                            f32x16 (&o)[16], float& l_run) {
  prologue<FP8>(c);
  bool ovf = false;
  for (int k = 0; k < c.nst; ++k) {
    const lu8* st = advance<FP8>(c, k);
    f32x16 sc = stage_scores(c, st, qf);
    float mloc = mask_max(c, sc, k);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    if (!fixed && k == 0) m_ref = mloc;
    ovf |= mloc > m_ref + HEADROOM;
    bf16x8 pb[2];
    float ls = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // raw v_exp_f32: results below 2^-126 flush to zero, harmless here
      const float pv = __builtin_amdgcn_exp2f(fminf(sc[r] - m_ref, HEADROOM));
      ls += pv;
      pb[r >> 3][r & 7] = (bf16_t)pv;
    }
    l_run += ls;

    // O^T[c][h] += V^T[c][t] P^T[t][h] for the stage's tokens 16hf..16hf+15;
    // consecutive MFMAs go to different accumulators
    // The per-stage lane bases are made opaque so that the compiler keeps one
    // base register each and folds every (cb, hf) offset into the instruction.
    uint32_t b1 = (uint32_t)(uintptr_t)(st + c.vofs1), b2 = (uint32_t)(uintptr_t)(st + c.vofs2);
    asm volatile("" : "+v"(b1), "+v"(b2));
    const lu8* p1 = (const lu8*)(uintptr_t)b1;
    const lu8* p2 = (const lu8*)(uintptr_t)b2;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) {
        const lu8* a1 = p1 + cb * (4 * ST_T * 16) + hf * 256;
        const lu8* a2 = p2 + cb * (4 * ST_T * 16) + hf * 256;
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)a1);
        const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)a2);
        const short s8 __attribute__((ext_vector_type(8))) = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
        o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, s8), pb[hf], o[cb], 0, 0, 0);
      }
    }
  }
  return ovf;
}

// Scores only: the exact row maximum over the split.
template <bool FP8>
__device__ __forceinline__ float max_pass(const SplitCtx& c, const bf16x8 (&qf)[32]) {
  prologue<FP8>(c);
  float mx = -INFINITY;
  for (int k = 0; k < c.nst; ++k) {
    const lu8* st = advance<FP8>(c, k);
    f32x16 sc = stage_scores(c, st, qf);
    mx = fmaxf(mx, mask_max(c, sc, k));
  }
  return fmaxf(mx, __shfl_xor(mx, 32, 64));
}

template <bool FP8>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_attn_v3(int s_q, int S, int pps, int P_items, const bf16_t* __restrict__ qt,
               const uint8_t* __restrict__ pages, size_t page_bytes, size_t f8_scale_off, size_t f8_rope_off,
               const int32_t* __restrict__ bt, int max_pages, const int32_t* __restrict__ seqlens,
               bf16_t* __restrict__ opart, float* __restrict__ lpart, int32_t* __restrict__ hdr, int batch) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lu8* lds = (lu8*)lds_raw;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (blockIdx.x == 0 && threadIdx.x == 0) {  // the split plan, for the combine
    hdr[HDR_MAGIC] = WS_MAGIC; hdr[HDR_S] = S; hdr[HDR_PPS] = pps; hdr[HDR_BATCH] = batch;
    hdr[HDR_SQ] = s_q; hdr[HDR_H] = H; hdr[HDR_DC] = DC; hdr[HDR_PDT] = MLA_BF16;
  }
  const int RB = s_q;
  // The RB row blocks of one (b, s) share blockIdx % 8, i.e. one XCD and its
  // L2, and are dispatched next to each other.
  const int bid = blockIdx.x;
  const int p = (bid / (8 * RB)) * 8 + bid % 8;
  const int j = (bid / 8) % RB;
  if (p >= P_items) return;
  const int b = p / S, s = p % S;

  const int L = seqlens[b];
  int vis = L > 0 ? L - s_q + j + 1 : 0;
  vis = vis < 0 ? 0 : vis;
  SplitCtx c;
  c.t_begin = s * pps * PAGE;
  const int t_end = min(vis, c.t_begin + pps * PAGE);
  c.ntok = t_end > c.t_begin ? t_end - c.t_begin : 0;
  c.nst = (c.ntok + ST_T - 1) / ST_T;

  const int cg = lane >> 5;  // lane half: k-group / token quad in the MFMA layouts
  const int hrow = wave * 32 + (lane & 31);
  const size_t prow = (((size_t)b * S + s) * s_q + j) * H + hrow;
  bf16_t* orow = opart + prow * DC;

  if (c.nst == 0) {
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) *(uint2*)(orow + 32 * cb + 8 * r4 + 4 * cg) = make_uint2(0u, 0u);
    if (cg == 0) lpart[prow] = -INFINITY;
    return;
  }

  // This wave's 32 query rows as MFMA B operands: lane holds qt[hrow][16kk + 8cg .. +8]
  // for the 32 absorbed k-steps; the RoPE part of all 128 rows goes to LDS,
  // row h at QR_OFF + 128h with its eight 16-byte chunks permuted by (h/2)%8.
  const bf16_t* qblk = qt + (size_t)(b * s_q + j) * H * DKV;
  const bf16_t* qrow = qblk + (size_t)hrow * DKV + 8 * cg;
  bf16x8 qf[32];
#pragma unroll
  for (int kk = 0; kk < 32; ++kk) qf[kk] = *(const bf16x8*)(qrow + 16 * kk);
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int i = wave + 4 * n;
    const int pos = 64 * i + lane, h = pos >> 3, lc = (pos & 7) ^ ((h >> 1) & 7);
    __builtin_amdgcn_global_load_lds((gbl_void*)(qblk + (size_t)h * DKV + DC + 8 * lc),
                                     (lds_void*)(lds + (FP8 ? F8_QR_OFF : QR_OFF) + i * 1024), 16, 0, 0);
  }

  c.pages = pages;
  c.page_bytes = page_bytes;
  c.bt_row = bt + (size_t)b * max_pages;
  c.p0 = c.t_begin / PAGE;
  {
    const int np = (c.ntok + PAGE - 1) / PAGE;
    c.bt_lane = lane < np ? c.bt_row[c.p0 + lane] : 0;
  }
  c.lds = lds;
  c.wave = wave;
  c.lane = lane;
  c.cg = cg;
  const int tr = lane & 31;
  c.kofs_even = cg * (ST_T * 16) + (tr ^ slot_x(cg)) * 16;       // chunk 2kk+cg, kk even
  c.kofs_odd = cg * (ST_T * 16) + (tr ^ slot_x(2 + cg)) * 16;  // chunk 2kk+cg, kk odd
  c.qr_lds = lds + (FP8 ? F8_QR_OFF : QR_OFF) + hrow * 128;
  c.f8_scale_off = f8_scale_off;
  c.f8_rope_off = f8_rope_off;
  c.f8_issue = wave == 0 ? 6 : 5;
  c.qr_x = (hrow >> 1) & 7;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int tq = i16 >> 2, qq = i16 & 3;
  // V^T reads: chunk C = 4cb + 2(g16&1) + (qq>>1), so C&3 is lane-constant
  const int cl = 2 * (g16 & 1) + (qq >> 1);
  const int cx = slot_x(cl);
  c.vofs1 = cl * (ST_T * 16) + ((4 * (g16 >> 1) + tq) ^ cx) * 16 + (qq & 1) * 8;
  c.vofs2 = cl * (ST_T * 16) + ((8 + 4 * (g16 >> 1) + tq) ^ cx) * 16 + (qq & 1) * 8;

  f32x16 o[16];
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) o[cb] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.0f;
  // Normally one pass.  If some score rose more than 2^96 above the first
  // stage's maximum, the item is redone: a scores-only pass finds the exact
  // maximum, then a full pass accumulates against it.
  bool fixed = false;
#pragma clang loop unroll(disable)
  for (;;) {
    const bool ovf = attend_pass<FP8>(c, qf, fixed, m_ref, o, l_run);
    __syncthreads();  // every wave is done with the ring
    if (fixed || !__syncthreads_or(ovf)) break;
    m_ref = max_pass<FP8>(c, qf);
    __syncthreads();
    fixed = true;
    l_run = 0.0f;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) o[cb] = f32x16{};
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (bf16_t)(o[cb][4 * r4 + e] * inv);
      *(bf16x4*)(orow + 32 * cb + 8 * r4 + 4 * cg) = v;
    }
    __builtin_amdgcn_sched_barrier(0);  // one accumulator block at a time through VGPRs
  }
  if (cg == 0) lpart[prow] = m_ref + log2f(l_tot);
}

}  // namespace

hipError_t fast_attention_v1(const DecodeArgs& a) {
  const bool fp8 = a.cache_dtype == MLA_FP8_E4M3;
  auto kern = fp8 ? &k_attn_v3<true> : &k_attn_v3<false>;
  const int lds = fp8 ? LDS_BYTES_FP8 : LDS_BYTES;
  static bool attr_set[2] = {false, false};
  if (!attr_set[fp8]) {
    MLA_TRY(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    attr_set[fp8] = true;
  }
  const int P_items = a.batch * a.S;
  const int RB = a.s_q;
  const int grid = ((P_items + 7) / 8) * 8 * RB;
  MLA_TRY(launch(kern, dim3(grid), dim3(256), lds, a.stream, a.s_q, a.S, a.pages_per_split, P_items,
                 (const bf16_t*)(a.ws + a.L.qt), a.pages, a.g.page_bytes, a.g.fp8_scale_off, a.g.fp8_rope_off,
                 a.block_table, a.max_pages, a.seqlens, (bf16_t*)(a.ws + a.L.opart), (float*)(a.ws + a.L.lpart),
                 (int32_t*)(a.ws + a.L.header), a.batch));
  return hipSuccess;
}

}  // namespace mla

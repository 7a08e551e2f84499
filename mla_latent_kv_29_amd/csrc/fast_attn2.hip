// Split-KV MLA decode attention on MFMA for the DeepSeek-V3 shape
// (d_c 512, d_rope 64, 128 heads, 64-token bf16 or fp8 pages), gfx950.
//
// What it computes (absorbed form; DeepSeek-V3 reading lesson, §2.1.1 and
// Question 2): for every query row (head i, query j) of sequence b and every
// cached token t visible to it inside this split,
//     s_t = qt_i . [c_t ; k^R_t]      (qt = tau*log2(e)*[W^UK_i^T q^C_i ; q^R_i])
// exp2-domain softmax weights, and O_i = sum_t p_t c_t / sum_t p_t (the
// attention-weighted latent; W^UV is applied later by the combine).
//
// Work item = (sequence b, split s, query j): all 128 heads over the split's
// tokens.  Four waves, one per SIMD, split the two products differently:
//   * scores: wave w owns heads 32w..32w+31.  S^T[16 tokens][16 heads]
//     blocks = K . Q^T with v_mfma_f32_16x16x32_bf16 (each K fragment read
//     from LDS feeds two of them); the wave's 512-wide absorbed query rows
//     sit in 128 VGPRs, the 64-wide RoPE rows of all heads in LDS.
//   * P.V: wave w owns latent channels 128w..128w+127 of all 128 heads.
//     O^T[128 ch][128 heads] += V^T . P^T with v_mfma_f32_32x32x16_bf16 into
//     all 256 AGPRs; V^T comes from the staged tokens with the transposing
//     ds_read_b64_tr_b16, P^T from an LDS buffer that every wave writes its
//     heads' weights to.
// Splitting P.V by channel means each wave reads only a quarter of V.  A
// step covers two 16-token stages: the scores of stages 2m, 2m+1 and the P.V
// of stages 2m-2, 2m-1 run between the same two barriers, so one barrier per
// 32 tokens publishes both the new stages and the previous weights.  The
// softmax VALU work is interleaved one slot at a time with the P.V MFMAs, so
// it issues while the matrix unit is busy.
//
// The score MFMAs are written as inline asm with VGPR accumulators: with O
// holding every AGPR, compiler-selected MFMAs would put the scores in AGPRs
// too and shuttle O through VGPRs each step.  Their one hazard the compiler
// cannot see -- a VALU read of an accumulator right after the MFMA that
// writes it -- is covered by s_nop wait states after each chain's last MFMA.
//
// Cache tokens stream HBM -> LDS with global_load_lds_dwordx4 (no VGPR
// staging) through a 7-slot ring of 16-token stages: two being scored, two
// in P.V, three in flight.  The chunk-major swizzled page layout makes that
// copy verbatim and every LDS access pattern bank-conflict free.
//
// FP8 cache (E4M3 codes with one fp32 scale per token and 1x128 channel tile,
// lesson §3.3; bf16 k^R): the copies land in a 5-slot ring of fp8 stages
// (three in flight), and after the step's first barrier the block widens the
// two stages it is about to score into bf16 images (code * scale, rounded
// once to bf16) in a 4-slot ring; a second barrier publishes them, and the
// bf16 step code above runs unchanged.  Products stay bf16 x bf16 with fp32
// accumulation.  The fp8 copies are issued in the widening phase rather than
// between the score MFMAs, which keeps the step loop free of spills.
//
// Softmax reference: the first step's row maximum, with 96 log2 units of
// headroom, so O is never rescaled.  The pass also collects the exact row
// maximum.  If some score exceeded the reference by more than the headroom,
// the block runs the pass again against that maximum.  Both passes are one
// runtime loop over the same code: a second copy of the pass would not fit
// the register file.
//
// The normalised partial rows leave through LDS so that each store writes a
// whole 1 KiB row.
#include <utility>
#include "internal.hpp"
#include "layout.hpp"

namespace mla {
namespace {

constexpr int H = 128, DC = 512, DKV = 576, PAGE = 64;
constexpr int NW = 4;                      // waves per block
constexpr int T = 16;                      // tokens per stage
constexpr int NCH = DKV / 8;               // 72 sixteen-byte chunks per token
constexpr int ST_BYTES = NCH * T * 16;     // 18 432
constexpr int P_STAGE = H * T * 2;         // 4 096
constexpr int P_BYTES = 2 * P_STAGE;       // 8 192
// fp8 stage in LDS: the 16 tokens' E4M3 codes (32 sixteen-channel chunks x 16
// slots), their bf16 k^R (8 eight-channel chunks x 16 slots), then their fp32
// scales (4 per token); in page order, so one 1 KiB copy instruction n lands
// at 1024 n.
constexpr int F8_ST = 8192 + 2048 + 256;   // 10 496
constexpr int F8_ROPE = 8192, F8_SCALES = 10240;
// the same three blocks inside a 64-token fp8 page
constexpr int F8_PG_SCALES = PAGE * DC, F8_PG_ROPE = F8_PG_SCALES + PAGE * (DC / 128) * 4;  // 32 768, 33 792

// LDS layout.  bf16 cache: a 7-slot ring of 16-token stages.  fp8 cache: the
// copies land in a 5-slot ring of fp8 stages, and each stage is widened to
// its bf16 image in a 4-slot ring (two being scored, two in P.V).  Then two
// P buffers, the RoPE query rows (128 x 64 bf16) and the per-head sums.
template <bool F8>
struct Lay {
  static constexpr int NST = F8 ? 4 : 7;                 // bf16 stage slots
  static constexpr int NF8 = F8 ? 5 : 0;                 // fp8 stage slots
  static constexpr int F8_OFF = NST * ST_BYTES;          // 73 728 (fp8 ring)
  static constexpr int P_OFF = F8_OFF + NF8 * F8_ST;     // 129 024 | 126 208
  static constexpr int QR_OFF = P_OFF + 2 * P_BYTES;
  static constexpr int L_OFF = QR_OFF + H * 64 * 2;
  static constexpr int LDS_BYTES = L_OFF + H * 4;        // 162 304 | 159 488
  static constexpr int COPIES = F8 ? 11 : NCH / 4;       // 1 KiB copy instructions per stage
};
static_assert(Lay<false>::LDS_BYTES <= 160 * 1024 && Lay<true>::LDS_BYTES <= 160 * 1024, "LDS");

typedef __attribute__((address_space(3))) uint8_t lu8;
typedef __attribute__((address_space(3))) const bf16x8 lbf16x8;
typedef __attribute__((address_space(3))) i16x4 li16x4;

// One wave-wide 1 KiB copy HBM -> LDS: lane l moves 16 bytes from
// sbase + voff(l) to lds_addr + 16 l.  sbase and lds_addr are wave-uniform.
// Written as inline asm so that the compiler does not track these copies: it
// would otherwise make every later LDS read wait for all of them, draining
// the ring each step.  Completion is waited for explicitly (wait_vmcnt)
// before the barrier that publishes a stage.  Nothing else in this kernel
// uses M0.
__device__ __forceinline__ void dma_1k(const uint8_t* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory");
}

// The same with M0 = lds_base + OFS (one scalar add instead of an address
// computation and a move per copy).
template <int OFS>
__device__ __forceinline__ void dma_1k_at(const uint8_t* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base), "i"(OFS)
               : "memory", "scc");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

struct Ctx {
  const uint8_t* pages;
  size_t page_bytes;
  const int32_t* bt_row;
  int p0, bt_lane;
  int t_begin, ntok, nst, nsteps;
  lu8* lds;
  uint32_t lds_addr;
  int wave, lane;
  uint32_t dma_ofs;           // lane part of a stage copy
  uint32_t dma_ofs_w;         // bf16: the same plus this wave's first copy (4096 * wave)
  uint32_t koff;              // K fragment of the scores MFMA
  uint32_t qr_ofs0, qr_ofs1;  // RoPE query fragments (k-steps 16, 17)
  uint32_t vofs1, vofs2;      // V^T transposing reads (wave's first channel block)
  uint32_t pw_ofs, pr_ofs;    // P write (scores layout) / read (P.V layout)
};

template <bool F8>
__device__ __forceinline__ int wrap(int x) { return x >= Lay<F8>::NST ? x - Lay<F8>::NST : x; }
__device__ __forceinline__ int wrap5(int x) { return x >= 5 ? x - 5 : x; }

__device__ __forceinline__ const uint8_t* stage_page(const Ctx& c, int t0) {
  const int idx = t0 / PAGE - c.p0;
  const int page = __builtin_amdgcn_readfirstlane(idx < 64 ? __builtin_amdgcn_readlane(c.bt_lane, idx) : c.bt_row[t0 / PAGE]);
  return c.pages + (size_t)page * c.page_bytes;
}

// Copy instruction ii of a stage whose quarter-page base is src (the page
// plus 256 bytes per earlier 16-token quarter) into the stage at dst.  bf16:
// 18 instructions of four 256-byte chunk runs.  fp8: 8 of codes, 2 of k^R, and
// the 256 bytes of scales on lanes 0-15.
template <bool F8>
__device__ __forceinline__ void copy_1k(const Ctx& c, const uint8_t* src, uint32_t dst, int ii) {
  if constexpr (!F8) {
    dma_1k(src + 4096 * ii, c.dma_ofs, dst + 1024 * ii);
  } else {
    const uint8_t* s = ii < 8 ? src + 4096 * ii : ii < 10 ? src + F8_PG_ROPE + 4096 * (ii - 8) : src + F8_PG_SCALES;
    if (ii < 10 || c.lane < 16) dma_1k(s, c.dma_ofs, dst + 1024 * ii);
  }
}
template <bool F8>
__device__ __forceinline__ uint32_t stage_dst(const Ctx& c, int slot) {
  return c.lds_addr + (F8 ? Lay<F8>::F8_OFF + slot * F8_ST : slot * ST_BYTES);
}

// Stage i (tokens t_begin + 16 i ..) into ring slot `slot` (fp8: the fp8
// ring); wave w issues copy instructions w, w+4, ...
template <bool F8>
__device__ __forceinline__ void issue_stage(const Ctx& c, int i, int slot) {
  if (i >= c.nst) return;
  const int t0 = c.t_begin + i * T;
  const uint8_t* src = stage_page(c, t0) + ((t0 / T) & 3) * (T * 16);
  const uint32_t dst = stage_dst<F8>(c, slot);
#pragma unroll
  for (int n = 0; n < 5; ++n) {
    const int ii = c.wave + NW * n;
    if (ii < Lay<F8>::COPIES) copy_1k<F8>(c, src, dst, ii);
  }
}

// A stage copy prepared for issue one instruction at a time, so that the
// copies can be spread between matrix instructions: a wave whose copies wait
// for the address unit cannot issue anything else meanwhile.
struct StageCopy {
  const uint8_t* src;  // nullptr: nothing to copy
  uint32_t dst;
};
template <bool F8>
__device__ __forceinline__ StageCopy plan_stage(const Ctx& c, int i, int slot) {
  StageCopy s;
  s.src = nullptr;
  s.dst = stage_dst<F8>(c, slot) + (F8 ? 0 : 1024 * c.wave);  // bf16: this wave's first copy
  if (i < c.nst) {
    const int t0 = c.t_begin + i * T;
    s.src = stage_page(c, t0) + ((t0 / T) & 3) * (T * 16);
  }
  return s;
}
// Instruction n (0..4) of this wave's share of a stage copy.
// bf16: copy ii = wave + 4n reads src + 4096 ii into dst + 1024 ii; the
// wave's part sits in dma_ofs_w and s.dst, n's part in the offsets below.
template <int N>
__device__ __forceinline__ void copy_part(const Ctx& c, const StageCopy& s) {
  static_assert(Lay<false>::COPIES == 18, "five copies on waves 0-1, four on waves 2-3");
  if (s.src != nullptr && (N < 4 || c.wave < 2)) dma_1k_at<4096 * N>(s.src, c.dma_ofs_w + 16384 * N, s.dst);
}
// n is a constant once the k-step loop is unrolled
__device__ __forceinline__ void copy_at(const Ctx& c, const StageCopy& s, int n) {
  switch (n) {
    case 0: copy_part<0>(c, s); break;
    case 1: copy_part<1>(c, s); break;
    case 2: copy_part<2>(c, s); break;
    case 3: copy_part<3>(c, s); break;
    default: copy_part<4>(c, s); break;
  }
}

// Before step m: stages 2m and 2m+1 have landed once at most the copies of
// stage 2m+2 (issued one step earlier) are outstanding.
template <bool F8>
__device__ __forceinline__ void wait_step(const Ctx& c, int m) {
  if (2 * m + 2 < c.nst) {
    if constexpr (F8) {  // 11 copies: three on waves 0-2, two on wave 3
      if (c.wave < 3) wait_vmcnt<3>();
      else wait_vmcnt<2>();
    } else {  // 18 copies: five on waves 0-1, four on waves 2-3
      if (c.wave < 2) wait_vmcnt<5>();
      else wait_vmcnt<4>();
    }
  } else {
    wait_vmcnt<0>();
  }
}

// Score MFMA with a VGPR accumulator (see the file comment).
__device__ __forceinline__ f32x4 mfma_s0(bf16x8 a, bf16x8 b) {
  f32x4 c;
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
  return c;
}
__device__ __forceinline__ f32x4 mfma_s(bf16x8 a, bf16x8 b, f32x4 c) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  return c;
}
// Last MFMA of a chain: 12 wait states before anything may read the result.
__device__ __forceinline__ f32x4 mfma_s_last(bf16x8 a, bf16x8 b, f32x4 c) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 3" : "+v"(c) : "v"(a), "v"(b));
  return c;
}

// S^T[16 tokens][16 heads] for stages A, B x head blocks 0, 1: 72 MFMAs in
// four chains; every K fragment feeds two.  The K fragments of k-step ks+KD
// are read while k-step ks multiplies; sched_barrier keeps that order (the
// scheduler would otherwise sink each read to its use).
constexpr int KD = 4;
template <bool F8>
__device__ __forceinline__ bf16x8 rope_q(const Ctx& c, int ks, int hb) {
  return *(lbf16x8*)(c.lds + Lay<F8>::QR_OFF + (ks == 16 ? c.qr_ofs0 : c.qr_ofs1) + 16 * 128 * hb);
}
template <bool F8>
__device__ __forceinline__ void step_scores(const Ctx& c, const lu8* stA, const lu8* stB, const bf16x8 (&qf)[16][2],
                                            f32x4 (&sc)[2][2], const StageCopy& cx, const StageCopy& cy) {
  const lu8* ka = stA + c.koff;
  const lu8* kb = stB + c.koff;
  bf16x8 fa[KD], fb[KD];
#pragma unroll
  for (int d = 0; d < KD; ++d) {
    fa[d] = *(lbf16x8*)(ka + 1024 * d);
    fb[d] = *(lbf16x8*)(kb + 1024 * d);
  }
  bf16x8 r0[2], r1[2];
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    if (ks == 12) {  // RoPE query fragments for k-steps 16, 17
      r0[0] = rope_q<F8>(c, 16, 0); r0[1] = rope_q<F8>(c, 16, 1);
      r1[0] = rope_q<F8>(c, 17, 0); r1[1] = rope_q<F8>(c, 17, 1);
    }
    const bf16x8 a = fa[ks % KD], b = fb[ks % KD];
    const bf16x8 q0 = ks < 16 ? qf[ks][0] : (ks == 16 ? r0[0] : r1[0]);
    const bf16x8 q1 = ks < 16 ? qf[ks][1] : (ks == 16 ? r0[1] : r1[1]);
    __builtin_amdgcn_sched_barrier(0);
    if (ks == 0) {
      sc[0][0] = mfma_s0(a, q0);
      sc[0][1] = mfma_s0(a, q1);
      sc[1][0] = mfma_s0(b, q0);
      sc[1][1] = mfma_s0(b, q1);
    } else if (ks < 17) {
      sc[0][0] = mfma_s(a, q0, sc[0][0]);
      sc[0][1] = mfma_s(a, q1, sc[0][1]);
      sc[1][0] = mfma_s(b, q0, sc[1][0]);
      sc[1][1] = mfma_s(b, q1, sc[1][1]);
    } else {
      sc[0][0] = mfma_s_last(a, q0, sc[0][0]);
      sc[0][1] = mfma_s_last(a, q1, sc[0][1]);
      sc[1][0] = mfma_s_last(b, q0, sc[1][0]);
      sc[1][1] = mfma_s_last(b, q1, sc[1][1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (ks + KD < 18) {
      fa[ks % KD] = *(lbf16x8*)(ka + 1024 * (ks + KD));
      fb[ks % KD] = *(lbf16x8*)(kb + 1024 * (ks + KD));
    }
    // the next two stages' copies go out between these MFMAs, early in the
    // step: the first at k-steps 1..5, the second at 6..10
    if constexpr (!F8) {  // (the fp8 copies go out in the widening phase)
      if (ks >= 1 && ks <= 5) copy_at(c, cx, ks - 1);
      if (ks >= 6 && ks <= 10) copy_at(c, cy, ks - 6);
    }
  }
}

// Lane layout of S^T: head 16w + lane%16, tokens 4*(lane/16) + r.  Masks
// tokens past the end of the split (nvalid may be <= 0: a padding stage).
__device__ __forceinline__ void mask(const Ctx& c, f32x4& s, int nvalid) {
  if (nvalid < T) {
    const int tb = 4 * (c.lane >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (tb + r >= nvalid) s[r] = -INFINITY;
  }
}

constexpr float HEADROOM = 96.0f;

// Maxima as single instructions: fmaxf on values the compiler cannot prove
// quiet (the scores come from inline asm) costs two extra canonicalising
// instructions per call.  Scores are finite or -inf.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Maximum over the lanes l, l^16 (permlane16 swap leaves the two values of
// each pair in the two results) and over l, l^32.
__device__ __forceinline__ float max_x16(float m) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float m) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// P.V MFMAs of stages 2m-2, 2m-1 interleaved with the softmax of this
// step's (masked) scores: the VALU instructions issue while each MFMA
// occupies the matrix unit.  A wave issues about one instruction per four
// cycles and a 32x32x16 MFMA keeps the unit busy for 32, so the softmax is
// cut into 12 items of a few instructions, spread over the 32 slots
// (generated at compile time; sched_barrier pins their order); head blocks
// 0 and 1 alternate, which also spaces each item from the one it needs.  Weights go to P buffer m&1 as bf16; lane
// heads 32w + 16hb + lane%16 (hb = 0, 1).
struct PvwState {
  const Ctx& c;
  int m;
  const f32x4 (&sc)[2][2];
  const bf16x8 (&v)[2][4];
  const bf16x8 (&p)[2][4];
  f32x16 (&o)[4][4];
  float (&m_ref)[2];
  float (&m_all)[2];
  float (&l_run)[2];
  bool& ovf;
  lu8* pw;
  float ml[2];
  f32x4 xa[2], xb[2];
};

template <int K>
__device__ __forceinline__ void pvw_slot(PvwState& st) {
  {
    constexpr int j = K >> 4, hb = (K >> 2) & 3, i = K & 3;
    st.o[i][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.v[j][i], st.p[j][hb], st.o[i][hb], 0, 0, 0);
  }
  // item i (0..11) sits in slot 8i/3: part i/2 of head block i%2
  constexpr int item = (3 * K + 7) / 8;
  if constexpr (item < 12 && (8 * item) / 3 == K) {
    constexpr int h = item & 1, part = item >> 1;
    const f32x4 sA = st.sc[0][h], sB = st.sc[1][h];
    if constexpr (part == 0) {
      st.ml[h] = vmax(vmax3(sA[0], sA[1], sA[2]), vmax3(sA[3], sB[0], vmax3(sB[1], sB[2], sB[3])));
    } else if constexpr (part == 1) {
      st.ml[h] = max_x16(st.ml[h]);
    } else if constexpr (part == 2) {
      st.ml[h] = max_x32(st.ml[h]);
      st.m_all[h] = vmax(st.m_all[h], st.ml[h]);
      // the reference: the first step's maximum, or the exact maximum
      // already in m_ref when the pass is redone (it is never smaller)
      if (st.m == 0) st.m_ref[h] = vmax(st.m_ref[h], st.ml[h]);
      st.ovf |= st.ml[h] > st.m_ref[h] + HEADROOM;
    } else if constexpr (part == 3) {
      // raw v_exp_f32: results below 2^-126 flush to zero, harmless here; a
      // score above the headroom only occurs in a pass that is redone
#pragma unroll
      for (int r = 0; r < 4; ++r) st.xa[h][r] = __builtin_amdgcn_exp2f(sA[r] - st.m_ref[h]);
    } else if constexpr (part == 4) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st.xb[h][r] = __builtin_amdgcn_exp2f(sB[r] - st.m_ref[h]);
    } else {
      const f32x4 xa = st.xa[h], xb = st.xb[h];
      st.l_run[h] += (xa[0] + xa[1]) + (xa[2] + xa[3]) + (xb[0] + xb[1]) + (xb[2] + xb[3]);
      bf16x4 pa, pb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pa[r] = (bf16_t)xa[r];
        pb[r] = (bf16_t)xb[r];
      }
      *(__attribute__((address_space(3))) bf16x4*)(st.pw + 512 * h) = pa;
      *(__attribute__((address_space(3))) bf16x4*)(st.pw + 512 * h + P_STAGE) = pb;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int... K>
__device__ __forceinline__ void pvw_slots(PvwState& st, std::integer_sequence<int, K...>) {
  (pvw_slot<K>(st), ...);
}

template <bool F8>
__device__ __forceinline__ void pv_weights_step(const Ctx& c, int m, const f32x4 (&sc)[2][2], const lu8* stA,
                                                const lu8* stB, const lu8* prd, f32x16 (&o)[4][4],
                                                float (&m_ref)[2], float (&m_all)[2], float (&l_run)[2], bool& ovf) {
  bf16x8 v[2][4], p[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const lu8* st = j ? stB : stA;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)(st + c.vofs1 + 1024 * i));
      const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)(st + c.vofs2 + 1024 * i));
      const short s8 __attribute__((ext_vector_type(8))) = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
      v[j][i] = __builtin_bit_cast(bf16x8, s8);
    }
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) p[j][hb] = *(lbf16x8*)(prd + j * P_STAGE + 1024 * hb);
  }
  __builtin_amdgcn_sched_barrier(0);
  PvwState st{c, m, sc, v, p, o, m_ref, m_all, l_run, ovf, c.lds + Lay<F8>::P_OFF + (m & 1) * P_BYTES + c.pw_ofs,
              {0.0f, 0.0f}, {}, {}};
  pvw_slots(st, std::make_integer_sequence<int, 32>{});
}

// Zeroes the latent part of the tokens past the end of the split in its last
// stage, so that whatever bytes the page holds there cannot turn a zero
// weight into NaN in P.V.  Runs after the barrier that publishes the stage
// and before the one that precedes its P.V.
__device__ __forceinline__ void zero_tail(const Ctx& c, int slot) {
  const int nvalid = c.ntok - (c.nst - 1) * T;
  if (nvalid >= T) return;
  lu8* st = c.lds + slot * ST_BYTES;
  const int tid = c.wave * 64 + c.lane;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int idx = tid + 256 * n;  // 64 latent chunks x 16 token slots
    const int C = idx >> 4, t = idx & 15;
    if (t >= nvalid) *(__attribute__((address_space(3))) bf16x8*)(st + 256 * C + 16 * (t ^ slot_x(C))) = bf16x8{};
  }
}

// The pass over the split.  Step m: score MFMAs of stages 2m, 2m+1 with the
// copies of stages 2m+3, 2m+4 (into the slots of 2m-4, 2m-3) between them,
// then the P.V of stages 2m-2, 2m-1 interleaved with the softmax of 2m, 2m+1.  Step 0 has no
// P.V: it multiplies zero weights (P buffer 1 starts zeroed) with the RoPE
// query rows standing in for V; after the last scores, all-(-inf) scores give
// zero weights.  So one copy of the step code serves every step.  A missing
// second stage is scored from the first one's slot with every token masked.
// m_all collects the exact maximum of each of the wave's heads; the return
// value says whether a score exceeded the reference by more than the
// headroom (only possible with fixed == false).
template <bool F8>
__device__ __forceinline__ void zero_p1(const Ctx& c) {
  const int tid = c.wave * 64 + c.lane;
  *(__attribute__((address_space(3))) bf16x8*)(c.lds + Lay<F8>::P_OFF + P_BYTES + 16 * tid) = bf16x8{};
  *(__attribute__((address_space(3))) bf16x8*)(c.lds + Lay<F8>::P_OFF + P_BYTES + 16 * (tid + 256)) = bf16x8{};
}

// fp8: widens stage slot `fs` of the fp8 ring into the bf16 image in slot
// `bs`: code * scale, rounded once to bf16 (products then stay bf16 x bf16
// with fp32 accumulation); k^R is copied.  Thread: token tid%16, 8-channel
// chunks tid/16 + 16 j (scale tile j), and k^R chunk tid/16 on threads < 128.
__device__ __forceinline__ void widen_stage(const Ctx& c, int fs, int bs) {
  const int tid = c.wave * 64 + c.lane, t = tid & 15, cq = tid >> 4;
  // chunks cq + 16 j share the slot permutation (x depends on the chunk mod
  // 4), so one source and one destination offset serve all four
  const int dofs = 256 * cq + 16 * (t ^ slot_x(cq));
  const lu8* f8 = c.lds + Lay<true>::F8_OFF + fs * F8_ST;
  const lu8* src = f8 + 256 * (cq >> 1) + 16 * (t ^ slot_x(cq >> 1)) + 8 * (cq & 1);
  const lu8* scl = f8 + F8_SCALES + 16 * t;
  lu8* dst = c.lds + bs * ST_BYTES + dofs;
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // 8-channel chunk cq + 16 j = 16-channel chunk cq/2 + 8 j, scale tile j
    const u32x2 code = *(__attribute__((address_space(3))) const u32x2*)(src + 2048 * j);
    const float sc = *(__attribute__((address_space(3))) const float*)(scl + 4 * j);
    bf16x8 v;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)code[w], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)code[w], true);
      v[4 * w + 0] = (bf16_t)(lo[0] * sc);
      v[4 * w + 1] = (bf16_t)(lo[1] * sc);
      v[4 * w + 2] = (bf16_t)(hi[0] * sc);
      v[4 * w + 3] = (bf16_t)(hi[1] * sc);
    }
    *(__attribute__((address_space(3))) bf16x8*)(dst + 4096 * j) = v;
  }
  // k^R chunk cq (threads < 128): the same slot order in both (x(64 + m) = x(m))
  if (tid < 128) *(__attribute__((address_space(3))) bf16x8*)(dst + 256 * 64) = *(lbf16x8*)(f8 + F8_ROPE + dofs);
}
template <bool F8>
__device__ __forceinline__ bool run_pass(const Ctx& c, const bf16x8 (&qf)[16][2], float (&m_ref)[2],
                                         float (&m_all)[2], float (&l_run)[2], f32x16 (&o)[4][4]) {
  using Ly = Lay<F8>;
  zero_p1<F8>(c);
  bool ovf = false;
  int sa = 0;  // slot of stage 2m
  int fa = 0;  // fp8: fp8-ring slot of stage 2m
  for (int m = 0; m <= c.nsteps; ++m) {
    if (m < c.nsteps) wait_step<F8>(c, m);
    ring_barrier();
    if constexpr (F8) {
      // this step's two stages into the bf16 slots freed by the last P.V
      if (m < c.nsteps) {
        widen_stage(c, fa, sa);
        if (2 * m + 1 < c.nst) widen_stage(c, wrap5(fa + 1), wrap<F8>(sa + 1));
      }
      // copies of stages 2m+3, 2m+4 into the fp8 slots widened last step
      issue_stage<F8>(c, 2 * m + 3, wrap5(fa + 3));
      issue_stage<F8>(c, 2 * m + 4, wrap5(fa + 4));
      ring_barrier();
    }
    const int pa = wrap<F8>(sa + Ly::NST - 2), pb = 2 * m - 1 < c.nst ? wrap<F8>(sa + Ly::NST - 1) : pa;
    const lu8* va = m > 0 ? c.lds + pa * ST_BYTES : c.lds + Ly::QR_OFF;
    const lu8* vb = m > 0 ? c.lds + pb * ST_BYTES : c.lds + Ly::QR_OFF;
    const lu8* prd = c.lds + Ly::P_OFF + ((m - 1) & 1) * P_BYTES + c.pr_ofs;
    // copies of stages 2m+3, 2m+4 (none past the last step)
    StageCopy cx{nullptr, 0}, cy{nullptr, 0};
    if constexpr (!F8) {
      cx = plan_stage<F8>(c, 2 * m + 3, wrap<F8>(sa + 3));
      cy = plan_stage<F8>(c, 2 * m + 4, wrap<F8>(sa + 4));
    }
    f32x4 sc[2][2];
    if (m < c.nsteps) {
      const int sb = 2 * m + 1 < c.nst ? wrap<F8>(sa + 1) : sa;
      if ((c.nst - 1) >> 1 == m) zero_tail(c, (c.nst - 1) & 1 ? sb : sa);
      step_scores<F8>(c, c.lds + sa * ST_BYTES, c.lds + sb * ST_BYTES, qf, sc, cx, cy);
      const int nv = c.ntok - 2 * m * T;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        mask(c, sc[0][hb], nv);
        mask(c, sc[1][hb], nv - T);
      }
    } else {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) sc[0][hb] = sc[1][hb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    pv_weights_step<F8>(c, m, sc, va, vb, prd, o, m_ref, m_all, l_run, ovf);
    sa = wrap<F8>(sa + 2);
    if constexpr (F8) fa = wrap5(fa + 2);
  }
  return ovf;
}

// Normalised partial output of the item: O / l per head (bf16) and the
// per-head log2-sum-exp2 m_ref + log2(l).
template <bool F8>
__device__ __forceinline__ void write_out(const Ctx& c, const f32x16 (&o)[4][4], const float (&m_ref)[2],
                                          const float (&l_run)[2], bf16_t* opart, float* lpart, size_t prow0) {
  const int lane = c.lane, wave = c.wave;
  const int g = lane >> 4, hq = 32 * wave + (lane & 15);
  // per-head sums of the weights: the 4 token groups of a head are lanes i16 + 16g
  float* lsum = (float*)(c.lds + Lay<F8>::L_OFF);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    float l_tot = l_run[hb] + __shfl_xor(l_run[hb], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (g == 0) {
      lsum[hq + 16 * hb] = l_tot;
      lpart[prow0 + hq + 16 * hb] = m_ref[hb] + log2f(l_tot);
    }
  }
  __syncthreads();

  // The rows go out through LDS (the ring is free by now): row h at 1024 h,
  // 16-byte chunk C at 16 (C ^ h%16), so that the register-layout writes
  // spread over the banks and every global store writes one whole 1 KiB row.
  // O^T lane layout: head 32 hb + lane%32, channels 32 cb + 8 (r/4) + 4 (lane/32) + r%4
  const int n = lane & 31, cg = lane >> 5;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int h = 32 * hb + n;
    const float inv = 1.0f / lsum[h];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16_t)(o[i][hb][4 * r4 + e] * inv);
        const int C = 16 * wave + 4 * i + r4;
        *(__attribute__((address_space(3))) bf16x4*)(c.lds + 1024 * h + 16 * (C ^ (h & 15)) + 8 * cg) = v;
      }
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int k = 0; k < H / NW; ++k) {
    const int h = NW * k + wave;
    const bf16x8 v = *(lbf16x8*)(c.lds + 1024 * h + 16 * (lane ^ (h & 15)));
    *(bf16x8*)(opart + (prow0 + h) * DC + 8 * lane) = v;
  }
}

template <bool F8>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_attn_v3b(int s_q, int S, int pps, int P_items, const bf16_t* __restrict__ qt,
                const uint8_t* __restrict__ pages, size_t page_bytes, const int32_t* __restrict__ bt, int max_pages,
                const int32_t* __restrict__ seqlens, bf16_t* __restrict__ opart, float* __restrict__ lpart,
                int32_t* __restrict__ hdr, int batch) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lu8* lds = (lu8*)lds_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, in an SGPR
  if (blockIdx.x == 0 && threadIdx.x == 0) {  // the split plan, for the combine
    hdr[HDR_MAGIC] = WS_MAGIC; hdr[HDR_S] = S; hdr[HDR_PPS] = pps; hdr[HDR_BATCH] = batch;
    hdr[HDR_SQ] = s_q; hdr[HDR_H] = H; hdr[HDR_DC] = DC; hdr[HDR_PDT] = MLA_BF16;
  }
  // Blocks are dealt to the 8 XCDs round-robin (blockIdx % 8).  Work items
  // (b, s) are numbered so that each XCD takes a contiguous run: the splits
  // of one sequence then share that XCD's L2 (its query rows are fetched from
  // HBM once), and the s_q query rows of one item are dispatched together.
  const int RB = s_q;
  const int n_per = (P_items + 7) / 8;
  const int u = blockIdx.x / 8;
  const int p = (blockIdx.x % 8) * n_per + u / RB;
  const int j = u % RB;
  if (u / RB >= n_per || p >= P_items) return;
  const int b = p / S, s = p % S;

  const int g = lane >> 4, i16 = lane & 15;
  const int hq = 32 * wave + i16;  // head of this lane in head block 0 of the scores layout
  const bf16_t* qblk = qt + (size_t)(b * s_q + j) * H * DKV;
  const int32_t* bt_row = bt + (size_t)b * max_pages;
  const int p0 = s * pps;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  // Everything that needs only the block index goes out at once: the length
  // and the split's page ids side by side, then the query rows; the stage
  // copies follow as soon as the length and the page ids are in.
  const int L = seqlens[b];
  const int bt_lane = lane < pps && p0 + lane < max_pages ? bt_row[p0 + lane] : 0;
  // RoPE rows of all heads to LDS: row h at QR_OFF + 128h, its eight 16-byte
  // chunks permuted by (h/2)%8 (conflict-free B-operand reads).
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int i = wave + NW * n;
    const int pos = 64 * i + lane, h = pos >> 3, lc = (pos & 7) ^ ((h >> 1) & 7);
    dma_1k((const uint8_t*)qblk, (uint32_t)((h * DKV + DC + 8 * lc) * 2), lds_addr + Lay<F8>::QR_OFF + i * 1024);
  }
  // Absorbed query rows as B operands: lane holds qt[hq + 16 hb][32 ks + 8 g .. +8].
  bf16x8 qf[16][2];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) qf[ks][hb] = *(const bf16x8*)(qblk + (size_t)(hq + 16 * hb) * DKV + 32 * ks + 8 * g);

  int vis = L > 0 ? L - s_q + j + 1 : 0;
  vis = vis < 0 ? 0 : vis;
  Ctx c;
  c.t_begin = p0 * PAGE;
  const int t_end = min(vis, c.t_begin + pps * PAGE);
  c.ntok = t_end > c.t_begin ? t_end - c.t_begin : 0;
  c.nst = (c.ntok + T - 1) / T;
  c.nsteps = (c.nst + 1) / 2;

  const size_t item = ((size_t)b * S + s) * s_q + j;
  const size_t prow0 = item * H;  // partial row of head 0
  if (c.nst == 0) {  // an empty split: lse = -inf, which the merge skips without reading its rows
    if (threadIdx.x < H) lpart[prow0 + threadIdx.x] = -INFINITY;
    wait_vmcnt<0>();  // nothing in flight into LDS when the block leaves
    return;
  }

  c.pages = pages;
  c.page_bytes = page_bytes;
  c.bt_row = bt_row;
  c.p0 = p0;
  c.bt_lane = bt_lane;
  c.lds = lds;
  c.lds_addr = lds_addr;
  c.wave = wave;
  c.lane = lane;
  c.dma_ofs = (uint32_t)(g * 1024 + i16 * 16);
  c.dma_ofs_w = c.dma_ofs + 4096u * (uint32_t)wave;
  // the first three stages go out before anything waits
  issue_stage<F8>(c, 0, 0);
  issue_stage<F8>(c, 1, 1);
  issue_stage<F8>(c, 2, 2);
  wait_vmcnt<0>();  // the compiler's own loads are then known complete (and stages 0-2 have landed)

  // K fragment: token i16, chunk 4 ks + g (chunk % 4 = g)
  c.koff = (uint32_t)(256 * g + 16 * (i16 ^ slot_x(g)));
  // (head block 1, heads hq + 16, sits 16 rows further with the same permutation)
  c.qr_ofs0 = (uint32_t)(hq * 128 + 16 * ((0 + g) ^ ((hq >> 1) & 7)));
  c.qr_ofs1 = (uint32_t)(hq * 128 + 16 * ((4 + g) ^ ((hq >> 1) & 7)));
  {
    // V^T[32 ch][16 tokens] of channel block 4w (+1, +2, +3): chunk 4cb + cl,
    // lane group layout of the transposing read
    const int tq = i16 >> 2, qq = i16 & 3;
    const int cl = 2 * (g & 1) + (qq >> 1);
    c.vofs1 = (uint32_t)(4096 * wave + 256 * cl + 16 * ((4 * (g >> 1) + tq) ^ slot_x(cl)) + 8 * (qq & 1));
    c.vofs2 = (uint32_t)(4096 * wave + 256 * cl + 16 * ((8 + 4 * (g >> 1) + tq) ^ slot_x(cl)) + 8 * (qq & 1));
  }
  {
    // P row of head h (one per stage): 16 bf16 weights in token order 0-3,
    // 8-11, 4-7, 12-15 (the k order of the transposed V^T fragment), 16-byte
    // halves swapped when bit 3 of h is set.  Writer: tokens 4g..4g+3 of head
    // hq (head hq + 16 is 512 bytes further, same swap).
    const int pos = ((g & 1) << 1) | (g >> 1);
    c.pw_ofs = (uint32_t)(hq * 32 + 16 * ((pos >> 1) ^ ((hq >> 3) & 1)) + 8 * (pos & 1));
    const int n = lane & 31;  // reader: head 32 hb + n, half lane/32
    c.pr_ofs = (uint32_t)(n * 32 + 16 * ((lane >> 5) ^ ((n >> 3) & 1)));
  }

  f32x16 o[4][4];
  float m_ref[2] = {-INFINITY, -INFINITY}, m_all[2], l_run[2];
  // A second pass, against the exact maximum, only if a score outgrew the
  // first step's reference.  Both passes run the same code (a runtime loop,
  // nothing to specialise on), so the step code exists once.
#pragma clang loop unroll(disable)
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) o[i][hb] = f32x16{};
    m_all[0] = m_all[1] = -INFINITY;
    l_run[0] = l_run[1] = 0.0f;
    const bool ovf = run_pass<F8>(c, qf, m_ref, m_all, l_run, o);
    const bool again = __syncthreads_or(ovf);  // also: every wave is done with the ring
    if (pass > 0 || !again) break;
    m_ref[0] = m_all[0];
    m_ref[1] = m_all[1];
    issue_stage<F8>(c, 0, 0);
    issue_stage<F8>(c, 1, 1);
    issue_stage<F8>(c, 2, 2);
  }
  write_out<F8>(c, o, m_ref, l_run, opart, lpart, prow0);
}

}  // namespace

template <bool F8>
static hipError_t launch_attn(const DecodeArgs& a) {
  constexpr int lds = Lay<F8>::LDS_BYTES;
  static bool attr_set = false;  // one flag per instantiation
  if (!attr_set) {
    MLA_TRY(hipFuncSetAttribute((const void*)&k_attn_v3b<F8>, hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    attr_set = true;
  }
  const int P_items = a.batch * a.S;
  const int grid = ((P_items + 7) / 8) * 8 * a.s_q;
  return launch(&k_attn_v3b<F8>, dim3(grid), dim3(256), lds, a.stream, a.s_q, a.S, a.pages_per_split, P_items,
                (const bf16_t*)(a.ws + a.L.qt), a.pages, a.g.page_bytes, a.block_table, a.max_pages, a.seqlens,
                (bf16_t*)(a.ws + a.L.opart), (float*)(a.ws + a.L.lpart), (int32_t*)(a.ws + a.L.header), a.batch);
}

hipError_t fast_attention_b(const DecodeArgs& a) {
  if (a.cache_dtype == MLA_FP8_E4M3) {
    // the page geometry the fp8 stage copies are compiled for
    if (a.g.fp8_scale_off != (size_t)F8_PG_SCALES || a.g.fp8_rope_off != (size_t)F8_PG_ROPE) return hipErrorInvalidValue;
    return launch_attn<true>(a);
  }
  return launch_attn<false>(a);
}

}  // namespace mla

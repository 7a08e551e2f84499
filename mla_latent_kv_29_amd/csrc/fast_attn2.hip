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
//   * scores: wave w owns heads 32w..32w+31.  A step's S^T[32 tokens][32
//     heads] = K . Q^T is one chain of 36 v_mfma_f32_32x32x16_bf16 over the
//     576 channels (k-steps of 16): the K fragments (tokens of the step's
//     two 16-token stages) come from LDS, the wave's 512-wide absorbed query
//     rows sit in 128 VGPRs, the 64-wide RoPE rows of all heads in LDS.
//   * P.V: wave w owns latent channels 128w..128w+127 of all 128 heads.
//     O^T[128 ch][128 heads] += V^T . P^T with v_mfma_f32_32x32x16_bf16 into
//     all 256 AGPRs; V^T comes from the staged tokens with the transposing
//     ds_read_b64_tr_b16, P^T from an LDS buffer that every wave writes its
//     heads' weights to.
// Splitting P.V by channel means each wave reads only a quarter of V.  Step
// m scores stages 2m, 2m+1 and multiplies the weights of stages 2m-2, 2m-1
// by V between the same two barriers, so one barrier per 32 tokens
// publishes both the new stages and the previous weights; the last step's
// P.V runs on its own afterwards.  The P.V MFMAs are interleaved with the
// score chain and the softmax VALU work with the P.V MFMAs, so that the
// vector work issues while the matrix unit is busy.
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
// FP8 cache with power-of-two (UE8M0) scales, a format the lesson's
// continuation of §3.5 reports DeepSeek V3.1 moving to: here
// v_cvt_scalef32_pk_bf16_fp8, which applies only the exponent of its scale
// operand, widens codes exactly in one instruction per two values, so the
// step needs one barrier.  Each lane reads its K fragments from the fp8
// stage (8 code bytes, half the LDS bytes of a bf16 fragment) and widens
// them in registers one k-step ahead of their MFMA; V is still multiplied
// from bf16 images in LDS, which the block writes one step ahead, as eight
// small jobs between the score MFMAs.  On data that both formats store alike
// the two kernels give the same bits.
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
  uint32_t koff_e, koff_o;    // K fragment of the scores MFMA (even / odd k-step), inside its stage
  uint32_t k8base;            // power-of-two FP8 cache: lane part of its K codes (16 token + 8 half)
  int kst;                    // 1 if this lane's score rows are tokens of the step's second stage
  uint32_t qr_base;           // RoPE query fragments: row of the lane's head, its k-half
  int qr_key;                 // ... and the chunk-pair permutation of that row
  uint32_t vofs1, vofs2;      // V^T transposing reads (wave's first channel block)
  uint32_t pw_ofs, pr_ofs;    // P write (this wave's head block) / read (P.V layout)
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

// Score MFMA with a VGPR accumulator (see the file comment).  One
// v_mfma_f32_32x32x16_bf16 chain per step: dependent MFMAs that accumulate
// into exactly the same registers issue back to back (the hardware forwards
// the accumulator), and on gfx950 this shape runs at the full matrix rate,
// which the 16x16x32 shape does not reach from one wave.
__device__ __forceinline__ f32x16 mfma_s0(bf16x8 a, bf16x8 b) {
  f32x16 c;
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
  return c;
}
__device__ __forceinline__ f32x16 mfma_s(bf16x8 a, bf16x8 b, f32x16 c) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  return c;
}
// Last MFMA of the chain: 12 wait states before a VALU instruction may read
// the result (what the compiler itself inserts for this shape).
__device__ __forceinline__ f32x16 mfma_s_last(bf16x8 a, bf16x8 b, f32x16 c) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 3" : "+v"(c) : "v"(a), "v"(b));
  return c;
}
// Power-of-two FP8 cache: eight E4M3 codes (two dwords, channel order) times
// the tile's scale 2^e, as bf16.  v_cvt_scalef32_pk_bf16_fp8 applies only
// the exponent of its scale operand, which for these scales is the whole
// scale, so every result is exact.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x2 lu32x2;
__device__ __forceinline__ bf16x8 cvt8_pow2(unsigned w0, unsigned w1, float sc) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, sc, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, sc, true);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, sc, false);
  const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, sc, true);
  return bf16x8{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
}

// S^T[32 tokens][32 heads] of the step's two stages (rows 0-15: the first
// stage, 16-31: the second) = K . Q^T over the 576 channels: 36 k-steps of
// 16.  Lane l reads token l%32 of its stage, channels 16 ks + 8 (l/32) .. +7:
// one 16-byte chunk, 2 ks + l/32, at the chunk-major offset of its token.
// The K fragments of k-step ks+KD are read while k-step ks multiplies;
// sched_barrier keeps that order (the scheduler would otherwise sink each
// read to its use).  The RoPE query fragments (k-steps 32-35) come from LDS.
constexpr int KD = 4;
constexpr int KSTEPS = DKV / 16;  // 36
template <bool F8>
__device__ __forceinline__ bf16x8 rope_q(const Ctx& c, int r) {
  return *(lbf16x8*)(c.lds + c.qr_base + 32 * (r ^ c.qr_key));
}
__device__ __forceinline__ bf16x8 kfrag(const lu8* kb, const Ctx& c, int ks) {
  return *(lbf16x8*)(kb + (ks & 1 ? c.koff_o : c.koff_e) + 512 * ks);
}
// Lane layout of S^T: head 32w + lane%32, value i is row (token of the step)
// 8 (i/4) + 4 (lane/32) + i%4.  Masks tokens past the end of the split (nv
// may be <= 0: a padding step).
__device__ __forceinline__ void mask(const Ctx& c, f32x16& s, int nv) {
  if (nv < 2 * T) {
    const int hi = 4 * (c.lane >> 5);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (8 * (i >> 2) + hi + (i & 3) >= nv) s[i] = -INFINITY;
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

// Maximum over the lanes l and l^32 (the permlane32 swap leaves the two
// values of each pair in its two results).
__device__ __forceinline__ float max_x32(float m) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// One step of the pass, as one compile-time schedule of 68 MFMAs:
//   part 1: the 36-MFMA score chain of stages 2m, 2m+1, with the 16 P.V
//           MFMAs of stage 2m-2 (the previous step's first stage) slotted
//           after every second score MFMA from k-step 3 on;
//   part 2: the 16 P.V MFMAs of stage 2m-1 with the softmax of this step's
//           scores cut into 9 items between them (the VALU work issues
//           while each MFMA occupies the matrix unit).
// So the matrix unit always has independent work queued: the fill of one
// product's operand reads is covered by the other's MFMAs.  The weights go
// to P buffer m&1 (see the softmax items) for the next step's P.V.
//
// P.V: O^T[128 ch][128 heads] of this wave's channel blocks += V^T . P^T;
// MFMA t of a stage is channel block t%4 of head block t/4 (V^T fragment t%4
// of the stage, P^T fragment t/4).  The stage's four V^T fragments are read
// once per stage; the P^T fragments stream two ahead.
//
// The lane's 16 scores belong to head 32w + lane%32: values 0-7 are tokens
// of the first stage in exactly the order the P.V operand takes them (tokens
// 0-3, 8-11 on lanes 0-31; 4-7, 12-15 on lanes 32-63), values 8-15 those of
// the second stage.  So the weights leave as two 16-byte stores, at the
// place where the P.V read of head block w expects them.
struct Fused {
  const Ctx& c;
  int m;
  const lu8* kb;                 // K fragments: the lane's stage
  const bf16x8 (&qf)[32];
  bf16x8 f[KD];                  // K fragments in flight
  bf16x8 r[4];                   // RoPE query fragments (k-steps 32-35)
  f32x16 sc;
  const lu8 *va, *vb, *prd;      // previous step's two stages and P buffer
  bf16x8 v[4], p[4];             // V^T of the current P.V stage; P^T ring
  f32x16 (&o)[4][4];
  float& m_ref;
  float& m_all;
  float& l_run;
  bool& ovf;
  lu8* pw;
  const StageCopy &cx, &cy;
  float ml;
  float x[16];
  // power-of-two FP8 cache: the 4 tile scales of the lane's token, and the
  // converted K operands of the next k-steps (three: a conversion runs two
  // k-steps ahead and never rewrites the operand of the MFMA just issued)
  f32x4 ksc;
  bf16x8 cv[3];
  // ... and the V images of this step's stages, widened between the score
  // MFMAs: eight jobs (stage k/4, tile k%4) of one 8-channel chunk a thread
  const lu8* wsrc[2];            // fp8 stages (wave-uniform)
  lu8* wdst[2];                  // their bf16 V slots
  int wnv[2];                    // tokens of each stage to keep (the rest are zeroed)
  uint32_t wr_ofs, ww_ofs, ws_ofs;  // the thread's code, image and scale offsets
  int wt;                        // the thread's token
  u32x2 wcode;
  float wscl;
};

// E8 V-image job K (a constant): read the thread's 8 codes and their tile
// scale; two parts later, widen and store them (tokens past the split's end
// as zeros, so that whatever bytes the page holds there cannot turn a zero
// weight into NaN in P.V).  Thread: token tid%16, 8-channel chunk tid/16 + 16 j.
// Without a second stage, wsrc[1] is the first stage and wdst[1] a slot that
// nothing reads (the next P.V takes the first stage's image for both), so
// the jobs run unconditionally.
template <int K>
__device__ __forceinline__ void wload(Fused& F) {
  constexpr int st = K / 4, j = K % 4;
  F.wcode = *(lu32x2*)(F.wsrc[st] + F.wr_ofs + 2048 * j);
  F.wscl = *(__attribute__((address_space(3))) const float*)(F.wsrc[st] + F.ws_ofs + 4 * j);
}
template <int K>
__device__ __forceinline__ void wstore(Fused& F) {
  constexpr int st = K / 4, j = K % 4;
  const bf16x8 v = cvt8_pow2(F.wcode[0], F.wcode[1], F.wscl);
  *(__attribute__((address_space(3))) bf16x8*)(F.wdst[st] + F.ww_ofs + 4096 * j) = F.wt < F.wnv[st] ? v : bf16x8{};
}

// Power-of-two FP8 cache, k-step K (a constant): the lane's raw K fragment,
// read KD k-steps ahead from the fp8 stage.  Content k-steps: the 8 code
// bytes of 16-channel chunk K, half lane/32, in the low half (chunk K of
// token t at 256 K + 16 (t ^ x(K))); RoPE k-steps: 8 bf16 k^R channels, laid
// out like the bf16 stage's chunks.
template <int K>
__device__ __forceinline__ bf16x8 kraw_e8(const Fused& F) {
  const Ctx& c = F.c;
  if constexpr (K < 32) {
    const u32x2 w = *(lu32x2*)(F.kb + ((c.k8base ^ (uint32_t)(16 * slot_x(K))) + 256 * K));
    const u32x4 r = __builtin_shufflevector(w, w, 0, 1, -1, -1);
    return __builtin_bit_cast(bf16x8, r);
  } else {
    return *(lbf16x8*)(F.kb + F8_ROPE + ((K & 1) ? c.koff_o : c.koff_e) + 512 * (K - 32));
  }
}
// ... and its MFMA operand: content codes widened with the tile's scale (tile
// K/8), k^R as read.
template <int K>
__device__ __forceinline__ bf16x8 kop_e8(const Fused& F) {
  if constexpr (K < 32) {
    const u32x4 r = __builtin_bit_cast(u32x4, F.f[K % KD]);
    return cvt8_pow2(r[0], r[1], F.ksc[K / 8]);
  } else {
    return F.f[K % KD];
  }
}

__device__ __forceinline__ void read_v(Fused& F, const lu8* st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)(st + F.c.vofs1 + 1024 * i));
    const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)(st + F.c.vofs2 + 1024 * i));
    const short s8 __attribute__((ext_vector_type(8))) = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
    F.v[i] = __builtin_bit_cast(bf16x8, s8);
  }
}
__device__ __forceinline__ void read_p(Fused& F, int j, int hb) {
  F.p[hb] = *(lbf16x8*)(F.prd + j * P_STAGE + 1024 * hb);
}
// P.V MFMA t (0..15) of the current stage
template <int T_>
__device__ __forceinline__ void pv_mfma(Fused& F) {
  constexpr int hb = T_ >> 2, i = T_ & 3;
  F.o[i][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.v[i], F.p[hb], F.o[i][hb], 0, 0, 0);
}

// Part 1, k-step KS: score MFMA, K read KD ahead, and the P.V MFMA of stage
// 2m-2 that follows it (after k-steps 3, 5, .., 33); the P^T fragment of
// head block hb is read two P.V MFMAs before its first use.
template <bool F8, bool E8, int KS>
__device__ __forceinline__ void part1(Fused& F) {
  const Ctx& c = F.c;
  if constexpr (KS == 26) {
#pragma unroll
    for (int q = 0; q < 4; ++q) F.r[q] = rope_q<F8>(c, q);
  }
  if constexpr (E8) {
    // operand of k-step KS converted two parts earlier (a whole MFMA lies
    // between a conversion's VALU writes and the MFMA that reads them);
    // convert the one after next, then read the raw fragment KD k-steps
    // ahead into the slot just used
    const bf16x8 a = F.cv[KS % 3];
    const bf16x8 q = KS < 32 ? F.qf[KS] : F.r[KS - 32];
    if constexpr (KS == 0) F.sc = mfma_s0(a, q);
    else if constexpr (KS < KSTEPS - 1) F.sc = mfma_s(a, q, F.sc);
    else F.sc = mfma_s_last(a, q, F.sc);
    if constexpr (KS + 2 < KSTEPS) F.cv[(KS + 2) % 3] = kop_e8<KS + 2>(F);
    if constexpr (KS + KD < KSTEPS) F.f[KS % KD] = kraw_e8<KS + KD>(F);
  } else {
    const bf16x8 a = F.f[KS % KD];
    const bf16x8 q = KS < 32 ? F.qf[KS] : F.r[KS - 32];
    if constexpr (KS == 0) F.sc = mfma_s0(a, q);
    else if constexpr (KS < KSTEPS - 1) F.sc = mfma_s(a, q, F.sc);
    else F.sc = mfma_s_last(a, q, F.sc);
    if constexpr (KS + KD < KSTEPS) F.f[KS % KD] = kfrag(F.kb, c, KS + KD);
  }
  constexpr int t = (KS - 3) / 2;
  if constexpr (KS >= 3 && (KS - 3) % 2 == 0 && t < 16) {
    pv_mfma<t>(F);
    // P^T of head block hb+2, one MFMA into head block hb
    if constexpr ((t & 3) == 1 && t < 9) read_p(F, 0, (t >> 2) + 2);
    if constexpr (t == 15) read_v(F, F.vb);  // the second stage's V^T, for part 2
    if constexpr (t == 15) { read_p(F, 1, 0); read_p(F, 1, 1); }
  }
  // stage copies: the first at k-steps 1, 8, 15, 22, 29
  if constexpr (!F8) {
    if constexpr (KS % 7 == 1) copy_at(c, F.cx, KS / 7);
  }
  // E8 V images: job k read at k-step 1 + 4k, widened and stored at 3 + 4k
  if constexpr (E8) {
    if constexpr (KS % 4 == 1 && KS / 4 < 8) wload<KS / 4>(F);
    if constexpr (KS % 4 == 3 && KS / 4 < 8) wstore<KS / 4>(F);
  }
  __builtin_amdgcn_sched_barrier(0);
}
template <bool F8, bool E8, int... K>
__device__ __forceinline__ void part1_all(Fused& F, std::integer_sequence<int, K...>) {
  (part1<F8, E8, K>(F), ...);
}

// Part 2, P.V MFMA T of stage 2m-1 and the softmax item that follows it.
template <bool F8, int T_>
__device__ __forceinline__ void part2(Fused& F) {
  pv_mfma<T_>(F);
  if constexpr ((T_ & 3) == 1 && T_ < 9) read_p(F, 1, (T_ >> 2) + 2);
  // items at slots 0, 1, 2, 4, 6, 8, 10, 12, 14
  constexpr int item = T_ < 3 ? T_ : (T_ % 2 == 0 ? T_ / 2 + 1 : -1);
  if constexpr (item >= 0 && item < 9) {
    const f32x16& s = F.sc;
    if constexpr (item == 0) {
      F.ml = vmax(vmax3(s[0], s[1], s[2]), vmax3(s[3], s[4], vmax3(s[5], s[6], s[7])));
    } else if constexpr (item == 1) {
      F.ml = vmax3(F.ml, vmax3(s[8], s[9], s[10]), vmax3(s[11], s[12], vmax3(s[13], s[14], s[15])));
    } else if constexpr (item == 2) {
      F.ml = max_x32(F.ml);
      F.m_all = vmax(F.m_all, F.ml);
      // the reference: the first step's maximum, or the exact maximum
      // already in m_ref when the pass is redone (it is never smaller)
      if (F.m == 0) F.m_ref = vmax(F.m_ref, F.ml);
      F.ovf |= F.ml > F.m_ref + HEADROOM;
    } else if constexpr (item <= 6) {
      // raw v_exp_f32: results below 2^-126 flush to zero, harmless here; a
      // score above the headroom only occurs in a pass that is redone
      constexpr int q = item - 3;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) F.x[4 * q + rr] = __builtin_amdgcn_exp2f(s[4 * q + rr] - F.m_ref);
    } else {
      constexpr int h = item - 7;  // stage
      const float* x = F.x + 8 * h;
      F.l_run += ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
      bf16x8 pk;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) pk[rr] = (bf16_t)x[rr];
      *(__attribute__((address_space(3))) bf16x8*)(F.pw + h * P_STAGE) = pk;
    }
  }
  // the second stage copy: at P.V MFMAs 3, 6, 9, 12, 15
  if constexpr (!F8) {
    if constexpr (T_ % 3 == 0 && T_ > 0) copy_at(F.c, F.cy, T_ / 3 - 1);
  }
  __builtin_amdgcn_sched_barrier(0);
}
template <bool F8, int... K>
__device__ __forceinline__ void part2_all(Fused& F, std::integer_sequence<int, K...>) {
  (part2<F8, K>(F), ...);
}

// After the last step: the P.V of its two stages alone (32 MFMAs, no scores).
template <bool F8>
__device__ __forceinline__ void pv_tail(Fused& F) {
  read_v(F, F.va);
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) read_p(F, 0, hb);
  __builtin_amdgcn_sched_barrier(0);
  pv_mfma<0>(F); pv_mfma<1>(F); pv_mfma<2>(F); pv_mfma<3>(F);
  pv_mfma<4>(F); pv_mfma<5>(F); pv_mfma<6>(F); pv_mfma<7>(F);
  pv_mfma<8>(F); pv_mfma<9>(F); pv_mfma<10>(F); pv_mfma<11>(F);
  pv_mfma<12>(F); pv_mfma<13>(F); pv_mfma<14>(F); pv_mfma<15>(F);
  __builtin_amdgcn_sched_barrier(0);
  read_v(F, F.vb);
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) read_p(F, 1, hb);
  __builtin_amdgcn_sched_barrier(0);
  pv_mfma<0>(F); pv_mfma<1>(F); pv_mfma<2>(F); pv_mfma<3>(F);
  pv_mfma<4>(F); pv_mfma<5>(F); pv_mfma<6>(F); pv_mfma<7>(F);
  pv_mfma<8>(F); pv_mfma<9>(F); pv_mfma<10>(F); pv_mfma<11>(F);
  pv_mfma<12>(F); pv_mfma<13>(F); pv_mfma<14>(F); pv_mfma<15>(F);
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
// E8 (power-of-two FP8 cache) step m, with one barrier: the barrier
// publishes the fp8 stages 2m, 2m+1, the V images of 2m-2, 2m-1 (widened
// during step m-1) and the weights of step m-1; the block then issues the
// copies of 2m+3, 2m+4, widens the V images of 2m, 2m+1 (for step m+1),
// scores 2m, 2m+1 with K read from the fp8 stages and widened in registers,
// and multiplies the weights of 2m-2, 2m-1 with their V images; the V-image
// jobs of 2m, 2m+1 run between the score MFMAs (wload / wstore).
template <bool F8, bool E8>
__device__ __forceinline__ bool run_pass(const Ctx& c, const bf16x8 (&qf)[32], float& m_ref, float& m_all,
                                         float& l_run, f32x16 (&o)[4][4]) {
  static_assert(!E8 || F8, "the power-of-two format is an FP8 cache");
  using Ly = Lay<F8>;
  zero_p1<F8>(c);
  bool ovf = false;
  int sa = 0;  // slot of stage 2m
  int fa = 0;  // fp8: fp8-ring slot of stage 2m
  for (int m = 0; m < c.nsteps; ++m) {
    wait_step<F8>(c, m);
    ring_barrier();
    if constexpr (E8) {
      issue_stage<F8>(c, 2 * m + 3, wrap5(fa + 3));
      issue_stage<F8>(c, 2 * m + 4, wrap5(fa + 4));
    } else if constexpr (F8) {
      // this step's two stages into the bf16 slots freed by the last P.V
      widen_stage(c, fa, sa);
      if (2 * m + 1 < c.nst) widen_stage(c, wrap5(fa + 1), wrap<F8>(sa + 1));
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
    const int sb = 2 * m + 1 < c.nst ? wrap<F8>(sa + 1) : sa;
    if (!E8 && (c.nst - 1) >> 1 == m) zero_tail(c, (c.nst - 1) & 1 ? sb : sa);  // E8: wstore zeroes
    const lu8* stA = c.lds + sa * ST_BYTES;
    const lu8* stB = c.lds + sb * ST_BYTES;
    // K source: the lane's bf16 stage, or (E8) its fp8 stage
    const int fb = 2 * m + 1 < c.nst ? wrap5(fa + 1) : fa;
    const lu8* kb = E8 ? c.lds + Ly::F8_OFF + (c.kst ? fb : fa) * F8_ST : (c.kst ? stB : stA);
    Fused F{c, m, kb, qf, {}, {}, {}, va, vb, prd, {}, {}, o, m_ref, m_all, l_run, ovf,
            c.lds + Ly::P_OFF + (m & 1) * P_BYTES + c.pw_ofs, cx, cy, 0.0f, {}};
    if constexpr (E8) {
      static_assert(KD == 4, "E8 prologue");
      F.f[0] = kraw_e8<0>(F);
      F.f[1] = kraw_e8<1>(F);
      F.f[2] = kraw_e8<2>(F);
      F.f[3] = kraw_e8<3>(F);
      F.ksc = *(__attribute__((address_space(3))) const f32x4*)(kb + F8_SCALES + 16 * (c.lane & 15));
      F.cv[0] = kop_e8<0>(F);
      F.cv[1] = kop_e8<1>(F);
      // the V images of stages 2m, 2m+1 (for step m+1) go to the bf16 slots of
      // 2m-4, 2m-3, multiplied last step
      const int nv_last = c.ntok - (c.nst - 1) * T;
      const int tid = c.wave * 64 + c.lane, cq = tid >> 4;
      F.wt = tid & 15;
      F.wr_ofs = (uint32_t)(256 * (cq >> 1) + 16 * (F.wt ^ slot_x(cq >> 1)) + 8 * (cq & 1));
      F.ww_ofs = (uint32_t)(256 * cq + 16 * (F.wt ^ slot_x(cq)));
      F.ws_ofs = (uint32_t)(F8_SCALES + 16 * F.wt);
      F.wsrc[0] = c.lds + Ly::F8_OFF + fa * F8_ST;
      F.wsrc[1] = c.lds + Ly::F8_OFF + fb * F8_ST;
      F.wdst[0] = c.lds + sa * ST_BYTES;
      F.wdst[1] = c.lds + wrap<F8>(sa + 1) * ST_BYTES;
      F.wnv[0] = 2 * m == c.nst - 1 ? nv_last : T;
      F.wnv[1] = 2 * m + 1 == c.nst - 1 ? nv_last : T;
    } else {
#pragma unroll
      for (int d = 0; d < KD; ++d) F.f[d] = kfrag(F.kb, c, d);
    }
    read_v(F, va);
    read_p(F, 0, 0);
    read_p(F, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
    part1_all<F8, E8>(F, std::make_integer_sequence<int, KSTEPS>{});
    mask(c, F.sc, c.ntok - 2 * m * T);
    part2_all<F8>(F, std::make_integer_sequence<int, 16>{});
    sa = wrap<F8>(sa + 2);
    if constexpr (F8) fa = wrap5(fa + 2);
  }
  // the P.V of the last step's stages, once every wave has written its weights
  ring_barrier();
  {
    const int m = c.nsteps;
    const int pa = wrap<F8>(sa + Ly::NST - 2), pb = 2 * m - 1 < c.nst ? wrap<F8>(sa + Ly::NST - 1) : pa;
    const StageCopy none{nullptr, 0};
    Fused F{c, m, c.lds, qf, {}, {}, {}, c.lds + pa * ST_BYTES, c.lds + pb * ST_BYTES,
            c.lds + Ly::P_OFF + ((m - 1) & 1) * P_BYTES + c.pr_ofs, {}, {}, o, m_ref, m_all, l_run, ovf,
            c.lds, none, none, 0.0f, {}};
    pv_tail<F8>(F);
  }
  return ovf;
}

// Normalised partial output of the item: O / l per head (bf16) and the
// per-head log2-sum-exp2 m_ref + log2(l).
template <bool F8>
__device__ __forceinline__ void write_out(const Ctx& c, const f32x16 (&o)[4][4], float m_ref, float l_run,
                                          bf16_t* opart, float* lpart, size_t prow0) {
  const int lane = c.lane, wave = c.wave;
  const int hq = 32 * wave + (lane & 31);
  // per-head sums of the weights: the two token halves of a head are lanes l, l^32
  float* lsum = (float*)(c.lds + Lay<F8>::L_OFF);
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (lane < 32) {
    lsum[hq] = l_tot;
    lpart[prow0 + hq] = m_ref + log2f(l_tot);
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

template <bool F8, bool E8>
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

  const int g = lane >> 4, i16 = lane & 15, hi = lane >> 5;
  const int hq = 32 * wave + (lane & 31);  // head of this lane in the scores layout
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
  // Absorbed query rows as B operands of the score MFMAs: lane holds
  // qt[hq][16 ks + 8 (lane/32) .. +8] for the 32 k-steps of the latent part.
  bf16x8 qf[32];
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) qf[ks] = *(const bf16x8*)(qblk + (size_t)hq * DKV + 16 * ks + 8 * hi);

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

  // K fragment of k-step ks: token i16 of the stage chosen by lane bit 4,
  // chunk 2 ks + lane/32, i.e. chunk % 4 = lane/32 (even ks) or 2 + lane/32
  // (odd ks); the k-step adds 512 ks.
  c.kst = (lane >> 4) & 1;
  c.koff_e = (uint32_t)(256 * hi + 16 * (i16 ^ slot_x(hi)));
  c.koff_o = (uint32_t)(256 * hi + 16 * (i16 ^ slot_x(2 + hi)));
  c.k8base = (uint32_t)(16 * i16 + 8 * hi);
  // RoPE query fragment r (k-step 32 + r): chunk 2r + lane/32 of row hq,
  // stored at 16 (chunk ^ key), key = (hq/2) % 8
  {
    const int key = (hq >> 1) & 7;
    c.qr_base = (uint32_t)(Lay<F8>::QR_OFF + hq * 128 + 16 * (hi ^ (key & 1)));
    c.qr_key = key >> 1;
  }
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
    // halves swapped when bit 3 of h is set.  Reader: head 32 hb + n, half
    // lane/32.  Writer: the same lane pattern in this wave's head block.
    const int n = lane & 31;
    c.pr_ofs = (uint32_t)(n * 32 + 16 * ((lane >> 5) ^ ((n >> 3) & 1)));
    c.pw_ofs = c.pr_ofs + 1024u * (uint32_t)wave;
  }

  f32x16 o[4][4];
  float m_ref = -INFINITY, m_all, l_run;
  // A second pass, against the exact maximum, only if a score outgrew the
  // first step's reference.  Both passes run the same code (a runtime loop,
  // nothing to specialise on), so the step code exists once.
#pragma clang loop unroll(disable)
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) o[i][hb] = f32x16{};
    m_all = -INFINITY;
    l_run = 0.0f;
    const bool ovf = run_pass<F8, E8>(c, qf, m_ref, m_all, l_run, o);
    const bool again = __syncthreads_or(ovf);  // also: every wave is done with the ring
    if (pass > 0 || !again) break;
    m_ref = m_all;
    issue_stage<F8>(c, 0, 0);
    issue_stage<F8>(c, 1, 1);
    issue_stage<F8>(c, 2, 2);
  }
  write_out<F8>(c, o, m_ref, l_run, opart, lpart, prow0);
}

}  // namespace

template <bool F8, bool E8 = false>
static hipError_t launch_attn(const DecodeArgs& a) {
  constexpr int lds = Lay<F8>::LDS_BYTES;
  MLA_TRY(lds_limit((const void*)&k_attn_v3b<F8, E8>, lds));
  const int P_items = a.batch * a.S;
  const int grid = ((P_items + 7) / 8) * 8 * a.s_q;
  return launch(&k_attn_v3b<F8, E8>, dim3(grid), dim3(256), lds, a.stream, a.s_q, a.S, a.pages_per_split, P_items,
                (const bf16_t*)(a.ws + a.L.qt), a.pages, a.g.page_bytes, a.block_table, a.max_pages, a.seqlens,
                (bf16_t*)(a.ws + a.L.opart), (float*)(a.ws + a.L.lpart), (int32_t*)(a.ws + a.L.header), a.batch);
}

hipError_t fast_attention(const DecodeArgs& a) {
  if (is_fp8_cache(a.cache_dtype)) {
    // the page geometry the fp8 stage copies are compiled for
    if (a.g.fp8_scale_off != (size_t)F8_PG_SCALES || a.g.fp8_rope_off != (size_t)F8_PG_ROPE) return hipErrorInvalidValue;
    return a.cache_dtype == MLA_FP8_E4M3_E8 ? launch_attn<true, true>(a) : launch_attn<true>(a);
  }
  return launch_attn<false>(a);
}

}  // namespace mla

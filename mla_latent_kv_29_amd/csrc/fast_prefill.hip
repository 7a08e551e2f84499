// Causal MLA prefill attention on MFMA for the DeepSeek-V3 shape (gfx950).
//
// What it computes (DeepSeek-V3 reading lesson, §2.1.1, in the non-absorbed
// form: per head i an explicit key k_{t,i} = [k^C_{t,i} ; k^R_t] with
// k^C = W^UK c^KV and the shared RoPE key k^R, value v^C = W^UV c^KV; the
// scaled softmax of q_{j,i} . k_{t,i} over the tokens t <= j of the same
// sequence): for every token j of every packed sequence and every head i,
//     o_{j,i} = sum_{t<=j} p_t v^C_{t,i},  p = softmax_t(tau q_{j,i} . k_{t,i}),
// and lse_{j,i} (natural log).  q arrives pre-scaled by tau log2(e), so the
// softmax runs in the exp2 domain.
//
// Work item = (sequence, head, tile of 64 query rows); four waves of 16 rows.
// Per 64-key tile (keys up to the tile's last query):
//   S^T[16 keys][16 queries] blocks = K . Q^T with v_mfma_f32_16x16x32_bf16:
//     K fragments from LDS (192-wide rows: k^C of the head, then k^R), the
//     wave's Q^T fragments in 24 VGPRs for the whole kernel.
//   Online softmax (running row maximum m and sum l): a lane holds four keys
//     of one query per 16-key block, so the row maximum needs two lane swaps;
//     O is rescaled by 2^(m_old - m_new) when the maximum moves.
//   O^T[16 channels][16 queries] += V^T . P^T: P^T is the S^T register
//     layout itself (keys 4g..4g+3 of two 16-key blocks make a lane's eight
//     k-slots), and the transposing LDS read delivers V^T in the same key
//     order, so P never leaves the registers.
// K and V tiles stream HBM/L2 -> LDS with global_load_lds into two 40 KiB
// buffers (one tile in flight while the other is multiplied); at 80 KiB a
// block, two blocks share a CU, i.e. two waves per SIMD.  The LDS layouts
// (16-byte chunk q of row r at slot q ^ f(r)) make the K fragment reads and
// the transposing V reads bank-conflict free.
#include "internal.hpp"

namespace mla {
namespace {

constexpr int PH = 128, PDH = 128, PDR = 64, PDQK = PDH + PDR;  // heads, d_head (= d_v), d_rope, q.k width
constexpr int BQ = 64, BKT = 64;                                 // query rows per block, keys per tile
constexpr int KC_BYTES = BKT * PDH * 2;                          // 16 KiB
constexpr int KR_BYTES = BKT * PDR * 2;                          // 8 KiB
constexpr int V_BYTES = BKT * PDH * 2;                           // 16 KiB
constexpr int STAGE = KC_BYTES + KR_BYTES + V_BYTES;             // 40 KiB
constexpr int PA_LDS = 2 * STAGE;                                // 80 KiB
constexpr int COPIES = STAGE / 1024;                             // 40 wave-instructions per tile
static_assert(COPIES == 40, "ten copies per wave");

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
// V rows (256 B).
__device__ __forceinline__ int kc_slot(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int kr_slot(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ int v_swz(int r) { return 2 * (r & 3) + 8 * ((r >> 2) & 1); }

struct PaArgs {
  const bf16_t* q;   // [H][n_tok][192], pre-scaled by tau log2(e)
  const bf16_t* kc;  // [H][n_tok][128]
  const bf16_t* vc;  // [H][n_tok][128]
  const bf16_t* kr;  // [n_tok][64]
  const int32_t* cu; // [n_seq + 1]
  int n_tok, qtiles;
  bf16_t* out;       // [n_tok][H][128]
  float* lse;        // [n_tok][H] or null
};

// Tile kt (keys 64 kt .. +63 of the sequence, clamped to its last token) into
// stage buffer `buf`: wave w issues copies w, w+4, ..., w+36 of the 40
// (0-15 k^C rows, 16-23 k^R rows, 24-39 V rows).
__device__ __forceinline__ void issue_tile(const bf16_t* kc_h, const bf16_t* vc_h, const bf16_t* kr, int start,
                                           int len, int kt, uint32_t buf, int wave, int lane) {
  const int k0 = kt * BKT;
#pragma unroll
  for (int n = 0; n < 10; ++n) {
    const int j = wave + 4 * n;  // wave-uniform
    if (j < 16) {
      const int r = 4 * j + (lane >> 4), c = kc_slot(r, lane & 15);
      const int key = min(k0 + r, len - 1);
      pa_dma(kc_h, (uint32_t)(((start + key) * PDH + 8 * c) * 2), buf + 1024 * j);
    } else if (j < 24) {
      const int jj = j - 16, r = 8 * jj + (lane >> 3), c = kr_slot(r, lane & 7);
      const int key = min(k0 + r, len - 1);
      pa_dma(kr, (uint32_t)(((start + key) * PDR + 8 * c) * 2), buf + KC_BYTES + 1024 * jj);
    } else {
      const int jj = j - 24, r = 4 * jj + (lane >> 4), c = (lane & 15) ^ v_swz(r);
      const int key = min(k0 + r, len - 1);
      pa_dma(vc_h, (uint32_t)(((start + key) * PDH + 8 * c) * 2), buf + KC_BYTES + KR_BYTES + 1024 * jj);
    }
  }
}

__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__global__ __launch_bounds__(256, 2) void k_prefill_attn(PaArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lu8* lds = (lu8*)lds_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, i16 = lane & 15;
  const int b = blockIdx.y, h = blockIdx.z;
  const int start = a.cu[b], len = a.cu[b + 1] - start;
  const int qt = a.qtiles - 1 - (int)blockIdx.x;  // the longest (last) query tiles first
  const int q0 = qt * BQ;
  if (q0 >= len) return;
  const int ntiles = qt + 1;  // causal: keys 0 .. q0 + 63
  const bf16_t* kc_h = a.kc + (size_t)h * a.n_tok * PDH;
  const bf16_t* vc_h = a.vc + (size_t)h * a.n_tok * PDH;
  const uint32_t ring = (uint32_t)(uintptr_t)lds;

  // Q^T fragments (B operand): query row q0 + 16 wave + i16 (clamped: rows
  // past the sequence are computed and never stored), k = 32 ks + 8 g.
  const int qrow = q0 + 16 * wave + i16;
  bf16x8 qf[6];
  {
    const bf16_t* qp = a.q + ((size_t)h * a.n_tok + start + min(qrow, len - 1)) * PDQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) qf[ks] = *(const bf16x8*)(qp + 32 * ks);
  }
  wait_vmcnt<0>();  // the compiler's loads are done before the copies go out
  issue_tile(kc_h, vc_h, a.kr, start, len, 0, ring, wave, lane);
  if (ntiles > 1) issue_tile(kc_h, vc_h, a.kr, start, len, 1, ring + STAGE, wave, lane);

  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{};
  float m = -INFINITY, l = 0.0f;  // running maximum (all of the lane's row) and this lane's partial sum
  // V^T transposing reads: lane (e, qq) of group g addresses key row 4g + e
  // (+16 for the second read), channels 16 db + 4 qq .. +3
  const int e = i16 >> 2, qq = i16 & 3;

  for (int kt = 0; kt < ntiles; ++kt) {
    if (kt == 0 && ntiles > 1) wait_vmcnt<10>();  // tile 1 may stay in flight
    else wait_vmcnt<0>();
    ring_barrier();  // tile kt is in; every wave is done with tile kt-1, whose buffer takes tile kt+1
    if (kt >= 1 && kt + 1 < ntiles) issue_tile(kc_h, vc_h, a.kr, start, len, kt + 1, ring + ((kt + 1) & 1) * STAGE, wave, lane);
    const lu8* st = lds + (kt & 1) * STAGE;

    // S^T blocks: keys 16 nb + 4g + r of this lane's query i16
    f32x4 s[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int r = 16 * nb + i16;
      f32x4 acc = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) {
        const lu8* p = ks < 4 ? st + r * 256 + 16 * kc_slot(r, 4 * ks + g)
                              : st + KC_BYTES + r * 128 + 16 * kr_slot(r, 4 * (ks - 4) + g);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const lbf16x8*)p, qf[ks], acc, 0, 0, 0);
      }
      s[nb] = acc;
    }
    if (kt == qt) {  // the diagonal tile: keys after the query are masked
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (q0 + 16 * nb + 4 * g + r > qrow) s[nb][r] = -INFINITY;
    }
    // online softmax
    float mt = vmax3(vmax3(s[0][0], s[0][1], s[0][2]), vmax3(s[0][3], s[1][0], s[1][1]), vmax3(s[1][2], s[1][3], s[2][0]));
    mt = vmax3(mt, vmax3(s[2][1], s[2][2], s[2][3]), vmax3(s[3][0], s[3][1], vmax3(s[3][2], s[3][3], s[3][3])));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m, mt);  // finite: every query sees key 0 in tile 0
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    float ls = 0.0f;
    bf16x8 pb[2];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[nb][r] - mn);
        ls += p;
        pb[nb >> 1][4 * (nb & 1) + r] = (bf16_t)p;
      }
    l = l * alpha + ls;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] *= alpha;
    // O^T += V^T P^T: k-step kk covers keys 32 kk .. +31 in the order of the
    // S^T registers (keys 32kk + 4g + 0..3, then 32kk + 16 + 4g + 0..3)
    const lu8* vt = st + KC_BYTES + KR_BYTES;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int r1 = 32 * kk + 4 * g + e, r2 = r1 + 16;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int c = 2 * db + (qq >> 1), half = qq & 1;
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)(vt + r1 * 256 + 16 * (c ^ v_swz(r1)) + 8 * half));
        const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4*)(vt + r2 * 256 + 16 * (c ^ v_swz(r2)) + 8 * half));
        const short s8 __attribute__((ext_vector_type(8))) = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, s8), pb[kk], o[db], 0, 0, 0);
      }
    }
  }
  wait_vmcnt<0>();  // nothing in flight into LDS when the block leaves

  // O^T lane layout: channels 16 db + 4 g + r of query i16; the row's sum is
  // spread over the four lanes i16 + 16 g'
  float lt = l + __shfl_xor(l, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (qrow < len) {
    const float inv = 1.0f / lt;
    bf16_t* op = a.out + ((size_t)(start + qrow) * PH + h) * PDH + 4 * g;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (bf16_t)(o[db][r] * inv);
      *(bf16x4*)(op + 16 * db) = v;
    }
    if (a.lse && g == 0) a.lse[(size_t)(start + qrow) * PH + h] = (m + __log2f(lt)) * 0.6931471805599453f;
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
            (const bf16_t*)(a.ws + a.L.kr), a.cu_seqlens, a.n_tok, qtiles, a.out, a.lse_out};
  static bool attr_set = false;
  if (!attr_set) {
    MLA_TRY(hipFuncSetAttribute((const void*)&k_prefill_attn, hipFuncAttributeMaxDynamicSharedMemorySize, PA_LDS));
    attr_set = true;
  }
  return launch(&k_prefill_attn, dim3(qtiles, a.n_seq, PH), dim3(256), PA_LDS, a.stream, pa);
}

hipError_t fast_prefill(const PrefillArgs& a) {
  MLA_TRY(prefill_projections(a));
  return prefill_attention(a);
}

}  // namespace mla

// Host-side plumbing shared by the API layer and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include "common.hpp"

namespace mla {

// Workspace layout of one decode step (every region 256-byte aligned).
//   header   : int32[64] plan written by mla_decode, read by mla_combine
//   cq_part  : f32 [KSPLIT_MAX][R][d_cq]   split-K partials of c^Q = W^DQ h
//   cq       : act [R][d_cq]               c^Q
//   u        : f32 [R][H][d_head+d_rope]   W^UQ c^Q (bf16 q^C for the MFMA path)
//   qt       : act [R][H][d_c+d_rope]      absorbed, scaled query [q_abs | q^R]
//   olat     : act [R][H][d_c]             merged latent rows (the combine's own
//                                          scratch when it merges before W^UV)
//   lpart    : f32 [B][S][s_q][H]          per-split log2-sum-exp2 of scores
//   opart    : f32 or bf16 [B][S][s_q][H][d_c]  per-split normalised latent outputs
//                                        (sized for f32; element type in the header)
// R = batch * s_q.  Everything up to lpart is independent of the split count
// S; opart follows lpart, so a kernel that reads S from the header finds it
// with opart_offset().
constexpr int KSPLIT_MAX = 16;
constexpr int MAX_SPLITS = 4096;
constexpr int WS_HEADER_INTS = 64;
constexpr int32_t WS_MAGIC = 0x4d4c4144;  // "MLAD"

struct WsLayout {
  size_t header, cq_part, cq, u, qt, olat, opart, lpart, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline size_t opart_offset(size_t lpart_off, int batch, int S, int s_q, int H) {
  return lpart_off + align256((size_t)batch * S * s_q * H * 4);
}

inline WsLayout ws_layout(const mla_dims& d, int act, int batch, int s_q, int S) {
  const size_t R = (size_t)batch * s_q, H = d.n_heads;
  const size_t es = act == MLA_F32 ? 4 : 2;
  WsLayout w;
  size_t o = 0;
  w.header = o;  o = align256(o + WS_HEADER_INTS * 4);
  w.cq_part = o; o = align256(o + (size_t)KSPLIT_MAX * R * d.d_cq * 4);
  w.cq = o;      o = align256(o + R * d.d_cq * es);
  w.u = o;       o = align256(o + R * H * (d.d_head + d.d_rope) * 4);
  w.qt = o;      o = align256(o + R * H * (d.d_c + d.d_rope) * es);
  w.olat = o;    o = align256(o + R * H * d.d_c * es);
  w.lpart = o;   o = align256(o + (size_t)batch * S * s_q * H * 4);
  w.opart = o;   o = align256(o + (size_t)batch * S * s_q * H * d.d_c * 4);
  w.total = o;
  return w;
}

// Header fields (int32 indices).
enum { HDR_MAGIC = 0, HDR_S = 1, HDR_PPS = 2, HDR_BATCH = 3, HDR_SQ = 4, HDR_H = 5, HDR_DC = 6, HDR_PDT = 7 };
// HDR_PDT: element type of opart, MLA_F32 or MLA_BF16 (the MFMA attention writes bf16)

struct DecodeArgs {
  mla_dims d;
  int act, cache_dtype;
  const void* hq;
  int batch, s_q;
  const void *W_DQ, *W_UQ, *W_UK;
  const uint8_t* pages;
  CacheGeom g;
  const int32_t* block_table;
  int max_pages;
  const int32_t* seqlens;
  float scale;           // softmax scale tau
  int S, pages_per_split;
  uint8_t* ws;
  WsLayout L;
  hipStream_t stream;
};

struct CombineArgs {
  mla_dims d;
  int act;
  int batch, s_q;
  int S;  // split count of the decode that filled ws (validated against ws_bytes on the host)
  uint8_t* ws;
  WsLayout L;
  const void* W_UV;
  void* out;
  float* lse_out;
  hipStream_t stream;
};

struct AppendArgs {
  mla_dims d;
  int act;
  const void* h;        // append: hidden states; write: c_kv
  const void* k_rope;   // write only
  int n_tok;
  const int32_t *seq_id, *pos;
  const void *W_DKV, *W_KR;
  uint8_t* pages;
  CacheGeom g;
  const int32_t* block_table;
  int max_pages;
  hipStream_t stream;
};

// Prefill workspace (every region 256-byte aligned), n = n_tok:
//   pos : int32 [n]                token position within its sequence
//   ckv : bf16  [n][d_c]           c^KV = W^DKV h
//   kr  : bf16  [n][d_rope]        k^R = RoPE(W^KR h)
//   cq  : bf16  [n][d_cq]          c^Q = W^DQ h
//   q   : bf16  [H][n][d_head + d_rope]  [q^C ; RoPE(q^R)] * tau * log2(e)
//   kc  : bf16  [H][n][d_head]     k^C = W^UK c^KV (explicit, per head)
//   vc  : bf16  [H][n][d_head]     v^C = W^UV c^KV
struct PrefillLayout {
  size_t freq, pos, rope, ckv, kr, cq, q, kc, vc, total;
};

inline PrefillLayout prefill_layout(const mla_dims& d, int n_tok) {
  const size_t n = (size_t)n_tok, H = d.n_heads;
  PrefillLayout w;
  size_t o = 0;
  w.freq = o; o = align256(o + 32 * 8);  // RoPE frequencies (double)
  w.pos = o; o = align256(o + n * 4);
  w.rope = o; o = align256(o + n * (d.d_rope / 2) * 8);  // (cos, sin) per token and RoPE pair
  w.ckv = o; o = align256(o + n * d.d_c * 2);
  w.kr = o;  o = align256(o + n * d.d_rope * 2);
  w.cq = o;  o = align256(o + n * d.d_cq * 2);
  w.q = o;   o = align256(o + H * n * (d.d_head + d.d_rope) * 2);
  w.kc = o;  o = align256(o + H * n * d.d_head * 2);
  w.vc = o;  o = align256(o + H * n * d.d_head * 2);
  w.total = o;
  return w;
}

struct PrefillArgs {
  mla_dims d;
  const bf16_t* h;  // [n_tok][d_model]
  int n_tok, n_seq, max_seqlen;
  const int32_t* cu_seqlens;  // [n_seq + 1]
  const bf16_t *W_DQ, *W_UQ, *W_UK, *W_UV, *W_DKV, *W_KR;
  float scale;                // softmax scale tau
  bf16_t* out;                // [n_tok][H][d_head]
  float* lse_out;             // [n_tok][H] or null
  uint8_t* ws;
  PrefillLayout L;
  hipStream_t stream;
};

// Output projection y = W^O [o_1; ...; o_H] for `rows` rows.
struct OutProjArgs {
  int rows, N, K;  // N = d_model, K = H * d_head
  int act;         // MLA_F32 or MLA_BF16 (o, W_O and y)
  const void* o;   // [rows][K]
  const void* W_O; // [N][K]
  void* y;         // [rows][N]
  uint8_t* ws;     // fp32 partials (out_proj_ws_bytes)
  hipStream_t stream;
};
// Plan of the bf16 MFMA path: k-groups of the skinny kernel (rows <= 64) or
// K splits of the general GEMM; 0 when the shape takes the generic path.
int out_proj_splits(int act, int rows, int N, int K);
size_t out_proj_ws_bytes(int act, int rows, int N, int K);

// The decode step without a caller workspace (noalloc.hip): the workspace of
// the MFMA path inside the library's static per-device array.
WsLayout noalloc_layout(const mla_dims& d, int batch, int s_q, int S);
hipError_t noalloc_decode_step(DecodeArgs& a, CombineArgs& c);

// Streaming read of `bytes` (a multiple of 16) from src (probe.hip).
hipError_t read_probe(const void* src, size_t bytes, int* sink, hipStream_t st);
hipError_t mfma_probe(const void* ops, int iters, float* sink, hipStream_t st);  // ops: 12 x 64 bf16x8
double mfma_probe_flops(int iters);
hipError_t check_metadata(int batch, int max_pages, int page_size, int num_pages, const int32_t* bt,
                          const int32_t* seqlens, int32_t* bad, hipStream_t st);

// Raises the dynamic LDS limit of `kernel` to `bytes` on the current device,
// once per (kernel, device); safe to call from several threads.
hipError_t lds_limit(const void* kernel, int bytes);

// Launchers (return the first HIP error of the enqueue, hipSuccess otherwise).
hipError_t generic_append(const AppendArgs& a);
hipError_t generic_write(const AppendArgs& a);
hipError_t generic_query(const DecodeArgs& a);       // header, c^Q, W^UQ, RoPE, absorption -> qt
hipError_t generic_attention(const DecodeArgs& a);   // qt + cache -> per-split partials
hipError_t generic_combine(const CombineArgs& a);
hipError_t write_header(const DecodeArgs& a);

bool fast_append_supported(const mla_dims& d, int act, int cache_dtype);
bool fast_append_shape(const mla_dims& d);
bool fast_decode_supported(const mla_dims& d, int act, int cache_dtype, int s_q);
hipError_t fast_append(const AppendArgs& a);
// decode-step append with a workspace (at most 64 tokens, V3 head shape):
// k-group partials of the latent rows (k_skinny), then their sum, RoPE,
// conversion and page scatter (k_append_reduce)
bool skinny_append_supported(const mla_dims& d, int n_tok);
int skinny_append_kgroups(const mla_dims& d);
hipError_t skinny_append_partials(const AppendArgs& a, float* part);
hipError_t append_reduce(const AppendArgs& a, const float* part, int kgroups);
hipError_t fast_combine(const CombineArgs& a);
hipError_t fast_attention(const DecodeArgs& a);
hipError_t fast_query(const DecodeArgs& a);
bool skinny_query_supported(const mla_dims& d, int R);
hipError_t skinny_query(const DecodeArgs& a);
bool merge_uv_supported(const mla_dims& d, int R, int S);
hipError_t merge_uv(const CombineArgs& a);
// W^UQ + RoPE + W^UK absorption for more than 64 rows (V3 shape), from c^Q
bool rows_query_supported(const mla_dims& d, int R);
hipError_t rows_query(const DecodeArgs& a, const bf16_t* cq);
hipError_t merge_uv_f8(const CombineArgs& a, const uint8_t* uv_c, const float* uv_s);  // E4M3 W^UV
bool prefill_supported(const mla_dims& d, int act);
hipError_t prefill_projections(const PrefillArgs& a);  // positions, c^KV, k^R, c^Q, q, k^C, v^C
hipError_t prefill_attention(const PrefillArgs& a);    // causal attention over q, k, v -> out, lse
hipError_t fast_prefill(const PrefillArgs& a);
// FP8 (E4M3) block-scaled GEMM Y = Q(X) Q(W)^T: weights in 128 x 128 blocks,
// activations quantised in 1 x 128 tiles into the workspace.
struct F8Plan {
  int kb, kgroups, nb;  // k-blocks per wave, k-groups, column blocks of 16 per block
  // workspace (one 64-row chunk at a time): activation codes, their scales,
  // fp32 partials of the k-groups
  size_t xc_off, xs_off, part_off, ws_bytes;
};
bool fp8_gemm_supported(int N, int K);
F8Plan fp8_plan(int M, int N, int K);
hipError_t fp8_quantize_weight(int N, int K, const bf16_t* W, uint8_t* codes, float* scales, hipStream_t st);
// With yc: Y also quantised in 1 x 128 tiles (codes yc [M][N], scales ys
// [M][N / 128]); at most 64 rows, N a multiple of 128.
hipError_t fp8_gemm(int M, int N, int K, const bf16_t* X, const uint8_t* Wc, const float* Ws, bf16_t* Y, uint8_t* ws,
                    hipStream_t st, uint8_t* yc = nullptr, float* ys = nullptr);
// Decode with FP8 block-scaled projection weights: the step's query phase
// and combine on E4M3 weights (the attention is the bf16 step's).  W^UK is
// given per head transposed, [H][d_c][d_head], so that every projection is
// Y = X . W^T with W stored [out][in].
struct Fp8Weights {
  const uint8_t *dq_c, *uq_c, *ukt_c;
  const float *dq_s, *uq_s, *ukt_s;
};
bool fp8w_supported(const mla_dims& d);
hipError_t fp8_quantize_weight_t(int batch, int R, int C, const bf16_t* W, uint8_t* codes, float* scales,
                                 hipStream_t st);
size_t fp8w_scratch_offset(const WsLayout& L);
size_t fp8w_scratch_bytes(const mla_dims& d, int R);
hipError_t fp8w_query(const DecodeArgs& a, const Fp8Weights& w);
// u = W^UQ c^Q on FP8 weights: q^C into qc [R][H][d_head], RoPE pairs into qt
hipError_t fp8w_uq(const DecodeArgs& a, const uint8_t* Wc, const float* Ws, const bf16_t* cq, bf16_t* qc,
                   uint8_t* ws);
hipError_t fp8w_combine(const CombineArgs& a, const uint8_t* uv_c, const float* uv_s);
hipError_t merge_partials(const CombineArgs& a);  // split partials -> O_lat (ws olat) and lse
bool skinny_out_supported(int rows, int N, int K);
hipError_t skinny_out(const OutProjArgs& a, int kgroups);  // rows <= 64: k-groups + their sum
hipError_t generic_out_project(const OutProjArgs& a);
hipError_t out_project(const OutProjArgs& a);

}  // namespace mla

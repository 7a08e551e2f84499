// bf16 MFMA GEMMs of the MLA decode path (gfx950) and their epilogues.
//
//   c^Q  = W^DQ h                      (split-K partials, then a reduction)
//   u    = W^UQ c^Q -> q^C, RoPE(q^R)   (summary "Báo cáo Kỹ thuật DeepSeek-V3",
//                                       Phương pháp item 1; lesson's V3
//                                       practice docstring for the W_UQ split)
//   qt_i = tau log2(e) W^UK_i^T q^C_i   (absorption, lesson §2.1.1 Question 2)
//   o_i  = W^UV_i O_lat_i               (value up-projection after attention)
//
// One kernel template: Y[M x N] = X[M x K] . B with B given either as W[N][K]
// (k contiguous, "X W^T") or as W[K][N] (n contiguous, read with the gfx950
// transposing LDS load).  64x64 output tile per 256-thread block, 64-deep k
// steps (whole 128-byte lines of every weight row) through an NS-stage LDS
// ring filled by global_load_lds_dwordx4, four waves of 32x32 (2x2
// v_mfma_f32_16x16x32_bf16, two k-halves per step), optional split-K over
// blockIdx.z and a batch (head) index in blockIdx.y.  The decode GEMMs have
// only 64-256 activation rows: they stream the weights, so what matters is
// keeping enough full cache lines in flight per CU.
#include <algorithm>
#include <type_traits>
#include <math.h>
#include "internal.hpp"

namespace mla {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

constexpr int NS = 4;             // ring depth (three k-steps in flight)
constexpr int BK = 64;
constexpr int TILE_BYTES = 8192;  // 64 rows x 64 k x bf16 (or 64 k x 64 n)
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr float LOG2E = 1.4426950408889634f;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

struct GemmArgs {
  int M, N, K;              // per batch
  int mtiles;               // ceil(M / 64)
  int xcd_map;              // column tiles a multiple of 8: keep a tile's row tiles on one XCD
  int k_per_split;          // multiple of BK
  const bf16_t* X;          // [batch][M][ldx]
  long ldx, bsx;
  const bf16_t* W;          // W_NK: [batch][N][ldw]; else [batch][K][ldw]
  long ldw, bsw;
};

// Row tile: 64 rows x 64 k, row r chunk q (16 B, 8 k) stored at r*8 + (q ^ (r & 7)).
__device__ __forceinline__ int xtile_pos(int r, int q) { return r * 8 + (q ^ (r & 7)); }
// K-major tile: 64 k-rows x 64 n, row k chunk q (8 n) stored at k*8 + (q ^ swz(k)).
__device__ __forceinline__ int ktile_pos(int k, int q) { return k * 8 + (q ^ (4 * ((k >> 1) & 1)) ^ (2 * ((k >> 3) & 1))); }

// Copies one 64 x 64 row tile (rows r0.., columns k0..) into LDS: 8 instructions of
// 1 KiB (8 rows of 128 B each); instruction i covers LDS positions 64i..64i+63.
// Rows >= rows_valid read the last valid row (never stored).
__device__ __forceinline__ void load_rows_tile(const bf16_t* base, long ld, int r0, int rows_valid, int k0,
                                               uint8_t* dst, int i, int lane) {
  const int pos = 64 * i + lane;
  const int r = pos >> 3, phys = pos & 7, q = phys ^ (r & 7);
  int row = r0 + r;
  row = row < rows_valid ? row : rows_valid - 1;
  __builtin_amdgcn_global_load_lds((gbl_void*)(base + (long)row * ld + k0 + 8 * q), (lds_void*)(dst + i * 1024), 16,
                                   0, 0);
}

// Copies a 64 k x 64 n tile of a K-major matrix into LDS (8 instructions).
__device__ __forceinline__ void load_kmajor_tile(const bf16_t* base, long ld, int k0, int n0, uint8_t* dst, int i,
                                                 int lane) {
  const int pos = 64 * i + lane;
  const int k = pos >> 3, phys = pos & 7;
  const int q = phys ^ (4 * ((k >> 1) & 1)) ^ (2 * ((k >> 3) & 1));
  __builtin_amdgcn_global_load_lds((gbl_void*)(base + (long)(k0 + k) * ld + n0 + 8 * q), (lds_void*)(dst + i * 1024),
                                   16, 0, 0);
}

template <bool W_NK, class Epi>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g, Epi epi) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * STAGE_BYTES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // The row tiles of one column tile are neighbours in the dispatch order, so
  // that its weight tiles are fetched from HBM once and then hit in cache;
  // blocks are dealt to the 8 XCDs round-robin, so with xcd_map they also
  // share one L2 (blockIdx.x % 8 picks the XCD).
  int nt, mt;
  if (g.xcd_map) {
    const int loc = blockIdx.x >> 3;
    mt = loc % g.mtiles;
    nt = (loc / g.mtiles) * 8 + (blockIdx.x & 7);
  } else {
    mt = blockIdx.x % g.mtiles;
    nt = blockIdx.x / g.mtiles;
  }
  const int n0 = nt * 64;
  const int batch = blockIdx.y, m0 = mt * 64;
  const int kb = blockIdx.z * g.k_per_split;
  const int ke = min(g.K, kb + g.k_per_split);
  const int nsteps = (ke - kb) / BK;
  const bf16_t* X = g.X + (long)batch * g.bsx;
  const bf16_t* W = g.W + (long)batch * g.bsw;

  // two instructions per wave per tile: X tile (8 instr), W tile (8 instr)
  auto issue = [&](int step) {
    uint8_t* st = lds + (step % NS) * STAGE_BYTES;
    const int k0 = kb + step * BK;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      load_rows_tile(X, g.ldx, m0, g.M, k0, st, wave + 4 * h, lane);
      if (W_NK) load_rows_tile(W, g.ldw, n0, g.N, k0, st + TILE_BYTES, wave + 4 * h, lane);
      else load_kmajor_tile(W, g.ldw, k0, n0, st + TILE_BYTES, wave + 4 * h, lane);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{};

  for (int s = 0; s < NS - 1 && s < nsteps; ++s) issue(s);
  const int g16 = lane >> 4, i16 = lane & 15;
  for (int step = 0; step < nsteps; ++step) {
    // loads of `step` are complete once at most (issued after it) remain
    const int after = min(NS - 2, nsteps - 1 - step);
    switch (after) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<4>(); break;
      default: wait_vmcnt<8>(); break;
    }
    ring_barrier();
    if (step + NS - 1 < nsteps) issue(step + NS - 1);
    const uint8_t* st = lds + (step % NS) * STAGE_BYTES;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {  // two 32-deep MFMA k-steps per stage
      bf16x8 a[2], b[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int r = 32 * wm + 16 * mi + i16;
        a[mi] = *(const bf16x8*)(st + xtile_pos(r, 4 * kh + g16) * 16);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        if (W_NK) {
          const int r = 32 * wn + 16 * ni + i16;
          b[ni] = *(const bf16x8*)(st + TILE_BYTES + xtile_pos(r, 4 * kh + g16) * 16);
        } else {
          // B[k][n]: lane needs k = 32kh + 8*g16 + e, n = 32wn + 16ni + i16 (two transposed reads)
          const int e = i16 >> 2, qq = i16 & 3;
          const int nq = 32 * wn + 16 * ni + 4 * qq;  // first n of this lane's 4-wide source
          const int c = nq >> 3, half = (nq >> 2) & 1;
          const int k1 = 32 * kh + 8 * g16 + e, k2 = k1 + 4;
          const uint8_t* p1 = st + TILE_BYTES + ktile_pos(k1, c) * 16 + half * 8;
          const uint8_t* p2 = st + TILE_BYTES + ktile_pos(k2, c) * 16 + half * 8;
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
          const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p2);
          const short s8 __attribute__((ext_vector_type(8))) = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
          b[ni] = __builtin_bit_cast(bf16x8, s8);
        }
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
  }
  // C layout: lane holds rows 4*g16 .. +3 of column i16 of each 16x16 block
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
      epi(batch, m0 + 32 * wm + 16 * mi + 4 * g16, n0 + 32 * wn + 16 * ni + i16, acc[mi][ni], blockIdx.z, g.M);
}

// ------------------------------------------------------------ epilogues
// fp32 split-K partial: Y[split][row][col]
struct EpiPartial {
  float* Y;
  int ld;       // N
  long split_stride;
  __device__ void operator()(int, int row, int col, f32x4 v, int split, int M) const {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row + r < M) Y[split * split_stride + (long)(row + r) * ld + col] = v[r];
  }
};

// u = W^UQ c^Q: head i = col / (d_head + d_rope); content columns -> q^C (bf16
// [R][H][d_head]); RoPE columns -> rotated at the row's position, scaled by
// tau log2 e, into qt[R][H][d_c + ...].  Adjacent columns form a RoPE pair and
// sit in neighbouring lanes.
struct EpiUQ {
  bf16_t* qc;
  bf16_t* qt;
  const int32_t* seqlens;
  int H, d_head, d_rope, d_c, s_q;
  float scale2;
  double freq[32];  // theta^(-2m/d_rope) of RoPE pair m
  __device__ void operator()(int, int row, int col, f32x4 v, int, int M) const {
    const int w = d_head + d_rope;
    const int i = col / w, d = col % w;
    if (d < d_head) {  // wave-uniform: 16-column blocks never straddle the boundary (d_head % 16 == 0)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (row + r < M) qc[((long)(row + r) * H + i) * d_head + d] = (bf16_t)v[r];
      return;
    }
    const int m = (d - d_head) >> 1;
    const bool odd = (d - d_head) & 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float other = __shfl_xor(v[r], 1, 64);
      const int rr = row + r;
      if (rr >= M) continue;
      const int b = rr / s_q, j = rr % s_q;
      int p = seqlens[b] - s_q + j;
      p = p < 0 ? 0 : p;
      float cs, sn;
      rope_cs_w(p, freq[m], &cs, &sn);
      const float x0 = odd ? other : v[r], x1 = odd ? v[r] : other;
      const float y = odd ? x0 * sn + x1 * cs : x0 * cs - x1 * sn;
      qt[((long)rr * H + i) * (d_c + d_rope) + d_c + (d - d_head)] = (bf16_t)(scale2 * y);
    }
  }
};

// Absorption: qt[row][head][col] = scale2 * v (content part of the query)
struct EpiAbsorb {
  bf16_t* qt;
  int H, d_c, d_rope;
  float scale2;
  __device__ void operator()(int head, int row, int col, f32x4 v, int, int M) const {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row + r < M) qt[((long)(row + r) * H + head) * (d_c + d_rope) + col] = (bf16_t)(scale2 * v[r]);
  }
};

// Output: out[row][head][col] = v (bf16)
struct EpiOut {
  bf16_t* out;
  int H, d_head;
  __device__ void operator()(int head, int row, int col, f32x4 v, int, int M) const {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row + r < M) out[((long)(row + r) * H + head) * d_head + col] = (bf16_t)v[r];
  }
};

// c^Q = sum of the split-K partials, rounded to bf16.
__global__ void k_reduce_cq(int R, int N, int splits, const float* part, bf16_t* cq) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)R * N) return;
  float s = 0.0f;
  for (int k = 0; k < splits; ++k) s += part[(long)k * R * N + idx];
  cq[idx] = (bf16_t)s;
}

// Merge of the per-split attention partials into O_lat (bf16 [R][H][d_c]) and
// the row's log-sum-exp: weights exp2(lse_s - max_s lse), empty splits
// (lse = -inf) skipped.  One wave per (row, head); each lane owns 8 channels
// per pass (16-byte partial reads).  S splits (the host's, already checked
// against the workspace size); partials are fp32 or bf16 (header).
__global__ __launch_bounds__(256) void k_merge(int batch, int H, int s_q, int S, int d_c, const uint8_t* ws,
                                               size_t lpart_off, bf16_t* olat, float* lse_out) {
  const bool pbf16 = ((const int32_t*)ws)[HDR_PDT] == MLA_BF16;
  const float* lpart = (const float*)(ws + lpart_off);
  const uint8_t* opart = ws + opart_offset(lpart_off, batch, S, s_q, H);
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // (b*s_q + j)*H + i
  if (row >= batch * s_q * H) return;
  const int i = row % H, bj = row / H, j = bj % s_q, b = bj / s_q;
  const size_t p0 = (((size_t)b * S) * s_q + j) * H + i, pstep = (size_t)s_q * H;  // partial row of split s
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, lpart[p0 + s * pstep]);
  M = wave_max(M);
  float W = 0.0f;
  for (int s = lane; s < S; s += 64) {
    const float l = lpart[p0 + s * pstep];
    W += l == -INFINITY ? 0.0f : exp2f(l - M);
  }
  W = wave_sum(W);
  const float invW = W > 0.0f ? 1.0f / W : 0.0f;
  if (lse_out && lane == 0) lse_out[row] = W > 0.0f ? (M + log2f(W)) * 0.6931471805599453f : -INFINITY;
  for (int c = 8 * lane; c < d_c; c += 512) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (pbf16) {
      // Lane t of a chunk of 64 splits holds split t's weight; the rows of 8
      // splits are loaded together (a long split list would otherwise pay
      // one memory latency per split).  Empty splits are never read.
      for (int s0 = 0; s0 < S; s0 += 64) {
        const int n = min(64, S - s0);
        const float lt = lane < n ? lpart[p0 + (size_t)(s0 + lane) * pstep] : -INFINITY;
        const float wt = lt == -INFINITY ? 0.0f : exp2f(lt - M);
        for (int u0 = 0; u0 < n; u0 += 8) {
          float w[8];
          bf16x8 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            w[u] = __shfl(wt, u0 + u, 64);  // 0 past the chunk (lanes >= n hold 0)
            v[u] = bf16x8{};
            if (w[u] != 0.0f)
              v[u] = *(const bf16x8*)((const bf16_t*)opart + (p0 + (size_t)(s0 + u0 + u) * pstep) * d_c + c);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += w[u] * (float)v[u][e];
        }
      }
    } else {
      for (int s = 0; s < S; ++s) {
        const float l = lpart[p0 + s * pstep];
        if (l == -INFINITY) continue;
        const float w = exp2f(l - M);
        const size_t off = (p0 + s * pstep) * d_c + c;
        const f32x4 v0 = *(const f32x4*)((const float*)opart + off);
        const f32x4 v1 = *(const f32x4*)((const float*)opart + off + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { acc[e] += w * v0[e]; acc[4 + e] += w * v1[e]; }
      }
    }
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16_t)(acc[e] * invW);
    *(bf16x8*)(olat + (size_t)row * d_c + c) = o;
  }
}

template <bool W_NK, class Epi>
hipError_t launch_gemm(const GemmArgs& g, int batch, int splits, const Epi& epi, hipStream_t st) {
  dim3 grid((g.N / 64) * g.mtiles, batch, splits);
  MLA_TRY(launch(&k_gemm<W_NK, Epi>, grid, dim3(256), 0, st, g, epi));
  return hipSuccess;
}

GemmArgs gemm_args(int M, int N, int K, const bf16_t* X, long ldx, long bsx, const bf16_t* W, long ldw, long bsw,
                   int splits) {
  GemmArgs g;
  g.M = M; g.N = N; g.K = K; g.mtiles = (M + 63) / 64;
  g.xcd_map = (N / 64) % 8 == 0;
  int kps = (K + splits - 1) / splits;
  g.k_per_split = (kps + BK - 1) / BK * BK;
  g.X = X; g.ldx = ldx; g.bsx = bsx; g.W = W; g.ldw = ldw; g.bsw = bsw;
  return g;
}

}  // namespace

// Query side of the decode on MFMA: qt = [tau log2e W^UK^T q^C | tau log2e RoPE(q^R)].
hipError_t fast_query(const DecodeArgs& a) {
  const mla_dims& d = a.d;
  const int R = a.batch * a.s_q, H = d.n_heads;
  if (skinny_query_supported(d, R)) return skinny_query(a);
  const float scale2 = a.scale * LOG2E;
  bf16_t* qt = (bf16_t*)(a.ws + a.L.qt);
  bf16_t* qc = (bf16_t*)(a.ws + a.L.u);  // q^C, bf16 [R][H][d_head]
  hipError_t e = hipSuccess;
  const bf16_t* cq = (const bf16_t*)a.hq;
  if (a.W_DQ) {
    // c^Q = W^DQ h: split K so that the grid fills the GPU's 512 block slots
    // (two 64 KiB blocks a CU) in one round: rounding up left a second round
    // of a few blocks (576 blocks at 256 rows, 528 at 128)
    const int ntile = d.d_cq / 64 * ((R + 63) / 64);
    int splits = std::max(1, 512 / ntile);
    splits = splits > KSPLIT_MAX ? KSPLIT_MAX : splits;
    while (splits > 1 && d.d_model / splits < 2 * BK) --splits;
    GemmArgs g = gemm_args(R, d.d_cq, d.d_model, (const bf16_t*)a.hq, d.d_model, 0, (const bf16_t*)a.W_DQ,
                           d.d_model, 0, splits);
    splits = (d.d_model + g.k_per_split - 1) / g.k_per_split;
    float* part = (float*)(a.ws + a.L.cq_part);
    e = launch_gemm<true>(g, 1, splits, EpiPartial{part, d.d_cq, (long)R * d.d_cq}, a.stream);
    if (e != hipSuccess) return e;
    bf16_t* cqb = (bf16_t*)(a.ws + a.L.cq);
    const long n = (long)R * d.d_cq;
    MLA_TRY(launch(&k_reduce_cq, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, a.stream, R, d.d_cq, splits,
                       (const float*)part, cqb));
    cq = cqb;
  }
  if (rows_query_supported(d, R)) return rows_query(a, cq);
  {
    GemmArgs g = gemm_args(R, H * (d.d_head + d.d_rope), d.d_cq, cq, d.d_cq, 0, (const bf16_t*)a.W_UQ, d.d_cq, 0, 1);
    EpiUQ epi{qc, qt, a.seqlens, H, d.d_head, d.d_rope, d.d_c, a.s_q, scale2, {}};
    for (int m = 0; m < d.d_rope / 2; ++m) epi.freq[m] = pow((double)d.rope_theta, -2.0 * m / d.d_rope);
    e = launch_gemm<true>(g, 1, 1, epi, a.stream);
    if (e != hipSuccess) return e;
  }
  {
    // per head: qt[:, i, 0:d_c] = scale2 * q^C_i (R x d_head) . W^UK_i (d_head x d_c)
    GemmArgs g = gemm_args(R, d.d_c, d.d_head, qc, (long)H * d.d_head, d.d_head, (const bf16_t*)a.W_UK, d.d_c,
                           (long)d.d_head * d.d_c, 1);
    e = launch_gemm<false>(g, H, 1, EpiAbsorb{qt, H, d.d_c, d.d_rope, scale2}, a.stream);
  }
  return e;
}

// ------------------------------------------------------------ prefill
// The projections of the non-absorbed prefill (lesson §2.1.1: c^KV, k^R,
// c^Q, q; k^C = W^UK c^KV and v^C = W^UV c^KV explicitly per head), one
// general GEMM each, with the layout the causal attention kernel reads.

namespace {

// RoPE frequencies theta^(-2m/d_rope), computed on the host in double, into
// device memory: epilogues index them per lane, which a by-value kernel
// argument would turn into a private-memory copy in every thread.
struct FreqTable {
  double f[32];
};
__global__ void k_store_freq(FreqTable t, int half, double* __restrict__ out) {
  if ((int)threadIdx.x < half) out[threadIdx.x] = t.f[threadIdx.x];
}

// (cos, sin) of every token's RoPE angles pos_t * theta^(-2m/d_rope): one
// thread per (token, pair), the same reduction as everywhere else.  The
// projections' epilogues read them, once per head.
__global__ void k_rope_table(int n_tok, int half, const int32_t* __restrict__ pos, const double* __restrict__ freq,
                             float2* __restrict__ tab) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)n_tok * half) return;
  const int t = (int)(i / half), m = (int)(i % half);
  float cs, sn;
  rope_cs_w(pos[t], freq[m], &cs, &sn);
  tab[i] = make_float2(cs, sn);
}

// Position of token t in its sequence: t - cu_seqlens[b] for the b with
// cu_seqlens[b] <= t < cu_seqlens[b + 1] (binary search).
__global__ void k_positions(const int32_t* __restrict__ cu, int n_seq, int n_tok, int32_t* __restrict__ pos) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_tok) return;
  int lo = 0, hi = n_seq;  // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  pos[t] = t - cu[lo];
}

// Y[row][col] (bf16, row stride ld)
struct EpiRowStore {
  static constexpr bool kRows8 = true;  // has mul() and store8() for the staged 256 x 256 epilogue
  bf16_t* y;
  int ld;
  __device__ float mul() const { return 1.0f; }
  __device__ void store8(int row, int col, bf16x8 v) const { *(bf16x8*)(y + (long)row * ld + col) = v; }
  __device__ void operator()(int, int row, int col, f32x4 v, int, int M) const {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row + r < M) y[(long)(row + r) * ld + col] = (bf16_t)v[r];
  }
};

// k^R = RoPE(W^KR h) at the row's position; columns (2m, 2m+1) are a pair in
// neighbouring lanes.
struct EpiRopeRows {
  bf16_t* y;
  int ld;
  const float2* cs_tab;  // [n_tok][d_rope / 2] (cos, sin) of the token's angles
  __device__ void operator()(int, int row, int col, f32x4 v, int, int M) const {
    const int m = col >> 1, half = ld >> 1;
    const bool odd = col & 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float other = __shfl_xor(v[r], 1, 64);
      const int rr = row + r;
      if (rr >= M) continue;
      const float2 t = cs_tab[(long)rr * half + m];
      const float cs = t.x, sn = t.y;
      const float x0 = odd ? other : v[r], x1 = odd ? v[r] : other;
      y[(long)rr * ld + col] = (bf16_t)(odd ? x0 * sn + x1 * cs : x0 * cs - x1 * sn);
    }
  }
};

// q = W^UQ c^Q, column n = (d_head + d_rope) i + d -> q[i][row][d] scaled by
// tau log2(e), the RoPE columns rotated at the row's position first.  A
// 16-column block is all content or all RoPE (d_head % 16 == 0), so the
// branch is wave-uniform.
struct EpiPrefillQ {
  static constexpr bool kRows8 = true;
  bf16_t* q;
  int n_tok, d_head, d_rope;
  float scale2;
  __device__ float mul() const { return scale2; }
  __device__ void store8(int row, int col, bf16x8 v) const {  // 8 columns never straddle a head (w % 8 == 0)
    const int w = d_head + d_rope, i = col / w, d = col % w;
    *(bf16x8*)(q + ((long)i * n_tok + row) * w + d) = v;
  }
  // q[i][row][d] = scale2 * v for column d_head_rope i + d; the RoPE of q^R
  // is left to the attention kernel, which rotates its query fragments as it
  // loads them: a table load here would wait (vmcnt counts stores too) for
  // every store before it.
  __device__ void operator()(int, int row, int col, f32x4 v, int, int M) const {
    const int w = d_head + d_rope;
    const int i = col / w, d = col % w;
    bf16_t* qi = q + (long)i * n_tok * w;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row + r < M) qi[(long)(row + r) * w + d] = (bf16_t)(scale2 * v[r]);
  }
};

// k^C or v^C: column n = d_head i + d -> y[i][row][d]
struct EpiHeadMajor {
  static constexpr bool kRows8 = true;
  bf16_t* y;
  int n_tok, d_head;
  __device__ float mul() const { return 1.0f; }
  __device__ void store8(int row, int col, bf16x8 v) const {
    const int i = col / d_head, d = col % d_head;
    *(bf16x8*)(y + ((long)i * n_tok + row) * d_head + d) = v;
  }
  __device__ void operator()(int, int row, int col, f32x4 v, int, int M) const {
    const int i = col / d_head, d = col % d_head;
    bf16_t* yi = y + (long)i * n_tok * d_head;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row + r < M) yi[(long)(row + r) * d_head + d] = (bf16_t)v[r];
  }
};

// ------------------------------------------------------------ 256 x 256 tiles
// Y = X W^T (W[N][K]) for hundreds of rows and more (the prefill
// projections).  256 x 256 output tile per 256-thread block, four waves of
// 128 x 128 (4 x 4 v_mfma_f32_32x32x16_bf16 accumulators, 256 AGPRs), 32-deep
// k-steps through a ring of four 32 KiB LDS stages (X tile, then W tile:
// 256 rows x 64 B each) filled by global_load_lds_dwordx4 from asm, three
// k-steps ahead; one block per CU.  The fragments of the next k-step are read
// from LDS between the current step's MFMAs (two register sets).  Row r of a tile keeps its 16-byte chunk
// c at slot c ^ ((r >> 2) & 3), so that the 16 lanes of each phase of a
// fragment read (rows r .. r+15, one chunk) hit 16 different bank groups.
// The 8 XCDs take contiguous ranges of tiles, ordered GB_GM row tiles x
// successive column tiles, so the blocks running together on an XCD share
// their X and W tiles in its L2.
constexpr int GB_T = 256;                 // tile rows and columns
constexpr int GB_BK = 32;                 // k per step
constexpr int GB_TILE = GB_T * GB_BK * 2; // 16 KiB
constexpr int GB_STAGE = 2 * GB_TILE;     // 32 KiB
constexpr int GB_NS = 4;                  // stages
constexpr int GB_LDS = GB_NS * GB_STAGE;  // 128 KiB
constexpr int GB_GM = 4;

struct BigArgs {
  int M, N, K, mt, nt;
  const bf16_t* X;  // [M][ldx]
  long ldx;
  const bf16_t* W;  // [N][ldw]
  long ldw;
};

__device__ __forceinline__ void gb_dma(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds_addr)
               : "memory");
}

// An accumulator element read out of its AGPR where the code stands (the
// compiler otherwise moves every accumulator of the tile to VGPRs at once).
__device__ __forceinline__ float agpr_read(float x) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
  return r;
}

// Epilogues that can take eight consecutive columns of a row at once
template <class E, class = void>
struct has_rows8 : std::false_type {};
template <class E>
struct has_rows8<E, std::void_t<decltype(E::kRows8)>> : std::bool_constant<E::kRows8> {};

template <class Epi>
__global__ __launch_bounds__(256, 1) void k_gemm_big(BigArgs a, Epi epi) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t gb_raw[];
  typedef __attribute__((address_space(3))) bf16x8 lbf16x8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hw = lane >> 5;
  const int T = a.mt * a.nt, per = (T + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (w >= T) return;
  const int grp = w / (GB_GM * a.nt), gm0 = grp * GB_GM, gsz = min(GB_GM, a.mt - gm0);
  const int rr = w - grp * GB_GM * a.nt;
  const int m0 = (gm0 + rr % gsz) * GB_T, n0 = (rr / gsz) * GB_T;
  const uint32_t lds = (uint32_t)(uintptr_t)gb_raw;

  // copies: wave w issues rows 16 (4w + n) + lane / 4 of each tile
  // (n = 0..3), chunk slot lane % 4; the k position goes into the scalar base
  uint32_t xo[4], wo[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row = 16 * (4 * wave + n) + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    xo[n] = (uint32_t)(min(row, a.M - 1 - m0) * a.ldx * 2 + 16 * c);
    wo[n] = (uint32_t)(row * a.ldw * 2 + 16 * c);
  }
  const uint8_t* xb = (const uint8_t*)(a.X + (long)m0 * a.ldx);
  const uint8_t* wb = (const uint8_t*)(a.W + (long)n0 * a.ldw);
  auto issue = [&](int ks, int stg) {
    const uint8_t* xk = xb + ks * 64;
    const uint8_t* wk = wb + ks * 64;
    const uint32_t d = lds + stg * GB_STAGE + 4096 * wave;
#pragma unroll
    for (int n = 0; n < 4; ++n) gb_dma(xk, xo[n], d + 1024 * n);
#pragma unroll
    for (int n = 0; n < 4; ++n) gb_dma(wk, wo[n], d + GB_TILE + 1024 * n);
  };

  // fragment read addresses of stages 0 and 2 (stages 1 and 3 add GB_STAGE):
  // row 128 wm + 32 mi + l32 of the X tile, 128 wn + 32 ni + l32 of the W
  // tile, chunk 2 k16 + hw
  const int wm = wave >> 1, wn = wave & 1;
  uint32_t fx[2][2], fw[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int k16 = 0; k16 < 2; ++k16) {
      const uint32_t o = lds + 2 * h * GB_STAGE + l32 * 64 + 16 * ((2 * k16 + hw) ^ ((l32 >> 2) & 3));
      fx[h][k16] = o + 128 * wm * 64;
      fw[h][k16] = o + GB_TILE + 128 * wn * 64;
    }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int nk = a.K / GB_BK;  // a multiple of 4
  // Fragments of a k-step: X rows 32 i (+ 128 wm), W rows 32 j (+ 128 wn), the
  // two 16-deep halves k16.  Step ks multiplies the fragments read during
  // step ks-1 and reads those of ks+1 between its MFMAs, so no MFMA waits for
  // an LDS read issued after the barrier.
  bf16x8 fa[2][2][4], fb[2][2][4];  // [register set][k16][i or j]
  auto read_frags = [&](auto stg_c, auto set_c, int k16, int i) {
    constexpr int STG = decltype(stg_c)::value, SET = decltype(set_c)::value;
    constexpr int H = STG >> 1;
    constexpr uint32_t SO = (STG & 1) * GB_STAGE;
    fa[SET][k16][i] = *(const lbf16x8*)(fx[H][k16] + SO + 2048 * i);
    fb[SET][k16][i] = *(const lbf16x8*)(fw[H][k16] + SO + 2048 * i);
  };
  issue(0, 0);
  issue(1, 1);
  issue(2, 2);
  issue(3, 3);
  wait_vmcnt<24>();  // this wave's copies of k-step 0 landed
  ring_barrier();
#pragma unroll
  for (int k16 = 0; k16 < 2; ++k16)
#pragma unroll
    for (int i = 0; i < 4; ++i) read_frags(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, k16, i);
  // Step ks (stage ks & 3, register set ks & 1): after the barrier, every
  // wave's copies of k-step ks+1 have landed and every wave has read k-step
  // ks's fragments, so the stage of ks takes k-step ks+4; past the last
  // k-step a repeat of it (never used), so that the loop body has no branch:
  // a branch there makes the compiler move the accumulators between AGPRs
  // and VGPRs.  The fragments read for ks+1 at the last step are never used.
  // The step's eight copies are spread over its MFMA groups, one after each
  // group of four: a wave whose copy waits for the address unit issues
  // nothing else meanwhile, so copies issued back to back after the barrier
  // left the matrix unit idle.
  auto step = [&](auto stg_c, int ks) {
    constexpr int STG = decltype(stg_c)::value;
    constexpr int SET = STG & 1;
    wait_vmcnt<16>();  // this wave's copies of ks+1 landed (ks+2, ks+3 may be in flight)
    ring_barrier();
    const int kc = min(ks + 4, nk - 1);
    const uint8_t* xk = xb + kc * 64;
    const uint8_t* wk = wb + kc * 64;
    const uint32_t d = lds + STG * GB_STAGE + 4096 * wave;
#pragma unroll
    for (int k16 = 0; k16 < 2; ++k16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[SET][k16][i], fb[SET][k16][j], acc[i][j], 0, 0, 0);
        read_frags(std::integral_constant<int, (STG + 1) & 3>{}, std::integral_constant<int, 1 - SET>{}, k16, i);
        // copy n = i of the X tile (k16 = 0) or of the W tile (k16 = 1)
        if (k16 == 0) gb_dma(xk, xo[i], d + 1024 * i);
        else gb_dma(wk, wo[i], d + GB_TILE + 1024 * i);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int ks = 0; ks < nk; ks += 4) {
    step(std::integral_constant<int, 0>{}, ks);
    step(std::integral_constant<int, 1>{}, ks + 1);
    step(std::integral_constant<int, 2>{}, ks + 2);
    step(std::integral_constant<int, 3>{}, ks + 3);
  }
  wait_vmcnt<0>();  // the repeat copies land before the block leaves

  if constexpr (has_rows8<Epi>::value) {
    // Staged epilogue: the wave's 128 x 128 tile goes to LDS (free now) as
    // bf16, row-major with 256-byte rows (the 64-byte quarter q of row r at
    // q ^ ((r >> 2) & 1): the two half-waves' rows r and r + 4 use other
    // banks), then leaves in whole rows: 16 lanes store one row's 256 bytes.
    ring_barrier();  // every wave is done with the stages
    const uint32_t tile = lds + 32768 * wave;
    const float mul = epi.mul();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = 32 * i + 8 * (e >> 2) + 4 * hw + (e & 3), c = 32 * j + l32;
          const uint32_t off = r * 256 + ((2 * c) ^ (((r >> 2) & 1) * 64));
          *(__attribute__((address_space(3))) bf16_t*)(tile + off) = (bf16_t)(mul * agpr_read(acc[i][j][e]));
        }
    const int rbase = m0 + 128 * wm, cbase = n0 + 128 * wn;
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
      const int r = 4 * it + (lane >> 4), k = lane & 15;
      const bf16x8 v = *(const lbf16x8*)(tile + r * 256 + 16 * (k ^ (((r >> 2) & 1) * 4)));
      if (rbase + r < a.M) epi.store8(rbase + r, cbase + 8 * k, v);
    }
    return;
  }
  // C lane layout: column l32 of each 32 x 32 block, rows 8 j + 4 hw + 0..3.
  // The tile origin passes through an empty asm statement so that no output
  // address is computed before the k-loop and held across it.
  int row0 = m0 + 128 * wm + 4 * hw, col0 = n0 + 128 * wn + l32;
  asm volatile("" : "+v"(row0), "+v"(col0));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // one accumulator block at a time leaves the AGPRs (volatile reads,
      // in program order); a fresh opaque copy of the origin per block keeps
      // the compiler from holding every block's row addresses at once
      int rb = row0, cb = col0;
      asm volatile("" : "+v"(rb), "+v"(cb));
      f32x16 t;
#pragma unroll
      for (int e = 0; e < 16; ++e) t[e] = agpr_read(acc[i][j][e]);
      // a block entirely past the last row stores nothing
      if (__builtin_amdgcn_readfirstlane(m0 + 128 * wm + 32 * i) >= a.M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
        epi(0, rb + 32 * i + 8 * q, cb + 32 * j, v, 0, a.M);
      }
    }
}

bool big_gemm_ok(int M, int N, int K) { return M >= GB_T && N % GB_T == 0 && K % 128 == 0; }

template <class Epi>
hipError_t launch_big(int M, int N, int K, const bf16_t* X, long ldx, const bf16_t* W, long ldw, const Epi& epi,
                      hipStream_t st) {
  BigArgs a{M, N, K, (M + GB_T - 1) / GB_T, N / GB_T, X, ldx, W, ldw};
  MLA_TRY(lds_limit((const void*)&k_gemm_big<Epi>, GB_LDS));
  const int T = a.mt * a.nt;
  return launch(&k_gemm_big<Epi>, dim3(8 * ((T + 7) / 8)), dim3(256), GB_LDS, st, a, epi);
}

// Y = X W^T with the 256 x 256 kernel when the shape fits it, else the
// 64 x 64 one.
template <class Epi>
hipError_t gemm_xwt(int M, int N, int K, const bf16_t* X, long ldx, const bf16_t* W, long ldw, const Epi& epi,
                    hipStream_t st) {
  if (big_gemm_ok(M, N, K)) return launch_big(M, N, K, X, ldx, W, ldw, epi, st);
  GemmArgs g = gemm_args(M, N, K, X, ldx, 0, W, ldw, 0, 1);
  return launch_gemm<true>(g, 1, 1, epi, st);
}

}  // namespace

hipError_t prefill_projections(const PrefillArgs& a) {
  const mla_dims& d = a.d;
  const int n = a.n_tok, H = d.n_heads, w = d.d_head + d.d_rope;
  int32_t* pos = (int32_t*)(a.ws + a.L.pos);
  bf16_t* ckv = (bf16_t*)(a.ws + a.L.ckv);
  bf16_t* kr = (bf16_t*)(a.ws + a.L.kr);
  bf16_t* cq = (bf16_t*)(a.ws + a.L.cq);
  bf16_t* q = (bf16_t*)(a.ws + a.L.q);
  bf16_t* kc = (bf16_t*)(a.ws + a.L.kc);
  bf16_t* vc = (bf16_t*)(a.ws + a.L.vc);
  MLA_TRY(launch(&k_positions, dim3((n + 255) / 256), dim3(256), 0, a.stream, a.cu_seqlens, a.n_seq, n, pos));
  FreqTable ft{};
  for (int m = 0; m < d.d_rope / 2; ++m) ft.f[m] = pow((double)d.rope_theta, -2.0 * m / d.d_rope);
  double* freq = (double*)(a.ws + a.L.freq);
  MLA_TRY(launch(&k_store_freq, dim3(1), dim3(64), 0, a.stream, ft, d.d_rope / 2, freq));
  float2* cs_tab = (float2*)(a.ws + a.L.rope);
  const long nrope = (long)n * (d.d_rope / 2);
  MLA_TRY(launch(&k_rope_table, dim3((unsigned)((nrope + 255) / 256)), dim3(256), 0, a.stream, n, d.d_rope / 2,
                 (const int32_t*)pos, (const double*)freq, cs_tab));
  MLA_TRY(gemm_xwt(n, d.d_c, d.d_model, a.h, d.d_model, a.W_DKV, d.d_model, EpiRowStore{ckv, d.d_c}, a.stream));
  EpiRopeRows er{kr, d.d_rope, cs_tab};
  MLA_TRY(gemm_xwt(n, d.d_rope, d.d_model, a.h, d.d_model, a.W_KR, d.d_model, er, a.stream));
  MLA_TRY(gemm_xwt(n, d.d_cq, d.d_model, a.h, d.d_model, a.W_DQ, d.d_model, EpiRowStore{cq, d.d_cq}, a.stream));
  EpiPrefillQ eq{q, n, d.d_head, d.d_rope, a.scale * LOG2E};
  MLA_TRY(gemm_xwt(n, H * w, d.d_cq, cq, d.d_cq, a.W_UQ, d.d_cq, eq, a.stream));
  MLA_TRY(gemm_xwt(n, H * d.d_head, d.d_c, ckv, d.d_c, a.W_UK, d.d_c, EpiHeadMajor{kc, n, d.d_head}, a.stream));
  return gemm_xwt(n, H * d.d_head, d.d_c, ckv, d.d_c, a.W_UV, d.d_c, EpiHeadMajor{vc, n, d.d_head}, a.stream);
}

// Combine on MFMA: merge the splits into O_lat, then out_i = W^UV_i O_lat_i
// (one fused kernel for at most 64 rows).
// ------------------------------------------------------------ W^O
int out_proj_splits(int act, int rows, int N, int K) {
  if (act != MLA_BF16 || rows < 1) return 0;
  if (skinny_out_supported(rows, N, K)) return K / 1024;
  if (N % 64 || K % BK) return 0;
  // general GEMM: split K until about 1024 blocks, at most 8 splits
  const long tiles = (long)((rows + 63) / 64) * (N / 64);
  const int want = (int)std::min<long>(8, std::max<long>(1, (1024 + tiles - 1) / tiles));
  return std::min(want, K / BK);
}

// fp32 partials of the MFMA path, and never less than the fp32 result of
// the generic path for bf16 (which MLA_FORCE_GENERIC may select).
size_t out_proj_ws_bytes(int act, int rows, int N, int K) {
  if (rows < 1 || act == MLA_F32) return 0;
  const int s = out_proj_splits(act, rows, N, K);
  return (size_t)std::max(s, 1) * rows * N * 4;
}

// y = W^O o: the skinny kernel for at most 64 rows, the general GEMM (split
// over K into fp32 partials when the tiles alone do not fill the chip)
// otherwise, the generic kernel for other shapes and for fp32.
hipError_t out_project(const OutProjArgs& a) {
  const int s = out_proj_splits(a.act, a.rows, a.N, a.K);
  if (s == 0) return generic_out_project(a);
  if (skinny_out_supported(a.rows, a.N, a.K)) return skinny_out(a, s);
  // one pass (enough tiles without a K split): the 256 x 256 kernel where it
  // fits and still gives a block per CU
  const EpiRowStore ey{(bf16_t*)a.y, a.N};
  if (s == 1 && big_gemm_ok(a.rows, a.N, a.K) && (long)((a.rows + 255) / 256) * (a.N / 256) >= 256)
    return launch_big(a.rows, a.N, a.K, (const bf16_t*)a.o, a.K, (const bf16_t*)a.W_O, a.K, ey, a.stream);
  GemmArgs g = gemm_args(a.rows, a.N, a.K, (const bf16_t*)a.o, a.K, 0, (const bf16_t*)a.W_O, a.K, 0, s);
  if (s == 1) return launch_gemm<true>(g, 1, 1, ey, a.stream);
  float* part = (float*)a.ws;
  MLA_TRY(launch_gemm<true>(g, 1, s, EpiPartial{part, a.N, (long)a.rows * a.N}, a.stream));
  return launch(&k_reduce_cq, dim3((a.rows * a.N + 255) / 256), dim3(256), 0, a.stream, a.rows, a.N, s,
                (const float*)part, (bf16_t*)a.y);
}

// O_lat (bf16, the combine's own region: the queries stay intact) and the
// rows' lse from the split partials.
hipError_t merge_partials(const CombineArgs& a) {
  const int R = a.batch * a.s_q, H = a.d.n_heads;
  return launch(&k_merge, dim3((R * H + 3) / 4), dim3(256), 0, a.stream, a.batch, H, a.s_q, a.S, a.d.d_c,
                (const uint8_t*)a.ws, a.L.lpart, (bf16_t*)(a.ws + a.L.olat), a.lse_out);
}

hipError_t fast_combine(const CombineArgs& a) {
  const mla_dims& d = a.d;
  const int R = a.batch * a.s_q, H = d.n_heads;
  if (merge_uv_supported(d, R, a.S)) return merge_uv(a);
  MLA_TRY(merge_partials(a));
  const bf16_t* olat = (const bf16_t*)(a.ws + a.L.olat);
  hipError_t e;
  GemmArgs g = gemm_args(R, d.d_head, d.d_c, olat, (long)H * d.d_c, d.d_c, (const bf16_t*)a.W_UV, d.d_c,
                         (long)d.d_head * d.d_c, 1);
  e = launch_gemm<true>(g, H, 1, EpiOut{(bf16_t*)a.out, H, d.d_head}, a.stream);
  return e;
}

}  // namespace mla

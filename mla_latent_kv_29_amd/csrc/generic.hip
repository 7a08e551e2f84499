// Generic MLA kernels: any supported dims, F32 or BF16 activations, F32 /
// BF16 / FP8 caches.  Plain VALU code with fp32 accumulation; the MFMA kernels
// for the DeepSeek-V3 shape live in fast_*.hip.  These serve the small float32
// configuration and every shape the MFMA kernels do not cover.
//
// Formulas: DeepSeek-V3 reading lesson "Читаем техотчёт DeepSeek-V3 вместе",
// §2.1.1 (latents, concatenated per-head key, absorption in Question 2) and
// the summary "Báo cáo Kỹ thuật DeepSeek-V3", Phương pháp item 1 (c^Q).
#include "internal.hpp"
#include "layout.hpp"
#include <math.h>

namespace mla {

static constexpr float LOG2E = 1.4426950408889634f;
static constexpr float LN2 = 0.6931471805599453f;

// ------------------------------------------------------------ cache access
__device__ __forceinline__ const uint8_t* page_ptr(const CacheGeom& g, const uint8_t* pages,
                                                   const int32_t* bt, int max_pages, int b, int t) {
  int page = bt[(size_t)b * max_pages + t / g.page_size];
  return pages + (size_t)page * g.page_bytes;
}

__device__ __forceinline__ float cache_lat(const CacheGeom& g, const uint8_t* pg, int slot, int c) {
  if (g.dtype == MLA_F32) return ((const float*)pg)[(size_t)slot * (g.d_c + g.d_rope) + c];
  if (g.dtype == MLA_BF16) return (float)*(const bf16_t*)(pg + bf16_page_off(slot, c, g.page_size));
  float s = ((const float*)(pg + g.fp8_scale_off))[slot * (g.d_c / 128) + c / 128];
  return e4m3_to_f32(pg[fp8_code_off(slot, c, g.page_size)]) * s;
}

__device__ __forceinline__ float cache_rope(const CacheGeom& g, const uint8_t* pg, int slot, int m) {
  if (g.dtype == MLA_F32) return ((const float*)pg)[(size_t)slot * (g.d_c + g.d_rope) + g.d_c + m];
  if (g.dtype == MLA_BF16) return (float)*(const bf16_t*)(pg + bf16_page_off(slot, g.d_c + m, g.page_size));
  return (float)*(const bf16_t*)(pg + g.fp8_rope_off + fp8_rope_elem_off(slot, m, g.page_size));
}

// Block of 256 threads stores one fp32 latent row (c^KV then rotated k^R,
// held in LDS) into its page slot, converting or quantising per 1x128 tile.
__device__ void store_row(const CacheGeom& g, uint8_t* pg, int slot, const float* row) {
  const int tid = threadIdx.x, D = g.d_c + g.d_rope;
  if (g.dtype == MLA_F32) {
    for (int k = tid; k < D; k += blockDim.x) ((float*)pg)[(size_t)slot * D + k] = row[k];
  } else if (g.dtype == MLA_BF16) {
    for (int k = tid; k < D; k += blockDim.x) *(bf16_t*)(pg + bf16_page_off(slot, k, g.page_size)) = (bf16_t)row[k];
  } else {
    const int lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6, nt = g.d_c / 128;
    for (int tile = wave; tile < nt; tile += nw) {
      float v0 = row[tile * 128 + lane], v1 = row[tile * 128 + 64 + lane];
      float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
      float s = tile_scale(amax, g.dtype);
      pg[fp8_code_off(slot, tile * 128 + lane, g.page_size)] = f32_to_e4m3(v0 / s);
      pg[fp8_code_off(slot, tile * 128 + 64 + lane, g.page_size)] = f32_to_e4m3(v1 / s);
      if (lane == 0) ((float*)(pg + g.fp8_scale_off))[slot * nt + tile] = s;
    }
    for (int m = tid; m < g.d_rope; m += blockDim.x)
      *(bf16_t*)(pg + g.fp8_rope_off + fp8_rope_elem_off(slot, m, g.page_size)) = (bf16_t)row[g.d_c + m];
  }
}

// ------------------------------------------------------------ append / write
// MODE 0: row = [W_DKV; W_KR] h_r, then RoPE on the last d_rope entries.
// MODE 1: row = given [c_kv | k_rope] (k_rope already rotated).
template <typename AT, int MODE>
__global__ __launch_bounds__(256) void k_latent_row(int d_model, CacheGeom g, float theta,
                                                     const AT* h, const AT* k_rope,
                                                     const int32_t* seq_id, const int32_t* pos,
                                                     const AT* W_DKV, const AT* W_KR, uint8_t* pages,
                                                     const int32_t* bt, int max_pages) {
  extern __shared__ float row[];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = g.d_c + g.d_rope;
  const int p = pos[r];
  if (MODE == 0) {
    const AT* hr = h + (size_t)r * d_model;
    for (int col = wave; col < D; col += 4) {
      const AT* w = col < g.d_c ? W_DKV + (size_t)col * d_model : W_KR + (size_t)(col - g.d_c) * d_model;
      float acc = 0.0f;
      for (int k = lane; k < d_model; k += 64) acc += to_f32(hr[k]) * to_f32(w[k]);
      acc = wave_sum(acc);
      if (lane == 0) row[col] = acc;
    }
    __syncthreads();
    for (int m = tid; m < g.d_rope / 2; m += blockDim.x) {
      float cs, sn;
      rope_cs(p, m, g.d_rope, theta, &cs, &sn);
      float x0 = row[g.d_c + 2 * m], x1 = row[g.d_c + 2 * m + 1];
      row[g.d_c + 2 * m] = x0 * cs - x1 * sn;
      row[g.d_c + 2 * m + 1] = x0 * sn + x1 * cs;
    }
  } else {
    for (int k = tid; k < g.d_c; k += blockDim.x) row[k] = to_f32(h[(size_t)r * g.d_c + k]);
    for (int k = tid; k < g.d_rope; k += blockDim.x) row[g.d_c + k] = to_f32(k_rope[(size_t)r * g.d_rope + k]);
  }
  __syncthreads();
  uint8_t* pg = (uint8_t*)page_ptr(g, pages, bt, max_pages, seq_id[r], p);
  store_row(g, pg, p % g.page_size, row);
}

// ------------------------------------------------------------ Y = X W^T
// One wave per output element, lanes stride over K.  Y is fp32.
template <typename XT, typename WT>
__global__ __launch_bounds__(256) void k_gemm_xwT(int M, int N, int K, const XT* X, const WT* W, float* Y) {
  const int lane = threadIdx.x & 63;
  const long idx = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= (long)M * N) return;
  const int m = (int)(idx / N), n = (int)(idx % N);
  const XT* x = X + (size_t)m * K;
  const WT* w = W + (size_t)n * K;
  float acc = 0.0f;
  for (int k = lane; k < K; k += 64) acc += to_f32(x[k]) * to_f32(w[k]);
  acc = wave_sum(acc);
  if (lane == 0) Y[(size_t)m * N + n] = acc;
}

// Query RoPE part: qt[r,i,d_c:] = scale2 * RoPE(u[r,i,d_head:], p_j).
template <typename QT>
__global__ void k_qrope_generic(int H, int s_q, int d_head, int d_rope, int d_c, float theta, float scale2,
                                const int32_t* seqlens, const float* u, QT* qt) {
  const int ri = blockIdx.x, i = ri % H, r = ri / H, j = r % s_q, b = r / s_q;
  int p = seqlens[b] - s_q + j;
  if (p < 0) p = 0;
  const float* ur = u + ((size_t)r * H + i) * (d_head + d_rope) + d_head;
  QT* q = qt + ((size_t)r * H + i) * (d_c + d_rope) + d_c;
  for (int m = threadIdx.x; m < d_rope / 2; m += blockDim.x) {
    float cs, sn;
    rope_cs(p, m, d_rope, theta, &cs, &sn);
    float x0 = ur[2 * m], x1 = ur[2 * m + 1];
    q[2 * m] = from_f32<QT>(scale2 * (x0 * cs - x1 * sn));
    q[2 * m + 1] = from_f32<QT>(scale2 * (x0 * sn + x1 * cs));
  }
}

// Absorption (§2.1.1 Question 2): qt[r,i,c] = scale2 * sum_a W_UK[i*d_head+a][c] q^C[r,i,a].
template <typename QT, typename WT>
__global__ __launch_bounds__(256) void k_absorb_generic(int H, int d_head, int d_rope, int d_c, float scale2,
                                                         const float* u, const WT* W_UK, QT* qt) {
  const int ri = blockIdx.x, i = ri % H;
  const float* qc = u + (size_t)ri * (d_head + d_rope);
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
    float acc = 0.0f;
    for (int a = 0; a < d_head; ++a) acc += to_f32(W_UK[((size_t)i * d_head + a) * d_c + c]) * qc[a];
    qt[(size_t)ri * (d_c + d_rope) + c] = from_f32<QT>(scale2 * acc);
  }
}

__device__ float block_reduce(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = is_max ? wave_max(v) : wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < nw; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

// Split-KV attention for one (query row, head, split): online softmax in the
// exp2 domain (scores already carry tau*log2 e), partial output normalised by
// its own sum, log2-sum-exp2 beside it.  d_c <= 1024.
template <typename QT>
__global__ __launch_bounds__(256) void k_attn_generic(int H, int s_q, CacheGeom g, const QT* qt,
                                                       const uint8_t* pages, const int32_t* bt, int max_pages,
                                                       const int32_t* seqlens, int S, int pps,
                                                       float* opart, float* lpart) {
  extern __shared__ float sm[];
  const int D = g.d_c + g.d_rope;
  float* q = sm;
  float* pbuf = sm + D;
  float* red = pbuf + 256;
  const int tid = threadIdx.x;
  const int row = blockIdx.x, s = blockIdx.y;
  const int i = row % H, bj = row / H, j = bj % s_q, b = bj / s_q;
  for (int k = tid; k < D; k += 256) q[k] = to_f32(qt[(size_t)row * D + k]);
  __syncthreads();
  const int L = seqlens[b];
  int vis = L > 0 ? L - s_q + j + 1 : 0;
  if (vis < 0) vis = 0;
  const int ps = g.page_size;
  const int t_begin = s * pps * ps;
  const int t_end = min(vis, (s + 1) * pps * ps);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.0f;
  for (int t0 = t_begin; t0 < t_end; t0 += 256) {
    const int t = t0 + tid;
    float sc = -INFINITY;
    if (t < t_end) {
      const uint8_t* pg = page_ptr(g, pages, bt, max_pages, b, t);
      const int slot = t % ps;
      float a = 0.0f;
      for (int c = 0; c < g.d_c; ++c) a += q[c] * cache_lat(g, pg, slot, c);
      for (int mm = 0; mm < g.d_rope; ++mm) a += q[g.d_c + mm] * cache_rope(g, pg, slot, mm);
      sc = a;
    }
    const float m_new = fmaxf(m, block_reduce(sc, red, true));
    const float e = t < t_end ? exp2f(sc - m_new) : 0.0f;
    const float alpha = exp2f(m - m_new);
    l = l * alpha + block_reduce(e, red, false);
    pbuf[tid] = e;
    __syncthreads();
    for (int k = 0; k < 4; ++k) acc[k] *= alpha;
    const int n = min(256, t_end - t0);
    for (int tt = 0; tt < n; ++tt) {
      const uint8_t* pg = page_ptr(g, pages, bt, max_pages, b, t0 + tt);
      const int slot = (t0 + tt) % ps;
      const float pt = pbuf[tt];
      for (int k = 0; k < 4; ++k) {
        const int c = tid + 256 * k;
        if (c < g.d_c) acc[k] += pt * cache_lat(g, pg, slot, c);
      }
    }
    m = m_new;
    __syncthreads();
  }
  const size_t prow = (((size_t)b * S + s) * s_q + j) * H + i;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  for (int k = 0; k < 4; ++k) {
    const int c = tid + 256 * k;
    if (c < g.d_c) opart[prow * g.d_c + c] = acc[k] * inv;
  }
  if (tid == 0) lpart[prow] = l > 0.0f ? m + log2f(l) : -INFINITY;
}

// Merge the splits (log-sum-exp weights, empty splits skipped) and apply
// W^UV of the row's head: out = W^UV_i O_lat.
template <typename OT>
__global__ __launch_bounds__(256) void k_combine_generic(int batch, int H, int s_q, int S, int d_head, int d_c,
                                                          const uint8_t* ws, size_t lpart_off,
                                                          const OT* W_UV, OT* out, float* lse_out) {
  extern __shared__ float olat[];
  float* wsm = olat + d_c;  // S weights
  const bool pbf16 = ((const int32_t*)ws)[HDR_PDT] == MLA_BF16;
  const float* lpart = (const float*)(ws + lpart_off);
  const uint8_t* opart = ws + opart_offset(lpart_off, batch, S, s_q, H);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x, i = row % H, bj = row / H, j = bj % s_q, b = bj / s_q;
  auto prow = [&](int s) { return (((size_t)b * S + s) * s_q + j) * H + i; };
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, lpart[prow(s)]);
  float W = 0.0f;
  for (int s = tid; s < S; s += blockDim.x) {
    const float ls = lpart[prow(s)];
    const float w = ls == -INFINITY ? 0.0f : exp2f(ls - M);
    wsm[s] = w;
  }
  __syncthreads();
  for (int s = 0; s < S; ++s) W += wsm[s];
  const float invW = W > 0.0f ? 1.0f / W : 0.0f;
  for (int c = tid; c < d_c; c += blockDim.x) {
    float a = 0.0f;
    for (int s = 0; s < S; ++s)
      if (wsm[s] != 0.0f)
        a += wsm[s] * (pbf16 ? (float)((const bf16_t*)opart)[prow(s) * d_c + c] : ((const float*)opart)[prow(s) * d_c + c]);
    olat[c] = a * invW;
  }
  __syncthreads();
  for (int a = wave; a < d_head; a += 4) {
    const OT* w = W_UV + ((size_t)i * d_head + a) * d_c;
    float acc = 0.0f;
    for (int c = lane; c < d_c; c += 64) acc += to_f32(w[c]) * olat[c];
    acc = wave_sum(acc);
    if (lane == 0) out[(size_t)row * d_head + a] = from_f32<OT>(acc);
  }
  if (tid == 0 && lse_out) lse_out[row] = W > 0.0f ? (M + log2f(W)) * LN2 : -INFINITY;
}

__global__ void k_write_header(int32_t* hdr, int S, int pps, int batch, int s_q, int H, int d_c) {
  if (threadIdx.x == 0) {
    hdr[HDR_MAGIC] = WS_MAGIC; hdr[HDR_S] = S; hdr[HDR_PPS] = pps; hdr[HDR_BATCH] = batch;
    hdr[HDR_SQ] = s_q; hdr[HDR_H] = H; hdr[HDR_DC] = d_c; hdr[HDR_PDT] = MLA_F32;
  }
}

// ------------------------------------------------------------ launchers
hipError_t generic_append(const AppendArgs& a) {
  const size_t lds = (size_t)(a.g.d_c + a.g.d_rope) * 4;
  if (a.act == MLA_F32)
    MLA_TRY(launch(&k_latent_row<float, 0>, dim3(a.n_tok), dim3(256), lds, a.stream, a.d.d_model, a.g,
                       a.d.rope_theta, (const float*)a.h, (const float*)nullptr, a.seq_id, a.pos,
                       (const float*)a.W_DKV, (const float*)a.W_KR, a.pages, a.block_table, a.max_pages));
  else
    MLA_TRY(launch(&k_latent_row<bf16_t, 0>, dim3(a.n_tok), dim3(256), lds, a.stream, a.d.d_model, a.g,
                       a.d.rope_theta, (const bf16_t*)a.h, (const bf16_t*)nullptr, a.seq_id, a.pos,
                       (const bf16_t*)a.W_DKV, (const bf16_t*)a.W_KR, a.pages, a.block_table, a.max_pages));
  return hipSuccess;
}

hipError_t generic_write(const AppendArgs& a) {
  const size_t lds = (size_t)(a.g.d_c + a.g.d_rope) * 4;
  if (a.act == MLA_F32)
    MLA_TRY(launch(&k_latent_row<float, 1>, dim3(a.n_tok), dim3(256), lds, a.stream, a.d.d_model, a.g,
                       a.d.rope_theta, (const float*)a.h, (const float*)a.k_rope, a.seq_id, a.pos,
                       (const float*)nullptr, (const float*)nullptr, a.pages, a.block_table, a.max_pages));
  else
    MLA_TRY(launch(&k_latent_row<bf16_t, 1>, dim3(a.n_tok), dim3(256), lds, a.stream, a.d.d_model, a.g,
                       a.d.rope_theta, (const bf16_t*)a.h, (const bf16_t*)a.k_rope, a.seq_id, a.pos,
                       (const bf16_t*)nullptr, (const bf16_t*)nullptr, a.pages, a.block_table, a.max_pages));
  return hipSuccess;
}

hipError_t write_header(const DecodeArgs& a) {
  MLA_TRY(launch(&k_write_header, dim3(1), dim3(64), 0, a.stream, (int32_t*)(a.ws + a.L.header), a.S,
                     a.pages_per_split, a.batch, a.s_q, a.d.n_heads, a.d.d_c));
  return hipSuccess;
}

template <typename T>
static hipError_t generic_query_t(const DecodeArgs& a) {
  const mla_dims& d = a.d;
  const int R = a.batch * a.s_q, H = d.n_heads;
  const float scale2 = a.scale * LOG2E;
  float* u = (float*)(a.ws + a.L.u);
  T* qt = (T*)(a.ws + a.L.qt);
  const size_t nu = (size_t)R * H * (d.d_head + d.d_rope);
  if (a.W_DQ) {
    float* cq = (float*)(a.ws + a.L.cq_part);
    const long n1 = (long)R * d.d_cq;
    MLA_TRY(launch(&k_gemm_xwT<T, T>, dim3((unsigned)((n1 + 3) / 4)), dim3(256), 0, a.stream, R, d.d_cq,
                       d.d_model, (const T*)a.hq, (const T*)a.W_DQ, cq));
    MLA_TRY(launch(&k_gemm_xwT<float, T>, dim3((unsigned)((nu + 3) / 4)), dim3(256), 0, a.stream, R,
                       H * (d.d_head + d.d_rope), d.d_cq, (const float*)cq, (const T*)a.W_UQ, u));
  } else {
    MLA_TRY(launch(&k_gemm_xwT<T, T>, dim3((unsigned)((nu + 3) / 4)), dim3(256), 0, a.stream, R,
                       H * (d.d_head + d.d_rope), d.d_cq, (const T*)a.hq, (const T*)a.W_UQ, u));
  }
  MLA_TRY(launch(&k_qrope_generic<T>, dim3(R * H), dim3(64), 0, a.stream, H, a.s_q, d.d_head, d.d_rope, d.d_c,
                     d.rope_theta, scale2, a.seqlens, (const float*)u, qt));
  MLA_TRY(launch(&k_absorb_generic<T, T>, dim3(R * H), dim3(256), 0, a.stream, H, d.d_head, d.d_rope, d.d_c,
                     scale2, (const float*)u, (const T*)a.W_UK, qt));
  return hipSuccess;
}

template <typename T>
static hipError_t generic_attention_t(const DecodeArgs& a) {
  const mla_dims& d = a.d;
  const int R = a.batch * a.s_q, H = d.n_heads;
  const size_t lds = (size_t)(d.d_c + d.d_rope + 256 + 8) * 4;
  MLA_TRY(launch(&k_attn_generic<T>, dim3(R * H, a.S), dim3(256), lds, a.stream, H, a.s_q, a.g,
                     (const T*)(a.ws + a.L.qt), a.pages, a.block_table, a.max_pages, a.seqlens, a.S,
                     a.pages_per_split, (float*)(a.ws + a.L.opart), (float*)(a.ws + a.L.lpart)));
  return hipSuccess;
}

hipError_t generic_query(const DecodeArgs& a) {
  hipError_t e = write_header(a);
  if (e != hipSuccess) return e;
  return a.act == MLA_F32 ? generic_query_t<float>(a) : generic_query_t<bf16_t>(a);
}

hipError_t generic_attention(const DecodeArgs& a) {
  // the header is rewritten so that an attend-only call after a query call
  // with other arguments still leaves a consistent plan for the combine
  hipError_t e = write_header(a);
  if (e != hipSuccess) return e;
  return a.act == MLA_F32 ? generic_attention_t<float>(a) : generic_attention_t<bf16_t>(a);
}


// fp32 -> bf16 (round to nearest even), elementwise.
__global__ __launch_bounds__(256) void k_f32_to_bf16(long n, const float* __restrict__ x, bf16_t* __restrict__ y) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = (bf16_t)x[i];
}

// y = W^O o on the VALU: one wave per output element, fp32 accumulation;
// bf16 results go through an fp32 buffer in the workspace.
hipError_t generic_out_project(const OutProjArgs& a) {
  const long MN = (long)a.rows * a.N;
  const dim3 grid((unsigned)((MN + 3) / 4));
  if (a.act == MLA_F32)
    return launch(&k_gemm_xwT<float, float>, grid, dim3(256), 0, a.stream, a.rows, a.N, a.K, (const float*)a.o,
                  (const float*)a.W_O, (float*)a.y);
  float* tmp = (float*)a.ws;
  MLA_TRY(launch(&k_gemm_xwT<bf16_t, bf16_t>, grid, dim3(256), 0, a.stream, a.rows, a.N, a.K,
                 (const bf16_t*)a.o, (const bf16_t*)a.W_O, tmp));
  return launch(&k_f32_to_bf16, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, a.stream, MN,
                (const float*)tmp, (bf16_t*)a.y);
}

hipError_t generic_combine(const CombineArgs& a) {
  const mla_dims& d = a.d;
  const int R = a.batch * a.s_q;
  const size_t lds = (size_t)(d.d_c + a.S) * 4;
  if (a.act == MLA_F32)
    MLA_TRY(launch(&k_combine_generic<float>, dim3(R * d.n_heads), dim3(256), lds, a.stream, a.batch,
                       d.n_heads, a.s_q, a.S, d.d_head, d.d_c, (const uint8_t*)a.ws, a.L.lpart, (const float*)a.W_UV,
                       (float*)a.out, a.lse_out));
  else
    MLA_TRY(launch(&k_combine_generic<bf16_t>, dim3(R * d.n_heads), dim3(256), lds, a.stream, a.batch,
                       d.n_heads, a.s_q, a.S, d.d_head, d.d_c, (const uint8_t*)a.ws, a.L.lpart, (const bf16_t*)a.W_UV,
                       (bf16_t*)a.out, a.lse_out));
  return hipSuccess;
}

}  // namespace mla

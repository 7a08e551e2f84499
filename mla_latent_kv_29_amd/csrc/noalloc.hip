// The decode step (mla_decode, then mla_combine) for callers that cannot
// allocate device memory: its workspace lives in a file-scope device array
// instead of a caller's buffer.  Same kernels as the two entry points.
//
// `scratch` is a host-side stand-in in host code, not a device address.
// Each device's address of the array is taken once, on the first call on
// that device (with that device current), and only that pointer is handed
// to kernels.
#include <mutex>
#include "internal.hpp"

namespace mla {
namespace {

static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
uint8_t* g_ptr[MAX_DEVICES];  // per device: the array's device address (null until taken)

hipError_t scratch_ptr(uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = (uint8_t*)p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

// Workspace of the MFMA path inside the array: the regions of ws_layout that
// its kernels touch, with the split partials sized for their bf16 element
// (the attention writes bf16; the layout of the general entry points sizes
// them for the fp32 of the generic path).  The partials follow the lse
// values, as the combine expects.
WsLayout noalloc_layout(const mla_dims& d, int batch, int s_q, int S) {
  const size_t R = (size_t)batch * s_q, H = d.n_heads;
  WsLayout w;
  size_t o = 0;
  w.header = o;  o = align256(o + WS_HEADER_INTS * 4);
  w.cq_part = o; o = align256(o + (size_t)KSPLIT_MAX * R * d.d_cq * 4);
  w.cq = o;      o = align256(o + R * d.d_cq * 2);
  w.u = o;       // not used on the MFMA path
  w.qt = o;      o = align256(o + R * H * (d.d_c + d.d_rope) * 2);
  w.olat = o;    o = align256(o + R * H * d.d_c * 2);
  w.lpart = o;   o = align256(o + (size_t)batch * S * s_q * H * 4);
  w.opart = o;   o = align256(o + (size_t)batch * S * s_q * H * d.d_c * 2);
  w.total = o;
  return w;
}

hipError_t noalloc_decode_step(DecodeArgs& a, CombineArgs& c) {
  uint8_t* ws = nullptr;
  MLA_TRY(scratch_ptr(&ws));
  a.ws = ws;
  c.ws = ws;
  MLA_TRY(fast_query(a));
  MLA_TRY(fast_attention(a));
  return fast_combine(c);
}

}  // namespace mla

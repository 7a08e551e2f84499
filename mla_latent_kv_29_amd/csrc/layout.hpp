// Paged latent-cache layouts shared by every kernel that reads or writes a
// page.  Host and device.
//
// BF16 pages are stored chunk-major: the 576 (d_c + d_rope) channels of a
// token are cut into 16-byte chunks of 8 channels, and chunk C of all
// page_size tokens is stored together; inside that block, token t sits at
// slot t ^ (4 * (C % 4)).  A page can therefore be copied to LDS verbatim and
// read there without bank conflicts both row-wise (8 channels of 16 tokens,
// the QK^T operand) and column-wise (4 tokens x 16 channels, the transposed
// PV operand).
//
// FP8 pages hold, in order: E4M3 codes in the same chunk-major arrangement
// with 16-channel chunks (16 bytes), the fp32 scales [page_size][d_c/128], and
// the bf16 k^R rows [page_size][d_rope] in their own chunk-major block
// (8-channel chunks).
//
// F32 pages are plain row-major [page_size][d_c + d_rope].
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Byte offset of channel ch of token t inside a BF16 page.
__host__ __device__ __forceinline__ size_t bf16_page_off(int t, int ch, int page_size) {
  const int C = ch >> 3;
  return 16 * ((size_t)C * page_size + (t ^ (4 * (C & 3)))) + 2 * (ch & 7);
}

// Byte offset of latent channel ch (< d_c) of token t inside an FP8 page.
__host__ __device__ __forceinline__ size_t fp8_code_off(int t, int ch, int page_size) {
  const int C = ch >> 4;
  return 16 * ((size_t)C * page_size + (t ^ (4 * (C & 3)))) + (ch & 15);
}

// Byte offset of rope channel m (< d_rope) of token t inside the rope block of
// an FP8 page (add the block's offset).
__host__ __device__ __forceinline__ size_t fp8_rope_elem_off(int t, int m, int page_size) {
  return bf16_page_off(t, m, page_size);
}

}  // namespace mla

// Paged latent-cache layouts shared by every kernel that reads or writes a
// page.  Host and device.
//
// BF16 pages are stored chunk-major: the 576 (d_c + d_rope) channels of a
// token are cut into 16-byte chunks of 8 channels, and chunk C of all
// page_size tokens is stored together; inside that block, token t sits at
// slot t ^ slot_x(C), slot_x(C) = 4 * ((4 - C % 4) % 4), i.e. 0, 12, 8, 4.
// A page can therefore be copied to LDS verbatim and read there without bank
// conflicts both row-wise (8 channels of 16 tokens from four consecutive
// chunks, the score operand) and column-wise (4 tokens x 16 channels, the
// transposed P.V operand); both properties were measured on gfx950, where
// the plainer 4 * (C % 4) leaves the row-wise read two-way conflicted.
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

// Token-slot XOR of chunk C (see above).
__host__ __device__ __forceinline__ constexpr int slot_x(int C) { return 4 * ((4 - (C & 3)) & 3); }

// Byte offset of channel ch of token t inside a BF16 page.
__host__ __device__ __forceinline__ size_t bf16_page_off(int t, int ch, int page_size) {
  const int C = ch >> 3;
  return 16 * ((size_t)C * page_size + (t ^ slot_x(C))) + 2 * (ch & 7);
}

// Byte offset of latent channel ch (< d_c) of token t inside an FP8 page.
__host__ __device__ __forceinline__ size_t fp8_code_off(int t, int ch, int page_size) {
  const int C = ch >> 4;
  return 16 * ((size_t)C * page_size + (t ^ slot_x(C))) + (ch & 15);
}

// Byte offset of rope channel m (< d_rope) of token t inside the rope block of
// an FP8 page (add the block's offset).
__host__ __device__ __forceinline__ size_t fp8_rope_elem_off(int t, int m, int page_size) {
  return bf16_page_off(t, m, page_size);
}

}  // namespace mla

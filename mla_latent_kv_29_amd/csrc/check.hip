// Device-side check of the decode metadata that the host validation cannot
// see: sequence lengths and the block-table entries of the pages a sequence
// uses live in device memory, and an out-of-range page id would make the
// cache copies read outside the page pool.  One block walks the whole
// (batch, page) table; the counts meet in LDS and one thread stores them.
#include "internal.hpp"

namespace mla {
namespace {

__global__ __launch_bounds__(256) void k_check_metadata(int batch, int max_pages, int page_size, int num_pages,
                                                        const int32_t* __restrict__ bt,
                                                        const int32_t* __restrict__ seqlens, int32_t* __restrict__ bad) {
  __shared__ int n_len, n_page;
  if (threadIdx.x == 0) n_len = n_page = 0;
  __syncthreads();
  int my_len = 0, my_page = 0;
  const long cap = (long)max_pages * page_size;
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    const int L = seqlens[b];
    my_len += L < 0 || L > cap;
  }
  const long total = (long)batch * max_pages;
  for (long e = threadIdx.x; e < total; e += blockDim.x) {
    const int b = (int)(e / max_pages), p = (int)(e % max_pages);
    long L = seqlens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    if ((long)p * page_size < L) {  // a page the sequence uses
      const int id = bt[e];
      my_page += id < 0 || id >= num_pages;
    }
  }
  if (my_len) atomicAdd(&n_len, my_len);
  if (my_page) atomicAdd(&n_page, my_page);
  __syncthreads();
  if (threadIdx.x == 0) {
    bad[0] = n_len;
    bad[1] = n_page;
  }
}

}  // namespace

hipError_t check_metadata(int batch, int max_pages, int page_size, int num_pages, const int32_t* bt,
                          const int32_t* seqlens, int32_t* bad, hipStream_t st) {
  return launch(&k_check_metadata, dim3(1), dim3(256), 0, st, batch, max_pages, page_size, num_pages, bt, seqlens,
                bad);
}

}  // namespace mla

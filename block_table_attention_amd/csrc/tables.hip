// Block-table transforms at the one point where allocator tables become
// kernel tables ("M5.3 - KV Memory Layout and Exact Reuse", 0x0AB and 0x0AC).
//
//  * expansion: allocator blocks of P_a = q P_k tokens viewed as kernel blocks
//    of P_k tokens -- allocator id a becomes kernel ids a q .. a q + q - 1 in
//    place, so row r of width n becomes a row of width n q; negative (padding)
//    entries stay -1.
//  * packing: a dense [B, width] table becomes one array of each row's first
//    n_r entries back to back, n_r = row_offsets[r + 1] - row_offsets[r].
// One thread per output entry; both are bandwidth-trivial, single launches.
#include "pba_internal.h"

namespace pba {

__global__ __launch_bounds__(256) void expand_tables_kernel(const int32_t* __restrict__ src,
                                                            int64_t n_src, int32_t split_log2,
                                                            int32_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_dst = n_src << split_log2;
  if (i >= n_dst) return;
  const int32_t a = src[i >> split_log2];
  const int32_t sub = (int32_t)(i & ((1 << split_log2) - 1));
  dst[i] = a < 0 ? -1 : (a << split_log2) + sub;
}

__global__ __launch_bounds__(256) void pack_tables_kernel(const int32_t* __restrict__ src,
                                                          int32_t width,
                                                          const int64_t* __restrict__ offsets,
                                                          int32_t* __restrict__ dst) {
  const int r = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t o0 = offsets[r];
  const int64_t n = offsets[r + 1] - o0;
  if (j >= width || j >= n) return;
  dst[o0 + j] = src[(int64_t)r * width + j];
}

hipError_t launch_expand_tables(const int32_t* src, int64_t n_src, int split_log2, int32_t* dst,
                                hipStream_t stream) {
  const int64_t n_dst = n_src << split_log2;
  const unsigned blocks = (unsigned)((n_dst + 255) / 256);
  hipLaunchKernelGGL(expand_tables_kernel, dim3(blocks), dim3(256), 0, stream, src, n_src,
                     split_log2, dst);
  return hipGetLastError();
}

hipError_t launch_pack_tables(const int32_t* src, int32_t batch, int32_t width,
                              const int64_t* offsets, int32_t* dst, hipStream_t stream) {
  const dim3 grid((unsigned)((width + 255) / 256), (unsigned)batch);
  hipLaunchKernelGGL(pack_tables_kernel, grid, dim3(256), 0, stream, src, width, offsets, dst);
  return hipGetLastError();
}

}  // namespace pba

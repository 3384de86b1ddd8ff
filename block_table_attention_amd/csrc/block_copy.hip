// block_copy: the copy-on-write before divergence.  Each (src, dst) pair copies
// the whole physical block, K and V, every kv head, bit for bit ("M5.3 - KV
// Memory Layout and Exact Reuse", 0x04C: one fused block-copy launch over many
// pairs; 0x05A-0x05D).  One work-group copies one (pair, kv head, K|V) tile of
// P * d scalars, which is contiguous in both the K and the V tile layout, with
// 16-byte loads and stores, four in flight per lane.
#include "pba_internal.h"

namespace pba {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void block_copy_kernel(CopyArgs a) {
  const int64_t pair = blockIdx.x;
  const int h = blockIdx.y >> 1;
  const bool is_v = blockIdx.y & 1;
  const int64_t s = a.src[pair];
  const int64_t d = a.dst[pair];
  char* base = static_cast<char*>(is_v ? a.v : a.k);
  const int64_t sb = is_v ? a.v_sb : a.k_sb;
  const int64_t sh = is_v ? a.v_sh : a.k_sh;
  const u32x4* __restrict__ from = reinterpret_cast<const u32x4*>(base + (s * sb + h * sh) * a.esize);
  u32x4* __restrict__ to = reinterpret_cast<u32x4*>(base + (d * sb + h * sh) * a.esize);
  const int64_t n16 = a.tile_bytes / 16;
  constexpr int UNROLL = 4;
  for (int64_t i = threadIdx.x; i < n16; i += 256 * UNROLL) {
    u32x4 r[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if (i + u * 256 < n16) r[u] = __builtin_nontemporal_load(from + i + u * 256);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if (i + u * 256 < n16) to[i + u * 256] = r[u];
  }
}

hipError_t launch_block_copy(const CopyArgs& a, int64_t n_pairs, int kv_heads, hipStream_t stream) {
  dim3 grid((unsigned)n_pairs, (unsigned)(2 * kv_heads));
  hipLaunchKernelGGL(block_copy_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pba

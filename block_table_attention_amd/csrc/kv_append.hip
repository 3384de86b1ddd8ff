// kv_append: scatter new tokens' K/V rows into their physical slots.
//
// slot s -> (block s div P, offset s mod P) ("M5.3 - KV Memory Layout and
// Exact Reuse", 0x03C-0x03D); the rows are bit copies, so NaN payloads and
// signed zeros survive.  One 64-lane wave handles 64 consecutive tokens of one
// kv head:
//   K: the tile is token major, so a row is one contiguous run of d scalars;
//      lanes walk (token, 16-byte chunk) pairs, which keeps both the reads of
//      k_new and the writes into the pool coalesced.
//   V: the tile is dim major ([d][P]), so a row becomes d scalars P apart.
//      Lane i owns token i: it reads its row 16 bytes at a time and writes each
//      scalar into its dim's run; for a prefill whose slots are consecutive the
//      64 lanes of one store fill 64 neighbouring positions of that run.
#include "pba_internal.h"

namespace pba {

template <typename E>
__global__ __launch_bounds__(64) void kv_append_kernel(AppendArgs a) {
  const int lane = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  const int D = a.head_dim;
  const int P = 1 << a.log2P;
  const int chunks = D * (int)sizeof(E) / 16;  // 16-byte pieces per row
  constexpr int EPC = 16 / sizeof(E);           // scalars per piece

  // K rows.
  const char* knew = static_cast<const char*>(a.k_new);
  char* kpool = static_cast<char*>(a.k);
  for (int idx = lane; idx < 64 * chunks; idx += 64) {
    const int64_t i = i0 + idx / chunks;
    const int c = idx % chunks;
    if (i >= a.n) break;
    const int64_t s = a.slots[i];
    if (s < 0) continue;
    const int64_t blk = s >> a.log2P;
    const int64_t off = s & (P - 1);
    const uint4 val = *reinterpret_cast<const uint4*>(
        knew + ((i * a.kv_heads + h) * D) * (int64_t)sizeof(E) + c * 16);
    *reinterpret_cast<uint4*>(kpool + (blk * a.k_sb + h * a.k_sh + off * D) * (int64_t)sizeof(E) +
                              c * 16) = val;
  }

  // V rows, transposed into the dim-major tile.
  const int64_t i = i0 + lane;
  if (i >= a.n) return;
  const int64_t s = a.slots[i];
  if (s < 0) return;
  const int64_t blk = s >> a.log2P;
  const int64_t off = s & (P - 1);
  const char* vrow = static_cast<const char*>(a.v_new) + ((i * a.kv_heads + h) * D) * (int64_t)sizeof(E);
  E* vdst = static_cast<E*>(a.v) + blk * a.v_sb + h * a.v_sh + off;
  for (int c = 0; c < chunks; ++c) {
    union {
      uint4 u;
      E e[EPC];
    } piece;
    piece.u = *reinterpret_cast<const uint4*>(vrow + c * 16);
#pragma unroll
    for (int e = 0; e < EPC; ++e) vdst[(int64_t)(c * EPC + e) * P] = piece.e[e];
  }
}

hipError_t launch_kv_append(const AppendArgs& a, int esize, hipStream_t stream) {
  const int64_t tiles = (a.n + 63) / 64;
  dim3 grid((unsigned)tiles, (unsigned)a.kv_heads);
  if (esize == 2)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pba

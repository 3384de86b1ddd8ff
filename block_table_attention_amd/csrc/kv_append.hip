// kv_append: scatter new tokens' K/V rows into their physical slots.
//
// slot s -> (block s div P, offset s mod P) ("M5.3 - KV Memory Layout and
// Exact Reuse", 0x03C-0x03D); the rows are bit copies, so NaN payloads and
// signed zeros survive.  One thread moves one 16-byte piece of one token's row
// of one kv head, so every load is independent of every store.  The piece and
// the slot are both requested before the slot is tested (the piece is in
// bounds for every task), so they share one memory round trip:
//   K tasks (piece fastest): the K tile is token major, a row is one run of d
//      scalars, and neighbouring lanes read and write neighbouring pieces;
//   V tasks (token fastest): the V tile is dim major ([d][P]), a row becomes d
//      scalars P apart; neighbouring lanes hold neighbouring tokens, so when a
//      prefill's slots are consecutive, the lanes of one store fill
//      neighbouring positions of the same dim run.
#include "pba_internal.h"

namespace pba {

template <typename E>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  constexpr int EPC = 16 / sizeof(E);  // scalars per 16-byte piece
  const int D = a.head_dim;
  const int H = a.kv_heads;
  const int pieces = D / EPC;
  const int64_t per_kind = a.n * H * pieces;
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= 2 * per_kind) return;
  const int P = 1 << a.log2P;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

  if (t < per_kind) {
    const int c = (int)(t % pieces);
    const int64_t rest = t / pieces;
    const int h = (int)(rest % H);
    const int64_t i = rest / H;
    const u32x4 val = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.k_new) +
                                                      (i * H + h) * D + c * EPC);
    const int64_t s = a.slots[i];
    asm volatile("" ::"v"(val), "v"(s));  // keeps the piece load above the test
    if (s < 0) return;
    const int64_t blk = s >> a.log2P, off = s & (P - 1);
    *reinterpret_cast<u32x4*>(static_cast<E*>(a.k) + blk * a.k_sb + h * a.k_sh + off * D +
                              c * EPC) = val;
  } else {
    t -= per_kind;
    const int64_t i = t % a.n;
    const int64_t rest = t / a.n;
    const int h = (int)(rest % H);
    const int c = (int)(rest / H);
    union {
      u32x4 u;
      E e[EPC];
    } piece;
    piece.u = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.v_new) + (i * H + h) * D +
                                              c * EPC);
    const int64_t s = a.slots[i];
    asm volatile("" ::"v"(piece.u), "v"(s));
    if (s < 0) return;
    const int64_t blk = s >> a.log2P, off = s & (P - 1);
    E* dst = static_cast<E*>(a.v) + blk * a.v_sb + h * a.v_sh + (int64_t)(c * EPC) * P + off;
#pragma unroll
    for (int e = 0; e < EPC; ++e) dst[(int64_t)e * P] = piece.e[e];
  }
}

hipError_t launch_kv_append(const AppendArgs& a, int esize, hipStream_t stream) {
  const int64_t tasks = 2 * a.n * a.kv_heads * (a.head_dim * esize / 16);
  const dim3 grid((unsigned)((tasks + 255) / 256));
  if (esize == 2)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pba

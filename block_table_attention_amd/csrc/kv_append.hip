// kv_append: scatter new tokens' K/V rows into their physical slots.
//
// slot s -> (block s div P, offset s mod P) ("M5.3 - KV Memory Layout and
// Exact Reuse", 0x03C-0x03D); the rows are bit copies, so NaN payloads and
// signed zeros survive.  The pieces and the slots are requested before any
// slot is tested (the pieces are in bounds for every task), so they share one
// memory round trip:
//   K tasks (piece fastest): one thread moves one 16-byte piece (E = 16 /
//      sizeof scalar scalars) of one token's row of one kv head; the K tile is
//      token major, so neighbouring lanes read and write neighbouring pieces;
//   V tasks of an append of fewer than kVBlockedMinTokens tokens (token
//      fastest): one thread moves one 16-byte piece of one token's V row; the
//      V tile is dim major ([d][P]), so the row becomes d scalars P apart.
//   V tasks of a larger append (piece fastest, then 8 token groups, then
//      head): one thread moves an E x E block -- piece c of the rows of E
//      consecutive tokens -- and transposes it in registers.  When the E
//      tokens' slots are consecutive and start at a multiple of E (a
//      prefill), each of the E dims becomes one 16-byte store; otherwise the
//      block's scalars are stored one by one.  Neighbouring lanes read
//      neighbouring pieces of a row, and the 8 groups of 8 E consecutive
//      tokens sit in two neighbouring waves, so a prefill's 128-byte dim runs
//      are written whole by one work-group (one XCD's L2) instead of in
//      pieces by work-groups on several XCDs.
#include "append_internal.h"
#include "pba_internal.h"

namespace pba {

template <typename E>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  constexpr int EPC = 16 / sizeof(E);  // scalars per 16-byte piece
  const int D = a.head_dim;
  const int H = a.kv_heads;
  const int pieces = D / EPC;
  const int64_t per_kind = a.n * H * pieces;
  const bool blocked = a.n >= kVBlockedMinTokens;
  const int64_t v_tasks = blocked ? v_append_groups<E>(a.n) * H * pieces : per_kind;
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= per_kind + v_tasks) return;
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
  } else if (!blocked) {
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
  } else {
    t -= per_kind;
    const int c = (int)(t % pieces);
    const int64_t r1 = t / pieces;
    const int gl = (int)(r1 % kVGroupRun);
    const int64_t r2 = r1 / kVGroupRun;
    const int h = (int)(r2 % H);
    const int64_t i0 = ((r2 / H) * kVGroupRun + gl) * EPC;  // first token of the group
    if (i0 >= a.n) return;
    append_v_block<E>(static_cast<const E*>(a.v_new) + (int64_t)h * D + c * EPC, (int64_t)H * D,
                      a.slots, i0, a.n, static_cast<E*>(a.v) + h * a.v_sh + (int64_t)(c * EPC) * P,
                      a.v_sb, a.log2P);
  }
}

hipError_t launch_kv_append(const AppendArgs& a, int esize, hipStream_t stream) {
  const int64_t per_head = a.head_dim * esize / 16;  // 16-byte pieces per row
  const int64_t groups = a.n < kVBlockedMinTokens ? a.n
                         : esize == 2               ? v_append_groups<uint16_t>(a.n)
                                                    : v_append_groups<uint32_t>(a.n);
  const int64_t tasks = (a.n + groups) * a.kv_heads * per_head;
  const dim3 grid((unsigned)((tasks + 255) / 256));
  if (esize == 2)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pba

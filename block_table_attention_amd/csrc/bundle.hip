// Cache groups with a layer axis: one launch writes new tokens into every
// layer of every group, one launch copies whole blocks of every layer of
// every group ("M5.3 - KV Memory Layout and Exact Reuse", 0x03B: a group's
// token row spans its layers, each group has its own pool; 0x04C: one fused
// block-copy launch over many pairs and layers; 0x04E and 0x05C: the new row
// is written, and the tail bundle copied, in every group).
//
// Work is flattened over the groups: group g owns the tasks (or work-groups)
// [task0_g, task0_{g+1}), and a thread finds its group by comparing its index
// with the at most eight starts held in the kernel arguments.
#include "append_internal.h"
#include "bundle_internal.h"

namespace pba {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Append, per group:
//   K tasks (piece fastest): one thread moves one 16-byte piece of one
//      (token, layer, head) row; a K row is head_dim consecutive scalars of
//      the token-major tile, so neighbouring lanes copy neighbouring pieces.
//   V tasks, appends of fewer than kVBlockedMinTokens tokens (token
//      fastest): one thread moves one 16-byte piece of one row into the
//      dim-major V tile, head_dim scalars P apart;
//   V tasks, larger appends (piece, then 8 token groups, then head, then layer
//      fastest): one thread moves piece c of 16 / es consecutive tokens' rows,
//      as kv_append does (append_v_block).
__global__ __launch_bounds__(256) void kv_append_bundle_kernel(BundleAppendArgs a) {
  const int32_t t = (int32_t)(blockIdx.x * 256u + threadIdx.x);
  if (t >= a.total) return;
  int gi = 0;
#pragma unroll
  for (int j = 1; j < PBA_MAX_GROUPS; ++j)
    if (j < a.n_groups && t >= a.g[j].task0) gi = j;
  const GroupAppend& G = a.g[gi];
  const int es = G.esize;
  const int D = G.head_dim;
  const int H = G.heads;
  const int L = G.layers;
  const int pieces = D * es / 16;
  const int P = 1 << G.log2P;
  int32_t local = t - G.task0;
  if (local < G.per_kind) {
    const int c = local % pieces;
    int32_t r = local / pieces;
    const int h = r % H;
    r /= H;
    const int l = r % L;
    const int i = r / L;
    // The piece and the slot go out together (the piece is in bounds for every task).
    const u32x4 val = *reinterpret_cast<const u32x4*>(
        G.k_new + ((((int64_t)i * L + l) * H + h) * D) * es + 16 * c);
    const int64_t s = G.slots[i];
    asm volatile("" ::"v"(val), "v"(s));  // keeps the piece load above the test
    if (s < 0) return;
    const int64_t blk = s >> G.log2P, off = s & (P - 1);
    *reinterpret_cast<u32x4*>(G.k + (l * G.k_sl + blk * G.k_sb + h * G.k_sh + off * D) * es +
                              16 * c) = val;
  } else if (a.n < kVBlockedMinTokens) {
    local -= G.per_kind;
    const int i = local % a.n;
    int32_t r = local / a.n;
    const int h = r % H;
    r /= H;
    const int l = r % L;
    const int c = r / L;
    const u32x4 piece = *reinterpret_cast<const u32x4*>(
        G.v_new + ((((int64_t)i * L + l) * H + h) * D) * es + 16 * c);
    const int64_t s = G.slots[i];
    asm volatile("" ::"v"(piece), "v"(s));
    if (s < 0) return;
    const int64_t blk = s >> G.log2P, off = s & (P - 1);
    const int epc = 16 / es;
    const int64_t e0 = l * G.v_sl + blk * G.v_sb + h * G.v_sh + (int64_t)(c * epc) * P + off;
    if (es == 2) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(G.v) + e0;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[(int64_t)e * P] = (uint16_t)(piece[e >> 1] >> (16 * (e & 1)));
    } else {
      uint32_t* dst = reinterpret_cast<uint32_t*>(G.v) + e0;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(int64_t)e * P] = piece[e];
    }
  } else {
    // V: piece c of a group of 16 / es tokens, the groups in runs of 8 inside
    // two neighbouring waves (append_v_block).
    local -= G.per_kind;
    if (local >= G.v_tasks) return;
    const int c = local % pieces;
    int32_t r = local / pieces;
    const int gl = r % kVGroupRun;
    r /= kVGroupRun;
    const int h = r % H;
    r /= H;
    const int l = r % L;
    const int64_t i0 = ((int64_t)(r / L) * kVGroupRun + gl) * (16 / es);
    if (i0 >= a.n) return;
    const int64_t row = (int64_t)L * H * D;                       // scalars between tokens
    const int64_t src0 = ((int64_t)l * H + h) * D + (int64_t)c * (16 / es);
    const int64_t dst0 = l * G.v_sl + h * G.v_sh + (int64_t)c * (16 / es) * P;
    if (es == 2)
      append_v_block<uint16_t>(reinterpret_cast<const uint16_t*>(G.v_new) + src0, row, G.slots,
                               i0, a.n, reinterpret_cast<uint16_t*>(G.v) + dst0, G.v_sb, G.log2P);
    else
      append_v_block<uint32_t>(reinterpret_cast<const uint32_t*>(G.v_new) + src0, row, G.slots,
                               i0, a.n, reinterpret_cast<uint32_t*>(G.v) + dst0, G.v_sb, G.log2P);
  }
}

// Copy: one work-group copies one (pair, K|V, layer, head) tile of P * head_dim
// scalars, contiguous in both tile layouts, with 16-byte loads and stores.
// Heads vary fastest, then layers, so neighbouring work-groups copy
// neighbouring tiles of one block (adjacent memory in a block-major group).
__global__ __launch_bounds__(256) void block_copy_bundle_kernel(BundleCopyArgs a) {
  const int32_t w = (int32_t)blockIdx.x;
  int gi = 0;
#pragma unroll
  for (int j = 1; j < PBA_MAX_GROUPS; ++j)
    if (j < a.n_groups && w >= a.g[j].wg0) gi = j;
  const GroupCopy& G = a.g[gi];
  int32_t r = w - G.wg0;
  const int h = r % G.heads;
  r /= G.heads;
  const int l = r % G.layers;
  r /= G.layers;
  const bool is_v = r & 1;
  const int32_t pair = r >> 1;
  const int64_t s = G.src[pair];
  const int64_t d = G.dst[pair];
  char* base = is_v ? G.v : G.k;
  const int64_t sl = is_v ? G.v_sl : G.k_sl;
  const int64_t sb = is_v ? G.v_sb : G.k_sb;
  const int64_t sh = is_v ? G.v_sh : G.k_sh;
  const int64_t tile = l * sl + h * sh;
  const u32x4* __restrict__ from = reinterpret_cast<const u32x4*>(base + tile + s * sb);
  u32x4* __restrict__ to = reinterpret_cast<u32x4*>(base + tile + d * sb);
  const int n16 = G.tile16;
  constexpr int UNROLL = 4;
  for (int i = threadIdx.x; i < n16; i += 256 * UNROLL) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if (i + u * 256 < n16) v[u] = __builtin_nontemporal_load(from + i + u * 256);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if (i + u * 256 < n16) to[i + u * 256] = v[u];
  }
}

hipError_t launch_kv_append_bundle(const BundleAppendArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.total + 255) / 256));
  hipLaunchKernelGGL(kv_append_bundle_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_block_copy_bundle(const BundleCopyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(block_copy_bundle_kernel, dim3((unsigned)a.total), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pba

// Internal declarations shared by the libpba.so translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pba.h"

namespace pba {

// Argument bundle of the append kernel (all pointers device, strides elements).
struct AppendArgs {
  void* k;
  void* v;
  int64_t k_sb, k_sh, v_sb, v_sh;
  const int64_t* slots;
  const void* k_new;
  const void* v_new;
  int64_t n;
  int32_t log2P;
  int32_t head_dim;
  int32_t kv_heads;
};

struct CopyArgs {
  void* k;
  void* v;
  int64_t k_sb, k_sh, v_sb, v_sh;
  const int32_t* src;
  const int32_t* dst;
  int64_t tile_bytes;  // P * head_dim * scalar bytes
  int32_t esize;
};

// How a decode row finds its blocks: a dense table row, a ragged table row,
// or no table (contiguous slots: `tables` holds one slot index per request and
// `max_blocks` the blocks of a slot).
constexpr int kTablesDense = 0;
constexpr int kTablesRagged = 1;
constexpr int kTablesContiguous = 2;

// Decode: one work-group per (partition, kv head, request).  The decode kernel
// takes k_sb and k_sh as int32 (the host rejects larger strides).
struct DecodeArgs {
  const void* k;
  const void* v;
  int64_t k_sb, k_sh, v_sb, v_sh;
  const void* q;
  const int32_t* tables;
  const int32_t* seq_lens;
  float* out;
  float* lse;
  float* ws_ml;  // [B][H_q][n_parts][2]: running max (log2 domain), sum
  float* ws_u;   // [B][H_q][n_parts][D]: unnormalised output
  int32_t* counters;  // [B][H_kv]: partitions finished; zero between calls
  const int64_t* row_offsets;  // ragged tables: row r = tables[row_offsets[r] ..
                               // row_offsets[r + 1]); nullptr for dense tables
  int32_t table_mode;  // kTablesDense / kTablesRagged / kTablesContiguous
  int32_t max_blocks;
  int32_t num_blocks;  // pool size: clamp for block ids read ahead of the length
  int32_t log2P;
  int32_t G;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t batch;
  int32_t part_tokens;
  int32_t n_parts;
  float scale_log2;  // scale * log2(e): scores live in the log2 domain
  int32_t split_log2;  // kernel view of an allocator pool: tiles of P << split rows
  // Fused append (nullptr: none): row r's new token -- its position T - 1 --
  // goes to slot new_slots[r] (negative: none) from k_new / v_new [B][H_kv][D].
  const int64_t* new_slots;
  const void* k_new;
  const void* v_new;
};

// Shared-prefix decode: chunk-first items (int32 x 8 each: row0, nrows, tb,
// te, slot, tiles, 0, 0) and each row's private range (first token, slot).
struct SharedArgs {
  const int32_t* items;
  const int32_t* row_private;  // [batch][2]
  int32_t n_items;
  int32_t n_packed;  // work-groups of four rows' private ranges before the items (0: none)
  int32_t nz_items;  // grid z planes of items and packed groups: ceil((n_items + n_packed) / batch)
};

// Private ranges of at most this many positions (four 32-token chunks) are
// walked one wave per row, four rows per work-group.
constexpr int kPackedPrivateTokens = 128;

// Balanced decode: partial states of segments cut by work-group range
// boundaries, two slots per work-group ([slots][G][2], [slots][G][D]).
struct FlatArgs {
  float* piece_ml;
  float* piece_u;
  int32_t seg_cost;  // fixed cost of a (request, kv head) segment, in kChunkUnits per chunk
};
constexpr int kChunkUnits = 8;  // cost of one 32-token chunk on the balancing axis
constexpr int kFlatMaxBatch = 2048;        // rows the balanced decode takes
constexpr int64_t kFlatMaxLds = 64 * 1024;  // its dynamic LDS, bytes

// The library's own fixed scratch (the allocation-free decode): completion
// counters in a region of their own, which no call's partial states overlap,
// so the counters' zero invariant holds across calls of any layout.
struct ScratchArea {
  int32_t* counters;
  size_t counter_bytes;
  char* states;
  size_t state_bytes;
};

// The step's new tokens, one per row, appended in the decode launch: row r's
// token goes to slot slots[r] (negative: none), its rows k[r], v[r] [H_kv][D].
struct NewTokens {
  const int64_t* slots;
  const void* k;
  const void* v;
};

// The decode entry points' common host path (argument checks, plan, validate
// mode, launch).  mode: kTablesDense / kTablesRagged / kTablesContiguous (a
// dense call with row_offsets is ragged); scratch: nullptr to use `workspace`;
// fused: nullptr, or the step's new tokens.
int decode_impl(const pba_kv_pool* pool, const void* q, int32_t num_q_heads,
                const int32_t* block_tables, const int64_t* row_offsets,
                int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch, float scale,
                float* out, float* lse, int32_t partition_tokens, void* workspace,
                size_t workspace_bytes, void* stream, int mode, const ScratchArea* scratch,
                const NewTokens* fused);

hipError_t launch_paged_decode_flat(const DecodeArgs& a, const FlatArgs& f, int head_dim,
                                    int n_wg, hipStream_t stream);
hipError_t launch_expand_tables(const int32_t* src, int64_t n_src, int split_log2, int32_t* dst,
                                hipStream_t stream);
hipError_t launch_pack_tables(const int32_t* src, int32_t batch, int32_t width,
                              const int64_t* offsets, int32_t* dst, hipStream_t stream);
hipError_t launch_kv_append(const AppendArgs& a, int esize, hipStream_t stream);
hipError_t launch_block_copy(const CopyArgs& a, int64_t n_pairs, int kv_heads, hipStream_t stream);
hipError_t launch_paged_decode(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream);
// bf16 only; a.n_parts is the slot stride (max_slots); private_parts bounds the
// private pieces of any row (ceil(max T / part_tokens)).
hipError_t launch_paged_decode_shared(const DecodeArgs& a, const SharedArgs& sa, int head_dim,
                                      int private_parts, hipStream_t stream);
// Work-group size and the token granule partitions are cut at, per dtype.
#ifndef PBA_DECODE_WAVES
#define PBA_DECODE_WAVES 4
#endif
constexpr int kDecodeThreads = 64 * PBA_DECODE_WAVES;

// Dynamic LDS of the balanced decode (4-byte words): T[B], pre[B + 1], the
// waves' chunk totals and piece segments, then the waves' pieces,
// (m, l)[2 waves][G][2] and u[2 waves][G * D].
constexpr int64_t flat_head_words(int B) {
  return (2 * (int64_t)B + 1 + 3 * PBA_DECODE_WAVES + 3) / 4 * 4;
}
constexpr int64_t flat_lds_bytes(int B, int G, int D) {
  return 4 * (flat_head_words(B) + 2 * PBA_DECODE_WAVES * (int64_t)G * (2 + D));
}
inline int decode_granule(int dtype) { return (dtype == PBA_BF16 ? 32 : 64) * PBA_DECODE_WAVES; }

}  // namespace pba

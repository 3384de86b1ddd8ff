/*
 * pba.h -- paged block-table attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpba.so: the data-plane calls of decode-time attention over a
 * paged KV cache.  A request keeps one logical token order; its block table
 * maps logical block j (tokens [j*P, (j+1)*P)) to a physical block of a shared
 * pool, and the last block holds T mod P rows (P when that is 0).
 * ("M5.3 - KV Memory Layout and Exact Reuse", sections 0x00A, 0x03A-0x03D,
 * 0x0A; "7. Memory Management and Local Model State", "Logical tokens,
 * physical blocks".)
 *
 * Allocation of blocks (free FIFO, reference counts, fork, copy-on-write
 * decisions) belongs to the caller; the library only moves and reads bytes.
 *
 * Conventions for every call
 *   - All buffers are device memory owned by the caller; the library never
 *     allocates, frees or retains them past the call.  Every call is
 *     asynchronous on `stream` (a hipStream_t; NULL = the null stream) and is
 *     ordered against other work only by that stream.
 *   - Return value: PBA_OK (0) or a negative pba_status.  Arguments the host
 *     can check (pointers, sizes, shapes, strides, dtypes, workspace size) are
 *     checked before any launch, so a rejected call changes no device byte.
 *     Values that live on the device (block ids, slots, sequence lengths) are
 *     checked only in validate mode (pba_set_validate); outside it,
 *     out-of-range device values are undefined behaviour.
 *   - n == 0 (tokens, pairs, batch) is a successful no-op.
 *   - Thread safety: calls may be made from several host threads; they share
 *     no mutable state except the process-wide validate flag.
 */
#ifndef PBA_H_
#define PBA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pba_status {
  PBA_OK = 0,
  PBA_ERR_NULL_ARG = -1,            /* a required pointer is NULL              */
  PBA_ERR_BAD_DTYPE = -2,           /* dtype not PBA_F32 / PBA_BF16            */
  PBA_ERR_BAD_SHAPE = -3,           /* negative size, head counts, strides     */
  PBA_ERR_UNSUPPORTED = -4,         /* valid but not built: P, head_dim, G     */
  PBA_ERR_WORKSPACE_TOO_SMALL = -5, /* workspace NULL or smaller than needed   */
  PBA_ERR_OUT_OF_RANGE = -6,        /* validate mode: bad id, slot or length   */
  PBA_ERR_OVERLAP = -7,             /* validate mode: duplicate slot / pair    */
  PBA_ERR_HIP = -8,                 /* a HIP runtime call failed               */
  PBA_ERR_HALF_BUNDLE = -9,         /* validate mode: a token or copy list that
                                       would move some cache groups only       */
  PBA_ERR_OUT_OF_MEMORY = -10,      /* contiguous arena: no free or reclaimable
                                       physical page for the request           */
  PBA_ERR_SCRATCH_LIMIT = -11       /* allocation-free decode: the arguments need
                                       more than the library's fixed scratch    */
} pba_status;

typedef enum pba_dtype { PBA_F32 = 0, PBA_BF16 = 1 } pba_dtype;

/* partition_tokens value of the decode calls: balance the batch's work over
 * the CUs instead of cutting rows into equal partitions. */
#define PBA_PARTITIONS_BALANCED (-1)
/* partition_tokens value of pba_paged_decode_plan_ex only: let the library
 * choose from the caller's summary of the row lengths. */
#define PBA_PARTITIONS_AUTO (-2)

/*
 * The K/V pool of one layer (one cache group): a fixed set of physical blocks
 * of P token rows each.  Element (block b, kv head h, in-block token o, dim c):
 *
 *   K: k[b * k_stride_block + h * k_stride_head + o * head_dim + c]
 *   V: v[b * v_stride_block + h * v_stride_head + c * block_size + o]
 *
 * i.e. inside one (block, head) tile K is [P][head_dim] (token major) and V is
 * [head_dim][P] (dim major).  The default dense pool is
 *   K [num_blocks, num_kv_heads, P, head_dim],  V [num_blocks, num_kv_heads, head_dim, P]
 * with k_stride_head = v_stride_head = P * head_dim and
 * k_stride_block = v_stride_block = num_kv_heads * P * head_dim.
 * Strides are in elements; block ids are widened to int64 before they are
 * multiplied by a stride ("Cache Concepts: Prefix Matching vs. Storage",
 * int64 widening of page ids).  Axis order -> strides -> address follows
 * "M5.3", section 0x03E.
 *
 * Requirements: block_size (P) in {16, 32, 64, 128, 256}; head_dim in
 * {64, 128}; k, v and every tile 16-byte aligned; a (block, head) tile of
 * P * head_dim elements must fit inside its stride.
 *
 * Kernel view of an allocator pool ("M5.3", 0x0AC): with split_log2 = s > 0
 * the memory holds tiles of P_a = P << s rows (allocator blocks), and the
 * descriptor exposes each as q = 2^s kernel blocks of P rows: kernel block b
 * is rows [(b mod q) P, (b mod q + 1) P) of tile b >> s, so
 *   K: k[(b >> s) * k_stride_block + h * k_stride_head + ((b mod q) P + o) * head_dim + c]
 *   V: v[(b >> s) * v_stride_block + h * v_stride_head + c * P_a + (b mod q) P + o]
 * num_blocks counts kernel blocks (a multiple of q), and block tables hold
 * kernel ids (pba_expand_block_tables makes them from allocator ids).  Slot
 * ids are the same in both views (b P + o = a P_a + i P + o).  Only the
 * decode calls accept s > 0 (at most 4); kv_append and block_copy take the
 * allocator view (s = 0, block_size P_a) of the same memory.
 */
typedef struct pba_kv_pool {
  void* k;
  void* v;
  int32_t dtype;         /* pba_dtype of every stored K/V scalar            */
  int32_t num_blocks;    /* physical blocks in the pool                      */
  int32_t block_size;    /* P: tokens per block (block_granularity)          */
  int32_t num_kv_heads;  /* H_kv                                             */
  int32_t head_dim;      /* d                                                */
  int32_t split_log2;    /* 0, or the kernel view of an allocator pool: see above */
  int64_t k_stride_block, k_stride_head;
  int64_t v_stride_block, v_stride_head;
} pba_kv_pool;

/*
 * pba_kv_append -- scatter new tokens' K/V rows into their physical slots.
 *
 * For each i < n_tokens with s = slot_mapping[i] >= 0: block = s div P,
 * offset = s mod P, and for every kv head h the row k_new[i, h, :] becomes
 * K(block, h, offset, :) and v_new[i, h, :] becomes V(block, h, offset, :).
 * A negative slot skips the token.  ("M5.3", 0x03C-0x03D slot = block * P +
 * offset; 0x04E the appended row o; "Cache Concepts", backend-owned write
 * locations.)  The copy is bit exact: NaN payloads and signed zeros survive.
 *
 *   slot_mapping  device int64 [n_tokens]
 *   k_new, v_new  device [n_tokens, num_kv_heads, head_dim], pool dtype,
 *                 contiguous, 16-byte aligned
 * Slots must be distinct within one call (validate mode: PBA_ERR_OVERLAP) and
 * below num_blocks * P (validate mode: PBA_ERR_OUT_OF_RANGE).
 */
int pba_kv_append(const pba_kv_pool* pool, const int64_t* slot_mapping, int64_t n_tokens,
                  const void* k_new, const void* v_new, void* stream);

/*
 * pba_block_copy -- copy-on-write before divergence: for each pair k the whole
 * physical block src[k] (every row, every kv head, K and V) is copied bit for
 * bit onto block dst[k].  ("M5.3", 0x04C a fused block-copy launch for COW,
 * 0x05A-0x05D; "7. Memory Management and Local Model State", "Sharing and
 * copy-on-write".)
 *
 *   src, dst  device int32 [n_pairs], ids in [0, num_blocks)
 * No block may appear twice as a destination, nor as both a source and a
 * destination, within one call (validate mode: PBA_ERR_OVERLAP).
 */
int pba_block_copy(const pba_kv_pool* pool, const int32_t* src, const int32_t* dst,
                   int64_t n_pairs, void* stream);

/*
 * Cache groups with a layer axis ("M5.3", 0x03B: each cache group has its
 * own pool and its own block table per request, and a token row of the group
 * spans all of its layers; 0x03C-0x03E: the group-local layer index is one
 * more coordinate of the stride rule; 0x04E: a bundle is one block of every
 * group, P_g * B_row,g bytes in group g).
 *
 * A group holds num_layers consecutive layers.  `pool` describes layer 0
 * (dtype, block count, P, kv heads, head_dim, block and head strides;
 * split_log2 must be 0); layer l is the same description with k and v
 * advanced by l * k_stride_layer and l * v_stride_layer elements:
 *   K: k[l * k_stride_layer + b * k_stride_block + h * k_stride_head + o * head_dim + c]
 *   V: v[l * v_stride_layer + b * v_stride_block + h * v_stride_head + c * P + o]
 * Layer-major groups ([L][NB][H] tiles) and block-major groups ([NB][L][H]
 * tiles: one block's layers adjacent) are both expressed by the strides.  The
 * (layer, block, head) tiles must be pairwise disjoint: sorted by stride,
 * every stride is at least the span of the axes below it (PBA_ERR_BAD_SHAPE).
 * Strides are multiples of 16 bytes.
 */
typedef struct pba_kv_group {
  pba_kv_pool pool;          /* layer 0 */
  int32_t num_layers;        /* L >= 1 */
  int32_t reserved0;         /* must be 0 */
  int64_t k_stride_layer, v_stride_layer;
} pba_kv_group;

#define PBA_MAX_GROUPS 8

/* The pba_kv_pool of layer `layer` of a group, for pba_paged_decode and the
 * other single-layer calls.  Host only: checks the group and writes *out. */
int pba_group_layer_pool(const pba_kv_group* group, int32_t layer, pba_kv_pool* out);

/*
 * pba_kv_append_bundle -- write new tokens into every layer of every cache
 * group in one launch ("M5.3", 0x04E: the appended row is written in every
 * group's destination; 0x05C step 6).
 *
 * For group g < num_groups and token i < n_tokens with s = slot_mappings[g][i]
 * >= 0: block s div P_g, offset s mod P_g, and for every layer l and kv head h
 * the row k_new[g][i, l, h, :] goes to K(l, block, h, offset, :) and
 * v_new[g][i, l, h, :] to V(l, block, h, offset, :), bit exact.
 *
 *   groups         host array [num_groups], 1 <= num_groups <= PBA_MAX_GROUPS
 *   slot_mappings  host array [num_groups] of device int64 [n_tokens]
 *   k_new, v_new   host arrays [num_groups] of device
 *                  [n_tokens, num_layers_g, num_kv_heads_g, head_dim_g] in the
 *                  group's dtype, contiguous, 16-byte aligned
 * A token is written to every group or, when its slot is negative in every
 * group, to none; validate mode rejects a token skipped in some groups only
 * (PBA_ERR_HALF_BUNDLE), a repeated slot within a group (PBA_ERR_OVERLAP) and
 * a slot beyond a group's pool (PBA_ERR_OUT_OF_RANGE), before any launch.
 */
int pba_kv_append_bundle(const pba_kv_group* groups, int32_t num_groups,
                         const int64_t* const* slot_mappings, const void* const* k_new,
                         const void* const* v_new, int64_t n_tokens, void* stream);

/*
 * pba_block_copy_bundle -- the copies of one publication, every layer of
 * every group, in one launch ("M5.3", 0x04C one fused block-copy launch over
 * many pairs and layers; 0x05B-0x05C the tail bundle of every group is copied
 * and all groups' replacements are published together).
 *
 * For group g and pair k < n_pairs[g]: block src_blocks[g][k] -> block
 * dst_blocks[g][k], whole blocks (every layer, kv head, row; K and V).
 *
 *   src_blocks, dst_blocks  host arrays [num_groups] of device int32 [n_pairs[g]]
 *   n_pairs                 host int64 [num_groups]; groups whose block sizes
 *                           differ may copy different numbers of blocks
 * Validate mode checks every group's pairs (ids in range: PBA_ERR_OUT_OF_RANGE;
 * no block twice as a destination or as both source and destination within a
 * group: PBA_ERR_OVERLAP) before anything is copied, so a rejected call moves
 * no group.
 */
int pba_block_copy_bundle(const pba_kv_group* groups, int32_t num_groups,
                          const int32_t* const* src_blocks, const int32_t* const* dst_blocks,
                          const int64_t* n_pairs, void* stream);

/*
 * pba_paged_decode -- one decode query row per request over its logical
 * history ("M5.3", 0x0A the paged decode loop, 0x0BA partial states and their
 * merge).
 *
 * For request r with T = seq_lens[r] and q-head i (kv head h = i / G,
 * G = num_q_heads / num_kv_heads), over the visible tokens t < T read through
 * block_tables[r, t div P] at offset t mod P:
 *   s_t = scale * <q[r, i, :], K_t>
 *   out[r, i, :] = sum_t exp(s_t - m) V_t / sum_t exp(s_t - m),  m = max_t s_t
 *   lse[r, i]    = m + ln sum_t exp(s_t - m)
 * Rows at positions >= T (tail padding, rows another request materialised in
 * a shared block, stale rows of a recycled block) are never used, even if
 * they hold NaN.
 *
 *   q             device [batch, num_q_heads, head_dim], pool dtype, contiguous
 *   block_tables  device int32 [batch, max_blocks_per_seq], row major; entries
 *                 at j >= ceil(T/P) are never read (any value)
 *   seq_lens      device int32 [batch]; 1 <= T <= max_blocks_per_seq * P
 *                 (validate mode: PBA_ERR_OUT_OF_RANGE)
 *   scale         score scale, normally 1/sqrt(head_dim)
 *   out           device float32 [batch, num_q_heads, head_dim]
 *   lse           device float32 [batch, num_q_heads], or NULL
 *   partition_tokens  0: the library splits each row into partitions of its
 *                 choice (sized so that all work-groups are resident at once);
 *                 PBA_PARTITIONS_BALANCED: the batch's 32-token chunks, laid
 *                 end to end, are split evenly over one work-group per CU,
 *                 whatever the row lengths (bf16 batches of at most 2048 rows
 *                 whose work-group state -- eight partial states of G x
 *                 (head_dim + 2) floats and the rows' prefix sums -- fits in
 *                 64 KiB of LDS, i.e. not G = 16 at head_dim 128; otherwise
 *                 as 0) -- for ragged batches, where equal
 *                 partitions leave most work-groups empty; otherwise the
 *                 partition length in tokens, a positive multiple of 256.
 *                 Partitions are reduced by the log-sum-exp merge; an empty
 *                 partition is the identity.
 *   workspace     device scratch of at least
 *                 pba_paged_decode_workspace_bytes(...) bytes, 16-byte aligned
 *                 (NULL allowed when that is 0).  Its first 4 * batch *
 *                 num_kv_heads bytes are completion counters that must be zero
 *                 before the first call that uses the workspace; every call
 *                 leaves them zero again, so a workspace zero-filled once
 *                 serves any number of calls ordered on one stream.  Calls
 *                 that overlap in time must not share a workspace.  The rest
 *                 needs no initialisation.
 * Supported: num_q_heads a multiple of num_kv_heads with G <= 16.
 * The result is deterministic for fixed arguments and does not depend on where
 * the blocks lie physically.
 */
int pba_paged_decode(const pba_kv_pool* pool, const void* q, int32_t num_q_heads,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* seq_lens, int32_t batch, float scale, float* out, float* lse,
                     int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * pba_paged_decode_append -- one decode step: the step's new tokens, one per
 * row, appended and the batch decoded in one call ("M5.3", 0x04E the appended
 * row o is written before the decode reads it; 0x0A the decode loop).  The
 * result equals pba_kv_append(new_slots, k_new, v_new, batch) followed by
 * pba_paged_decode(...) on the same stream, bit for bit in the pool and in
 * out / lse.
 *
 *   new_slots     device int64 [batch]: row r's new token goes to slot
 *                 new_slots[r] (negative: row r appends nothing this step).
 *                 That slot must be row r's last position, T_r - 1, through
 *                 its block table (block_tables[r][(T_r - 1) / P] * P +
 *                 (T_r - 1) % P), in a block no other row of the batch
 *                 references (a shared block is copied before it is written,
 *                 so no work-group reads a position another one writes).
 *                 Validate mode checks the position (PBA_ERR_OUT_OF_RANGE),
 *                 that slots are distinct and that the block is the row's
 *                 alone (PBA_ERR_OVERLAP); outside it, another slot is
 *                 undefined
 *   k_new, v_new  device [batch, num_kv_heads, head_dim], pool dtype,
 *                 contiguous, 16-byte aligned: the new tokens' K and V rows
 * Other arguments as pba_paged_decode (the same workspace size).  Each new
 * token is written, in the decode launch, by the wave that reads it (bf16
 * and fp32 pools; partitions and PBA_PARTITIONS_BALANCED alike).
 */
int pba_paged_decode_append(const pba_kv_pool* pool, const int64_t* new_slots, const void* k_new,
                            const void* v_new, const void* q, int32_t num_q_heads,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t batch, float scale, float* out,
                            float* lse, int32_t partition_tokens, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * pba_paged_decode_ragged -- pba_paged_decode over a compact block table
 * ("M5.3", 0x0AB): row r's entries are block_entries[row_offsets[r] ..
 * row_offsets[r + 1]) (at least ceil(T_r / P) of them) instead of a dense
 * [batch, max_blocks_per_seq] row.  row_offsets: device int64 [batch + 1],
 * non-decreasing, from 0 or more; max_blocks_per_seq bounds every row's entry
 * count and plans the partitions exactly as for the dense call (the same
 * workspace size).  Validate mode checks the offsets and the visible entries.
 * Each work-group reads its row's two offsets before its first table entry
 * (one more scalar round trip than the dense call).
 */
int pba_paged_decode_ragged(const pba_kv_pool* pool, const void* q, int32_t num_q_heads,
                            const int32_t* block_entries, const int64_t* row_offsets,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                            float scale, float* out, float* lse, int32_t partition_tokens,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * pba_expand_block_tables -- allocator ids to kernel ids ("M5.3", 0x0AC): for
 * each of the n_entries input entries a, the q = 2^split_log2 outputs at
 * positions q*i .. q*i + q - 1 are a*q .. a*q + q - 1, or -1 when a < 0
 * (padding).  A dense [B, n] table becomes a dense [B, n q] one, a compact one
 * a compact one with every offset times q.  dst: device int32 [n_entries * q].
 * Ids times q must fit in int32 (validate mode: PBA_ERR_OUT_OF_RANGE).
 */
int pba_expand_block_tables(const int32_t* src, int64_t n_entries, int32_t split_log2,
                            int32_t* dst, void* stream);

/*
 * pba_pack_block_tables -- dense [batch, width] table to a compact one
 * ("M5.3", 0x0AB): dst[row_offsets[r] + j] = src[r, j] for
 * j < row_offsets[r + 1] - row_offsets[r] (<= width; validate mode checks the
 * offsets).  The caller computes the offsets (prefix sums of its rows' block
 * counts) and sizes dst to row_offsets[batch] entries; batch <= 65535.
 */
int pba_pack_block_tables(const int32_t* src, int32_t batch, int32_t width,
                          const int64_t* row_offsets, int32_t* dst, void* stream);

/*
 * Workspace bytes pba_paged_decode (and its ragged and contiguous forms) needs
 * for these arguments; 0 when one partition per row suffices, and 0 for
 * arguments the call would reject.  Host only, no device access.
 *
 * The workspace holds what the pages call the partition API's canonical
 * state of every independently computed key partition of a score row,
 * (m_p, l_p, u_p) per (request, q-head, partition), until the log-sum-exp
 * merge combines them ("M5.3", 0x0BA: one score row, disjoint key partitions,
 * one denominator), plus one completion counter per (request, kv head):
 *   [int32 counters, batch * num_kv_heads | pad to 256 B]
 *   [float (m, l), batch * num_q_heads * n_partitions * 2 | pad to 256 B]
 *   [float u, batch * num_q_heads * n_partitions * head_dim]
 * (the balanced decomposition holds two work-group partial states per CU in
 * place of the per-partition ones).  The same arguments always give the same
 * size and layout.
 */
size_t pba_paged_decode_workspace_bytes(const pba_kv_pool* pool, int32_t num_q_heads,
                                        int32_t batch, int32_t max_blocks_per_seq,
                                        int32_t partition_tokens);

/*
 * pba_paged_decode_noalloc -- pba_paged_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and results as
 * pba_paged_decode (dense block tables, any partition_tokens), without the
 * workspace: the completion counters and partial states live in a fixed
 * array of device memory inside the library, PBA_NOALLOC_COUNTER_BYTES of
 * counters and PBA_NOALLOC_STATE_BYTES of partial states, which every GPU the
 * library runs on holds until the process ends.  The call allocates nothing:
 * no hipMalloc, no hipFree, no allocating library routine.  The first call on
 * a device looks up the array's address there and clears its counters with a
 * kernel on `stream`; every call leaves them at zero again.
 *
 * Limits: batch * num_kv_heads * 4 <= PBA_NOALLOC_COUNTER_BYTES and
 * pba_paged_decode_workspace_bytes(...) minus its counter part (batch *
 * num_kv_heads * 4 rounded up to 256) <= PBA_NOALLOC_STATE_BYTES; larger
 * arguments return PBA_ERR_SCRATCH_LIMIT before anything is launched.
 * Calls on one GPU share the array: calls that overlap in time on one GPU
 * (on two streams, or from host threads without ordering) race and give
 * undefined results.  Validate mode works as for pba_paged_decode (it
 * copies device ids to host memory and synchronises the stream).
 */
#define PBA_NOALLOC_COUNTER_BYTES (256u * 1024u)
#define PBA_NOALLOC_STATE_BYTES (32u * 1024u * 1024u)
int pba_paged_decode_noalloc(const pba_kv_pool* pool, const void* q, int32_t num_q_heads,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* seq_lens, int32_t batch, float scale, float* out,
                             float* lse, int32_t partition_tokens, void* stream);

/* The partition length (tokens) and count pba_paged_decode would use; returns
 * a pba_status.  Either output pointer may be NULL.  For the balanced
 * decomposition the length is 0 and the count is the number of waves the
 * batch's chunks are spread over. */
int pba_paged_decode_plan(const pba_kv_pool* pool, int32_t num_q_heads, int32_t batch,
                          int32_t max_blocks_per_seq, int32_t partition_tokens,
                          int32_t* partition_tokens_out, int32_t* num_partitions_out);

/*
 * pba_paged_decode_plan_ex -- the decomposition a decode call will use, and
 * why ("M5.3", 0x0A: a row's keys cut into partitions merged by the LSE rule;
 * 0x0BL: the dispatch's selected decomposition and its fallback reason are
 * part of what a run must report).  Host only.
 *
 * partition_tokens: as the decode calls take it (0, a length, or
 * PBA_PARTITIONS_BALANCED), or PBA_PARTITIONS_AUTO: the library chooses from
 * `hint`, the caller's summary of the batch's row lengths (the decode calls
 * cannot see them without a device synchronisation):
 *   - every CU holds a (row, kv head) and the longest row is over 4x the
 *     mean: the balanced decomposition (reason PBA_PLAN_RAGGED), or where it
 *     is not built partitions of about twice the mean (fallback says why);
 *   - the longest row is over 1.3x the mean and at least 1536 tokens and the
 *     batch covers over half the CUs: 512-token partitions, 1024 from 4096
 *     tokens on (PBA_PLAN_MILD);
 *   - otherwise the table-width plan (PBA_PLAN_UNIFORM, or PBA_PLAN_FEW_ROWS
 *     when the batch covers at most half the CUs).
 * Without a hint AUTO is the table-width plan (PBA_PLAN_WIDTH).  The decode
 * calls do not take PBA_PARTITIONS_AUTO: pass out->partition_request.
 */
typedef struct pba_length_hint {
  int64_t sum_tokens;   /* sum over the batch of seq_lens */
  int32_t max_tokens;   /* largest seq_lens */
  int32_t reserved0;    /* 0 */
} pba_length_hint;

typedef enum pba_decomposition {
  PBA_DECOMP_GRID = 0,      /* (kv head, request, partition) work-groups */
  PBA_DECOMP_BALANCED = 1   /* the batch's chunks split evenly, one work-group per CU */
} pba_decomposition;

typedef enum pba_plan_reason {
  PBA_PLAN_OK = 0,               /* (fallback) none */
  PBA_PLAN_REQUESTED = 1,        /* the caller's partition length or balanced request */
  PBA_PLAN_WIDTH = 2,            /* library plan from the table width, no lengths given */
  PBA_PLAN_UNIFORM = 3,          /* lengths near uniform: the table-width plan */
  PBA_PLAN_FEW_ROWS = 4,         /* at most half the CUs have a (row, kv head) */
  PBA_PLAN_RAGGED = 5,           /* longest row over 4x the mean, CUs full */
  PBA_PLAN_MILD = 6,             /* mildly ragged, over half the CUs */
  PBA_PLAN_FALLBACK_DTYPE = 7,   /* balanced not built: fp32 pool */
  PBA_PLAN_FALLBACK_BATCH = 8,   /* balanced not built: more than 2048 rows */
  PBA_PLAN_FALLBACK_LDS = 9,     /* balanced not built: its LDS exceeds 64 KiB (G 16, d 128) */
  PBA_PLAN_FALLBACK_CHUNKS = 10  /* balanced not built: 2^31 chunks or more */
} pba_plan_reason;

typedef struct pba_decode_plan_info {
  int32_t partition_request;  /* the partition_tokens value to pass to the decode calls */
  int32_t decomposition;      /* pba_decomposition */
  int32_t partition_tokens;   /* grid: partition length; balanced: 0 */
  int32_t num_partitions;     /* grid: partitions per row; balanced: waves */
  int32_t reason;             /* pba_plan_reason: why this partition request */
  int32_t fallback;           /* pba_plan_reason: why a balanced choice became the grid (0: none) */
  uint64_t workspace_bytes;   /* pba_paged_decode_workspace_bytes for the request */
} pba_decode_plan_info;

int pba_paged_decode_plan_ex(const pba_kv_pool* pool, int32_t num_q_heads, int32_t batch,
                             int32_t max_blocks_per_seq, int32_t partition_tokens,
                             const pba_length_hint* hint, pba_decode_plan_info* out);

/*
 * Shared-prefix execution reuse ("M5.3", 0x0BA-0x0BE: disjoint key partitions
 * of one score row merged by log-sum-exp; Hydragen's batching of the queries
 * that share K/V; ChunkAttention's chunk-first / sequence-first phases).
 *
 * The batch is described as chunks: a chunk is a run of whole blocks that every
 * row of a contiguous range of the batch maps to the same physical ids.  The
 * plan lists chunk-first work items and each row's private range:
 *
 *   items        device int32 [num_items][8], one work item per entry:
 *                  [0] row0, [1] nrows: the batch rows [row0, row0 + nrows)
 *                  [2] tb, [3] te: the key positions [tb, te) of those rows
 *                  [4] slot: index of the item's partial state in each row
 *                  [5] tiles: 1, 2 or 4 tiles of 16/G rows (16 columns);
 *                      nrows <= tiles * (16/G).  Tiles go in groups of two:
 *                      the waves of a group split its positions and each
 *                      wave serves both tiles from one K/V read (up to 64
 *                      query columns per work-group)
 *                  [6], [7]: 0
 *   row_private  device int32 [batch][2]: (pb, ps): row r's positions
 *                [pb, T) are decoded alone in pieces of partition_tokens from
 *                pb, the k-th piece writing slot ps + k.
 *
 * Contract (checked in validate mode, PBA_ERR_OUT_OF_RANGE / PBA_ERR_OVERLAP):
 * for every row the item ranges covering it and its private pieces tile
 * [0, T) exactly, its slots are exactly 0 .. n-1 with n <= max_slots, its
 * private pieces number at most private_parts (when that is nonzero) and its
 * private positions T - pb at most private_tokens (when that is nonzero); tb
 * and pb are multiples of min(P, 32); te <= T of every covered row; every
 * covered row maps blocks [tb/P, ceil(te/P)) to the same ids as row0.  Outside
 * validate mode a plan that breaks the contract gives undefined results but
 * stays inside the caller's buffers.  The result equals pba_paged_decode's up
 * to rounding and is deterministic for a fixed plan.
 *
 * bf16 pools only (PBA_ERR_UNSUPPORTED otherwise); batch <= 65535.
 */
typedef struct pba_shared_plan {
  int32_t num_items;
  int32_t max_slots;         /* partial states per (row, q-head) in the workspace */
  int32_t partition_tokens;  /* piece length: a positive multiple of 256 */
  int32_t private_parts;     /* bound on any row's private pieces, ceil((T - pb) /
                                partition_tokens); 0: from the table width */
  const int32_t* items;
  const int32_t* row_private;
  int32_t private_tokens;    /* bound on any row's private positions T - pb; 0:
                                none given.  At most 128 (four 32-token chunks):
                                four rows' private ranges share a work-group,
                                one wave each, instead of a work-group per
                                private piece */
  int32_t reserved0;         /* 0 */
} pba_shared_plan;

/*
 * pba_shared_plan_build -- the host side of the shared-prefix decode: from the
 * batch's block tables and lengths (host memory), the order in which rows that
 * share leading blocks are adjacent, the shared chunks, and the plan's items
 * and private ranges ("M5.3", 0x0BB: chunks over a coverage interval of
 * sequences, each sequence's ordered chunk path; 0x0BD: the chunk-first /
 * sequence-first metadata is built on the host before the launch).  Host only.
 *
 *   tables      host int32 [batch][width], the caller's row order
 *   seq_lens    host int32 [batch], 0 <= T <= width * P
 *   order       out, host int64 [batch]: row i of the plan is caller row
 *               order[i] (rows sorted lexicographically by table row, stable).
 *               items, row_private and chunks refer to rows in this order: the
 *               decode gets tables, seq_lens and q permuted the same way
 *   items       out, host int32 [items_capacity][8] (pba_shared_plan.items), or
 *               NULL to only size the plan
 *   row_private out, host int32 [batch][2]
 *   chunks      out, host int32 [chunks_capacity][4] (row_begin, row_end,
 *               tok_begin, tok_end) in tree pre-order, or NULL
 *   info        out: the plan's scalars and ledgers
 * A chunk is a maximal run of whole, fully visible blocks that every row of a
 * contiguous row range maps to the same physical ids, below its ancestors'
 * chunks; runs covering more than params->threshold rows become chunks.
 * Every chunk is cut into pieces of partition_tokens keys from its first key;
 * the rows of a piece form 16-column tiles of 16 / G rows, up to
 * tiles_per_item per item.  A row's slots are its chunks' pieces in path
 * order, then its private pieces.  Items are listed longest walk first (32-key
 * chunks per wave, then tiles), the order the decode starts them in; their
 * slots do not depend on it.  Returns PBA_ERR_WORKSPACE_TOO_SMALL (info
 * filled, nothing else written) when items or chunks exceed their capacity.
 */
typedef struct pba_shared_plan_params {
  int32_t block_size;        /* P of the tables (kernel blocks) */
  int32_t group;             /* G = num_q_heads / num_kv_heads, 1 .. 16 */
  int32_t partition_tokens;  /* piece length, a positive multiple of 256 */
  int32_t threshold;         /* chunks cover more than this many rows (>= 0) */
  int32_t tiles_per_item;    /* 1, 2 or 4 */
  int32_t reserved0;         /* 0 */
} pba_shared_plan_params;

typedef struct pba_shared_plan_info {
  int32_t num_items;         /* items of the plan */
  int32_t num_chunks;        /* shared chunks */
  int32_t max_slots;         /* the pba_shared_plan fields of the same names */
  int32_t private_parts;
  int32_t private_tokens;
  int32_t partition_tokens;
  int64_t chunk_rows;        /* rows covered, summed over chunks */
  int64_t kv_rows_read;      /* key positions the plan's work-groups read per kv head
                                (a piece once per pair of tiles, private ranges once) */
  int64_t chunk_visits;      /* 32-token chunk reads per kv head, counted the same way */
  int64_t partial_states;    /* (row, slot) partial states written per kv head (rows of
                                more than one slot): G * (head_dim + 2) floats each */
} pba_shared_plan_info;

int pba_shared_plan_build(const int32_t* tables, int32_t width, const int32_t* seq_lens,
                          int32_t batch, const pba_shared_plan_params* params, int64_t* order,
                          int32_t* items, int32_t items_capacity, int32_t* row_private,
                          int32_t* chunks, int32_t chunks_capacity, pba_shared_plan_info* info);

/* Workspace bytes pba_paged_decode_shared needs (0 when max_slots == 1);
 * returns 0 for arguments it would reject.  The first 4 * batch *
 * num_kv_heads bytes are completion counters with the same zero-once rule as
 * pba_paged_decode's workspace. */
size_t pba_paged_decode_shared_workspace_bytes(const pba_kv_pool* pool, int32_t num_q_heads,
                                               int32_t batch, int32_t max_blocks_per_seq,
                                               const pba_shared_plan* plan);

/* paged_decode over a batch described by a shared-prefix plan; arguments as
 * pba_paged_decode, with the plan in place of partition_tokens. */
int pba_paged_decode_shared(const pba_kv_pool* pool, const void* q, int32_t num_q_heads,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t batch, float scale, float* out,
                            float* lse, const pba_shared_plan* plan, void* workspace,
                            size_t workspace_bytes, void* stream);

/* pba_paged_decode_shared_append -- one shared-prefix decode step: the
 * step's new tokens appended and the batch decoded in one launch, as
 * pba_paged_decode_append does for pba_paged_decode ("M5.3", 0x03C-0x03D:
 * slot s is block s div P, offset s mod P; 0x0BA-0x0BE: the shared-prefix
 * decode).  new_slots, k_new, v_new: as pba_paged_decode_append, rows in the
 * batch's (sharing) order and under the same rules (the row's position
 * T - 1, in a block only that row references); the position must also lie
 * in the row's private range (row_private pb <= T - 1: a chunk's blocks are
 * shared), where the wave that reads T - 1 writes it first.  Validate mode
 * checks all three (PBA_ERR_OUT_OF_RANGE, PBA_ERR_OVERLAP) with nothing
 * written; outside it, a slot elsewhere is undefined.  Other arguments as
 * pba_paged_decode_shared. */
int pba_paged_decode_shared_append(const pba_kv_pool* pool, const int64_t* new_slots,
                                   const void* k_new, const void* v_new, const void* q,
                                   int32_t num_q_heads, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   int32_t batch, float scale, float* out, float* lse,
                                   const pba_shared_plan* plan, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Contiguous virtual K/V ("M5.3", 0x06A-0x06F; vAttention): a second kernel
 * boundary with no user block table.  One virtual reservation holds the K and
 * V tensor of every layer for num_slots request slots; physical pages of
 * page_bytes are created as HIP virtual-memory handles and mapped into a
 * slot's range on demand, in page bundles (page q of the slot in every K and
 * V tensor, mapped and made accessible together before the slot's frontier
 * moves).
 *
 * Layout: tensor x = 2 * layer + (0: K, 1: V) starts at x * num_slots * R
 * bytes from the reservation; slot r's range of a tensor is [r R, (r+1) R),
 * R = page_bytes * ceil(ceil(max_tokens / P) * P * row / page_bytes) with
 * row = num_kv_heads * head_dim * scalar bytes; inside it, token t sits in
 * tile t / P (P rows of every head) in the library's K and V tile layouts.
 * The arena is therefore also a cache group (pba_vkv_group) whose block j of
 * slot r is block id r * blocks_per_slot + j, and token t of slot r has slot
 * id r * blocks_per_slot * P + t for pba_kv_append / pba_kv_append_bundle.
 *
 * Rows may be written and read only below the slot's mapped frontier
 * (pba_vkv_capacity); reading or writing past it touches unmapped memory.
 * In validate mode the append, copy and decode calls on an arena's memory
 * check the frontier (PBA_ERR_OUT_OF_RANGE).  Unmapping (pba_vkv_free without
 * retain, reclamation in pba_vkv_map) first waits for the device to be idle.
 */
typedef struct pba_vkv_arena pba_vkv_arena;

typedef struct pba_vkv_config {
  int32_t dtype;         /* PBA_BF16 or PBA_F32 */
  int32_t num_layers;    /* L: K and V tensors per layer */
  int32_t num_slots;     /* B: request slots */
  int32_t num_kv_heads;  /* H_kv */
  int32_t head_dim;      /* 64 or 128 */
  int32_t block_size;    /* P: rows of one tile, a power of two in 16..256 */
  int64_t max_tokens;    /* T_max: rows reserved per slot */
  int64_t page_bytes;    /* G: a multiple of the device's virtual-memory
                            granularity and of P * row */
  int64_t num_handles;   /* physical pages created up front (a multiple of 2L);
                            0: pages are created when needed, without limit */
} pba_vkv_config;

typedef struct pba_vkv_ledgers {  /* 0x06A: the ledgers are separate quantities */
  int64_t reserved_bytes;           /* M_VA: virtual reservation */
  int64_t pool_bytes;               /* M_phys,pool: handles created */
  int64_t mapped_bytes;             /* M_mapped: handles mapped into slots */
  int64_t inactive_retained_bytes;  /* mapped into freed slots, kept for reuse */
  int64_t free_bytes;               /* created, not mapped */
  int64_t bundle_maps, bundle_unmaps;  /* page bundles mapped / unmapped so far */
  int64_t slot_bytes;               /* R */
} pba_vkv_ledgers;

/* Reserve the arena on the current device; creates num_handles pages. */
int pba_vkv_create(const pba_vkv_config* cfg, pba_vkv_arena** out);
/* Wait for the device, unmap and release every page, free the reservation. */
int pba_vkv_destroy(pba_vkv_arena* arena);
/* Back the first `tokens` rows of the slot (0x06D: map before use).  A freed
 * slot becomes active for a new request generation: its retained pages are
 * reused as capacity, none of its old rows are valid (0x06E).  Pages come
 * from free handles, then from the highest bundle of the lowest-numbered
 * inactive slot; if the pool cannot supply them the call changes nothing and
 * returns PBA_ERR_OUT_OF_MEMORY.  Synchronous on the host. */
int pba_vkv_map(pba_vkv_arena* arena, int32_t slot, int64_t tokens);
/* Mark the slot inactive; retain != 0 keeps its pages mapped (delayed
 * reclamation), otherwise they are unmapped and return to the pool. */
int pba_vkv_free(pba_vkv_arena* arena, int32_t slot, int32_t retain);
/* The arena as a cache group (every layer) and the blocks of one slot. */
int pba_vkv_group(const pba_vkv_arena* arena, pba_kv_group* out, int32_t* blocks_per_slot);
/* Rows of the slot below its mapped frontier. */
int pba_vkv_capacity(const pba_vkv_arena* arena, int32_t slot, int64_t* tokens);
int pba_vkv_get_ledgers(const pba_vkv_arena* arena, pba_vkv_ledgers* out);

/*
 * pba_paged_decode_contiguous -- pba_paged_decode with a request-slot index
 * in place of the block table ("M5.3", 0x06C: the kernel reads no block table,
 * only the slot of each request, as FlashAttention's cache_batch_idx): row r
 * reads rows [0, seq_lens[r]) of slot slot_index[r], i.e. blocks
 * slot_index[r] * blocks_per_slot + j of `pool` (a layer of pba_vkv_group, or
 * any pool laid out that way).  No block past the row's last one is
 * addressed.  slot_index: device int32 [batch], in [0, num_blocks /
 * blocks_per_slot); 1 <= seq_lens[r] <= blocks_per_slot * P (validate mode,
 * which also checks arena frontiers).  Partitions are planned as for the dense
 * call with max_blocks_per_seq = blocks_per_slot.  bf16 pools only.
 */
int pba_paged_decode_contiguous(const pba_kv_pool* pool, const void* q, int32_t num_q_heads,
                                const int32_t* slot_index, int32_t blocks_per_slot,
                                const int32_t* seq_lens, int32_t batch, float scale, float* out,
                                float* lse, int32_t partition_tokens, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* pba_status_string(int status);

/*
 * Validate mode (process wide, default off).  When on, every call first copies
 * its device-resident ids, slots and lengths to the host (synchronising the
 * stream), checks them, and returns PBA_ERR_OUT_OF_RANGE / PBA_ERR_OVERLAP /
 * PBA_ERR_HALF_BUNDLE without launching anything if one is bad, so a rejected
 * call changes no device byte.  This is the pages' rule that every id is
 * checked against its bound before any byte is touched ("Cache Concepts:
 * Prefix Matching vs. Storage", "Virtual block placement within a shared
 * physical plan": ids are validated before any bytes are cleared) and that a
 * failed or rejected operation leaves the predecessor state unchanged
 * ("M5.3", 0x05G Failure Lab).  Host-visible arguments are checked in either
 * mode.  Returns the previous setting.
 */
int pba_set_validate(int on);

/* ABI version: major * 10000 + minor * 100 + patch. */
int pba_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PBA_H_ */

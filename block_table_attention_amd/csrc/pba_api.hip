// Host side of libpba.so: argument checks, the split planner, validate mode
// and kernel launches.  Everything the host can check is checked before any
// launch, so a rejected call leaves every device byte unchanged ("M5.3 - KV
// Memory Layout and Exact Reuse", 0x05G: rejected operations preserve the
// predecessor state; "Cache Concepts: Prefix Matching vs. Storage": validate
// every id before touching bytes).
#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "bundle_internal.h"
#include "append_internal.h"
#include "pba_internal.h"
#include "vkv_internal.h"

namespace {

std::atomic<int> g_validate{0};

constexpr int kPartGranule = 256;  // partition lengths are multiples of this

int log2_exact(int x) {
  if (x <= 0 || (x & (x - 1))) return -1;
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

int esize_of(int dtype) { return dtype == PBA_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// True when the tiles of `tile` elements at sum_i idx_i * stride_i (idx_i <
// count_i) are pairwise disjoint: taken by increasing stride, every axis with
// more than one index strides at least over the span of the axes below it.
bool tiles_disjoint(int64_t tile, std::vector<std::pair<int64_t, int64_t>> axes) {
  std::sort(axes.begin(), axes.end());
  int64_t span = tile;
  for (const auto& a : axes) {
    if (a.second <= 1) continue;
    if (a.first < span) return false;
    if (a.first > (INT64_MAX - span) / (a.second - 1)) return false;
    span += a.first * (a.second - 1);
  }
  return true;
}

// Checks the pool descriptor; everything here is host-visible.
int check_pool(const pba_kv_pool* pool) {
  if (!pool) return PBA_ERR_NULL_ARG;
  if (pool->dtype != PBA_F32 && pool->dtype != PBA_BF16) return PBA_ERR_BAD_DTYPE;
  if (pool->num_blocks <= 0 || pool->num_kv_heads <= 0 || pool->block_size <= 0 ||
      pool->head_dim <= 0 || pool->split_log2 < 0)
    return PBA_ERR_BAD_SHAPE;
  const int lp = log2_exact(pool->block_size);
  if (lp < 4 || lp > 8) return PBA_ERR_UNSUPPORTED;  // P in {16, ..., 256}
  if (pool->head_dim != 64 && pool->head_dim != 128) return PBA_ERR_UNSUPPORTED;
  if (pool->split_log2 > 4) return PBA_ERR_UNSUPPORTED;  // at most 16 kernel blocks per tile
  if (pool->num_blocks % (1 << pool->split_log2)) return PBA_ERR_BAD_SHAPE;
  if (!pool->k || !pool->v) return PBA_ERR_NULL_ARG;
  // An allocator tile holds P << split_log2 rows.
  const int64_t tile = ((int64_t)pool->block_size << pool->split_log2) * pool->head_dim;
  const int64_t tiles = pool->num_blocks >> pool->split_log2;
  const int es = esize_of(pool->dtype);
  const int64_t strides[4] = {pool->k_stride_block, pool->k_stride_head, pool->v_stride_block,
                              pool->v_stride_head};
  for (int64_t s : strides) {
    if (s < 0) return PBA_ERR_BAD_SHAPE;
    if ((s * es) % 16) return PBA_ERR_UNSUPPORTED;
  }
  // The (block, head) tiles of K, and of V, must not overlap.
  if (!tiles_disjoint(tile, {{pool->k_stride_block, tiles}, {pool->k_stride_head, pool->num_kv_heads}}) ||
      !tiles_disjoint(tile, {{pool->v_stride_block, tiles}, {pool->v_stride_head, pool->num_kv_heads}}))
    return PBA_ERR_BAD_SHAPE;
  if (!aligned16(pool->k) || !aligned16(pool->v)) return PBA_ERR_UNSUPPORTED;
  return PBA_OK;
}

// Checks a cache group: its layer-0 pool (allocator view), the layer count and
// strides, and that no two (layer, block, head) tiles of K, or of V, overlap.
int check_group(const pba_kv_group* g) {
  if (!g) return PBA_ERR_NULL_ARG;
  if (g->pool.split_log2) return PBA_ERR_UNSUPPORTED;  // groups are allocator views
  const int st = check_pool(&g->pool);
  if (st) return st;
  const pba_kv_pool& p = g->pool;
  if (g->num_layers < 1 || g->reserved0 != 0 || g->k_stride_layer < 0 || g->v_stride_layer < 0)
    return PBA_ERR_BAD_SHAPE;
  const int es = esize_of(p.dtype);
  if ((g->k_stride_layer * es) % 16 || (g->v_stride_layer * es) % 16) return PBA_ERR_UNSUPPORTED;
  const int64_t tile = (int64_t)p.block_size * p.head_dim;
  if (!tiles_disjoint(tile, {{g->k_stride_layer, g->num_layers}, {p.k_stride_block, p.num_blocks},
                             {p.k_stride_head, p.num_kv_heads}}) ||
      !tiles_disjoint(tile, {{g->v_stride_layer, g->num_layers}, {p.v_stride_block, p.num_blocks},
                             {p.v_stride_head, p.num_kv_heads}}))
    return PBA_ERR_BAD_SHAPE;
  return PBA_OK;
}

int check_groups(const pba_kv_group* groups, int32_t num_groups) {
  if (!groups) return PBA_ERR_NULL_ARG;
  if (num_groups < 1) return PBA_ERR_BAD_SHAPE;
  if (num_groups > PBA_MAX_GROUPS) return PBA_ERR_UNSUPPORTED;
  for (int32_t g = 0; g < num_groups; ++g) {
    const int st = check_group(&groups[g]);
    if (st) return st;
  }
  return PBA_OK;
}

// Shape checks shared by the decode entry points (pool checked first).  The
// decode kernel takes the K strides as int32 and the kv heads on a grid axis
// (at most 65535; the partitions, checked by the planner, likewise).
int check_decode_shape(const pba_kv_pool* pool, int32_t num_q_heads, int32_t batch,
                       int32_t max_blocks_per_seq) {
  const int st = check_pool(pool);
  if (st) return st;
  if (num_q_heads <= 0 || batch < 0 || max_blocks_per_seq <= 0) return PBA_ERR_BAD_SHAPE;
  if (num_q_heads % pool->num_kv_heads) return PBA_ERR_BAD_SHAPE;
  if (num_q_heads / pool->num_kv_heads > 16) return PBA_ERR_UNSUPPORTED;
  if (pool->k_stride_block > INT32_MAX || pool->k_stride_head > INT32_MAX ||
      pool->num_kv_heads > 65535)
    return PBA_ERR_UNSUPPORTED;
  return PBA_OK;
}

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Split planner.  Partition lengths are multiples of the dtype's token granule
// (128 tokens for bf16 = 4 waves x 32-token chunks, 256 for fp32), so chunks
// never straddle a partition; an explicit length must be a multiple of 256.
// Without one, the planner cuts every row into the largest number of equal
// partitions for which the (request, kv head, partition) work-groups number
// at most one per CU, measured over the longest row the table can describe
// (the host does not see seq_lens).  More resident work-groups per CU only
// add bytes in flight: measured on MI355X, one 4-wave work-group per CU
// already keeps the HBM stream at its chunked-access ceiling, while three
// per CU lose ~10% and lengthen the final merges.
int plan_partitions(const pba_kv_pool* pool, int32_t batch, int32_t max_blocks, int32_t requested,
                    int32_t* part_tokens, int32_t* n_parts) {
  const int64_t max_T = (int64_t)max_blocks * pool->block_size;
  if (max_T <= 0) return PBA_ERR_BAD_SHAPE;
  const int64_t granule = pba::decode_granule(pool->dtype);
  int64_t pt;
  if (requested > 0) {
    if (requested % kPartGranule) return PBA_ERR_UNSUPPORTED;
    pt = requested;
  } else if (requested < 0) {
    return PBA_ERR_BAD_SHAPE;
  } else {
    const int64_t slots = device_cu_count();
    const int64_t units = (int64_t)batch * pool->num_kv_heads;
    const int64_t max_splits = (max_T + granule - 1) / granule;
    int64_t splits = slots / units;
    if (splits < 1) splits = 1;
    if (splits > max_splits) splits = max_splits;
    const int64_t per = (max_T + splits - 1) / splits;
    pt = (per + granule - 1) / granule * granule;
  }
  const int64_t np = (max_T + pt - 1) / pt;
  // Partitions go on a grid axis of at most 65535.
  if (pt > INT32_MAX || np > 65535) return PBA_ERR_UNSUPPORTED;
  *part_tokens = (int32_t)pt;
  *n_parts = (int32_t)np;
  return PBA_OK;
}

// Workspace: [counters int32 B*H_kv | pad to 256 B][m, l: B*H_q*n_parts*2 f32
// | pad][u: B*H_q*n_parts*d f32].  Only rows with more than one partition use
// it.  The counters must be zero before the first call; every call leaves them
// zero again.
struct WsLayout {
  size_t ml_off, u_off, bytes;
};

WsLayout workspace_layout(int32_t batch, int32_t kv_heads, int64_t rows, int32_t n_parts,
                          int head_dim) {
  WsLayout w{0, 0, 0};
  if (n_parts <= 1) return w;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  w.ml_off = up((size_t)batch * kv_heads * sizeof(int32_t));
  w.u_off = w.ml_off + up((size_t)rows * n_parts * 2 * sizeof(float));
  w.bytes = w.u_off + (size_t)rows * n_parts * head_dim * sizeof(float);
  return w;
}

// The balanced decode (one 4-wave work-group per CU, the batch's chunks split
// evenly over the waves) serves partition_tokens == PBA_PARTITIONS_BALANCED
// for bf16 batches of at most kFlatMaxBatch rows whose LDS (row prefix sums
// and the waves' pieces) fits in kFlatMaxLds bytes; everything else uses the
// grid of (kv head, request, partition).
// Why the balanced decomposition cannot serve a batch (PBA_PLAN_OK: it can).
int flat_fallback(const pba_kv_pool* pool, int32_t num_q_heads, int32_t batch,
                  int32_t max_blocks_per_seq) {
  if (pool->dtype != PBA_BF16) return PBA_PLAN_FALLBACK_DTYPE;
  if (batch < 1 || batch > pba::kFlatMaxBatch) return PBA_PLAN_FALLBACK_BATCH;
  // Chunk counts are int32 in the kernel: B * H_kv * ceil(max T / 32) < 2^31.
  const int64_t max_T = (int64_t)max_blocks_per_seq * pool->block_size;
  const int64_t chunks = (int64_t)batch * pool->num_kv_heads * ((max_T + 31) / 32);
  if (chunks >= INT32_MAX) return PBA_PLAN_FALLBACK_CHUNKS;
  const int G = num_q_heads / pool->num_kv_heads;
  if (pba::flat_lds_bytes(batch, G, pool->head_dim) > pba::kFlatMaxLds)
    return PBA_PLAN_FALLBACK_LDS;
  return PBA_PLAN_OK;
}

bool use_flat(const pba_kv_pool* pool, int32_t num_q_heads, int32_t batch,
              int32_t partition_tokens, int32_t max_blocks_per_seq) {
  return partition_tokens == PBA_PARTITIONS_BALANCED &&
         flat_fallback(pool, num_q_heads, batch, max_blocks_per_seq) == PBA_PLAN_OK;
}

// A balanced request that the balanced decode cannot serve falls back to the
// library's own partition plan.
int32_t grid_request(int32_t partition_tokens) {
  return partition_tokens == PBA_PARTITIONS_BALANCED ? 0 : partition_tokens;
}

int flat_workgroups() { return device_cu_count(); }  // one work-group per CU

// Fixed cost of one (request, kv head) segment in the balanced decode, in
// units of 1/kChunkUnits of a 32-token chunk, by kernel block size.  Per-wave
// loop times grow with the segments a wave crosses (about a third of a chunk
// each at 64+ token blocks); on lognormal batches (128 requests, median 100
// tokens) half a chunk at 64+ token blocks and three eighths at 16 and 32
// gave the shortest kernels, 4-10% below an even split of the chunks.
int32_t flat_seg_cost(int kernel_block) { return kernel_block >= 64 ? 4 : 3; }

// Balanced-decode workspace: [counters int32 B*H_kv | pad][piece (m, l) |
// pad][piece u], two work-group piece slots per work-group, G columns each
// (the waves' pieces stay in LDS).
int64_t flat_slots() { return 2 * (int64_t)flat_workgroups(); }

WsLayout flat_layout(int32_t batch, int32_t kv_heads, int32_t G, int head_dim) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t pieces = (size_t)flat_slots() * G;
  WsLayout w;
  w.ml_off = up((size_t)batch * kv_heads * sizeof(int32_t));
  w.u_off = w.ml_off + up(pieces * 2 * sizeof(float));
  w.bytes = w.u_off + pieces * head_dim * sizeof(float);
  return w;
}

template <typename T>
bool copy_to_host(std::vector<T>& dst, const T* src, int64_t n, hipStream_t stream) {
  dst.resize((size_t)n);
  if (n == 0) return true;
  if (hipMemcpyAsync(dst.data(), src, (size_t)n * sizeof(T), hipMemcpyDeviceToHost, stream) !=
      hipSuccess)
    return false;
  return hipStreamSynchronize(stream) == hipSuccess;
}

}  // namespace

extern "C" {

int pba_version(void) { return 400; }

int pba_set_validate(int on) { return g_validate.exchange(on ? 1 : 0); }

const char* pba_status_string(int status) {
  switch (status) {
    case PBA_OK: return "ok";
    case PBA_ERR_NULL_ARG: return "a required pointer is NULL";
    case PBA_ERR_BAD_DTYPE: return "unsupported or unknown dtype";
    case PBA_ERR_BAD_SHAPE: return "bad size, head count or stride";
    case PBA_ERR_UNSUPPORTED: return "block size, head_dim, head ratio, alignment or partition length not supported";
    case PBA_ERR_WORKSPACE_TOO_SMALL: return "workspace missing or too small";
    case PBA_ERR_OUT_OF_RANGE: return "block id, slot or sequence length out of range";
    case PBA_ERR_OVERLAP: return "duplicate slot or overlapping copy pairs";
    case PBA_ERR_HIP: return "HIP runtime error";
    case PBA_ERR_HALF_BUNDLE: return "a token or copy would move some cache groups only";
    case PBA_ERR_OUT_OF_MEMORY: return "no free or reclaimable physical page in the arena";
    case PBA_ERR_SCRATCH_LIMIT:
      return "the call needs more than the allocation-free entry point's fixed scratch";
    default: return "unknown status";
  }
}

int pba_kv_append(const pba_kv_pool* pool, const int64_t* slot_mapping, int64_t n_tokens,
                  const void* k_new, const void* v_new, void* stream) {
  int st = check_pool(pool);
  if (st) return st;
  if (pool->split_log2) return PBA_ERR_UNSUPPORTED;  // writes use the allocator view
  if (n_tokens < 0) return PBA_ERR_BAD_SHAPE;
  if (n_tokens == 0) return PBA_OK;
  if (!slot_mapping || !k_new || !v_new) return PBA_ERR_NULL_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return PBA_ERR_UNSUPPORTED;
  // K tasks: one per 16-byte piece; V tasks: one per piece of E tokens (runs
  // of 8 groups), at most n_tokens + 64 tokens' worth.
  const int64_t tasks =
      (2 * n_tokens + 64) * pool->num_kv_heads * (pool->head_dim * esize_of(pool->dtype) / 16);
  if ((tasks + 255) / 256 > INT32_MAX) return PBA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g_validate.load()) {
    std::vector<int64_t> slots;
    if (!copy_to_host(slots, slot_mapping, n_tokens, s)) return PBA_ERR_HIP;
    const int64_t limit = (int64_t)pool->num_blocks * pool->block_size;
    std::unordered_set<int64_t> seen;
    for (int64_t x : slots) {
      if (x < 0) continue;
      if (x >= limit) return PBA_ERR_OUT_OF_RANGE;
      if (!seen.insert(x).second) return PBA_ERR_OVERLAP;
    }
    if ((st = pba::vkv_check_slot_ids(pool->k, slots.data(), n_tokens))) return st;
  }
  pba::AppendArgs a;
  a.k = pool->k;
  a.v = pool->v;
  a.k_sb = pool->k_stride_block;
  a.k_sh = pool->k_stride_head;
  a.v_sb = pool->v_stride_block;
  a.v_sh = pool->v_stride_head;
  a.slots = slot_mapping;
  a.k_new = k_new;
  a.v_new = v_new;
  a.n = n_tokens;
  a.log2P = log2_exact(pool->block_size);
  a.head_dim = pool->head_dim;
  a.kv_heads = pool->num_kv_heads;
  return pba::launch_kv_append(a, esize_of(pool->dtype), s) == hipSuccess ? PBA_OK : PBA_ERR_HIP;
}

int pba_block_copy(const pba_kv_pool* pool, const int32_t* src, const int32_t* dst,
                   int64_t n_pairs, void* stream) {
  int st = check_pool(pool);
  if (st) return st;
  if (pool->split_log2) return PBA_ERR_UNSUPPORTED;  // copies use the allocator view
  if (n_pairs < 0) return PBA_ERR_BAD_SHAPE;
  if (n_pairs == 0) return PBA_OK;
  if (!src || !dst) return PBA_ERR_NULL_ARG;
  if (n_pairs > INT32_MAX || 2LL * pool->num_kv_heads > 65535) return PBA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g_validate.load()) {
    std::vector<int32_t> hs, hd;
    if (!copy_to_host(hs, src, n_pairs, s) || !copy_to_host(hd, dst, n_pairs, s)) return PBA_ERR_HIP;
    std::unordered_set<int32_t> dsts, srcs(hs.begin(), hs.end());
    for (int64_t i = 0; i < n_pairs; ++i) {
      if (hs[i] < 0 || hs[i] >= pool->num_blocks || hd[i] < 0 || hd[i] >= pool->num_blocks)
        return PBA_ERR_OUT_OF_RANGE;
      if (!dsts.insert(hd[i]).second || srcs.count(hd[i])) return PBA_ERR_OVERLAP;
    }
    if ((st = pba::vkv_check_blocks(pool->k, hs.data(), n_pairs)) ||
        (st = pba::vkv_check_blocks(pool->k, hd.data(), n_pairs)))
      return st;
  }
  pba::CopyArgs a;
  a.k = pool->k;
  a.v = pool->v;
  a.k_sb = pool->k_stride_block;
  a.k_sh = pool->k_stride_head;
  a.v_sb = pool->v_stride_block;
  a.v_sh = pool->v_stride_head;
  a.src = src;
  a.dst = dst;
  a.esize = esize_of(pool->dtype);
  a.tile_bytes = (int64_t)pool->block_size * pool->head_dim * a.esize;
  return pba::launch_block_copy(a, n_pairs, pool->num_kv_heads, s) == hipSuccess ? PBA_OK
                                                                                 : PBA_ERR_HIP;
}

int pba_group_layer_pool(const pba_kv_group* group, int32_t layer, pba_kv_pool* out) {
  const int st = check_group(group);
  if (st) return st;
  if (!out) return PBA_ERR_NULL_ARG;
  if (layer < 0 || layer >= group->num_layers) return PBA_ERR_BAD_SHAPE;
  const int es = esize_of(group->pool.dtype);
  *out = group->pool;
  out->k = static_cast<char*>(group->pool.k) + (int64_t)layer * group->k_stride_layer * es;
  out->v = static_cast<char*>(group->pool.v) + (int64_t)layer * group->v_stride_layer * es;
  return PBA_OK;
}

int pba_kv_append_bundle(const pba_kv_group* groups, int32_t num_groups,
                         const int64_t* const* slot_mappings, const void* const* k_new,
                         const void* const* v_new, int64_t n_tokens, void* stream) {
  int st = check_groups(groups, num_groups);
  if (st) return st;
  if (n_tokens < 0) return PBA_ERR_BAD_SHAPE;
  if (n_tokens == 0) return PBA_OK;
  if (!slot_mappings || !k_new || !v_new) return PBA_ERR_NULL_ARG;
  int64_t tasks_per_token = 0;  // K and V pieces of one token over every group
  for (int32_t g = 0; g < num_groups; ++g) {
    if (!slot_mappings[g] || !k_new[g] || !v_new[g]) return PBA_ERR_NULL_ARG;
    if (!aligned16(k_new[g]) || !aligned16(v_new[g])) return PBA_ERR_UNSUPPORTED;
    const pba_kv_pool& p = groups[g].pool;
    tasks_per_token += 2LL * groups[g].num_layers * p.num_kv_heads * (p.head_dim * esize_of(p.dtype) / 16);
  }
  // Tokens per launch: every task index of a launch fits in int32 (the V
  // tasks of a group cover up to 64 tokens past the launch's).
  const int64_t chunk = std::min<int64_t>(n_tokens, (INT32_MAX - 256) / tasks_per_token - 64);
  if (chunk < 1) return PBA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g_validate.load()) {
    std::vector<std::vector<int64_t>> slots(num_groups);
    for (int32_t g = 0; g < num_groups; ++g) {
      if (!copy_to_host(slots[g], slot_mappings[g], n_tokens, s)) return PBA_ERR_HIP;
      const int64_t limit = (int64_t)groups[g].pool.num_blocks * groups[g].pool.block_size;
      std::unordered_set<int64_t> seen;
      for (int64_t x : slots[g]) {
        if (x < 0) continue;
        if (x >= limit) return PBA_ERR_OUT_OF_RANGE;
        if (!seen.insert(x).second) return PBA_ERR_OVERLAP;
      }
      if ((st = pba::vkv_check_slot_ids(groups[g].pool.k, slots[g].data(), n_tokens))) return st;
    }
    for (int64_t i = 0; i < n_tokens; ++i) {
      int skipped = 0;
      for (int32_t g = 0; g < num_groups; ++g) skipped += slots[g][i] < 0;
      if (skipped != 0 && skipped != num_groups) return PBA_ERR_HALF_BUNDLE;
    }
  }
  for (int64_t t0 = 0; t0 < n_tokens; t0 += chunk) {
    const int64_t n = std::min(chunk, n_tokens - t0);
    pba::BundleAppendArgs a{};
    a.n_groups = num_groups;
    a.n = (int32_t)n;
    int64_t task = 0;
    for (int32_t g = 0; g < num_groups; ++g) {
      const pba_kv_group& G = groups[g];
      const pba_kv_pool& p = G.pool;
      const int es = esize_of(p.dtype);
      const int64_t row = (int64_t)G.num_layers * p.num_kv_heads * p.head_dim * es;  // bytes
      pba::GroupAppend& A = a.g[g];
      A.k = static_cast<char*>(p.k);
      A.v = static_cast<char*>(p.v);
      A.k_new = static_cast<const char*>(k_new[g]) + t0 * row;
      A.v_new = static_cast<const char*>(v_new[g]) + t0 * row;
      A.slots = slot_mappings[g] + t0;
      A.k_sl = G.k_stride_layer;
      A.k_sb = p.k_stride_block;
      A.k_sh = p.k_stride_head;
      A.v_sl = G.v_stride_layer;
      A.v_sb = p.v_stride_block;
      A.v_sh = p.v_stride_head;
      A.layers = G.num_layers;
      A.heads = p.num_kv_heads;
      A.head_dim = p.head_dim;
      A.log2P = log2_exact(p.block_size);
      A.esize = es;
      A.task0 = (int32_t)task;
      const int64_t lhp = (int64_t)G.num_layers * p.num_kv_heads * (p.head_dim * es / 16);
      A.per_kind = (int32_t)(n * lhp);
      A.v_tasks = (int32_t)((n < pba::kVBlockedMinTokens ? n
                             : es == 2 ? pba::v_append_groups<uint16_t>(n)
                                       : pba::v_append_groups<uint32_t>(n)) * lhp);
      task += (int64_t)A.per_kind + A.v_tasks;
    }
    a.total = (int32_t)task;
    if (pba::launch_kv_append_bundle(a, s) != hipSuccess) return PBA_ERR_HIP;
  }
  return PBA_OK;
}

int pba_block_copy_bundle(const pba_kv_group* groups, int32_t num_groups,
                          const int32_t* const* src_blocks, const int32_t* const* dst_blocks,
                          const int64_t* n_pairs, void* stream) {
  int st = check_groups(groups, num_groups);
  if (st) return st;
  if (!src_blocks || !dst_blocks || !n_pairs) return PBA_ERR_NULL_ARG;
  int64_t total = 0;
  for (int32_t g = 0; g < num_groups; ++g) {
    if (n_pairs[g] < 0) return PBA_ERR_BAD_SHAPE;
    if (n_pairs[g] > 0 && (!src_blocks[g] || !dst_blocks[g])) return PBA_ERR_NULL_ARG;
    total += n_pairs[g] * 2 * groups[g].num_layers * groups[g].pool.num_kv_heads;
    if (total > INT32_MAX) return PBA_ERR_UNSUPPORTED;
  }
  if (total == 0) return PBA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g_validate.load()) {
    for (int32_t g = 0; g < num_groups; ++g) {
      std::vector<int32_t> hs, hd;
      if (!copy_to_host(hs, src_blocks[g], n_pairs[g], s) ||
          !copy_to_host(hd, dst_blocks[g], n_pairs[g], s))
        return PBA_ERR_HIP;
      const int32_t nb = groups[g].pool.num_blocks;
      std::unordered_set<int32_t> dsts, srcs(hs.begin(), hs.end());
      for (int64_t i = 0; i < n_pairs[g]; ++i) {
        if (hs[i] < 0 || hs[i] >= nb || hd[i] < 0 || hd[i] >= nb) return PBA_ERR_OUT_OF_RANGE;
        if (!dsts.insert(hd[i]).second || srcs.count(hd[i])) return PBA_ERR_OVERLAP;
      }
      if ((st = pba::vkv_check_blocks(groups[g].pool.k, hs.data(), n_pairs[g])) ||
          (st = pba::vkv_check_blocks(groups[g].pool.k, hd.data(), n_pairs[g])))
        return st;
    }
  }
  pba::BundleCopyArgs a{};
  a.n_groups = num_groups;
  int64_t wg = 0;
  for (int32_t g = 0; g < num_groups; ++g) {
    const pba_kv_group& G = groups[g];
    const pba_kv_pool& p = G.pool;
    const int es = esize_of(p.dtype);
    pba::GroupCopy& C = a.g[g];
    C.k = static_cast<char*>(p.k);
    C.v = static_cast<char*>(p.v);
    C.src = src_blocks[g];
    C.dst = dst_blocks[g];
    C.k_sl = G.k_stride_layer * es;
    C.k_sb = p.k_stride_block * es;
    C.k_sh = p.k_stride_head * es;
    C.v_sl = G.v_stride_layer * es;
    C.v_sb = p.v_stride_block * es;
    C.v_sh = p.v_stride_head * es;
    C.layers = G.num_layers;
    C.heads = p.num_kv_heads;
    C.tile16 = (int32_t)((int64_t)p.block_size * p.head_dim * es / 16);
    C.wg0 = (int32_t)wg;
    wg += n_pairs[g] * 2 * G.num_layers * p.num_kv_heads;
  }
  a.total = (int32_t)wg;
  return pba::launch_block_copy_bundle(a, s) == hipSuccess ? PBA_OK : PBA_ERR_HIP;
}

int pba_paged_decode_plan(const pba_kv_pool* pool, int32_t num_q_heads, int32_t batch,
                          int32_t max_blocks_per_seq, int32_t partition_tokens,
                          int32_t* partition_tokens_out, int32_t* num_partitions_out) {
  int st = check_decode_shape(pool, num_q_heads, batch, max_blocks_per_seq);
  if (st) return st;
  int32_t pt = 0, np = 0;
  if (use_flat(pool, num_q_heads, batch, partition_tokens, max_blocks_per_seq)) {
    np = flat_workgroups() * pba::kDecodeThreads / 64;  // waves the batch is spread over
  } else {
    st = plan_partitions(pool, batch > 0 ? batch : 1, max_blocks_per_seq,
                         grid_request(partition_tokens), &pt, &np);
    if (st) return st;
  }
  if (partition_tokens_out) *partition_tokens_out = pt;
  if (num_partitions_out) *num_partitions_out = np;
  return PBA_OK;
}

size_t pba_paged_decode_workspace_bytes(const pba_kv_pool* pool, int32_t num_q_heads,
                                        int32_t batch, int32_t max_blocks_per_seq,
                                        int32_t partition_tokens) {
  int32_t pt = 0, np = 0;
  if (pba_paged_decode_plan(pool, num_q_heads, batch, max_blocks_per_seq, partition_tokens, &pt,
                            &np))
    return 0;
  if (use_flat(pool, num_q_heads, batch, partition_tokens, max_blocks_per_seq))
    return flat_layout(batch, pool->num_kv_heads, num_q_heads / pool->num_kv_heads,
                       pool->head_dim).bytes;
  return workspace_layout(batch, pool->num_kv_heads, (int64_t)batch * num_q_heads, np,
                          pool->head_dim).bytes;
}

// The partition request for a batch whose lengths the caller summarises
// (sum and maximum).  Measured on MI355X over 146 batch shapes (8-128 rows,
// 4-8 kv heads, rows up to 8192 tokens, uniform and ragged lengths):
//  * when every CU already holds a (row, kv head) and the longest row is over
//    4x the mean, equal partitions leave most work-groups idle: the balanced
//    decomposition (lognormal batches: 50 us against 61-77 us with 1024-token
//    partitions), or partitions of about twice the mean where it is not built;
//  * mildly ragged batches (longest over 1.3x the mean and at least 1536
//    tokens) over more than half the CUs: 512-token partitions (1024 from 4096
//    tokens), 4-16 % faster than a whole row per work-group;
//  * otherwise the table-width plan, within ~3 % of the best on uniform batches.
static int32_t auto_request(const pba_kv_pool* pool, int32_t num_q_heads, int32_t batch,
                            int32_t max_blocks_per_seq, const pba_length_hint* hint,
                            int32_t* reason, int32_t* fallback) {
  *fallback = PBA_PLAN_OK;
  if (!hint || batch < 1) {
    *reason = PBA_PLAN_WIDTH;
    return 0;
  }
  const double mean = (double)hint->sum_tokens / batch;
  const int64_t longest = hint->max_tokens;
  const int64_t units = (int64_t)batch * pool->num_kv_heads;
  const int64_t cus = device_cu_count();
  if (units >= cus && longest > 4.0 * mean) {
    const int fb = flat_fallback(pool, num_q_heads, batch, max_blocks_per_seq);
    if (fb == PBA_PLAN_OK) {
      *reason = PBA_PLAN_RAGGED;
      return PBA_PARTITIONS_BALANCED;
    }
    *fallback = fb;
    *reason = PBA_PLAN_RAGGED;
    int64_t pt = ((int64_t)(2.0 * mean) + 255) / 256 * 256;
    pt = std::max<int64_t>(512, pt);
    return pt >= longest ? 0 : (int32_t)std::min<int64_t>(pt, 1 << 30);
  }
  if (2 * units > cus && longest > 1.3 * mean && longest >= 1536) {
    *reason = PBA_PLAN_MILD;
    return longest < 4096 ? 512 : 1024;
  }
  *reason = 2 * units > cus ? PBA_PLAN_UNIFORM : PBA_PLAN_FEW_ROWS;
  return 0;
}

int pba_paged_decode_plan_ex(const pba_kv_pool* pool, int32_t num_q_heads, int32_t batch,
                             int32_t max_blocks_per_seq, int32_t partition_tokens,
                             const pba_length_hint* hint, pba_decode_plan_info* out) {
  if (!out) return PBA_ERR_NULL_ARG;
  int st = check_decode_shape(pool, num_q_heads, batch, max_blocks_per_seq);
  if (st) return st;
  if (hint && (hint->sum_tokens < 0 || hint->max_tokens < 0 || hint->reserved0 != 0))
    return PBA_ERR_BAD_SHAPE;
  pba_decode_plan_info info{};
  info.fallback = PBA_PLAN_OK;
  int32_t request = partition_tokens;
  if (partition_tokens == PBA_PARTITIONS_AUTO) {
    request = auto_request(pool, num_q_heads, batch, max_blocks_per_seq, hint, &info.reason,
                           &info.fallback);
  } else if (partition_tokens == PBA_PARTITIONS_BALANCED) {
    info.reason = PBA_PLAN_REQUESTED;
    info.fallback = flat_fallback(pool, num_q_heads, batch > 0 ? batch : 1, max_blocks_per_seq);
  } else {
    info.reason = partition_tokens == 0 ? PBA_PLAN_WIDTH : PBA_PLAN_REQUESTED;
  }
  info.partition_request = request;
  int32_t pt = 0, np = 0;
  st = pba_paged_decode_plan(pool, num_q_heads, batch, max_blocks_per_seq, request, &pt, &np);
  if (st) return st;
  info.decomposition = use_flat(pool, num_q_heads, batch, request, max_blocks_per_seq)
                           ? PBA_DECOMP_BALANCED
                           : PBA_DECOMP_GRID;
  info.partition_tokens = pt;
  info.num_partitions = np;
  info.workspace_bytes =
      pba_paged_decode_workspace_bytes(pool, num_q_heads, batch, max_blocks_per_seq, request);
  *out = info;
  return PBA_OK;
}

}  // extern "C"

namespace pba {

// Validate mode, fused steps: each new token is its row's position T - 1
// through the row's table (block_of(r, j) = row r's j-th block), the slots
// are distinct, and no other row of the batch references a new token's block
// (a block that several rows share is copied before it is written, so a new
// position is visible to its own row alone and no work-group reads it while
// another writes it).
template <typename BlockOf>
int check_new_tokens(const std::vector<int64_t>& ns, const std::vector<int32_t>& lens,
                     int32_t batch, int P, BlockOf block_of) {
  std::unordered_set<int64_t> seen;
  std::unordered_map<int64_t, int32_t> owner;
  for (int32_t r = 0; r < batch; ++r) {
    if (ns[r] < 0) continue;
    const int64_t t = lens[r] - 1;
    const int64_t blk = block_of(r, t / P);
    if (ns[r] != blk * P + t % P) return PBA_ERR_OUT_OF_RANGE;
    if (!seen.insert(ns[r]).second || !owner.emplace(blk, r).second) return PBA_ERR_OVERLAP;
  }
  for (int32_t r = 0; r < batch && !owner.empty(); ++r) {
    const int64_t nb = (lens[r] + P - 1) / P;
    for (int64_t j = 0; j < nb; ++j) {
      const auto it = owner.find(block_of(r, j));
      if (it != owner.end() && it->second != r) return PBA_ERR_OVERLAP;
    }
  }
  return PBA_OK;
}

// Dense (row r at r * max_blocks_per_seq), ragged (row r =
// block_tables[row_offsets[r] .. row_offsets[r + 1])) or contiguous
// (block_tables = slot index, max_blocks_per_seq = blocks per slot) decode.
// The counters and partial states go to the caller's workspace (counters
// first), or, with `scratch`, to its two fixed regions.
int decode_impl(const pba_kv_pool* pool, const void* q, int32_t num_q_heads,
                const int32_t* block_tables, const int64_t* row_offsets,
                int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch, float scale,
                float* out, float* lse, int32_t partition_tokens, void* workspace,
                size_t workspace_bytes, void* stream, int mode, const ScratchArea* scratch,
                const NewTokens* fused) {
  int st = check_decode_shape(pool, num_q_heads, batch, max_blocks_per_seq);
  if (st) return st;
  if (mode == pba::kTablesContiguous && pool->dtype != PBA_BF16) return PBA_ERR_UNSUPPORTED;
  const int G = num_q_heads / pool->num_kv_heads;
  if (batch == 0) return PBA_OK;
  if (!q || !block_tables || !seq_lens || !out) return PBA_ERR_NULL_ARG;
  if (!aligned16(q)) return PBA_ERR_UNSUPPORTED;
  if (fused && (!fused->slots || !fused->k || !fused->v)) return PBA_ERR_NULL_ARG;
  if (fused && (!aligned16(fused->k) || !aligned16(fused->v))) return PBA_ERR_UNSUPPORTED;
  const bool flat = use_flat(pool, num_q_heads, batch, partition_tokens, max_blocks_per_seq);
  int32_t pt = 0, np = 0;
  if (!flat) {
    st = plan_partitions(pool, batch, max_blocks_per_seq, grid_request(partition_tokens), &pt,
                         &np);
    if (st) return st;
  }
  const int64_t rows = (int64_t)batch * num_q_heads;
  if (rows > INT32_MAX) return PBA_ERR_UNSUPPORTED;
  const WsLayout ws = flat ? flat_layout(batch, pool->num_kv_heads, G, pool->head_dim)
                           : workspace_layout(batch, pool->num_kv_heads, rows, np, pool->head_dim);
  const size_t need = ws.bytes;
  // Counters, then the (m, l) and u states: at the layout's offsets in the
  // caller's workspace, or in the scratch's two regions (states from its
  // state region's start).
  int32_t* counters = nullptr;
  float* ws_ml = nullptr;
  float* ws_u = nullptr;
  if (need > 0 && scratch) {
    if ((size_t)batch * pool->num_kv_heads * sizeof(int32_t) > scratch->counter_bytes ||
        need - ws.ml_off > scratch->state_bytes)
      return PBA_ERR_SCRATCH_LIMIT;
    counters = scratch->counters;
    ws_ml = reinterpret_cast<float*>(scratch->states);
    ws_u = reinterpret_cast<float*>(scratch->states + (ws.u_off - ws.ml_off));
  } else if (need > 0) {
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
      return PBA_ERR_WORKSPACE_TOO_SMALL;
    char* wsb = static_cast<char*>(workspace);
    counters = reinterpret_cast<int32_t*>(wsb);
    ws_ml = reinterpret_cast<float*>(wsb + ws.ml_off);
    ws_u = reinterpret_cast<float*>(wsb + ws.u_off);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g_validate.load()) {
    std::vector<int32_t> lens, tab;
    std::vector<int64_t> offs;
    if (!copy_to_host(lens, seq_lens, batch, s)) return PBA_ERR_HIP;
    if (mode == pba::kTablesContiguous) {
      if (!copy_to_host(tab, block_tables, batch, s)) return PBA_ERR_HIP;
      const int64_t n_slots = pool->num_blocks / max_blocks_per_seq;
      const int64_t cap = (int64_t)max_blocks_per_seq * pool->block_size;
      for (int32_t r = 0; r < batch; ++r)
        if (tab[r] < 0 || tab[r] >= n_slots || lens[r] < 1 || lens[r] > cap)
          return PBA_ERR_OUT_OF_RANGE;
      if ((st = pba::vkv_check_rows(pool->k, tab.data(), lens.data(), batch))) return st;
    } else if (row_offsets) {
      if (!copy_to_host(offs, row_offsets, (int64_t)batch + 1, s)) return PBA_ERR_HIP;
      if (offs[0] < 0) return PBA_ERR_OUT_OF_RANGE;
      for (int32_t r = 0; r < batch; ++r)
        if (offs[r + 1] < offs[r] || offs[r + 1] - offs[r] > max_blocks_per_seq)
          return PBA_ERR_OUT_OF_RANGE;
      if (!copy_to_host(tab, block_tables, offs[batch], s)) return PBA_ERR_HIP;
    } else {
      if (!copy_to_host(tab, block_tables, (int64_t)batch * max_blocks_per_seq, s)) return PBA_ERR_HIP;
    }
    const int64_t cap = (int64_t)max_blocks_per_seq * pool->block_size;
    for (int32_t r = 0; r < batch && mode != pba::kTablesContiguous; ++r) {
      const int64_t T = lens[r];
      if (T < 1 || T > cap) return PBA_ERR_OUT_OF_RANGE;
      const int64_t nb = (T + pool->block_size - 1) / pool->block_size;
      const int64_t base = row_offsets ? offs[r] : (int64_t)r * max_blocks_per_seq;
      if (row_offsets && offs[r + 1] - offs[r] < nb) return PBA_ERR_OUT_OF_RANGE;
      for (int64_t j = 0; j < nb; ++j) {
        const int32_t b = tab[(size_t)(base + j)];
        if (b < 0 || b >= pool->num_blocks) return PBA_ERR_OUT_OF_RANGE;
      }
      if ((st = pba::vkv_check_blocks(pool->k, tab.data() + base, nb))) return st;
    }
    if (fused) {
      std::vector<int64_t> ns;
      if (!copy_to_host(ns, fused->slots, batch, s)) return PBA_ERR_HIP;
      const int64_t mb = max_blocks_per_seq;
      st = check_new_tokens(ns, lens, batch, pool->block_size, [&](int32_t r, int64_t j) {
        if (mode == pba::kTablesContiguous) return (int64_t)tab[r] * mb + j;
        return (int64_t)tab[(size_t)((row_offsets ? offs[r] : r * mb) + j)];
      });
      if (st) return st;
    }
  }
  pba::DecodeArgs a;
  a.k = pool->k;
  a.v = pool->v;
  a.k_sb = pool->k_stride_block;
  a.k_sh = pool->k_stride_head;
  a.v_sb = pool->v_stride_block;
  a.v_sh = pool->v_stride_head;
  a.q = q;
  a.tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  a.counters = counters;
  a.ws_ml = ws_ml;
  a.ws_u = ws_u;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = pool->num_blocks;
  a.split_log2 = pool->split_log2;
  a.row_offsets = row_offsets;
  a.table_mode = mode == pba::kTablesContiguous ? mode
                 : row_offsets                  ? pba::kTablesRagged
                                                : pba::kTablesDense;
  a.log2P = log2_exact(pool->block_size);
  a.G = G;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.batch = batch;
  a.part_tokens = pt;
  a.n_parts = np;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.new_slots = nullptr;
  a.k_new = a.v_new = nullptr;
  if (fused) {
    // Every decomposition writes the step's tokens in its own launch, from
    // the wave that reads each of them (fused steps come with dense tables).
    if (a.table_mode != pba::kTablesDense) return PBA_ERR_UNSUPPORTED;
    a.new_slots = fused->slots;
    a.k_new = fused->k;
    a.v_new = fused->v;
  }
  if (flat) {
    pba::FlatArgs f;
    f.piece_ml = ws_ml;
    f.piece_u = ws_u;
    f.seg_cost = flat_seg_cost(pool->block_size);  // the kernel block
    return pba::launch_paged_decode_flat(a, f, pool->head_dim, flat_workgroups(), s) == hipSuccess
               ? PBA_OK
               : PBA_ERR_HIP;
  }
  return pba::launch_paged_decode(a, pool->dtype, pool->head_dim, s) == hipSuccess ? PBA_OK
                                                                                  : PBA_ERR_HIP;
}

}  // namespace pba

extern "C" {

int pba_paged_decode(const pba_kv_pool* pool, const void* q, int32_t num_q_heads,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* seq_lens, int32_t batch, float scale, float* out, float* lse,
                     int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return pba::decode_impl(pool, q, num_q_heads, block_tables, nullptr, max_blocks_per_seq,
                          seq_lens, batch, scale, out, lse, partition_tokens, workspace,
                          workspace_bytes, stream, pba::kTablesDense, nullptr, nullptr);
}

int pba_paged_decode_append(const pba_kv_pool* pool, const int64_t* new_slots, const void* k_new,
                            const void* v_new, const void* q, int32_t num_q_heads,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t batch, float scale, float* out,
                            float* lse, int32_t partition_tokens, void* workspace,
                            size_t workspace_bytes, void* stream) {
  const pba::NewTokens fused{new_slots, k_new, v_new};
  return pba::decode_impl(pool, q, num_q_heads, block_tables, nullptr, max_blocks_per_seq,
                          seq_lens, batch, scale, out, lse, partition_tokens, workspace,
                          workspace_bytes, stream, pba::kTablesDense, nullptr, &fused);
}

int pba_paged_decode_ragged(const pba_kv_pool* pool, const void* q, int32_t num_q_heads,
                            const int32_t* block_entries, const int64_t* row_offsets,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                            float scale, float* out, float* lse, int32_t partition_tokens,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (batch > 0 && !row_offsets) return PBA_ERR_NULL_ARG;
  return pba::decode_impl(pool, q, num_q_heads, block_entries, row_offsets, max_blocks_per_seq,
                          seq_lens, batch, scale, out, lse, partition_tokens, workspace,
                          workspace_bytes, stream, pba::kTablesDense, nullptr, nullptr);
}

int pba_paged_decode_contiguous(const pba_kv_pool* pool, const void* q, int32_t num_q_heads,
                                const int32_t* slot_index, int32_t blocks_per_slot,
                                const int32_t* seq_lens, int32_t batch, float scale, float* out,
                                float* lse, int32_t partition_tokens, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (pool && blocks_per_slot > 0 && pool->num_blocks % blocks_per_slot) return PBA_ERR_BAD_SHAPE;
  if (pool && pool->split_log2) return PBA_ERR_UNSUPPORTED;
  return pba::decode_impl(pool, q, num_q_heads, slot_index, nullptr, blocks_per_slot, seq_lens,
                          batch, scale, out, lse, partition_tokens, workspace, workspace_bytes,
                          stream, pba::kTablesContiguous, nullptr, nullptr);
}

int pba_expand_block_tables(const int32_t* src, int64_t n_entries, int32_t split_log2,
                            int32_t* dst, void* stream) {
  if (n_entries < 0 || split_log2 < 0) return PBA_ERR_BAD_SHAPE;
  if (split_log2 > 4) return PBA_ERR_UNSUPPORTED;
  if (n_entries == 0) return PBA_OK;
  if (!src || !dst) return PBA_ERR_NULL_ARG;
  if ((n_entries << split_log2) / 256 + 1 > INT32_MAX) return PBA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g_validate.load()) {
    std::vector<int32_t> h;
    if (!copy_to_host(h, src, n_entries, s)) return PBA_ERR_HIP;
    for (int32_t a : h)
      if (a >= 0 && (int64_t)a << split_log2 > INT32_MAX) return PBA_ERR_OUT_OF_RANGE;
  }
  return pba::launch_expand_tables(src, n_entries, split_log2, dst, s) == hipSuccess ? PBA_OK
                                                                                     : PBA_ERR_HIP;
}

int pba_pack_block_tables(const int32_t* src, int32_t batch, int32_t width,
                          const int64_t* row_offsets, int32_t* dst, void* stream) {
  if (batch < 0 || width < 0) return PBA_ERR_BAD_SHAPE;
  if (batch == 0 || width == 0) return PBA_OK;
  if (batch > 65535) return PBA_ERR_UNSUPPORTED;
  if (!src || !row_offsets || !dst) return PBA_ERR_NULL_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g_validate.load()) {
    std::vector<int64_t> offs;
    if (!copy_to_host(offs, row_offsets, (int64_t)batch + 1, s)) return PBA_ERR_HIP;
    if (offs[0] < 0) return PBA_ERR_OUT_OF_RANGE;
    for (int32_t r = 0; r < batch; ++r)
      if (offs[r + 1] < offs[r] || offs[r + 1] - offs[r] > width) return PBA_ERR_OUT_OF_RANGE;
  }
  return pba::launch_pack_tables(src, batch, width, row_offsets, dst, s) == hipSuccess
             ? PBA_OK
             : PBA_ERR_HIP;
}

}  // extern "C"

namespace {

// Host-visible checks of a shared-prefix plan (the device arrays are checked
// in validate mode only).
int check_shared_plan(const pba_kv_pool* pool, int32_t num_q_heads, int32_t batch,
                      int32_t max_blocks, const pba_shared_plan* plan, int32_t* nz_items,
                      int32_t* private_parts, int32_t* n_packed = nullptr) {
  if (!plan) return PBA_ERR_NULL_ARG;
  if (pool->dtype != PBA_BF16) return PBA_ERR_UNSUPPORTED;
  if (plan->private_parts < 0 || plan->num_items < 0 || plan->max_slots < 1 ||
      plan->private_tokens < 0 || plan->reserved0 != 0)
    return PBA_ERR_BAD_SHAPE;
  const int32_t pt = plan->partition_tokens;
  if (pt <= 0 || pt % kPartGranule) return PBA_ERR_UNSUPPORTED;
  if (batch > 65535) return PBA_ERR_UNSUPPORTED;
  if (batch > 0 && (!plan->row_private || (plan->num_items > 0 && !plan->items)))
    return PBA_ERR_NULL_ARG;
  const int64_t max_T = (int64_t)max_blocks * pool->block_size;
  // Short private ranges go four rows per work-group, in the items' planes;
  // otherwise each private piece has a work-group of its own, one plane per
  // piece index.
  const bool packed = plan->private_tokens > 0 && plan->private_tokens <= pba::kPackedPrivateTokens;
  const int64_t npk = packed ? ((int64_t)batch + 3) / 4 : 0;
  const int64_t pp = packed                   ? 0
                     : plan->private_parts > 0 ? plan->private_parts
                                               : (max_T + pt - 1) / pt;
  const int64_t nz = batch > 0 ? ((int64_t)plan->num_items + npk + batch - 1) / batch : 0;
  if (pp + nz > 65535) return PBA_ERR_UNSUPPORTED;
  if ((int64_t)batch * num_q_heads > INT32_MAX) return PBA_ERR_UNSUPPORTED;
  *nz_items = (int32_t)nz;
  *private_parts = (int32_t)pp;
  if (n_packed) *n_packed = (int32_t)npk;
  return PBA_OK;
}

// Validate mode: every row's key positions [0, T) are covered exactly once by
// the chunk-first items covering it and its private pieces, its slots are
// exactly 0 .. n-1 with n <= max_slots, and every row an item covers maps the
// item's blocks to the same physical ids as the item's first row.
int validate_shared_plan(const pba_kv_pool* pool, int32_t num_q_heads, int32_t batch,
                         int32_t max_blocks, const pba_shared_plan* plan,
                         const std::vector<int32_t>& lens, const std::vector<int32_t>& tab,
                         hipStream_t s) {
  const int P = pool->block_size;
  const int align = P < 32 ? P : 32;
  const int G = num_q_heads / pool->num_kv_heads;
  const int rpt = 16 / G;
  const int32_t pt = plan->partition_tokens;
  std::vector<int32_t> items, priv;
  if (!copy_to_host(items, plan->items, (int64_t)plan->num_items * 8, s)) return PBA_ERR_HIP;
  if (!copy_to_host(priv, plan->row_private, (int64_t)batch * 2, s)) return PBA_ERR_HIP;
  // Per row: (token begin, token end) pieces and slots.
  std::vector<std::vector<std::pair<int64_t, int64_t>>> spans(batch);
  std::vector<std::vector<int32_t>> slots(batch);
  for (int32_t i = 0; i < plan->num_items; ++i) {
    const int32_t* it = &items[(size_t)i * 8];
    const int32_t row0 = it[0], nrows = it[1], tb = it[2], te = it[3], slot = it[4];
    const int32_t tiles = it[5];
    if ((tiles != 1 && tiles != 2 && tiles != 4) || it[6] || it[7]) return PBA_ERR_OUT_OF_RANGE;
    if (row0 < 0 || nrows < 1 || nrows > tiles * rpt || (int64_t)row0 + nrows > batch)
      return PBA_ERR_OUT_OF_RANGE;
    if (tb < 0 || te <= tb || tb % align || slot < 0 || slot >= plan->max_slots)
      return PBA_ERR_OUT_OF_RANGE;
    const int64_t j0 = tb / P, j1 = ((int64_t)te + P - 1) / P;
    for (int32_t r = row0; r < row0 + nrows; ++r) {
      if (te > lens[r]) return PBA_ERR_OUT_OF_RANGE;
      for (int64_t j = j0; j < j1; ++j)
        if (tab[(size_t)r * max_blocks + j] != tab[(size_t)row0 * max_blocks + j])
          return PBA_ERR_OUT_OF_RANGE;
      spans[r].push_back({tb, te});
      slots[r].push_back(slot);
    }
  }
  for (int32_t r = 0; r < batch; ++r) {
    const int32_t T = lens[r], pb = priv[2 * (size_t)r], ps = priv[2 * (size_t)r + 1];
    if (pb < 0 || pb > T || pb % align || ps < 0) return PBA_ERR_OUT_OF_RANGE;
    int32_t k = 0;
    for (int64_t t = pb; t < T; t += pt, ++k) {
      spans[r].push_back({t, std::min<int64_t>(T, t + pt)});
      slots[r].push_back(ps + k);
    }
    if (plan->private_parts > 0 && k > plan->private_parts) return PBA_ERR_OUT_OF_RANGE;
    if (plan->private_tokens > 0 && T - pb > plan->private_tokens) return PBA_ERR_OUT_OF_RANGE;
    std::sort(spans[r].begin(), spans[r].end());
    int64_t at = 0;
    for (const auto& sp : spans[r]) {
      if (sp.first != at) return sp.first < at ? PBA_ERR_OVERLAP : PBA_ERR_OUT_OF_RANGE;
      at = sp.second;
    }
    if (at != T) return PBA_ERR_OUT_OF_RANGE;
    std::sort(slots[r].begin(), slots[r].end());
    for (size_t q = 0; q < slots[r].size(); ++q) {
      if (q > 0 && slots[r][q] == slots[r][q - 1]) return PBA_ERR_OVERLAP;
      if (slots[r][q] != (int32_t)q) return PBA_ERR_OUT_OF_RANGE;
    }
    if ((int64_t)slots[r].size() > plan->max_slots) return PBA_ERR_OUT_OF_RANGE;
  }
  return PBA_OK;
}

}  // namespace

extern "C" {

size_t pba_paged_decode_shared_workspace_bytes(const pba_kv_pool* pool, int32_t num_q_heads,
                                               int32_t batch, int32_t max_blocks_per_seq,
                                               const pba_shared_plan* plan) {
  if (check_decode_shape(pool, num_q_heads, batch, max_blocks_per_seq)) return 0;
  int32_t nz = 0, pp = 0;
  if (check_shared_plan(pool, num_q_heads, batch, max_blocks_per_seq, plan, &nz, &pp)) return 0;
  return workspace_layout(batch, pool->num_kv_heads, (int64_t)batch * num_q_heads,
                          plan->max_slots, pool->head_dim).bytes;
}

}  // extern "C"

namespace {

// pba_paged_decode_shared, and with `fused` pba_paged_decode_shared_append.
int shared_decode(const pba_kv_pool* pool, const void* q, int32_t num_q_heads,
                  const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                  int32_t batch, float scale, float* out, float* lse, const pba_shared_plan* plan,
                  void* workspace, size_t workspace_bytes, void* stream,
                  const pba::NewTokens* fused) {
  int st = check_decode_shape(pool, num_q_heads, batch, max_blocks_per_seq);
  if (st) return st;
  int32_t nz = 0, pp = 0, npk = 0;
  st = check_shared_plan(pool, num_q_heads, batch, max_blocks_per_seq, plan, &nz, &pp, &npk);
  if (st) return st;
  if (batch == 0) return PBA_OK;
  if (!q || !block_tables || !seq_lens || !out) return PBA_ERR_NULL_ARG;
  if (!aligned16(q)) return PBA_ERR_UNSUPPORTED;
  if (fused && (!fused->slots || !fused->k || !fused->v)) return PBA_ERR_NULL_ARG;
  if (fused && (!aligned16(fused->k) || !aligned16(fused->v))) return PBA_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)batch * num_q_heads;
  const WsLayout ws = workspace_layout(batch, pool->num_kv_heads, rows, plan->max_slots,
                                       pool->head_dim);
  if (ws.bytes > 0 && (!workspace || workspace_bytes < ws.bytes || !aligned16(workspace)))
    return PBA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g_validate.load()) {
    std::vector<int32_t> lens, tab;
    if (!copy_to_host(lens, seq_lens, batch, s)) return PBA_ERR_HIP;
    if (!copy_to_host(tab, block_tables, (int64_t)batch * max_blocks_per_seq, s)) return PBA_ERR_HIP;
    const int64_t cap = (int64_t)max_blocks_per_seq * pool->block_size;
    for (int32_t r = 0; r < batch; ++r) {
      const int64_t T = lens[r];
      if (T < 1 || T > cap) return PBA_ERR_OUT_OF_RANGE;
      const int64_t nb = (T + pool->block_size - 1) / pool->block_size;
      for (int64_t j = 0; j < nb; ++j) {
        const int32_t b = tab[(size_t)r * max_blocks_per_seq + j];
        if (b < 0 || b >= pool->num_blocks) return PBA_ERR_OUT_OF_RANGE;
      }
    }
    st = validate_shared_plan(pool, num_q_heads, batch, max_blocks_per_seq, plan, lens, tab, s);
    if (st) return st;
    if (fused) {
      // Besides check_new_tokens: the new position lies in the row's private
      // range (a chunk's work-groups do not write).
      std::vector<int64_t> ns;
      std::vector<int32_t> priv;
      if (!copy_to_host(ns, fused->slots, batch, s)) return PBA_ERR_HIP;
      if (!copy_to_host(priv, plan->row_private, (int64_t)batch * 2, s)) return PBA_ERR_HIP;
      for (int32_t r = 0; r < batch; ++r)
        if (ns[r] >= 0 && priv[2 * (size_t)r] > lens[r] - 1) return PBA_ERR_OUT_OF_RANGE;
      const int64_t mb = max_blocks_per_seq;
      st = pba::check_new_tokens(ns, lens, batch, pool->block_size, [&](int32_t r, int64_t j) {
        return (int64_t)tab[(size_t)(r * mb + j)];
      });
      if (st) return st;
    }
  }
  pba::DecodeArgs a;
  a.k = pool->k;
  a.v = pool->v;
  a.k_sb = pool->k_stride_block;
  a.k_sh = pool->k_stride_head;
  a.v_sb = pool->v_stride_block;
  a.v_sh = pool->v_stride_head;
  a.q = q;
  a.tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  char* wsb = static_cast<char*>(workspace);
  a.counters = ws.bytes ? reinterpret_cast<int32_t*>(wsb) : nullptr;
  a.ws_ml = ws.bytes ? reinterpret_cast<float*>(wsb + ws.ml_off) : nullptr;
  a.ws_u = ws.bytes ? reinterpret_cast<float*>(wsb + ws.u_off) : nullptr;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = pool->num_blocks;
  a.split_log2 = pool->split_log2;
  a.row_offsets = nullptr;
  a.table_mode = pba::kTablesDense;
  a.log2P = log2_exact(pool->block_size);
  a.G = num_q_heads / pool->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.batch = batch;
  a.part_tokens = plan->partition_tokens;
  a.n_parts = plan->max_slots;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.new_slots = fused ? fused->slots : nullptr;
  a.k_new = fused ? fused->k : nullptr;
  a.v_new = fused ? fused->v : nullptr;
  pba::SharedArgs sa;
  sa.items = plan->items;
  sa.row_private = plan->row_private;
  sa.n_items = plan->num_items;
  sa.n_packed = npk;
  sa.nz_items = nz;
  return pba::launch_paged_decode_shared(a, sa, pool->head_dim, (int)pp, s) == hipSuccess
             ? PBA_OK
             : PBA_ERR_HIP;
}

}  // namespace

extern "C" {

int pba_paged_decode_shared(const pba_kv_pool* pool, const void* q, int32_t num_q_heads,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t batch, float scale, float* out,
                            float* lse, const pba_shared_plan* plan, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return shared_decode(pool, q, num_q_heads, block_tables, max_blocks_per_seq, seq_lens, batch,
                       scale, out, lse, plan, workspace, workspace_bytes, stream, nullptr);
}

int pba_paged_decode_shared_append(const pba_kv_pool* pool, const int64_t* new_slots,
                                   const void* k_new, const void* v_new, const void* q,
                                   int32_t num_q_heads, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   int32_t batch, float scale, float* out, float* lse,
                                   const pba_shared_plan* plan, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const pba::NewTokens fused{new_slots, k_new, v_new};
  return shared_decode(pool, q, num_q_heads, block_tables, max_blocks_per_seq, seq_lens, batch,
                       scale, out, lse, plan, workspace, workspace_bytes, stream, &fused);
}

}  // extern "C"

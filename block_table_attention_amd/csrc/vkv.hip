// Contiguous virtual K/V (vAttention, "M5.3 - KV Memory Layout and Exact
// Reuse", 0x06A-0x06E): one virtual reservation holds every layer's K and V
// tensor for B request slots; physical pages are created as handles and
// mapped into a slot's range on demand, so a kernel addresses a request's rows
// by its slot index alone, with no block table.
//
// Reservation: tensor x = 2 * layer + (0 for K, 1 for V) starts at x * B * R
// bytes; slot r's range of a tensor is [r R, (r + 1) R) with
// R = G * ceil(ceil(T_max / P) * P * row / G), row = H_kv * d * b; page q of a
// slot is [q G, (q + 1) G) of that range.  Inside a slot's range the rows are
// laid out as a pool of tiles of P tokens (the library's K and V tile
// layouts), so the arena is also a pba_kv_group whose block ids are
// slot * R / (P row) + j, and the ordinary append, copy and per-layer views
// work on it.  G must be a multiple of P * row, so a page always holds whole
// tiles and a mapped frontier covers a whole number of tiles.
//
// A page bundle (page q of a slot in all 2L tensors) is mapped as one unit:
// a slot's frontier advances only when every tensor's page is mapped and
// accessible (0x06D).  Freed slots may keep their pages (0x06E); a growing
// slot takes free handles first, then reclaims the highest bundle of the
// lowest-numbered inactive slot that has one.
#include <algorithm>
#include <mutex>
#include <vector>

#include "pba_internal.h"
#include "vkv_internal.h"

struct pba_vkv_arena {
  pba_vkv_config cfg;
  int device = 0;
  char* va = nullptr;
  size_t va_bytes = 0;
  int64_t row = 0;           // bytes of one token row of one tensor
  int64_t R = 0;             // bytes of one slot's range of one tensor
  int64_t pages_per_slot = 0;
  int64_t tiles_per_slot = 0;
  int tensors = 0;           // 2L
  int64_t created = 0;       // handles created
  std::vector<hipMemGenericAllocationHandle_t> free_handles;
  // mapped[slot][q * tensors + x]: handle of page q of tensor x
  std::vector<std::vector<hipMemGenericAllocationHandle_t>> mapped;
  std::vector<int64_t> frontier;  // mapped pages per slot (every tensor)
  std::vector<uint8_t> active;
  std::vector<int64_t> generation;
  int64_t maps = 0, unmaps = 0;  // page bundles
  mutable std::mutex mu;
};

namespace {

std::mutex g_registry_mu;
std::vector<pba_vkv_arena*> g_registry;

char* page_va(const pba_vkv_arena* a, int x, int64_t slot, int64_t q) {
  return a->va + ((int64_t)x * a->cfg.num_slots + slot) * a->R + q * a->cfg.page_bytes;
}

hipMemAllocationProp page_prop(int device) {
  hipMemAllocationProp prop = {};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

// Unmap the slot's highest page bundle; its handles join the free list.
bool unmap_top(pba_vkv_arena* a, int64_t slot) {
  const int64_t q = a->frontier[slot] - 1;
  auto& m = a->mapped[slot];
  bool ok = true;
  for (int x = 0; x < a->tensors; ++x) {
    ok &= hipMemUnmap(page_va(a, x, slot, q), a->cfg.page_bytes) == hipSuccess;
    a->free_handles.push_back(m[q * a->tensors + x]);
  }
  m.resize(q * a->tensors);
  a->frontier[slot] = q;
  ++a->unmaps;
  return ok;
}

// Map page q of every tensor of the slot with handles taken from the free list.
bool map_bundle(pba_vkv_arena* a, int64_t slot, int64_t q) {
  hipMemAccessDesc acc = {};
  acc.location.type = hipMemLocationTypeDevice;
  acc.location.id = a->device;
  acc.flags = hipMemAccessFlagsProtReadWrite;
  const size_t G = a->cfg.page_bytes;
  std::vector<hipMemGenericAllocationHandle_t> hs(a->free_handles.begin(),
                                                  a->free_handles.begin() + a->tensors);
  int done = 0;
  for (; done < a->tensors; ++done) {
    char* p = page_va(a, done, slot, q);
    if (hipMemMap(p, G, 0, hs[done], 0) != hipSuccess) break;
    if (hipMemSetAccess(p, G, &acc, 1) != hipSuccess) {
      (void)hipMemUnmap(p, G);
      break;
    }
  }
  if (done < a->tensors) {  // undo this bundle; the handles stay free
    for (int x = 0; x < done; ++x) (void)hipMemUnmap(page_va(a, x, slot, q), G);
    return false;
  }
  a->free_handles.erase(a->free_handles.begin(), a->free_handles.begin() + a->tensors);
  auto& m = a->mapped[slot];
  m.insert(m.end(), hs.begin(), hs.end());
  a->frontier[slot] = q + 1;
  ++a->maps;
  return true;
}

// Rows of the slot below its frontier, at most max_tokens (the rows reserved).
int64_t capacity_tokens(const pba_vkv_arena* a, int64_t slot) {
  const int64_t t = a->frontier[slot] * a->cfg.page_bytes / a->row;
  return std::min<int64_t>(t, a->cfg.max_tokens);
}

}  // namespace

namespace pba {

// Validate-mode checks of calls whose K base lies inside an arena: every row
// a call would touch must lie below its slot's mapped frontier.
int vkv_check_rows(const void* k_base, const int32_t* slots, const int32_t* lens, int64_t n) {
  std::lock_guard<std::mutex> lock(g_registry_mu);
  for (const pba_vkv_arena* a : g_registry) {
    const char* p = static_cast<const char*>(k_base);
    if (p < a->va || p >= a->va + a->va_bytes) continue;
    std::lock_guard<std::mutex> al(a->mu);
    for (int64_t i = 0; i < n; ++i) {
      if (slots[i] < 0 || slots[i] >= a->cfg.num_slots) return PBA_ERR_OUT_OF_RANGE;
      if (lens[i] > capacity_tokens(a, slots[i])) return PBA_ERR_OUT_OF_RANGE;
    }
  }
  return PBA_OK;
}

int vkv_check_slot_ids(const void* k_base, const int64_t* ids, int64_t n) {
  std::lock_guard<std::mutex> lock(g_registry_mu);
  for (const pba_vkv_arena* a : g_registry) {
    const char* p = static_cast<const char*>(k_base);
    if (p < a->va || p >= a->va + a->va_bytes) continue;
    std::lock_guard<std::mutex> al(a->mu);
    const int64_t per_slot = a->tiles_per_slot * a->cfg.block_size;
    for (int64_t i = 0; i < n; ++i) {
      if (ids[i] < 0) continue;
      const int64_t slot = ids[i] / per_slot, t = ids[i] % per_slot;
      if (slot >= a->cfg.num_slots || t >= capacity_tokens(a, slot)) return PBA_ERR_OUT_OF_RANGE;
    }
  }
  return PBA_OK;
}

// Blocks are whole tiles: a block is usable when its tile lies below the
// slot's mapped pages.
int vkv_check_blocks(const void* k_base, const int32_t* ids, int64_t n) {
  std::lock_guard<std::mutex> lock(g_registry_mu);
  for (const pba_vkv_arena* a : g_registry) {
    const char* p = static_cast<const char*>(k_base);
    if (p < a->va || p >= a->va + a->va_bytes) continue;
    std::lock_guard<std::mutex> al(a->mu);
    for (int64_t i = 0; i < n; ++i) {
      const int64_t slot = ids[i] / a->tiles_per_slot, j = ids[i] % a->tiles_per_slot;
      if (ids[i] < 0 || slot >= a->cfg.num_slots ||
          (j + 1) * a->cfg.block_size > a->frontier[slot] * a->cfg.page_bytes / a->row)
        return PBA_ERR_OUT_OF_RANGE;
    }
  }
  return PBA_OK;
}

}  // namespace pba

extern "C" {

int pba_vkv_create(const pba_vkv_config* cfg, pba_vkv_arena** out) {
  if (!cfg || !out) return PBA_ERR_NULL_ARG;
  *out = nullptr;
  const pba_vkv_config& c = *cfg;
  if (c.dtype != PBA_BF16 && c.dtype != PBA_F32) return PBA_ERR_BAD_DTYPE;
  if (c.num_layers < 1 || c.num_slots < 1 || c.num_kv_heads < 1 || c.max_tokens < 1 ||
      c.page_bytes <= 0 || c.num_handles < 0)
    return PBA_ERR_BAD_SHAPE;
  if (c.head_dim != 64 && c.head_dim != 128) return PBA_ERR_UNSUPPORTED;
  if (c.block_size < 16 || c.block_size > 256 || (c.block_size & (c.block_size - 1)))
    return PBA_ERR_UNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PBA_ERR_HIP;
  const hipMemAllocationProp prop = page_prop(dev);
  size_t gran = 0;
  if (hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityMinimum) !=
      hipSuccess)
    return PBA_ERR_HIP;
  const int64_t es = c.dtype == PBA_BF16 ? 2 : 4;
  const int64_t row = (int64_t)c.num_kv_heads * c.head_dim * es;
  const int64_t tile_set = c.block_size * row;  // P rows of every head
  if (c.page_bytes % (int64_t)gran || c.page_bytes % tile_set) return PBA_ERR_UNSUPPORTED;
  const int64_t tiles = (c.max_tokens + c.block_size - 1) / c.block_size;
  const int64_t pages = (tiles * tile_set + c.page_bytes - 1) / c.page_bytes;
  const int64_t R = pages * c.page_bytes;
  const int64_t tps = R / tile_set;
  const int tensors = 2 * c.num_layers;
  // Block ids (slot * tiles_per_slot + j) are int32 in the pool descriptor.
  if (tps * c.num_slots > INT32_MAX || tps * c.block_size > INT32_MAX) return PBA_ERR_UNSUPPORTED;
  if (c.num_handles && c.num_handles % tensors) return PBA_ERR_BAD_SHAPE;  // whole bundles
  auto* a = new pba_vkv_arena();
  a->cfg = c;
  a->device = dev;
  a->row = row;
  a->R = R;
  a->pages_per_slot = pages;
  a->tiles_per_slot = tps;
  a->tensors = tensors;
  a->va_bytes = (size_t)tensors * c.num_slots * R;
  void* va = nullptr;
  if (hipMemAddressReserve(&va, a->va_bytes, (size_t)c.page_bytes, nullptr, 0) != hipSuccess) {
    delete a;
    return PBA_ERR_HIP;
  }
  a->va = static_cast<char*>(va);
  a->mapped.resize(c.num_slots);
  a->frontier.assign(c.num_slots, 0);
  a->active.assign(c.num_slots, 0);
  a->generation.assign(c.num_slots, 0);
  for (int64_t i = 0; i < c.num_handles; ++i) {
    hipMemGenericAllocationHandle_t h;
    if (hipMemCreate(&h, (size_t)c.page_bytes, &prop, 0) != hipSuccess) {
      pba_vkv_destroy(a);
      return PBA_ERR_HIP;
    }
    a->free_handles.push_back(h);
    ++a->created;
  }
  {
    std::lock_guard<std::mutex> lock(g_registry_mu);
    g_registry.push_back(a);
  }
  *out = a;
  return PBA_OK;
}

int pba_vkv_destroy(pba_vkv_arena* a) {
  if (!a) return PBA_ERR_NULL_ARG;
  {
    std::lock_guard<std::mutex> lock(g_registry_mu);
    g_registry.erase(std::remove(g_registry.begin(), g_registry.end(), a), g_registry.end());
  }
  bool ok = hipDeviceSynchronize() == hipSuccess;
  for (int64_t s = 0; s < a->cfg.num_slots; ++s)
    while (a->frontier[s] > 0) ok &= unmap_top(a, s);
  for (auto h : a->free_handles) ok &= hipMemRelease(h) == hipSuccess;
  if (a->va) ok &= hipMemAddressFree(a->va, a->va_bytes) == hipSuccess;
  delete a;
  return ok ? PBA_OK : PBA_ERR_HIP;
}

int pba_vkv_map(pba_vkv_arena* a, int32_t slot, int64_t tokens) {
  if (!a) return PBA_ERR_NULL_ARG;
  std::lock_guard<std::mutex> lock(a->mu);
  if (slot < 0 || slot >= a->cfg.num_slots || tokens < 0) return PBA_ERR_BAD_SHAPE;
  if (tokens > a->cfg.max_tokens) return PBA_ERR_OUT_OF_RANGE;
  const int64_t need = (tokens * a->row + a->cfg.page_bytes - 1) / a->cfg.page_bytes;
  const int64_t missing = std::max<int64_t>(0, need - a->frontier[slot]);
  // Feasibility first, so that a call that cannot finish changes nothing.
  if (a->cfg.num_handles) {
    int64_t avail = (int64_t)a->free_handles.size() / a->tensors;
    for (int64_t v = 0; v < a->cfg.num_slots; ++v)
      if (v != slot && !a->active[v]) avail += a->frontier[v];
    if (avail < missing) return PBA_ERR_OUT_OF_MEMORY;
  }
  if (!a->active[slot]) {  // a new request generation: no row of the slot is valid
    a->active[slot] = 1;
    ++a->generation[slot];
  }
  const hipMemAllocationProp prop = page_prop(a->device);
  for (int64_t q = a->frontier[slot]; q < need; ++q) {
    while ((int64_t)a->free_handles.size() < a->tensors) {
      if (!a->cfg.num_handles) {  // no fixed pool: create the bundle's handles
        hipMemGenericAllocationHandle_t h;
        if (hipMemCreate(&h, (size_t)a->cfg.page_bytes, &prop, 0) != hipSuccess) return PBA_ERR_HIP;
        a->free_handles.push_back(h);
        ++a->created;
        continue;
      }
      int64_t victim = -1;
      for (int64_t v = 0; v < a->cfg.num_slots && victim < 0; ++v)
        if (v != slot && !a->active[v] && a->frontier[v] > 0) victim = v;
      // Work launched before the victim was freed may still read its pages.
      if (victim < 0 || hipDeviceSynchronize() != hipSuccess || !unmap_top(a, victim))
        return PBA_ERR_HIP;
    }
    if (!map_bundle(a, slot, q)) return PBA_ERR_HIP;
  }
  return PBA_OK;
}

int pba_vkv_free(pba_vkv_arena* a, int32_t slot, int32_t retain) {
  if (!a) return PBA_ERR_NULL_ARG;
  std::lock_guard<std::mutex> lock(a->mu);
  if (slot < 0 || slot >= a->cfg.num_slots) return PBA_ERR_BAD_SHAPE;
  if (!a->active[slot]) return PBA_ERR_OUT_OF_RANGE;
  a->active[slot] = 0;
  if (!retain) {
    if (hipDeviceSynchronize() != hipSuccess) return PBA_ERR_HIP;  // no kernel may still read it
    while (a->frontier[slot] > 0)
      if (!unmap_top(a, slot)) return PBA_ERR_HIP;
  }
  return PBA_OK;
}

int pba_vkv_group(const pba_vkv_arena* a, pba_kv_group* out, int32_t* blocks_per_slot) {
  if (!a || !out) return PBA_ERR_NULL_ARG;
  const pba_vkv_config& c = a->cfg;
  const int64_t es = c.dtype == PBA_BF16 ? 2 : 4;
  const int64_t tensor = (int64_t)c.num_slots * a->R;  // bytes of one K or V tensor
  pba_kv_group g = {};
  g.pool.k = a->va;
  g.pool.v = a->va + tensor;
  g.pool.dtype = c.dtype;
  g.pool.num_blocks = (int32_t)(a->tiles_per_slot * c.num_slots);
  g.pool.block_size = c.block_size;
  g.pool.num_kv_heads = c.num_kv_heads;
  g.pool.head_dim = c.head_dim;
  g.pool.split_log2 = 0;
  g.pool.k_stride_block = g.pool.v_stride_block = (int64_t)c.block_size * c.num_kv_heads * c.head_dim;
  g.pool.k_stride_head = g.pool.v_stride_head = (int64_t)c.block_size * c.head_dim;
  g.num_layers = c.num_layers;
  g.k_stride_layer = g.v_stride_layer = 2 * tensor / es;
  *out = g;
  if (blocks_per_slot) *blocks_per_slot = (int32_t)a->tiles_per_slot;
  return PBA_OK;
}

int pba_vkv_capacity(const pba_vkv_arena* a, int32_t slot, int64_t* tokens) {
  if (!a || !tokens) return PBA_ERR_NULL_ARG;
  std::lock_guard<std::mutex> lock(a->mu);
  if (slot < 0 || slot >= a->cfg.num_slots) return PBA_ERR_BAD_SHAPE;
  *tokens = capacity_tokens(a, slot);
  return PBA_OK;
}

int pba_vkv_get_ledgers(const pba_vkv_arena* a, pba_vkv_ledgers* out) {
  if (!a || !out) return PBA_ERR_NULL_ARG;
  std::lock_guard<std::mutex> lock(a->mu);
  const int64_t G = a->cfg.page_bytes;
  pba_vkv_ledgers l = {};
  l.reserved_bytes = (int64_t)a->va_bytes;
  l.pool_bytes = a->created * G;
  int64_t mapped = 0, inactive = 0;
  for (int64_t s = 0; s < a->cfg.num_slots; ++s) {
    mapped += a->frontier[s];
    if (!a->active[s]) inactive += a->frontier[s];
  }
  l.mapped_bytes = mapped * a->tensors * G;
  l.inactive_retained_bytes = inactive * a->tensors * G;
  l.free_bytes = (int64_t)a->free_handles.size() * G;
  l.bundle_maps = a->maps;
  l.bundle_unmaps = a->unmaps;
  l.slot_bytes = a->R;
  *out = l;
  return PBA_OK;
}

}  // extern "C"

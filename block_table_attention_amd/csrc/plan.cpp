// Host-side planner of the shared-prefix decode: from host block tables and
// lengths, the batch order in which rows that share leading blocks are
// adjacent, the shared chunks (a chunk tree over row ranges), and the work
// items and private ranges of a pba_shared_plan ("M5.3 - KV Memory Layout and
// Exact Reuse", 0x0BB: chunks with a coverage interval of sequences and each
// sequence's ordered chunk path; 0x0BD: chunk-first work for chunks covering
// more than a threshold of sequences, sequence-first work for the rest; the
// metadata is built on the host side of the kernel boundary).  No device
// access.
#include <algorithm>
#include <cstring>
#include <numeric>
#include <vector>

#include "pba.h"

namespace {

int log2_exact(int x) {
  if (x <= 0 || (x & (x - 1))) return -1;
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

struct Chunk {
  int32_t row_begin, row_end, tok_begin, tok_end;
};

// The chunk tree of rows already in sharing order.  A chunk is a maximal run
// of whole, fully visible blocks that every row of [a, b) maps to the same
// physical ids, below its ancestors' chunks; only runs covering more than
// `threshold` rows become chunks.  Chunks come in pre-order (an ancestor
// before its descendants, siblings in row order); private[r] is the first
// token of row r that no chunk covers.
void chunk_tree(const std::vector<int32_t>& t, int width, const std::vector<int32_t>& lens, int P,
                int threshold, std::vector<Chunk>& chunks, std::vector<int64_t>& priv) {
  const int B = (int)lens.size();
  std::vector<int32_t> full(B);
  for (int r = 0; r < B; ++r) full[r] = lens[r] / P;  // whole blocks row r sees
  priv.assign(B, 0);
  chunks.clear();
  struct Node {
    int a, b, j0;
  };
  std::vector<Node> stack;
  if (B > 0) stack.push_back({0, B, 0});
  auto cell = [&](int r, int j) { return t[(size_t)r * width + j]; };
  while (!stack.empty()) {
    const Node nd = stack.back();
    stack.pop_back();
    const int a = nd.a, b = nd.b, j0 = nd.j0;
    if (b - a <= threshold) {
      for (int r = a; r < b; ++r) priv[r] = (int64_t)j0 * P;
      continue;
    }
    int lim = full[a];
    for (int r = a + 1; r < b; ++r) lim = std::min(lim, full[r]);
    int j = j0;
    while (j < lim) {
      bool same = true;
      for (int r = a + 1; r < b && same; ++r) same = cell(r, j) == cell(a, j);
      if (!same) break;
      ++j;
    }
    if (j > j0) chunks.push_back({a, b, j0 * P, j * P});
    // Children: runs of rows that continue past block j with the same id.
    std::vector<Node> kids;
    for (int r = a; r < b;) {
      if (full[r] <= j) {
        priv[r] = (int64_t)j * P;
        ++r;
        continue;
      }
      int e = r + 1;
      while (e < b && full[e] > j && cell(e, j) == cell(r, j)) ++e;
      kids.push_back({r, e, j});
      r = e;
    }
    for (auto it = kids.rbegin(); it != kids.rend(); ++it) stack.push_back(*it);
  }
}

}  // namespace

extern "C" int pba_shared_plan_build(const int32_t* tables, int32_t width, const int32_t* seq_lens,
                                     int32_t batch, const pba_shared_plan_params* params,
                                     int64_t* order, int32_t* items, int32_t items_capacity,
                                     int32_t* row_private, int32_t* chunks_out,
                                     int32_t chunks_capacity, pba_shared_plan_info* info) {
  if (!params || !info) return PBA_ERR_NULL_ARG;
  const int P = params->block_size, G = params->group, pt = params->partition_tokens;
  const int tpi = params->tiles_per_item;
  if (batch < 0 || width < 1 || items_capacity < 0 || chunks_capacity < 0 ||
      params->threshold < 0 || params->reserved0 != 0 || G < 1 || pt <= 0)
    return PBA_ERR_BAD_SHAPE;
  const int lp = log2_exact(P);
  if (lp < 4 || lp > 8 || G > 16 || pt % 256 || (tpi != 1 && tpi != 2 && tpi != 4))
    return PBA_ERR_UNSUPPORTED;
  if (batch > 0 && (!tables || !seq_lens || !order || !row_private)) return PBA_ERR_NULL_ARG;
  for (int32_t r = 0; r < batch; ++r)
    if (seq_lens[r] < 0 || (int64_t)seq_lens[r] > (int64_t)width * P) return PBA_ERR_OUT_OF_RANGE;

  // Sharing order: rows sorted lexicographically by their table rows (stable),
  // so every shared chunk covers one contiguous range of rows.
  std::vector<int32_t> idx(batch);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
    const int32_t* a = tables + (size_t)x * width;
    const int32_t* b = tables + (size_t)y * width;
    return std::lexicographical_compare(a, a + width, b, b + width);
  });
  std::vector<int32_t> t((size_t)batch * width);
  std::vector<int32_t> lens(batch);
  for (int32_t i = 0; i < batch; ++i) {
    std::memcpy(&t[(size_t)i * width], tables + (size_t)idx[i] * width, sizeof(int32_t) * width);
    lens[i] = seq_lens[idx[i]];
  }
  std::vector<Chunk> chunks;
  std::vector<int64_t> priv;
  chunk_tree(t, width, lens, P, params->threshold, chunks, priv);

  // Items: every chunk cut into pieces of pt keys from its first key; the rows
  // of a piece in 16-column tiles of 16 / G rows, up to tiles_per_item per item.
  const int rpt = 16 / G;
  std::vector<int32_t> its;
  std::vector<int64_t> next_slot(batch, 0);
  int64_t chunk_rows = 0, kv_rows = 0, visits = 0;
  for (const Chunk& c : chunks) {
    const int64_t base = next_slot[c.row_begin];
    for (int r = c.row_begin; r < c.row_end; ++r)
      if (next_slot[r] != base) return PBA_ERR_BAD_SHAPE;  // not reached: a chunk's rows share their path
    const int64_t pieces = ((int64_t)c.tok_end - c.tok_begin + pt - 1) / pt;
    const int tiles = (c.row_end - c.row_begin + rpt - 1) / rpt;
    chunk_rows += c.row_end - c.row_begin;
    for (int64_t k = 0; k < pieces; ++k) {
      const int64_t tb = c.tok_begin + k * pt;
      const int64_t te = std::min<int64_t>(c.tok_end, tb + pt);
      for (int ti = 0; ti < tiles;) {
        const int left = tiles - ti;
        const int nt = std::min(tpi, left >= 4 ? 4 : (left >= 2 ? 2 : 1));
        const int row0 = c.row_begin + ti * rpt;
        const int nrows = std::min(c.row_end, c.row_begin + (ti + nt) * rpt) - row0;
        const int32_t it[8] = {row0, nrows, (int32_t)tb, (int32_t)te, (int32_t)(base + k), nt, 0, 0};
        its.insert(its.end(), it, it + 8);
        const int reads = nt == 4 ? 2 : 1;  // a group of two tiles shares one read
        kv_rows += reads * (te - tb);
        visits += reads * ((te - tb + 31) / 32);
        ti += nt;
      }
    }
    for (int r = c.row_begin; r < c.row_end; ++r) next_slot[r] += pieces;
  }
  // Longest walk first: a work-group's waves split an item's 32-key chunks
  // (all four waves over one or two tiles, two waves per tile pair of a
  // four-tile item), and the grid starts items in array order as CUs free
  // up, so an item with many steps per wave that came last would finish
  // last.  Slots are fixed per item, so the order changes no result.
  {
    const int64_t n = (int64_t)its.size() / 8;
    std::vector<int64_t> perm(n), steps(n);
    for (int64_t i = 0; i < n; ++i) {
      const int32_t* it = &its[(size_t)i * 8];
      const int64_t chunks = ((int64_t)it[3] - it[2] + 31) / 32;
      const int waves = it[5] == 4 ? 2 : 4;  // waves that split one tile group's chunks
      steps[i] = (chunks + waves - 1) / waves;
      perm[i] = i;
    }
    std::stable_sort(perm.begin(), perm.end(), [&](int64_t x, int64_t y) {
      if (steps[x] != steps[y]) return steps[x] > steps[y];
      return its[(size_t)x * 8 + 5] > its[(size_t)y * 8 + 5];
    });
    std::vector<int32_t> sorted(its.size());
    for (int64_t i = 0; i < n; ++i)
      std::copy(&its[(size_t)perm[i] * 8], &its[(size_t)perm[i] * 8] + 8, &sorted[(size_t)i * 8]);
    its.swap(sorted);
  }
  int64_t max_slots = 1, priv_parts = 1, priv_tokens = 1, partial = 0;
  for (int32_t r = 0; r < batch; ++r) {
    const int64_t rest = std::max<int64_t>(0, (int64_t)lens[r] - priv[r]);
    const int64_t pp = (rest + pt - 1) / pt;
    const int64_t slots = next_slot[r] + pp;
    max_slots = std::max(max_slots, slots);
    priv_parts = std::max(priv_parts, pp);
    priv_tokens = std::max(priv_tokens, rest);
    if (slots > 1) partial += slots;
    kv_rows += rest;
    visits += (rest + 31) / 32;
  }
  const int64_t n_items = (int64_t)its.size() / 8;
  if (n_items > INT32_MAX || max_slots > INT32_MAX) return PBA_ERR_UNSUPPORTED;
  info->num_items = (int32_t)n_items;
  info->num_chunks = (int32_t)chunks.size();
  info->max_slots = (int32_t)max_slots;
  info->private_parts = (int32_t)priv_parts;
  info->private_tokens = (int32_t)priv_tokens;
  info->partition_tokens = pt;
  info->chunk_rows = chunk_rows;
  info->kv_rows_read = kv_rows;
  info->chunk_visits = visits;
  info->partial_states = partial;
  // Sizes first: a short output buffer writes nothing.
  if (items && n_items > items_capacity) return PBA_ERR_WORKSPACE_TOO_SMALL;
  if (chunks_out && (int64_t)chunks.size() > chunks_capacity) return PBA_ERR_WORKSPACE_TOO_SMALL;
  for (int32_t i = 0; i < batch; ++i) {
    order[i] = idx[i];
    row_private[2 * i] = (int32_t)priv[i];
    row_private[2 * i + 1] = (int32_t)next_slot[i];
  }
  if (items) std::copy(its.begin(), its.end(), items);
  if (chunks_out)
    for (size_t c = 0; c < chunks.size(); ++c) {
      chunks_out[4 * c] = chunks[c].row_begin;
      chunks_out[4 * c + 1] = chunks[c].row_end;
      chunks_out[4 * c + 2] = chunks[c].tok_begin;
      chunks_out[4 * c + 3] = chunks[c].tok_end;
    }
  return PBA_OK;
}

// paged_decode: one decode query row per request over its logical K/V history.
//
// The method ("M5.3 - KV Memory Layout and Exact Reuse", 0x0A): for each logical
// block of the request, translate it through the block table, read its visible
// rows (all P, or T mod P in the last block), score them against q, and fold
// them into an online-softmax state (m, l, u); finally O = u / l.  Long rows
// are cut into partitions of `part_tokens` tokens whose states are merged with
// the log-sum-exp rule of 0x0BA (an empty partition is the identity; outputs
// are never averaged).
//
// Work decomposition on gfx950 (256 CUs, 64-lane waves):
//   work-group = (partition, kv head h, request r), 4 waves.  Wave w walks
//   the partition's chunks w, w+4, w+8, ...; the four waves merge their states
//   through LDS.  A row with one partition is written directly.  Otherwise
//   each work-group stores its partition state, and the last work-group of the
//   (request, kv head) to finish -- found with one atomic counter per pair --
//   merges the partitions in index order (deterministic) and resets the
//   counter, so no second kernel is launched.
//
// bf16 path: the G query heads of kv head h are processed together, so the
// scores of a 32-token chunk are the small dense product S^T[32 x G] =
// K[32 x d] Q^T[d x G] and the value update is O^T[d x G] += V^T[d x 32]
// P^T[32 x G].  Both run on v_mfma_f32_16x16x32_bf16 (G padded to 16 columns):
//   * the K tile is token major, so each lane's A-operand fragment (one token
//     row, 8 consecutive dims) is one 16-byte load straight from HBM;
//   * the V tile is dim major ([d][P]), so each lane's A-operand fragment for
//     the value product (one dim, 8 consecutive tokens) is again one 16-byte
//     load;
//   * the token order inside a chunk is permuted so that the score fragment a
//     lane receives (tokens 8g..8g+7 of its head) is exactly the B-operand
//     fragment it needs for the value product: no cross-lane traffic.
// No LDS staging: every loaded byte feeds exactly one MFMA of the wave that
// loaded it.  Loads are software pipelined: the next chunk's K is requested as
// soon as the score MFMAs have consumed the current K, and the next V as soon
// as the value MFMAs have consumed the current V, so each wave keeps a chunk
// of loads in flight while it computes.  Probabilities enter the value MFMA as
// a bf16 pair p = hi + lo (hi = bf16(p), lo = bf16(p - hi)), ~16 significant
// bits.  The running output is rescaled only when some head's maximum moved.
//
// Visibility: positions t >= T (tail padding, rows materialised in a shared
// block by a longer request, stale rows) are removed by selects -- scores to
// -inf, V scalars to 0 -- never by multiplying by zero, since they may hold NaN.
// Table entries at j >= ceil(T/P) are never read.
#include "pba_internal.h"

namespace pba {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kDecodeThreads / 64;
// s_waitcnt encoding (gfx9 family): vmcnt(0), expcnt and lgkmcnt unconstrained.
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-wave partial states, staged in LDS for the work-group merge.
template <int D>
struct WaveStates {
  float m[kWaves][16];
  float l[kWaves][16];
  float o[kWaves][16][D + 4];  // [head][dim]; rows padded against bank conflicts
  int last;
};

// Partition states cross work-groups (and XCDs, whose L2s are not coherent
// with each other) through memory.  Every state word is written and read by
// agent-scope atomic accesses (global_store / global_load with sc1: written
// through the XCD's L2 to the device coherence point, and read from it), so
// each word is coherent across XCDs on its own.  What the handoff adds is the
// order between a work-group's state words and its completion count: every
// wave waits until its state stores have completed (s_waitcnt vmcnt(0)), the
// work-group barrier follows, and only then does one thread increment the
// counter; the work-group that reads the final count issues its state loads
// after that increment returns.  The language-level form of this order -- a
// release increment plus an acquire fence in the merging work-group --
// compiles to an L2 write-back (buffer_wbl2) before every increment and an L2
// invalidate in the merger; both only matter for plain stores and loads,
// which the handoff does not use, and measured on MI355X they cost 6 %
// (8 x 16,384 tokens) to 85 % (the shared-prefix batch) of the decode time.
__device__ __forceinline__ int count_done(int32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_state(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two neighbouring state words in one 8-byte store (p 8-byte aligned).
__device__ __forceinline__ void st_state2(float* p, float lo, float hi) {
  const uint64_t v = (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float ld_state(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Final merge of the partition states of one (request, kv head):
//   O = sum_p w_p u_p / L,  w_p = 2^(m_p - M),  M = max_p m_p,  L = sum_p w_p l_p,
// partitions in index order, TILE at a time with a running (M, L, O).
// A thread owns dims c, c + D/4, c + D/2, c + 3D/4 of one q-head row, so it
// needs only that row's (m, l), and each load or store instruction of a wave
// covers whole runs of consecutive dims.  Every load of a tile is issued
// before any is used and none sits under a lane-dependent branch (partition
// indices are clamped in bounds and the surplus ignored), so a tile costs one
// memory round trip and the merge needs no LDS and no barrier.
template <int D, int TILE>
__device__ __forceinline__ void merge_dims(const DecodeArgs& a, int64_t row, int c, int np_r) {
  constexpr int C4 = D / 4;
  const float* ml = a.ws_ml + row * a.n_parts * 2;
  const float* uu = a.ws_u + row * a.n_parts * D + c;
  float M = -INFINITY, L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < np_r; p0 += TILE) {
    float mt[TILE], lt[TILE];
    f32x4 ut[TILE];
#pragma unroll
    for (int j = 0; j < TILE; ++j) {
      const int64_t pp = min(p0 + j, np_r - 1);
      mt[j] = ld_state(ml + 2 * pp);
      lt[j] = ld_state(ml + 2 * pp + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) ut[j][e] = ld_state(uu + pp * D + C4 * e);
    }
    float Mt = M;
#pragma unroll
    for (int j = 0; j < TILE; ++j)
      if (p0 + j < np_r) Mt = fmaxf(Mt, mt[j]);
    if (Mt == -INFINITY) continue;  // only empty states so far: identity
    const float sc = (M == -INFINITY) ? 0.f : fast_exp2(M - Mt);
    L *= sc;
    O *= sc;
#pragma unroll
    for (int j = 0; j < TILE; ++j) {
      if (p0 + j < np_r && mt[j] != -INFINITY) {
        const float w = fast_exp2(mt[j] - Mt);
        L += w * lt[j];
        O += w * ut[j];
      }
    }
    M = Mt;
  }
  const f32x4 res = (L > 0.f) ? O * (1.f / L) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4; ++e) a.out[row * D + c + C4 * e] = res[e];
  if (a.lse && c == 0) a.lse[row] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

template <int D, int TILE>
__device__ void merge_partitions(const DecodeArgs& a, int r, int h, int np_r) {
  constexpr int C4 = D / 4;
  const int G = a.G;
  const int64_t row0 = (int64_t)r * a.num_q_heads + (int64_t)h * G;
  for (int idx = threadIdx.x; idx < G * C4; idx += kDecodeThreads) {
    const int n = idx / C4;
    merge_dims<D, TILE>(a, row0 + n, idx - n * C4, np_r);
  }
}

// The final merges of nm requests of kv head h at once (rows[k] with nps[k]
// partitions): one pass of the whole work-group, so the rows' load round
// trips overlap instead of following one another.
template <int D, int TILE>
__device__ void merge_rows(const DecodeArgs& a, const int* rows, const int* nps, int nm, int h) {
  constexpr int C4 = D / 4;
  const int G = a.G;
  const int per = G * C4;
  for (int idx = threadIdx.x; idx < nm * per; idx += kDecodeThreads) {
    const int k = idx / per;
    const int rem = idx - k * per;
    const int n = rem / C4;
    merge_dims<D, TILE>(a, (int64_t)rows[k] * a.num_q_heads + (int64_t)h * G + n, rem - n * C4,
                        nps[k]);
  }
}

// The tile is sized to the partition count: clamped surplus loads in a tile
// are real memory requests.
template <int D>
__device__ void merge_row(const DecodeArgs& a, int r, int h, int np_r) {
  if (np_r <= 4)
    merge_partitions<D, 4>(a, r, h, np_r);
  else if (np_r <= 8)
    merge_partitions<D, 8>(a, r, h, np_r);
  else
    merge_partitions<D, 16>(a, r, h, np_r);
}

// Merge the wave states of one work-group; write the row (one partition) or
// the partition state; the last partition of a (request, kv head) merges all.
template <int D>
__device__ void finish_workgroup(const DecodeArgs& a, WaveStates<D>& st, int r, int h, int part,
                                 int T) {
  constexpr int C4 = D / 4;
  const int G = a.G;
  const int np_r = (T + a.part_tokens - 1) / a.part_tokens;
  for (int idx = threadIdx.x; idx < G * C4; idx += kDecodeThreads) {
    const int n = idx / C4;
    const int c = idx - n * C4;  // dims c + C4 * e, e < 4
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, st.m[w][n]);
    float L = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = st.m[w][n];
        if (mw == -INFINITY) continue;  // a wave that saw no chunk: identity
        const float wt = fast_exp2(mw - M);
        L += wt * st.l[w][n];
#pragma unroll
        for (int e = 0; e < 4; ++e) O[e] += wt * st.o[w][n][c + C4 * e];
      }
    }
    const int64_t row = (int64_t)r * a.num_q_heads + (int64_t)h * G + n;
    if (np_r == 1) {
      const f32x4 res = (L > 0.f) ? O * (1.f / L) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) a.out[row * D + c + C4 * e] = res[e];
      if (a.lse && c == 0) a.lse[row] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
    } else {
      const int64_t prow = row * a.n_parts + part;
#pragma unroll
      for (int e = 0; e < 4; ++e) st_state(a.ws_u + prow * D + c + C4 * e, O[e]);
      if (c == 0) {
        st_state(a.ws_ml + prow * 2 + 0, M);
        st_state(a.ws_ml + prow * 2 + 1, L);
      }
    }
  }
  if (np_r == 1) return;
  int32_t* counter = a.counters + (int64_t)r * a.num_kv_heads + h;
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's state stores are complete
  __syncthreads();
  if (threadIdx.x == 0) st.last = count_done(counter) == np_r - 1;
  __syncthreads();
  if (!st.last) return;
  merge_row<D>(a, r, h, np_r);
  if (threadIdx.x == 0) *counter = 0;  // ready for the next call on this workspace
}

// ---------------------------------------------------------------------------
// bf16 K/V, MFMA path
// ---------------------------------------------------------------------------
// Block tables are read-only for the whole launch: reading them through the
// constant address space lets wave-uniform lookups use scalar loads, which do
// not queue behind the vector K/V loads.
typedef const int32_t __attribute__((address_space(4))) table_t;

// What the first loads of a work-group depend on: its block-table row, the
// pool bases and strides.  These values reach the kernel as separate scalar
// arguments ahead of the argument bundle, which the build preloads into SGPRs
// (kernarg preload), so the first table read does not wait for a fetch of the
// kernel arguments.
struct PoolView {
  table_t* trow;
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_sb, k_sh, v_sb, v_sh;
  int max_blocks;
  int last_block;  // num_blocks - 1: clamp for ids read ahead of the length
  int log2P;
  int split;       // kernel view: allocator tiles hold P << split rows
  int64_t base_block = 0;  // contiguous slots: block j of the row is base_block + j
};

// Kernel block pb of a (possibly split) pool: allocator tile pb >> split, its
// rows starting at (pb mod 2^split) * P.
__device__ __forceinline__ int64_t tile_of(const PoolView& pv, int64_t pb) { return pb >> pv.split; }
__device__ __forceinline__ int row_of(const PoolView& pv, int64_t pb) {
  return (int)(pb & ((1 << pv.split) - 1)) << pv.log2P;
}

// Physical block ids of the chunk starting at t0 (one when P >= 32, two when
// P == 16).  Ids are clamped into the pool so that a lookup made before the
// request length is known (or past it) only ever addresses pool memory; rows
// past the length are masked out of the result regardless.
// Contiguous slots (IMPLICIT): no table; block j of the row is base_block + j,
// with j clamped below the row's last block so that no address past the
// request's mapped rows is formed.
template <bool IMPLICIT = false>
__device__ __forceinline__ void chunk_blocks(const PoolView& pv, int t0, int64_t& pb0,
                                             int64_t& pb1) {
  const int j0 = min(t0 >> pv.log2P, pv.max_blocks - 1);
  if constexpr (IMPLICIT) {
    pb0 = pv.base_block + j0;
    pb1 = pv.log2P == 4 ? pv.base_block + min(j0 + 1, pv.max_blocks - 1) : pb0;
  } else {
    pb0 = min(max(pv.trow[j0], 0), pv.last_block);
    pb1 = pb0;
    if (pv.log2P == 4) pb1 = min(max(pv.trow[min(j0 + 1, pv.max_blocks - 1)], 0), pv.last_block);
  }
}

template <int D>
// Rows at or past t_end (a tail chunk) are read as row t_end - 1: the same
// lines as a visible row, so a tail chunk fetches no K row beyond the end;
// their scores are masked.
__device__ __forceinline__ void load_k(u32x4 (&kf)[2][D / 32], const PoolView& pv, int h, int t0,
                                       int64_t pb0, int64_t pb1, int n, int g, int t_end) {
  const int P = 1 << pv.log2P;
#pragma unroll
  for (int at = 0; at < 2; ++at) {
    // A-operand row n of tile `at` holds chunk token 8(n>>2) + 4at + (n&3).
    const int tk = min(8 * (n >> 2) + 4 * at + (n & 3), max(t_end - 1 - t0, 0));
    const int64_t pb = (tk >= 16 && pv.log2P == 4) ? pb1 : pb0;
    const int off = row_of(pv, pb) + ((t0 + tk) & (P - 1));
    const uint16_t* kp =
        pv.k + tile_of(pv, pb) * pv.k_sb + (int64_t)h * pv.k_sh + (int64_t)off * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) kf[at][kk] = *reinterpret_cast<const u32x4*>(kp + 32 * kk);
  }
}

template <int D>
__device__ __forceinline__ void load_v(u32x4 (&vf)[D / 16], const PoolView& pv, int h, int t0,
                                       int64_t pb0, int64_t pb1, int n, int g) {
  const int P = 1 << pv.log2P;
  // A-operand row n of tile mt is dim 16mt + n; its k-slots are tokens 8g..8g+7.
  const int tv = 8 * g;
  const int64_t pb = (tv >= 16 && pv.log2P == 4) ? pb1 : pb0;
  const int Pa = P << pv.split;  // rows of an allocator tile: V's dim stride
  const int off = row_of(pv, pb) + ((t0 + tv) & (P - 1));
  const uint16_t* vp =
      pv.v + tile_of(pv, pb) * pv.v_sb + (int64_t)h * pv.v_sh + (int64_t)n * Pa + off;
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt)
    vf[mt] = *reinterpret_cast<const u32x4*>(vp + (int64_t)(16 * mt) * Pa);
}

// Fused append: the wave that reads a row's last position T - 1 writes the
// step's new token there first (the kv_append of one token per row), so the
// decode of that row reads it in the same launch.  Lanes 0 .. D/8 - 1 hold
// 16 bytes of the K row each, every lane two scalars of the V row (dims
// 2 lane, 2 lane + 1); they are loaded when the wave starts and stored just
// before the wave prefetches the chunk holding T - 1.  The address is the
// caller's slot, which the contract makes the row's position T - 1 through
// its table (validate mode checks it), so the stores hit the bytes that
// chunk's loads read; a wavefront-scope release/acquire orders the stores of
// some lanes before the loads of others (the wave's memory operations are
// performed in order, so the fences need no instruction).
struct NewToken {
  u32x4 k;      // 8 K scalars (lanes < D / 8)
  uint32_t v;   // 2 V scalars
  int64_t slot;
};

template <int D>
__device__ __forceinline__ void load_new_token(NewToken& nt, const DecodeArgs& a, int r, int h,
                                               int lane) {
  const int64_t row = ((int64_t)r * a.num_kv_heads + h) * D;
  const uint16_t* kn = static_cast<const uint16_t*>(a.k_new) + row;
  const uint16_t* vn = static_cast<const uint16_t*>(a.v_new) + row;
  if (lane < D / 8) nt.k = *reinterpret_cast<const u32x4*>(kn + 8 * lane);
  if (lane < D / 2) nt.v = *reinterpret_cast<const uint32_t*>(vn + 2 * lane);
}

template <int D>
__device__ __forceinline__ void store_new_token(const NewToken& nt, const PoolView& pv, int h,
                                                int lane) {
  const int P = 1 << pv.log2P;
  const int64_t pb = nt.slot >> pv.log2P;  // kernel block of the slot
  const int off = row_of(pv, pb) + (int)(nt.slot & (P - 1));
  uint16_t* kp = const_cast<uint16_t*>(pv.k) + tile_of(pv, pb) * pv.k_sb + (int64_t)h * pv.k_sh +
                 (int64_t)off * D;
  const int Pa = P << pv.split;
  uint16_t* vp = const_cast<uint16_t*>(pv.v) + tile_of(pv, pb) * pv.v_sb + (int64_t)h * pv.v_sh + off;
  if (lane < D / 8) *reinterpret_cast<u32x4*>(kp + 8 * lane) = nt.k;
  if (lane < D / 2) {
    vp[(int64_t)(2 * lane) * Pa] = (uint16_t)(nt.v & 0xFFFFu);
    vp[(int64_t)(2 * lane + 1) * Pa] = (uint16_t)(nt.v >> 16);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The running maximum moves only when a chunk's maximum exceeds it by more
// than this many log2 units, so probabilities stay below 2^kRescaleSlack and
// the accumulators are rescaled (a multiply per accumulator) only a few times
// per row instead of whenever the maximum grows.  Every (m, l, u) state keeps
// l and u relative to its own m, so merges are unaffected.
constexpr float kRescaleSlack = 8.f;

// Scores enter the softmax unscaled and |scale| * log2(e) is folded into the
// exponent (one fma per score).  A negative scale is carried by the queries:
// their bf16 sign bits are flipped when they are loaded.
__device__ __forceinline__ float abs_scale(float scale_log2) { return fabsf(scale_log2); }
__device__ __forceinline__ uint32_t q_sign_mask(float scale_log2) {
  return scale_log2 < 0.f ? 0x80008000u : 0u;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Online-softmax update of one 16-column tile over a 32-token chunk.  s holds
// this lane's raw scores: tokens tbase + 4 at + i (tbase = t0 + 8 g) of
// column n.  In a tail chunk (tail = true) tokens at or past t_end are
// removed; columns without a query (zero q, padding) are computed like the
// others and never stored.  Returns the probabilities as the B operand of
// the value product, split p = hi + lo into two bf16 parts (~16 significant
// bits).
template <int MT>
__device__ __forceinline__ void softmax_tile(const f32x4 (&s)[2], bool tail, int tbase, int t_end,
                                             float sl, float& m_run, float& l_run,
                                             f32x4 (&acc)[MT], bf16x8& phi, bf16x8& plo) {
  float x[8];
#pragma unroll
  for (int at = 0; at < 2; ++at)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * at + i] = s[at][i];
  if (tail) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (tbase + j < t_end) ? x[j] : -INFINITY;
  }
  float cmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
  const float cm = cmax * sl;
  if (__any(cm > m_run + kRescaleSlack)) {  // the first chunk always takes this
    const float m_new = fmaxf(m_run, cm);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
  }
  const float nm = -m_run;
  float p[8];
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = fast_exp2(fmaf(x[j], sl, nm));
    psum += p[j];
  }
  l_run += psum;
  u32x4 hi, lo;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hi[q] = pack_bf16(p[2 * q], p[2 * q + 1]);
    const float h0 = __uint_as_float(hi[q] << 16);
    const float h1 = __uint_as_float(hi[q] & 0xFFFF0000u);
    lo[q] = pack_bf16(p[2 * q] - h0, p[2 * q + 1] - h1);
  }
  phi = __builtin_bit_cast(bf16x8, hi);
  plo = __builtin_bit_cast(bf16x8, lo);
}

// One 32-token chunk of a wave: the score product over its K fragments, the
// online-softmax update of (m_run, l_run), the value product into acc, and
// the loads of the wave's next chunk tn, each issued as soon as the registers
// it overwrites are consumed.  Tokens at or past t_end are masked out;
// columns at or past ncols carry no probability mass.
// `pv`, `h` and `tn_end` describe the chunk being prefetched (the same row as
// the current chunk, except in the balanced kernel, where the next chunk may
// belong to another (request, kv head)); t0 and t_end describe the current one.
// vmode (balanced kernel, blocks of 64 or more tokens): the V rows of a
// 64-token half-tile share 128-byte lines, which a wave that walks its chunks
// in order would read one chunk apart (the line may leave the L2 in between).
//   0: load the V of chunk tn;
//   1: also load the V of chunk tn + 32 (same block) into vf2;
//   2: chunk tn's V is already in vf2 (loaded with the previous chunk).
// pf = false: the wave's last chunk, nothing to prefetch.  The loop exits
// right after it, so every iteration that reaches the next one has the same
// loads in flight (the waits in the loop stay exact), and the wave's final
// waits do not cover reloads of a chunk it no longer needs.
template <int D, bool IMPLICIT = false>
__device__ __forceinline__ void chunk_step(const PoolView& pv, int h, int t0, int tn, int t_end,
                                           int tn_end, int ncols, float scale_log2,
                                           const bf16x8 (&qf)[D / 32], u32x4 (&kf)[2][D / 32],
                                           u32x4 (&vf)[D / 16], float& m_run, float& l_run,
                                           f32x4 (&acc)[D / 16], int n, int g, bool pf = true,
                                           u32x4 (*vf2)[D / 16] = nullptr, int vmode = 0) {
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  constexpr int CH = 32;
  int64_t nb0, nb1;
  chunk_blocks<IMPLICIT>(pv, tn, nb0, nb1);
  // A second block that starts at or past the end holds no visible row: its
  // loads go to the first block instead (and are masked), so no block past
  // the row's last one is ever read.
  if (tn + 16 >= tn_end) nb1 = nb0;

  // Scores S^T = K Q^T: lane gets tokens 8g + 4a + i (i < 4) of head n.
  f32x4 s[2];
#pragma unroll
  for (int at = 0; at < 2; ++at) {
    s[at] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      s[at] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[at][kk]),
                                                       qf[kk], s[at], 0, 0, 0);
  }
  if (pf) load_k<D>(kf, pv, h, tn, nb0, nb1, n, g, tn_end);

  const int tbase = t0 + 8 * g;  // token of k-slot j = 0 of this lane
  const bool tail = t0 + CH > t_end;  // wave uniform
  bf16x8 phi, plo;
  softmax_tile<MT>(s, tail, tbase, t_end, scale_log2, m_run, l_run, acc, phi, plo);

  // Tail chunk: zero the V scalars of tokens >= t_end (they may hold NaN).
  if (tail) {
    const int cnt = t_end - tbase;  // valid tokens among this lane's 8
    u32x4 mask;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      mask[q] = (cnt >= 2 * q + 2) ? 0xFFFFFFFFu : ((cnt == 2 * q + 1) ? 0x0000FFFFu : 0u);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) vf[mt] &= mask;
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const bf16x8 va = __builtin_bit_cast(bf16x8, vf[mt]);
    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, acc[mt], 0, 0, 0);
    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, acc[mt], 0, 0, 0);
  }
  if (vmode == 2) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) vf[mt] = (*vf2)[mt];
  } else if (pf) {
    load_v<D>(vf, pv, h, tn, nb0, nb1, n, g);
    if (vmode == 1) load_v<D>(*vf2, pv, h, tn + CH, nb0, nb0, n, g);
  }
}

// Grid: x = kv head, y = request, z = partition.  Work-groups reach the
// XCDs round-robin in linear order, so with the partition as the slowest axis
// every XCD gets an even share of the first partitions (never empty) and of
// the later ones (empty past a short request's end).
// MODE: kTablesDense, kTablesRagged, or kTablesContiguous (`tables` is the
// request-slot index [batch] and `max_blocks` the blocks of one slot: row r
// reads blocks slot*max_blocks + j, with no table).
template <int D, int MODE>
__global__ __launch_bounds__(kDecodeThreads) void decode_bf16_kernel(
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens,
    const void* __restrict__ kbase, const void* __restrict__ vbase, int32_t max_blocks,
    int32_t part_tokens, int32_t log2P, int32_t last_block, int32_t k_sb, int32_t k_sh,
    DecodeArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int KK = D / 32;  // k-steps of the score product
  constexpr int MT = D / 16;  // 16-dim tiles of the value product
  constexpr int CH = 32;      // tokens per chunk

  __shared__ WaveStates<D> st;

  const int h = blockIdx.x;
  const int r = blockIdx.y;
  const int part = blockIdx.z;
  const int lane = threadIdx.x & 63;
  // Wave-uniform (SGPR): chunk positions and block-table reads become scalar.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;  // head column of this lane
  const int g = lane >> 4;  // k-group of this lane
  const int G = a.G;
  const int p_begin = part * part_tokens;
  // Dense tables: row r at r * max_blocks.  Ragged tables: row r is entries
  // [row_offsets[r], row_offsets[r + 1]) of one array (one more scalar round
  // trip before the first table read).
  int64_t toff = (int64_t)r * max_blocks;
  int nblk = max_blocks;
  if constexpr (MODE == kTablesRagged) {
    const int64_t __attribute__((address_space(4)))* ro =
        (const int64_t __attribute__((address_space(4)))*)a.row_offsets;
    toff = ro[r];
    nblk = (int)(ro[r + 1] - toff);
    if (nblk < 1) return;  // an empty row (rejected in validate mode)
  }
  // Start-up: the request length and this wave's first block-table entries
  // (or its slot) come back in one scalar round trip; q and the first
  // chunk's K and V are requested right after, and only by waves that have a
  // chunk, so the work-groups of partitions past a short request's end, and
  // waves past it, read nothing else.  Issue order q, K, V keeps the in-loop
  // waits exact.
  const int T = seq_lens[r];
  PoolView pv{(table_t*)(tables + toff),
              static_cast<const uint16_t*>(kbase),
              static_cast<const uint16_t*>(vbase),
              k_sb, k_sh, a.v_sb, a.v_sh, nblk, last_block, log2P, a.split_log2};
  constexpr bool IMPLICIT = MODE == kTablesContiguous;
  if constexpr (IMPLICIT) {
    const int slot = ((const int32_t __attribute__((address_space(4)))*)tables)[r];
    pv.base_block = (int64_t)slot * max_blocks;
    pv.max_blocks = max(1, (T + (1 << log2P) - 1) >> log2P);
  }
  int t0 = p_begin + wave * CH;
  int64_t pb0, pb1;
  chunk_blocks<IMPLICIT>(pv, t0, pb0, pb1);
  // The bundle fields the first loads need are fetched with the length, not
  // after the test on it (which would add a scalar round trip).
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);
  const int num_q_heads = a.num_q_heads;
  asm volatile("" ::"s"(qbase), "s"(num_q_heads), "s"(G), "s"(pv.v_sb), "s"(pv.v_sh),
               "s"(pv.split));
  if (p_begin >= T) return;  // empty partition: never counted, never read
  if (t0 + 16 >= T) pb1 = pb0;  // no block past the row's last one is read
  const int p_end = min(T, p_begin + part_tokens);
  // This wave's chunks: p_begin + wave*CH + k*kWaves*CH for k < n_w.
  const int span = p_end - p_begin - wave * CH;
  const int n_w = span > 0 ? (span + kWaves * CH - 1) / (kWaves * CH) : 0;
  // Fused append: this wave writes the row's new token if it reads T - 1,
  // before prefetching the chunk that holds it (t_new).
  NewToken nt;
  nt.slot = -1;
  int t_new = -1;
  if (a.new_slots && p_end == T) {
    const int64_t slot = ((const int64_t __attribute__((address_space(4)))*)a.new_slots)[r];
    const int c_new = (T - 1 - p_begin) / CH;
    if (slot >= 0 && c_new % kWaves == wave) {
      nt.slot = slot;
      t_new = p_begin + c_new * CH;
    }
  }
  if (t_new == t0) {  // the wave's first chunk: write before its first loads
    load_new_token<D>(nt, a, r, h, lane);
    store_new_token<D>(nt, pv, h, lane);
    t_new = -1;
  }

  u32x4 qraw[KK];
  u32x4 kf[2][KK];
  u32x4 vf[MT];
  if (n_w > 0) {
    // Q^T fragments (B operand of the score product): lane holds dims
    // 32kk + 8g .. +8 of query head n (padding lanes read head 0).
    const uint16_t* qrow =
        qbase + ((int64_t)r * num_q_heads + (int64_t)h * G + (n < G ? n : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qraw[kk] = *reinterpret_cast<const u32x4*>(qrow + 32 * kk + 8 * g);
    __builtin_amdgcn_sched_barrier(0);
    load_k<D>(kf, pv, h, t0, pb0, pb1, n, g, T);
    __builtin_amdgcn_sched_barrier(0);
    load_v<D>(vf, pv, h, t0, pb0, pb1, n, g);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (t_new >= 0) load_new_token<D>(nt, a, r, h, lane);
  // Padding heads (n >= G) get zero queries; applied after every first load
  // is in flight.
  const uint32_t qs = q_sign_mask(a.scale_log2);
  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[kk] = __builtin_bit_cast(bf16x8, (n < G ? qraw[kk] : u32x4{0u, 0u, 0u, 0u}) ^ qs);

  float m_run = -INFINITY;  // running max (log2 domain) of head n
  float l_run = 0.f;        // this lane's share of the running sum
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < n_w; ++it, t0 += kWaves * CH) {
    // Next chunk of this wave (none after the last).
    const bool more = it + 1 < n_w;
    const int tn = more ? t0 + kWaves * CH : t0;
    if (tn == t_new && more) store_new_token<D>(nt, pv, h, lane);
    chunk_step<D, IMPLICIT>(pv, h, t0, tn, T, T, G, abs_scale(a.scale_log2), qf, kf, vf, m_run, l_run, acc, n,
                            g, more);
  }

  // Wave state -> LDS.  acc[mt][i] is O^T[dim 16mt + 4g + i][head n]: four
  // consecutive dims of one head per lane.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (g == 0) {
    st.m[wave][n] = m_run;
    st.l[wave][n] = l_run;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4*>(&st.o[wave][n][16 * mt + 4 * g]) = acc[mt];
  __syncthreads();
  finish_workgroup<D>(a, st, r, h, part, T);
}

// ---------------------------------------------------------------------------
// Balanced decode: the batch's chunks spread evenly over the chip
// ---------------------------------------------------------------------------
// The (request, kv head) segments of the batch -- ceil(T/32) chunks each --
// are laid end to end, request major, on a cost axis: a chunk spans
// kChunkUnits and every segment seg_cost more in front of its chunks (its
// fixed cost: the q load, a new table row, the epilogue, the pieces), so
// waves over many short segments get fewer chunks.  With V units and NG
// work-groups (one per CU), work-group w owns the chunks that start in
// [w V / NG, (w+1) V / NG), and its wave i those in the i-th quarter of that
// range (seg_cost = 0 splits the chunk count evenly).
// A wave walks its range chunk by chunk with the grid kernel's software
// pipeline, the prefetch crossing from one segment into the next (the next
// segment's q is requested with it), so a ragged batch keeps every CU
// streaming until the end instead of waiting on its longest rows.  With
// blocks of 64 or more tokens, the prefetch of an even chunk also loads its
// odd partner's V, which shares the same 128-byte lines.
// A segment inside one wave's range is written by that wave.  A segment cut
// by wave boundaries leaves one partial state per wave, in LDS; after the
// loops the work-group merges the pieces of each such segment that lie in its
// range (in range order): into the rows if the segment lies inside the
// work-group's range, otherwise into one work-group piece in memory, which is
// counted with one atomic per (request, kv head); the work-group that brings
// the count to the number of work-groups over the segment merges their pieces
// and resets the counter.
// Dynamic LDS (flat_lds_bytes): row lengths T[B] and their chunk prefix sums
// pre[B + 1] (the host keeps the chunk total below 2^31), the waves' chunk
// totals, the segment of each wave piece (r * H + h, or -1), and the wave
// pieces themselves in the accumulator order of piece_at.

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Pieces are stored in the accumulator order of the MFMA tiles, columns
// fastest: value (dim 16 mt + 4 q + i, column cn) of slot s sits at
//   s G D + ((mt 4 + i) 4 + q) G + cn,
// so a wave's store of one accumulator register covers 4 G consecutive floats
// and a merge load of 64 consecutive items covers whole 4 G-float runs: no
// bank conflicts for the wave pieces in LDS, and whole 64-byte runs for the
// work-group pieces in memory, whose device-coherent stores and loads (they
// bypass the XCD's L2) would otherwise each fill a quarter of every 64-byte
// write or read.
__device__ __forceinline__ int64_t piece_at(int64_t s, int G, int D, int mt, int i, int q, int cn) {
  return s * G * D + (int64_t)((mt * 4 + i) * 4 + q) * G + cn;
}

// Merge n pieces (slot_of(j), j < n, in order) of item j (column j % G, dims
// 16 mt + 4 q .. + 3 with q = (j / G) % 4, mt = j / (4 G)) into (M, L, O) and
// write the rows, or store one piece at dst_slot.  The loads of a tile of
// pieces are all issued before any is used.
template <int D, typename SlotOf>
__device__ void flat_merge_item(const DecodeArgs& a, const FlatArgs& f, SlotOf slot_of, int n,
                                int64_t row0, int item, bool to_rows, int64_t dst_slot) {
  const int G = a.G;
  const int cn = item % G;
  const int rq = item / G;
  const int q = rq & 3;
  const int mt = rq >> 2;
  float M = -INFINITY, L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  constexpr int TILE = 8;
  for (int j0 = 0; j0 < n; j0 += TILE) {
    float mt_[TILE], lt[TILE];
    f32x4 ut[TILE];
#pragma unroll
    for (int j = 0; j < TILE; ++j) {
      const int64_t s = slot_of(min(j0 + j, n - 1));
      mt_[j] = ld_state(f.piece_ml + (s * G + cn) * 2);
      lt[j] = ld_state(f.piece_ml + (s * G + cn) * 2 + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) ut[j][e] = ld_state(f.piece_u + piece_at(s, G, D, mt, e, q, cn));
    }
#pragma unroll
    for (int j = 0; j < TILE; ++j) {
      if (j0 + j >= n || mt_[j] == -INFINITY) continue;
      const float Mn = fmaxf(M, mt_[j]);
      const float sa = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
      const float sb = fast_exp2(mt_[j] - Mn);
      L = L * sa + lt[j] * sb;
      O = O * sa + ut[j] * sb;
      M = Mn;
    }
  }
  if (to_rows) {
    const f32x4 res = L > 0.f ? O * (1.f / L) : f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(a.out + (row0 + cn) * D + 16 * mt + 4 * q) = res;
    if (a.lse && rq == 0) a.lse[row0 + cn] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) st_state(f.piece_u + piece_at(dst_slot, G, D, mt, e, q, cn), O[e]);
    if (rq == 0) {
      st_state(f.piece_ml + (dst_slot * G + cn) * 2, M);
      st_state(f.piece_ml + (dst_slot * G + cn) * 2 + 1, L);
    }
  }
}

// Merge the n wave pieces of item `item` held in LDS (local slots packed 3
// bits each, in range order) and write the rows, or store one work-group
// piece at dst_slot in memory.
template <int D>
__device__ void lds_merge_item(const DecodeArgs& a, const FlatArgs& f, const float* l_ml,
                               const float* l_u, uint32_t packed, int n, int64_t row0, int item,
                               bool to_rows, int64_t dst_slot) {
  const int G = a.G;
  const int cn = item % G;
  const int rq = item / G;
  const int q = rq & 3;
  const int mt = rq >> 2;
  float M = -INFINITY, L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < n; ++j) {
    const int ls = (packed >> (3 * j)) & 7;
    const float m = l_ml[(ls * G + cn) * 2];
    if (m == -INFINITY) continue;
    const float l = l_ml[(ls * G + cn) * 2 + 1];
    f32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = l_u[piece_at(ls, G, D, mt, e, q, cn)];
    const float Mn = fmaxf(M, m);
    const float sa = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
    const float sb = fast_exp2(m - Mn);
    L = L * sa + l * sb;
    O = O * sa + u * sb;
    M = Mn;
  }
  if (to_rows) {
    const f32x4 res = L > 0.f ? O * (1.f / L) : f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(a.out + (row0 + cn) * D + 16 * mt + 4 * q) = res;
    if (a.lse && rq == 0) a.lse[row0 + cn] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) st_state(f.piece_u + piece_at(dst_slot, G, D, mt, e, q, cn), O[e]);
    if (rq == 0) {
      st_state(f.piece_ml + (dst_slot * G + cn) * 2, M);
      st_state(f.piece_ml + (dst_slot * G + cn) * 2 + 1, L);
    }
  }
}

// kFused (dense tables): the step's new tokens are written in the launch.  A
// row's token for kv head h goes to the pool from the wave that walks the
// last chunk of segment (row, h), before that wave requests the chunk (with
// 64-token or larger blocks, before the request of the even chunk whose V
// load also brings the last chunk's V).  Each wave keeps the token of the
// segment it is walking in registers and requests the next segment's token
// when it writes one, so the rows arrive a step ahead of their store.
template <int D, int MODE, bool kFused = false>
__global__ __launch_bounds__(kDecodeThreads) void decode_bf16_flat_kernel(
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens,
    const void* __restrict__ kbase, const void* __restrict__ vbase, int32_t max_blocks,
    int32_t log2P, int32_t last_block, int32_t k_sb, int32_t k_sh, DecodeArgs a, FlatArgs f) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  constexpr int CH = 32;
  constexpr bool IMPLICIT = MODE == kTablesContiguous;

  extern __shared__ __align__(16) int32_t flat_lds[];
  const int B = a.batch;
  const int H = a.num_kv_heads;
  const int G = a.G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int P = 1 << log2P;
  const int wave = uni(tid >> 6);
  int32_t* const s_T = flat_lds;                 // [B]
  int32_t* const s_pre = s_T + B;                // [B + 1]
  int32_t* const s_wsum = s_pre + B + 1;         // [kWaves]
  int32_t* const s_pend = s_wsum + kWaves;       // [2 kWaves]
  float* const l_ml = reinterpret_cast<float*>(flat_lds + flat_head_words(B));
  float* const l_u = l_ml + 2 * kWaves * G * 2;

  // Rows and their chunk counts; prefix sums over the batch.  A row with no
  // visible token (rejected in validate mode) has no chunk and gets out = 0,
  // lse = -inf from work-group 0: the identity state.
  const int per = (B + kDecodeThreads - 1) / kDecodeThreads;
  const int rb = min(B, tid * per), re = min(B, rb + per);
  int local = 0;
  for (int r = rb; r < re; ++r) {
    const int T = seq_lens[r];
    s_T[r] = T;
    if (T > 0) {
      local += H * ((T + CH - 1) / CH);
    } else if (blockIdx.x == 0) {
      for (int i = 0; i < a.num_q_heads; ++i) {
        const int64_t row = (int64_t)r * a.num_q_heads + i;
        for (int c = 0; c < D; ++c) a.out[row * D + c] = 0.f;
        if (a.lse) a.lse[row] = -INFINITY;
      }
    }
  }
  // Inclusive scan of the thread totals: within each wave by shuffles, then
  // over the waves' totals.
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wsum[wave] = incl;
  if (tid < 2 * kWaves) s_pend[tid] = -1;
  __syncthreads();
  {
    int run = incl - local;
    for (int w = 0; w < wave; ++w) run += s_wsum[w];
    for (int r = rb; r < re; ++r) {
      s_pre[r] = run;
      const int T = s_T[r];
      if (T > 0) run += H * ((T + CH - 1) / CH);
    }
    if (tid == kDecodeThreads - 1) s_pre[B] = run;
  }
  __syncthreads();

  // Ranges: this work-group's, then this wave's quarter of it.
  const int64_t C = uni(s_pre[B]);
  // NG <= C: every work-group range spans at least kChunkUnits, so no range
  // between two chunks of one segment is empty (the merge counts every
  // work-group between a segment's first and last chunk).
  const int64_t NG = min((int64_t)gridDim.x, C);
  const int64_t wg = blockIdx.x;
  if (wg >= NG) return;
  const int64_t A = f.seg_cost;
  const int64_t V = kChunkUnits * C + A * H * B;
  // Start of row r on the cost axis, and the position of chunk k of head h of
  // row r (nch chunks per head).
  auto vpre = [&](int r) -> int64_t { return kChunkUnits * (int64_t)s_pre[r] + A * H * r; };
  auto chunk_pos = [&](int r, int h, int k, int nch) -> int64_t {
    return vpre(r) + h * (kChunkUnits * (int64_t)nch + A) + A + kChunkUnits * (int64_t)k;
  };
  // The largest row r with mul pre[r] + add r <= x (a nondecreasing key that
  // row 0 meets): a binary search over groups of 64 rows, then one compare
  // per lane and a ballot, so the dependent LDS reads number log2(B / 64) + 1.
  auto last_row_le = [&](int64_t mul, int64_t add, int64_t x) -> int {
    int glo = 0, ghi = (B - 1) >> 6;
    while (glo < ghi) {
      const int mid = (glo + ghi + 1) >> 1;
      if (mul * uni(s_pre[64 * mid]) + add * (64 * mid) <= x) glo = mid; else ghi = mid - 1;
    }
    const int rr = 64 * glo + lane;
    const bool ok = rr < B && mul * (int64_t)s_pre[min(rr, B)] + add * rr <= x;
    return uni(64 * glo + (int)__popcll(__ballot(ok)) - 1);
  };
  // The first chunk that starts at or after position x (C past the end).
  auto first_chunk = [&](int64_t x) -> int64_t {
    if (x >= V) return C;
    const int r = last_row_le(kChunkUnits, A * H, x);
    const int T = uni(s_T[r]);
    const int64_t nch = T > 0 ? (T + CH - 1) / CH : 0;
    const int64_t span = kChunkUnits * nch + A;
    const int64_t rel = x - vpre(r);
    const int64_t base = uni(s_pre[r]);
    const int64_t hh = span > 0 ? rel / span : H;
    if (hh >= H) return base + H * nch;
    const int64_t off = rel - hh * span;
    const int64_t k = off <= A ? 0 : (off - A + kChunkUnits - 1) / kChunkUnits;
    return k >= nch ? base + (hh + 1) * nch : base + hh * nch + k;
  };
  const int64_t x0 = wg * V / NG, x1 = (wg + 1) * V / NG;
  const int64_t cb = first_chunk(x0 + (x1 - x0) * wave / kWaves);
  const int64_t ce = first_chunk(x0 + (x1 - x0) * (wave + 1) / kWaves);
  // The work-group's chunks [gb, ge): the first wave's start, the last one's end.
  __shared__ int64_t s_gbe[2];
  if (lane == 0 && wave == 0) s_gbe[0] = cb;
  if (lane == 0 && wave == kWaves - 1) s_gbe[1] = ce;
  // Work-group owning the chunk at position p: the largest w with
  // floor(w V / NG) <= p.
  auto wg_owner = [&](int64_t p) -> int64_t { return ((p + 1) * NG + V - 1) / V - 1; };

  // Reads of one row's table: dense rows at r * max_blocks; ragged rows from
  // row_offsets; contiguous rows are a slot's blocks.
  auto view = [&](int rr, int TT) {
    int64_t toff = (int64_t)rr * max_blocks;
    int nb = max_blocks;
    if constexpr (MODE == kTablesRagged) {
      const int64_t __attribute__((address_space(4)))* ro =
          (const int64_t __attribute__((address_space(4)))*)a.row_offsets;
      toff = ro[rr];
      nb = (int)(ro[rr + 1] - toff);
    } else if constexpr (MODE == kTablesContiguous) {
      toff = (int64_t)((const int32_t __attribute__((address_space(4)))*)tables)[rr] * max_blocks;
    }
    PoolView pv{(table_t*)(tables + toff),
                static_cast<const uint16_t*>(kbase),
                static_cast<const uint16_t*>(vbase),
                k_sb, k_sh, a.v_sb, a.v_sh, nb, last_block, log2P, a.split_log2};
    if constexpr (IMPLICIT) {
      pv.trow = nullptr;
      pv.base_block = toff;
      pv.max_blocks = max(1, (TT + P - 1) >> log2P);
    }
    return pv;
  };
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q);
  auto load_q = [&](u32x4 (&qr)[KK], int rr, int hh) {
    const uint16_t* qrow =
        qbase + ((int64_t)rr * a.num_q_heads + (int64_t)hh * G + (n < G ? n : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qr[kk] = *reinterpret_cast<const u32x4*>(qrow + 32 * kk + 8 * g);
  };

  if (cb < ce) {
    // Segment cursor at cb: row r (the largest with pre[r] <= cb), head h, chunk k.
    int r = last_row_le(1, 0, cb);
    int T = uni(s_T[r]);
    int nch = (T + CH - 1) / CH;
    const int off0 = (int)(cb - uni(s_pre[r]));
    int h = off0 / nch;
    int k = off0 - h * nch;

    PoolView pv = view(r, T);
    u32x4 qraw[KK];
    u32x4 kf[2][KK];
    u32x4 vf[MT];
    u32x4 vf2[MT];
    // Chunk pairs (2j, 2j + 1) of one segment share V lines when the kernel
    // block holds 64 tokens or more: the even chunk's load brings both.
    const bool pairs = log2P >= 6;
    bool have2 = false;  // vf2 holds the V of the chunk after the one in vf
    // Fused step: the token of segment (nt_r, nt_h), written before the
    // request of chunk kx of that segment when kx (or, in pairs, kx + 1) is
    // its last chunk.
    NewToken nt;
    nt.slot = -1;
    int nt_r = -1, nt_h = 0;
    auto load_token = [&](int rr, int hh) {
      nt_r = rr;
      nt_h = hh;
      nt.slot = -1;
      if (rr >= 0) {
        nt.slot = ((const int64_t __attribute__((address_space(4)))*)a.new_slots)[rr];
        load_new_token<D>(nt, a, rr, hh, lane);
      }
    };
    auto write_token_before = [&](const PoolView& pw, int rx, int hx, int kx, int nchx) {
      if (rx == nt_r && hx == nt_h &&
          (kx == nchx - 1 || (pairs && !(kx & 1) && kx + 1 == nchx - 1))) {
        if (nt.slot >= 0) store_new_token<D>(nt, pw, hx, lane);
        // The next segment: the next kv head, else the next row with tokens.
        int r3 = rx, h3 = hx + 1;
        if (h3 == H) {
          h3 = 0;
          do {
            ++r3;
          } while (r3 < B && uni(s_T[r3]) <= 0);
          if (r3 >= B) r3 = -1;
        }
        load_token(r3, h3);
      }
    };
    if constexpr (kFused) {
      load_token(r, h);
      write_token_before(pv, r, h, k, nch);
    }
    {
      load_q(qraw, r, h);
      int64_t pb0, pb1;
      const int t0 = k * CH;
      chunk_blocks<IMPLICIT>(pv, t0, pb0, pb1);
      if (t0 + 16 >= T) pb1 = pb0;
      __builtin_amdgcn_sched_barrier(0);
      load_k<D>(kf, pv, h, t0, pb0, pb1, n, g, T);
      __builtin_amdgcn_sched_barrier(0);
      load_v<D>(vf, pv, h, t0, pb0, pb1, n, g);
      if (pairs && !(k & 1) && k + 1 < nch && cb + 1 < ce) {
        load_v<D>(vf2, pv, h, t0 + CH, pb0, pb0, n, g);
        have2 = true;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const uint32_t qs = q_sign_mask(a.scale_log2);
    bf16x8 qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, (n < G ? qraw[kk] : u32x4{0u, 0u, 0u, 0u}) ^ qs);

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool first_seg = true;
    int k_first = k;  // first chunk of this wave's piece of the current segment

    for (int64_t c = cb; c < ce; ++c) {
      const bool last = c + 1 == ce;
      const bool seg_end = last || k + 1 == nch;
      const bool new_seg = !last && k + 1 == nch;
      int r2 = r, h2 = h, k2 = k, T2 = T, nch2 = nch;
      if (!last) {
        if (k + 1 < nch) {
          k2 = k + 1;
        } else {
          k2 = 0;
          if (h + 1 < H) {
            h2 = h + 1;
          } else {
            h2 = 0;
            do {
              ++r2;
              T2 = uni(s_T[r2]);
            } while (T2 <= 0);
            nch2 = (T2 + CH - 1) / CH;
          }
        }
      }
      const PoolView pvn = r2 == r ? pv : view(r2, T2);
      if constexpr (kFused) {
        if (!last) write_token_before(pvn, r2, h2, k2, nch2);
      }
      u32x4 qnext[KK];
      if (new_seg) load_q(qnext, r2, h2);
      // The prefetched chunk (k2): its V came with the previous load, or it
      // starts a pair whose second chunk this wave also reads.
      int vmode = 0;
      if (have2) {
        vmode = 2;
        have2 = false;
      } else if (pairs && !last && !(k2 & 1) && k2 + 1 < nch2 && c + 2 < ce) {
        vmode = 1;
        have2 = true;
      }
      chunk_step<D, IMPLICIT>(pvn, h2, k * CH, k2 * CH, T, T2, G, abs_scale(a.scale_log2), qf, kf, vf,
                              m_run, l_run, acc, n, g, !last, &vf2, vmode);
      if (seg_end) {
        float l_tot = l_run + __shfl_xor(l_run, 16, 64);
        l_tot += __shfl_xor(l_tot, 32, 64);
        if (k_first == 0 && k + 1 == nch) {
          // The whole segment is this wave's: write the rows.
          const int64_t row = (int64_t)r * a.num_q_heads + (int64_t)h * G + n;
          if (n < G) {
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              *reinterpret_cast<f32x4*>(a.out + row * D + 16 * mt + 4 * g) = acc[mt] * inv;
            if (a.lse && g == 0)
              a.lse[row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
          }
        } else {
          // A cut segment: this wave's piece goes to its LDS slot.
          const int ls = wave * 2 + (first_seg ? 0 : 1);
          if (n < G) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int i = 0; i < 4; ++i) l_u[piece_at(ls, G, D, mt, i, g, n)] = acc[mt][i];
            if (g == 0) {
              l_ml[(ls * G + n) * 2] = m_run;
              l_ml[(ls * G + n) * 2 + 1] = l_tot;
            }
          }
          if (lane == 0) s_pend[ls] = r * H + h;
        }
        m_run = -INFINITY;
        l_run = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        first_seg = false;
        k_first = 0;
      }
      if (new_seg) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          qf[kk] = __builtin_bit_cast(bf16x8, (n < G ? qnext[kk] : u32x4{0u, 0u, 0u, 0u}) ^ qs);
      }
      if (r2 != r) pv = pvn;
      r = r2;
      h = h2;
      k = k2;
      T = T2;
      nch = nch2;
    }
  }
  // Pieces: every wave's LDS pieces are written, then the work-group merges.
  // All cut segments of the range go through each step together: (1) merge
  // each segment's wave pieces -- into the rows if it lies inside this range,
  // else into one work-group piece in memory; (2) count the work-group pieces;
  // (3) the last work-group of a segment merges its work-group pieces into
  // the rows.
  __syncthreads();
  __shared__ int s_seg[2 * kWaves];
  __shared__ uint32_t s_packed[2 * kWaves];  // wave pieces: 3-bit local slots 2w + which
  __shared__ int s_np[2 * kWaves];
  __shared__ int s_last[2 * kWaves];
  __shared__ int64_t s_w0[2 * kWaves];
  __shared__ int s_nseg;
  if (tid == 0) {
    int ns = 0;
    for (int qi = 0; qi < 2 * kWaves; ++qi) {
      const int seg = s_pend[qi];
      if (seg < 0) continue;
      int at = 0;
      while (at < ns && s_seg[at] != seg) ++at;
      if (at == ns) {
        s_seg[ns] = seg;
        s_packed[ns] = 0;
        s_np[ns] = 0;
        ++ns;
      }
      s_packed[at] |= (uint32_t)qi << (3 * s_np[at]);
      ++s_np[at];
    }
    s_nseg = ns;
  }
  __syncthreads();
  const int nseg = uni(s_nseg);
  if (nseg == 0) return;
  constexpr int C4 = D / 4;
  const int items = G * C4;
  // This work-group's chunks [gb, ge).
  const int64_t gb = s_gbe[0], ge = s_gbe[1];
  // A segment's rows and its chunks [s0, s1).
  auto seg_info = [&](int si, int& pr, int& ph, int64_t& s0, int64_t& s1) {
    const int seg = s_seg[si];
    pr = seg / H;
    ph = seg - pr * H;
    const int pn = (s_T[pr] + CH - 1) / CH;
    s0 = (int64_t)s_pre[pr] + (int64_t)ph * pn;
    s1 = s0 + pn;
  };
  for (int idx = tid; idx < nseg * items; idx += kDecodeThreads) {
    const int si = idx / items;
    const int item = idx - si * items;
    int pr, ph;
    int64_t s0, s1;
    seg_info(si, pr, ph, s0, s1);
    const int64_t row0 = (int64_t)pr * a.num_q_heads + (int64_t)ph * G;
    const bool inside = s0 >= gb && s1 <= ge;
    // Work-group slot 0: the segment began before this range; 1: it ends after it.
    const int64_t wslot = wg * 2 + (s0 < gb ? 0 : 1);
    lds_merge_item<D>(a, f, l_ml, l_u, s_packed[si], s_np[si], row0, item, inside, wslot);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (tid < nseg) {
    int pr, ph;
    int64_t s0, s1;
    seg_info(tid, pr, ph, s0, s1);
    int last = 0;
    if (!(s0 >= gb && s1 <= ge)) {
      // The work-groups over the segment: owners of its first and last chunk.
      const int pn = (int)(s1 - s0);
      const int64_t w0 = wg_owner(chunk_pos(pr, ph, 0, pn));
      const int nwg = (int)(wg_owner(chunk_pos(pr, ph, pn - 1, pn)) - w0 + 1);
      last = count_done(a.counters + (int64_t)pr * H + ph) == nwg - 1 ? nwg : 0;
      s_w0[tid] = w0;
    }
    s_last[tid] = last;  // the number of work-group pieces when this one merges
  }
  __syncthreads();
  for (int idx = tid; idx < nseg * items; idx += kDecodeThreads) {
    const int si = idx / items;
    if (!s_last[si]) continue;
    const int item = idx - si * items;
    int pr, ph;
    int64_t s0, s1;
    seg_info(si, pr, ph, s0, s1);
    const int64_t w0 = s_w0[si];
    // Work-group w0 holds the segment's start (its slot 1); the others hold
    // segments that began before their ranges (slot 0).
    auto wg_slot = [&](int j) { return (w0 + j) * 2 + (j == 0 ? 1 : 0); };
    const int64_t row0 = (int64_t)pr * a.num_q_heads + (int64_t)ph * G;
    flat_merge_item<D>(a, f, wg_slot, s_last[si], row0, item, true, 0);
  }
  if (tid < nseg && s_last[tid]) {
    int pr, ph;
    int64_t s0, s1;
    seg_info(tid, pr, ph, s0, s1);
    a.counters[(int64_t)pr * H + ph] = 0;  // ready for the next call on this workspace
  }
}

// ---------------------------------------------------------------------------
// Shared-prefix execution: chunk-first and sequence-first items in one launch
// ---------------------------------------------------------------------------
// A chunk is a run of whole blocks that every row of a contiguous range of the
// batch maps to the same physical ids.  Each (row, q-head) pair is one column
// of the MFMA products; a 16-column tile holds 16/G rows of one kv head.
//  * chunk-first item (grid z < nz_items): a piece [tb, te) of a chunk and the
//    rows it covers, in 1, 2 or 4 tiles of 16 columns.  Tiles go in groups of
//    two; the waves of a group split its 32-token chunks and each wave serves
//    both tiles from one K/V load, so one read serves up to 64 query columns.
//  * sequence-first item (grid z >= nz_items): a piece of one row's private
//    range [private_begin, T), split from private_begin.  These planes come
//    last in dispatch order, after the chunk-first items (which the planner
//    lists longest walk first).
//  * packed private group (flat index 0 .. n_packed - 1 of the chunk-first
//    planes, ahead of the items; only when the plan bounds every private
//    range to a few chunks): the private ranges of four consecutive rows,
//    one wave each, in place of the sequence-first planes.  Short and first,
//    they store their states and leave, so the rows' merges fall to the
//    items that end last.
// Every item leaves one partial state per column in its row's slot list; the
// last contributor of a (row, kv head) merges the row's slots in slot order,
// so the result does not depend on which work-group finishes last.
// Grid: x = kv head, y = request (chunk-first: item index low part), z as above.
typedef const int32_t __attribute__((address_space(4))) item_t;

constexpr int kItemInts = 8;      // row0, nrows, tb, te, slot, tiles, 0, 0
constexpr int kMaxItemRows = 64;  // 4 tiles x 16 rows (G = 1)

// One 32-token chunk for NT 16-column tiles that share its K and V (the
// chunk-first items): one K load and one V load serve every tile, each tile
// keeps its own online-softmax state.  Otherwise as chunk_step.
template <int D, int NT>
__device__ __forceinline__ void chunk_step_nt(const PoolView& pv, int h, int t0, int tn, int t_end,
                                              const int (&ncols)[NT], float scale_log2,
                                              const bf16x8 (&qf)[NT][D / 32],
                                              u32x4 (&kf)[2][D / 32], u32x4 (&vf)[D / 16],
                                              float (&m_run)[NT], float (&l_run)[NT],
                                              f32x4 (&acc)[NT][D / 16], int n, int g, bool pf) {
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  constexpr int CH = 32;
  int64_t nb0, nb1;
  chunk_blocks(pv, tn, nb0, nb1);
  if (tn + 16 >= t_end) nb1 = nb0;  // no block past the piece's last one is read

  f32x4 s[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int at = 0; at < 2; ++at) {
      s[t][at] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        s[t][at] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, kf[at][kk]), qf[t][kk], s[t][at], 0, 0, 0);
    }
  if (pf) load_k<D>(kf, pv, h, tn, nb0, nb1, n, g, t_end);

  const int tbase = t0 + 8 * g;
  const bool tail = t0 + CH > t_end;  // wave uniform
  bf16x8 phi[NT], plo[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    softmax_tile<MT>(s[t], tail, tbase, t_end, scale_log2, m_run[t], l_run[t], acc[t], phi[t],
                     plo[t]);

  // Tail chunk: zero the V scalars of tokens >= t_end (they may hold NaN).
  if (tail) {
    const int cnt = t_end - tbase;
    u32x4 mask;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      mask[q] = (cnt >= 2 * q + 2) ? 0xFFFFFFFFu : ((cnt == 2 * q + 1) ? 0x0000FFFFu : 0u);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) vf[mt] &= mask;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const bf16x8 va = __builtin_bit_cast(bf16x8, vf[mt]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi[t], acc[t][mt], 0, 0, 0);
      acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo[t], acc[t][mt], 0, 0, 0);
    }
  }
  if (pf) load_v<D>(vf, pv, h, tn, nb0, nb1, n, g);
}

// The walk of one piece [tb, te) for an item's tiles, and the merge of the
// waves' states into each column's row or slot.  The tiles form groups of NT
// (NT = 2 for items of 2 or 4 tiles): the waves of a group split the piece's
// chunks and each wave serves all NT tiles of its group from one K/V load,
// so a wave walks piece / (32 * waves per group) chunks whatever the tiles.
// The states go through LDS one tile of each group at a time.
// kFused (a fused step's kernel) and new_slot >= 0 (a private piece holding
// its row's position te - 1): the wave that reads te - 1 first writes the
// row's new token there, as the grid kernel does.
template <int D, int NT, bool kFused = false>
__device__ __forceinline__ void shared_item(const DecodeArgs& a, WaveStates<D>& st, int* s_slots,
                                            const PoolView& pv, int h, int row0, int nrows, int tb,
                                            int te, int tiles, int slot, int rT, int rpb, int rps,
                                            int part_tokens, int wave, int n, int g,
                                            int64_t new_slot = -1) {
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  constexpr int CH = 32;
  constexpr int C4 = D / 4;
  const int G = a.G;
  const int rpt = 16 / G;           // rows per 16-column tile
  const int groups = tiles / NT;
  const int wpg = kWaves / groups;  // waves per group
  const int grp = wave / wpg;
  const int sub = wave - grp * wpg;
  int ncols[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) ncols[j] = max(0, min(rpt, nrows - (grp * NT + j) * rpt)) * G;
  const int first = tb + sub * CH;
  const int stride = wpg * CH;
  const int span = te - first;
  const int n_w = (span > 0 && ncols[0] > 0) ? (span + stride - 1) / stride : 0;

  int t0 = first;
  // Fused append: the chunk holding te - 1 is this wave's if it is one of
  // first + k stride.
  const int lane = threadIdx.x & 63;
  NewToken nt;
  nt.slot = -1;
  int t_new = -1;
  if (kFused && new_slot >= 0 && n_w > 0) {
    const int c_new = (te - 1 - tb) / CH;
    if (c_new % wpg == sub) {
      nt.slot = new_slot;
      t_new = tb + c_new * CH;
    }
  }
  // The token's rows are requested with the chunk's table entries, so a
  // write into the wave's first chunk costs no round trip of its own.
  if (kFused && t_new >= 0) load_new_token<D>(nt, a, row0, h, lane);
  u32x4 qraw[NT][KK];
  u32x4 kf[2][KK];
  u32x4 vf[MT];
  if (n_w > 0) {
    int64_t pb0, pb1;
    chunk_blocks(pv, t0, pb0, pb1);
    if (t0 + 16 >= te) pb1 = pb0;  // no block past the piece's last one is read
    if (kFused && t_new == first) {  // the wave's first chunk: written before its loads
      store_new_token<D>(nt, pv, h, lane);
      t_new = -1;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int cn = n < ncols[j] ? n : 0;
      const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                             ((int64_t)(row0 + (grp * NT + j) * rpt + cn / G) * a.num_q_heads +
                              (int64_t)h * G + cn % G) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qraw[j][kk] = *reinterpret_cast<const u32x4*>(qrow + 32 * kk + 8 * g);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_k<D>(kf, pv, h, t0, pb0, pb1, n, g, te);
    __builtin_amdgcn_sched_barrier(0);
    load_v<D>(vf, pv, h, t0, pb0, pb1, n, g);
    __builtin_amdgcn_sched_barrier(0);
  }
  bf16x8 qf[NT][KK];
  float m_run[NT], l_run[NT];
  f32x4 acc[NT][MT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[j][kk] = __builtin_bit_cast(bf16x8, (n < ncols[j] ? qraw[j][kk] : u32x4{0u, 0u, 0u, 0u}) ^
                                                 q_sign_mask(a.scale_log2));
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int it = 0; it < n_w; ++it, t0 += stride) {
    const bool more = it + 1 < n_w;
    const int tn = more ? t0 + stride : t0;
    if (kFused && tn == t_new && more) store_new_token<D>(nt, pv, h, lane);
    chunk_step_nt<D, NT>(pv, h, t0, tn, te, ncols, abs_scale(a.scale_log2), qf, kf, vf, m_run, l_run, acc, n,
                         g, more);
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    l_run[j] += __shfl_xor(l_run[j], 16, 64);
    l_run[j] += __shfl_xor(l_run[j], 32, 64);
  }
  // Slot count of each row, clamped to the workspace's slots per row.
  if ((int)threadIdx.x < nrows) {
    const int ns = rps + (rT > rpb ? (rT - rpb + part_tokens - 1) / part_tokens : 0);
    s_slots[threadIdx.x] = min(max(ns, 0), a.n_parts);
  }
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    if (p) __syncthreads();  // the previous tile's merge has read the LDS states
    if (g == 0) {
      st.m[wave][n] = m_run[p];
      st.l[wave][n] = l_run[p];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4*>(&st.o[wave][n][16 * mt + 4 * g]) = acc[p][mt];
    __syncthreads();
    // Columns of tile gi * NT + p of every group gi: column n -> item row
    // t * rpt + n / G, q-head h * G + n % G; the tile's state merges the
    // states of its group's waves.
    for (int idx = threadIdx.x; idx < groups * 16 * C4; idx += kDecodeThreads) {
      const int col = idx / C4;
      const int c = idx - col * C4;  // dims c + C4 * e, e < 4
      const int gi = col >> 4;
      const int cn = col & 15;
      const int t = gi * NT + p;
      const int ri = t * rpt + cn / G;
      if (cn >= rpt * G || ri >= nrows) continue;
      const int w0 = gi * wpg;
      const int w1 = w0 + wpg;
      float M = -INFINITY;
      for (int w = w0; w < w1; ++w) M = fmaxf(M, st.m[w][cn]);
      float L = 0.f;
      f32x4 O = {0.f, 0.f, 0.f, 0.f};
      if (M != -INFINITY) {
        for (int w = w0; w < w1; ++w) {
          const float mw = st.m[w][cn];
          if (mw == -INFINITY) continue;
          const float wt = fast_exp2(mw - M);
          L += wt * st.l[w][cn];
#pragma unroll
          for (int e = 0; e < 4; ++e) O[e] += wt * st.o[w][cn][c + C4 * e];
        }
      }
      const int64_t row = (int64_t)(row0 + ri) * a.num_q_heads + (int64_t)h * G + cn % G;
      if (s_slots[ri] == 1) {
        const f32x4 res = (L > 0.f) ? O * (1.f / L) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) a.out[row * D + c + C4 * e] = res[e];
        if (a.lse && c == 0) a.lse[row] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
      } else {
        const int64_t prow = row * a.n_parts + slot;
#pragma unroll
        for (int e = 0; e < 4; ++e) st_state(a.ws_u + prow * D + c + C4 * e, O[e]);
        if (c == 0) st_state2(a.ws_ml + prow * 2, M, L);
      }
    }
  }
}

// Private ranges of up to four rows [row0, row0 + nrows), one wave each, for
// plans that bound every private range to a few chunks: wave w walks row
// row0 + w's positions [pb, T) alone and writes the state to the row's slot,
// or the row itself when that is its only slot.  s_slots[w] gets the row's
// slot count, 0 when the row has no private position (nothing to count).
template <int D, bool kFused>
__device__ __forceinline__ void packed_private(const DecodeArgs& a, const SharedArgs& sa,
                                               int* s_slots, const int32_t* tables,
                                               const PoolView& pv0, int h, int row0, int nrows,
                                               int part_tokens, int wave, int lane, int n, int g,
                                               float (*o)[D + 4]) {
  constexpr int KK = D / 32;
  constexpr int MT = D / 16;
  constexpr int CH = 32;
  const int G = a.G;
  const int r = row0 + wave;
  int T = 0, pb = 0, ps = -1;
  // Fused step: the row's new slot and rows are requested with its length.
  NewToken nt;
  nt.slot = -1;
  if (wave < nrows) {
    T = a.seq_lens[r];
    pb = sa.row_private[2 * r];
    ps = sa.row_private[2 * r + 1];
    if (kFused) {
      nt.slot = a.new_slots[r];
      load_new_token<D>(nt, a, r, h, lane);
    }
  }
  const bool work = wave < nrows && pb >= 0 && pb < T && ps >= 0 && ps < a.n_parts;
  const int ns = work ? min(ps + (T - pb + part_tokens - 1) / part_tokens, a.n_parts) : 0;
  if (lane == 0 && wave < nrows) s_slots[wave] = ns;
  if (!work) return;

  PoolView pv = pv0;
  pv.trow = (table_t*)(tables + (int64_t)r * pv0.max_blocks);
  const int ncols[1] = {G};
  // Fused append: the row's new token, at position T - 1 of this range, is
  // written just before the wave requests the chunk holding it.
  const int t_new = kFused && nt.slot >= 0 ? pb + (T - 1 - pb) / CH * CH : -1;
  u32x4 qraw[1][KK];
  u32x4 kf[2][KK];
  u32x4 vf[MT];
  {
    int64_t pb0, pb1;
    chunk_blocks(pv, pb, pb0, pb1);
    if (pb + 16 >= T) pb1 = pb0;  // no block past the row's last one is read
    if (kFused && t_new == pb) store_new_token<D>(nt, pv, h, lane);
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((int64_t)r * a.num_q_heads + (int64_t)h * G + (n < G ? n : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qraw[0][kk] = *reinterpret_cast<const u32x4*>(qrow + 32 * kk + 8 * g);
    __builtin_amdgcn_sched_barrier(0);
    load_k<D>(kf, pv, h, pb, pb0, pb1, n, g, T);
    __builtin_amdgcn_sched_barrier(0);
    load_v<D>(vf, pv, h, pb, pb0, pb1, n, g);
    __builtin_amdgcn_sched_barrier(0);
  }
  bf16x8 qf[1][KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[0][kk] = __builtin_bit_cast(bf16x8, (n < G ? qraw[0][kk] : u32x4{0u, 0u, 0u, 0u}) ^
                                               q_sign_mask(a.scale_log2));
  float m_run[1] = {-INFINITY}, l_run[1] = {0.f};
  f32x4 acc[1][MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[0][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int n_w = (T - pb + CH - 1) / CH;
  int t0 = pb;
  for (int it = 0; it < n_w; ++it, t0 += CH) {
    const bool more = it + 1 < n_w;
    if (kFused && more && t0 + CH == t_new) store_new_token<D>(nt, pv, h, lane);
    chunk_step_nt<D, 1>(pv, h, t0, more ? t0 + CH : t0, T, ncols, abs_scale(a.scale_log2), qf, kf,
                        vf, m_run, l_run, acc, n, g, more);
  }
  float L = l_run[0] + __shfl_xor(l_run[0], 16, 64);
  L += __shfl_xor(L, 32, 64);
  const float M = m_run[0];
  if (ns == 1) {
    if (n >= G) return;
    const int64_t row = (int64_t)r * a.num_q_heads + (int64_t)h * G + n;
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4*>(a.out + row * D + 16 * mt + 4 * g) = acc[0][mt] * inv;
    if (a.lse && g == 0) a.lse[row] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
  } else {
    // The state goes out through the wave's own LDS rows: each lane holds 4
    // dims of a head 16 bytes apart from its neighbours', so stored directly
    // every 64-byte write request would carry 16 bytes; read back, a store
    // instruction writes whole runs of D words (8 bytes per lane).
    const int64_t prow0 = ((int64_t)r * a.num_q_heads + (int64_t)h * G) * a.n_parts + ps;
    if (n < G) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4*>(&o[n][16 * mt + 4 * g]) = acc[0][mt];
      if (g == 0) st_state2(a.ws_ml + (prow0 + (int64_t)n * a.n_parts) * 2, M, L);
    }
    // The LDS writes of every lane precede the reads (one wave: in order).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    for (int e = lane; e < G * (D / 2); e += 64) {
      const int cn = e / (D / 2);
      const int d = 2 * (e - cn * (D / 2));
      const f32x2 v = *reinterpret_cast<const f32x2*>(&o[cn][d]);
      st_state2(a.ws_u + (prow0 + (int64_t)cn * a.n_parts) * D + d, v[0], v[1]);
    }
  }
}

// kFused: a fused step (a.new_slots set), in a kernel of its own so that the
// plain decode keeps its registers.
template <int D, bool kFused>
__global__ __launch_bounds__(kDecodeThreads) void decode_bf16_shared_kernel(
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens,
    const void* __restrict__ kbase, const void* __restrict__ vbase, int32_t max_blocks,
    int32_t part_tokens, int32_t log2P, int32_t last_block, int32_t k_sb, int32_t k_sh,
    DecodeArgs a, SharedArgs sa) {
  static_assert(D == 64 || D == 128, "head_dim");

  __shared__ WaveStates<D> st;
  __shared__ int s_slots[kMaxItemRows];  // slot count of each row of the item
  __shared__ int s_last[kMaxItemRows];

  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int G = a.G;
  const int rpt = 16 / G;  // rows per 16-column tile

  int row0, nrows, tb = 0, te = 0, slot = 0, tiles = 1;
  int64_t new_slot = -1;  // fused step: the row's new token, for its last private piece
  bool packed = false;
  if ((int)blockIdx.z < sa.nz_items) {
    const int fa = blockIdx.y + gridDim.y * blockIdx.z;
    if (fa >= sa.n_items + sa.n_packed) return;
    packed = fa < sa.n_packed;
  }
  if (packed) {
    // Four rows' private ranges, one wave each, ahead of the items in the
    // same planes: short groups that store their states and leave, so that
    // the rows' merges fall to the items (longest first) that end last.
    row0 = 4 * (blockIdx.y + gridDim.y * blockIdx.z);
    nrows = min(4, a.batch - row0);
  } else if ((int)blockIdx.z < sa.nz_items) {
    const int fa = blockIdx.y + gridDim.y * blockIdx.z - sa.n_packed;
    item_t* it = (item_t*)(sa.items + (int64_t)kItemInts * fa);
    row0 = it[0];
    nrows = it[1];
    tb = it[2];
    te = it[3];
    slot = it[4];
    tiles = it[5];
    // Items are device data checked only in validate mode: a malformed one
    // must not address outside the batch, the LDS row arrays or the slots.
    if ((tiles != 1 && tiles != 2 && tiles != 4) || row0 < 0 || nrows < 1 ||
        nrows > tiles * rpt || row0 + nrows > a.batch || tb < 0 || te <= tb)
      return;
  } else {
    const int r = blockIdx.y;
    const int part = blockIdx.z - sa.nz_items;
    item_t* rp = (item_t*)(sa.row_private + 2 * (int64_t)r);
    const int T = seq_lens[r];
    const int pbeg = rp[0];
    // Fused step: the row's new slot, requested with its length.
    const int64_t slot_r =
        kFused ? ((const int64_t __attribute__((address_space(4)))*)a.new_slots)[r] : -1;
    tb = pbeg + part * part_tokens;
    if (tb >= T || pbeg < 0) return;  // empty piece: never counted, never read
    te = min(T, tb + part_tokens);
    row0 = r;
    nrows = 1;
    slot = rp[1] + part;
    tiles = 1;
    if (kFused && te == T) new_slot = slot_r;
  }
  if (slot < 0 || slot >= a.n_parts) return;
  // Length and private range of the item's rows: requested now, used after
  // the loop (slot counts), so the loads wait in flight meanwhile.
  int rT = 0, rpb = 0, rps = 0;
  if (!packed && (int)threadIdx.x < nrows) {
    const int rr = row0 + threadIdx.x;
    rT = seq_lens[rr];
    rpb = sa.row_private[2 * rr];
    rps = sa.row_private[2 * rr + 1];
  }

  const PoolView pv{(table_t*)(tables + (int64_t)row0 * max_blocks),
                    static_cast<const uint16_t*>(kbase), static_cast<const uint16_t*>(vbase),
                    k_sb, k_sh, a.v_sb, a.v_sh, max_blocks, last_block, log2P, a.split_log2};
  if (packed)
    packed_private<D, kFused>(a, sa, s_slots, tables, pv, h, row0, nrows, part_tokens, wave, lane,
                              n, g, st.o[wave]);
  else if (tiles >= 2)
    shared_item<D, 2>(a, st, s_slots, pv, h, row0, nrows, tb, te, tiles, slot, rT, rpb, rps,
                      part_tokens, wave, n, g);
  else
    shared_item<D, 1, kFused>(a, st, s_slots, pv, h, row0, nrows, tb, te, tiles, slot, rT, rpb,
                              rps, part_tokens, wave, n, g, new_slot);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's state stores are complete
  __syncthreads();
  if ((int)threadIdx.x < nrows) {
    const int ns = s_slots[threadIdx.x];
    int last = 0;
    if (ns > 1) {
      int32_t* counter = a.counters + (int64_t)(row0 + threadIdx.x) * a.num_kv_heads + h;
      last = count_done(counter) == ns - 1;
    }
    s_last[threadIdx.x] = last;
  }
  __syncthreads();
  // The rows this work-group completed, merged together.
  __shared__ int s_mrow[kMaxItemRows];
  __shared__ int s_mnp[kMaxItemRows];
  __shared__ int s_nm, s_maxnp;
  if (threadIdx.x == 0) {
    int nm = 0, mx = 0;
    for (int i = 0; i < nrows; ++i) {
      if (!s_last[i]) continue;
      s_mrow[nm] = row0 + i;
      s_mnp[nm] = s_slots[i];
      mx = max(mx, s_slots[i]);
      ++nm;
    }
    s_nm = nm;
    s_maxnp = mx;
  }
  __syncthreads();
  const int nm = s_nm;
  if (nm == 0) return;
  if (s_maxnp <= 4)
    merge_rows<D, 4>(a, s_mrow, s_mnp, nm, h);
  else if (s_maxnp <= 8)
    merge_rows<D, 8>(a, s_mrow, s_mnp, nm, h);
  else
    merge_rows<D, 16>(a, s_mrow, s_mnp, nm, h);
  if ((int)threadIdx.x < nm) a.counters[(int64_t)s_mrow[threadIdx.x] * a.num_kv_heads + h] = 0;
}

// ---------------------------------------------------------------------------
// fp32 K/V, VALU path (64-token chunks; lane = token for scores, lane = dim
// for the value update)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_f32_kernel(DecodeArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int CH = 64;
  constexpr int DPL = D / 64;  // dims per lane in the value update

  __shared__ WaveStates<D> st;
  __shared__ float sq[16][D];
  __shared__ float sp[kWaves][16][CH];

  const int h = blockIdx.x;
  const int r = blockIdx.y;
  const int part = blockIdx.z;

  const int T = a.seq_lens[r];
  const int p_begin = part * a.part_tokens;
  if (p_begin >= T) return;
  const int p_end = min(T, p_begin + a.part_tokens);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = a.G;
  const int log2P = a.log2P;
  const int P = 1 << log2P;
  const int nblk = (T + P - 1) >> log2P;

  const float* qsrc = static_cast<const float*>(a.q) + ((int64_t)r * a.num_q_heads + (int64_t)h * G) * D;
  for (int i = threadIdx.x; i < 16 * D; i += kDecodeThreads) {
    const int gg = i / D;
    sq[gg][i - gg * D] = (gg < G) ? qsrc[i] : 0.f;
  }
  __syncthreads();

  const float* kpool = static_cast<const float*>(a.k);
  const float* vpool = static_cast<const float*>(a.v);
  // Dense or ragged row of the block table (see decode_bf16_kernel).
  const int32_t* trow =
      a.tables + (a.row_offsets ? a.row_offsets[r] : (int64_t)r * a.max_blocks);
  const int split = a.split_log2;
  const int qmask = (1 << split) - 1;

  float m_run[16], l_run[16], u[16][DPL];
#pragma unroll
  for (int gg = 0; gg < 16; ++gg) {
    m_run[gg] = -INFINITY;
    l_run[gg] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) u[gg][e] = 0.f;
  }

  // Fused step: the wave whose chunk holds T - 1 writes the row's new token
  // (K: D / 4 lanes of four floats; V: a lane per dim, P apart) just before
  // it reads that chunk.
  int t_new = -1;
  int64_t slot_new = -1;
  if (a.new_slots && p_end == T) {
    slot_new = a.new_slots[r];
    const int c_new = (T - 1 - p_begin) / CH;
    if (slot_new >= 0 && c_new % kWaves == wave) t_new = p_begin + c_new * CH;
  }

  for (int t0 = p_begin + wave * CH; t0 < p_end; t0 += kWaves * CH) {
    if (t0 == t_new) {
      const int64_t pbn = slot_new >> log2P;
      const int offn = (int)(slot_new & (P - 1));
      const int rown = ((int)(pbn & qmask) << log2P) + offn;
      const int64_t src = ((int64_t)r * a.num_kv_heads + h) * D;
      if (lane < D / 4)
        *reinterpret_cast<f32x4*>(const_cast<float*>(kpool) + (pbn >> split) * a.k_sb +
                                  (int64_t)h * a.k_sh + (int64_t)rown * D + 4 * lane) =
            *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.k_new) + src + 4 * lane);
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const int c = lane + 64 * e;
        const_cast<float*>(vpool)[(pbn >> split) * a.v_sb + (int64_t)h * a.v_sh +
                                  (int64_t)c * (P << split) + rown] =
            static_cast<const float*>(a.v_new)[src + c];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    const int t = t0 + lane;
    const bool valid = t < T;
    const int j = min(t >> log2P, nblk - 1);
    const int64_t pb = trow[j];
    const float* krow = kpool + (pb >> split) * a.k_sb + (int64_t)h * a.k_sh +
                        (int64_t)(((int)(pb & qmask) << log2P) + (t & (P - 1))) * D;
    float s[16];
#pragma unroll
    for (int gg = 0; gg < 16; ++gg) s[gg] = 0.f;
    for (int c = 0; c < D; c += 4) {
      const f32x4 kv = *reinterpret_cast<const f32x4*>(krow + c);
#pragma unroll
      for (int gg = 0; gg < 16; ++gg)
        if (gg < G) s[gg] += sq[gg][c] * kv[0] + sq[gg][c + 1] * kv[1] + sq[gg][c + 2] * kv[2] +
                             sq[gg][c + 3] * kv[3];
    }
    float alpha[16];
#pragma unroll
    for (int gg = 0; gg < 16; ++gg) {
      if (gg >= G) continue;
      const float x = valid ? s[gg] * a.scale_log2 : -INFINITY;
      float cm = x;
#pragma unroll
      for (int msk = 32; msk >= 1; msk >>= 1) cm = fmaxf(cm, __shfl_xor(cm, msk, 64));
      const float m_new = fmaxf(m_run[gg], cm);
      alpha[gg] = fast_exp2(m_run[gg] - m_new);
      m_run[gg] = m_new;
      const float pv = fast_exp2(x - m_new);
      l_run[gg] = l_run[gg] * alpha[gg] + pv;
      sp[wave][gg][lane] = pv;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int gg = 0; gg < 16; ++gg)
      if (gg < G)
#pragma unroll
        for (int e = 0; e < DPL; ++e) u[gg][e] *= alpha[gg];
    // Value update: lane = dim c (+64), tokens t0 .. t0+63 in runs of 4.
    for (int t4 = 0; t4 < CH; t4 += 4) {
      const int tt = t0 + t4;
      if (tt >= T) break;
      const int jj = tt >> log2P;
      const int64_t pbv = trow[jj];
      const int off = tt & (P - 1);
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const int c = lane + 64 * e;
        f32x4 vv = *reinterpret_cast<const f32x4*>(
            vpool + (pbv >> split) * a.v_sb + (int64_t)h * a.v_sh + (int64_t)c * (P << split) +
            ((int)(pbv & qmask) << log2P) + off);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (tt + q >= T) vv[q] = 0.f;
#pragma unroll
        for (int gg = 0; gg < 16; ++gg)
          if (gg < G)
            u[gg][e] += sp[wave][gg][t4] * vv[0] + sp[wave][gg][t4 + 1] * vv[1] +
                        sp[wave][gg][t4 + 2] * vv[2] + sp[wave][gg][t4 + 3] * vv[3];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // Wave state -> LDS: lane-partial sums reduce across the wave.
#pragma unroll
  for (int gg = 0; gg < 16; ++gg) {
    if (gg >= G) continue;
    float l = l_run[gg];
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) l += __shfl_xor(l, msk, 64);
    if (lane == 0) {
      st.m[wave][gg] = m_run[gg];
      st.l[wave][gg] = l;
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) st.o[wave][gg][lane + 64 * e] = u[gg][e];
  }
  __syncthreads();
  finish_workgroup<D>(a, st, r, h, part, T);
}

hipError_t launch_paged_decode(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream) {
  // Requests go on the grid's y axis, at most kMaxGridY per launch; a larger
  // batch is launched in slices whose per-request pointers are offset.
  constexpr int kMaxGridY = 65535;
  for (int r0 = 0; r0 < a.batch; r0 += kMaxGridY) {
    const int nb = min(a.batch - r0, kMaxGridY);
    DecodeArgs s = a;
    const int64_t rows = (int64_t)r0 * a.num_q_heads;
    s.q = static_cast<const char*>(a.q) + rows * head_dim * (dtype == PBA_BF16 ? 2 : 4);
    if (a.table_mode == kTablesRagged)
      s.row_offsets = a.row_offsets + r0;  // entries stay put: offsets are absolute
    else if (a.table_mode == kTablesContiguous)
      s.tables = a.tables + r0;            // one slot index per request
    else
      s.tables = a.tables + (int64_t)r0 * a.max_blocks;
    s.seq_lens = a.seq_lens + r0;
    s.out = a.out + rows * head_dim;
    s.lse = a.lse ? a.lse + rows : nullptr;
    s.ws_ml = a.ws_ml ? a.ws_ml + rows * a.n_parts * 2 : nullptr;
    s.ws_u = a.ws_u ? a.ws_u + rows * a.n_parts * head_dim : nullptr;
    s.counters = a.counters ? a.counters + (int64_t)r0 * a.num_kv_heads : nullptr;
    if (a.new_slots) {
      const int64_t new_row =
          (int64_t)r0 * a.num_kv_heads * head_dim * (dtype == PBA_BF16 ? 2 : 4);  // bytes
      s.new_slots = a.new_slots + r0;
      s.k_new = static_cast<const char*>(a.k_new) + new_row;
      s.v_new = static_cast<const char*>(a.v_new) + new_row;
    }
    s.batch = nb;
    const dim3 grid((unsigned)a.num_kv_heads, (unsigned)nb, (unsigned)a.n_parts);
    const dim3 block(kDecodeThreads);
    if (dtype == PBA_BF16) {
      auto kern = a.table_mode == kTablesRagged
                      ? (head_dim == 128 ? decode_bf16_kernel<128, kTablesRagged>
                                         : decode_bf16_kernel<64, kTablesRagged>)
                  : a.table_mode == kTablesContiguous
                      ? (head_dim == 128 ? decode_bf16_kernel<128, kTablesContiguous>
                                         : decode_bf16_kernel<64, kTablesContiguous>)
                      : (head_dim == 128 ? decode_bf16_kernel<128, kTablesDense>
                                         : decode_bf16_kernel<64, kTablesDense>);
      hipLaunchKernelGGL(kern, grid, block, 0, stream, s.tables, s.seq_lens, s.k, s.v,
                         s.max_blocks, s.part_tokens, s.log2P, s.num_blocks - 1,
                         (int32_t)s.k_sb, (int32_t)s.k_sh, s);
    } else {
      auto kern = head_dim == 128 ? decode_f32_kernel<128> : decode_f32_kernel<64>;
      hipLaunchKernelGGL(kern, grid, block, 0, stream, s);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_paged_decode_flat(const DecodeArgs& a, const FlatArgs& f, int head_dim,
                                    int n_wg, hipStream_t stream) {
  const dim3 grid((unsigned)n_wg), block(kDecodeThreads);
  const unsigned lds = (unsigned)flat_lds_bytes(a.batch, a.G, head_dim);
#define PBA_FLAT(DD, MM)                                                                         \
  hipLaunchKernelGGL((decode_bf16_flat_kernel<DD, MM>), grid, block, lds, stream, a.tables,     \
                     a.seq_lens, a.k, a.v, a.max_blocks, a.log2P, a.num_blocks - 1,            \
                     (int32_t)a.k_sb, (int32_t)a.k_sh, a, f)
  if (a.new_slots) {  // fused steps come with dense tables only
    if (a.table_mode != kTablesDense) return hipErrorInvalidValue;
    if (head_dim == 128)
      hipLaunchKernelGGL((decode_bf16_flat_kernel<128, kTablesDense, true>), grid, block, lds,
                         stream, a.tables, a.seq_lens, a.k, a.v, a.max_blocks, a.log2P,
                         a.num_blocks - 1, (int32_t)a.k_sb, (int32_t)a.k_sh, a, f);
    else
      hipLaunchKernelGGL((decode_bf16_flat_kernel<64, kTablesDense, true>), grid, block, lds,
                         stream, a.tables, a.seq_lens, a.k, a.v, a.max_blocks, a.log2P,
                         a.num_blocks - 1, (int32_t)a.k_sb, (int32_t)a.k_sh, a, f);
    return hipGetLastError();
  }
  if (head_dim == 128) {
    if (a.table_mode == kTablesRagged) PBA_FLAT(128, kTablesRagged);
    else if (a.table_mode == kTablesContiguous) PBA_FLAT(128, kTablesContiguous);
    else PBA_FLAT(128, kTablesDense);
  } else {
    if (a.table_mode == kTablesRagged) PBA_FLAT(64, kTablesRagged);
    else if (a.table_mode == kTablesContiguous) PBA_FLAT(64, kTablesContiguous);
    else PBA_FLAT(64, kTablesDense);
  }
#undef PBA_FLAT
  return hipGetLastError();
}

hipError_t launch_paged_decode_shared(const DecodeArgs& a, const SharedArgs& sa, int head_dim,
                                      int private_parts, hipStream_t stream) {
  const dim3 grid((unsigned)a.num_kv_heads, (unsigned)a.batch,
                  (unsigned)(sa.nz_items + private_parts));
  const dim3 block(kDecodeThreads);
  auto kern = a.new_slots ? (head_dim == 128 ? decode_bf16_shared_kernel<128, true>
                                              : decode_bf16_shared_kernel<64, true>)
                          : (head_dim == 128 ? decode_bf16_shared_kernel<128, false>
                                              : decode_bf16_shared_kernel<64, false>);
  hipLaunchKernelGGL(kern, grid, block, 0, stream, a.tables, a.seq_lens, a.k, a.v, a.max_blocks,
                     a.part_tokens, a.log2P, a.num_blocks - 1, (int32_t)a.k_sb, (int32_t)a.k_sh, a,
                     sa);
  return hipGetLastError();
}

}  // namespace pba

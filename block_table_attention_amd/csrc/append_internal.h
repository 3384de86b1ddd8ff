// The V half of the appends (kv_append, kv_append_bundle): one thread moves
// an E x E block of scalars (E = 16 / sizeof scalar) -- piece c of the V rows
// of tokens i0 .. i0 + E - 1 -- into the dim-major V tile ([d][P] per block
// and head), transposing it in registers.  When the E tokens' slots are
// consecutive and start at a multiple of E (a prefill; P is a multiple of E,
// so they share a block), each of the E dims of the piece is one 16-byte
// store; otherwise the scalars are stored one by one ("M5.3 - KV Memory
// Layout and Exact Reuse", 0x03C-0x03D: slot s -> block s div P, offset s
// mod P).  Tokens at or past n read token n - 1 (in bounds) and store
// nothing; negative slots store nothing.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pba {

// Appends of at least this many tokens move V in blocks (a prefill's slots
// are consecutive); smaller ones -- a decode step's one token per request,
// scattered over the pool -- move one token's piece per thread, so that the
// scattered scalar stores spread over many threads instead of queueing 64
// deep in each.
constexpr int64_t kVBlockedMinTokens = 1024;

// Token groups of E per (head, piece), in runs of 8 groups: a run's 8 E
// tokens fill whole 128-byte dim runs of a prefill, and a task order with
// the run inside two neighbouring waves writes them from one work-group.
constexpr int kVGroupRun = 8;

template <typename E>
__host__ __device__ inline int64_t v_append_groups(int64_t n) {
  constexpr int EPC = 16 / sizeof(E);
  return (n + EPC * kVGroupRun - 1) / (EPC * kVGroupRun) * kVGroupRun;
}

// src: piece c of token 0's row (token i's at src + i * row_stride);
// dst: dims c E .. c E + E - 1 of the (layer, head) V tile of block 0
// (block b's at dst + b * block_stride); all in scalars.
template <typename E>
__device__ __forceinline__ void append_v_block(const E* src, int64_t row_stride,
                                               const int64_t* slots, int64_t i0, int64_t n,
                                               E* dst, int64_t block_stride, int log2P) {
  constexpr int EPC = 16 / sizeof(E);
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  union Piece {
    u32x4 u;
    E e[EPC];
  };
  const int P = 1 << log2P;
  Piece in[EPC];
  int64_t s[EPC];
#pragma unroll
  for (int j = 0; j < EPC; ++j) {
    const int64_t i = i0 + j < n ? i0 + j : n - 1;
    in[j].u = *reinterpret_cast<const u32x4*>(src + i * row_stride);
    s[j] = i0 + j < n ? slots[i] : -1;
  }
#pragma unroll
  for (int j = 0; j < EPC; ++j) asm volatile("" ::"v"(in[j].u), "v"(s[j]));
  bool run = s[0] >= 0 && (s[0] & (EPC - 1)) == 0;
#pragma unroll
  for (int j = 1; j < EPC; ++j) run = run && s[j] == s[0] + j;
  if (run) {
    E* d = dst + (s[0] >> log2P) * block_stride + (s[0] & (P - 1));
#pragma unroll
    for (int k = 0; k < EPC; ++k) {
      Piece out;
#pragma unroll
      for (int j = 0; j < EPC; ++j) out.e[j] = in[j].e[k];
      *reinterpret_cast<u32x4*>(d + (int64_t)k * P) = out.u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPC; ++j) {
      if (s[j] < 0) continue;
      E* d = dst + (s[j] >> log2P) * block_stride + (s[j] & (P - 1));
#pragma unroll
      for (int k = 0; k < EPC; ++k) d[(int64_t)k * P] = in[j].e[k];
    }
  }
}

}  // namespace pba

// pba_paged_decode_noalloc: pba_paged_decode for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The split-K partial states and completion counters that
// pba_paged_decode keeps in the caller's workspace live here in one fixed
// array of device memory, `scratch`, which each GPU the library runs on holds
// until the process ends.
//
// Layout of the array: [completion counters | partial states].  The counters
// have a region of their own, so no call's partial states ever overlap any
// call's counters, and every call leaves the counters it used at zero (the
// same invariant pba_paged_decode's workspace relies on): the counters are
// cleared once per device, at set-up, and stay zero between calls of any
// layout.  Calls on one GPU share the array: calls that overlap in time on one
// GPU (two streams, or host threads without ordering) race.
#include <mutex>
#include <vector>

#include "pba_internal.h"

namespace {

constexpr size_t kCounterBytes = PBA_NOALLOC_COUNTER_BYTES;
constexpr size_t kStateBytes = PBA_NOALLOC_STATE_BYTES;
static_assert(kCounterBytes % 256 == 0, "the state region starts 256-byte aligned");

static __device__ __align__(256) unsigned char scratch[kCounterBytes + kStateBytes];

// Zero n 32-bit words (the counter region at set-up): a kernel rather than a
// memset node, so a first call made under stream capture records no memset.
__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

std::mutex g_mu;
std::vector<unsigned char*> g_scratch;  // device address of `scratch`, per device

// The array's device address on the current device (host code must not use
// the symbol itself: it names a host-side stand-in).  Found once per device
// with that device current; the counter region is cleared on `stream` then.
int scratch_on_current_device(hipStream_t stream, unsigned char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PBA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1, nullptr);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PBA_ERR_HIP;
    const int64_t words = kCounterBytes / 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                       stream, static_cast<uint32_t*>(p), words);
    if (hipGetLastError() != hipSuccess) return PBA_ERR_HIP;
    g_scratch[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_scratch[dev];
  return PBA_OK;
}

}  // namespace

extern "C" int pba_paged_decode_noalloc(const pba_kv_pool* pool, const void* q,
                                        int32_t num_q_heads, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                        int32_t batch, float scale, float* out, float* lse,
                                        int32_t partition_tokens, void* stream) {
  // Arguments the host can check (and sizes beyond the scratch) are rejected
  // before the scratch is set up or anything is launched.
  const size_t need = pba_paged_decode_workspace_bytes(pool, num_q_heads, batch,
                                                       max_blocks_per_seq, partition_tokens);
  pba::ScratchArea area{nullptr, kCounterBytes, nullptr, kStateBytes};
  if (need > 0) {
    // (need > 0: the pool and shapes passed the decode's checks.)
    if (!q || !block_tables || !seq_lens || !out) return PBA_ERR_NULL_ARG;
    // Every workspace layout puts the counters first, padded to 256 bytes;
    // the rest are partial states.  The decode path checks both again.
    const size_t counters = (size_t)batch * pool->num_kv_heads * sizeof(int32_t);
    if (counters > kCounterBytes || need - (counters + 255) / 256 * 256 > kStateBytes)
      return PBA_ERR_SCRATCH_LIMIT;
    unsigned char* base = nullptr;
    const int st = scratch_on_current_device(static_cast<hipStream_t>(stream), &base);
    if (st) return st;
    area.counters = reinterpret_cast<int32_t*>(base);
    area.states = reinterpret_cast<char*>(base + kCounterBytes);
  }
  return pba::decode_impl(pool, q, num_q_heads, block_tables, nullptr, max_blocks_per_seq,
                          seq_lens, batch, scale, out, lse, partition_tokens, nullptr, 0, stream,
                          pba::kTablesDense, &area, nullptr);
}

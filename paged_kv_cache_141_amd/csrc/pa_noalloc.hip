// pa_noalloc.hip -- pa_attention without a caller workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, serving
// loops and harnesses that forbid hipMalloc).  The step's work lists and
// split-context partials go to `scratch`, a static device array that every
// device the library runs on holds until the process ends; the kernels are
// those of pa_attention, handed the array's device address as their
// workspace.
#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace {

static_assert(PA_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte units");

// The shared scratch.  In host code its name stands for a host-side shadow,
// not for device memory: the kernels only ever receive the device address
// hipGetSymbolAddress gives for it on the current device.
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device (null: not looked up yet)

// The scratch's address on the current device, looked up on the first call
// there (with that device current) and kept; null if the lookup fails.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> hold(g_lock);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" pa_status_t pa_attention_noalloc(const void* q, int32_t q_dtype, const void* k_cache,
                                            const void* v_cache, const pa_cache_t* cache,
                                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                                            const int32_t* seq_lens, const int32_t* query_start_loc,
                                            int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                            int32_t max_seq_len, int32_t max_query_len, float scale, void* out,
                                            void* stream) {
  // validate and size first: an error or a step too large for the scratch
  // is reported before the device is touched
  size_t need = 0;
  int st = pa::attention_entry(q, q_dtype, k_cache, v_cache, cache, block_tables, max_blocks_per_seq, seq_lens,
                               query_start_loc, num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, 0,
                               scale, out, nullptr, 0, stream, &need);
  if (st != PA_OK) return static_cast<pa_status_t>(st);
  if (need == 0) return PA_OK;   // an empty step
  if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_TOO_LARGE;
  void* ws = device_scratch();
  if (!ws) return PA_ERR_HIP;
  // the plan kernel rewrites the work counters and item lists on every call,
  // and partials are written before they are read: nothing needs clearing
  return static_cast<pa_status_t>(pa::attention_entry(q, q_dtype, k_cache, v_cache, cache, block_tables,
                                                      max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                                                      num_tokens, num_q_heads, max_seq_len, max_query_len, 0, scale,
                                                      out, ws, PA_NOALLOC_SCRATCH_BYTES, stream, nullptr));
}

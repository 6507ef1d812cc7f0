// pa_decode.hip -- the decode attention kernel: one wave per work item (a
// 16-row tile of one sequence and kv head over one context partition), with
// K/V read straight from the paged cache into MFMA operands.
//
// Method: the itwiki "vLLM" article, section "PagedAttention" -- the cache is
// cut into B-token blocks reached through a block table ("Block table"), and
// the attention of a query is a sum over those blocks, fetched one by one;
// the result is ordinary attention ("Block-wise attention").
#include "pa_decode_item.h"

namespace pa {

// Wave g starts on item g, then draws items from a counter until the list
// is done -- or, when the plan found decode-routed sequences starting in the
// same block (their tables share blocks) and the grid has at least eight
// waves, from its XCD's class of items (decode_items_dealt).  V is read with
// the non-temporal hint (STREAM; K without it).
template <int CT, int KV, int D, int BS>
__global__ __launch_bounds__(64, PA_DECODE_WAVES_PER_SIMD) void attn_kernel(AttnArgs a) {
  constexpr bool STREAM = true;
  // fp8 at head dim 256: two steps in flight (a deeper ring does not fit the registers)
  constexpr int PF8 = D == 256 ? 2 : PA_DECODE_PREFETCH_FP8;
  // the plan's header words, read together
  const int64_t total = decode_total(a);
  const int split_s = uniform(a.header[7]);
  const int shared = uniform(a.header[kShareWord]);
  decode_items_dealt<CT, KV, D, BS, PA_DECODE_PREFETCH, PF8, STREAM>(a, threadIdx.x, blockIdx.x, gridDim.x, total,
                                                                     split_s, shared != 0 && gridDim.x >= 8);
}

template <int CT, int KV, int D, int BS>
static int64_t decode_slots() {
  static const int64_t slots = resident_groups(reinterpret_cast<const void*>(&attn_kernel<CT, KV, D, BS>), 64);
  return slots;
}

int64_t decode_waves(int q, int kv, int d, int bs) {
  int64_t n = 0;
  (void)dispatch_attention(q, kv, d, bs, [&](auto ct, auto kvt, auto dt, auto bst) -> hipError_t {
    n = decode_slots<decltype(ct)::value, decltype(kvt)::value, decltype(dt)::value, decltype(bst)::value>();
    return hipSuccess;
  });
  return n;
}

// One wave per resident slot (the persistent grid); each loops over work
// items until the list is done.
hipError_t launch_decode(int q, int kv, int d, int bs, const AttnArgs& a, hipStream_t stream) {
  return dispatch_attention(q, kv, d, bs, [&](auto ct, auto kvt, auto dt, auto bst) -> hipError_t {
    constexpr int CT = decltype(ct)::value, KV = decltype(kvt)::value;
    constexpr int D = decltype(dt)::value, BS = decltype(bst)::value;
    const int64_t slots = decode_slots<CT, KV, D, BS>();
    const int64_t want = a.max_items * a.num_kv_heads;
    const int64_t waves = want < slots ? (want > 0 ? want : 1) : slots;
    hipLaunchKernelGGL((attn_kernel<CT, KV, D, BS>), dim3(static_cast<unsigned>(waves)), dim3(64), 0, stream, a);
    return hipGetLastError();
  });
}

}  // namespace pa

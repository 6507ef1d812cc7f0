// pa_chunk.hip -- the chunked-prefill attention kernel: 8-wave workgroups
// over 256-row blocks of prompt chunks (the loop itself is chunk_items).
//
// Method: a step mixes one-token decode rows with causal prompt chunks
// (techknowgenie "vLLM V1 core refactoring", section "Dynamic Chunked
// Prefill"); the chunk's queries see the cached prefix and the chunk's own
// earlier tokens, through the block table (itwiki "vLLM", "PagedAttention").
#include "pa_chunk_item.h"

namespace pa {

template <int CT, int KV, int D, int BS>
__global__ __launch_bounds__(kChunkThreads, kChunkWavesPerSimd) void chunk_kernel(AttnArgs a) {
  chunk_items<CT, KV, D, BS, kChunkPartition>(a, blockIdx.x, gridDim.x, a.prefix_pass != 0);
}

// One workgroup per resident slot, looping over chunk items.
hipError_t launch_chunk(int q, int kv, int d, int bs, const AttnArgs& a, hipStream_t stream) {
  return dispatch_attention(q, kv, d, bs, [&](auto ct, auto kvt, auto dt, auto bst) -> hipError_t {
    constexpr int CT = decltype(ct)::value, KV = decltype(kvt)::value;
    constexpr int D = decltype(dt)::value, BS = decltype(bst)::value;
    if constexpr (CT == DT_F32) {
      return hipErrorInvalidValue;   // the chunk kernel stages 16-bit operands
    } else {
      if (!a.prefix_pass && a.chunk_partition != kChunkPartition) return hipErrorInvalidValue;   // plan mismatch
      static const int64_t groups =
          resident_groups(reinterpret_cast<const void*>(&chunk_kernel<CT, KV, D, BS>), kChunkThreads);
      const int64_t want = a.prefix_pass ? a.prefix_items : a.max_citems * a.num_kv_heads;
      const int64_t grid = want < groups ? (want > 0 ? want : 1) : groups;
      hipLaunchKernelGGL((chunk_kernel<CT, KV, D, BS>), dim3(static_cast<unsigned>(grid)), dim3(kChunkThreads), 0,
                         stream, a);
      return hipGetLastError();
    }
  });
}

}  // namespace pa

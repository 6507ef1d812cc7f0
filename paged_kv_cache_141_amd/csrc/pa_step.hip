// pa_step.hip -- the fused step kernel: the decode items and the prompt-chunk
// items of one step in a single launch of one 8-wave workgroup per CU.  The
// plan kernel gives the first header[6] workgroups to decode items (each wave
// draws its own) and the rest to chunk items; a chunk workgroup that finds
// the chunk list done turns to decode items, so the two lists finish
// together.  Decode items are HBM-bound and chunk items MFMA-bound: side by
// side, each mostly uses what the other leaves idle.
//
// Method: one step serves decode rows and prompt chunks together
// (techknowgenie "vLLM V1 core refactoring", section "Dynamic Chunked
// Prefill": decode is bandwidth-bound, prefill compute-bound, and the two are
// batched so that the GPU is used by both).
#include "pa_chunk_item.h"
#include "pa_decode_item.h"

namespace pa {

// Decode waves here share their SIMD with a second wave (8 waves per CU), so
// 16-bit K/V keep one step in flight instead of two: the register budget of
// a wave is half the SIMD's.
#ifndef PA_STEP_DECODE_PREFETCH
#define PA_STEP_DECODE_PREFETCH 1
#endif
constexpr int kStepDecodePrefetch = PA_STEP_DECODE_PREFETCH;
constexpr int kStepDecodePrefetchFp8 = 2;   // fp8 steps are half the bytes: two fit the same registers

template <int CT, int KV, int D, int BS>
__global__ __launch_bounds__(kChunkThreads, kChunkWavesPerSimd) void step_kernel(AttnArgs a) {
  const int ndec = uniform(a.header[6]);
  const int g = blockIdx.x;
  const int wave = uniform(static_cast<int>(threadIdx.x) >> 6);
  const int nchunk = static_cast<int>(gridDim.x) - ndec;
  if (g >= ndec) {
    chunk_items<CT, KV, D, BS, kChunkPartitionFused>(a, g - ndec, nchunk, false);
    decode_items<CT, KV, D, BS, kStepDecodePrefetch, kStepDecodePrefetchFp8, true>(
        a, threadIdx.x & 63, -1, ndec * kChunkWaves, decode_total(a), uniform(a.header[7]));
  } else {
    decode_items<CT, KV, D, BS, kStepDecodePrefetch, kStepDecodePrefetchFp8, true>(
        a, threadIdx.x & 63, g * kChunkWaves + wave, ndec * kChunkWaves, decode_total(a), uniform(a.header[7]));
  }
}

int64_t step_groups(int q, int kv, int d, int bs) {
  int64_t g = 0;
  (void)dispatch_attention(q, kv, d, bs, [&](auto ct, auto kvt, auto dt, auto bst) -> hipError_t {
    constexpr int CT = decltype(ct)::value, KV = decltype(kvt)::value;
    constexpr int D = decltype(dt)::value, BS = decltype(bst)::value;
    if constexpr (CT != DT_F32 && D <= 128) {
      static const int64_t groups =
          resident_groups(reinterpret_cast<const void*>(&step_kernel<CT, KV, D, BS>), kChunkThreads);
      g = groups;
    }
    return hipSuccess;
  });
  return g;
}

// One workgroup per resident slot (one per CU): the split in header[6] counts
// workgroups of exactly this grid.
hipError_t launch_step(int q, int kv, int d, int bs, const AttnArgs& a, hipStream_t stream) {
  return dispatch_attention(q, kv, d, bs, [&](auto ct, auto kvt, auto dt, auto bst) -> hipError_t {
    constexpr int CT = decltype(ct)::value, KV = decltype(kvt)::value;
    constexpr int D = decltype(dt)::value, BS = decltype(bst)::value;
    if constexpr (CT == DT_F32 || D > 128) {
      return hipErrorInvalidValue;   // chunk items stage 16-bit operands; d 256 runs the kernels apart
    } else {
      if (a.chunk_partition != kChunkPartitionFused) return hipErrorInvalidValue;   // plan mismatch
      hipLaunchKernelGGL((step_kernel<CT, KV, D, BS>), dim3(static_cast<unsigned>(a.step_groups)),
                         dim3(kChunkThreads), 0, stream, a);
      return hipGetLastError();
    }
  });
}

}  // namespace pa

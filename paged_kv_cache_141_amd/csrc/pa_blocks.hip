// pa_blocks.hip -- whole-block copies between KV pools.
//
// Copy-on-write: a physical block shared by several sequences (reference
// count above one) is copied before one of them writes a token into it; and
// preemption moves all blocks of a request out to host memory and back
// (itwiki "vLLM", sections on block sharing with copy-on-write and on
// scheduling and preemption).  Both are the same operation here: block
// mapping[k].src of a source pool becomes block mapping[k].dst of a
// destination pool, K and V, every kv head; the pools may be one pool
// (copy-on-write) or a device pool and a pinned host pool (swap).
#include "pa_device.h"

namespace pa {

// Grid: x = (pair, K or V), y = 16 KB piece of the block's tensor.  Each
// block's tensor is one contiguous run of Hkv * B * d * eb bytes (a multiple
// of 16); a thread moves four 16-byte pieces, loads first, so every thread has
// four loads in flight.  Pairs whose ids fall outside their pool are skipped.
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int kCopyPiece = kCopyThreads * kCopyUnroll * 16;   // bytes per workgroup

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(BlockCopyArgs a) {
  const int pair = blockIdx.x >> 1;
  const bool v = blockIdx.x & 1;
  const int64_t src = a.mapping[2 * pair];
  const int64_t dst = a.mapping[2 * pair + 1];
  if (src < 0 || src >= a.src_blocks || dst < 0 || dst >= a.dst_blocks) return;
  const int64_t base = static_cast<int64_t>(blockIdx.y) * kCopyPiece;
  const u32x4* s = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(v ? a.src_v : a.src_k) +
                                                   src * a.block_bytes + base);
  u32x4* d = reinterpret_cast<u32x4*>(static_cast<uint8_t*>(v ? a.dst_v : a.dst_k) + dst * a.block_bytes + base);
  const int64_t n = min(static_cast<int64_t>(kCopyPiece), a.block_bytes - base) / 16;
  u32x4 x[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = threadIdx.x + u * kCopyThreads;
    if (i < n) x[u] = s[i];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = threadIdx.x + u * kCopyThreads;
    if (i < n) d[i] = x[u];
  }
}

hipError_t launch_copy_blocks(const BlockCopyArgs& a, hipStream_t stream) {
  if (a.num_pairs <= 0) return hipSuccess;
  const int64_t pieces = (a.block_bytes + kCopyPiece - 1) / kCopyPiece;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<unsigned>(2 * a.num_pairs), static_cast<unsigned>(pieces)),
                     dim3(kCopyThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa

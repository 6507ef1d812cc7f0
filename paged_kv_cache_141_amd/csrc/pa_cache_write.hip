// pa_cache_write.hip -- reshape_and_cache: scatter this step's new K/V rows
// into their cache slots through the slot mapping (llm-wiki "vLLM 0.25 Model
// Runner V2", section "Redesign 4": a flat per-token slot index; slot s is
// offset s % B of physical block s / B, the itwiki "vLLM" article, section
// "PagedAttention", "Block table").
#include <mutex>

#include "pa_device.h"

namespace pa {

#if PA_DEBUG
// The debug words of one device: the first violation's code and index.
static __device__ int32_t g_debug_words[2] = {0, 0};
#endif

// 8 consecutive source elements -> fp32 (exact widening).
template <int SRC>
__device__ __forceinline__ void load8_src(const uint8_t* p, float (&x)[8]) {
  if constexpr (SRC == DT_F32) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p + 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = u2f(a[e]); x[e + 4] = u2f(b[e]); }
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = a[e];
      if constexpr (SRC == DT_BF16) {
        x[2 * e] = bf16_to_f32(w & 0xFFFFu);
        x[2 * e + 1] = bf16_to_f32(w >> 16);
      } else {
        x[2 * e] = f16_to_f32(w & 0xFFFFu);
        x[2 * e + 1] = f16_to_f32(w >> 16);
      }
    }
  }
}

template <int KV>
__device__ __forceinline__ uint32_t encode1(float x, float scale) {
  if constexpr (KV == DT_F32) return f2u(x);
  else if constexpr (KV == DT_F16) return f32_to_f16(x);
  else if constexpr (KV == DT_BF16) return f32_to_bf16(x);
  else return f32_to_e4m3(x, scale);
}

// One row of 8 consecutive elements (16-byte source loads for 16-bit
// sources) encoded to the cache type and stored as one run.
template <int KV>
__device__ __forceinline__ void store8(uint8_t* dst, const float (&x)[8], float scale) {
  if constexpr (KV == DT_F32) {
    u32x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) { lo[e] = f2u(x[e]); hi[e] = f2u(x[e + 4]); }
    reinterpret_cast<u32x4*>(dst)[0] = lo;
    reinterpret_cast<u32x4*>(dst)[1] = hi;
  } else if constexpr (Bytes<KV>::v == 2) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = encode1<KV>(x[2 * e], 1.f) | (encode1<KV>(x[2 * e + 1], 1.f) << 16);
    *reinterpret_cast<u32x4*>(dst) = w;
  } else {
    u32x2 w;
#pragma unroll
    for (int e = 0; e < 2; ++e)
      w[e] = encode1<KV>(x[4 * e], scale) | (encode1<KV>(x[4 * e + 1], scale) << 8) |
             (encode1<KV>(x[4 * e + 2], scale) << 16) | (encode1<KV>(x[4 * e + 3], scale) << 24);
    *reinterpret_cast<u32x2*>(dst) = w;
  }
}

// One workgroup = kWriteTokens consecutive tokens of one kv head; a thread
// takes 8 consecutive elements of one token's K row and the same 8 of its V
// row.  Both land as one contiguous run in the token's row of the [B][d]
// tile, so the tokens of a prompt chunk, which sit in consecutive slots of
// one block, fill whole cache lines.
constexpr int kWriteTokens = 16;

template <int SRC, int KV>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheWriteArgs a) {
  constexpr int EBS = Bytes<SRC>::v;
  constexpr int EBK = Bytes<KV>::v;
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * kWriteTokens;
  const int nt = min(kWriteTokens, a.num_tokens - t0);
  const int d = a.head_dim;
  const int chunks = d / 8;
  for (int x = threadIdx.x; x < nt * chunks; x += 256) {
    const int tt = x / chunks;
    const int c = x - tt * chunks;
    const int64_t s = a.slots[t0 + tt];
    if (s < 0) continue;                                 // padding
#if PA_DEBUG
    if (s >= a.num_slots) {                              // past the pool: recorded and skipped
      if (h == 0 && c == 0) debug_record(a.debug, kDebugSlot, t0 + tt);
      continue;
    }
#endif
    const int64_t blk = s / a.block_size;
    const int off = static_cast<int>(s - blk * a.block_size);
    const int64_t src_off = ((static_cast<int64_t>(t0 + tt) * a.num_kv_heads + h) * d + 8 * c) * EBS;
    float xk[8], xv[8];
    load8_src<SRC>(static_cast<const uint8_t*>(a.key) + src_off, xk);
    load8_src<SRC>(static_cast<const uint8_t*>(a.value) + src_off, xv);
    // element (off, dim) of the (blk, h) tile
    const int64_t dst = ((blk * a.num_kv_heads + h) * static_cast<int64_t>(a.block_size) + off) * d + 8 * c;
    store8<KV>(static_cast<uint8_t*>(a.k_cache) + dst * EBK, xk, a.k_scale);
    store8<KV>(static_cast<uint8_t*>(a.v_cache) + dst * EBK, xv, a.v_scale);
  }
}

template <int SRC, int KV>
static hipError_t launch_rc(const CacheWriteArgs& a, hipStream_t stream) {
  if (a.head_dim > 256 || a.head_dim % 8 != 0) return hipErrorInvalidValue;
  const int64_t groups = (static_cast<int64_t>(a.num_tokens) + kWriteTokens - 1) / kWriteTokens;
  if (groups > 0x7FFFFFFF || a.num_kv_heads > 65535) return hipErrorInvalidValue;
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL((reshape_and_cache_kernel<SRC, KV>), dim3(static_cast<unsigned>(groups), a.num_kv_heads),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int SRC>
static hipError_t launch_rc_kv(int kv, const CacheWriteArgs& a, hipStream_t stream) {
  switch (kv) {
    case DT_F32: return launch_rc<SRC, DT_F32>(a, stream);
    case DT_F16: return launch_rc<SRC, DT_F16>(a, stream);
    case DT_BF16: return launch_rc<SRC, DT_BF16>(a, stream);
    case DT_FP8: return launch_rc<SRC, DT_FP8>(a, stream);
  }
  return hipErrorInvalidValue;
}

int32_t* debug_words() {
#if PA_DEBUG
  static std::mutex lock;
  static int32_t* addr[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> hold(lock);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_debug_words)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = static_cast<int32_t*>(p);
  }
  return addr[dev];
#else
  return nullptr;
#endif
}

hipError_t read_debug_words(int32_t* code, int32_t* index, hipStream_t stream) {
#if PA_DEBUG
  int32_t* words = debug_words();
  if (!words) return hipErrorInvalidSymbol;
  int32_t w[2] = {0, 0};
  const int32_t zero[2] = {0, 0};
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemcpy(w, words, sizeof(w), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(words, zero, sizeof(zero), hipMemcpyHostToDevice);
  *code = w[0];
  *index = w[1];
  return e;
#else
  (void)stream;
  *code = -1;
  *index = -1;
  return hipErrorNotSupported;
#endif
}

hipError_t launch_reshape_and_cache(int src, int kv, const CacheWriteArgs& a, hipStream_t stream) {
  switch (src) {
    case DT_F32: return launch_rc_kv<DT_F32>(kv, a, stream);
    case DT_F16: return launch_rc_kv<DT_F16>(kv, a, stream);
    case DT_BF16: return launch_rc_kv<DT_BF16>(kv, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa

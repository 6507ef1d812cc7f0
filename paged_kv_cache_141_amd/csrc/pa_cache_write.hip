// pa_cache_write.hip -- reshape_and_cache: scatter this step's new K/V rows
// into their cache slots through the slot mapping (llm-wiki "vLLM 0.25 Model
// Runner V2", section "Redesign 4": a flat per-token slot index; slot s is
// offset s % B of physical block s / B, the itwiki "vLLM" article, section
// "PagedAttention", "Block table").
#include <mutex>

#include "pa_cache_write.h"

namespace pa {

#if PA_DEBUG
// The debug words of one device: the first violation's code and index.
static __device__ int32_t g_debug_words[2] = {0, 0};
#endif

// One workgroup = kWriteTokens consecutive tokens of one kv head.
constexpr int kWriteTokens = 16;

template <int SRC, int KV>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheWriteArgs a) {
  const int t0 = blockIdx.x * kWriteTokens;
  write_rows<SRC, KV>(a, t0, min(kWriteTokens, a.num_tokens - t0), blockIdx.y, threadIdx.x, 256);
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

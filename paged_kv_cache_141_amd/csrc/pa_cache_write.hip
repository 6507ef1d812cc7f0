// pa_cache_write.hip -- reshape_and_cache: scatter this step's new K/V rows
// into their cache slots through the slot mapping (llm-wiki "vLLM 0.25 Model
// Runner V2", section "Redesign 4": a flat per-token slot index; slot s is
// offset s % B of physical block s / B, the itwiki "vLLM" article, section
// "PagedAttention", "Block table").
#include "pa_device.h"

namespace pa {

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

// One source element -> fp32 (exact widening).
template <int SRC>
__device__ __forceinline__ float load1_src(const uint8_t* p) {
  if constexpr (SRC == DT_F32) return *reinterpret_cast<const float*>(p);
  else if constexpr (SRC == DT_BF16) return bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
  else return f16_to_f32(*reinterpret_cast<const uint16_t*>(p));
}

template <int KV>
__device__ __forceinline__ uint32_t encode1(float x, float scale) {
  if constexpr (KV == DT_F32) return f2u(x);
  else if constexpr (KV == DT_F16) return f32_to_f16(x);
  else if constexpr (KV == DT_BF16) return f32_to_bf16(x);
  else return f32_to_e4m3(x, scale);
}

// One thread = 8 elements of one (token, kv head) row, C = d / 8 threads per
// row.  K: thread c takes the 8 consecutive elements 8c .. 8c+7 (one 16-byte
// chunk for 16-bit sources) and lands them as one contiguous run.  V: the
// row goes down one column of the transposed [d][B] tile, one element per
// dim row, B elements apart; thread c takes dims c, C + c, 2C + c, ..., so
// that each store instruction writes C consecutive dims of a row -- stores
// that fall in one cache line (4 dims of 16-bit bf16 at B = 16) merge into
// one request instead of four.
template <int SRC, int KV>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheWriteArgs a) {
  const int chunks = a.head_dim / 8;
  const int per_tok = a.num_kv_heads * chunks;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(a.num_tokens) * per_tok) return;
  const int t = static_cast<int>(idx / per_tok);
  const int rem = static_cast<int>(idx - static_cast<int64_t>(t) * per_tok);
  const int h = rem / chunks;
  const int c = rem - h * chunks;
  const int64_t s = a.slots[t];
  if (s < 0) return;
  const int64_t blk = s / a.block_size;
  const int off = static_cast<int>(s - blk * a.block_size);
  constexpr int EBS = Bytes<SRC>::v;
  constexpr int EBK = Bytes<KV>::v;
  const int64_t src_off = ((static_cast<int64_t>(t) * a.num_kv_heads + h) * a.head_dim + 8 * c) * EBS;
  float xk[8], xv[8];
  load8_src<SRC>(static_cast<const uint8_t*>(a.key) + src_off, xk);
  {
    const uint8_t* vsrc = static_cast<const uint8_t*>(a.value) +
                          ((static_cast<int64_t>(t) * a.num_kv_heads + h) * a.head_dim + c) * EBS;
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[e] = load1_src<SRC>(vsrc + static_cast<int64_t>(e) * chunks * EBS);
  }

  const int64_t tile = (blk * a.num_kv_heads + h) * static_cast<int64_t>(a.block_size) * a.head_dim;
  uint8_t* kdst = static_cast<uint8_t*>(a.k_cache) + (tile + static_cast<int64_t>(off) * a.head_dim + 8 * c) * EBK;
  if constexpr (KV == DT_F32) {
    u32x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) { lo[e] = f2u(xk[e]); hi[e] = f2u(xk[e + 4]); }
    reinterpret_cast<u32x4*>(kdst)[0] = lo;
    reinterpret_cast<u32x4*>(kdst)[1] = hi;
  } else if constexpr (EBK == 2) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = encode1<KV>(xk[2 * e], 1.f) | (encode1<KV>(xk[2 * e + 1], 1.f) << 16);
    *reinterpret_cast<u32x4*>(kdst) = w;
  } else {
    u32x2 w;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      w[e] = encode1<KV>(xk[4 * e], a.k_scale) | (encode1<KV>(xk[4 * e + 1], a.k_scale) << 8) |
             (encode1<KV>(xk[4 * e + 2], a.k_scale) << 16) |
             (encode1<KV>(xk[4 * e + 3], a.k_scale) << 24);
    }
    *reinterpret_cast<u32x2*>(kdst) = w;
  }

  // V tile is [d][B]: element (dim, off) at dim * B + off; this thread's dims
  // are c + e * chunks
  uint8_t* vdst = static_cast<uint8_t*>(a.v_cache) +
                  (tile + static_cast<int64_t>(c) * a.block_size + off) * EBK;
  const int64_t vstride = static_cast<int64_t>(chunks) * a.block_size * EBK;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t code = encode1<KV>(xv[e], a.v_scale);
    uint8_t* p = vdst + e * vstride;
    if constexpr (EBK == 4) *reinterpret_cast<uint32_t*>(p) = code;
    else if constexpr (EBK == 2) *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(code);
    else *p = static_cast<uint8_t>(code);
  }
}

template <int SRC, int KV>
static hipError_t launch_rc(const CacheWriteArgs& a, hipStream_t stream) {
  const int64_t work = static_cast<int64_t>(a.num_tokens) * a.num_kv_heads * (a.head_dim / 8);
  const int64_t blocks = (work + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((reshape_and_cache_kernel<SRC, KV>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, a);
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

hipError_t launch_reshape_and_cache(int src, int kv, const CacheWriteArgs& a, hipStream_t stream) {
  switch (src) {
    case DT_F32: return launch_rc_kv<DT_F32>(kv, a, stream);
    case DT_F16: return launch_rc_kv<DT_F16>(kv, a, stream);
    case DT_BF16: return launch_rc_kv<DT_BF16>(kv, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa

// pa_cache_write.h -- the cache write's device code: new K/V rows of some
// tokens scattered into their slots (llm-wiki "vLLM 0.25 Model Runner V2",
// section "Redesign 4": a flat per-token slot index; slot s is offset s % B of
// physical block s / B, the itwiki "vLLM" article, section "PagedAttention",
// "Block table").  Used by the cache-write kernel and by the launch that
// writes a step's tokens beside its work-list build.
#pragma once

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

// Tokens [t0, t0 + nt) of kv head h, by `nthreads` threads (thread tid): a
// thread takes 8 consecutive elements of one token's K row and the same 8 of
// its V row.  Both land as one contiguous run in the token's row of the
// [B][d] tile, so the tokens of a prompt chunk, which sit in consecutive
// slots of one block, fill whole cache lines.
template <int SRC, int KV>
__device__ __forceinline__ void write_rows(const CacheWriteArgs& a, int t0, int nt, int h, int tid, int nthreads) {
  constexpr int EBS = Bytes<SRC>::v;
  constexpr int EBK = Bytes<KV>::v;
  const int d = a.head_dim;
  const int chunks = d / 8;
  for (int x = tid; x < nt * chunks; x += nthreads) {
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

}  // namespace pa

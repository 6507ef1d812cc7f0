// pa_device.h -- device-side building blocks of the attention kernels:
// vector types, element sizes, MFMA operand fragments, and the online-softmax
// step.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_codec.h"
#include "pa_internal.h"

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3 };

template <int DT> struct Bytes;
template <> struct Bytes<DT_F32> { static constexpr int v = 4; };
template <> struct Bytes<DT_F16> { static constexpr int v = 2; };
template <> struct Bytes<DT_BF16> { static constexpr int v = 2; };
template <> struct Bytes<DT_FP8> { static constexpr int v = 1; };

// Does sequence i (rows = q_len * G) use the chunk kernel?
__device__ __forceinline__ bool is_chunk_seq(const AttnArgs& a, int rows) {
  return a.chunk_path && rows >= kChunkMinRows;
}

// First partial row of (token, q head) -- the row of sequence seq whose
// local query index is `local` -- in the workspace's partial lists (the
// layout of WorkspaceLayout: decode-routed rows by sequence slot or token,
// chunk-routed rows by token after chunk_row_base); -1 where the workspace
// holds no list for it (a chunk row in a step the hints kept chunk-free, or
// a decode row past its sequence's slots, both outside the contract).
__device__ __forceinline__ int64_t partial_row(const AttnArgs& a, bool chunk_kind, int seq, int token, int local,
                                               int head) {
  if (chunk_kind) {
    if (a.chunk_parts == 0) return -1;
    return a.chunk_row_base + (static_cast<int64_t>(token) * a.num_q_heads + head) * a.chunk_parts;
  }
  int64_t slot = token;
  if (a.dec_per_seq > 0) {
    if (local < 0 || local >= a.dec_per_seq) return -1;
    slot = static_cast<int64_t>(seq) * a.dec_per_seq + local;
  }
  return (slot * a.num_q_heads + head) * a.dec_parts;
}

// The sequence whose query rows hold `token`: the last i with
// query_start_loc[i] <= token (binary search, one lane at a time).
__device__ __forceinline__ int seq_of_token(const AttnArgs& a, int token) {
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.qsl[mid] <= token) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Eight operand elements of one lane for a K=32 MFMA step (or eight K=4
// steps for fp32): 16 bytes for 16-bit types, 32 bytes for fp32.
template <int CT> struct Frag { u32x4 w; };
template <> struct Frag<DT_F32> { u32x4 w[2]; };

template <int CT>
__device__ __forceinline__ Frag<CT> frag_zero() {
  Frag<CT> f;
  if constexpr (CT == DT_F32) { f.w[0] = u32x4{0, 0, 0, 0}; f.w[1] = f.w[0]; }
  else f.w = u32x4{0, 0, 0, 0};
  return f;
}

// Eight consecutive elements of storage type SRC as loaded from memory
// (kept raw so that prefetched data costs the fewest registers).
template <int SRC> struct Raw { u32x4 w; };
template <> struct Raw<DT_F32> { u32x4 w[2]; };
template <> struct Raw<DT_FP8> { u32x2 w; };

// Cache data a decode item reads once: STREAM gives the loads the
// non-temporal hint (global_load ... nt).  The decode items give it to their
// V loads, not their K loads.  Decode kernel us in one session, no hint / V
// only / K and V: LLaMA-7B 777 / 712 / 733, GQA 439 / 406 / 428, GQA fp8
// 235 / 221 / 231; the fused mixed step with K too 624 against 595.
template <bool STREAM, typename T>
__device__ __forceinline__ T load_once(const T* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int SRC, bool STREAM>
__device__ __forceinline__ Raw<SRC> load_kv(const uint8_t* p) {
  Raw<SRC> r;
  if constexpr (SRC == DT_F32) {
    r.w[0] = load_once<STREAM>(reinterpret_cast<const u32x4*>(p));
    r.w[1] = load_once<STREAM>(reinterpret_cast<const u32x4*>(p) + 1);
  } else if constexpr (SRC == DT_FP8) {
    r.w = load_once<STREAM>(reinterpret_cast<const u32x2*>(p));
  } else {
    r.w = load_once<STREAM>(reinterpret_cast<const u32x4*>(p));
  }
  return r;
}

template <int SRC>
__device__ __forceinline__ Raw<SRC> load_raw(const uint8_t* p) {
  Raw<SRC> r;
  if constexpr (SRC == DT_F32) {
    r.w[0] = reinterpret_cast<const u32x4*>(p)[0];
    r.w[1] = reinterpret_cast<const u32x4*>(p)[1];
  } else if constexpr (SRC == DT_FP8) {
    r.w = *reinterpret_cast<const u32x2*>(p);
  } else {
    r.w = *reinterpret_cast<const u32x4*>(p);
  }
  return r;
}

// Two fp8 codes (the low or high 16 bits of w) -> two elements of the 16-bit
// compute type, packed.  gfx950's scaled conversion does it in one
// instruction; with scale 1 it is exact (every E4M3 value, subnormals
// included, is a normal bf16 and f16 value).
template <int CT>
__device__ __forceinline__ uint32_t widen2(uint32_t w, bool high) {
  static_assert(CT == DT_BF16 || CT == DT_F16, "fp8 codes widen to a 16-bit compute type");
  if constexpr (CT == DT_BF16) {
    return high ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
                : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  } else {
    return high ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))
                : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  }
}

// Raw elements -> MFMA operand of compute type CT.  fp8 codes widen exactly
// to bf16/f16 (every E4M3 value is representable in both).
template <int CT, int SRC>
__device__ __forceinline__ Frag<CT> to_frag(const Raw<SRC>& r) {
  Frag<CT> f;
  if constexpr (SRC == DT_FP8) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      f.w[2 * e] = widen2<CT>(r.w[e], false);
      f.w[2 * e + 1] = widen2<CT>(r.w[e], true);
    }
  } else if constexpr (SRC == DT_F32) {
    f.w[0] = r.w[0];
    f.w[1] = r.w[1];
  } else {
    f.w = r.w;
  }
  return f;
}

template <int CT, int SRC>
__device__ __forceinline__ Frag<CT> load_frag(const uint8_t* p) {
  return to_frag<CT, SRC>(load_raw<SRC>(p));
}

// acc += A(16 x 32) * B(32 x 16).  A lane's 8 elements sit in the same K
// slots of A and B, so the pairing of A and B elements only needs both
// operands to use one assignment of data to (lane group, element).
template <int CT>
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<CT>& a, const Frag<CT>& b) {
  if constexpr (CT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.w),
                                                   __builtin_bit_cast(bf16x8, b.w), acc, 0, 0, 0);
  } else if constexpr (CT == DT_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a.w),
                                                  __builtin_bit_cast(f16x8, b.w), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(u2f(a.w[h][e]), u2f(b.w[h][e]), acc, 0, 0, 0);
    return acc;
  }
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// Two fp32 -> two packed 16-bit values (hardware conversion, round to nearest
// even; used for probabilities and outputs, never for cache contents).
template <int CT>
__device__ __forceinline__ uint32_t cvt2(float x, float y) {
  if constexpr (CT == DT_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{x, y}, bf16x2v));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{x, y}, f16x2v));
}

// fp32 probabilities -> operand elements.
template <int CT>
__device__ __forceinline__ Frag<CT> pack_p(const float (&p)[8]) {
  Frag<CT> f;
  if constexpr (CT == DT_F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.w[0][e] = f2u(p[e]); f.w[1][e] = f2u(p[e + 4]); }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) f.w[e] = cvt2<CT>(p[2 * e], p[2 * e + 1]);
  }
  return f;
}

template <int OT>
__device__ __forceinline__ void store4(uint8_t* p, float a, float b, float c, float d) {
  if constexpr (OT == DT_F32)
    *reinterpret_cast<u32x4*>(p) = u32x4{f2u(a), f2u(b), f2u(c), f2u(d)};
  else
    *reinterpret_cast<u32x2*>(p) = u32x2{cvt2<OT>(a, b), cvt2<OT>(c, d)};
}

// ---- V operands from token-major V rows (the decode items; the chunk
// items read theirs from LDS with transposing loads instead).
//
// The PV product O^T += V^T P^T takes V^T as its A operand: lane (r, lg)
// must hold, for one output dim, the values of the eight keys of its K slots.
// A V row in the cache holds one key's d values, so each lane reads, for
// each of its eight keys, a run of SEG consecutive dims, and the operands
// are transposed in registers.  The runs
// of lane r are segments c = 0 .. NSEG-1 at dims 16*SEG*c + SEG*r; output
// tile j = SEG*c + jj then holds dims 16*SEG*c + SEG*n + jj in its rows n, so
// the accumulator element v of lane (r, lg) in tile j is dim
// 16*SEG*c + SEG*(4*lg + v) + jj of query row r.
template <int EB, int D>
struct VGeo {
  static constexpr int NT = D / 16;                     // 16-dim output tiles
  // dims per run: 16 bytes of 16-bit values (8 dims at most), all NT dims of
  // fp8 codes (4 to 16 bytes), 4 fp32 values
  static constexpr int SEG = EB == 1 ? NT : (EB == 4 ? 4 : (NT < 8 ? NT : 8));
  static constexpr int NSEG = NT / SEG;
  static constexpr int WORDS = SEG * EB / 4;             // 32-bit words per run
  static_assert(NSEG * SEG == NT && WORDS >= 1 && WORDS <= 4, "V run geometry");
};

template <int N> struct Words { uint32_t w[N]; };

template <int N, bool STREAM>
__device__ __forceinline__ Words<N> load_words(const uint8_t* p) {
  Words<N> r;
  if constexpr (N == 4) {
    const u32x4 x = load_once<STREAM>(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int e = 0; e < 4; ++e) r.w[e] = x[e];
  } else if constexpr (N == 2) {
    const u32x2 x = load_once<STREAM>(reinterpret_cast<const u32x2*>(p));
    r.w[0] = x[0];
    r.w[1] = x[1];
  } else {
    r.w[0] = load_once<STREAM>(reinterpret_cast<const uint32_t*>(p));
  }
  return r;
}

// Operand of tile jj (within a run) from the eight runs v[0..7] of 16-bit
// values, slot e of the lane taking run e: element jj of each run, two runs
// per 32-bit word (one byte permute each).
template <int CT, int N>
__device__ __forceinline__ Frag<CT> vt_frag16(const Words<N> (&v)[8], int jj) {
  const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
  Frag<CT> f;
#pragma unroll
  for (int q = 0; q < 4; ++q) f.w[q] = __builtin_amdgcn_perm(v[2 * q + 1].w[jj >> 1], v[2 * q].w[jj >> 1], sel);
  return f;
}

// fp32 values: element jj of run e goes to slot e unchanged.
__device__ __forceinline__ Frag<DT_F32> vt_frag32(const Words<4> (&v)[8], int jj) {
  Frag<DT_F32> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.w[e >> 2][e & 3] = v[e].w[jj];
  return f;
}

// 4x4 byte transpose: x[b] = byte b of a, b, c, d (in that order, low first).
__device__ __forceinline__ void byte_transpose4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t (&x)[4]) {
  const uint32_t ab0 = __builtin_amdgcn_perm(b, a, 0x06020400u);   // a0 b0 a2 b2
  const uint32_t ab1 = __builtin_amdgcn_perm(b, a, 0x07030501u);   // a1 b1 a3 b3
  const uint32_t cd0 = __builtin_amdgcn_perm(d, c, 0x06020400u);
  const uint32_t cd1 = __builtin_amdgcn_perm(d, c, 0x07030501u);
  x[0] = __builtin_amdgcn_perm(cd0, ab0, 0x05040100u);
  x[1] = __builtin_amdgcn_perm(cd1, ab1, 0x05040100u);
  x[2] = __builtin_amdgcn_perm(cd0, ab0, 0x07060302u);
  x[3] = __builtin_amdgcn_perm(cd1, ab1, 0x07060302u);
}

// Online-softmax update for one query row whose keys are spread over the four
// lanes r, r+16, r+32, r+48 (N raw scores per lane, already -inf where
// masked).  m is the row's reference max in raw-score units, the same in the
// four lanes; c = scale * k_scale * log2(e) > 0 turns raw scores into log2
// units.  The reference moves -- and lsum and the accumulator are rescaled
// -- only when some lane of the wave holds a score more than `slack`
// (kRescaleSlack / c, AttnArgs::rescale_slack) above it; only then is the
// cross-lane row max taken.
// Returns the probabilities 2^(c*(s - m)) <= 2^kRescaleSlack in p.
template <int N, int NACC>
__device__ __forceinline__ void softmax_update(const float (&s)[N], float& m, float& lsum,
                                               f32x4 (&acc)[NACC], float c, float slack, float (&p)[N]) {
  float lm = s[0];
#pragma unroll
  for (int e = 1; e < N; ++e) lm = fmaxf(lm, s[e]);
  if (__any(lm > m + slack)) {
    float rm = fmaxf(lm, __shfl_xor(lm, 16));
    rm = fmaxf(rm, __shfl_xor(rm, 32));
    const float mnew = fmaxf(m, rm);
    const float alpha = (mnew == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f((m - mnew) * c);
    lsum *= alpha;
#pragma unroll
    for (int n = 0; n < NACC; ++n) acc[n] *= alpha;
    m = mnew;
  }
  const float cm = (m == -__builtin_inff()) ? 0.f : m * c;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], c, -cm));
    lsum += p[e];
  }
}

// Reference max in log2 units, as stored for the partition merge.
__device__ __forceinline__ float max_log2(float m, float c) { return m == -__builtin_inff() ? m : m * c; }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

#if PA_DEBUG
// Debug build: record a violation in the debug words ([0] the first
// violation's code, 0 for none; [1] its sequence or token) unless one is
// recorded already (the code word is taken with a compare-and-swap from 0).
__device__ __forceinline__ void debug_record(int32_t* words, int32_t code, int32_t index) {
  if (atomicCAS(&words[0], 0, code) == 0) atomicExch(&words[1], index);
}
#endif

// Host-side dispatch of a runtime (q dtype, kv dtype, head dim, block size)
// to f(ct, kv, d, bs), each an std::integral_constant, for the combinations
// the kernels are built for; others give hipErrorInvalidValue.
template <int V> using IC = std::integral_constant<int, V>;

template <int CT, int KV, class F>
hipError_t dispatch_shape(int d, int bs, F&& f) {
  if (d == 64) {
    if (bs == 16) return f(IC<CT>{}, IC<KV>{}, IC<64>{}, IC<16>{});
    if (bs == 32) return f(IC<CT>{}, IC<KV>{}, IC<64>{}, IC<32>{});
    if (bs == 64) return f(IC<CT>{}, IC<KV>{}, IC<64>{}, IC<64>{});
  } else if (d == 128) {
    if (bs == 16) return f(IC<CT>{}, IC<KV>{}, IC<128>{}, IC<16>{});
    if (bs == 32) return f(IC<CT>{}, IC<KV>{}, IC<128>{}, IC<32>{});
    if (bs == 64) return f(IC<CT>{}, IC<KV>{}, IC<128>{}, IC<64>{});
  } else if (d == 256) {
    if constexpr (CT != DT_F32) {   // 16-bit queries only at d = 256
      if (bs == 16) return f(IC<CT>{}, IC<KV>{}, IC<256>{}, IC<16>{});
      if (bs == 32) return f(IC<CT>{}, IC<KV>{}, IC<256>{}, IC<32>{});
      if (bs == 64) return f(IC<CT>{}, IC<KV>{}, IC<256>{}, IC<64>{});
    }
  }
  return hipErrorInvalidValue;
}

template <class F>
hipError_t dispatch_attention(int q, int kv, int d, int bs, F&& f) {
  if (q == DT_F32 && kv == DT_F32) return dispatch_shape<DT_F32, DT_F32>(d, bs, f);
  if (q == DT_F16 && kv == DT_F16) return dispatch_shape<DT_F16, DT_F16>(d, bs, f);
  if (q == DT_F16 && kv == DT_FP8) return dispatch_shape<DT_F16, DT_FP8>(d, bs, f);
  if (q == DT_BF16 && kv == DT_BF16) return dispatch_shape<DT_BF16, DT_BF16>(d, bs, f);
  if (q == DT_BF16 && kv == DT_FP8) return dispatch_shape<DT_BF16, DT_FP8>(d, bs, f);
  return hipErrorInvalidValue;
}

}  // namespace pa

// pa_kernels.hip -- HIP kernels of the paged-attention hot path for gfx950.
//
//   reshape_and_cache_kernel : scatter new K/V into their cache slots.
//   plan_kernel              : per-step work list (sequence, row tile, partition).
//   attn_kernel              : block-table gather + QK^T + online softmax + PV on
//                              MFMA, one 16-row tile x one context partition per
//                              work item.
//   reduce_kernel            : log-sum-exp merge of a row's partitions.
//
// Method: the itwiki "vLLM" article, section "PagedAttention" -- the cache is
// cut into B-token blocks reached through a block table ("Block table"), and
// the attention of query i is a sum over those blocks that the kernel fetches
// one by one; the result is ordinary attention ("Block-wise attention").  A
// step mixes decode rows and causal prompt chunks (techknowgenie "vLLM V1
// core refactoring", "Dynamic Chunked Prefill").
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

// Decode-kernel tuning: steps of 16-bit K/V kept in flight ahead of the one
// being computed, and the occupancy the register budget is cut for.
#ifndef PA_DECODE_PREFETCH
#define PA_DECODE_PREFETCH 2
#endif
#ifndef PA_DECODE_WAVES_PER_SIMD
#define PA_DECODE_WAVES_PER_SIMD 1
#endif

template <int DT> struct Bytes;
template <> struct Bytes<DT_F32> { static constexpr int v = 4; };
template <> struct Bytes<DT_F16> { static constexpr int v = 2; };
template <> struct Bytes<DT_BF16> { static constexpr int v = 2; };
template <> struct Bytes<DT_FP8> { static constexpr int v = 1; };

// ============================================================================
// cache write
// ============================================================================

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

// One thread = 8 consecutive elements (one 16-byte source chunk for 16-bit
// sources) of one (token, kv head) row.  K lands as one contiguous run of
// 8 elements; V goes to 8 rows of the transposed tile at the token's offset.
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
  load8_src<SRC>(static_cast<const uint8_t*>(a.value) + src_off, xv);

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

  // V tile is [d][B]: element (dim, off) at dim * B + off
  uint8_t* vdst = static_cast<uint8_t*>(a.v_cache) +
                  (tile + static_cast<int64_t>(8 * c) * a.block_size + off) * EBK;
  const int64_t vstride = static_cast<int64_t>(a.block_size) * EBK;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t code = encode1<KV>(xv[e], a.v_scale);
    uint8_t* p = vdst + e * vstride;
    if constexpr (EBK == 4) *reinterpret_cast<uint32_t*>(p) = code;
    else if constexpr (EBK == 2) *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(code);
    else *p = static_cast<uint8_t>(code);
  }
}

// ============================================================================
// step plan: the work list
// ============================================================================

// Does sequence i (rows = q_len * G) use the chunk kernel?
__device__ __forceinline__ bool is_chunk_seq(const AttnArgs& a, int rows) {
  return a.chunk_path && rows >= kChunkMinRows;
}

// One workgroup.  For each sequence with q_len > 0 it counts work items --
// decode: ceil(rows/16) row tiles x ceil(L/P) partitions (P = 512 or 1024); chunk:
// ceil(rows/128) row blocks x ceil(L/4096) partitions -- takes exclusive
// prefix sums and appends the items in (tile, partition) order to the two
// lists.  It also resets the work counters the attention kernels draw from.
__global__ __launch_bounds__(1024) void plan_kernel(AttnArgs a) {
  __shared__ int32_t scan[2][1024];
  __shared__ int64_t carry[2];
  const int tid = threadIdx.x;
  if (tid < 2) carry[tid] = 0;
  __syncthreads();
  for (int base = 0; base < a.num_seqs; base += 1024) {
    const int i = base + tid;
    int n[2] = {0, 0}, parts[2] = {1, 1};
    if (i < a.num_seqs) {
      const int L = a.seq_lens[i];
      const int ql = a.qsl[i + 1] - a.qsl[i];
      const int rows = ql * a.group;
      if (ql > 0 && L > 0) {
        if (is_chunk_seq(a, rows)) {
          parts[1] = (L + kChunkPartition - 1) / kChunkPartition;
          n[1] = ((rows + kChunkRows - 1) / kChunkRows) * parts[1];
        } else {
          parts[0] = (L + a.partition - 1) / a.partition;
          n[0] = ((rows + kTileRows - 1) / kTileRows) * parts[0];
        }
      }
    }
    scan[0][tid] = n[0];
    scan[1][tid] = n[1];
    __syncthreads();
    for (int ofs = 1; ofs < 1024; ofs <<= 1) {   // inclusive Hillis-Steele scans
      const int v0 = tid >= ofs ? scan[0][tid - ofs] : 0;
      const int v1 = tid >= ofs ? scan[1][tid - ofs] : 0;
      __syncthreads();
      scan[0][tid] += v0;
      scan[1][tid] += v1;
      __syncthreads();
    }
#pragma unroll
    for (int list = 0; list < 2; ++list) {
      int32_t* out = list ? a.citems : a.items;
      const int64_t cap = list ? a.max_citems : a.max_items;
      const int64_t start = carry[list] + scan[list][tid] - n[list];
      for (int k = 0; k < n[list]; ++k) {
        const int64_t pos = start + k;
        if (pos >= cap) break;              // only with metadata beyond the host bounds
        const int tile = k / parts[list];
        const int part = k - tile * parts[list];
        out[2 * pos] = i;
        out[2 * pos + 1] = (tile << 16) | part;
      }
    }
    __syncthreads();
    if (tid == 1023) {
      carry[0] += scan[0][1023];
      carry[1] += scan[1][1023];
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.header[0] = 0;
    a.header[1] = static_cast<int32_t>(carry[0] < a.max_items ? carry[0] : a.max_items);
    a.header[2] = 0;
    a.header[3] = static_cast<int32_t>(carry[1] < a.max_citems ? carry[1] : a.max_citems);
  }
}

// ============================================================================
// attention
// ============================================================================

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

// Raw elements -> MFMA operand of compute type CT.  fp8 codes widen exactly
// to bf16/f16 (every E4M3 value is representable in both).
template <int CT, int SRC>
__device__ __forceinline__ Frag<CT> to_frag(const Raw<SRC>& r) {
  Frag<CT> f;
  if constexpr (SRC == DT_FP8) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(r.w[e], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(r.w[e], true);
      if constexpr (CT == DT_BF16) {
        // exact: an E4M3 value has at most 4 significant bits, so the low half is zero
        f.w[2 * e] = __builtin_amdgcn_perm(f2u(lo[1]), f2u(lo[0]), 0x07060302u);
        f.w[2 * e + 1] = __builtin_amdgcn_perm(f2u(hi[1]), f2u(hi[0]), 0x07060302u);
      } else {
        f.w[2 * e] = f32_to_f16(lo[0]) | (f32_to_f16(lo[1]) << 16);
        f.w[2 * e + 1] = f32_to_f16(hi[0]) | (f32_to_f16(hi[1]) << 16);
      }
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

// Per-element keep-masks for an 8-element operand whose element e is kept
// when e < n (n may be <= 0 or >= 8): zeroes elements by selection, no branches.
template <int CT>
__device__ __forceinline__ void frag_keep_first(Frag<CT>& f, int n) {
  if constexpr (CT == DT_F32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.w[e >> 2][e & 3] = e < n ? f.w[e >> 2][e & 3] : 0u;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t keep = (2 * q < n ? 0x0000FFFFu : 0u) | (2 * q + 1 < n ? 0xFFFF0000u : 0u);
      f.w[q] &= keep;
    }
  }
}

// Rescale threshold (log2 units): the running reference max of a row moves
// only when a new score exceeds it by more than this, so the accumulator
// rescale is skipped for most tiles; probabilities stay below 2^8.
constexpr float kRescaleSlack = 8.f;

// Online-softmax update for one query row whose keys are spread over the four
// lanes r, r+16, r+32, r+48 (N raw scores per lane, already -inf where
// masked).  m is the row's reference max in raw-score units, the same in the
// four lanes; c = scale * k_scale * log2(e) > 0 turns raw scores into log2
// units.  The reference moves -- and lsum and the accumulator are rescaled
// -- only when some lane of the wave holds a score more than `slack`
// (kRescaleSlack / c) above it; only then is the cross-lane row max taken.
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

// One work item: sequence i, kv head h, rows [16*tile, 16*tile+16) of the
// sequence's q_len*G (token, head-in-group) rows, keys of partition `part`.
//
// Lane l = r + 16*lg (r = l % 16, lg = l / 16).  The 16x16 MFMA result tile
// puts column r in lane r + 16*(row/4), element row%4.  The score tile is
// computed transposed, S^T = K * Q^T (rows = keys, columns = query rows), with
// K-tile row m of sub-tile tau holding key 8*(m/4) + 4*tau + m%4 of the
// 32-key step: then lane l ends up with the scores of query row r for the
// eight consecutive keys 8*lg .. 8*lg+7, exactly the K slots the PV product
// O^T = V^T * P^T needs from P^T, and V^T's rows (dims) are contiguous over
// keys in the [d][B] tile, so both MFMA operands load straight from memory.
template <int CT, int KV, int D, int BS>
__device__ __forceinline__ void attn_item(const AttnArgs& a, int i, int tile, int part, int h,
                                          int lane) {
  constexpr int EBQ = Bytes<CT>::v;
  constexpr int EBK = Bytes<KV>::v;
  constexpr int KS = D / 32;     // K-steps of the QK^T product
  constexpr int NT = D / 16;     // 16-dim output tiles
  const int r = lane & 15;
  const int lg = lane >> 4;

  const int L = a.seq_lens[i];
  const int q0 = a.qsl[i];
  const int ql = a.qsl[i + 1] - q0;
  const int G = a.group;
  const int rows = ql * G;
  const int row0 = tile * kTileRows;
  const int R = row0 + r;
  const bool valid = R < rows;
  const int t = R / G;
  const int g = R - t * G;
  const int token = q0 + t;
  const int head = h * G + g;
  const int base_pos = L - ql;
  const int row_pos = valid ? base_pos + t : -1;
  const int last_R = min(rows, row0 + kTileRows) - 1;
  const int max_pos = base_pos + last_R / G;
  const int min_pos = base_pos + row0 / G;
  const int kstart = part * a.partition;
  const int kend = min(min(L, kstart + a.partition), max_pos + 1);
  if (kstart >= kend) return;

  // Q^T operand: row r's dims [32s + 8lg, +8)
  Frag<CT> qf[KS];
  {
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                        ((static_cast<int64_t>(token) * a.num_q_heads + head) * D + 8 * lg) * EBQ;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = valid ? load_frag<CT, CT>(qp + 32 * s * EBQ) : frag_zero<CT>();
  }

  const int nblk = (L + BS - 1) / BS;
  const int64_t tile_bytes = static_cast<int64_t>(BS) * D * EBK;
  const int64_t blk_stride = tile_bytes * a.num_kv_heads;
  const uint8_t* kc = static_cast<const uint8_t*>(a.k_cache) + h * tile_bytes;
  const uint8_t* vc = static_cast<const uint8_t*>(a.v_cache) + h * tile_bytes;

  // The partition's block-table entries, one per lane (at most P/B <= 64):
  // each step then reads its physical block ids with readlane, no memory trip.
  const int jbase = kstart / BS;
  const int nbt = min(nblk - jbase, a.partition / BS);
  const int32_t* bt = a.block_tables + static_cast<int64_t>(i) * a.max_blocks_per_seq + jbase;
  const int btv = lane < nbt ? bt[lane] : 0;

  // per-lane key offsets inside a 32-key step
  const int kkey0 = 8 * (r >> 2) + (r & 3);      // sub-tile 0; sub-tile 1 adds 4
  const int vkey = 8 * lg;                        // first of the lane's 8 keys for V / P

  float m = -__builtin_inff();
  float lsum = 0.f;
  const float slack = kRescaleSlack / a.score_scale;
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Step {
    Raw<KV> k[2][KS];
    Raw<KV> v[NT];
  };
  // Issue the loads of the 32-key step starting at key k0 (block-table
  // gather: physical block(s) from the table register, then 16-byte reads).
  auto issue = [&](Step& st, int k0) {
    const int j0 = k0 / BS;
    const int64_t p0 = __builtin_amdgcn_readlane(btv, j0 - jbase);
    int64_t p1 = p0;
    if constexpr (BS == 16) p1 = __builtin_amdgcn_readlane(btv, min(j0 + 1, nblk - 1) - jbase);
    const int inblk = k0 - j0 * BS;   // 0 for BS <= 32; 0 or 32 for BS = 64
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int kk = kkey0 + 4 * tau;                  // key within the step
      const int64_t pb = (BS == 16 && kk >= 16) ? p1 : p0;
      const int off = (BS == 16) ? (kk & 15) : inblk + kk;
      const uint8_t* kp = kc + pb * blk_stride + (static_cast<int64_t>(off) * D + 8 * lg) * EBK;
#pragma unroll
      for (int s = 0; s < KS; ++s) st.k[tau][s] = load_raw<KV>(kp + 32 * s * EBK);
    }
    const int64_t pb = (BS == 16 && vkey >= 16) ? p1 : p0;
    const int off = (BS == 16) ? (vkey & 15) : inblk + vkey;
    const uint8_t* vp = vc + pb * blk_stride + (static_cast<int64_t>(r) * BS + off) * EBK;
#pragma unroll
    for (int n = 0; n < NT; ++n) st.v[n] = load_raw<KV>(vp + static_cast<int64_t>(16 * n) * BS * EBK);
  };

  auto compute = [&](const Step& st, int k0) {
    // ---- S^T = K Q^T
    f32x4 sf[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      sf[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) sf[tau] = mma<CT>(sf[tau], to_frag<CT, KV>(st.k[tau][s]), qf[s]);
    }
    float sc[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) { sc[e] = sf[0][e]; sc[4 + e] = sf[1][e]; }
    if (k0 + 31 > min_pos) {   // some key of this step is past some row's position
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[e] = (k0 + vkey + e <= row_pos) ? sc[e] : -__builtin_inff();
    }
    // ---- online softmax (row r; the four lane groups share the row)
    float p[8];
    softmax_update<8, NT>(sc, m, lsum, acc, a.score_scale, slack, p);

    // ---- O^T += V^T P^T (keys past the end hold poison: their V elements
    // are replaced by zero, by selection)
    const Frag<CT> pf = pack_p<CT>(p);
    const bool tail = k0 + 32 > L;
    const int keep = L - (k0 + vkey);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      Frag<CT> vf = to_frag<CT, KV>(st.v[n]);
      if (tail) frag_keep_first<CT>(vf, keep);
      acc[n] = mma<CT>(acc[n], vf, pf);
    }
  };

  // Software pipeline: the loads of step s + PF are in flight while step s
  // computes.  fp8 steps are half the bytes, so they run one step deeper.
  constexpr int PF = (KV == DT_FP8) ? 2 : (KV == DT_F32 ? 0 : PA_DECODE_PREFETCH);
  constexpr int NB = PF + 1;
  Step buf[NB];
  const int nsteps = (kend - kstart + 31) / 32;
#pragma unroll
  for (int s = 0; s < PF; ++s)
    if (s < nsteps) issue(buf[s], kstart + 32 * s);
  for (int s0 = 0; s0 < nsteps; s0 += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int s = s0 + b;
      if (s >= nsteps) break;
      if (s + PF < nsteps) issue(buf[(b + PF) % NB], kstart + 32 * (s + PF));
      compute(buf[b], kstart + 32 * s);
    }
  }

  // ---- finish: whole-row denominator, then the output or a partial
  float ltot = lsum + __shfl_xor(lsum, 16);
  ltot += __shfl_xor(ltot, 32);
  if (!valid || row_pos < kstart) return;
  const int nparts_row = row_pos / a.partition + 1;
  if (nparts_row == 1) {
    const float inv = a.v_scale / ltot;
    uint8_t* op = static_cast<uint8_t*>(a.out) +
                  ((static_cast<int64_t>(token) * a.num_q_heads + head) * D + 4 * lg) * EBQ;
#pragma unroll
    for (int n = 0; n < NT; ++n)
      store4<CT>(op + 16 * n * EBQ, acc[n][0] * inv, acc[n][1] * inv, acc[n][2] * inv, acc[n][3] * inv);
  } else {
    const int64_t rowp = (static_cast<int64_t>(token) * a.num_q_heads + head) * a.max_parts + part;
    if (lg == 0) {
      a.part_m[rowp] = max_log2(m, a.score_scale);
      a.part_l[rowp] = ltot;
    }
    float* pa = a.part_acc + rowp * D + 4 * lg;
#pragma unroll
    for (int n = 0; n < NT; ++n)
      *reinterpret_cast<f32x4*>(pa + 16 * n) = acc[n] * a.v_scale;
  }
}

// Waves draw work items from a counter; item w covers list entry w / Hkv and
// kv head w % Hkv.  Every wave exits once the counter passes the item count.
template <int CT, int KV, int D, int BS>
__global__ __launch_bounds__(64, PA_DECODE_WAVES_PER_SIMD) void attn_kernel(AttnArgs a) {
  const int lane = threadIdx.x;
  const int64_t total = static_cast<int64_t>(uniform(a.header[1])) * a.num_kv_heads;
  while (true) {
    int w = 0;
    if (lane == 0) w = atomicAdd(a.header, 1);
    w = uniform(__shfl(w, 0));
    if (w >= total) break;
    const int e = w / a.num_kv_heads;
    const int h = w - e * a.num_kv_heads;
    const int i = uniform(a.items[2 * e]);
    const int tp = uniform(a.items[2 * e + 1]);
    attn_item<CT, KV, D, BS>(a, i, tp >> 16, tp & 0xFFFF, h, lane);
  }
}

// ============================================================================
// chunked prefill: 128-row blocks over LDS-staged 64-key tiles
// ============================================================================

// LDS image of one 64-key tile in the 16-bit compute type: K rows [64][d]
// and V^T rows [d][64], unpadded.  The 16-byte chunks of a row are XOR-
// swizzled so that the 16 lanes of each MFMA operand read (16 different
// rows, one chunk column) land in 16 different 16-byte bank groups.
template <int D>
struct ChunkLds {
  static constexpr int KROW = D * 2;                   // bytes per K row
  static constexpr int VROW = kChunkKeys * 2;          // bytes per V^T row (128)
  static constexpr int KBYTES = kChunkKeys * KROW;
  static constexpr int BUF = KBYTES + D * VROW;
  // The K rows one read touches are {8*(r/4) + 4*tau + r%4} (mod 32).
  static __device__ __forceinline__ int kswz(int key) {
    if constexpr (D == 128) return (key & 3) | (((key >> 3) & 3) << 2);
    else return ((key >> 1) & 1) | (((key >> 3) & 3) << 1);   // 128-byte rows pair up per 256 bytes
  }
  // The V^T rows one read touches are 16 consecutive dims.
  static __device__ __forceinline__ int vswz(int dim) { return (dim >> 1) & 7; }
  static __device__ __forceinline__ int koff(int key, int chunk) { return key * KROW + ((chunk ^ kswz(key)) << 4); }
  static __device__ __forceinline__ int voff(int dim, int chunk) { return KBYTES + dim * VROW + ((chunk ^ vswz(dim)) << 4); }
};

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4):
// lane l's data lands at LDS byte offset lds_base + 16 * l, lds_base being
// wave-uniform.  Issued as inline assembly so that the compiler does not
// guard every later LDS read with a wait for it (it cannot tell the ring
// buffers apart); the kernel waits for these loads itself, with s_waitcnt
// vmcnt and a barrier, before any wave reads the buffer they fill.
// M0 carries the LDS address; it is saved and restored around the load so
// that the compiler's own use of M0 is never disturbed.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_base)
      : "memory");
}

// s_waitcnt immediate: at most n vector-memory operations outstanding
// (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return 0xF70 | (n & 15) | ((n >> 4) << 14); }

// 16 raw fp8 codes -> 16 elements of the 16-bit compute type (two 16-byte halves).
template <int CT>
__device__ __forceinline__ void widen16(const u32x4& raw, u32x4& lo, u32x4& hi) {
  Raw<DT_FP8> a, b;
  a.w = u32x2{raw[0], raw[1]};
  b.w = u32x2{raw[2], raw[3]};
  lo = to_frag<CT, DT_FP8>(a).w;
  hi = to_frag<CT, DT_FP8>(b).w;
}

// One workgroup (8 waves, two per SIMD) per work item: sequence i, kv head h,
// rows [256*rb, 256*rb + 256) of the sequence's (token, head-in-group) rows, keys
// of context partition `part` (4096 keys).  Wave w owns rows 32w..32w+31 as
// two 16-row tiles.  Each 64-key tile is gathered through the block table by
// all 512 threads with 16-byte loads -- straight into LDS for 16-bit caches
// (global_load_lds), through registers for fp8, which is widened to the
// compute type on the way -- while the previous tile computes; each wave
// then runs the same transposed-score MFMA scheme as the decode kernel,
// every LDS operand read feeding both of its row tiles.  Keys past the end
// are never used: their scores are replaced by -inf and their V elements by
// zero, by selection.
template <int CT, int KV, int D, int BS>
__global__ __launch_bounds__(kChunkThreads, 1) void chunk_kernel(AttnArgs a) {
  using Lds = ChunkLds<D>;
  // 16-bit caches: three tile buffers (two tiles in flight); fp8: two
  // buffers plus two register sets.
  constexpr bool DIRECT = (KV != DT_FP8);                // 16-bit cache: global -> LDS directly
  constexpr int NBUF = DIRECT ? 3 : 2;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * Lds::BUF];
  __shared__ int32_t btl[kChunkPartition / BS];          // the partition's physical block ids
  __shared__ int slot;
  constexpr int EBQ = Bytes<CT>::v;
  constexpr int EBK = Bytes<KV>::v;
  constexpr int KS = D / 32;
  constexpr int NT = D / 16;
  constexpr int RT = 2;                                  // row tiles per wave

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);                    // wave-uniform: keeps its branches scalar
  const int lane = tid & 63;
  const int r = lane & 15;
  const int lg = lane >> 4;
  const int64_t total = static_cast<int64_t>(uniform(a.header[3])) * a.num_kv_heads;
  const int64_t tile_bytes = static_cast<int64_t>(BS) * D * EBK;
  const int64_t blk_stride = tile_bytes * a.num_kv_heads;
  const uint32_t blk_stride32 = static_cast<uint32_t>(blk_stride);   // Hkv * B * d * eb < 2^32

  // Direct-to-LDS loads: wave w's load j fills tile bytes [base, base + 1 KB).
  // Tiles start at multiples of 64 >= B, so which key (or dim) and which
  // 16-byte chunk a lane fetches, its block relative to the tile's first
  // block and its offset inside that block are the same for every tile.
  constexpr int NI = Lds::BUF / 1024 / kChunkWaves;       // loads per wave per tile
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  int dma_base[NI], dma_rel[NI], dma_off[NI];
  bool dma_is_v[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int base = (wave * NI + j) * 1024;
    const int pos = base + lane * 16;
    dma_base[j] = base;
    dma_is_v[j] = base >= Lds::KBYTES;
    if (!dma_is_v[j]) {
      const int kk = pos / Lds::KROW;
      const int chunk = ((pos % Lds::KROW) >> 4) ^ Lds::kswz(kk);
      dma_rel[j] = kk / BS;
      dma_off[j] = ((kk % BS) * D + 8 * chunk) * EBK;
    } else {
      const int pv = pos - Lds::KBYTES;
      const int dim = pv / Lds::VROW;
      const int kk = 8 * (((pv % Lds::VROW) >> 4) ^ Lds::vswz(dim));   // first of the chunk's 8 keys
      dma_rel[j] = kk / BS;
      dma_off[j] = (dim * BS + kk % BS) * EBK;
    }
  }

  // LDS operand reads: lane (r, lg) reads K row kg*32 + 4*tau + rb, chunk
  // 4s + lg, and V^T row 16n + r, chunk 4kg + lg.  The swizzle of those rows
  // depends on r alone, so each lane needs one offset per s (K) and per kg
  // (V); kg, tau and n then enter as immediate offsets.
  const int rb = 8 * (r >> 2) + (r & 3);
  int kls[KS], vls[2];
#pragma unroll
  for (int s = 0; s < KS; ++s) kls[s] = Lds::koff(rb, 4 * s + lg);
#pragma unroll
  for (int kg = 0; kg < 2; ++kg) vls[kg] = Lds::voff(r, 4 * kg + lg);

  while (true) {
    if (tid == 0) slot = atomicAdd(a.header + 2, 1);
    __syncthreads();
    const int w = slot;
    if (w >= total) break;
    const int e = w / a.num_kv_heads;
    const int h = w - e * a.num_kv_heads;
    const int i = a.citems[2 * e];
    const int tp = a.citems[2 * e + 1];
    const int rb = tp >> 16;
    const int part = tp & 0xFFFF;

    const int L = a.seq_lens[i];
    const int q0 = a.qsl[i];
    const int ql = a.qsl[i + 1] - q0;
    const int G = a.group;
    const int rows = ql * G;
    const int base_pos = L - ql;
    const int wrow0 = rb * kChunkRows + wave * (16 * RT);
    const int wlast = min(rows, wrow0 + 16 * RT) - 1;     // last row of this wave (< wrow0: none)
    const int wave_min_pos = base_pos + wrow0 / G;
    const int wave_max_pos = wlast >= wrow0 ? base_pos + wlast / G : -1;
    const int wg_max_pos = base_pos + (min(rows, rb * kChunkRows + kChunkRows) - 1) / G;
    const int kstart = part * kChunkPartition;
    const int kend = min(min(L, kstart + kChunkPartition), wg_max_pos + 1);

    if (kstart < kend) {
      int row_pos[RT], token[RT], head[RT];
      bool valid[RT];
      Frag<CT> qf[RT][KS];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int R = wrow0 + 16 * rt + r;
        valid[rt] = R < rows;
        const int t = R / G;
        token[rt] = q0 + t;
        head[rt] = h * G + (R - t * G);
        row_pos[rt] = valid[rt] ? base_pos + t : -1;
        const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                            ((static_cast<int64_t>(token[rt]) * a.num_q_heads + head[rt]) * D + 8 * lg) * EBQ;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          qf[rt][s] = valid[rt] ? load_frag<CT, CT>(qp + 32 * s * EBQ) : frag_zero<CT>();
      }
      float m[RT], lsum[RT];
      const float slack = kRescaleSlack / a.score_scale;
      f32x4 acc[RT][NT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        m[rt] = -__builtin_inff();
        lsum[rt] = 0.f;
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[rt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      }

      const int nblk = (L + BS - 1) / BS;
      const int jbase = kstart / BS;
      {
        const int32_t* bt = a.block_tables + static_cast<int64_t>(i) * a.max_blocks_per_seq + jbase;
        for (int j = tid; j < min(nblk - jbase, kChunkPartition / BS); j += kChunkThreads) btl[j] = bt[j];
      }
      __syncthreads();
      const uint8_t* kc = static_cast<const uint8_t*>(a.k_cache) + h * tile_bytes;
      const uint8_t* vc = static_cast<const uint8_t*>(a.v_cache) + h * tile_bytes;
      // physical block of tile-relative key index kk (clamped to the last block:
      // keys past the end are loaded but never used)
      auto phys_of = [&](int kt, int kk) -> int64_t { return btl[min((kt + kk) / BS, nblk - 1) - jbase]; };

      // ---- 16-bit caches: the tile goes straight to LDS, 1 KB per wave instruction
      auto issue_direct = [&](int b, int kt) {
        const int jt = kt / BS - jbase;                     // tile's first block, table-relative
        const int jlast = nblk - 1 - jbase;
        uint32_t phys[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) phys[j] = static_cast<uint32_t>(btl[min(jt + dma_rel[j], jlast)]);
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          // a block id times the per-block stride (< 2^32 bytes) needs one 32x32->64 multiply-add
          const uint8_t* src = (dma_is_v[j] ? vc : kc) +
                               (static_cast<uint64_t>(phys[j]) * blk_stride32 + static_cast<uint32_t>(dma_off[j]));
          lds_dma16(src, uniform(static_cast<int>(lds0 + b * Lds::BUF + dma_base[j])));
        }
      };

      // ---- fp8 caches: 16 codes per thread-chunk through registers, widened
      constexpr int FCH = kChunkKeys * D / 16;                // 16-code chunks of K (and of V) per tile
      constexpr int FPT = (FCH + kChunkThreads - 1) / kChunkThreads;
      using Regs = u32x4[DIRECT ? 1 : FPT];
      Regs kreg0, vreg0, kreg1, vreg1;
      auto gather_fp8 = [&](Regs& kreg, Regs& vreg, int kt) {
#pragma unroll
        for (int j = 0; j < FPT; ++j) {
          const int c = tid + kChunkThreads * j;
          if (FCH % kChunkThreads != 0 && c >= FCH) break;
          const int kk = c / (D / 16);
          const int cc = c % (D / 16);
          kreg[j] = *reinterpret_cast<const u32x4*>(
              kc + phys_of(kt, kk) * blk_stride + static_cast<int64_t>((kt + kk) % BS) * D + cc * 16);
          const int dim = c / (kChunkKeys / 16);
          const int kv0 = (c % (kChunkKeys / 16)) * 16;      // first of 16 keys
          vreg[j] = *reinterpret_cast<const u32x4*>(
              vc + phys_of(kt, kv0) * blk_stride + static_cast<int64_t>(dim) * BS + (kt + kv0) % BS);
        }
      };
      auto stage_fp8 = [&](const Regs& kreg, const Regs& vreg, uint8_t* buf) {
#pragma unroll
        for (int j = 0; j < FPT; ++j) {
          const int c = tid + kChunkThreads * j;
          if (FCH % kChunkThreads != 0 && c >= FCH) break;
          u32x4 lo, hi;
          const int kk = c / (D / 16);
          const int cc = c % (D / 16);                       // 16 codes = 16-bit chunks 2cc, 2cc+1
          widen16<CT>(kreg[j], lo, hi);
          *reinterpret_cast<u32x4*>(buf + Lds::koff(kk, 2 * cc)) = lo;
          *reinterpret_cast<u32x4*>(buf + Lds::koff(kk, 2 * cc + 1)) = hi;
          const int dim = c / (kChunkKeys / 16);
          const int vc2 = (c % (kChunkKeys / 16)) * 2;
          widen16<CT>(vreg[j], lo, hi);
          *reinterpret_cast<u32x4*>(buf + Lds::voff(dim, vc2)) = lo;
          *reinterpret_cast<u32x4*>(buf + Lds::voff(dim, vc2 + 1)) = hi;
        }
      };

      // ---- one tile on this wave's rows
      auto compute = [&](const uint8_t* buf, int kt) {
        f32x4 sf[RT][2][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int kg = 0; kg < 2; ++kg)
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) sf[rt][kg][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kg = 0; kg < 2; ++kg)
#pragma unroll
          for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
              Frag<CT> kf;
              kf.w = *reinterpret_cast<const u32x4*>(buf + kls[s] + (kg * 32 + 4 * tau) * Lds::KROW);
#pragma unroll
              for (int rt = 0; rt < RT; ++rt) sf[rt][kg][tau] = mma<CT>(sf[rt][kg][tau], kf, qf[rt][s]);
            }
          }
        Frag<CT> pf[RT][2];
        const bool edge = kt + kChunkKeys - 1 > wave_min_pos;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          float sc[16];
#pragma unroll
          for (int kg = 0; kg < 2; ++kg)
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
              float v = sf[rt][kg][e2 >> 2][e2 & 3];
              if (edge && kt + kg * 32 + 8 * lg + e2 > row_pos[rt]) v = -__builtin_inff();
              sc[kg * 8 + e2] = v;
            }
          float p[16];
          softmax_update<16, NT>(sc, m[rt], lsum[rt], acc[rt], a.score_scale, slack, p);
#pragma unroll
          for (int kg = 0; kg < 2; ++kg) {
            float pk[8];
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) pk[e2] = p[kg * 8 + e2];
            pf[rt][kg] = pack_p<CT>(pk);
          }
        }
        const bool tail = kt + kChunkKeys > L;   // V of keys past the end: replaced by zero
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int kg = 0; kg < 2; ++kg) {
            Frag<CT> vf;
            vf.w = *reinterpret_cast<const u32x4*>(buf + vls[kg] + 16 * n * Lds::VROW);
            if (tail) frag_keep_first<CT>(vf, L - (kt + kg * 32 + 8 * lg));
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc[rt][n] = mma<CT>(acc[rt][n], vf, pf[rt][kg]);
          }
      };

      const int ntiles = (kend - kstart + kChunkKeys - 1) / kChunkKeys;
      auto tile_key = [&](int ti) { return kstart + ti * kChunkKeys; };
      if constexpr (DIRECT) {
        // The compiler cannot see the LDS loads; retire its own loads (q) here
        // so that it has no reason to wait on the vector-memory counter later.
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        // tile ti lives in buffer ti % 3; tiles ti+1 and ti+2 load while ti computes
        issue_direct(0, tile_key(0));
        if (ntiles > 1) {
          issue_direct(1, tile_key(1));
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(NI));
        } else {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        __syncthreads();
        for (int ti = 0; ti < ntiles; ++ti) {
          const int kt = tile_key(ti);
          const bool ahead = ti + 2 < ntiles;
          if (ahead) issue_direct((ti + 2) % 3, tile_key(ti + 2));
          if (kt <= wave_max_pos) compute(lds + (ti % 3) * Lds::BUF, kt);
          if (ahead) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NI));   // tile ti+1 has landed
          else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
          __syncthreads();
        }
      } else {
        // tile ti lives in buffer ti % 2 and, before that, register set ti % 2
        gather_fp8(kreg0, vreg0, tile_key(0));
        stage_fp8(kreg0, vreg0, lds);
        if (ntiles > 1) gather_fp8(kreg1, vreg1, tile_key(1));
        __syncthreads();
        for (int ti = 0; ti < ntiles; ti += 2) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int tj = ti + half;
            if (tj < ntiles) {
              Regs& kr = half ? kreg1 : kreg0;   // holds tile tj (already staged): free
              Regs& vr = half ? vreg1 : vreg0;
              Regs& kn = half ? kreg0 : kreg1;   // holds tile tj + 1
              Regs& vn = half ? vreg0 : vreg1;
              if (tj + 2 < ntiles) gather_fp8(kr, vr, tile_key(tj + 2));
              const int kt = tile_key(tj);
              if (kt <= wave_max_pos) compute(lds + half * Lds::BUF, kt);
              if (tj + 1 < ntiles) stage_fp8(kn, vn, lds + (1 - half) * Lds::BUF);
              __syncthreads();
            }
          }
        }
      }

#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float ltot = lsum[rt] + __shfl_xor(lsum[rt], 16);
        ltot += __shfl_xor(ltot, 32);
        if (!valid[rt] || row_pos[rt] < kstart) continue;
        if (row_pos[rt] / kChunkPartition == 0) {
          const float inv = a.v_scale / ltot;
          uint8_t* op = static_cast<uint8_t*>(a.out) +
                        ((static_cast<int64_t>(token[rt]) * a.num_q_heads + head[rt]) * D + 4 * lg) * EBQ;
#pragma unroll
          for (int n = 0; n < NT; ++n)
            store4<CT>(op + 16 * n * EBQ, acc[rt][n][0] * inv, acc[rt][n][1] * inv, acc[rt][n][2] * inv,
                       acc[rt][n][3] * inv);
        } else {
          const int64_t rowp = (static_cast<int64_t>(token[rt]) * a.num_q_heads + head[rt]) * a.max_parts + part;
          if (lg == 0) {
            a.part_m[rowp] = max_log2(m[rt], a.score_scale);
            a.part_l[rowp] = ltot;
          }
          float* pp = a.part_acc + rowp * D + 4 * lg;
#pragma unroll
          for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(pp + 16 * n) = acc[rt][n] * a.v_scale;
        }
      }
    }
    __syncthreads();
  }
}

// One workgroup per (token, q head); rows whose keys fit one partition were
// written by the attention kernel and are skipped here.
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p
template <int OT, int D>
__global__ __launch_bounds__(64) void reduce_kernel(AttnArgs a) {
  const int token = blockIdx.x;
  const int head = blockIdx.y;
  // sequence of this token: last i with qsl[i] <= token
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (uniform(a.qsl[mid]) <= token) lo = mid; else hi = mid - 1;
  }
  const int i = lo;
  const int q0 = a.qsl[i];
  const int ql = a.qsl[i + 1] - q0;
  const int row_pos = a.seq_lens[i] - ql + (token - q0);
  const int np = row_pos / (is_chunk_seq(a, ql * a.group) ? kChunkPartition : a.partition) + 1;
  if (np <= 1) return;
  const int64_t row = (static_cast<int64_t>(token) * a.num_q_heads + head) * a.max_parts;
  float M = -__builtin_inff();
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.part_m[row + p]);
  float den = 0.f;
  constexpr int PER = D / 64;
  float num[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) num[k] = 0.f;
  for (int p = 0; p < np; ++p) {
    const float wgt = __builtin_amdgcn_exp2f(a.part_m[row + p] - M);
    den += wgt * a.part_l[row + p];
    const float* ap = a.part_acc + (row + p) * D;
#pragma unroll
    for (int k = 0; k < PER; ++k) num[k] += wgt * ap[threadIdx.x + 64 * k];
  }
  constexpr int EBO = Bytes<OT>::v;
  uint8_t* op = static_cast<uint8_t*>(a.out) + ((static_cast<int64_t>(token) * a.num_q_heads + head) * D) * EBO;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const float v = num[k] / den;
    const int dd = threadIdx.x + 64 * k;
    if constexpr (OT == DT_F32) reinterpret_cast<float*>(op)[dd] = v;
    else if constexpr (OT == DT_BF16) reinterpret_cast<uint16_t*>(op)[dd] = static_cast<uint16_t>(f32_to_bf16(v));
    else reinterpret_cast<uint16_t*>(op)[dd] = static_cast<uint16_t>(f32_to_f16(v));
  }
}

// ============================================================================
// launchers
// ============================================================================

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

// Workgroups of `threads` threads of `kernel` that fit on the device at once.
static int64_t resident_groups(const void* kernel, int threads) {
  int dev = 0, per_cu = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu <= 0)
    return 512;
  return static_cast<int64_t>(per_cu) * prop.multiProcessorCount;
}

// plan -> decode kernel -> chunk kernel (when a prompt chunk can be present)
// -> partition merge.  ev[0..1] bracket the decode kernel, ev[2..3] the chunk
// kernel (each may be null).
template <int CT, int KV, int D, int BS>
static hipError_t launch_attn(const AttnArgs& a, hipStream_t stream, const hipEvent_t* ev) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one wave per resident slot; each loops over work items until the list is done
  static const int64_t slots = resident_groups(reinterpret_cast<const void*>(&attn_kernel<CT, KV, D, BS>), 64);
  const int64_t want = a.max_items * a.num_kv_heads;
  const int64_t waves = want < slots ? (want > 0 ? want : 1) : slots;
  if (ev[0] && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((attn_kernel<CT, KV, D, BS>), dim3(static_cast<unsigned>(waves)), dim3(64), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev[1] && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
  if constexpr (CT != DT_F32) {
    if (a.chunk_path && static_cast<int64_t>(a.max_query_len) * a.group >= kChunkMinRows) {
      static const int64_t groups =
          resident_groups(reinterpret_cast<const void*>(&chunk_kernel<CT, KV, D, BS>), kChunkThreads);
      const int64_t cwant = a.max_citems * a.num_kv_heads;
      const int64_t cgrid = cwant < groups ? (cwant > 0 ? cwant : 1) : groups;
      if (ev[2] && (e = hipEventRecord(ev[2], stream)) != hipSuccess) return e;
      hipLaunchKernelGGL((chunk_kernel<CT, KV, D, BS>), dim3(static_cast<unsigned>(cgrid)), dim3(kChunkThreads), 0, stream,
                         a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (ev[3] && (e = hipEventRecord(ev[3], stream)) != hipSuccess) return e;
    }
  }
  if (a.max_parts > 1 && a.num_tokens > 0) {
    hipLaunchKernelGGL((reduce_kernel<CT, D>), dim3(a.num_tokens, a.num_q_heads), dim3(64), 0, stream, a);
    e = hipGetLastError();
  }
  return e;
}

template <int CT, int KV>
static hipError_t launch_attn_shape(int d, int bs, const AttnArgs& a, hipStream_t s, const hipEvent_t* ev) {
  if (d == 64) {
    if (bs == 16) return launch_attn<CT, KV, 64, 16>(a, s, ev);
    if (bs == 32) return launch_attn<CT, KV, 64, 32>(a, s, ev);
    if (bs == 64) return launch_attn<CT, KV, 64, 64>(a, s, ev);
  } else if (d == 128) {
    if (bs == 16) return launch_attn<CT, KV, 128, 16>(a, s, ev);
    if (bs == 32) return launch_attn<CT, KV, 128, 32>(a, s, ev);
    if (bs == 64) return launch_attn<CT, KV, 128, 64>(a, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention(int q, int kv, int d, int bs, const AttnArgs& a, hipStream_t s,
                            const hipEvent_t* ev) {
  if (q == DT_F32 && kv == DT_F32) return launch_attn_shape<DT_F32, DT_F32>(d, bs, a, s, ev);
  if (q == DT_F16 && kv == DT_F16) return launch_attn_shape<DT_F16, DT_F16>(d, bs, a, s, ev);
  if (q == DT_F16 && kv == DT_FP8) return launch_attn_shape<DT_F16, DT_FP8>(d, bs, a, s, ev);
  if (q == DT_BF16 && kv == DT_BF16) return launch_attn_shape<DT_BF16, DT_BF16>(d, bs, a, s, ev);
  if (q == DT_BF16 && kv == DT_FP8) return launch_attn_shape<DT_BF16, DT_FP8>(d, bs, a, s, ev);
  return hipErrorInvalidValue;
}

}  // namespace pa

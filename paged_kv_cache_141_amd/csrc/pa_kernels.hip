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

// One workgroup.  For each sequence with q_len > 0: tiles = ceil(q_len*G/16)
// row tiles, parts = ceil(L/P) context partitions; its tiles*parts items are
// appended in (tile, partition) order after an exclusive prefix sum.  Also
// resets the work counter the attention kernel's waves draw from.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ seq_lens,
                                                    const int32_t* __restrict__ qsl, int num_seqs,
                                                    int group, int32_t* __restrict__ header,
                                                    int32_t* __restrict__ items,
                                                    int64_t max_items) {
  __shared__ int32_t scan[1024];
  __shared__ int64_t carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < num_seqs; base += 1024) {
    const int i = base + tid;
    int n = 0, parts = 1;
    if (i < num_seqs) {
      const int L = seq_lens[i];
      const int ql = qsl[i + 1] - qsl[i];
      if (ql > 0 && L > 0) {
        const int tiles = (ql * group + kTileRows - 1) / kTileRows;
        parts = (L + kPartition - 1) / kPartition;
        n = tiles * parts;
      }
    }
    scan[tid] = n;
    __syncthreads();
    for (int ofs = 1; ofs < 1024; ofs <<= 1) {   // inclusive Hillis-Steele scan
      const int v = tid >= ofs ? scan[tid - ofs] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int64_t start = carry + scan[tid] - n;
    for (int k = 0; k < n; ++k) {
      const int64_t pos = start + k;
      if (pos >= max_items) break;          // only with metadata beyond the host bounds
      const int tile = k / parts;
      const int part = k - tile * parts;
      items[2 * pos] = i;
      items[2 * pos + 1] = (tile << 16) | part;
    }
    __syncthreads();
    if (tid == 1023) carry += scan[1023];
    __syncthreads();
  }
  if (tid == 0) {
    header[0] = 0;
    header[1] = static_cast<int32_t>(carry < max_items ? carry : max_items);
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

// Zero element e of a fragment (used to drop NaN-poisoned V slots past the end).
template <int CT>
__device__ __forceinline__ void frag_zero_elem(Frag<CT>& f, int e) {
  if constexpr (CT == DT_F32) {
    f.w[e >> 2][e & 3] = 0u;
  } else {
    const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
    f.w[e >> 1] &= keep;
  }
}

// fp32 probabilities -> operand elements (round to nearest even).
template <int CT>
__device__ __forceinline__ Frag<CT> pack_p(const float (&p)[8]) {
  Frag<CT> f;
  if constexpr (CT == DT_F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.w[0][e] = f2u(p[e]); f.w[1][e] = f2u(p[e + 4]); }
  } else if constexpr (CT == DT_BF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f.w[e] = f32_to_bf16(p[2 * e]) | (f32_to_bf16(p[2 * e + 1]) << 16);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) f.w[e] = f32_to_f16(p[2 * e]) | (f32_to_f16(p[2 * e + 1]) << 16);
  }
  return f;
}

template <int OT>
__device__ __forceinline__ void store4(uint8_t* p, float a, float b, float c, float d) {
  if constexpr (OT == DT_F32) {
    *reinterpret_cast<u32x4*>(p) = u32x4{f2u(a), f2u(b), f2u(c), f2u(d)};
  } else if constexpr (OT == DT_BF16) {
    *reinterpret_cast<u32x2*>(p) =
        u32x2{f32_to_bf16(a) | (f32_to_bf16(b) << 16), f32_to_bf16(c) | (f32_to_bf16(d) << 16)};
  } else {
    *reinterpret_cast<u32x2*>(p) =
        u32x2{f32_to_f16(a) | (f32_to_f16(b) << 16), f32_to_f16(c) | (f32_to_f16(d) << 16)};
  }
}

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
  const int kstart = part * kPartition;
  const int kend = min(min(L, kstart + kPartition), max_pos + 1);
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

  // The partition's block-table entries, one per lane (at most P/B <= 32):
  // each step then reads its physical block ids with readlane, no memory trip.
  const int jbase = kstart / BS;
  const int nbt = min(nblk - jbase, kPartition / BS);
  const int32_t* bt = a.block_tables + static_cast<int64_t>(i) * a.max_blocks_per_seq + jbase;
  const int btv = lane < nbt ? bt[lane] : 0;

  // per-lane key offsets inside a 32-key step
  const int kkey0 = 8 * (r >> 2) + (r & 3);      // sub-tile 0; sub-tile 1 adds 4
  const int vkey = 8 * lg;                        // first of the lane's 8 keys for V / P

  float m = -__builtin_inff();
  float lsum = 0.f;
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
    for (int e = 0; e < 4; ++e) { sc[e] = sf[0][e] * a.score_scale; sc[4 + e] = sf[1][e] * a.score_scale; }
    if (k0 + 31 > min_pos) {   // some key of this step is past some row's position
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[e] = (k0 + vkey + e <= row_pos) ? sc[e] : -__builtin_inff();
    }

    // ---- online softmax (row r; the four lane groups share the row)
    float mt = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sc[e]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(m, mt);
    const float mref = (mnew == -__builtin_inff()) ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - mref);
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { p[e] = __builtin_amdgcn_exp2f(sc[e] - mref); ps += p[e]; }
    lsum = lsum * alpha + ps;
    m = mnew;
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] *= alpha;

    // ---- O^T += V^T P^T
    const Frag<CT> pf = pack_p<CT>(p);
    const bool tail = k0 + 32 > L;   // keys past the end hold poison: drop them by selection
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      Frag<CT> vf = to_frag<CT, KV>(st.v[n]);
      if (tail) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k0 + vkey + e >= L) frag_zero_elem<CT>(vf, e);
      }
      acc[n] = mma<CT>(acc[n], vf, pf);
    }
  };

  // Software pipeline: the loads of step s + PF are in flight while step s
  // computes.  fp8 steps are half the bytes, so they run one step deeper.
  constexpr int PF = (KV == DT_FP8) ? 2 : (KV == DT_F32 ? 0 : 1);
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
  const int nparts_row = row_pos / kPartition + 1;
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
      a.part_m[rowp] = m;
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
__global__ __launch_bounds__(64, 2) void attn_kernel(AttnArgs a) {
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
  const int np = row_pos / kPartition + 1;
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

// Waves of a 64-thread kernel that fit on the device at once (0 -> a default).
static int64_t resident_waves(const void* kernel) {
  int dev = 0, per_cu = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64, 0) != hipSuccess || per_cu <= 0)
    return 2048;
  return static_cast<int64_t>(per_cu) * prop.multiProcessorCount;
}

template <int CT, int KV, int D, int BS>
static hipError_t launch_attn(const AttnArgs& a, hipStream_t stream, hipEvent_t before, hipEvent_t after) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, a.seq_lens, a.qsl, a.num_seqs,
                     a.group, a.header, a.items, a.max_items);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one wave per resident slot; each loops over work items until the list is done
  static const int64_t slots = resident_waves(reinterpret_cast<const void*>(&attn_kernel<CT, KV, D, BS>));
  const int64_t want = a.max_items * a.num_kv_heads;
  const int64_t waves = want < slots ? (want > 0 ? want : 1) : slots;
  if (before && (e = hipEventRecord(before, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((attn_kernel<CT, KV, D, BS>), dim3(static_cast<unsigned>(waves)), dim3(64), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (after && (e = hipEventRecord(after, stream)) != hipSuccess) return e;
  if (e != hipSuccess) return e;
  if (a.max_parts > 1 && a.num_tokens > 0) {
    hipLaunchKernelGGL((reduce_kernel<CT, D>), dim3(a.num_tokens, a.num_q_heads), dim3(64), 0, stream, a);
    e = hipGetLastError();
  }
  return e;
}

template <int CT, int KV>
static hipError_t launch_attn_shape(int d, int bs, const AttnArgs& a, hipStream_t s, hipEvent_t b,
                                    hipEvent_t e) {
  if (d == 64) {
    if (bs == 16) return launch_attn<CT, KV, 64, 16>(a, s, b, e);
    if (bs == 32) return launch_attn<CT, KV, 64, 32>(a, s, b, e);
    if (bs == 64) return launch_attn<CT, KV, 64, 64>(a, s, b, e);
  } else if (d == 128) {
    if (bs == 16) return launch_attn<CT, KV, 128, 16>(a, s, b, e);
    if (bs == 32) return launch_attn<CT, KV, 128, 32>(a, s, b, e);
    if (bs == 64) return launch_attn<CT, KV, 128, 64>(a, s, b, e);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention(int q, int kv, int d, int bs, const AttnArgs& a, hipStream_t s,
                            hipEvent_t b, hipEvent_t e) {
  if (q == DT_F32 && kv == DT_F32) return launch_attn_shape<DT_F32, DT_F32>(d, bs, a, s, b, e);
  if (q == DT_F16 && kv == DT_F16) return launch_attn_shape<DT_F16, DT_F16>(d, bs, a, s, b, e);
  if (q == DT_F16 && kv == DT_FP8) return launch_attn_shape<DT_F16, DT_FP8>(d, bs, a, s, b, e);
  if (q == DT_BF16 && kv == DT_BF16) return launch_attn_shape<DT_BF16, DT_BF16>(d, bs, a, s, b, e);
  if (q == DT_BF16 && kv == DT_FP8) return launch_attn_shape<DT_BF16, DT_FP8>(d, bs, a, s, b, e);
  return hipErrorInvalidValue;
}

}  // namespace pa

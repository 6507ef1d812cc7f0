// pa_chunk_item.h -- the chunked-prefill work loop: a workgroup of 8 waves
// draws 256-row blocks of prompt chunks and runs them over 64-key tiles of
// the paged cache staged in LDS, MFMA for both products, causal mask by
// selection.  Used by the chunk kernel and by the fused step kernel.
//
// Method: a step mixes one-token decode rows with causal prompt chunks
// (techknowgenie "vLLM V1 core refactoring", section "Dynamic Chunked
// Prefill"); the chunk's queries see the cached prefix and the chunk's own
// earlier tokens, through the block table (itwiki "vLLM", "PagedAttention").
#pragma once

#include <type_traits>

#include "pa_device.h"

namespace pa {

// LDS image of one 64-key tile in the 16-bit compute type: K rows [64][d]
// and V rows [64][d], unpadded.  The 16-byte chunks of a K row are XOR-
// swizzled so that the 16 lanes of each MFMA operand read (16 different
// rows, one chunk column) land in 16 different 16-byte bank groups.  V rows
// are read with transposing loads (lds_read_tr16), each 32-lane half of one
// touching 8 rows at one 32-byte column; the 32-byte units of a V row are
// XOR-swizzled by the row bits that differ inside such a half (bits 0, 1
// and 3), so those 8 reads land in 8 different 32-byte bank groups.
template <int D>
struct ChunkLds {
  static constexpr int KROW = D * 2;                   // bytes per K row
  static constexpr int VROW = D * 2;                   // bytes per V row
  static constexpr int KBYTES = kChunkKeys * KROW;
  static constexpr int BUF = KBYTES + kChunkKeys * VROW;
  // The K rows one read touches are {8*(r/4) + 4*tau + r%4} (mod 32).
  static __device__ __forceinline__ int kswz(int key) {
    if constexpr (D >= 128) return (key & 3) | (((key >> 3) & 3) << 2);   // 16 distinct 16-byte groups
    else return ((key >> 1) & 1) | (((key >> 3) & 3) << 1);   // 128-byte rows pair up per 256 bytes
  }
  // 32-byte unit swizzle of V row `key`; at d = 64 a row is half the banks,
  // and bit 0 of the row already picks the half
  static __device__ __forceinline__ int vswz(int key) {
    if constexpr (D >= 128) return (key & 3) | (((key >> 3) & 1) << 2);
    else return ((key >> 1) & 1) | (((key >> 3) & 1) << 1);
  }
  static __device__ __forceinline__ int koff(int key, int chunk) { return key * KROW + ((chunk ^ kswz(key)) << 4); }
  // LDS byte of logical byte `byte` of V row `key`
  static __device__ __forceinline__ int voff(int key, int byte) {
    return KBYTES + key * VROW + ((((byte >> 5) ^ vswz(key))) << 5) + (byte & 31);
  }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group,
// lane 4e + a passes the address of 4 consecutive 16-bit elements, and lane
// 4a + b receives element b of the four runs passed by lanes 4e + a, e = 0..3
// (layout measured on gfx950).  With lane 4e + a pointing at row k0 + e,
// columns 4a .. 4a+3 of a row-major matrix, lane n receives rows k0 .. k0+3
// of column n.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, x);
}

#ifndef PA_CHUNK_DMA_HINT
#define PA_CHUNK_DMA_HINT ""
#endif
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
      "global_load_lds_dwordx4 %1, off" PA_CHUNK_DMA_HINT "\n\t"
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

// Softmax step of one 16-row tile over one 64-key tile, without the row sum
// (the row sums come from the PV product with an all-ones operand): updates
// the reference max m (lazily, as in softmax_update) and rescales the
// accumulators, returns p = 2^(c*s - c*m) in the MFMA operand type.
template <int CT, int NACC>
__device__ __forceinline__ void chunk_softmax(const float (&s)[16], float& m, f32x4 (&acc)[NACC], f32x4& lacc,
                                              float c, float slack, Frag<CT> (&pf)[2]) {
  float lm = s[0];
#pragma unroll
  for (int e = 1; e < 16; ++e) lm = fmaxf(lm, s[e]);
  if (__any(lm > m + slack)) {
    float rm = fmaxf(lm, __shfl_xor(lm, 16));
    rm = fmaxf(rm, __shfl_xor(rm, 32));
    const float mnew = fmaxf(m, rm);
    const float alpha = (mnew == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f((m - mnew) * c);
    lacc *= alpha;
#pragma unroll
    for (int n = 0; n < NACC; ++n) acc[n] *= alpha;
    m = mnew;
  }
  const float cm = (m == -__builtin_inff()) ? 0.f : m * c;
#pragma unroll
  for (int kg = 0; kg < 2; ++kg) {
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * kg + e], c, -cm));
    pf[kg] = pack_p<CT>(p);
  }
}

// One workgroup (8 waves, two per SIMD) per work item: sequence i, kv head h,
// rows [256*rb, 256*rb + 256) of the sequence's (token, head-in-group) rows,
// keys of context partition `part` (a.chunk_partition keys: 8192, 16384 in
// the fused step).  Wave w owns rows 32w..32w+31 as two 16-row tiles.  Each
// 64-key tile is gathered through the block table by all 512 threads with
// 16-byte loads -- straight into LDS for 16-bit caches (global_load_lds),
// through registers for fp8, which is
// widened to the compute type on the way -- kChunkAhead tiles ahead of the
// one being computed.  Each wave runs the transposed-score MFMA scheme of
// the decode kernel, every LDS operand read feeding both of its row tiles;
// the V^T operands come from the V rows through transposing LDS reads.
//
// Keys past a row's position get score -inf by selection, on the tiles that
// hold such keys only; V rows of keys past the end of the sequence (they
// hold whatever the pool has there) are overwritten with zero in LDS.
#ifndef PA_CHUNK_AHEAD
#define PA_CHUNK_AHEAD 2
#endif
constexpr int kChunkAhead = PA_CHUNK_AHEAD;              // tiles in flight (16-bit caches)

// The workgroup's first item is `first` (dealt out in advance, -1 for
// none); after that it draws item base + k from the counter.  `prefix`: the
// items are those of the shared-prefix pass instead of the chunk list.
// CPART: keys per partition of the chunk list, the value the plan used
// (a.chunk_partition); the shared-prefix pass uses a.prefix_part <= CPART.
template <int CT, int KV, int D, int BS, int CPART>
__device__ __forceinline__ void chunk_items(const AttnArgs& a, int first, int base, bool prefix) {
  using Lds = ChunkLds<D>;
  constexpr bool DIRECT = (KV != DT_FP8);                // 16-bit cache: global -> LDS directly
  // 16-bit caches: tile t and the kChunkAhead tiles loading behind it; fp8:
  // tiles t and t+1 (staged from registers after round t computes).
  constexpr int AHEAD = D == 256 ? 1 : kChunkAhead;      // a 64 KB tile at d = 256: two buffers fit LDS
  constexpr int NBUF = DIRECT ? AHEAD + 1 : 2;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * Lds::BUF];
  __shared__ int32_t btl[CPART / BS];                    // the partition's physical block ids
  __shared__ int slot;
  constexpr int EBQ = Bytes<CT>::v;
  constexpr int EBK = Bytes<KV>::v;
  constexpr int KS = D / 32;
  constexpr int NT = D / 16;
  constexpr int RT = D == 256 ? kChunkRowTiles / 2 : kChunkRowTiles;   // row tiles per wave
  constexpr int ROWS = kChunkWaves * 16 * RT;            // rows of one item
  static_assert(ROWS == chunk_rows_for(D), "the plan and the kernel must agree on an item's rows");

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);                    // wave-uniform: keeps its branches scalar
  const int lane = tid & 63;
  const int r = lane & 15;
  const int lg = lane >> 4;
  // the prefix pass has (row block, prefix partition, kv head) items known on
  // the host; otherwise the plan's chunk list times the kv heads
  const int64_t total = prefix ? a.prefix_items : static_cast<int64_t>(uniform(a.header[3])) * a.num_kv_heads;
  const int64_t tile_bytes = static_cast<int64_t>(BS) * D * EBK;
  const int64_t blk_stride = tile_bytes * a.num_kv_heads;
  const uint32_t blk_stride32 = static_cast<uint32_t>(blk_stride);   // Hkv * B * d * eb < 2^32

  // Direct-to-LDS loads: wave w's load j fills tile bytes [base, base + 1 KB).
  // Tiles start at multiples of 64 >= B, so which key (or dim) and which
  // 16-byte chunk a lane fetches, its block relative to the tile's first
  // block and its offset inside that block are the same for every tile.
  constexpr int NI = Lds::BUF / 1024 / kChunkWaves;       // loads per wave per tile
  static_assert(Lds::BUF % (1024 * kChunkWaves) == 0, "a tile splits evenly over the waves");
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  // Per load: the block relative to the tile's first block, and the byte
  // offset inside the block.
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
      const int kk = pv / Lds::VROW;
      const int pb = pv % Lds::VROW;                       // this LDS byte holds logical byte lb of row kk
      const int lb = (((pb >> 5) ^ Lds::vswz(kk)) << 5) | (pb & 31);
      dma_rel[j] = kk / BS;
      dma_off[j] = (kk % BS) * D * EBK + lb;
    }
  }

  // LDS operand reads: lane (r, lg) reads K row kg*32 + 4*tau + rb, chunk
  // 4s + lg; the swizzle of those rows depends on r alone, so each lane
  // needs one offset per s, and kg and tau enter as immediate offsets.  V:
  // slot e of the lane's P^T operand in key group kg is key 32*kg + 8*lg + e;
  // the V^T operand of output tile n (dims 16n .. 16n+15) takes two
  // transposing reads, h = 0 and 1, in which lane (r, lg) points at row
  // 32*kg + 8*lg + 4*h + r/4, dims 16n + 4*(r%4) .. +3.  The swizzle of those
  // rows depends on r and lg alone: one offset per n (mod 8), the rest
  // immediate.
  constexpr int NV = NT < 8 ? NT : 8;
  const int rb = 8 * (r >> 2) + (r & 3);
  int kls[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) kls[s] = Lds::koff(rb, 4 * s + lg);
  int vto[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) vto[n] = Lds::voff(8 * lg + (r >> 2), 32 * n + 8 * (r & 3));

  // all-ones A operand: the PV product with it yields the row sums of P
  Frag<CT> ones;
  {
    const uint32_t one2 = CT == DT_BF16 ? 0x3F803F80u : 0x3C003C00u;
    ones.w = u32x4{one2, one2, one2, one2};
  }

  while (true) {
    int w = first;
    if (w < 0) {
      if (base >= total) break;   // every item was dealt out: a draw could only come back empty
      if (tid == 0) slot = atomicAdd(a.header + (prefix ? 4 : 2), 1);
      __syncthreads();
      w = base + uniform(slot);
      __syncthreads();   // every wave has read slot before thread 0 writes it again
    }
    first = -1;
    if (w >= total) break;
    const int G = a.group;
    int i, h, rblk, part, L, q0, rows, base_pos, tstep, cpart, kstart, pslot;
    if (prefix) {
      // all rows of the step (every token x its kv head's group) against keys
      // [part * P, ...) of the shared prefix, which every row sees whole: as if
      // each row sat at position prefix_len - 1.  Row blocks vary fastest, so
      // items that read the same keys run side by side.
      rblk = w % a.prefix_rblocks;
      const int ph = w / a.prefix_rblocks;
      h = ph % a.num_kv_heads;
      part = ph / a.num_kv_heads;
      i = 0;                                 // the prefix blocks, read from sequence 0's table row
      L = a.prefix_len;
      q0 = 0;
      rows = a.num_tokens * G;
      base_pos = a.prefix_len - 1;
      tstep = 0;
      cpart = a.prefix_part;
      kstart = part * cpart;
      pslot = part;
    } else {
      const int e = w / a.num_kv_heads;
      h = w - e * a.num_kv_heads;
      i = uniform(a.citems[2 * e]);
      const int tp = uniform(a.citems[2 * e + 1]);
      rblk = static_cast<int>(static_cast<uint32_t>(tp) >> 16);
      part = tp & 0xFFFF;
      L = min(uniform(a.seq_lens[i]), a.max_seq_len);
      q0 = uniform(a.qsl[i]);
      const int ql = uniform(a.qsl[i + 1]) - q0;
      rows = ql * G;
      base_pos = L - ql;
      tstep = 1;
      cpart = CPART;
      kstart = a.prefix_len + part * cpart;   // keys past a shared prefix only
      pslot = a.prefix_parts + part;
    }
    const int wrow0 = rblk * ROWS + wave * (16 * RT);
    const int wlast = min(rows, wrow0 + 16 * RT) - 1;     // last row of this wave (< wrow0: none)
    const int wave_min_pos = base_pos + tstep * (wrow0 / G);
    const int wave_max_pos = wlast >= wrow0 ? base_pos + tstep * (wlast / G) : -1;
    const int wg_max_pos = base_pos + tstep * ((min(rows, rblk * ROWS + ROWS) - 1) / G);
    const int kend = min(min(L, kstart + cpart), wg_max_pos + 1);

    if (kstart < kend) {
      int row_pos[RT];
      Frag<CT> qf[RT][KS];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int R = wrow0 + 16 * rt + r;
        const bool valid = R < rows;
        const int t = R / G;
        row_pos[rt] = valid ? base_pos + tstep * t : -1;
        const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                            ((static_cast<int64_t>(q0 + t) * a.num_q_heads + h * G + (R - t * G)) * D + 8 * lg) * EBQ;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          qf[rt][s] = valid ? load_frag<CT, CT>(qp + 32 * s * EBQ) : frag_zero<CT>();
      }
      float m[RT];
      f32x4 lacc[RT];
      const float slack = a.rescale_slack;
      f32x4 acc[RT][NT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        m[rt] = -__builtin_inff();
        lacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[rt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      }

      const int nblk = (L + BS - 1) / BS;
      const int jbase = kstart / BS;
      {
        // the partition's block ids; past the sequence's last block the
        // table repeats that block (keys past the end are loaded but never
        // used), so tile loads need no clamp
        const int32_t* bt = a.block_tables + static_cast<int64_t>(i) * a.max_blocks_per_seq + jbase;
        const int nb = min(nblk - jbase, cpart / BS);
        for (int j = tid; j < cpart / BS; j += kChunkThreads) {
          int id = bt[min(j, nb - 1)];
#if PA_DEBUG
          // debug build: an id outside the pool is recorded and replaced by block 0
          if (id < 0 || id >= a.num_blocks) {
            debug_record(a.debug, kDebugBlockId, i);
            id = 0;
          }
#endif
          btl[j] = id;
        }
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
        uint32_t phys[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) phys[j] = static_cast<uint32_t>(btl[jt + dma_rel[j]]);
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          // a block id times the per-block stride (< 2^32 bytes) needs one 32x32->64 multiply-add
          const uint8_t* src = ((dma_is_v[j] ? vc : kc) + dma_off[j]) + static_cast<uint64_t>(phys[j]) * blk_stride32;
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
          const int64_t src = phys_of(kt, kk) * blk_stride + static_cast<int64_t>((kt + kk) % BS) * D + cc * 16;
          kreg[j] = *reinterpret_cast<const u32x4*>(kc + src);
          vreg[j] = *reinterpret_cast<const u32x4*>(vc + src);
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
          widen16<CT>(vreg[j], lo, hi);
          *reinterpret_cast<u32x4*>(buf + Lds::voff(kk, 32 * cc)) = lo;
          *reinterpret_cast<u32x4*>(buf + Lds::voff(kk, 32 * cc + 16)) = hi;
        }
      };
      // V rows of keys kt + [live, 64) are past the end: overwrite them with
      // zero (all threads; the caller fences with a barrier).
      auto zero_tail = [&](uint8_t* buf, int live) {
        constexpr int CPR = Lds::VROW / 16;                 // 16-byte chunks per row
        for (int x = live * CPR + tid; x < kChunkKeys * CPR; x += kChunkThreads)
          *reinterpret_cast<u32x4*>(buf + Lds::voff(x / CPR, 16 * (x % CPR))) = u32x4{0u, 0u, 0u, 0u};
      };

      // ---- a tile's work on this wave's rows: scores (MFMA), softmax (VALU),
      // then the PV product (MFMA)
      f32x4 sf[RT][2][2];                                    // raw scores of the last qk
      Frag<CT> pf[RT][2];                                    // P of the last softmax, MFMA operand
      // Operand fragments are read from LDS a key group (32 keys) at a time
      // into registers, then multiplied: the group's reads are all in flight
      // together instead of each MFMA waiting for the read just before it.
      auto qk = [&](const uint8_t* buf) {
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
          Frag<CT> kf[2][KS];
#pragma unroll
          for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int s = 0; s < KS; ++s)
              kf[tau][s].w = *reinterpret_cast<const u32x4*>(buf + kls[s] + (kg * 32 + 4 * tau) * Lds::KROW);
#pragma unroll
          for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              sf[rt][kg][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s = 0; s < KS; ++s) sf[rt][kg][tau] = mma<CT>(sf[rt][kg][tau], kf[tau][s], qf[rt][s]);
            }
        }
      };
      auto softmax = [&](int kt) {
        float sc[RT][16];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int x = 0; x < 16; ++x) sc[rt][x] = sf[rt][x >> 3][(x >> 2) & 1][x & 3];
        if (kt + kChunkKeys - 1 > wave_min_pos) {
          // the lane's keys are kt + 8lg + {0..7} and kt + 8lg + 32 + {0..7}
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int vis = row_pos[rt] - kt - 8 * lg;      // visible: offset <= vis
#pragma unroll
            for (int x = 0; x < 16; ++x)
              sc[rt][x] = ((x >> 3) * 32 + (x & 7) > vis) ? -__builtin_inff() : sc[rt][x];
          }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          chunk_softmax<CT, NT>(sc[rt], m[rt], acc[rt], lacc[rt], a.score_scale, slack, pf[rt]);
      };
      auto qk_softmax = [&](const uint8_t* buf, int kt) {
        qk(buf);
        softmax(kt);
      };
      auto pv = [&](const uint8_t* buf) {
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
          // rows 32kg + 8lg + {0..3} and {4..7}: slots 0-3 and 4-7 of tile n
          u32x2 lo[NT], hi[NT];
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const uint8_t* p = buf + vto[n % NV] + 256 * (n / NV) + 32 * kg * Lds::VROW;
            lo[n] = lds_read_tr16(p);
            hi[n] = lds_read_tr16(p + 4 * Lds::VROW);
          }
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            Frag<CT> vf;
            vf.w = u32x4{lo[n][0], lo[n][1], hi[n][0], hi[n][1]};
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc[rt][n] = mma<CT>(acc[rt][n], vf, pf[rt][kg]);
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) lacc[rt] = mma<CT>(lacc[rt], ones, pf[rt][kg]);
        }
      };

      const int ntiles = (kend - kstart + kChunkKeys - 1) / kChunkKeys;
      auto tile_key = [&](int ti) { return kstart + ti * kChunkKeys; };
      auto bufp = [&](int ti) { return lds + (ti % NBUF) * Lds::BUF; };
      // wait until at most the loads of the n most recently issued tiles are outstanding
      auto wait_later = [&](int n) {
        static_assert(AHEAD >= 1 && AHEAD <= 3, "tiles in flight: 1 to 3");
        if (AHEAD >= 3 && n >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NI));
        else if (AHEAD >= 2 && n >= 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NI));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      };
      // one round: tile ti is in LDS
      auto do_round = [&](int ti) {
        const int kt = tile_key(ti);
        if (kt + kChunkKeys > L) {                           // the sequence's last keys: V tail to zero
          zero_tail(bufp(ti), L - kt);
          __syncthreads();
        }
        if (kt <= wave_max_pos) {
          qk_softmax(bufp(ti), kt);
          pv(bufp(ti));
        }
      };

      if constexpr (DIRECT) {
        // The compiler cannot see the LDS loads; retire its own loads (q) here
        // so that it has no reason to wait on the vector-memory counter later.
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        // tiles 0 .. AHEAD-1 in flight, then wait for tile 0
#pragma unroll
        for (int x = 0; x < AHEAD; ++x)
          if (x < ntiles) issue_direct(x, tile_key(x));
        wait_later(min(ntiles, AHEAD) - 1);
        __syncthreads();
        for (int ti = 0; ti < ntiles; ++ti) {
          // buffer (ti + ahead) % NBUF last held tile ti-1, finished in round ti-1
          if (ti + AHEAD < ntiles) issue_direct((ti + AHEAD) % NBUF, tile_key(ti + AHEAD));
          do_round(ti);
          // tile ti+1 has landed once at most the loads of the tiles after it are outstanding
          wait_later(min(ntiles - 2 - ti, AHEAD - 1));
          __syncthreads();
        }
      } else {
        // register set ti % 2 holds tile ti between its gather and its staging
        gather_fp8(kreg0, vreg0, tile_key(0));
        stage_fp8(kreg0, vreg0, bufp(0));
        if (ntiles > 1) gather_fp8(kreg1, vreg1, tile_key(1));
        __syncthreads();
        for (int ti = 0; ti < ntiles; ti += 2) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int tj = ti + half;
            if (tj < ntiles) {
              Regs& kr = half ? kreg1 : kreg0;   // held tile tj (already staged): free
              Regs& vr = half ? vreg1 : vreg0;
              Regs& kn = half ? kreg0 : kreg1;   // holds tile tj + 1
              Regs& vn = half ? vreg0 : vreg1;
              if (tj + 2 < ntiles) gather_fp8(kr, vr, tile_key(tj + 2));
              do_round(tj);
              // buffer (tj+1) % 2 last held tile tj-1, finished in round tj-1
              if (tj + 1 < ntiles) stage_fp8(kn, vn, bufp(tj + 1));
              __syncthreads();
            }
          }
        }
      }

#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int R = wrow0 + 16 * rt + r;
        if (R >= rows || row_pos[rt] < kstart) continue;
        const int t = R / G;
        const int token = q0 + t;
        const int head = h * G + (R - t * G);
        const float ltot = lacc[rt][0];
        // accumulator element v of tile n is dim 16n + 4lg + v
        if (a.prefix_len == 0 && row_pos[rt] / CPART == 0) {
          const float inv = a.v_scale / ltot;
          uint8_t* op = static_cast<uint8_t*>(a.out) +
                        ((static_cast<int64_t>(token) * a.num_q_heads + head) * D + 4 * lg) * EBQ;
#pragma unroll
          for (int n = 0; n < NT; ++n)
            store4<CT>(op + 16 * n * EBQ, acc[rt][n][0] * inv, acc[rt][n][1] * inv, acc[rt][n][2] * inv,
                       acc[rt][n][3] * inv);
        } else {
          // the row's list: a prompt chunk's (this item's sequence), or for
          // the prefix pass the list of the row's own sequence and kind
          int64_t row0;
          if (prefix) {
            const int s = seq_of_token(a, token);
            const int s0 = a.qsl[s];
            row0 = partial_row(a, is_chunk_seq(a, (a.qsl[s + 1] - s0) * G), s, token, token - s0, head);
          } else {
            row0 = partial_row(a, true, i, token, t, head);
          }
          if (row0 < 0) continue;
          const int64_t rowp = row0 + pslot;
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

}  // namespace pa

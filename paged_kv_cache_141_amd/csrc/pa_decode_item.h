// pa_decode_item.h -- one decode work item (a 16-row tile of one sequence
// and kv head over one context partition) on one wave, and the loop by which
// a wave draws such items from the decode list.  Used by the decode kernel
// and by the fused step kernel.
//
// Method: the itwiki "vLLM" article, section "PagedAttention" -- the cache is
// cut into B-token blocks reached through a block table ("Block table"), and
// the attention of a query is a sum over those blocks, fetched one by one;
// the result is ordinary attention ("Block-wise attention").
#pragma once

#include "pa_device.h"

namespace pa {

// Decode-kernel tuning: steps of 16-bit K/V kept in flight ahead of the one
// being computed, and the occupancy the register budget is cut for.
#ifndef PA_DECODE_PREFETCH
#define PA_DECODE_PREFETCH 2
#endif
#ifndef PA_DECODE_PREFETCH_FP8
#define PA_DECODE_PREFETCH_FP8 2
#endif
#ifndef PA_DECODE_FP8_WIDE
#define PA_DECODE_FP8_WIDE 1
#endif
#ifndef PA_DECODE_PAIR_V
#define PA_DECODE_PAIR_V 1
#endif
#ifndef PA_DECODE_NT_B64
#define PA_DECODE_NT_B64 0
#endif
#ifndef PA_DECODE_WAVES_PER_SIMD
#define PA_DECODE_WAVES_PER_SIMD 1
#endif

// The physical block ids of one partition (at most 128 blocks), two per
// lane: entry j sits in lane j % 64 of register j / 64, so a step reads its
// block with a readlane instead of a memory trip.
struct PartTable {
  int lo, hi;
  __device__ __forceinline__ void load(const int32_t* bt, int nbt, int lane) {
    lo = lane < nbt ? bt[lane] : 0;
    hi = lane + 64 < nbt ? bt[lane + 64] : 0;
  }
#if PA_DEBUG
  // debug build: an id outside the pool is recorded and replaced by block 0
  __device__ __forceinline__ void check(const AttnArgs& a, int seq) {
    if (lo < 0 || lo >= a.num_blocks) { debug_record(a.debug, kDebugBlockId, seq); lo = 0; }
    if (hi < 0 || hi >= a.num_blocks) { debug_record(a.debug, kDebugBlockId, seq); hi = 0; }
  }
#endif
  __device__ __forceinline__ int64_t operator[](int j) const {   // j wave-uniform
    const int a = __builtin_amdgcn_readlane(lo, j & 63);
    const int b = __builtin_amdgcn_readlane(hi, j & 63);
    return j < 64 ? a : b;
  }
};

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
template <int CT, int KV, int D, int BS, int PF16, int PF8, bool STREAM>
__device__ __forceinline__ void attn_item(const AttnArgs& a, int i, int tile, int part, int h,
                                          int lane) {
  constexpr int EBQ = Bytes<CT>::v;
  constexpr int EBK = Bytes<KV>::v;
  constexpr int KS = D / 32;     // K-steps of the QK^T product
  constexpr int NT = D / 16;     // 16-dim output tiles
  const int r = lane & 15;
  const int lg = lane >> 4;

  const int L = min(a.seq_lens[i], a.max_seq_len);
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
  const int kstart = a.prefix_len + part * a.partition;   // keys past a shared prefix only
  const int kend = min(min(L, kstart + a.partition), max_pos + 1);
  if (kstart >= kend) return;

  // Which dims K-step s gives lane group lg: [32s + 8lg, +8) -- or, for fp8
  // K, [64(s/2) + 16lg + 8(s%2), +8), so that one 16-byte load per lane fills
  // the lane's slots of two K-steps.  A dot product does not depend on the
  // order of its terms; Q and K only have to agree on it.
  constexpr bool WIDE = KV == DT_FP8 && PA_DECODE_FP8_WIDE;
  auto kdim = [&](int s) { return WIDE ? 64 * (s >> 1) + 16 * lg + 8 * (s & 1) : 32 * s + 8 * lg; };

  // Q^T operand: row r's dims of each K-step
  Frag<CT> qf[KS];
  {
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                        (static_cast<int64_t>(token) * a.num_q_heads + head) * D * EBQ;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = valid ? load_frag<CT, CT>(qp + kdim(s) * EBQ) : frag_zero<CT>();
  }

  const int nblk = (L + BS - 1) / BS;
  const int64_t tile_bytes = static_cast<int64_t>(BS) * D * EBK;
  const int64_t blk_stride = tile_bytes * a.num_kv_heads;
  const uint8_t* kc = static_cast<const uint8_t*>(a.k_cache) + h * tile_bytes;
  const uint8_t* vc = static_cast<const uint8_t*>(a.v_cache) + h * tile_bytes;

  // The partition's block-table entries, held in registers.
  const int jbase = kstart / BS;
  const int nbt = min(nblk - jbase, a.partition / BS);
  PartTable btv;
  btv.load(a.block_tables + static_cast<int64_t>(i) * a.max_blocks_per_seq + jbase, nbt, lane);
#if PA_DEBUG
  btv.check(a, i);
#endif

  // per-lane key offsets inside a 32-key step
  const int kkey0 = 8 * (r >> 2) + (r & 3);      // sub-tile 0; sub-tile 1 adds 4
  const int vkey = 8 * lg;                        // first of the lane's 8 keys for V / P

  float m = -__builtin_inff();
  float lsum = 0.f;
  const float slack = a.rescale_slack;
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Step {
    Raw<KV> k[2][KS];
    Raw<KV> v[NT];
  };
  // Issue the loads of the 32-key step starting at key k0 (block-table
  // gather: physical block(s) from the table register, then 16-byte reads):
  // K, then V.
  auto issue_k = [&](Step& st, int k0) {
    const int j0 = k0 / BS;
    const int64_t p0 = btv[j0 - jbase];
    int64_t p1 = p0;
    if constexpr (BS == 16) p1 = btv[min(j0 + 1, nblk - 1) - jbase];
    const int inblk = k0 - j0 * BS;   // 0 for BS <= 32; 0 or 32 for BS = 64
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int kk = kkey0 + 4 * tau;                  // key within the step
      const int64_t pb = (BS == 16 && kk >= 16) ? p1 : p0;
      const int off = (BS == 16) ? (kk & 15) : inblk + kk;
      const uint8_t* kp = kc + pb * blk_stride + static_cast<int64_t>(off) * D * EBK;
      if constexpr (WIDE) {
#pragma unroll
        for (int s = 0; s < KS; s += 2) {
          const u32x4 x = load_once<false>(reinterpret_cast<const u32x4*>(kp + kdim(s)));
          st.k[tau][s].w = u32x2{x[0], x[1]};
          st.k[tau][s + 1].w = u32x2{x[2], x[3]};
        }
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) st.k[tau][s] = load_kv<KV, false>(kp + kdim(s) * EBK);
      }
    }
  };
  auto issue_v = [&](Step& st, int k0) {
    const int j0 = k0 / BS;
    const int64_t p0 = btv[j0 - jbase];
    const int64_t pb = (BS == 16 && vkey >= 16) ? btv[min(j0 + 1, nblk - 1) - jbase] : p0;
    const int inblk = k0 - j0 * BS;
    const int off = (BS == 16) ? (vkey & 15) : inblk + vkey;
    const uint8_t* vp = vc + pb * blk_stride + (static_cast<int64_t>(r) * BS + off) * EBK;
#pragma unroll
    for (int n = 0; n < NT; ++n) st.v[n] = load_kv<KV, STREAM>(vp + static_cast<int64_t>(16 * n) * BS * EBK);
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
  // computes (PF16 steps for 16-bit caches).
  constexpr int PF = (KV == DT_FP8) ? PF8 : (KV == DT_F32 ? 0 : PF16);
  // 64-key blocks: a step reads half of each 128-byte V^T row, so the V loads
  // of a block's two steps go out together (with the first step's K), and
  // whole rows are read at once.  That takes one more step buffer: the second
  // step's V lands a step earlier than its K.  (kstart is a multiple of 64,
  // so even steps start blocks.)
  constexpr bool PAIRV = BS == 64 && PF >= 2 && PA_DECODE_PAIR_V;
  constexpr int NB = PAIRV ? (PF + 3) / 2 * 2 : PF + 1;   // PAIRV: PF + 2 rounded up to even
  static_assert(!PAIRV || NB % 2 == 0, "step parity must be static in the ring");
  Step buf[NB];
  const int nsteps = (kend - kstart + 31) / 32;
  // issue step s into buf[b]
  auto issue = [&](int b, int s) {
    issue_k(buf[b], kstart + 32 * s);
    if constexpr (PAIRV) {
      if ((b & 1) == 0) {
        issue_v(buf[b], kstart + 32 * s);
        if (s + 1 < nsteps) issue_v(buf[(b + 1) % NB], kstart + 32 * (s + 1));
      }
    } else {
      issue_v(buf[b], kstart + 32 * s);
    }
  };
#pragma unroll
  for (int s = 0; s < PF; ++s)
    if (s < nsteps) issue(s, s);
  for (int s0 = 0; s0 < nsteps; s0 += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int s = s0 + b;
      if (s >= nsteps) break;
      if (s + PF < nsteps) issue((b + PF) % NB, s + PF);
      compute(buf[b], kstart + 32 * s);
    }
  }

  // ---- finish: whole-row denominator, then the output or a partial
  float ltot = lsum + __shfl_xor(lsum, 16);
  ltot += __shfl_xor(ltot, 32);
  if (!valid || row_pos < kstart) return;
  const int nparts_row = (row_pos - a.prefix_len) / a.partition + 1;
  if (nparts_row == 1 && a.prefix_len == 0) {
    const float inv = a.v_scale / ltot;
    uint8_t* op = static_cast<uint8_t*>(a.out) +
                  ((static_cast<int64_t>(token) * a.num_q_heads + head) * D + 4 * lg) * EBQ;
#pragma unroll
    for (int n = 0; n < NT; ++n)
      store4<CT>(op + 16 * n * EBQ, acc[n][0] * inv, acc[n][1] * inv, acc[n][2] * inv, acc[n][3] * inv);
  } else {
    const int64_t row0 = partial_row(a, false, i, token, t, head);
    if (row0 < 0) return;
    const int64_t rowp = row0 + a.prefix_parts + part;
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

// A wave runs decode work items; item w covers list entry w / Hkv and kv
// head w % Hkv.  Items 0 .. base-1 are dealt out one per wave in advance
// (`first`, -1 for none): the first round costs no atomic, so a short step is
// not held up by a queue of atomics on one counter.  After that the wave
// draws item base + k from the counter, and returns once it passes the
// item count.
template <int CT, int KV, int D, int BS, int PF16, int PF8, bool STREAM>
__device__ __forceinline__ void decode_items(const AttnArgs& a, int lane, int first, int base) {
  const int64_t total = static_cast<int64_t>(uniform(a.header[1])) * a.num_kv_heads;
  int w = first;
  while (true) {
    if (w < 0) {
      int k = 0;
      if (lane == 0) k = atomicAdd(a.header, 1);
      w = base + uniform(__shfl(k, 0));
    }
    if (w >= total) break;
    // head dim 256: a 32-key step is 32 KiB of 16-bit K/V, so one step is in
    // flight while the other computes
    constexpr int PFD = D == 256 ? 1 : PF16;
    const int e = w / a.num_kv_heads;
    const int h = w - e * a.num_kv_heads;
    const int i = uniform(a.items[2 * e]);
    const int tp = uniform(a.items[2 * e + 1]);
    // the hint only where a step reads whole V rows (B no more than the
    // step's keys): a step that reads half of each row and leaves the other
    // half to the next step measured 1.5x slower with it (B 64: 1,080 against
    // 733 us for the LLaMA-7B decode kernel at B 16)
    // (tile, partition) are the unsigned 16-bit halves of tp: tiles reach 0xFFFF
    attn_item<CT, KV, D, BS, PFD, PF8, STREAM && (BS <= 32 || PA_DECODE_NT_B64)>(
        a, i, static_cast<int>(static_cast<uint32_t>(tp) >> 16), tp & 0xFFFF, h, lane);
    w = -1;
  }
}

}  // namespace pa

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
// sequence's q_len*G (token, head-in-group) rows, the keys of item `part` of
// the tile's DecodeCut (S = split_s split partitions).
//
// Lane l = r + 16*lg (r = l % 16, lg = l / 16).  The 16x16 MFMA result tile
// puts column r in lane r + 16*(row/4), element row%4.  The score tile is
// computed transposed, S^T = K * Q^T (rows = keys, columns = query rows), with
// K-tile row m of sub-tile tau holding key 8*(m%4) + 4*tau + m/4 of the
// 32-key step: then lane l ends up with the scores of query row r for the
// eight keys 4*e + lg (e = 0..7), and slot e of the lane's P^T operand is key
// 4*e + lg.  The PV product O^T = V^T * P^T reads, for each of those keys, a
// run of consecutive dims of its V row (VGeo): one instruction covers four
// consecutive keys' whole rows, and the runs are transposed in registers.
template <int CT, int KV, int D, int BS, int PF16, int PF8, bool STREAM>
__device__ __forceinline__ void attn_item(const AttnArgs& a, int i, int tile, int part, int L, int ql,
                                          int split_s, int h, int lane) {
  constexpr int EBQ = Bytes<CT>::v;
  constexpr int EBK = Bytes<KV>::v;
  constexpr int KS = D / 32;     // K-steps of the QK^T product
  using VG = VGeo<EBK, D>;
  constexpr int NT = VG::NT;     // 16-dim output tiles
  constexpr int SEG = VG::SEG, NSEG = VG::NSEG, VW = VG::WORDS;
  const int r = lane & 15;
  const int lg = lane >> 4;

  const int q0 = a.qsl[i];
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
  const DecodeCut cut(L - a.prefix_len, a.partition, a.split_f, split_s);
  const int klen = cut.len(part);
  const int kstart = a.prefix_len + cut.start(part);       // keys past a shared prefix only
  const int kend = min(min(L, kstart + klen), max_pos + 1);
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
  // the lane's first V run (dims SEG*r ..) of a tile
  const uint8_t* vc = static_cast<const uint8_t*>(a.v_cache) + h * tile_bytes + SEG * r * EBK;

  // The partition's block-table entries, held in registers.
  const int jbase = kstart / BS;
  const int nbt = min(nblk - jbase, klen / BS);
  PartTable btv;
  btv.load(a.block_tables + static_cast<int64_t>(i) * a.max_blocks_per_seq + jbase, nbt, lane);
#if PA_DEBUG
  btv.check(a, i);
#endif

  // the key of the lane's K-tile row in sub-tile 0 (sub-tile 1 adds 4)
  const int kkey0 = 8 * (r & 3) + (r >> 2);

  float m = -__builtin_inff();
  float lsum = 0.f;
  const float slack = a.rescale_slack;
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Step {
    Raw<KV> k[2][KS];
    Words<VW> v[8][NSEG];          // run c of key 4e + lg
  };
  // Issue the loads of the 32-key step starting at key k0 (block-table
  // gather: physical block(s) from the table register, then the reads): K,
  // then V.
  auto issue = [&](Step& st, int k0) {
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
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kk = 4 * e + lg;
      const int64_t pb = (BS == 16 && e >= 4) ? p1 : p0;   // wave-uniform per e
      const int off = (BS == 16) ? (kk & 15) : inblk + kk;
      const uint8_t* vp = vc + pb * blk_stride + static_cast<int64_t>(off) * D * EBK;
#pragma unroll
      for (int c = 0; c < NSEG; ++c) st.v[e][c] = load_words<VW, STREAM>(vp + 16 * SEG * c * EBK);
    }
  };

  auto compute = [&](Step& st, int k0) {
    // ---- S^T = K Q^T
    f32x4 sf[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      sf[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) sf[tau] = mma<CT>(sf[tau], to_frag<CT, KV>(st.k[tau][s]), qf[s]);
    }
    // element i2 of sub-tile tau is key 8*i2 + 4*tau + lg = 4*e + lg, e = 2*i2 + tau
    float sc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sc[e] = sf[e & 1][e >> 1];
    if (k0 + 31 > min_pos) {   // some key of this step is past some row's position
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[e] = (k0 + 4 * e + lg <= row_pos) ? sc[e] : -__builtin_inff();
    }
    // ---- online softmax (row r; the four lane groups share the row)
    float p[8];
    softmax_update<8, NT>(sc, m, lsum, acc, a.score_scale, slack, p);

    // ---- O^T += V^T P^T (keys past the end hold poison: their V runs are
    // replaced by zero, by selection)
    const Frag<CT> pf = pack_p<CT>(p);
    if (k0 + 32 > L) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool dead = k0 + 4 * e + lg >= L;
#pragma unroll
        for (int c = 0; c < NSEG; ++c)
#pragma unroll
          for (int x = 0; x < VW; ++x) st.v[e][c].w[x] = dead ? 0u : st.v[e][c].w[x];
      }
    }
#pragma unroll
    for (int c = 0; c < NSEG; ++c) {
      if constexpr (KV == DT_FP8) {
        // byte jj of each run: 4x4 byte transposes of keys 0-3 and 4-7, then
        // widened two codes at a time
#pragma unroll
        for (int x = 0; x < VW; ++x) {
          uint32_t lo[4], hi[4];
          byte_transpose4(st.v[0][c].w[x], st.v[1][c].w[x], st.v[2][c].w[x], st.v[3][c].w[x], lo);
          byte_transpose4(st.v[4][c].w[x], st.v[5][c].w[x], st.v[6][c].w[x], st.v[7][c].w[x], hi);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            Frag<CT> vf;
            vf.w[0] = widen2<CT>(lo[b], false);
            vf.w[1] = widen2<CT>(lo[b], true);
            vf.w[2] = widen2<CT>(hi[b], false);
            vf.w[3] = widen2<CT>(hi[b], true);
            const int j = SEG * c + 4 * x + b;
            acc[j] = mma<CT>(acc[j], vf, pf);
          }
        }
      } else {
        Words<VW> run[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) run[e] = st.v[e][c];
#pragma unroll
        for (int jj = 0; jj < SEG; ++jj) {
          const int j = SEG * c + jj;
          if constexpr (KV == DT_F32) acc[j] = mma<CT>(acc[j], vt_frag32(run, jj), pf);
          else acc[j] = mma<CT>(acc[j], vt_frag16<CT>(run, jj), pf);
        }
      }
    }
  };

  // Software pipeline: the loads of step s + PF are in flight while step s
  // computes (PF16 steps for 16-bit caches).
  constexpr int PF = (KV == DT_FP8) ? PF8 : (KV == DT_F32 ? 0 : PF16);
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

  // ---- finish: whole-row denominator, then the output or a partial.  Lane
  // (r, lg) holds, for each run c, dims 16*SEG*c + 4*SEG*lg + [0, 4*SEG) of
  // row r: accumulator element v of tile SEG*c + jj is dim 16*SEG*c +
  // SEG*(4*lg + v) + jj.
  float ltot = lsum + __shfl_xor(lsum, 16);
  ltot += __shfl_xor(ltot, 32);
  if (!valid || row_pos < kstart) return;
  const int nparts_row = cut.item_of(row_pos - a.prefix_len) + 1;
  auto dim0 = [&](int c, int v) { return 16 * SEG * c + SEG * (4 * lg + v); };
  if (nparts_row == 1 && a.prefix_len == 0) {
    const float inv = a.v_scale / ltot;
    uint8_t* op = static_cast<uint8_t*>(a.out) + (static_cast<int64_t>(token) * a.num_q_heads + head) * D * EBQ;
#pragma unroll
    for (int c = 0; c < NSEG; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int jj = 0; jj < SEG; jj += 4) {
          const int j = SEG * c + jj;
          store4<CT>(op + (dim0(c, v) + jj) * EBQ, acc[j][v] * inv, acc[j + 1][v] * inv, acc[j + 2][v] * inv,
                     acc[j + 3][v] * inv);
        }
  } else {
    const int64_t prow = partial_row(a, false, i, token, t, head);
    if (prow < 0) return;
    const int64_t rowp = prow + a.prefix_parts + part;
    if (lg == 0) {
      a.part_m[rowp] = max_log2(m, a.score_scale);
      a.part_l[rowp] = ltot;
    }
    float* pp = a.part_acc + rowp * D;
    const float vs = a.v_scale;
#pragma unroll
    for (int c = 0; c < NSEG; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int jj = 0; jj < SEG; jj += 4) {
          const int j = SEG * c + jj;
          *reinterpret_cast<f32x4*>(pp + dim0(c, v) + jj) =
              f32x4{acc[j][v], acc[j + 1][v], acc[j + 2][v], acc[j + 3][v]} * vs;
        }
  }
}

// Decode item w: list entry w / Hkv, kv head w % Hkv.
template <int CT, int KV, int D, int BS, int PF16, int PF8, bool STREAM>
__device__ __forceinline__ void decode_item(const AttnArgs& a, int64_t w, int split_s, int lane) {
  // head dim 256: a 32-key step is 32 KiB of 16-bit K/V, so one step is in
  // flight while the other computes
  constexpr int PFD = D == 256 ? 1 : PF16;
  const int64_t e = w / a.num_kv_heads;
  const int h = static_cast<int>(w - e * a.num_kv_heads);
  const int4 rec = *reinterpret_cast<const int4*>(a.items + kDecodeItemWords * e);
  const int i = uniform(rec.x);
  const int tp = uniform(rec.y);
  // (tile, partition) are the unsigned 16-bit halves of tp: tiles reach 0xFFFF
  attn_item<CT, KV, D, BS, PFD, PF8, STREAM>(a, i, static_cast<int>(static_cast<uint32_t>(tp) >> 16), tp & 0xFFFF,
                                             uniform(rec.z), uniform(rec.w), split_s, h, lane);
}

// The decode items of a launch: the list's entries (plan header word 1)
// times the kv heads.
__device__ __forceinline__ int64_t decode_total(const AttnArgs& a) {
  return static_cast<int64_t>(uniform(a.header[1])) * a.num_kv_heads;
}

// A wave runs decode work items (`total` of them, from decode_total;
// `split_s` the tail split's partitions per row tile, plan header word 7);
// item w covers list entry w / Hkv and kv head w % Hkv.  Items 0 .. base-1 are dealt out one per wave in advance
// (`first`, -1 for none): the first round costs no atomic, so a short step is
// not held up by a queue of atomics on one counter.  After that the wave
// draws item base + k from the counter, and returns once it passes the
// item count -- or at once when base already does: with every item dealt
// out, a draw could only come back empty, and the waves' last draws would
// all queue on the counter together.
template <int CT, int KV, int D, int BS, int PF16, int PF8, bool STREAM>
__device__ __forceinline__ void decode_items(const AttnArgs& a, int lane, int first, int base, int64_t total,
                                             int split_s) {
  int w = first;
  while (true) {
    if (w < 0) {
      if (base >= total) break;
      int k = 0;
      if (lane == 0) k = atomicAdd(a.header, 1);
      w = base + uniform(__shfl(k, 0));
    }
    if (w >= total) break;
    decode_item<CT, KV, D, BS, PF16, PF8, STREAM>(a, w, split_s, lane);
    w = -1;
  }
}

// The decode kernel's item loop: wave b of nw starts on item b, dealt out in
// advance like decode_items' first round, and then draws -- from the one
// counter, or, with `by_xcd`, from its XCD's class of items.  The class form
// is for steps whose block tables share blocks.  Workgroups (here one wave
// each) go to the chip's eight XCDs in turn, each XCD with its own L2, so
// wave b runs on XCD b % 8; it takes only items of class b % 8 (item w is
// in class w % 8, so a class holds whole kv heads when 8 divides Hkv, and
// one XCD's L2 holds the shared blocks of its heads instead of every XCD's
// L2 holding all of them), drawing them from its class's counter (header
// words kXcdCounters .. +7, zeroed by the plan).  Every item runs once when
// the grid has at least eight waves (each class then has a wave); the
// caller asks for classes only then.  Without shared blocks the classes are
// slower: an XCD held to some heads reads fixed offsets of every block.  One
// call site of the item body for both forms keeps the kernel's code small.
template <int CT, int KV, int D, int BS, int PF16, int PF8, bool STREAM>
__device__ __forceinline__ void decode_items_dealt(const AttnArgs& a, int lane, int b, int nw, int64_t total,
                                                   int split_s, bool by_xcd) {
  const int c = b & 7;
  const int64_t dealt = by_xcd ? (nw - c + 7) >> 3 : nw;    // waves drawing from the same counter
  const int64_t stride = by_xcd ? 8 : 1;
  const int64_t first = by_xcd ? c : 0;                      // the counter's items: first + stride * m
  int32_t* const counter = by_xcd ? a.header + kXcdCounters + c : a.header;
  int64_t w = b;
  while (w < total) {
    decode_item<CT, KV, D, BS, PF16, PF8, STREAM>(a, w, split_s, lane);
    if (first + stride * dealt >= total) break;             // every item was dealt out
    int k = 0;
    if (lane == 0) k = atomicAdd(counter, 1);
    w = first + stride * (dealt + uniform(__shfl(k, 0)));
  }
}

}  // namespace pa

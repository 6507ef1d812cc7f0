// pa_attention.hip -- one attention step: the work-list kernel, the decode
// and chunk kernels (pa_decode.hip, pa_chunk.hip), and the log-sum-exp merge
// of split-context partials.
#include "pa_cache_write.h"
#include "pa_device.h"

namespace pa {

// Keys a work item visits (its keys [kstart, kstart + len) clipped to the
// sequence and to the causal reach of its last row), in units of the
// kernel's key step; 0 for an item with nothing to do.  Must agree with the
// kernels' own bounds.
__device__ __forceinline__ int item_size(int L, int ql, int G, int row0, int nrows, int kstart, int len,
                                         int step) {
  const int rows = ql * G;
  const int last = min(rows, row0 + nrows) - 1;
  const int max_pos = L - ql + last / G;
  const int kend = min(min(L, kstart + len), max_pos + 1);
  return kend > kstart ? (kend - kstart + step - 1) / step : 0;
}

// One workgroup builds both work lists -- decode: (sequence, 16-row tile,
// item of the tile's DecodeCut); chunk: (sequence, 256-row block, partition
// of a.chunk_partition keys) -- longest item first: items are bucketed by the
// number of key steps they visit (32 keys for decode, 64 for chunks, counted
// in pairs for 16384-key partitions) and the buckets
// are laid out in descending order, so the persistent kernels, which take
// items in list order, start the long ones first and end on short ones.
// Order within a bucket is arbitrary; no result depends on it.  It also
// resets the work counters the attention kernels draw from.
//
// Sequences are taken 1024 at a time; a scan of their item counts flattens
// the batch's items so that all threads share them evenly.
//
// Tail split (a.split_f > 1): with fewer than kSplitItemsPerWave whole
// partitions per decode wave the plan sets S, the partitions each row tile
// cuts into fine items, so that the fine items come to kSplitRounds
// partitions per wave: S = ceil(kSplitRounds * waves / (row tiles * Hkv)),
// at most a.split_max.  S goes to header[7] for the decode kernel and the
// merge.
__device__ __forceinline__ void plan_block(AttnArgs a) {
  constexpr int NB0 = kPartitionMax / 32 + 1;            // decode buckets: 0 .. 64 steps
  // chunk buckets: 0 .. 128, in units of cb tiles (2 for 16384-key partitions)
  constexpr int CBMAX = kChunkPartitionMax > 8192 ? kChunkPartitionMax / 8192 : 1;
  constexpr int NB1 = kChunkPartitionMax / (kChunkKeys * CBMAX) + 1;
  const int cb = a.chunk_partition > 8192 ? a.chunk_partition / 8192 : 1;
  constexpr int NBMAX = (NB0 > NB1 ? NB0 : NB1);
  static_assert(NBMAX <= 192, "the bucket scan covers 3 x 64 buckets");
  __shared__ int hist[2][NBMAX];
  __shared__ int scan[1024];                             // inclusive item-count scan of the batch
  __shared__ int sL[1024], sQ[1024], sNP[1024];          // per sequence: L, q_len, partitions (<0: chunk list)
  __shared__ int total[2];
  __shared__ int wtot[16];                               // per-wave totals of the batch scan
  __shared__ int hset[kShareSlots];                      // first blocks seen (one batch), -1 free
  __shared__ int shared_blocks;
  const int tid = threadIdx.x;
  const int G = a.group;
  for (int x = tid; x < 2 * NBMAX; x += 1024) hist[x / NBMAX][x % NBMAX] = 0;
  // sharing is looked for in steps of one batch with at least kShareMinSeqs
  // sequences and no declared prefix (a caller that declares one has said
  // what is shared; the decode items then read only the blocks past it)
  const bool find_sharing = a.num_seqs <= 1024 && a.num_seqs >= kShareMinSeqs && a.prefix_len == 0;
  if (find_sharing)
    for (int x = tid; x < kShareSlots; x += 1024) hset[x] = -1;
  if (tid == 0) shared_blocks = 0;
  int first_block = -1;                                  // this thread's sequence's first block

  int S = 0;                                             // tail split: partitions each row tile cuts
  const bool one_batch = a.num_seqs <= 1024;

  // batch of sequences [base, base + 1024): fill the per-sequence table and
  // the scan (`again`: the same batch counted again, L and q_len from the table)
  auto load_batch = [&](int base, bool again) {
    const int i = base + tid;
    int n = 0, L = 0, ql = 0, np = 0;
    if (again) {
      L = sL[tid];
      ql = sQ[tid];
    } else if (i < a.num_seqs) {
      L = min(a.seq_lens[i], a.max_seq_len);
      ql = a.qsl[i + 1] - a.qsl[i];
      if (find_sharing && a.max_blocks_per_seq > 0)
        first_block = a.block_tables[static_cast<int64_t>(i) * a.max_blocks_per_seq];
#if PA_DEBUG
      // debug build: a sequence whose metadata breaks the contract is
      // recorded and skipped (no work items)
      {
        const int Lraw = a.seq_lens[i];
        int code = kDebugNone;
        if (ql < 0 || (i == 0 && a.qsl[0] != 0) || (i == a.num_seqs - 1 && a.qsl[a.num_seqs] != a.num_tokens))
          code = kDebugQueryStart;
        else if (Lraw < 0 || Lraw > a.max_seq_len) code = kDebugSeqLen;
        else if (ql > Lraw) code = kDebugQueryLen;
        else if (ql > a.max_query_len) code = kDebugMaxQuery;
        else {
          const int nb = (L + a.block_size - 1) / a.block_size;
          if (nb > a.max_blocks_per_seq) code = kDebugBlockId;
          const int32_t* row = a.block_tables + static_cast<int64_t>(i) * a.max_blocks_per_seq;
          for (int j = 0; j < nb && code == kDebugNone; ++j)
            if (row[j] < 0 || row[j] >= a.num_blocks) code = kDebugBlockId;
        }
        if (code != kDebugNone) {
          debug_record(a.debug, code, i);
          ql = 0;
        }
      }
#endif
    }
    if (i < a.num_seqs) {
      const int rows = ql * G;
      const int own = L - a.prefix_len;                   // keys past the shared prefix
      if (ql > 0 && own > 0) {
        if (is_chunk_seq(a, rows)) {
          np = (own + a.chunk_partition - 1) / a.chunk_partition;
          n = ((rows + a.chunk_rows - 1) / a.chunk_rows) * np;
          np = -np;
        } else {
          np = DecodeCut(own, a.partition, a.split_f, S).n;
          n = ((rows + kTileRows - 1) / kTileRows) * np;
        }
      }
    }
    // inclusive scan of n: within each wave by shuffles, then the wave totals
    const int lane = tid & 63, wv = tid >> 6;
    int v = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o);
      if (lane >= o) v += u;
    }
    __syncthreads();                                     // the previous batch is done with the table
    sL[tid] = L;
    sQ[tid] = ql;
    sNP[tid] = np;
    if (lane == 63) wtot[wv] = v;
    __syncthreads();
    int before = 0;
    for (int x = 0; x < wv; ++x) before += wtot[x];
    scan[tid] = v + before;
    __syncthreads();
  };
  // item k of the batch: its sequence (batch-relative), list, tile, partition and bucket
  auto item = [&](int k, int& j, int& list, int& t, int& p, int& bucket) {
    int lo = 0, hi = 1023;                               // first j with scan[j] > k
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (scan[mid] > k) hi = mid; else lo = mid + 1;
    }
    j = lo;
    const int idx = k - (j ? scan[j - 1] : 0);
    const int L = sL[j], ql = sQ[j], np = sNP[j];
    list = np < 0 ? 1 : 0;
    const int npp = np < 0 ? -np : np;
    t = idx / npp;
    p = idx - t * npp;
    if (list) {
      bucket = (item_size(L, ql, G, t * a.chunk_rows, a.chunk_rows, a.prefix_len + p * a.chunk_partition,
                          a.chunk_partition, kChunkKeys) + cb - 1) / cb;
    } else {
      const DecodeCut cut(L - a.prefix_len, a.partition, a.split_f, S);
      bucket = item_size(L, ql, G, t * kTileRows, kTileRows, a.prefix_len + cut.start(p), cut.len(p), 32);
    }
  };

  // Tail split (the host allows it only below 1,024 (sequence, kv head)
  // pairs, so with one batch, and only in steps without chunk rows): the
  // batch's item count with whole partitions is then its partition count.
  // With fewer than kSplitItemsPerWave per decode wave, S follows from the
  // row tiles, and the batch is counted again with the split.
  if (one_batch) {
    load_batch(0, false);
    // Block sharing (find_sharing): do two of the batch's decode-routed
    // sequences start in the same block?  Then their tables share
    // blocks, and the decode kernel deals its items by XCD so that each L2
    // holds one class of kv heads (decode_items_dealt).  A hash set in LDS of
    // the first blocks finds a repeat; the loads were issued beside the
    // sequence's metadata.  (Load-balancing only: no result depends on it.)
    if (find_sharing && tid < a.num_seqs && sQ[tid] > 0 && sL[tid] > 0 && sNP[tid] > 0 && first_block >= 0) {
      int slot = static_cast<int>((static_cast<uint32_t>(first_block) * 2654435761u) >> (32 - kShareBits));
      for (int probe = 0; probe < kShareSlots; ++probe) {
        const int prev = atomicCAS(&hset[slot], -1, first_block);
        if (prev == -1) break;
        if (prev == first_block) {
          shared_blocks = 1;
          break;
        }
        slot = (slot + 1) & (kShareSlots - 1);
      }
    }
    if (find_sharing) __syncthreads();                   // (uniform)
    if (a.split_f > 1 && static_cast<int64_t>(scan[1023]) * a.num_kv_heads <
                             static_cast<int64_t>(kSplitItemsPerWave) * a.decode_waves) {
      const int own = sL[tid] - a.prefix_len;
      int tiles = sQ[tid] > 0 && own > 0 ? (sQ[tid] * G + kTileRows - 1) / kTileRows : 0;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) tiles += __shfl_xor(tiles, o);
      if ((tid & 63) == 0) wtot[tid >> 6] = tiles;
      __syncthreads();
      int pairs = 0;
      for (int x = 0; x < 16; ++x) pairs += wtot[x];
      if (pairs > 0) {
        const int64_t pk = static_cast<int64_t>(pairs) * a.num_kv_heads;
        const int64_t want = static_cast<int64_t>(ceilf(kSplitRounds * a.decode_waves / static_cast<float>(pk)));
        S = static_cast<int>(want < a.split_max ? want : a.split_max);
        load_batch(0, true);                             // (its first barrier orders the wtot reads)
      }
    }
  }

  // pass 1: bucket sizes.  With one batch, a thread's first KEEP items stay
  // in registers for pass 2.
  constexpr int KEEP = 4;
  int cj[KEEP], cl[KEEP], ct[KEEP], cp[KEEP], cb2[KEEP];
  for (int base = 0; base < a.num_seqs; base += 1024) {
    if (!one_batch) load_batch(base, false);
    const int nk = scan[1023];
#pragma unroll
    for (int m = 0; m < KEEP; ++m) {
      const int k = tid + 1024 * m;
      if (k < nk) {
        item(k, cj[m], cl[m], ct[m], cp[m], cb2[m]);
        atomicAdd(&hist[cl[m]][cb2[m]], 1);
      }
    }
    for (int k = tid + 1024 * KEEP; k < nk; k += 1024) {
      int j, list, t, p, bucket;
      item(k, j, list, t, p, bucket);
      atomicAdd(&hist[list][bucket], 1);
    }
  }
  __syncthreads();
  // fused step: split the step kernel's workgroups between the two lists by
  // their estimated times (the histograms hold the items' step / tile counts)
  if (a.fused) {
    if (tid < 64) {                                      // one wave sums the histograms
      float dsteps = 0.f, ctiles = 0.f;
      for (int b = 1 + tid; b < NB0; b += 64) dsteps += static_cast<float>(b) * hist[0][b];
      for (int b = 1 + tid; b < NB1; b += 64) ctiles += static_cast<float>(b * cb) * hist[1][b];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        dsteps += __shfl_xor(dsteps, o);
        ctiles += __shfl_xor(ctiles, o);
      }
      const float td = dsteps * a.num_kv_heads * a.step_dec_us;     // whole chip, full bandwidth
      const float tc = ctiles * a.num_kv_heads * a.step_chunk_us;   // whole chip
      const int n = a.step_groups;
      int nd = n;
      if (dsteps == 0.f) {
        nd = 0;
      } else if (ctiles > 0.f) {
        // k decode workgroups: decode takes td * s n / k (k <= s n, s the
        // saturation share; td beyond), chunks tc * n / (n - k).  The first
        // falls and the second rises with k: they meet at k = s td n / (tc + s td),
        // and past s n only the chunk time grows.
        const float sat = kFusedDecodeSaturation * n;
        const float k = fminf(sat, kFusedDecodeSaturation * td * n / (tc + kFusedDecodeSaturation * td));
        nd = min(max(static_cast<int>(k + 0.5f), 1), n - 1);
      }
      if (tid == 0) a.header[6] = nd;
    }
    __syncthreads();                                     // hist is rewritten below
  }
  // bucket starts, longest bucket first: one wave per list scans the reversed
  // histogram (lanes take buckets b, b + 64 and b + 128)
  if (tid < 128) {
    const int list = tid >> 6, lane = tid & 63;
    const int nb = list ? NB1 : NB0;
    int carry = 0;
    for (int half = 0; half < (nb + 63) / 64; ++half) {
      const int r = lane + 64 * half;                    // rank from the longest bucket
      const int b = nb - 1 - r;
      const int c = b >= 0 ? hist[list][b] : 0;
      int incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      if (b >= 0) hist[list][b] = carry + incl - c;
      carry += __shfl(incl, 63);
    }
    if (lane == 0) total[list] = carry;
  }
  __syncthreads();
  // pass 2: place every item in its bucket (a single batch is still loaded)
  auto place = [&](int base, int j, int list, int t, int p, int bucket) {
    const int pos = atomicAdd(&hist[list][bucket], 1);
    if (pos >= (list ? a.max_citems : a.max_items)) return;   // only with metadata beyond the host bounds
    const int32_t tp = static_cast<int32_t>((static_cast<uint32_t>(t) << 16) | static_cast<uint32_t>(p));
    if (list) {
      a.citems[2 * pos] = base + j;
      a.citems[2 * pos + 1] = tp;
    } else {
      // decode items also carry L (clipped to max_seq_len) and q_len
      *reinterpret_cast<int4*>(a.items + kDecodeItemWords * static_cast<int64_t>(pos)) =
          int4{base + j, tp, sL[j], sQ[j]};
    }
  };
  for (int base = 0; base < a.num_seqs; base += 1024) {
    if (!one_batch) load_batch(base, false);
    const int nk = scan[1023];
#pragma unroll
    for (int m = 0; m < KEEP; ++m) {
      const int k = tid + 1024 * m;
      if (k < nk) {
        if (!one_batch) item(k, cj[m], cl[m], ct[m], cp[m], cb2[m]);
        place(base, cj[m], cl[m], ct[m], cp[m], cb2[m]);
      }
    }
    for (int k = tid + 1024 * KEEP; k < nk; k += 1024) {
      int j, list, t, p, bucket;
      item(k, j, list, t, p, bucket);
      place(base, j, list, t, p, bucket);
    }
  }
  if (tid == 0) {
    a.header[0] = 0;
    a.header[1] = static_cast<int32_t>(total[0] < a.max_items ? total[0] : a.max_items);
    a.header[2] = 0;
    a.header[4] = 0;
    a.header[3] = static_cast<int32_t>(total[1] < a.max_citems ? total[1] : a.max_citems);
    a.header[7] = S;
    a.header[kShareWord] = shared_blocks;
  }
  if (tid < 8) a.header[kXcdCounters + tid] = 0;
}

__global__ __launch_bounds__(1024) void plan_kernel(AttnArgs a) { plan_block(a); }

// The plan beside a cache write of the step's new tokens, in one launch:
// workgroup 0 builds the work lists while the others scatter the new K/V
// rows, kPlanWriteTokens tokens of one kv head each.  The two are
// independent (the plan reads only the step's metadata), and the attention
// kernels that follow see both.
constexpr int kPlanWriteTokens = 64;

template <int SRC, int KV>
__global__ __launch_bounds__(1024) void plan_write_kernel(AttnArgs a, CacheWriteArgs w) {
  if (blockIdx.x == 0) {
    plan_block(a);
    return;
  }
  const int b = static_cast<int>(blockIdx.x) - 1;
  const int h = b % w.num_kv_heads;
  const int t0 = (b / w.num_kv_heads) * kPlanWriteTokens;
  write_rows<SRC, KV>(w, t0, min(kPlanWriteTokens, w.num_tokens - t0), h, threadIdx.x, 1024);
}

template <int SRC>
static hipError_t launch_plan_write_kv(int kv, const AttnArgs& a, const CacheWriteArgs& w, unsigned groups,
                                       hipStream_t stream) {
  switch (kv) {
    case DT_F32: hipLaunchKernelGGL((plan_write_kernel<SRC, DT_F32>), dim3(groups), dim3(1024), 0, stream, a, w); break;
    case DT_F16: hipLaunchKernelGGL((plan_write_kernel<SRC, DT_F16>), dim3(groups), dim3(1024), 0, stream, a, w); break;
    case DT_BF16: hipLaunchKernelGGL((plan_write_kernel<SRC, DT_BF16>), dim3(groups), dim3(1024), 0, stream, a, w); break;
    case DT_FP8: hipLaunchKernelGGL((plan_write_kernel<SRC, DT_FP8>), dim3(groups), dim3(1024), 0, stream, a, w); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

static hipError_t launch_plan_write(int src, int kv, const AttnArgs& a, const CacheWriteArgs& w, hipStream_t stream) {
  if (w.head_dim > 256 || w.head_dim % 8 != 0 || w.num_kv_heads <= 0) return hipErrorInvalidValue;
  const int64_t groups = 1 + (static_cast<int64_t>(w.num_tokens) + kPlanWriteTokens - 1) / kPlanWriteTokens *
                                 w.num_kv_heads;
  if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  switch (src) {
    case DT_F32: return launch_plan_write_kv<DT_F32>(kv, a, w, static_cast<unsigned>(groups), stream);
    case DT_F16: return launch_plan_write_kv<DT_F16>(kv, a, w, static_cast<unsigned>(groups), stream);
    case DT_BF16: return launch_plan_write_kv<DT_BF16>(kv, a, w, static_cast<unsigned>(groups), stream);
  }
  return hipErrorInvalidValue;
}

// Merge of split-context partials.  One workgroup (4 waves) per token and
// group of q heads, or per token and all its heads (in turn) when the step
// has many tokens; tokens whose keys fit one partition were written by the
// attention kernels and leave at once.  Each head takes D/4
// lanes, 4 dims per lane (16-byte loads):
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p
#ifndef PA_REDUCE_MANY_TOKENS
#define PA_REDUCE_MANY_TOKENS 1024
#endif
template <int OT, int D, int PG>
__global__ __launch_bounds__(256) void reduce_kernel(AttnArgs a) {
  constexpr int LPH = D / 4;                             // lanes per head
  constexpr int HPB = 4 * (64 / LPH);                    // heads per workgroup
  const int token = blockIdx.x;
  int lo = 0;
  if (a.num_tokens == a.num_seqs && a.max_query_len == 1) {
    // one query token per sequence (the counts leave no other way): token i
    // is sequence i's, with no search
    lo = token;
  } else {
    // sequence of this token: last i with qsl[i] <= token.  A 64-way search:
    // each round every lane probes one candidate and a ballot keeps the last
    // one at or before the token (qsl is non-decreasing, qsl[lo] <= token).
    const int lane = threadIdx.x & 63;
    int hi = a.num_seqs - 1;
    while (hi > lo) {
      const int step = (hi - lo + 64) / 64;
      const int cand = lo + lane * step;
      const uint64_t ok = __ballot(cand <= hi && a.qsl[cand] <= token);
      lo += (63 - __builtin_clzll(ok)) * step;
      hi = min(hi, lo + step - 1);
    }
  }
  const int i = uniform(lo);
  const int q0 = a.qsl[i];
  const int ql = a.qsl[i + 1] - q0;
  const int L = min(a.seq_lens[i], a.max_seq_len);
  const int row_pos = L - ql + (token - q0);
  const int own = row_pos - a.prefix_len;               // the row's keys past the shared prefix, minus one
  const bool chunk_kind = is_chunk_seq(a, ql * a.group);
  // the row's partials: the prefix pass's, then one per item up to the one
  // holding the row's last key
  int np = a.prefix_len > 0 ? a.prefix_parts : 0;
  if (own >= 0)
    np += chunk_kind ? own / a.chunk_partition + 1
                     : DecodeCut(L - a.prefix_len, a.partition, a.split_f, uniform(a.header[7])).item_of(own) + 1;
  if (np <= 1 && a.prefix_len == 0) return;
  // the token's partial lists (head 0; heads follow at a stride of the list length)
  const int64_t list0 = partial_row(a, chunk_kind, i, token, token - q0, 0);
  if (list0 < 0) return;
  const int list_len = chunk_kind ? a.chunk_parts : a.dec_parts;
  const int nparts = min(np, list_len);   // equal for metadata within the contract
  // head groups blockIdx.y, + gridDim.y, ... (one per workgroup, or all of
  // them in one workgroup when the step has many tokens)
  const int d0 = (threadIdx.x % LPH) * 4;
  const int ngroups = (a.num_q_heads + HPB - 1) / HPB;
  for (int hg = blockIdx.y; hg < ngroups; hg += gridDim.y) {
    const int head = hg * HPB + static_cast<int>(threadIdx.x) / LPH;
    if (head >= a.num_q_heads) break;
    const int64_t row = list0 + static_cast<int64_t>(head) * list_len;
    // One pass over the partials, PG at a time (all their loads issued
    // together): the running max moves to the group's max and what was summed
    // so far is rescaled to it.
    float M = -__builtin_inff();
    float den = 0.f;
    f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < nparts; p0 += PG) {
      float mv[PG], lv[PG];
      f32x4 av[PG];
#pragma unroll
      for (int j = 0; j < PG; ++j) {
        const bool in = p0 + j < nparts;
        mv[j] = in ? a.part_m[row + p0 + j] : -__builtin_inff();
        lv[j] = in ? a.part_l[row + p0 + j] : 0.f;
        av[j] = in ? *reinterpret_cast<const f32x4*>(a.part_acc + (row + p0 + j) * D + d0)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      float Mn = M;
#pragma unroll
      for (int j = 0; j < PG; ++j) Mn = fmaxf(Mn, mv[j]);
      const float r = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      den *= r;
      num *= r;
#pragma unroll
      for (int j = 0; j < PG; ++j) {
        const float wgt = mv[j] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mv[j] - Mn);
        den += wgt * lv[j];
        num += wgt * av[j];
      }
      M = Mn;
    }
    const float inv = 1.f / den;
    uint8_t* op = static_cast<uint8_t*>(a.out) +
                  ((static_cast<int64_t>(token) * a.num_q_heads + head) * D + d0) * Bytes<OT>::v;
    store4<OT>(op, num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv);
  }
}

template <int OT, int D>
static void launch_reduce(const AttnArgs& a, hipStream_t stream) {
  constexpr int HPB = 4 * (64 / (D / 4));
  // a step with many tokens (prompt chunks) has few that need a merge: one
  // workgroup per token then, so that the rest cost one early exit each
  const bool many = a.num_tokens >= PA_REDUCE_MANY_TOKENS;
  const int groups = (a.num_q_heads + HPB - 1) / HPB;
  const dim3 grid(a.num_tokens, many ? 1 : groups);
  // Rows with more than 8 partials (long contexts, a shared prefix's pass)
  // read 32 per round: fewer dependent load rounds.  Steps with many tokens
  // keep 8: the wider group's registers slow their early exits.
  if (!many && (a.dec_parts > 8 || a.chunk_parts > 8))
    hipLaunchKernelGGL((reduce_kernel<OT, D, 32>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((reduce_kernel<OT, D, 8>), grid, dim3(256), 0, stream, a);
}

// plan (with the step's cache write when `write` is given) -> [shared-prefix
// pass] -> decode kernel -> chunk kernel (when a prompt chunk can be present)
// -> partition merge.  ev[0..1] bracket the decode kernel, ev[4..5] the
// shared-prefix pass, ev[2..3] the chunk
// kernel (each may be null).
hipError_t launch_attention(int q, int kv, int d, int bs, const AttnArgs& a, hipStream_t stream,
                            const hipEvent_t* ev, const CacheWriteArgs* write, int write_src) {
  // the pairing and shape must exist before anything is enqueued
  hipError_t e = dispatch_attention(q, kv, d, bs, [](auto, auto, auto, auto) { return hipSuccess; });
  if (e != hipSuccess) return e;
  // a step that can hold prompt chunks: one fused launch where the shape has one
  const bool chunks = q != DT_F32 && a.chunk_path && static_cast<int64_t>(a.max_query_len) * a.group >= kChunkMinRows;
  AttnArgs f = a;                             // what every kernel of this step reads
  const bool fused = PA_FUSED_STEP && chunks && (f.step_groups = static_cast<int32_t>(step_groups(q, kv, d, bs))) > 0;
  f.chunk_partition = fused ? kChunkPartitionFused : kChunkPartition;
  // the tail split serves the decode kernel's own list (in the fused step,
  // chunk items make the tail)
  if (fused) f.split_f = 1;
  if (f.split_f > 1) f.decode_waves = static_cast<int32_t>(decode_waves(q, kv, d, bs));
  if (fused) {
    const double eb = kv == DT_F32 ? 4 : (kv == DT_FP8 ? 1 : 2);
    f.fused = 1;
    f.step_dec_us = static_cast<float>(32.0 * d * 2 * eb / kFusedDecodeBytesPerUs);
    f.step_chunk_us = static_cast<float>(64.0 * a.chunk_rows * d * 4 / kFusedChunkFlopsPerUs);
  }
  if (write && write->num_tokens > 0) {       // the step's cache write in the plan's launch
    if ((e = launch_plan_write(write_src, kv, f, *write, stream)) != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, f);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.prefix_len > 0) {                     // the shared prefix, all rows at once
    AttnArgs p = f;
    p.prefix_pass = 1;
    if (ev[4] && (e = hipEventRecord(ev[4], stream)) != hipSuccess) return e;
    if ((e = launch_chunk(q, kv, d, bs, p, stream)) != hipSuccess) return e;
    if (ev[5] && (e = hipEventRecord(ev[5], stream)) != hipSuccess) return e;
  }
  if (fused) {                                // decode + chunk items in one launch
    if (ev[0] && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
    if (ev[2] && (e = hipEventRecord(ev[2], stream)) != hipSuccess) return e;
    if ((e = launch_step(q, kv, d, bs, f, stream)) != hipSuccess) return e;
    if (ev[1] && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
    if (ev[3] && (e = hipEventRecord(ev[3], stream)) != hipSuccess) return e;
  } else {
    if (ev[0] && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
    if ((e = launch_decode(q, kv, d, bs, f, stream)) != hipSuccess) return e;
    if (ev[1] && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
    if (chunks) {
      if (ev[2] && (e = hipEventRecord(ev[2], stream)) != hipSuccess) return e;
      if ((e = launch_chunk(q, kv, d, bs, f, stream)) != hipSuccess) return e;
      if (ev[3] && (e = hipEventRecord(ev[3], stream)) != hipSuccess) return e;
    }
  }
  if ((a.dec_parts > 1 || a.chunk_parts > 1 || a.prefix_len > 0) && a.num_tokens > 0) {
    if (q == DT_F32) {
      if (d == 64) launch_reduce<DT_F32, 64>(f, stream);
      else launch_reduce<DT_F32, 128>(f, stream);
    } else if (q == DT_F16) {
      if (d == 64) launch_reduce<DT_F16, 64>(f, stream);
      else if (d == 128) launch_reduce<DT_F16, 128>(f, stream);
      else launch_reduce<DT_F16, 256>(f, stream);
    } else {
      if (d == 64) launch_reduce<DT_BF16, 64>(f, stream);
      else if (d == 128) launch_reduce<DT_BF16, 128>(f, stream);
      else launch_reduce<DT_BF16, 256>(f, stream);
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace pa

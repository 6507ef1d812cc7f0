// pa_internal.h -- host-side plumbing shared by the C-ABI layer and the
// kernel launchers.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "pa.h"

namespace pa {

// Debug build (-DPA_DEBUG=1, libpa_debug.so): the plan kernel checks every
// sequence's metadata and the cache write every slot before using them; the
// first violation is recorded in a device word pair (code, index) that
// pa_debug_check reads back, and the offending sequence or token is
// skipped, so no kernel reads or writes outside its buffers.  Release
// builds treat such metadata as undefined behaviour and check nothing.
#ifndef PA_DEBUG
#define PA_DEBUG 0
#endif
enum DebugCode : int32_t {
  kDebugNone = 0,
  kDebugQueryStart = 1,   // query_start_loc does not start at 0, end at num_tokens, or decreases
  kDebugQueryLen = 2,     // q_len > L
  kDebugSeqLen = 3,       // L > max_seq_len (or L < 0)
  kDebugMaxQuery = 4,     // q_len > max_query_len
  kDebugBlockId = 5,      // ceil(L/B) > max_blocks_per_seq, or a used block id outside [0, num_blocks)
  kDebugSlot = 6,         // a cache-write slot >= num_blocks * B
};

// Rows of one attention work item: a 16-row MFMA tile of (query token,
// q head) pairs of one sequence and kv head.
constexpr int kTileRows = 16;

// A decode item's record: sequence, (row tile << 16 | item of the tile's cut),
// and the sequence's context length and query count as the plan read them, so
// that an item's first loads need not wait for the sequence's metadata.
constexpr int kDecodeItemWords = 4;

// Workspace header words: [0]/[1] decode work counter and item count,
// [2]/[3] the chunk list's, [4] the shared-prefix pass's counter, [6] the
// fused launch's decode workgroups, [7] the tail split's partitions per row
// tile, [kShareWord] 1 when two decode-routed sequences start in the same
// block (looked for in steps without a declared prefix), [kXcdCounters ..
// +7] the decode kernel's per-XCD class counters.
constexpr int kShareWord = 8;
constexpr int kXcdCounters = 16;
// The plan's hash set of first blocks (LDS): 2^kShareBits slots; steps of
// fewer than kShareMinSeqs sequences are not looked at (too small for the
// L2 to matter, and the look costs the plan about half a microsecond).
constexpr int kShareBits = 11;
constexpr int kShareSlots = 1 << kShareBits;
constexpr int kShareMinSeqs = 8;

// Keys of one context partition handled by one decode work item.  A row
// whose keys span more than one partition gets partial (max, sum, acc)
// results that a log-sum-exp reduce merges.  Longer partitions mean fewer
// items (each pays a start-up latency before its first loads land) and
// fewer partials; shorter ones spread few long contexts over more waves.
// So: with at least kManyPairs (sequence, kv head) pairs -- one per decode
// wave the chip holds at one wave per SIMD (256 CUs x 4 SIMDs) -- whole
// contexts already keep every wave busy and partitions are as long as they
// go (kPartitionMax); with fewer pairs, steps whose longest context reaches
// kLongContext use kPartitionLong, shorter ones kPartitionShort.  (Shorter
// partitions for few, short contexts, to give every wave an item, measured
// slower: each item pays its start-up latency.)  Measured on MI355X: fp8
// decode of 128 sequences x 8 kv heads at 8.1k-8.5k keys runs 357 us with
// 2048-key partitions against 390 us with 1024; 64 x 8 pairs at 1k-32k keys
// run best at 1024 (bf16 405 us, fp8 221 us; 2048: fp8 230 us; 512: fp8 246 us).
// A partition holds at most 128 blocks (two block ids per lane of a wave)
// and at most kPartitionMax keys (64 steps of 32 keys).
#ifndef PA_PARTITION_SHORT
#define PA_PARTITION_SHORT 512
#endif
#ifndef PA_PARTITION_LONG
#define PA_PARTITION_LONG 1024
#endif
#ifndef PA_MANY_PAIRS
#define PA_MANY_PAIRS 1024
#endif
constexpr int kPartitionShort = PA_PARTITION_SHORT;
constexpr int kPartitionLong = PA_PARTITION_LONG;
constexpr int kPartitionMax = 2048;
static_assert(kPartitionShort % 32 == 0 && kPartitionLong % 32 == 0, "partitions hold whole 32-key steps");
static_assert(kPartitionShort <= kPartitionMax && kPartitionLong <= kPartitionMax, "at most 2048 keys");
#ifndef PA_LONG_CONTEXT
#define PA_LONG_CONTEXT 8192
#endif
constexpr int64_t kLongContext = PA_LONG_CONTEXT;
constexpr int64_t kManyPairs = PA_MANY_PAIRS;
// Contexts of 64k keys and more take the longest partitions whatever the
// pair count: each (sequence, kv head) still has 32 or more of them, and
// their partials -- a row's workspace share -- halve.
constexpr int64_t kVeryLongContext = 65536;
inline int decode_partition(int64_t max_seq_len, int64_t num_seqs, int64_t num_kv_heads) {
  if (num_seqs * num_kv_heads >= kManyPairs || max_seq_len >= kVeryLongContext) return kPartitionMax;
  return max_seq_len >= kLongContext ? kPartitionLong : kPartitionShort;
}

// Tail split of the decode list.  Waves take items longest first, so the
// step ends within about one item of the last wave's share; with few, large
// items per wave that imbalance is a large part of the step (at head dim
// 256, 2.5 items of 1 MB per wave, the last waves ran alone for the final
// 25 % of a 437 us kernel).  So when there are fewer (sequence, kv head)
// pairs than decode waves, partitions hold at least kSplitPartBytes of K and
// V, and there are fewer than kSplitItemsPerWave of them per wave, each row
// tile's last S partitions are cut into fine items; sorted longest first,
// those end the list and even the waves out.  Each item costs its wave a
// start-up (a chain of dependent loads that queue behind the step's KV
// stream), so fine items hold at least kSplitBytes (256 keys at head dim
// 256), and the plan kernel sizes the fine work to kSplitRounds partitions
// per decode wave (at most kSplitItems fine items per row tile).  Measured
// on 1k-32k contexts with 1024-key partitions: head dim 256 kernel 435 ->
// 408 us (bf16), 226 -> 215 us (fp8); slower where items are smaller or more
// numerous (fp8 at head dim 128, 256 KB partitions: 216 -> 228 us; bf16 at
// 128, five partitions per wave: 1-2 %), so the split stays off there.  The
// partial slots of a row tile are its items in key order.  Steps that can
// hold prompt chunks keep whole partitions: there the chunk items end the
// step.
#ifndef PA_SPLIT_ROUNDS
#define PA_SPLIT_ROUNDS 0.5
#endif
#ifndef PA_SPLIT_BYTES
#define PA_SPLIT_BYTES (128 << 10)
#endif
#ifndef PA_SPLIT_PART_BYTES
#define PA_SPLIT_PART_BYTES (512 << 10)
#endif
#ifndef PA_SPLIT_ITEMS_PER_WAVE
#define PA_SPLIT_ITEMS_PER_WAVE 4
#endif
constexpr int kSplitMinKeys = 256;
constexpr int64_t kSplitBytes = PA_SPLIT_BYTES;
constexpr int64_t kSplitPartBytes = PA_SPLIT_PART_BYTES;
constexpr int kSplitItems = 32;
constexpr float kSplitRounds = PA_SPLIT_ROUNDS;
constexpr int kSplitItemsPerWave = PA_SPLIT_ITEMS_PER_WAVE;
// Fine items per split partition (1: no split), for head_dim and KV
// elements of kv_bytes bytes.
inline int split_factor(int64_t partition, int64_t num_seqs, int64_t num_kv_heads, bool chunks,
                        int64_t head_dim, int64_t kv_bytes) {
  const int64_t key_bytes = head_dim * 2 * kv_bytes;   // K and V of one key
  if (!(kSplitRounds > 0.f) || chunks || num_seqs * num_kv_heads >= kManyPairs ||
      partition * key_bytes < kSplitPartBytes)
    return 1;
  int64_t fine = kSplitMinKeys;                          // keys per fine item: a power of two
  while (fine < partition && fine * key_bytes < kSplitBytes) fine *= 2;
  return fine < partition ? static_cast<int>(partition / fine) : 1;
}

// The decode items of one row tile of a sequence with `own` keys past the
// shared prefix: partitions of P keys, except that the last S of them (from
// partition ps on) are cut into items of P / F keys.  Item j < ps covers keys
// [j P, j P + P), item j >= ps covers [ps P + (j - ps) P/F, + P/F); item j
// writes partial slot j, so a row's slots are its items in key order.  The
// plan, the decode kernel and the merge all derive the cut from (own, P, F, S).
struct DecodeCut {
  int P, Pf, ps, n;   // n: the tile's items
  __host__ __device__ __forceinline__ DecodeCut(int own, int partition, int F, int S) {
    P = partition;
    Pf = partition / F;
    const int npc = own > 0 ? (own + P - 1) / P : 0;
    ps = F > 1 ? (npc > S ? npc - S : 0) : npc;
    const int rest = own - ps * P;   // keys of the split partitions
    n = ps + (rest > 0 ? (rest + Pf - 1) / Pf : 0);
  }
  __host__ __device__ __forceinline__ int start(int j) const { return j < ps ? j * P : ps * P + (j - ps) * Pf; }
  __host__ __device__ __forceinline__ int len(int j) const { return j < ps ? P : Pf; }
  // the item holding key k (k >= 0)
  __host__ __device__ __forceinline__ int item_of(int k) const { return k < ps * P ? k / P : ps + (k - ps * P) / Pf; }
};

inline int64_t kv_elem_bytes(int32_t kv_dtype) {
  return kv_dtype == PA_F32 ? 4 : (kv_dtype == PA_FP8_E4M3 ? 1 : 2);
}

// A sequence with more than kChunkMinRows - 1 (token, head) rows per kv head
// (a prompt chunk) goes to the chunk kernel: 256-row blocks, 64-key LDS
// tiles, context partitions of kChunkPartition keys.  Fewer rows (decode,
// short speculative runs) stay on the 16-row decode kernel.
constexpr int kChunkMinRows = 65;
#ifndef PA_CHUNK_WAVES
#define PA_CHUNK_WAVES 8
#endif
#ifndef PA_CHUNK_ROW_TILES
#define PA_CHUNK_ROW_TILES 2
#endif
#ifndef PA_CHUNK_WAVES_PER_SIMD
#define PA_CHUNK_WAVES_PER_SIMD 2
#endif
constexpr int kChunkWaves = PA_CHUNK_WAVES;    // waves per chunk workgroup
constexpr int kChunkThreads = 64 * kChunkWaves;
constexpr int kChunkRowTiles = PA_CHUNK_ROW_TILES;          // 16-row tiles per wave (head dim <= 128)
constexpr int kChunkWavesPerSimd = PA_CHUNK_WAVES_PER_SIMD; // register budget: 512 / this per wave
constexpr int kChunkRows = 16 * kChunkRowTiles * kChunkWaves;
// Rows of one chunk work item: 256 (two 16-row tiles per wave), or half that
// for head dim 256, whose accumulators leave room for half the row tiles.
constexpr int chunk_rows_for(int64_t head_dim) {
  return head_dim == 256 ? 16 * (kChunkRowTiles / 2) * kChunkWaves : kChunkRows;
}
constexpr int kChunkKeys = 64;
#ifndef PA_CHUNK_PARTITION
#define PA_CHUNK_PARTITION 8192
#endif
#ifndef PA_CHUNK_PARTITION_FUSED
#define PA_CHUNK_PARTITION_FUSED 16384
#endif
// Keys per chunk-item partition: kChunkPartition when the chunk kernel runs
// alone, kChunkPartitionFused in the fused step, whose decode items fill in
// behind the longer chunk items.  Workspace bounds use the shorter one.
constexpr int kChunkPartition = PA_CHUNK_PARTITION;
constexpr int kChunkPartitionFused = PA_CHUNK_PARTITION_FUSED;
constexpr int kChunkPartitionMax = kChunkPartition > kChunkPartitionFused ? kChunkPartition : kChunkPartitionFused;
static_assert(kChunkPartition <= kChunkPartitionFused, "workspace bounds assume the shorter partition apart");

// Rescale threshold (log2 units): the running reference max of a row moves
// only when a new score exceeds it by more than this, so the accumulator
// rescale is skipped for most tiles; probabilities stay below 2^8.
constexpr float kRescaleSlack = 8.f;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Fused step: a step with prompt chunks (head dim <= 128, 16-bit queries)
// runs its decode and chunk work in one launch of one 8-wave workgroup per
// CU, split between the two by the plan kernel so that the HBM-bound decode
// items and the MFMA-bound chunk items run side by side.  The split is sized
// with throughputs measured on MI355X (256 CUs): decode streams about
// 5.5 TB/s once it holds 60 % of the CUs, proportionally less on fewer (128
// CUs: 85 % of the full rate); the chunk loop retires about 0.8 PFLOP/s of
// algorithmic work on the whole chip, in proportion to its CUs.  Chunk
// workgroups that run out of chunk items go on to decode items.
#ifndef PA_FUSED_STEP
#define PA_FUSED_STEP 1
#endif
constexpr double kFusedDecodeBytesPerUs = 5.5e6;
constexpr double kFusedChunkFlopsPerUs = 0.8e9;
constexpr float kFusedDecodeSaturation = 0.6f;

// Upper bound on the number of (sequence, row tile, partition) work items,
// from host-side bounds only: sum_i ceil(q_i*G/rows) <= ceil(T*G/rows) + S.
inline int64_t max_work_items(int64_t num_seqs, int64_t num_tokens, int64_t group,
                              int64_t max_seq_len, int64_t rows_per_item, int64_t partition) {
  const int64_t tiles = ceil_div(num_tokens * group, rows_per_item) + num_seqs;
  const int64_t parts = ceil_div(max_seq_len > 0 ? max_seq_len : 1, partition);
  return tiles * parts;
}

// Workspace carve-up (byte offsets, each 256-byte aligned).
struct WorkspaceLayout {
  size_t header;   // int32 [64]: [0]/[1] decode work counter/count, [2]/[3] chunk's, [4] prefix pass's; [6] fused decode workgroups, [7] split partitions per row tile
  size_t items;    // int32x4 [max_items]: decode items (seq, tile << 16 | partition with unsigned halves, L, q_len)
  size_t citems;   // int32x2 [max_citems]: chunk items (seq, row block << 16 | partition)
  size_t part_m;   // float [rows]: running max (log2 units) per partition
  size_t part_l;   // float [rows]: softmax denominator per partition
  size_t part_acc; // float [rows][d]: un-normalised output per partition
  size_t total;
  int64_t max_items;
  int64_t max_citems;
  // Partial rows.  A (token, q head) row owns dec_parts consecutive partial
  // rows if its sequence is decode-routed (one per decode item of its row
  // tile, the tail split's fine items included), chunk_parts if chunk-routed.
  // Decode rows sit at slot (i * dec_per_seq + local token) when dec_per_seq
  // > 0, at the token index otherwise; chunk rows at chunk_row_base + their
  // token index.  Two layouts, the smaller is used: one token-indexed list
  // for both kinds (dec_parts = chunk_parts, chunk_row_base 0), or the split
  // one, where decode rows need slots for at most S * floor(64 / G) tokens
  // (a decode-routed sequence has q_len * G < kChunkMinRows) and only chunk
  // rows pay for long contexts at the chunk partition length.
  int64_t part_rows;
  int64_t chunk_row_base;
  int32_t dec_parts;
  int32_t chunk_parts;   // 0: the step has no chunk rows (the hints rule them out)
  int32_t dec_per_seq;
  int32_t partition;     // decode partition length in keys
  int32_t split_f;       // fine items per split partition (1: no tail split)
  int32_t split_max;     // most partitions a row tile has split (0 without the split)
  int32_t prefix_parts;  // partials of the shared-prefix pass (first in each row's list)
  int32_t prefix_part;   // keys per shared-prefix partition
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Shared-prefix (cascade) pass: keys per prefix partition.  The pass has
// (row blocks x partitions x kv heads) items of one workgroup each; they are
// sized to fill one round of kPrefixItems workgroups (one per CU of the
// GPU) without spilling a few into a second round: as many partitions as
// fit that round, each at least 256 keys, rounded up to whole 64-key tiles
// and at most 8192 keys.
#ifndef PA_PREFIX_ITEMS
#define PA_PREFIX_ITEMS 256
#endif
constexpr int64_t kPrefixItems = PA_PREFIX_ITEMS;
inline int32_t prefix_partition(int64_t prefix_len, int64_t num_tokens, int64_t group, int64_t num_kv_heads,
                                int64_t chunk_rows) {
  // (row blocks x kv heads; at least 1, so that an empty step sizes too)
  const int64_t units = std::max<int64_t>(1, ceil_div(num_tokens * group, chunk_rows) * num_kv_heads);
  int64_t parts = kPrefixItems / units > 1 ? kPrefixItems / units : 1;
  const int64_t most = ceil_div(prefix_len, 256);
  parts = parts < most ? parts : most;
  int64_t p = ceil_div(ceil_div(prefix_len, parts), kChunkKeys) * kChunkKeys;
  return static_cast<int32_t>(p < 256 ? 256 : (p > kChunkPartition ? kChunkPartition : p));
}

// chunk_path: 16-bit queries (fp32 queries stay on the decode kernel);
// max_query_len decides whether prompt chunks can occur at all.
inline WorkspaceLayout workspace_layout(int64_t num_seqs, int64_t num_tokens, int64_t num_q_heads,
                                        int64_t num_kv_heads, int64_t head_dim, int64_t max_seq_len,
                                        int64_t max_query_len, bool chunk_path, int64_t kv_bytes,
                                        int64_t prefix_len = 0) {
  WorkspaceLayout w{};
  const int64_t group = num_kv_heads > 0 ? num_q_heads / num_kv_heads : 1;
  // keys past the shared prefix: what the decode and chunk kernels cover
  const int64_t own = max_seq_len - prefix_len > 0 ? max_seq_len - prefix_len : 1;
  w.partition = decode_partition(own, num_seqs, num_kv_heads);
  const bool chunks = chunk_path && max_query_len * group >= kChunkMinRows;
  w.split_f = split_factor(w.partition, num_seqs, num_kv_heads, chunks, head_dim, kv_bytes);
  w.split_max = w.split_f > 1 ? kSplitItems / w.split_f : 0;
  // items (and partial slots) per decode row tile: its partitions, plus
  // split_f - 1 more for each split one
  const int64_t dec_items_per_tile = ceil_div(own, w.partition) + static_cast<int64_t>(w.split_max) * (w.split_f - 1);
  w.max_items = (ceil_div(num_tokens * group, kTileRows) + num_seqs) * dec_items_per_tile;
  w.max_citems = max_work_items(num_seqs, num_tokens, group, own, chunk_rows_for(head_dim), kChunkPartition);
  w.prefix_parts = 0;
  w.prefix_part = 0;
  if (prefix_len > 0) {
    w.prefix_part = prefix_partition(prefix_len, num_tokens, group, num_kv_heads, chunk_rows_for(head_dim));
    w.prefix_parts = static_cast<int32_t>(ceil_div(prefix_len, w.prefix_part));
  }
  const int64_t dparts = w.prefix_parts + dec_items_per_tile;
  const int64_t cparts = chunks ? w.prefix_parts + ceil_div(own, kChunkPartition) : 0;
  // one token-indexed list for both kinds ...
  const int64_t mp = dparts > cparts ? dparts : cparts;
  const double rows_shared = static_cast<double>(num_tokens) * num_q_heads * mp;
  // ... or decode rows by (sequence, local token), chunk rows by token
  const int64_t dq = chunk_path ? (kChunkMinRows - 1) / group : 0;
  const double dtok = static_cast<double>(dq) * num_seqs;
  const double rows_split = dtok * num_q_heads * dparts + (chunks ? static_cast<double>(num_tokens) * num_q_heads * cparts : 0.0);
  // (dq >= 1: dec_per_seq = 0 means token slots, so a split layout needs one
  // decode slot per sequence at least)
  const bool split = chunk_path && dq >= 1 && dtok < num_tokens && rows_split < rows_shared;
  const double rows_d = split ? rows_split : rows_shared;
  if (rows_d > 4.0e15) {             // beyond any device (the caller's check refuses it): no layout
    w.part_rows = -1;
    w.total = ~size_t(0);
    return w;
  }
  if (split) {
    w.dec_per_seq = static_cast<int32_t>(dq);
    w.dec_parts = static_cast<int32_t>(dparts);
    w.chunk_parts = static_cast<int32_t>(cparts);
    w.chunk_row_base = dq * num_seqs * num_q_heads * dparts;
  } else {
    w.dec_per_seq = 0;
    w.dec_parts = w.chunk_parts = static_cast<int32_t>(mp);
    w.chunk_row_base = 0;
  }
  w.part_rows = static_cast<int64_t>(rows_d);
  const size_t rows = static_cast<size_t>(w.part_rows);
  size_t off = 0;
  w.header = off;   off = align256(off + 64 * sizeof(int32_t));
  w.items = off;    off = align256(off + static_cast<size_t>(w.max_items) * kDecodeItemWords * sizeof(int32_t));
  w.citems = off;   off = align256(off + static_cast<size_t>(w.max_citems) * 2 * sizeof(int32_t));
  w.part_m = off;   off = align256(off + rows * sizeof(float));
  w.part_l = off;   off = align256(off + rows * sizeof(float));
  w.part_acc = off; off = align256(off + rows * head_dim * sizeof(float));
  w.total = off;
  return w;
}

struct CacheWriteArgs {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int64_t* slots;
  int32_t num_tokens, num_kv_heads, head_dim, block_size;
  int64_t num_slots;   // num_blocks * block_size (the debug build checks slots against it)
  int32_t* debug;      // debug build: the device's debug words (null in release builds)
  float k_scale, v_scale;
};

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* qsl;
  void* out;
  int32_t* header;
  int32_t* items;
  int32_t* citems;
  float* part_m;
  float* part_l;
  float* part_acc;
  int64_t max_items;
  int64_t max_citems;
  int32_t chunk_path;   // 1: sequences with >= kChunkMinRows rows use the chunk kernel
  int32_t max_blocks_per_seq;
  int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, group;
  int32_t max_query_len;
  // Host bound on the context lengths.  Every kernel reads a context
  // length as min(seq_lens[i], max_seq_len): a sequence past the bound gets
  // rows computed over its first max_seq_len keys -- wrong, but every
  // block-table, pool, partial and item access stays inside the buffers the
  // bound sized.
  int32_t max_seq_len;
  int32_t num_blocks;   // pool size N (the debug build checks block ids against it)
  int32_t block_size;
  int32_t* debug;       // debug build: the device's debug words (null in release builds)
  // partial rows (WorkspaceLayout): decode rows' and chunk rows' counts,
  // decode slots per sequence (0: by token), first chunk row
  int32_t dec_parts, chunk_parts, dec_per_seq;
  int64_t chunk_row_base;
  int32_t partition;   // decode partition length in keys (decode_partition)
  // Tail split (split_factor): fine items per split partition (1: none), the
  // most partitions per row tile the plan may split, and the decode waves
  // the plan sizes the fine work for.  The plan's choice of S is header[7].
  int32_t split_f, split_max, decode_waves;
  // Shared prefix (cascade): every sequence's first prefix_len keys are the
  // same blocks (sequence 0's table row is read for them) and every query row
  // sits at or past prefix_len.  The prefix pass attends all rows to those
  // keys (partials 0 .. prefix_parts-1); the decode and chunk kernels then
  // cover keys from prefix_len on (partials from prefix_parts on).
  int32_t prefix_len;
  int32_t prefix_part, prefix_parts, prefix_rblocks;
  int32_t prefix_pass;       // 1: this chunk-kernel launch is the prefix pass
  int32_t chunk_rows;        // rows of one chunk item: chunk_rows_for(head dim)
  int32_t chunk_partition;   // keys per chunk-item partition (kChunkPartition or kChunkPartitionFused)
  int64_t prefix_items;
  float score_scale;   // scale * k_scale * log2(e)
  float rescale_slack; // kRescaleSlack / score_scale (raw-score units)
  float v_scale;
  // Fused step (decode and chunk work in one launch): the plan kernel splits
  // the step kernel's step_groups workgroups (one per CU) into decode and
  // chunk roles, header[6] = workgroups that start on decode items.
  int32_t fused;
  int32_t step_groups;
  float step_dec_us;     // whole-chip time of one 32-key decode step of one kv head, us
  float step_chunk_us;   // whole-chip time of one 64-key chunk tile of one kv head, us
};

// Workgroups of `threads` threads of `kernel` that fit on the device at once.
inline int64_t resident_groups(const void* kernel, int threads) {
  int dev = 0, per_cu = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu <= 0)
    return 512;
  return static_cast<int64_t>(per_cu) * prop.multiProcessorCount;
}

struct BlockCopyArgs {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const int64_t* mapping;   // [num_pairs][2]: (src block, dst block)
  int64_t block_bytes;      // Hkv * B * d * eb: one block of K (or of V)
  int64_t src_blocks, dst_blocks;
  int32_t num_pairs;
};

struct TableWriteArgs {
  int32_t* table;           // [max_reqs][max_blocks]
  const int32_t* rows;      // [num_writes]
  const int32_t* starts;    // [num_writes]
  const int32_t* offsets;   // [num_writes + 1]: write k's values are values[offsets[k] .. offsets[k+1])
  const int32_t* values;    // [num_values]
  int32_t max_reqs, max_blocks, num_writes;
  int64_t num_values;
};

struct StepArgs {
  const int32_t* table;          // [max_reqs][max_blocks], by persistent slot
  const int32_t* idx_mapping;    // [num_reqs]: persistent slot of batch position b
  const int32_t* num_computed;   // [max_reqs]: tokens already in the cache, by slot
  const int32_t* num_scheduled;  // [num_reqs]: query tokens this step, by batch position
  int32_t* qsl;                  // [num_reqs + 1]
  int32_t* seq_lens;             // [num_reqs]
  int64_t* positions;            // [num_tokens]
  int64_t* slot_mapping;         // [num_tokens]
  int32_t* step_tables;          // [num_reqs][max_blocks]
  int32_t max_reqs, max_blocks, num_reqs, num_tokens, block_size;
};

struct CommitArgs {
  int32_t* num_computed;         // [max_reqs], by persistent slot
  const int32_t* idx_mapping;    // [num_reqs]
  const int32_t* num_scheduled;  // [num_reqs]
  int32_t max_reqs, num_reqs;
};

// The body of pa_attention / pa_attention_shared_prefix (a pa_status_t):
// validates, lays out the workspace and launches.  With `required` non-null
// it only writes the workspace bytes the step needs there (after the same
// validation) and launches nothing.  `write` (may be null; checked by the
// caller): the step's cache write of new tokens (source dtype write_src),
// launched beside the work-list build -- or alone when the step has no
// attention rows.  (pa_api.hip)
int attention_entry(const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                    const pa_cache_t* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                    int32_t num_tokens, int32_t num_q_heads, int32_t max_seq_len,
                    int32_t max_query_len, int32_t prefix_len, float scale, void* out,
                    void* workspace, size_t workspace_bytes, void* stream, size_t* required,
                    const CacheWriteArgs* write = nullptr, int32_t write_src = 0);

// Launchers.  Each returns hipSuccess or the launch error.

hipError_t launch_reshape_and_cache(int src_dtype, int kv_dtype, const CacheWriteArgs& a,
                                    hipStream_t stream);   // (pa_cache_write.hip)
// Debug build: the current device's debug words (a static device pair,
// looked up once per device; null in release builds or if the lookup
// fails), and a synchronous read-and-clear of them after the stream has
// drained.  (pa_cache_write.hip)
int32_t* debug_words();
hipError_t read_debug_words(int32_t* code, int32_t* index, hipStream_t stream);
hipError_t launch_copy_blocks(const BlockCopyArgs& a, hipStream_t stream);   // (pa_blocks.hip)
hipError_t launch_table_writes(const TableWriteArgs& a, hipStream_t stream);  // (pa_metadata.hip)
hipError_t launch_prepare_step(const StepArgs& a, hipStream_t stream);        // (pa_metadata.hip)
hipError_t launch_commit_step(const CommitArgs& a, hipStream_t stream);       // (pa_metadata.hip)
// kv_dtype, q_dtype: pa_dtype_t values; head_dim 64|128; block_size 16|32|64.
// events[0..1] (may be null) are recorded around the decode kernel,
// events[2..3] around the chunk kernel and events[4..5] around the
// shared-prefix pass.  (pa_attention.hip)
// write (may be null): the step's cache write (source dtype write_src),
// launched beside the work-list build instead of on its own.
hipError_t launch_attention(int q_dtype, int kv_dtype, int head_dim, int block_size,
                            const AttnArgs& a, hipStream_t stream, const hipEvent_t* events,
                            const CacheWriteArgs* write = nullptr, int write_src = 0);
// The decode kernel alone (pa_decode.hip) and the chunk kernel alone
// (pa_chunk.hip; 16-bit q only); both draw items from the plan's lists.
hipError_t launch_decode(int q_dtype, int kv_dtype, int head_dim, int block_size, const AttnArgs& a,
                         hipStream_t stream);
// The decode kernel's grid: one wave per resident slot (pa_decode.hip).
int64_t decode_waves(int q_dtype, int kv_dtype, int head_dim, int block_size);
hipError_t launch_chunk(int q_dtype, int kv_dtype, int head_dim, int block_size, const AttnArgs& a,
                        hipStream_t stream);
// The fused step kernel (pa_step.hip): its grid (one workgroup per CU, 0 if
// the shape has no fused form: f32 q or head dim 256) and its launch.
int64_t step_groups(int q_dtype, int kv_dtype, int head_dim, int block_size);
hipError_t launch_step(int q_dtype, int kv_dtype, int head_dim, int block_size, const AttnArgs& a,
                       hipStream_t stream);

}  // namespace pa

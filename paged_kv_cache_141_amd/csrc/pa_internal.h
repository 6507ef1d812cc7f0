// pa_internal.h -- host-side plumbing shared by the C-ABI layer and the
// kernel launchers.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Rows of one attention work item: a 16-row MFMA tile of (query token,
// q head) pairs of one sequence and kv head.
constexpr int kTileRows = 16;

// Keys of one context partition handled by one work item.  A row whose keys
// span more than one partition gets partial (max, sum, acc) results that a
// log-sum-exp reduce merges.
constexpr int kPartition = 512;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Upper bound on the number of (sequence, row tile, partition) work items,
// from host-side bounds only: sum_i ceil(q_i*G/16) <= ceil(T*G/16) + S.
inline int64_t max_work_items(int64_t num_seqs, int64_t num_tokens, int64_t group,
                              int64_t max_seq_len) {
  const int64_t tiles = ceil_div(num_tokens * group, kTileRows) + num_seqs;
  const int64_t parts = ceil_div(max_seq_len > 0 ? max_seq_len : 1, kPartition);
  return tiles * parts;
}

// Workspace carve-up (byte offsets, each 256-byte aligned).
struct WorkspaceLayout {
  size_t header;   // int32 [64]: [0] work counter, [1] item count
  size_t items;    // int32x2 [max_items]: (seq, tile << 16 | partition)
  size_t part_m;   // float [T][Hq][MP]: running max (log2 units) per partition
  size_t part_l;   // float [T][Hq][MP]: softmax denominator per partition
  size_t part_acc; // float [T][Hq][MP][d]: un-normalised output per partition
  size_t total;
  int64_t max_items;
  int32_t max_parts;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WorkspaceLayout workspace_layout(int64_t num_seqs, int64_t num_tokens, int64_t num_q_heads,
                                        int64_t num_kv_heads, int64_t head_dim,
                                        int64_t max_seq_len) {
  WorkspaceLayout w{};
  const int64_t group = num_kv_heads > 0 ? num_q_heads / num_kv_heads : 1;
  w.max_items = max_work_items(num_seqs, num_tokens, group, max_seq_len);
  w.max_parts = static_cast<int32_t>(ceil_div(max_seq_len > 0 ? max_seq_len : 1, kPartition));
  const size_t rows = static_cast<size_t>(num_tokens) * num_q_heads * w.max_parts;
  size_t off = 0;
  w.header = off;   off = align256(off + 64 * sizeof(int32_t));
  w.items = off;    off = align256(off + static_cast<size_t>(w.max_items) * 2 * sizeof(int32_t));
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
  float* part_m;
  float* part_l;
  float* part_acc;
  int64_t max_items;
  int32_t max_blocks_per_seq;
  int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, group;
  int32_t max_parts;
  float score_scale;   // scale * k_scale * log2(e)
  float v_scale;
};

// Launchers (defined in pa_kernels.hip).  Return hipSuccess or the launch error.
hipError_t launch_reshape_and_cache(int src_dtype, int kv_dtype, const CacheWriteArgs& a,
                                    hipStream_t stream);
// kv_dtype, q_dtype: pa_dtype_t values; head_dim 64|128; block_size 16|32|64.
// `before`/`after` (may be null) are recorded around the attention kernel.
hipError_t launch_attention(int q_dtype, int kv_dtype, int head_dim, int block_size,
                            const AttnArgs& a, hipStream_t stream, hipEvent_t before,
                            hipEvent_t after);

}  // namespace pa

// pa_api.hip -- the C ABI declared in include/pa.h: argument validation,
// workspace sizing and kernel dispatch.  Allocates nothing; the only state is
// the optional timing-event pair of pa_set_attention_events.
#include <math.h>
#include <string.h>

#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

using pa::ceil_div;

// The measurement hooks of pa_set_attention_events / pa_set_chunk_events /
// pa_set_prefix_events (the library's only state): decode kernel pair, chunk
// kernel pair, shared-prefix pass pair.
hipEvent_t g_events[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};

bool dtype_known(int32_t d) { return d >= PA_F32 && d <= PA_FP8_E4M3; }

pa_status_t check_cache(const pa_cache_t* c) {
  if (!c) return PA_ERR_NULL;
  if (!dtype_known(c->kv_dtype)) return PA_ERR_DTYPE;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0) return PA_ERR_SHAPE;
  if (c->block_size != 16 && c->block_size != 32 && c->block_size != 64) return PA_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return PA_ERR_UNSUPPORTED;
  // one block of all kv heads must stay below 4 GiB (32-bit block strides)
  if (static_cast<int64_t>(c->num_kv_heads) * c->block_size * c->head_dim * 4 >= (int64_t(1) << 32))
    return PA_ERR_UNSUPPORTED;
  if (c->kv_dtype == PA_FP8_E4M3) {
    if (!(c->k_scale > 0.f) || !(c->v_scale > 0.f) || !isfinite(c->k_scale) || !isfinite(c->v_scale))
      return PA_ERR_UNSUPPORTED;
  } else if (c->k_scale != 1.f || c->v_scale != 1.f) {
    return PA_ERR_UNSUPPORTED;
  }
  return PA_OK;
}

// The (q dtype, cache dtype) pairs the attention kernels compute: the MFMA
// operands share one type, fp8 codes widen exactly to the query's type.
bool pairing_ok(int32_t q, int32_t kv) {
  return (q == PA_F32 && kv == PA_F32) || (q == PA_F16 && (kv == PA_F16 || kv == PA_FP8_E4M3)) ||
         (q == PA_BF16 && (kv == PA_BF16 || kv == PA_FP8_E4M3));
}

pa_status_t check_attention_sizes(const pa_cache_t* c, int32_t num_q_heads, int32_t num_seqs,
                                  int32_t num_tokens, int32_t max_seq_len, int32_t max_query_len) {
  pa_status_t st = check_cache(c);
  if (st != PA_OK) return st;
  if (num_q_heads <= 0 || num_seqs < 0 || num_tokens < 0 || max_seq_len < 0 || max_query_len < 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % c->num_kv_heads != 0) return PA_ERR_SHAPE;
  if (max_query_len > max_seq_len) return PA_ERR_SHAPE;
  // every token belongs to a sequence with at most max_query_len of them
  if (static_cast<int64_t>(num_tokens) > static_cast<int64_t>(num_seqs) * max_query_len) return PA_ERR_SHAPE;
  const int64_t group = num_q_heads / c->num_kv_heads;
  // work items pack (tile, partition) into 16 bits each
  if (ceil_div(static_cast<int64_t>(max_query_len) * group, pa::kTileRows) > 0xFFFF) return PA_ERR_UNSUPPORTED;
  const pa::WorkspaceLayout w = pa::workspace_layout(num_seqs, num_tokens, num_q_heads, c->num_kv_heads,
                                                     c->head_dim, max_seq_len, max_query_len,
                                                     c->kv_dtype != PA_F32, pa::kv_elem_bytes(c->kv_dtype));
  if (ceil_div(max_seq_len, w.partition) + static_cast<int64_t>(w.split_max) * (w.split_f - 1) > 0xFFFF)
    return PA_ERR_UNSUPPORTED;
  if (w.max_items > 0x7FFFFFFF / 64 || w.max_citems > 0x7FFFFFFF / 64) return PA_ERR_UNSUPPORTED;
  // the partials' size (the layout computes it without wrap-around): at most 2^48 bytes
  if (w.part_rows < 0 || static_cast<double>(w.part_rows) * (c->head_dim + 2) * 4.0 > 281474976710656.0)
    return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// The address a kernel uses for pool pointer p: device memory of the current
// device as is, page-locked host memory through its device mapping.  False
// for anything else (pageable host memory, another device's memory).
bool kernel_address(const void* p, const void** out) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();   // clear the sticky error of the failed query
    return false;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (attr.type == hipMemoryTypeDevice && attr.device == dev) {
    *out = p;
    return true;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer) {
    *out = attr.devicePointer;
    return true;
  }
  return false;
}

// A shared prefix: whole blocks, no longer than the longest context, and a
// 16-bit query (the prefix pass runs on the chunk kernel).
pa_status_t check_prefix(const pa_cache_t* c, int32_t q_dtype, int32_t max_seq_len, int32_t prefix_len) {
  if (prefix_len == 0) return PA_OK;
  if (prefix_len < 0 || prefix_len % c->block_size != 0 || prefix_len > max_seq_len) return PA_ERR_SHAPE;
  if (q_dtype == PA_F32) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// The cache write's checks and launch arguments (pa_reshape_and_cache and
// pa_write_and_attend).  a.num_tokens == 0 means nothing to write.
pa_status_t cache_write_args(const void* key, const void* value, int32_t src_dtype, void* k_cache, void* v_cache,
                             const pa_cache_t* cache, const int64_t* slot_mapping, int32_t num_tokens,
                             pa::CacheWriteArgs& a) {
  a = pa::CacheWriteArgs{};
  pa_status_t st = check_cache(cache);
  if (st != PA_OK) return st;
  if (src_dtype != PA_F32 && src_dtype != PA_F16 && src_dtype != PA_BF16) return PA_ERR_DTYPE;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  a.key = key;
  a.value = value;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.block_size = cache->block_size;
  a.num_slots = static_cast<int64_t>(cache->num_blocks) * cache->block_size;
  a.debug = PA_DEBUG ? pa::debug_words() : nullptr;
  if (PA_DEBUG && !a.debug) return PA_ERR_HIP;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  return PA_OK;
}

}  // namespace

namespace pa {

int attention_entry(const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                    const pa_cache_t* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                    int32_t num_tokens, int32_t num_q_heads, int32_t max_seq_len,
                    int32_t max_query_len, int32_t prefix_len, float scale, void* out,
                    void* workspace, size_t workspace_bytes, void* stream, size_t* required,
                    const CacheWriteArgs* write, int32_t write_src) {
  if (required) *required = 0;
  pa_status_t st = check_attention_sizes(cache, num_q_heads, num_seqs, num_tokens, max_seq_len, max_query_len);
  if (st != PA_OK) return st;
  if ((st = check_prefix(cache, q_dtype, max_seq_len, prefix_len)) != PA_OK) return st;
  if (!dtype_known(q_dtype)) return PA_ERR_DTYPE;
  if (!pairing_ok(q_dtype, cache->kv_dtype)) return PA_ERR_DTYPE;
  if (!isfinite(scale) || !(scale > 0.f)) return PA_ERR_UNSUPPORTED;
  if (cache->head_dim == 256 && q_dtype == PA_F32) return PA_ERR_UNSUPPORTED;   // 16-bit queries only
  if (num_seqs == 0 || num_tokens == 0) {       // no attention: the cache write alone, if any
    if (!write || write->num_tokens == 0) return PA_OK;
    return pa::launch_reshape_and_cache(write_src, cache->kv_dtype, *write, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? PA_OK
               : PA_ERR_HIP;
  }
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start_loc || !out)
    return PA_ERR_NULL;
  if (max_blocks_per_seq <= 0 || static_cast<int64_t>(max_blocks_per_seq) * cache->block_size <
                                     static_cast<int64_t>(max_seq_len))
    return PA_ERR_SHAPE;
  const pa::WorkspaceLayout w = pa::workspace_layout(num_seqs, num_tokens, num_q_heads, cache->num_kv_heads,
                                                     cache->head_dim, max_seq_len, max_query_len,
                                                     q_dtype != PA_F32, pa::kv_elem_bytes(cache->kv_dtype),
                                                     prefix_len);
  if (required) {   // the caller sizes (or supplies) the workspace once it knows the need
    *required = w.total;
    return PA_OK;
  }
  if (!workspace || workspace_bytes < w.total) return PA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return PA_ERR_WORKSPACE;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  pa::AttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.qsl = query_start_loc;
  a.out = out;
  a.header = reinterpret_cast<int32_t*>(ws + w.header);
  a.items = reinterpret_cast<int32_t*>(ws + w.items);
  a.citems = reinterpret_cast<int32_t*>(ws + w.citems);
  a.part_m = reinterpret_cast<float*>(ws + w.part_m);
  a.part_l = reinterpret_cast<float*>(ws + w.part_l);
  a.part_acc = reinterpret_cast<float*>(ws + w.part_acc);
  a.max_items = w.max_items;
  a.max_citems = w.max_citems;
  a.chunk_path = q_dtype != PA_F32;   // the chunk kernel stages 16-bit operands
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.max_query_len = max_query_len;
  a.max_seq_len = max_seq_len;
  a.num_blocks = cache->num_blocks;
  a.block_size = cache->block_size;
  a.debug = PA_DEBUG ? pa::debug_words() : nullptr;
  if (PA_DEBUG && !a.debug) return PA_ERR_HIP;
  a.num_kv_heads = cache->num_kv_heads;
  a.group = num_q_heads / cache->num_kv_heads;
  a.dec_parts = w.dec_parts;
  a.chunk_parts = w.chunk_parts;
  a.dec_per_seq = w.dec_per_seq;
  a.chunk_row_base = w.chunk_row_base;
  a.partition = w.partition;
  a.split_f = w.split_f;
  a.split_max = w.split_max;
  a.prefix_len = prefix_len;
  a.prefix_part = w.prefix_part;
  a.prefix_parts = w.prefix_parts;
  a.chunk_rows = pa::chunk_rows_for(cache->head_dim);
  a.chunk_partition = pa::kChunkPartition;
  a.prefix_rblocks = static_cast<int32_t>(ceil_div(static_cast<int64_t>(num_tokens) * a.group, a.chunk_rows));
  a.prefix_items = static_cast<int64_t>(a.prefix_rblocks) * w.prefix_parts * cache->num_kv_heads;
  a.score_scale = scale * cache->k_scale * 1.4426950408889634f;
  a.rescale_slack = pa::kRescaleSlack / a.score_scale;
  a.v_scale = cache->v_scale;
  const hipError_t e = pa::launch_attention(q_dtype, cache->kv_dtype, cache->head_dim, cache->block_size, a,
                                            static_cast<hipStream_t>(stream), g_events, write, write_src);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa

extern "C" {

const char* pa_version(void) { return "0.1.0"; }

const char* pa_status_string(pa_status_t s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "inconsistent or invalid sizes";
    case PA_ERR_DTYPE: return "unknown dtype or unsupported dtype pairing";
    case PA_ERR_UNSUPPORTED: return "block size, head dim, scale or size outside the supported path";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_METADATA: return "invalid metadata contents";
    case PA_ERR_TOO_LARGE: return "the step needs more than the static scratch of pa_attention_noalloc";
  }
  return "unknown status";
}

pa_status_t pa_reshape_and_cache(const void* key, const void* value, int32_t src_dtype, void* k_cache,
                                 void* v_cache, const pa_cache_t* cache, const int64_t* slot_mapping,
                                 int32_t num_tokens, void* stream) {
  pa::CacheWriteArgs a;
  const pa_status_t st = cache_write_args(key, value, src_dtype, k_cache, v_cache, cache, slot_mapping, num_tokens, a);
  if (st != PA_OK || a.num_tokens == 0) return st;
  const hipError_t e = pa::launch_reshape_and_cache(src_dtype, cache->kv_dtype, a,
                                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status_t pa_write_and_attend(const void* key, const void* value, int32_t src_dtype, const int64_t* slot_mapping,
                                int32_t num_new_tokens, const void* q, int32_t q_dtype, void* k_cache,
                                void* v_cache, const pa_cache_t* cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                                int32_t num_q_heads, int32_t max_seq_len, int32_t max_query_len,
                                int32_t prefix_len, float scale, void* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  pa::CacheWriteArgs w;
  const pa_status_t st =
      cache_write_args(key, value, src_dtype, k_cache, v_cache, cache, slot_mapping, num_new_tokens, w);
  if (st != PA_OK) return st;
  return static_cast<pa_status_t>(pa::attention_entry(
      q, q_dtype, k_cache, v_cache, cache, block_tables, max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
      num_tokens, num_q_heads, max_seq_len, max_query_len, prefix_len, scale, out, workspace, workspace_bytes,
      stream, nullptr, w.num_tokens > 0 ? &w : nullptr, src_dtype));
}

pa_status_t pa_copy_blocks(const void* src_k, const void* src_v, const pa_cache_t* src_cache, void* dst_k,
                           void* dst_v, const pa_cache_t* dst_cache, const int64_t* block_mapping,
                           int32_t num_pairs, void* stream) {
  pa_status_t st = check_cache(src_cache);
  if (st != PA_OK) return st;
  if ((st = check_cache(dst_cache)) != PA_OK) return st;
  if (src_cache->block_size != dst_cache->block_size || src_cache->num_kv_heads != dst_cache->num_kv_heads ||
      src_cache->head_dim != dst_cache->head_dim || src_cache->kv_dtype != dst_cache->kv_dtype)
    return PA_ERR_SHAPE;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !block_mapping) return PA_ERR_NULL;
  pa::BlockCopyArgs a{};
  const void* p = nullptr;
  if (!kernel_address(src_k, &p)) return PA_ERR_UNSUPPORTED;
  a.src_k = p;
  if (!kernel_address(src_v, &p)) return PA_ERR_UNSUPPORTED;
  a.src_v = p;
  if (!kernel_address(dst_k, &p)) return PA_ERR_UNSUPPORTED;
  a.dst_k = const_cast<void*>(p);
  if (!kernel_address(dst_v, &p)) return PA_ERR_UNSUPPORTED;
  a.dst_v = const_cast<void*>(p);
  if (!kernel_address(block_mapping, &p)) return PA_ERR_UNSUPPORTED;
  a.mapping = static_cast<const int64_t*>(p);
  static const int kEb[] = {4, 2, 2, 1};
  a.block_bytes = static_cast<int64_t>(src_cache->num_kv_heads) * src_cache->block_size * src_cache->head_dim *
                  kEb[src_cache->kv_dtype];
  a.src_blocks = src_cache->num_blocks;
  a.dst_blocks = dst_cache->num_blocks;
  a.num_pairs = num_pairs;
  const hipError_t e = pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status_t pa_apply_block_table_writes(int32_t* block_table, int32_t max_reqs, int32_t max_blocks,
                                        const int32_t* write_rows, const int32_t* write_starts,
                                        const int32_t* write_offsets, const int32_t* write_values,
                                        int32_t num_writes, int32_t num_values, void* stream) {
  if (max_reqs <= 0 || max_blocks <= 0 || num_writes < 0 || num_values < 0) return PA_ERR_SHAPE;
  if (num_writes == 0 || num_values == 0) return PA_OK;
  if (!block_table || !write_rows || !write_starts || !write_offsets || !write_values) return PA_ERR_NULL;
  pa::TableWriteArgs a{};
  const void* p = nullptr;
  if (!kernel_address(block_table, &p)) return PA_ERR_UNSUPPORTED;
  a.table = static_cast<int32_t*>(const_cast<void*>(p));
  if (!kernel_address(write_rows, &p)) return PA_ERR_UNSUPPORTED;
  a.rows = static_cast<const int32_t*>(p);
  if (!kernel_address(write_starts, &p)) return PA_ERR_UNSUPPORTED;
  a.starts = static_cast<const int32_t*>(p);
  if (!kernel_address(write_offsets, &p)) return PA_ERR_UNSUPPORTED;
  a.offsets = static_cast<const int32_t*>(p);
  if (!kernel_address(write_values, &p)) return PA_ERR_UNSUPPORTED;
  a.values = static_cast<const int32_t*>(p);
  a.max_reqs = max_reqs;
  a.max_blocks = max_blocks;
  a.num_writes = num_writes;
  a.num_values = num_values;
  const hipError_t e = pa::launch_table_writes(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status_t pa_prepare_step(const int32_t* block_table, int32_t max_reqs, int32_t max_blocks,
                            const int32_t* idx_mapping, const int32_t* num_computed,
                            const int32_t* num_scheduled, int32_t num_reqs, int32_t num_tokens,
                            int32_t block_size, int32_t* query_start_loc, int32_t* seq_lens,
                            int64_t* positions, int64_t* slot_mapping, int32_t* step_block_tables,
                            void* stream) {
  if (max_reqs <= 0 || max_blocks <= 0 || num_reqs < 0 || num_tokens < 0 || block_size <= 0) return PA_ERR_SHAPE;
  if (num_reqs == 0) return PA_OK;
  if (!block_table || !idx_mapping || !num_computed || !num_scheduled || !query_start_loc || !seq_lens ||
      !step_block_tables || (num_tokens > 0 && (!positions || !slot_mapping)))
    return PA_ERR_NULL;
  pa::StepArgs a{};
  a.table = block_table;
  a.idx_mapping = idx_mapping;
  a.num_computed = num_computed;
  a.num_scheduled = num_scheduled;
  a.qsl = query_start_loc;
  a.seq_lens = seq_lens;
  a.positions = positions;
  a.slot_mapping = slot_mapping;
  a.step_tables = step_block_tables;
  a.max_reqs = max_reqs;
  a.max_blocks = max_blocks;
  a.num_reqs = num_reqs;
  a.num_tokens = num_tokens;
  a.block_size = block_size;
  const hipError_t e = pa::launch_prepare_step(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status_t pa_commit_step(int32_t* num_computed, int32_t max_reqs, const int32_t* idx_mapping,
                           const int32_t* num_scheduled, int32_t num_reqs, void* stream) {
  if (max_reqs <= 0 || num_reqs < 0) return PA_ERR_SHAPE;
  if (num_reqs == 0) return PA_OK;
  if (!num_computed || !idx_mapping || !num_scheduled) return PA_ERR_NULL;
  pa::CommitArgs a{};
  a.num_computed = num_computed;
  a.idx_mapping = idx_mapping;
  a.num_scheduled = num_scheduled;
  a.max_reqs = max_reqs;
  a.num_reqs = num_reqs;
  const hipError_t e = pa::launch_commit_step(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status_t pa_attention_workspace_size(const pa_cache_t* cache, int32_t num_q_heads, int32_t num_seqs,
                                        int32_t num_tokens, int32_t max_seq_len, int32_t max_query_len,
                                        size_t* bytes) {
  if (!bytes) return PA_ERR_NULL;
  pa_status_t st = check_attention_sizes(cache, num_q_heads, num_seqs, num_tokens, max_seq_len, max_query_len);
  if (st != PA_OK) return st;
  *bytes = pa::workspace_layout(num_seqs, num_tokens, num_q_heads, cache->num_kv_heads, cache->head_dim,
                                max_seq_len, max_query_len, cache->kv_dtype != PA_F32,
                                pa::kv_elem_bytes(cache->kv_dtype))
               .total;
  return PA_OK;
}

pa_status_t pa_attention_shared_prefix_workspace_size(const pa_cache_t* cache, int32_t num_q_heads,
                                                      int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len,
                                                      int32_t max_query_len, int32_t prefix_len, size_t* bytes) {
  if (!bytes) return PA_ERR_NULL;
  pa_status_t st = check_attention_sizes(cache, num_q_heads, num_seqs, num_tokens, max_seq_len, max_query_len);
  if (st != PA_OK) return st;
  if (prefix_len < 0 || (cache && prefix_len % cache->block_size != 0) || prefix_len > max_seq_len) return PA_ERR_SHAPE;
  *bytes = pa::workspace_layout(num_seqs, num_tokens, num_q_heads, cache->num_kv_heads, cache->head_dim,
                                max_seq_len, max_query_len, cache->kv_dtype != PA_F32,
                                pa::kv_elem_bytes(cache->kv_dtype), prefix_len)
               .total;
  return PA_OK;
}

pa_status_t pa_attention(const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                         const pa_cache_t* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                         int32_t num_tokens, int32_t num_q_heads, int32_t max_seq_len,
                         int32_t max_query_len, float scale, void* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return static_cast<pa_status_t>(pa::attention_entry(q, q_dtype, k_cache, v_cache, cache, block_tables,
                                                      max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                                                      num_tokens, num_q_heads, max_seq_len, max_query_len, 0, scale,
                                                      out, workspace, workspace_bytes, stream, nullptr));
}

pa_status_t pa_attention_shared_prefix(const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                                       const pa_cache_t* cache, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                       const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                                       int32_t num_q_heads, int32_t max_seq_len, int32_t max_query_len,
                                       int32_t prefix_len, float scale, void* out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return static_cast<pa_status_t>(pa::attention_entry(q, q_dtype, k_cache, v_cache, cache, block_tables,
                                                      max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                                                      num_tokens, num_q_heads, max_seq_len, max_query_len,
                                                      prefix_len, scale, out, workspace, workspace_bytes, stream,
                                                      nullptr));
}

pa_status_t pa_preferred_block_size(int32_t head_dim, int32_t kv_dtype, int32_t q_dtype, int32_t group,
                                    int32_t* block_size) {
  if (!block_size) return PA_ERR_NULL;
  if (!dtype_known(kv_dtype) || !dtype_known(q_dtype) || !pairing_ok(q_dtype, kv_dtype)) return PA_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PA_ERR_UNSUPPORTED;
  if (head_dim == 256 && q_dtype == PA_F32) return PA_ERR_UNSUPPORTED;
  if (group < 1) return PA_ERR_SHAPE;
  // Decode kernel time on MI355X (one session), B = 16 / 32 / 64, us:
  //   LLaMA-7B shape (group 1, d 128): bf16 708 / 709 / 716, fp8 383 / 377 / 380;
  //   GQA long context (group 4):      bf16 d 64 425 / 418 / 420, d 128 406 / 405 / 404,
  //                                    d 256 438 / 432 / 432;
  //                                    fp8  d 64 243 / 239 / 239, d 128 224 / 221 / 221,
  //                                    d 256 232 / 232 / 228.
  // A 32-key step reads whole K and V rows at every B, so B matters only
  // through the block-table lookups and the K rows a step gathers from one
  // block or two: 32 is within 0.5 % of the fastest everywhere except fp8
  // codes at d 256 (16-byte rows of 16 dims per lane), where 64 leads by 2 %.
  // fp32 caches follow the 16-bit choice (not measured separately).
  *block_size = (kv_dtype == PA_FP8_E4M3 && head_dim == 256) ? 64 : 32;
  return PA_OK;
}

pa_status_t pa_debug_check(int32_t* code, int32_t* index, void* stream) {
  if (!code || !index) return PA_ERR_NULL;
  if (!PA_DEBUG) {
    *code = -1;
    *index = -1;
    return PA_ERR_UNSUPPORTED;
  }
  if (pa::read_debug_words(code, index, static_cast<hipStream_t>(stream)) != hipSuccess) return PA_ERR_HIP;
  return *code == pa::kDebugNone ? PA_OK : PA_ERR_METADATA;
}

pa_status_t pa_set_attention_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return PA_ERR_NULL;
  g_events[0] = static_cast<hipEvent_t>(before);
  g_events[1] = static_cast<hipEvent_t>(after);
  return PA_OK;
}

pa_status_t pa_set_chunk_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return PA_ERR_NULL;
  g_events[2] = static_cast<hipEvent_t>(before);
  g_events[3] = static_cast<hipEvent_t>(after);
  return PA_OK;
}

pa_status_t pa_set_prefix_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return PA_ERR_NULL;
  g_events[4] = static_cast<hipEvent_t>(before);
  g_events[5] = static_cast<hipEvent_t>(after);
  return PA_OK;
}

pa_status_t pa_check_metadata(const pa_cache_t* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                              int32_t num_tokens, int32_t max_seq_len, int32_t max_query_len, int32_t* bad_seq,
                              void* stream) {
  pa_status_t st = check_cache(cache);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (bad_seq) *bad_seq = -1;
  if (num_seqs == 0) return num_tokens == 0 ? PA_OK : PA_ERR_METADATA;
  if (!block_tables || !seq_lens || !query_start_loc) return PA_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<int32_t> lens(num_seqs), qsl(num_seqs + 1),
      bt(static_cast<size_t>(num_seqs) * max_blocks_per_seq);
  if (hipMemcpyAsync(lens.data(), seq_lens, lens.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(qsl.data(), query_start_loc, qsl.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(bt.data(), block_tables, bt.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return PA_ERR_HIP;
  if (qsl[0] != 0 || qsl[num_seqs] != num_tokens) return PA_ERR_METADATA;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t ql = qsl[i + 1] - qsl[i];
    const int32_t L = lens[i];
    bool ok = ql >= 0 && ql <= L && L <= max_seq_len && ql <= max_query_len;
    const int64_t nb = ceil_div(L, cache->block_size);
    ok = ok && nb <= max_blocks_per_seq;
    for (int64_t j = 0; ok && j < nb; ++j) {
      const int32_t p = bt[static_cast<size_t>(i) * max_blocks_per_seq + j];
      ok = p >= 0 && p < cache->num_blocks;
    }
    if (!ok) {
      if (bad_seq) *bad_seq = i;
      return PA_ERR_METADATA;
    }
  }
  return PA_OK;
}

}  // extern "C"

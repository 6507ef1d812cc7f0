/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-attention library.
 *
 * The operation: attention over a KV cache split into fixed-size blocks of B
 * tokens, reached through a per-request block table that maps logical block
 * j to a physical block anywhere in a pool (itwiki "vLLM", section
 * "PagedAttention": "Block table" and "Block-wise attention"; the page states
 * the block-wise sum is mathematically ordinary attention).  One call serves
 * a token-budgeted step that mixes one-token decode rows with causal prompt
 * chunks (techknowgenie "vLLM V1 core refactoring", section "Dynamic Chunked
 * Prefill").  New K/V reach the cache through a per-token slot mapping, and
 * the step is described by seq_lens and query_start_loc (llm-wiki "vLLM 0.25
 * Model Runner V2", sections "Redesign 3" and "Redesign 4").
 *
 * Conventions for every entry point:
 *  - Pointers marked [device] are device pointers on the current HIP device;
 *    [host] pointers are read during the call only.  The library keeps no
 *    pointer after returning, allocates no memory, and is re-entrant.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without synchronising.  Inputs must stay valid and
 *    unmodified until the stream has executed the work; outputs are ready
 *    when the stream reaches that point.
 *  - Argument errors are detected before anything is enqueued and returned as
 *    a pa_status_t; nothing is launched then.  A failed launch returns
 *    PA_ERR_HIP.  There is no fallback path: an unsupported combination is an
 *    error, never a slower substitute.
 *  - The *contents* of metadata arrays are not checked (out-of-range block
 *    ids, q_len > seq_len or a decreasing query_start_loc are undefined
 *    behaviour); pa_check_metadata checks them on request.
 *
 * Cache layout (the pages give none; this is the library's definition):
 *    k_cache [num_blocks][num_kv_heads][block_size][head_dim]
 *    v_cache [num_blocks][num_kv_heads][block_size][head_dim]
 * i.e. every (block, kv head) tile is one contiguous run and a token's
 * head_dim elements are one row of it, in both pools.  Slot s of the pool is
 * token offset s % B of physical block s / B.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3 /* OCP E4M3FN: bias 7, max 448, NaN = S.1111.111, no inf */
} pa_dtype_t;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL                       */
  PA_ERR_SHAPE = 2,       /* a size is negative/zero where it must not be, or
                             shapes disagree (e.g. Hq % Hkv != 0)             */
  PA_ERR_DTYPE = 3,       /* unknown dtype, or a dtype pairing the path lacks  */
  PA_ERR_UNSUPPORTED = 4, /* block size / head dim / scale outside the path    */
  PA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required           */
  PA_ERR_HIP = 6,         /* a HIP runtime call or launch failed               */
  PA_ERR_METADATA = 7,    /* pa_check_metadata found an invalid entry          */
  PA_ERR_TOO_LARGE = 8    /* the step needs more device memory than the static
                             scratch of pa_attention_noalloc holds            */
} pa_status_t;

/* Description of a KV cache pool (host struct, read during the call only). */
typedef struct {
  int32_t num_blocks;   /* N: physical blocks in the pool                     */
  int32_t block_size;   /* B: tokens per block, one of 16, 32, 64             */
  int32_t num_kv_heads; /* Hkv                                                */
  int32_t head_dim;     /* d: 64, 128 or 256 (256 with 16-bit queries only)  */
  int32_t kv_dtype;     /* a pa_dtype_t                                       */
  float k_scale;        /* dequantisation multipliers: value = code * scale.  */
  float v_scale;        /* Must be 1.0f unless kv_dtype is PA_FP8_E4M3.       */
} pa_cache_t;

/*
 * Write new tokens' K and V into their cache slots.
 *
 * For each token t in [0, num_tokens) with s = slot_mapping[t] >= 0:
 *   k_cache[s / B][h][s % B][:] = enc(key[t][h][:])   for every kv head h
 *   v_cache[s / B][h][s % B][:] = enc(value[t][h][:])
 * where enc widens the source to fp32 exactly and then stores it as the
 * cache dtype: identity for fp32, round-to-nearest-even for fp16/bf16, and
 * for fp8 e4m3(fl32(x / scale)) with a correctly rounded fp32 division,
 * round-to-nearest-even, finite overflow and infinities saturated to +-448
 * and NaN kept as NaN.  Slots < 0 are skipped (padding).  Slot values must
 * be < num_blocks * B and unique among the non-negative entries.
 *
 *   key, value   [device] [num_tokens][num_kv_heads][head_dim], src_dtype
 *                (PA_F32, PA_F16 or PA_BF16), contiguous.
 *   k_cache, v_cache [device] pools in the layout above, cache->kv_dtype.
 *   slot_mapping [device] int64 [num_tokens].
 * num_tokens == 0 is a no-op returning PA_OK.
 */
pa_status_t pa_reshape_and_cache(const void* key, const void* value, int32_t src_dtype,
                                 void* k_cache, void* v_cache, const pa_cache_t* cache,
                                 const int64_t* slot_mapping, int32_t num_tokens,
                                 void* stream);

/*
 * Bytes of device workspace pa_attention needs for these sizes (written to
 * *bytes [host]).  The same arguments must be passed to pa_attention.
 */
pa_status_t pa_attention_workspace_size(const pa_cache_t* cache, int32_t num_q_heads,
                                        int32_t num_seqs, int32_t num_tokens,
                                        int32_t max_seq_len, int32_t max_query_len,
                                        size_t* bytes);

/*
 * Paged attention of one mixed step.
 *
 * Sequence i owns query rows [query_start_loc[i], query_start_loc[i+1]) of q;
 * q_len_i is their count and seq_lens[i] = L_i counts its cache tokens
 * including this step's (already written by pa_reshape_and_cache).  Query t
 * of sequence i sits at position L_i - q_len_i + t and sees the keys at
 * positions <= its own (causal within a chunk; a decode row sees all L_i).
 * Cache position p of sequence i is in physical block
 * block_tables[i * max_blocks_per_seq + p / B], offset p % B.  q head h
 * reads kv head h / (num_q_heads / num_kv_heads).  Then
 *   out[t][h][:] = sum_p softmax_p(scale * q[t][h] . k_p) v_p
 * computed with fp32 accumulation.
 *
 *   q        [device] [num_tokens][num_q_heads][head_dim], q_dtype, contiguous.
 *   out      [device] same shape and dtype as q; every row of a sequence with
 *            q_len > 0 is written (rounded to nearest even from fp32).
 *   block_tables [device] int32 [num_seqs][max_blocks_per_seq]; entries past
 *            a sequence's ceil(L/B) blocks are never read.
 *   seq_lens [device] int32 [num_seqs]; query_start_loc [device] int32
 *            [num_seqs + 1], 0 = qsl[0] <= ... <= qsl[num_seqs] = num_tokens.
 *   max_seq_len, max_query_len: host-side upper bounds of L_i and q_len_i
 *            (they size the launch; an actual value above them is undefined).
 *   workspace [device] at least pa_attention_workspace_size bytes, 256-byte
 *            aligned; its contents on entry do not matter.
 * scale must be finite and > 0 (PA_ERR_UNSUPPORTED otherwise).
 * dtype pairings: fp32 q with an fp32 cache; fp16 q with an fp16 or fp8
 * cache; bf16 q with a bf16 or fp8 cache.  Anything else is PA_ERR_DTYPE.
 * Sequences with q_len = 0 are no-ops.  num_seqs == 0 is a no-op.
 */
pa_status_t pa_attention(const void* q, int32_t q_dtype, const void* k_cache,
                         const void* v_cache, const pa_cache_t* cache,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, const int32_t* query_start_loc,
                         int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                         int32_t max_seq_len, int32_t max_query_len, float scale,
                         void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One step's cache write and attention in one call: the same result as
 * pa_reshape_and_cache(key, value, src_dtype, k_cache, v_cache, cache,
 * slot_mapping, num_new_tokens, stream) followed by pa_attention(q, ...,
 * stream) with the remaining arguments -- or, with prefix_len > 0,
 * pa_attention_shared_prefix(q, ..., prefix_len, ...) -- enqueued on
 * `stream` (the itwiki
 * "vLLM" article, section "PagedAttention": a step writes its new K/V into
 * the paged cache and then attends over it; the llm-wiki "vLLM 0.25 Model
 * Runner V2", section "Redesign 4", for the flat slot index).  The write
 * runs in the same launch as the step's work-list build, which does not
 * depend on it, so the step has one kernel launch fewer.
 *
 * Arguments, layouts and ownership are those of the two calls; the
 * workspace comes from pa_attention_workspace_size with the attention's
 * arguments (pa_attention_shared_prefix_workspace_size with prefix_len > 0).  Every argument of both is checked before anything is
 * enqueued, and on any error nothing is: the status is the first failing
 * check's (the cache write's checks first).  num_new_tokens == 0 is
 * pa_attention; num_seqs == 0 or num_tokens == 0 is the cache write alone.
 */
pa_status_t pa_write_and_attend(const void* key, const void* value, int32_t src_dtype,
                                const int64_t* slot_mapping, int32_t num_new_tokens,
                                const void* q, int32_t q_dtype, void* k_cache, void* v_cache,
                                const pa_cache_t* cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                const int32_t* query_start_loc, int32_t num_seqs,
                                int32_t num_tokens, int32_t num_q_heads, int32_t max_seq_len,
                                int32_t max_query_len, int32_t prefix_len, float scale, void* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged attention of a step whose sequences all share a prefix (cascade).
 *
 * Same arguments and result as pa_attention, plus prefix_len: every
 * sequence's first prefix_len cache positions are the same physical blocks
 * (block_tables[i][0 .. prefix_len/B) equal for all i; the kernels read
 * sequence 0's row for them), and every query row sits at or past
 * position prefix_len (seq_lens[i] - q_len_i >= prefix_len).  A prompt
 * shared by many requests, such as a system prompt, keeps its blocks once
 * with a reference count per block (itwiki "vLLM", section on block sharing
 * with copy-on-write; techknowgenie "vLLM V1 core refactoring", section on
 * restoring system prompts and multi-turn history without recomputation:
 * blocks whose token hash matches are re-linked by reference count, e.g. an
 * 8,000-token system prompt).  The shared keys are then read once for all
 * rows of the step:
 * one pass attends every query row to the prefix as a dense MFMA
 * contraction, the usual kernels attend each row to its own keys past the
 * prefix, and the log-sum-exp merge joins the two.  Mathematically the
 * result equals pa_attention's.
 *
 * prefix_len must be a multiple of the block size, at most max_seq_len
 * (PA_ERR_SHAPE otherwise); prefix_len == 0 is pa_attention.  A 16-bit
 * query is required (PA_ERR_UNSUPPORTED for fp32).  Sequences that break
 * the sharing or position conditions get undefined rows, never an
 * out-of-bounds access.  The workspace comes from
 * pa_attention_shared_prefix_workspace_size with the same arguments.
 */
pa_status_t pa_attention_shared_prefix_workspace_size(const pa_cache_t* cache, int32_t num_q_heads,
                                                      int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len,
                                                      int32_t max_query_len, int32_t prefix_len, size_t* bytes);

pa_status_t pa_attention_shared_prefix(const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                                       const pa_cache_t* cache, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                       const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                                       int32_t num_q_heads, int32_t max_seq_len, int32_t max_query_len,
                                       int32_t prefix_len, float scale, void* out, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Copy whole blocks: copy-on-write within a pool, or swapping between a
 * device pool and a host pool.
 *
 * For each pair k in [0, num_pairs) with s = block_mapping[2k] and
 * t = block_mapping[2k+1]: block t of the destination K pool (all kv heads)
 * becomes a copy of block s of the source K pool, and likewise for V.  A
 * block shared by several sequences is copied before one of them writes a
 * token into it (pass the same pool as source and destination), and the
 * blocks of a preempted request move out to host memory and back (itwiki
 * "vLLM", sections on block sharing with copy-on-write, and on scheduling
 * and preemption).  The copy is byte-exact.
 *
 *   src_k, src_v  source pool, [device] or page-locked [host], in the layout
 *                 above for src_cache.
 *   dst_k, dst_v  destination pool, [device] or page-locked [host], dst_cache.
 *   src_cache, dst_cache [host]: must agree on block_size, num_kv_heads,
 *                 head_dim and kv_dtype (PA_ERR_SHAPE otherwise); num_blocks
 *                 may differ; the scales are not used.
 *   block_mapping [device] int64 [num_pairs][2].
 * Host pools must be page-locked allocations the device can address
 * (hipHostMalloc, torch pin_memory); a pointer the runtime does not know,
 * or device memory of another device, is PA_ERR_UNSUPPORTED, detected
 * before anything is enqueued.  Pairs with an id outside its pool are
 * skipped.  Destination blocks must be distinct and, within one pool, no
 * destination may also be a source (the result would depend on order).
 * num_pairs == 0 is a no-op.
 */
pa_status_t pa_copy_blocks(const void* src_k, const void* src_v, const pa_cache_t* src_cache, void* dst_k,
                           void* dst_v, const pa_cache_t* dst_cache, const int64_t* block_mapping,
                           int32_t num_pairs, void* stream);

/*
 * Staged block-table writes.  The block table lives in device memory, one
 * row per persistent request slot; the host records only what changed, as
 * runs (row, start, values), packs them into one small buffer and has one
 * kernel apply them (llm-wiki "vLLM 0.25 Model Runner V2", "Redesign 3").
 *
 * For each write k in [0, num_writes):
 *   block_table[write_rows[k]][write_starts[k] + j] = write_values[write_offsets[k] + j]
 *   for j in [0, write_offsets[k+1] - write_offsets[k]).
 *
 *   block_table  [device] int32 [max_reqs][max_blocks], updated in place.
 *   write_rows, write_starts [device or page-locked host] int32 [num_writes].
 *   write_offsets [device or page-locked host] int32 [num_writes + 1],
 *                non-decreasing, write_offsets[0] = 0, last = num_values.
 *   write_values [device or page-locked host] int32 [num_values].
 * Staging buffers in page-locked host memory are read by the kernel over
 * the host link (no separate copy); other host memory is
 * PA_ERR_UNSUPPORTED.  Writes whose row or columns fall outside the table
 * are skipped.  Two writes to one entry leave either value.  A call with no
 * writes is a no-op.
 */
pa_status_t pa_apply_block_table_writes(int32_t* block_table, int32_t max_reqs, int32_t max_blocks,
                                        const int32_t* write_rows, const int32_t* write_starts,
                                        const int32_t* write_offsets, const int32_t* write_values,
                                        int32_t num_writes, int32_t num_values, void* stream);

/*
 * Inputs of one step from persistent request state, built on the GPU
 * (llm-wiki "vLLM 0.25 Model Runner V2", "Redesign 1": a request keeps its
 * slot while active and idx_mapping names the slot each batch position
 * reads; "Redesign 4": query_start_loc is the running sum of the per-request
 * token counts, and positions, seq_lens and the slot mapping are built on
 * the GPU).  For batch position b in [0, num_reqs) with s = idx_mapping[b]:
 *   query_start_loc[0] = 0, query_start_loc[b+1] = query_start_loc[b] + num_scheduled[b]
 *   seq_lens[b]  = num_computed[s] + num_scheduled[b]
 *   step_block_tables[b][:] = block_table[s][:]
 * and for query token t = query_start_loc[b] + i, i < num_scheduled[b]:
 *   positions[t]    = num_computed[s] + i
 *   slot_mapping[t] = block_table[s][positions[t] / block_size] * block_size
 *                     + positions[t] % block_size
 * num_computed counts the request's tokens already in the cache; the
 * outputs feed pa_reshape_and_cache and pa_attention directly.
 *
 *   block_table [device] int32 [max_reqs][max_blocks] (by persistent slot).
 *   idx_mapping [device] int32 [num_reqs]; num_computed [device] int32
 *               [max_reqs]; num_scheduled [device] int32 [num_reqs].
 *   query_start_loc [device] int32 [num_reqs + 1]; seq_lens [device] int32
 *               [num_reqs]; positions, slot_mapping [device] int64
 *               [num_tokens]; step_block_tables [device] int32
 *               [num_reqs][max_blocks].
 * num_tokens must equal the sum of num_scheduled (the scheduler knows it);
 * tokens past that sum, tokens whose block is past the table's width and
 * tokens of a batch position whose slot is outside [0, max_reqs) get
 * position -1 and slot -1 (a skipped cache write).  num_reqs == 0 is a no-op.
 */
pa_status_t pa_prepare_step(const int32_t* block_table, int32_t max_reqs, int32_t max_blocks,
                            const int32_t* idx_mapping, const int32_t* num_computed,
                            const int32_t* num_scheduled, int32_t num_reqs, int32_t num_tokens,
                            int32_t block_size, int32_t* query_start_loc, int32_t* seq_lens,
                            int64_t* positions, int64_t* slot_mapping, int32_t* step_block_tables,
                            void* stream);

/*
 * End of a step: its tokens are cached.  For b in [0, num_reqs):
 *   num_computed[idx_mapping[b]] += num_scheduled[b]
 * (positions outside [0, max_reqs) are skipped).  With pa_prepare_step this
 * keeps the step loop on the GPU: prepare, write the cache, attend, commit,
 * so several decode steps can run back to back -- captured once in a HIP
 * graph and replayed -- without the host preparing each step (techknowgenie
 * "vLLM V1 core refactoring", section on the PagedAttention V3 kernel
 * architecture: a GPU graph runner executes N decode steps on its own; the
 * blocks those steps fill must already be in the table).
 *
 *   num_computed [device] int32 [max_reqs], updated in place;
 *   idx_mapping, num_scheduled [device] int32 [num_reqs].
 * Batch positions must name distinct slots.  num_reqs == 0 is a no-op.
 */
pa_status_t pa_commit_step(int32_t* num_computed, int32_t max_reqs, const int32_t* idx_mapping,
                           const int32_t* num_scheduled, int32_t num_reqs, void* stream);

/*
 * Debug check of metadata contents.  Synchronous: copies the metadata to the
 * host (on `stream`) and returns PA_ERR_METADATA if any sequence has
 * q_len < 0, q_len > L, L > max_seq_len, q_len > max_query_len,
 * ceil(L/B) > max_blocks_per_seq, or a used block id outside [0, num_blocks);
 * PA_OK otherwise.  When it fails, *bad_seq [host, may be NULL] receives the
 * first offending sequence (-1 for a query_start_loc that does not start at
 * 0 or end at num_tokens).
 */
pa_status_t pa_check_metadata(const pa_cache_t* cache, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens,
                              const int32_t* query_start_loc, int32_t num_seqs,
                              int32_t num_tokens, int32_t max_seq_len, int32_t max_query_len,
                              int32_t* bad_seq, void* stream);

/*
 * Debug builds (the library compiled with -DPA_DEBUG=1, libpa_debug.so): the
 * step plan checks each sequence's metadata before it makes work items
 * (query_start_loc starts at 0, ends at num_tokens and does not decrease;
 * 0 <= L <= max_seq_len; q_len <= L and <= max_query_len; ceil(L/B) <=
 * max_blocks_per_seq and every used block id in [0, num_blocks)), the
 * attention kernels check each block id they load, and the cache write each
 * slot (< num_blocks * B).  The first violation is recorded as (code, index)
 * in a per-device word pair, and the offending sequence, block or token is
 * skipped (or read as block 0), so nothing is read or written outside the
 * caller's buffers; the affected rows are undefined.  Codes: 1 bad
 * query_start_loc, 2 q_len > L, 3 L outside [0, max_seq_len], 4 q_len >
 * max_query_len, 5 a block id outside the pool (or too many blocks), 6 a slot
 * outside the pool; index is the sequence (codes 1-5) or the token (6).
 *
 * pa_debug_check waits for `stream`, writes the recorded pair to *code and
 * *index [host] (0, 0 when nothing was recorded), clears it, and returns
 * PA_OK or PA_ERR_METADATA.  Release builds check nothing and return
 * PA_ERR_UNSUPPORTED (with -1, -1).
 */
pa_status_t pa_debug_check(int32_t* code, int32_t* index, void* stream);

/*
 * Measurement hook.  When both are non-NULL, every later pa_attention call
 * records hipEvent_t `before` on its stream immediately before launching the
 * decode attention kernel and `after` immediately after it, so
 * hipEventElapsedTime gives that one kernel's duration (the work-list, chunk
 * and partition-merge kernels fall outside).  Pass NULL, NULL to turn it off.  This is the
 * library's only global state; it is meant for timing harnesses and is not
 * thread-safe.
 */
pa_status_t pa_set_attention_events(void* before, void* after);

/*
 * The same hook for the chunk kernel, which pa_attention launches (after the
 * decode kernel) when some sequence may have at least 65 (query token, q head)
 * rows per kv head, i.e. a prompt chunk (max_query_len * Hq / Hkv >= 65 with
 * a 16-bit q); the events are recorded only on calls that launch it.
 */
pa_status_t pa_set_chunk_events(void* before, void* after);

/*
 * The same hook for the shared-prefix pass of pa_attention_shared_prefix
 * (recorded only on calls with prefix_len > 0).
 */
pa_status_t pa_set_prefix_events(void* before, void* after);

/*
 * The block size (tokens per cache block) the attention kernels run fastest
 * with for a head dim, a (q dtype, cache dtype) pairing and a query group
 * (group = q heads per kv head), as measured on MI355X over decode steps at
 * B = 16, 32 and 64: 64 for an fp8 cache at head dim 256, 32 otherwise (the
 * query group does not change the choice on this GPU; it is part of the
 * question).  The page chooses the block size among 16, 32 and 64 tokens
 * by head dim and precision (techknowgenie "vLLM V1 core refactoring",
 * section "PagedAttention V3 kernel architecture and hardware-level memory
 * alignment", adaptive block tiling).  Writes 16, 32 or 64 to *block_size [host].  Every
 * block size works with every entry point; this is a performance choice for
 * the caller that sizes the pool.  PA_ERR_UNSUPPORTED for a head dim outside
 * {64, 128, 256} (or 256 with fp32), PA_ERR_DTYPE for a pairing pa_attention
 * rejects, PA_ERR_SHAPE for group < 1, PA_ERR_NULL for a NULL block_size.
 */
pa_status_t pa_preferred_block_size(int32_t head_dim, int32_t kv_dtype, int32_t q_dtype, int32_t group,
                                    int32_t* block_size);

/*
 * pa_attention for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc.
 * Same arguments and result as pa_attention, without the workspace: the
 * step's work lists and split-context partials live in a static device
 * array of PA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on each
 * device it runs on until the process ends.  The call allocates nothing
 * (no hipMalloc, no allocating library routine).
 *
 * A step whose pa_attention_workspace_size exceeds PA_NOALLOC_SCRATCH_BYTES
 * returns PA_ERR_TOO_LARGE before anything is enqueued (the decode steps of
 * the LLaMA-7B shape need about 4 MiB, 64 sequences at 32k contexts with 8
 * kv heads of dim 128 about 57 MiB with a bf16 cache and 33 MiB with fp8; a
 * 3,840-token mixed step with 9k contexts needs about 305 MiB and
 * takes pa_attention with a caller workspace).  All calls on one device
 * share that device's array, which keeps the last call's contents: calls
 * that overlap on one device (two streams, or two host threads) race and
 * give undefined rows.  Calls ordered on one stream are safe.  The first
 * call on a device looks up the array's address there (PA_ERR_HIP if that
 * fails).
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status_t pa_attention_noalloc(const void* q, int32_t q_dtype, const void* k_cache,
                                 const void* v_cache, const pa_cache_t* cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens, const int32_t* query_start_loc,
                                 int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                 int32_t max_seq_len, int32_t max_query_len, float scale,
                                 void* out, void* stream);

/* Static text for a status code. */
const char* pa_status_string(pa_status_t status);

/* Library version, e.g. "0.1.0". */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */

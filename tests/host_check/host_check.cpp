// host_check.cpp -- the host validation layer of the C ABI (pa_api.hip and
// pa_noalloc.hip: argument checks, workspace sizing, the launch arguments it
// builds) compiled with AddressSanitizer and UndefinedBehaviorSanitizer and
// linked against stub launchers instead of the kernels.  Every entry point
// is driven with valid and invalid arguments, extremes included; each call
// that reaches a stub must hand it buffers that fit what the caller passed.
// Runs on the CPU; no device memory is touched (the pointers are never
// dereferenced).  Exit status 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <limits>
#include <random>

#include "pa.h"
#include "pa_internal.h"

namespace {
int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

pa::AttnArgs g_attn;
pa::CacheWriteArgs g_write;
int g_attn_launches = 0, g_write_launches = 0, g_other_launches = 0;
int g_joint_writes = 0, g_joint_src = -1;   // cache writes handed to the attention launcher
}  // namespace

// ---- stub launchers: record what the host layer would launch
namespace pa {
hipError_t launch_attention(int, int, int, int, const AttnArgs& a, hipStream_t, const hipEvent_t*,
                            const CacheWriteArgs* w, int src) {
  g_attn = a;
  ++g_attn_launches;
  if (w) {
    g_write = *w;
    g_joint_src = src;
    ++g_joint_writes;
  }
  return hipSuccess;
}
hipError_t launch_reshape_and_cache(int, int, const CacheWriteArgs& a, hipStream_t) {
  g_write = a;
  ++g_write_launches;
  return hipSuccess;
}
hipError_t launch_copy_blocks(const BlockCopyArgs&, hipStream_t) { ++g_other_launches; return hipSuccess; }
hipError_t launch_table_writes(const TableWriteArgs&, hipStream_t) { ++g_other_launches; return hipSuccess; }
hipError_t launch_prepare_step(const StepArgs&, hipStream_t) { ++g_other_launches; return hipSuccess; }
hipError_t launch_commit_step(const CommitArgs&, hipStream_t) { ++g_other_launches; return hipSuccess; }
int32_t* debug_words() { return nullptr; }
hipError_t read_debug_words(int32_t*, int32_t*, hipStream_t) { return hipErrorNotSupported; }
}  // namespace pa

namespace {

void* const FAKE = reinterpret_cast<void*>(uintptr_t(1) << 40);     // 256-aligned, never dereferenced
const int32_t* const FAKEI = static_cast<const int32_t*>(FAKE);

pa_cache_t cache(int32_t N, int32_t B, int32_t H, int32_t d, int32_t dt, float ks = 1.f, float vs = 1.f) {
  pa_cache_t c;
  c.num_blocks = N;
  c.block_size = B;
  c.num_kv_heads = H;
  c.head_dim = d;
  c.kv_dtype = dt;
  c.k_scale = ks;
  c.v_scale = vs;
  return c;
}

// The workspace regions handed to the kernels lie inside [ws, ws + bytes),
// in order, 256-byte aligned, each as large as the launch arguments say.
void check_layout(const pa::AttnArgs& a, uintptr_t ws, size_t bytes, int32_t d) {
  const uintptr_t end = ws + bytes;
  auto at = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
  CHECK(at(a.header) == ws);
  CHECK(at(a.items) >= ws + 64 * 4 && at(a.items) % 256 == 0);
  CHECK(at(a.items) + static_cast<uintptr_t>(a.max_items) * 16 <= at(a.citems));
  CHECK(at(a.citems) + static_cast<uintptr_t>(a.max_citems) * 8 <= at(a.part_m));
  // every row's partial list: decode rows at most (slots) x Hq x dec_parts,
  // then chunk rows T x Hq x chunk_parts from chunk_row_base (0 and equal
  // lengths when one token-indexed list serves both)
  const uintptr_t dslots = a.dec_per_seq > 0 ? uintptr_t(a.dec_per_seq) * a.num_seqs : uintptr_t(a.num_tokens);
  const uintptr_t drows = dslots * a.num_q_heads * a.dec_parts;
  const uintptr_t crows = uintptr_t(a.chunk_row_base) + uintptr_t(a.num_tokens) * a.num_q_heads * a.chunk_parts;
  CHECK(a.dec_per_seq == 0 || uintptr_t(a.chunk_row_base) == drows);
  const uintptr_t rows = drows > crows ? drows : crows;
  CHECK(at(a.part_m) + rows * 4 <= at(a.part_l));
  CHECK(at(a.part_l) + rows * 4 <= at(a.part_acc));
  CHECK(at(a.part_acc) + rows * d * 4 <= end);
  CHECK(a.dec_parts >= 1 && a.partition >= 32 && a.max_seq_len >= 0);
  // a decode-routed sequence (q_len * G < 65) fits its slots
  CHECK(a.dec_per_seq == 0 || int64_t(a.dec_per_seq) * a.group >= 64 / a.group * a.group);
}

pa_status_t attend(const pa_cache_t& c, int32_t q_dtype, int32_t Hq, int32_t S, int32_t T, int32_t max_seq,
                   int32_t max_q, int32_t mbps, void* ws, size_t bytes, int32_t prefix = 0, float scale = 0.125f) {
  if (prefix)
    return pa_attention_shared_prefix(FAKE, q_dtype, FAKE, FAKE, &c, FAKEI, mbps, FAKEI, FAKEI, S, T, Hq, max_seq,
                                      max_q, prefix, scale, FAKE, ws, bytes, nullptr);
  return pa_attention(FAKE, q_dtype, FAKE, FAKE, &c, FAKEI, mbps, FAKEI, FAKEI, S, T, Hq, max_seq, max_q, scale,
                      FAKE, ws, bytes, nullptr);
}

void argument_errors() {
  const pa_cache_t ok = cache(16, 16, 2, 64, PA_BF16);
  CHECK(attend(cache(16, 8, 2, 64, PA_BF16), PA_BF16, 4, 2, 2, 40, 1, 3, FAKE, 1 << 30) == PA_ERR_UNSUPPORTED);
  CHECK(attend(cache(16, 16, 2, 96, PA_BF16), PA_BF16, 4, 2, 2, 40, 1, 3, FAKE, 1 << 30) == PA_ERR_UNSUPPORTED);
  CHECK(attend(cache(16, 16, 2, 64, 9), PA_BF16, 4, 2, 2, 40, 1, 3, FAKE, 1 << 30) == PA_ERR_DTYPE);
  CHECK(attend(ok, PA_F32, 4, 2, 2, 40, 1, 3, FAKE, 1 << 30) == PA_ERR_DTYPE);
  CHECK(attend(ok, PA_BF16, 3, 2, 2, 40, 1, 3, FAKE, 1 << 30) == PA_ERR_SHAPE);
  CHECK(attend(ok, PA_BF16, 4, 2, 2, 40, 1, 2, FAKE, 1 << 30) == PA_ERR_SHAPE);       // 2 blocks < 40 tokens
  CHECK(attend(ok, PA_BF16, 4, 2, 2, 40, 41, 3, FAKE, 1 << 30) == PA_ERR_SHAPE);      // q bound above L bound
  CHECK(attend(ok, PA_BF16, 4, 2, 2, 40, 1, 3, nullptr, 1 << 30) == PA_ERR_WORKSPACE);
  CHECK(attend(ok, PA_BF16, 4, 2, 2, 40, 1, 3, static_cast<char*>(FAKE) + 16, 1 << 30) == PA_ERR_WORKSPACE);
  CHECK(attend(ok, PA_BF16, 4, 2, 2, 40, 1, 3, FAKE, 1 << 30, 8) == PA_ERR_SHAPE);    // prefix not whole blocks
  CHECK(attend(ok, PA_BF16, 4, -1, 2, 40, 1, 3, FAKE, 1 << 30) == PA_ERR_SHAPE);
  CHECK(attend(ok, PA_BF16, 4, 2, 2, 40, 1, 3, FAKE, 1 << 30, 0, -1.f) == PA_ERR_UNSUPPORTED);
  CHECK(attend(ok, PA_BF16, 4, 2, 2, 40, 1, 3, FAKE, 1 << 30, 0, std::numeric_limits<float>::quiet_NaN()) ==
        PA_ERR_UNSUPPORTED);
  CHECK(attend(cache(16, 16, 2, 64, PA_BF16, 2.f), PA_BF16, 4, 2, 2, 40, 1, 3, FAKE, 1 << 30) == PA_ERR_UNSUPPORTED);
  CHECK(attend(cache(0, 16, 2, 64, PA_BF16), PA_BF16, 4, 2, 2, 40, 1, 3, FAKE, 1 << 30) == PA_ERR_SHAPE);
  CHECK(attend(ok, PA_BF16, 4, 0, 0, 40, 1, 3, nullptr, 0) == PA_OK);                  // empty step: no-op
  CHECK(pa_attention(nullptr, PA_BF16, FAKE, FAKE, &ok, FAKEI, 3, FAKEI, FAKEI, 2, 2, 4, 40, 1, 0.1f, FAKE, FAKE,
                     1 << 30, nullptr) == PA_ERR_NULL);
  size_t b = 0;
  CHECK(pa_attention_workspace_size(nullptr, 4, 2, 2, 40, 1, &b) == PA_ERR_NULL);
  CHECK(pa_attention_workspace_size(&ok, 4, 2, 2, 40, 1, nullptr) == PA_ERR_NULL);
  // partials past 2^48 bytes are refused (2^20 tokens x 2^20 q heads)
  const pa_cache_t wide = cache(16, 16, 1 << 16, 64, PA_BF16);
  CHECK(pa_attention_workspace_size(&wide, 1 << 20, 1 << 20, 1 << 20, 4096, 1, &b) == PA_ERR_UNSUPPORTED);
  // more tokens than the sequences' query bound allows
  CHECK(pa_attention_workspace_size(&ok, 4, 2, 5, 40, 2, &b) == PA_ERR_SHAPE);
  // cache write
  CHECK(pa_reshape_and_cache(FAKE, FAKE, 7, FAKE, FAKE, &ok, static_cast<const int64_t*>(FAKE), 4, nullptr) ==
        PA_ERR_DTYPE);
  CHECK(pa_reshape_and_cache(FAKE, FAKE, PA_BF16, FAKE, FAKE, &ok, static_cast<const int64_t*>(FAKE), -1, nullptr) ==
        PA_ERR_SHAPE);
  CHECK(pa_reshape_and_cache(nullptr, FAKE, PA_BF16, FAKE, FAKE, &ok, static_cast<const int64_t*>(FAKE), 4,
                             nullptr) == PA_ERR_NULL);
  // block copies: a pointer the runtime does not know is refused before any launch
  CHECK(pa_copy_blocks(FAKE, FAKE, &ok, FAKE, FAKE, &ok, static_cast<const int64_t*>(FAKE), 1, nullptr) ==
        PA_ERR_UNSUPPORTED);
  const pa_cache_t other = cache(16, 32, 2, 64, PA_BF16);
  CHECK(pa_copy_blocks(FAKE, FAKE, &ok, FAKE, FAKE, &other, static_cast<const int64_t*>(FAKE), 1, nullptr) ==
        PA_ERR_SHAPE);
  // metadata checker: argument errors only (a valid call copies from the device)
  CHECK(pa_check_metadata(&ok, FAKEI, 0, FAKEI, FAKEI, 1, 1, 40, 1, nullptr, nullptr) == PA_ERR_SHAPE);
  CHECK(pa_check_metadata(&ok, nullptr, 3, FAKEI, FAKEI, 1, 1, 40, 1, nullptr, nullptr) == PA_ERR_NULL);
  // step inputs
  CHECK(pa_prepare_step(FAKEI, 0, 4, FAKEI, FAKEI, FAKEI, 1, 1, 16, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr) == PA_ERR_SHAPE);
  CHECK(pa_commit_step(nullptr, 4, FAKEI, FAKEI, 1, nullptr) == PA_ERR_NULL);
  CHECK(pa_apply_block_table_writes(nullptr, 4, 4, FAKEI, FAKEI, FAKEI, FAKEI, 1, 1, nullptr) == PA_ERR_NULL);
  // debug record: a release build checks nothing
  int32_t code = 0, index = 0;
  CHECK(pa_debug_check(&code, &index, nullptr) == PA_ERR_UNSUPPORTED && code == -1 && index == -1);
  // status strings and the version
  for (int s = 0; s <= 9; ++s) CHECK(pa_status_string(static_cast<pa_status_t>(s)) != nullptr);
  CHECK(strlen(pa_version()) > 0);
  int32_t bs = 0;
  CHECK(pa_preferred_block_size(128, PA_FP8_E4M3, PA_BF16, 4, &bs) == PA_OK && bs == 32);
  CHECK(pa_preferred_block_size(256, PA_FP8_E4M3, PA_BF16, 1, &bs) == PA_OK && bs == 64);
  CHECK(pa_preferred_block_size(128, PA_BF16, PA_BF16, 4, &bs) == PA_OK && bs == 32);
  CHECK(pa_preferred_block_size(128, PA_BF16, PA_BF16, 0, &bs) == PA_ERR_SHAPE);
  CHECK(pa_preferred_block_size(std::numeric_limits<int32_t>::min(), PA_BF16, PA_BF16, 1, &bs) == PA_ERR_UNSUPPORTED);
}

// Valid calls reach the stub with a workspace layout inside the caller's
// buffer; one byte less is refused.
void valid_calls() {
  const int32_t dts[][2] = {{PA_BF16, PA_BF16}, {PA_F16, PA_FP8_E4M3}, {PA_F32, PA_F32}, {PA_BF16, PA_FP8_E4M3}};
  for (auto& dt : dts) {
    for (int32_t d : {64, 128, 256}) {
      if (d == 256 && dt[0] == PA_F32) continue;
      const float sc = dt[1] == PA_FP8_E4M3 ? 0.03125f : 1.f;
      const pa_cache_t c = cache(1000, 16, 8, d, dt[1], sc, sc);
      for (int32_t max_seq : {1, 17, 2048, 9216, 131072}) {
        const int32_t S = 64, Hq = 32, max_q = max_seq < 1024 ? max_seq : 1024;
        const int32_t T = 64 + 1024 < S * max_q ? 64 + 1024 : S * max_q;
        const int32_t mbps = (max_seq + 15) / 16;
        size_t need = 0;
        CHECK(pa_attention_workspace_size(&c, Hq, S, T, max_seq, max_q, &need) == PA_OK);
        const int before = g_attn_launches;
        CHECK(attend(c, dt[0], Hq, S, T, max_seq, max_q, mbps, FAKE, need) == PA_OK);
        CHECK(g_attn_launches == before + 1);
        check_layout(g_attn, reinterpret_cast<uintptr_t>(FAKE), need, d);
        CHECK(g_attn.max_seq_len == max_seq && g_attn.num_blocks == 1000 && g_attn.block_size == 16);
        CHECK(attend(c, dt[0], Hq, S, T, max_seq, max_q, mbps, FAKE, need - 1) == PA_ERR_WORKSPACE);
        // shared prefix of whole blocks
        if (dt[0] != PA_F32 && max_seq >= 2048) {
          CHECK(pa_attention_shared_prefix_workspace_size(&c, Hq, S, T, max_seq, max_q, 1024, &need) == PA_OK);
          CHECK(attend(c, dt[0], Hq, S, T, max_seq, max_q, mbps, FAKE, need, 1024) == PA_OK);
          check_layout(g_attn, reinterpret_cast<uintptr_t>(FAKE), need, d);
          CHECK(g_attn.prefix_parts >= 1 && g_attn.dec_parts > g_attn.prefix_parts);
        }
      }
    }
  }
  // the cache write hands the stub the pool geometry
  const pa_cache_t c = cache(77, 32, 4, 128, PA_FP8_E4M3, 0.5f, 0.25f);
  CHECK(pa_reshape_and_cache(FAKE, FAKE, PA_BF16, FAKE, FAKE, &c, static_cast<const int64_t*>(FAKE), 9, nullptr) ==
        PA_OK);
  CHECK(g_write_launches == 1 && g_write.num_slots == 77 * 32 && g_write.num_tokens == 9 &&
        g_write.k_scale == 0.5f && g_write.v_scale == 0.25f);
  // the joint write-and-attend call: both argument sets checked before any
  // launch; the write goes to the attention launcher, or alone without rows
  {
    const pa_cache_t cb = cache(77, 32, 4, 128, PA_BF16);
    const int64_t* slots = static_cast<const int64_t*>(FAKE);
    const int a0 = g_attn_launches, w0 = g_write_launches, j0 = g_joint_writes;
    CHECK(pa_write_and_attend(FAKE, FAKE, PA_F32, slots, 5, FAKE, PA_BF16, FAKE, FAKE, &cb, FAKEI, 4, FAKEI, FAKEI,
                              2, 2, 8, 100, 1, 0, 0.1f, FAKE, FAKE, size_t(1) << 40, nullptr) == PA_OK);
    CHECK(g_attn_launches == a0 + 1 && g_joint_writes == j0 + 1 && g_write_launches == w0);
    CHECK(g_write.num_tokens == 5 && g_write.num_slots == 77 * 32 && g_joint_src == PA_F32);
    // a bad write argument or a bad attention argument: nothing launched
    CHECK(pa_write_and_attend(nullptr, FAKE, PA_F32, slots, 5, FAKE, PA_BF16, FAKE, FAKE, &cb, FAKEI, 4, FAKEI,
                              FAKEI, 2, 2, 8, 100, 1, 0, 0.1f, FAKE, FAKE, size_t(1) << 40, nullptr) == PA_ERR_NULL);
    CHECK(pa_write_and_attend(FAKE, FAKE, PA_FP8_E4M3, slots, 5, FAKE, PA_BF16, FAKE, FAKE, &cb, FAKEI, 4, FAKEI,
                              FAKEI, 2, 2, 8, 100, 1, 0, 0.1f, FAKE, FAKE, size_t(1) << 40, nullptr) == PA_ERR_DTYPE);
    CHECK(pa_write_and_attend(FAKE, FAKE, PA_F32, slots, 5, FAKE, PA_F16, FAKE, FAKE, &cb, FAKEI, 4, FAKEI, FAKEI,
                              2, 2, 8, 100, 1, 0, 0.1f, FAKE, FAKE, size_t(1) << 40, nullptr) == PA_ERR_DTYPE);
    CHECK(pa_write_and_attend(FAKE, FAKE, PA_F32, slots, 5, FAKE, PA_BF16, FAKE, FAKE, &cb, FAKEI, 4, FAKEI, FAKEI,
                              2, 2, 8, 100, 1, 0, 0.1f, FAKE, FAKE, 16, nullptr) == PA_ERR_WORKSPACE);
    CHECK(g_attn_launches == a0 + 1 && g_joint_writes == j0 + 1 && g_write_launches == w0);
    // no new tokens: pa_attention; no attention rows: the write alone
    CHECK(pa_write_and_attend(nullptr, nullptr, PA_F32, nullptr, 0, FAKE, PA_BF16, FAKE, FAKE, &cb, FAKEI, 4, FAKEI,
                              FAKEI, 2, 2, 8, 100, 1, 0, 0.1f, FAKE, FAKE, size_t(1) << 40, nullptr) == PA_OK);
    CHECK(g_attn_launches == a0 + 2 && g_joint_writes == j0 + 1);
    CHECK(pa_write_and_attend(FAKE, FAKE, PA_BF16, slots, 3, nullptr, PA_BF16, FAKE, FAKE, &cb, nullptr, 4, nullptr,
                              nullptr, 0, 0, 8, 100, 1, 0, 0.1f, nullptr, nullptr, 0, nullptr) == PA_OK);
    CHECK(g_attn_launches == a0 + 2 && g_write_launches == w0 + 1 && g_write.num_tokens == 3);
    // with a shared prefix (whole blocks, every query past it)
    CHECK(pa_write_and_attend(FAKE, FAKE, PA_F32, slots, 5, FAKE, PA_BF16, FAKE, FAKE, &cb, FAKEI, 4, FAKEI, FAKEI,
                              2, 2, 8, 100, 1, 64, 0.1f, FAKE, FAKE, size_t(1) << 40, nullptr) == PA_OK);
    CHECK(g_attn_launches == a0 + 3 && g_joint_writes == j0 + 2 && g_attn.prefix_len == 64 &&
          g_attn.prefix_parts >= 1);
    CHECK(pa_write_and_attend(FAKE, FAKE, PA_F32, slots, 5, FAKE, PA_BF16, FAKE, FAKE, &cb, FAKEI, 4, FAKEI, FAKEI,
                              2, 2, 8, 100, 1, 40, 0.1f, FAKE, FAKE, size_t(1) << 40, nullptr) == PA_ERR_SHAPE);
    CHECK(g_attn_launches == a0 + 3);
  }
  // step inputs and commit reach their launchers
  const int before = g_other_launches;
  CHECK(pa_prepare_step(FAKEI, 8, 4, FAKEI, FAKEI, FAKEI, 2, 3, 16, static_cast<int32_t*>(FAKE),
                        static_cast<int32_t*>(FAKE), static_cast<int64_t*>(FAKE), static_cast<int64_t*>(FAKE),
                        static_cast<int32_t*>(FAKE), nullptr) == PA_OK);
  CHECK(pa_commit_step(static_cast<int32_t*>(FAKE), 8, FAKEI, FAKEI, 2, nullptr) == PA_OK);
  CHECK(g_other_launches == before + 2);
}

// Random sizes, extremes included: every call either fails validation or
// reaches the stub with a layout that fits the size the library asked for
// (and the size arithmetic never overflows: UBSan checks the signed part).
void random_sizes() {
  std::mt19937_64 rng(141);
  const int32_t big = std::numeric_limits<int32_t>::max();
  const int32_t picks[] = {-1, 0, 1, 2, 15, 16, 17, 63, 64, 65, 1000, 4096, 65535, 65536, 1 << 20, big - 1, big};
  auto pick = [&]() { return picks[rng() % (sizeof(picks) / sizeof(picks[0]))]; };
  int reached = 0;
  for (int it = 0; it < 20000; ++it) {
    const int32_t H = (rng() % 3 == 0) ? pick() : int32_t(1 + rng() % 16);
    const int64_t hq = int64_t(H) * int64_t(1 + rng() % 8);
    const int32_t Hq = (rng() % 3 == 0) ? pick() : int32_t(hq < big ? hq : big);
    const int32_t d = (rng() % 4 == 0) ? pick() : (rng() % 2 ? 128 : 64);
    const int32_t B = (rng() % 4 == 0) ? pick() : (16 << (rng() % 3));
    const pa_cache_t c = cache((rng() % 4 == 0) ? pick() : 5000, B, H, d, PA_BF16);
    const int32_t S = (rng() % 2) ? pick() : int32_t(rng() % 300);
    const int32_t T = (rng() % 2) ? pick() : int32_t(rng() % 5000);
    const int32_t max_seq = (rng() % 2) ? pick() : int32_t(rng() % 200000);
    const int32_t max_q = (rng() % 2) ? pick() : int32_t(rng() % 5000);
    const int32_t prefix = (rng() % 4 == 0) ? 16 * int32_t(rng() % 100) : 0;
    size_t need = 0;
    const pa_status_t st = prefix ? pa_attention_shared_prefix_workspace_size(&c, Hq, S, T, max_seq, max_q, prefix, &need)
                                  : pa_attention_workspace_size(&c, Hq, S, T, max_seq, max_q, &need);
    if (st != PA_OK) continue;
    CHECK(need >= 256 && need < (size_t(1) << 52));
    const int32_t mbps = B > 0 ? int32_t((int64_t(max_seq) + B - 1) / B) : 1;
    const int before = g_attn_launches;
    const pa_status_t at = attend(c, PA_BF16, Hq, S, T, max_seq, max_q, mbps > 0 ? mbps : 1, FAKE, need, prefix);
    if (S == 0 || T == 0) {
      CHECK(at == PA_OK && g_attn_launches == before);
      continue;
    }
    CHECK(at == PA_OK);
    if (at == PA_OK && g_attn_launches == before + 1) {
      check_layout(g_attn, reinterpret_cast<uintptr_t>(FAKE), need, d);
      ++reached;
    }
    // the no-allocation entry point: too large, or it goes on to the device
    // (absent here) -- never a launch without its scratch
    const pa_status_t na = pa_attention_noalloc(FAKE, PA_BF16, FAKE, FAKE, &c, FAKEI, mbps > 0 ? mbps : 1, FAKEI, FAKEI,
                                                S, T, Hq, max_seq, max_q, 0.125f, FAKE, nullptr);
    if (!prefix) {
      if (need > PA_NOALLOC_SCRATCH_BYTES) CHECK(na == PA_ERR_TOO_LARGE);
      else CHECK(na == PA_ERR_HIP || na == PA_OK);   // no device here: the scratch lookup fails
    }
  }
  CHECK(reached > 100);
  fprintf(stderr, "random sizes: %d calls reached the launcher\n", reached);
}

}  // namespace

// The tail split's cut of a row tile's keys (pa::DecodeCut), which the plan,
// the decode items and the merge each derive on their own: its items tile
// [0, own) in key order with no gap or overlap, item_of maps every key to
// the item that holds it, the last item is not empty, only the last S
// partitions are cut, and the item count stays within the workspace's
// per-tile bound ceil(own / P) + split_max * (F - 1).
void decode_cut() {
  const int parts[] = {512, 1024, 2048};
  for (int P : parts)
    for (int F = 1; F <= 8; F *= 2) {
      const int smax = F > 1 ? pa::kSplitItems / F : 0;
      for (int S = 0; S <= smax + 2; ++S)
        for (int own = 0; own <= 5 * P + 3; own += (own < 3 * P ? 37 : 1)) {
          const int s = S < smax ? S : smax;   // the plan caps S at split_max
          const pa::DecodeCut cut(own, P, F, s);
          const int npc = (own + P - 1) / P;
          CHECK(cut.n <= npc + smax * (F - 1));
          CHECK(F > 1 || cut.n == npc);
          CHECK(cut.ps == (F > 1 ? (npc > s ? npc - s : 0) : npc));
          if (own == 0) {
            CHECK(cut.n == 0);
            continue;
          }
          CHECK(cut.start(0) == 0);
          for (int j = 0; j + 1 < cut.n; ++j) CHECK(cut.start(j + 1) == cut.start(j) + cut.len(j));
          CHECK(cut.start(cut.n - 1) < own && cut.start(cut.n - 1) + cut.len(cut.n - 1) >= own);
          for (int j = 0; j < cut.n; ++j) {
            CHECK(cut.len(j) == (j < cut.ps ? P : P / F));
            const int end = cut.start(j) + cut.len(j) < own ? cut.start(j) + cut.len(j) : own;
            CHECK(cut.item_of(cut.start(j)) == j && cut.item_of(end - 1) == j);
          }
          CHECK(cut.item_of(own - 1) == cut.n - 1);
        }
    }
}

int main() {
  argument_errors();
  valid_calls();
  random_sizes();
  decode_cut();
  if (g_fail) {
    fprintf(stderr, "host_check: %d checks failed\n", g_fail);
    return 1;
  }
  printf("host_check: all checks passed\n");
  return 0;
}

// pa_metadata.hip -- step inputs built on the GPU from persistent request
// state (llm-wiki "vLLM 0.25 Model Runner V2"):
//  * the block table lives on the GPU, indexed by a request's persistent
//    slot; the host sends only the changes, as (row, start, values) runs
//    packed into one small buffer, and one kernel applies them
//    ("Redesign 3");
//  * a step names its requests by persistent slot through idx_mapping; the
//    GPU gathers their block-table rows and builds query_start_loc (the
//    prefix sum of the scheduled token counts), seq_lens, each token's
//    position and its cache slot ("Redesign 1", "Redesign 4").
#include "pa_device.h"

namespace pa {

// One workgroup per staged run k: its row, start and value range are
// wave-uniform loads (a staging buffer in page-locked host memory costs one
// round trip for them, then one coalesced read of the values).  Runs whose
// row or start fall outside the table are skipped; values past the width
// are dropped.
__global__ __launch_bounds__(256) void table_writes_kernel(TableWriteArgs a) {
  const int k = blockIdx.x;
  const int row = a.rows[k];
  const int start = a.starts[k];
  const int v0 = a.offsets[k];
  const int v1 = a.offsets[k + 1];
  if (row < 0 || row >= a.max_reqs || start < 0 || v1 <= v0) return;
  int32_t* dst = a.table + static_cast<int64_t>(row) * a.max_blocks;
  for (int j = threadIdx.x; j < v1 - v0; j += 256)
    if (start + j < a.max_blocks) dst[start + j] = a.values[v0 + j];
}

// Workgroup 0 builds query_start_loc and seq_lens (a scan over the scheduled
// token counts, 1024 requests per pass) and then each query token's position
// and cache slot, finding the token's request by binary search in the scan,
// which it keeps in LDS for up to kScanLds requests (beyond that, in global
// memory).  The other workgroups copy the step's block-table rows, one int32
// per thread.  A token past the scheduled total, or whose block is past the
// table's width, or whose batch position names a slot outside the table,
// gets position -1 and slot -1 (a skipped cache write).
constexpr int kScanLds = 4096;

__global__ __launch_bounds__(1024) void step_inputs_kernel(StepArgs a) {
  if (blockIdx.x > 0) {
    const int64_t e = (static_cast<int64_t>(blockIdx.x) - 1) * 1024 + threadIdx.x;
    if (e >= static_cast<int64_t>(a.num_reqs) * a.max_blocks) return;
    const int b = static_cast<int>(e / a.max_blocks);
    const int col = static_cast<int>(e - static_cast<int64_t>(b) * a.max_blocks);
    const int slot = a.idx_mapping[b];
    a.step_tables[e] = (slot >= 0 && slot < a.max_reqs) ? a.table[static_cast<int64_t>(slot) * a.max_blocks + col]
                                                         : 0;
    return;
  }
  __shared__ int scan[1024];
  __shared__ int qs[kScanLds + 1];
  __shared__ int carry;
  const int tid = threadIdx.x;
  const bool in_lds = a.num_reqs <= kScanLds;
  if (tid == 0) {
    carry = 0;
    a.qsl[0] = 0;
    qs[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < a.num_reqs; base += 1024) {
    const int b = base + tid;
    int n = 0;
    if (b < a.num_reqs) {
      n = a.num_scheduled[b];
      const int slot = a.idx_mapping[b];
      const int done = (slot >= 0 && slot < a.max_reqs) ? a.num_computed[slot] : 0;
      a.seq_lens[b] = done + n;
    }
    scan[tid] = n;
    __syncthreads();
    for (int ofs = 1; ofs < 1024; ofs <<= 1) {            // inclusive Hillis-Steele scan
      const int x = tid >= ofs ? scan[tid - ofs] : 0;
      __syncthreads();
      scan[tid] += x;
      __syncthreads();
    }
    if (b < a.num_reqs) {
      a.qsl[b + 1] = carry + scan[tid];
      if (in_lds) qs[b + 1] = carry + scan[tid];
    }
    __syncthreads();
    if (tid == 1023) carry += scan[1023];
    __syncthreads();
  }
  if (!in_lds) __threadfence_block();                     // the global scan is read back below
  for (int t = tid; t < a.num_tokens; t += 1024) {
    int lo = 0, hi = a.num_reqs - 1;                      // last b with qsl[b] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((in_lds ? qs[mid] : a.qsl[mid]) <= t) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int q0 = in_lds ? qs[b] : a.qsl[b];
    const int q1 = in_lds ? qs[b + 1] : a.qsl[b + 1];
    int64_t pos = -1, slot_out = -1;
    const int slot = a.idx_mapping[b];
    if (t < q1 && slot >= 0 && slot < a.max_reqs) {
      pos = static_cast<int64_t>(a.num_computed[slot]) + (t - q0);
      const int64_t j = pos / a.block_size;
      if (j < a.max_blocks)
        slot_out = static_cast<int64_t>(a.table[static_cast<int64_t>(slot) * a.max_blocks + j]) * a.block_size +
                   pos % a.block_size;
      else
        pos = -1;
    }
    a.positions[t] = pos;
    a.slot_mapping[t] = slot_out;
  }
}

// num_computed[idx_mapping[b]] += num_scheduled[b]: the step's tokens are now
// cached (one thread per batch position; slots outside the table skipped).
__global__ __launch_bounds__(256) void commit_step_kernel(CommitArgs a) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= a.num_reqs) return;
  const int slot = a.idx_mapping[b];
  if (slot >= 0 && slot < a.max_reqs) a.num_computed[slot] += a.num_scheduled[b];
}

hipError_t launch_commit_step(const CommitArgs& a, hipStream_t stream) {
  if (a.num_reqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(commit_step_kernel, dim3(static_cast<unsigned>((a.num_reqs + 255) / 256)), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_table_writes(const TableWriteArgs& a, hipStream_t stream) {
  if (a.num_values <= 0 || a.num_writes <= 0) return hipSuccess;
  hipLaunchKernelGGL(table_writes_kernel, dim3(static_cast<unsigned>(a.num_writes)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prepare_step(const StepArgs& a, hipStream_t stream) {
  if (a.num_reqs <= 0) return hipSuccess;
  const int64_t gather = (static_cast<int64_t>(a.num_reqs) * a.max_blocks + 1023) / 1024;
  hipLaunchKernelGGL(step_inputs_kernel, dim3(static_cast<unsigned>(1 + gather)), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa

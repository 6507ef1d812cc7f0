// pa_attention.hip -- one attention step: the work-list kernel, the decode
// and chunk kernels (pa_decode.hip, pa_chunk.hip), and the log-sum-exp merge
// of split-context partials.
#include "pa_device.h"

namespace pa {

// One workgroup.  For each sequence with q_len > 0 it counts work items --
// decode: ceil(rows/16) row tiles x ceil(L/P) partitions (P = 512 or 1024); chunk:
// ceil(rows/256) row blocks x ceil(L/4096) partitions -- takes exclusive
// prefix sums and appends the items in (tile, partition) order to the two
// lists.  It also resets the work counters the attention kernels draw from.
__global__ __launch_bounds__(1024) void plan_kernel(AttnArgs a) {
  __shared__ int32_t scan[2][1024];
  __shared__ int64_t carry[2];
  const int tid = threadIdx.x;
  if (tid < 2) carry[tid] = 0;
  __syncthreads();
  for (int base = 0; base < a.num_seqs; base += 1024) {
    const int i = base + tid;
    int n[2] = {0, 0}, parts[2] = {1, 1};
    if (i < a.num_seqs) {
      const int L = a.seq_lens[i];
      const int ql = a.qsl[i + 1] - a.qsl[i];
      const int rows = ql * a.group;
      if (ql > 0 && L > 0) {
        if (is_chunk_seq(a, rows)) {
          parts[1] = (L + kChunkPartition - 1) / kChunkPartition;
          n[1] = ((rows + kChunkRows - 1) / kChunkRows) * parts[1];
        } else {
          parts[0] = (L + a.partition - 1) / a.partition;
          n[0] = ((rows + kTileRows - 1) / kTileRows) * parts[0];
        }
      }
    }
    scan[0][tid] = n[0];
    scan[1][tid] = n[1];
    __syncthreads();
    for (int ofs = 1; ofs < 1024; ofs <<= 1) {   // inclusive Hillis-Steele scans
      const int v0 = tid >= ofs ? scan[0][tid - ofs] : 0;
      const int v1 = tid >= ofs ? scan[1][tid - ofs] : 0;
      __syncthreads();
      scan[0][tid] += v0;
      scan[1][tid] += v1;
      __syncthreads();
    }
#pragma unroll
    for (int list = 0; list < 2; ++list) {
      int32_t* out = list ? a.citems : a.items;
      const int64_t cap = list ? a.max_citems : a.max_items;
      const int64_t start = carry[list] + scan[list][tid] - n[list];
      for (int k = 0; k < n[list]; ++k) {
        const int64_t pos = start + k;
        if (pos >= cap) break;              // only with metadata beyond the host bounds
        const int tile = k / parts[list];
        const int part = k - tile * parts[list];
        out[2 * pos] = i;
        out[2 * pos + 1] = (tile << 16) | part;
      }
    }
    __syncthreads();
    if (tid == 1023) {
      carry[0] += scan[0][1023];
      carry[1] += scan[1][1023];
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.header[0] = 0;
    a.header[1] = static_cast<int32_t>(carry[0] < a.max_items ? carry[0] : a.max_items);
    a.header[2] = 0;
    a.header[3] = static_cast<int32_t>(carry[1] < a.max_citems ? carry[1] : a.max_citems);
  }
}

// One workgroup per (token, q head); rows whose keys fit one partition were
// written by the attention kernel and are skipped here.
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p
template <int OT, int D>
__global__ __launch_bounds__(64) void reduce_kernel(AttnArgs a) {
  const int token = blockIdx.x;
  const int head = blockIdx.y;
  // sequence of this token: last i with qsl[i] <= token
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (uniform(a.qsl[mid]) <= token) lo = mid; else hi = mid - 1;
  }
  const int i = lo;
  const int q0 = a.qsl[i];
  const int ql = a.qsl[i + 1] - q0;
  const int row_pos = a.seq_lens[i] - ql + (token - q0);
  const int np = row_pos / (is_chunk_seq(a, ql * a.group) ? kChunkPartition : a.partition) + 1;
  if (np <= 1) return;
  const int64_t row = (static_cast<int64_t>(token) * a.num_q_heads + head) * a.max_parts;
  float M = -__builtin_inff();
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.part_m[row + p]);
  float den = 0.f;
  constexpr int PER = D / 64;
  float num[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) num[k] = 0.f;
  for (int p = 0; p < np; ++p) {
    const float wgt = __builtin_amdgcn_exp2f(a.part_m[row + p] - M);
    den += wgt * a.part_l[row + p];
    const float* ap = a.part_acc + (row + p) * D;
#pragma unroll
    for (int k = 0; k < PER; ++k) num[k] += wgt * ap[threadIdx.x + 64 * k];
  }
  constexpr int EBO = Bytes<OT>::v;
  uint8_t* op = static_cast<uint8_t*>(a.out) + ((static_cast<int64_t>(token) * a.num_q_heads + head) * D) * EBO;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const float v = num[k] / den;
    const int dd = threadIdx.x + 64 * k;
    if constexpr (OT == DT_F32) reinterpret_cast<float*>(op)[dd] = v;
    else if constexpr (OT == DT_BF16) reinterpret_cast<uint16_t*>(op)[dd] = static_cast<uint16_t>(f32_to_bf16(v));
    else reinterpret_cast<uint16_t*>(op)[dd] = static_cast<uint16_t>(f32_to_f16(v));
  }
}

// plan -> decode kernel -> chunk kernel (when a prompt chunk can be present)
// -> partition merge.  ev[0..1] bracket the decode kernel, ev[2..3] the chunk
// kernel (each may be null).
hipError_t launch_attention(int q, int kv, int d, int bs, const AttnArgs& a, hipStream_t stream,
                            const hipEvent_t* ev) {
  // the pairing and shape must exist before anything is enqueued
  hipError_t e = dispatch_attention(q, kv, d, bs, [](auto, auto, auto, auto) { return hipSuccess; });
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev[0] && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
  if ((e = launch_decode(q, kv, d, bs, a, stream)) != hipSuccess) return e;
  if (ev[1] && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
  if (q != DT_F32 && a.chunk_path && static_cast<int64_t>(a.max_query_len) * a.group >= kChunkMinRows) {
    if (ev[2] && (e = hipEventRecord(ev[2], stream)) != hipSuccess) return e;
    if ((e = launch_chunk(q, kv, d, bs, a, stream)) != hipSuccess) return e;
    if (ev[3] && (e = hipEventRecord(ev[3], stream)) != hipSuccess) return e;
  }
  if (a.max_parts > 1 && a.num_tokens > 0) {
    const dim3 grid(a.num_tokens, a.num_q_heads);
    if (q == DT_F32) {
      if (d == 64) hipLaunchKernelGGL((reduce_kernel<DT_F32, 64>), grid, dim3(64), 0, stream, a);
      else hipLaunchKernelGGL((reduce_kernel<DT_F32, 128>), grid, dim3(64), 0, stream, a);
    } else if (q == DT_F16) {
      if (d == 64) hipLaunchKernelGGL((reduce_kernel<DT_F16, 64>), grid, dim3(64), 0, stream, a);
      else hipLaunchKernelGGL((reduce_kernel<DT_F16, 128>), grid, dim3(64), 0, stream, a);
    } else {
      if (d == 64) hipLaunchKernelGGL((reduce_kernel<DT_BF16, 64>), grid, dim3(64), 0, stream, a);
      else hipLaunchKernelGGL((reduce_kernel<DT_BF16, 128>), grid, dim3(64), 0, stream, a);
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace pa

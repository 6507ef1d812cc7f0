// pa_attention.hip -- one attention step: the work-list kernel, the decode
// and chunk kernels (pa_decode.hip, pa_chunk.hip), and the log-sum-exp merge
// of split-context partials.
#include "pa_device.h"

namespace pa {

// Keys a work item visits (its partition clipped to the sequence and to the
// causal reach of its last row), in units of the kernel's key step; 0 for an
// item with nothing to do.  Must agree with the kernels' own bounds.
__device__ __forceinline__ int item_size(int L, int ql, int G, int row0, int nrows, int part, int P,
                                         int step) {
  const int rows = ql * G;
  const int last = min(rows, row0 + nrows) - 1;
  const int max_pos = L - ql + last / G;
  const int kstart = part * P;
  const int kend = min(min(L, kstart + P), max_pos + 1);
  return kend > kstart ? (kend - kstart + step - 1) / step : 0;
}

// One workgroup builds both work lists -- decode: (sequence, 16-row tile,
// partition of a.partition keys); chunk: (sequence, 256-row block, partition
// of 4096 keys) -- longest item first: items are bucketed by the number of
// key steps they visit (32 keys for decode, 64 for chunks) and the buckets
// are laid out in descending order, so the persistent kernels, which take
// items in list order, start the long ones first and end on short ones.
// Order within a bucket is arbitrary; no result depends on it.  It also
// resets the work counters the attention kernels draw from.
__global__ __launch_bounds__(1024) void plan_kernel(AttnArgs a) {
  constexpr int NB0 = kPartitionLong / 32 + 1;           // decode buckets: 0 .. 32 steps
  constexpr int NB1 = kChunkPartition / kChunkKeys + 1;   // chunk buckets: 0 .. 64 tiles
  __shared__ int hist0[NB0], hist1[NB1];
  __shared__ int total[2];
  const int tid = threadIdx.x;
  const int G = a.group;
  for (int b = tid; b < NB0; b += 1024) hist0[b] = 0;
  for (int b = tid; b < NB1; b += 1024) hist1[b] = 0;
  __syncthreads();

  // visit(list, i, tile, part, bucket) for every item of sequence i
  auto items_of = [&](int i, auto&& visit) {
    const int L = a.seq_lens[i];
    const int ql = a.qsl[i + 1] - a.qsl[i];
    const int rows = ql * G;
    if (ql <= 0 || L <= 0) return;
    if (is_chunk_seq(a, rows)) {
      const int np = (L + kChunkPartition - 1) / kChunkPartition;
      const int nt = (rows + kChunkRows - 1) / kChunkRows;
      for (int t = 0; t < nt; ++t)
        for (int p = 0; p < np; ++p)
          visit(1, t, p, item_size(L, ql, G, t * kChunkRows, kChunkRows, p, kChunkPartition, kChunkKeys));
    } else {
      const int np = (L + a.partition - 1) / a.partition;
      const int nt = (rows + kTileRows - 1) / kTileRows;
      for (int t = 0; t < nt; ++t)
        for (int p = 0; p < np; ++p)
          visit(0, t, p, item_size(L, ql, G, t * kTileRows, kTileRows, p, a.partition, 32));
    }
  };

  // pass 1: bucket sizes
  for (int i = tid; i < a.num_seqs; i += 1024)
    items_of(i, [&](int list, int, int, int bucket) { atomicAdd(list ? &hist1[bucket] : &hist0[bucket], 1); });
  __syncthreads();
  // bucket starts, longest bucket first
  if (tid < 2) {
    int* hist = tid ? hist1 : hist0;
    const int nb = tid ? NB1 : NB0;
    int run = 0;
    for (int b = nb - 1; b >= 0; --b) {
      const int c = hist[b];
      hist[b] = run;
      run += c;
    }
    total[tid] = run;
  }
  __syncthreads();
  // pass 2: place every item in its bucket
  for (int i = tid; i < a.num_seqs; i += 1024)
    items_of(i, [&](int list, int t, int p, int bucket) {
      const int pos = atomicAdd(list ? &hist1[bucket] : &hist0[bucket], 1);
      if (pos >= (list ? a.max_citems : a.max_items)) return;   // only with metadata beyond the host bounds
      int32_t* out = list ? a.citems : a.items;
      out[2 * pos] = i;
      out[2 * pos + 1] = (t << 16) | p;
    });
  if (tid == 0) {
    a.header[0] = 0;
    a.header[1] = static_cast<int32_t>(total[0] < a.max_items ? total[0] : a.max_items);
    a.header[2] = 0;
    a.header[3] = static_cast<int32_t>(total[1] < a.max_citems ? total[1] : a.max_citems);
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

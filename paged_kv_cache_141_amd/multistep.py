"""Several decode steps as one device-resident loop, capturable in a HIP graph.

Each step: ``prepare_step`` (step inputs from the persistent per-slot state)
-> ``write_and_attend`` (the step's new K/V written in the launch that
builds its work lists, then attention) -> ``commit_step`` (the tokens are
cached: num_computed advances).  Nothing in
the loop allocates, synchronises or needs the host, so the whole sequence of
launches can be captured once and replayed (techknowgenie "vLLM V1 core
refactoring", section on the PagedAttention V3 kernel architecture: a GPU
graph runner executes N decode steps on its own instead of the host
scheduler synchronising at every token).  The blocks the N steps fill must
already be in the block table.
"""

from __future__ import annotations

import paged_kv_cache_141_amd as pa


class DecodeLoop:
    """N decode steps of a fixed batch.

    block_table  int32 [max_reqs, max_blocks] (device), by persistent slot;
    num_computed int32 [max_reqs] (device), advanced by each step;
    idx_mapping  int32 [R] (device): the batch's persistent slots;
    q            [N, R, Hq, d]; key, value [N, R, Hkv, d] (device): per-step
                 inputs, in the dtypes pa.write_and_attend takes;
    max_seq_len  host bound on the context length at the last step.
    ``out[s]`` holds step s's attention output after ``run()`` (or a replay).
    """

    def __init__(self, k_cache, v_cache, block_table, num_computed, idx_mapping, q, key, value,
                 block_size: int, scale: float, max_seq_len: int, k_scale: float = 1.0, v_scale: float = 1.0):
        import ctypes
        import torch
        self.k_cache, self.v_cache, self.table = k_cache, v_cache, block_table
        self.num_computed, self.idx = num_computed, idx_mapping
        self.q, self.key, self.value = q, key, value
        self.N, self.R = q.shape[0], idx_mapping.numel()
        self.B, self.scale, self.max_seq_len = block_size, scale, max_seq_len
        self.k_scale, self.v_scale = k_scale, v_scale
        dev = q.device
        R, W = self.R, block_table.shape[1]
        self.sched = torch.ones(R, dtype=torch.int32, device=dev)
        self.meta = (torch.empty(R + 1, dtype=torch.int32, device=dev), torch.empty(R, dtype=torch.int32, device=dev),
                     torch.empty(R, dtype=torch.int64, device=dev), torch.empty(R, dtype=torch.int64, device=dev),
                     torch.empty(R, W, dtype=torch.int32, device=dev))
        self.out = torch.empty_like(q)
        spec = pa.cache_spec(k_cache, v_cache, k_scale, v_scale)
        need = ctypes.c_size_t(0)
        st = pa.library().pa_attention_workspace_size(ctypes.byref(spec), q.shape[2], R, R, max_seq_len, 1,
                                                      ctypes.byref(need))
        if st != 0:
            raise pa.PagedAttentionError(st, "pa_attention_workspace_size")
        self.workspace = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=dev)

    def step(self, s: int, stream=None):
        qsl, lens, _, slots, tables = pa.prepare_step(self.table, self.idx, self.num_computed, self.sched, self.R,
                                                      self.B, out=self.meta, stream=stream)
        pa.write_and_attend(self.key[s], self.value[s], slots, self.q[s], self.k_cache, self.v_cache, tables, lens,
                            qsl, self.scale, max_seq_len=self.max_seq_len, max_query_len=1, out=self.out[s],
                            workspace=self.workspace, k_scale=self.k_scale, v_scale=self.v_scale, stream=stream)
        pa.commit_step(self.num_computed, self.idx, self.sched, stream=stream)

    def run(self, stream=None):
        """Enqueue the N steps on the stream (the current one by default)."""
        for s in range(self.N):
            self.step(s, stream)
        return self.out

    def capture(self):
        """Record the N steps once into a graph; ``graph.replay()`` reruns them
        from whatever num_computed and cache the device holds then.

        The context bound and the workspace are fixed here: a replay is
        correct only while every context it reaches stays within
        ``max_seq_len``, e.g. when each replay starts from the captured state
        (restore num_computed first), or when max_seq_len was sized for all
        the replays.  A context past the bound is attended over its first
        max_seq_len keys only -- a wrong row, never an access outside the
        buffers."""
        import torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):      # captures on torch's capture stream, the current one inside
            self.run()
        return g

"""Benchmark one step of the paged-attention hot path on one MI355X.

A step is the whole path over one batch: the cache write of the step's new
tokens (pa_reshape_and_cache) followed by paged attention (pa_attention: the
work-list, attention and partition-merge kernels).  Inputs are seeded,
synthetic and resident in HBM before timing starts.

Default workload: the LLaMA-7B-shaped decode step (256 sequences, 32 q = 32 kv
heads, d = 128, bf16 KV, block size 16, contexts uniform in [128, 2048]).

Prints one JSON line: value = KV GB/s of the whole step (the KV bytes the
method must read, over the step's wall time); `roofline` prices the
attention kernel alone (timed with HIP events recorded on its own launch
stream around that one kernel) against 8 TB/s; `cpu_baseline` times the
fp64 CPU oracle on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn KV GB/s (% of HBM peak) + query tokens/s per step, 1×MI355X"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="llama7b_decode",
                    choices=["tiny_decode", "llama7b_decode", "gqa_long_decode", "mixed_chunked_prefill",
                             "fp8_shared_prefix"])
    ap.add_argument("--block-size", type=int, default=None, choices=[16, 32, 64], help="tokens per cache block")
    ap.add_argument("--kv-dtype", default=None, choices=["bf16", "f16", "fp8_e4m3"],
                    help="cache dtype override (fp8_e4m3: per-tensor scale 2^-5)")
    ap.add_argument("--head-dim", type=int, default=None, choices=[64, 128, 256],
                    help="for gqa_long_decode / mixed_chunked_prefill: 256 keeps the KV bytes per token "
                         "with half the heads (16q/4kv)")
    ap.add_argument("--placement", default=None, help="shuffled | identity | private")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the step: copy a MIB-mebibyte device buffer --steps times "
                         "(the known-size reference for HBM counter scaling)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the oracle's timed sample (0 disables it)")
    ap.add_argument("--op", default="step", choices=["step", "copy_blocks", "swap", "prepare", "multistep"],
                    help="step: the attention step (default).  copy_blocks: copy-on-write of "
                         "--pairs blocks within one pool.  swap: --pairs blocks out to page-locked "
                         "host memory and back in.  Both use the pool geometry of --config.  prepare: "
                         "the step inputs of --config built on the GPU from 1,024 persistent request "
                         "slots (staged block-table writes + pa_prepare_step).  multistep: --graph-steps "
                         "decode steps of --config (prepare, cache write, attention, commit per step) run "
                         "eagerly and replayed from one captured HIP graph.")
    ap.add_argument("--graph-steps", type=int, default=8, help="decode steps per graph for --op multistep")
    ap.add_argument("--pairs", type=int, default=2048, help="block pairs per copy for --op")
    ap.add_argument("--no-configs", action="store_true",
                    help="default run only: skip the records of the other configurations")
    ap.add_argument("--config-cpu-seconds", type=float, default=3.0,
                    help="oracle budget for each of the other configurations' records (0 disables it)")
    ap.add_argument("--separate-write", action="store_true",
                    help="time the step as pa_reshape_and_cache + pa_attention[_shared_prefix] instead of "
                         "pa_write_and_attend")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="attend through pa_attention_shared_prefix over the workload's common prefix "
                         "(fp8_shared_prefix): the prefix is attended once for all rows")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t pairs from the HIP runtime torch loaded (the one the library uses).

    The events only time work: they are read after a full device
    synchronize, so they are created without the system-scope fence that a
    default event performs when it is recorded (a cache writeback and
    invalidate, which costs the step it brackets several microseconds)."""

    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence

    def __init__(self, fence=False):
        import torch
        lib = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.hip = ctypes.CDLL(lib if os.path.exists(lib) else "libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.flags = 0 if fence else self.DISABLE_SYSTEM_FENCE

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.flags) == 0
        return ev.value

    def record(self, e, stream):
        """Record event e on a torch stream."""
        assert self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream.cuda_stream)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(ctypes.c_void_p(e))


# the files each kernel is compiled from, beside the shared device headers
KERNEL_SOURCES = {"attn_kernel": ("pa_decode.hip", "pa_decode_item.h"),
                  "chunk_kernel": ("pa_chunk.hip", "pa_chunk_item.h"),
                  "step_kernel": ("pa_step.hip", "pa_decode_item.h", "pa_chunk_item.h")}


def _code_only(text):
    """C++ source without its comments and blank space: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(kernel):
    """Hash of the code one kernel is compiled from (its own file plus the
    shared device headers, comments left out): counter runs stay valid until
    that code changes."""
    h = hashlib.sha256()
    for f in (*KERNEL_SOURCES[kernel], "pa_device.h", "pa_codec.h", "pa_internal.h"):
        h.update(_code_only(open(os.path.join(ROOT, "paged_kv_cache_141_amd", "csrc", f)).read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload_name, kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload_name}_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s):
    """Time the oracle (cache write of the new tokens + attention) sequence by
    sequence on a seeded random sample until ~budget_s of timed work."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from workloads import accounting

    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    cores = max([p.get("num_threads", 1) for p in blas] or [1])
    kp, vp = w.initial_pool()
    oracle.attention.validate_metadata(w.seq_lens, w.query_start_loc, w.block_tables,
                                       w.num_blocks, w.block_size)
    q = w.q_values()
    order = np.random.default_rng([w.seed, 99]).permutation(w.num_seqs)
    timed, kv_bytes, toks, n = 0.0, 0, 0, 0
    eb = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}[w.kv_dtype]
    per_tok = w.num_kv_heads * 2 * w.head_dim * eb
    if w.shared_prefix_len and w.prefix_blocks_shared:
        for kind, i, k, v, s in w.iter_token_writes([int(order[0])]):
            if i == -1:
                oracle.cache.reshape_and_cache(kp, vp, k, v, w.src_dtype, w.kv_dtype, s,
                                               w.block_size, w.k_scale, w.v_scale)
    for i in order:
        i = int(i)
        writes = [x for x in w.iter_token_writes([i]) if x[1] == i]
        for kind, _, k, v, s in writes:           # prior context: setup, untimed
            if kind == "prior":
                oracle.cache.reshape_and_cache(kp, vp, k, v, w.src_dtype, w.kv_dtype, s,
                                               w.block_size, w.k_scale, w.v_scale)
        t0 = time.perf_counter()
        for kind, _, k, v, s in writes:
            if kind == "new":
                oracle.cache.reshape_and_cache(kp, vp, k, v, w.src_dtype, w.kv_dtype, s,
                                               w.block_size, w.k_scale, w.v_scale)
        oracle.attention.paged_attention(q, w.q_dtype, kp, vp, w.kv_dtype, w.block_tables,
                                         w.seq_lens, w.query_start_loc, w.block_size, w.scale,
                                         w.k_scale, w.v_scale, seqs=[i], validate=False)
        timed += time.perf_counter() - t0
        kv_bytes += int(w.seq_lens[i]) * per_tok
        toks += int(w.query_lens[i])
        n += 1
        if timed >= budget_s:
            break
    return {
        "value": round(kv_bytes / timed / 1e9, 4), "unit": "GB/s", "cores": int(cores),
        "kind": "oracle",
        "query_tokens_per_s": round(toks / timed, 2),
        "seconds": round(timed, 2),
        "sample": f"{n} of {w.num_seqs} sequences (seeded random order), {toks} query tokens, "
                  f"{kv_bytes / 1e9:.3f} GB of KV; fp64 NumPy oracle, cache write of the new "
                  f"tokens + attention, prior-context cache fill untimed",
    }


def bench_block_copies(args):
    """Whole-block copies in the pool geometry of --config: copy-on-write of
    --pairs blocks within a device pool (HBM: each pair reads and writes one K
    and one V block), or a swap of --pairs blocks out to a page-locked host pool
    and back (each direction moves one K and one V block per pair across the
    host link).  Timed with events on the current stream."""
    import numpy as np
    import torch

    import workloads
    import paged_kv_cache_141_amd as pa

    w = workloads.make(args.config)
    eb = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}[w.kv_dtype]
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}[w.kv_dtype]
    H, B, d, n = w.num_kv_heads, w.block_size, w.head_dim, args.pairs
    block_bytes = H * B * d * eb
    nblocks = 2 * n + 1
    gen = torch.Generator(device="cuda").manual_seed(141)
    kd = torch.randint(0, 127, (nblocks, H, B, d), dtype=torch.int8, device="cuda", generator=gen)
    vd = torch.randint(0, 127, (nblocks, H, B, d), dtype=torch.int8, device="cuda", generator=gen)
    kd = kd.view(torch.uint8).view(dt) if eb == 1 else kd.view(torch.uint8).repeat_interleave(eb, -1).view(dt)
    vd = vd.view(torch.uint8).view(dt) if eb == 1 else vd.view(torch.uint8).repeat_interleave(eb, -1).view(dt)
    rng = np.random.default_rng(141)
    perm = rng.permutation(nblocks)
    stream = torch.cuda.current_stream()
    if args.op == "copy_blocks":
        mapping = torch.from_numpy(np.stack([perm[:n], perm[n:2 * n]], 1).astype(np.int64)).cuda()
        run = [lambda: pa.copy_blocks(kd, vd, kd, vd, mapping)]
        moved = 2 * 2 * block_bytes * n          # K and V, read and written
        names, bound, peak = ["copy_blocks"], "hbm", HBM_PEAK_GBS
    else:
        kh = torch.empty((n, H, B, d), dtype=dt, pin_memory=True)
        vh = torch.empty((n, H, B, d), dtype=dt, pin_memory=True)
        out = torch.from_numpy(np.stack([perm[:n], np.arange(n)], 1).astype(np.int64)).cuda()
        back = torch.from_numpy(np.stack([np.arange(n), perm[n:2 * n]], 1).astype(np.int64)).cuda()
        run = [lambda: pa.copy_blocks(kd, vd, kh, vh, out), lambda: pa.copy_blocks(kh, vh, kd, vd, back)]
        moved = 2 * block_bytes * n              # K and V cross the link once per direction
        names, bound, peak = ["swap_out", "swap_in"], "host link", None
        # the link's own rate for contiguous page-locked copies, for scale
        big = torch.empty(n * 2 * block_bytes, dtype=torch.uint8, pin_memory=True)
        dev = torch.empty(n * 2 * block_bytes, dtype=torch.uint8, device="cuda")
    res = {}
    for name, fn in zip(names, run):
        for _ in range(args.warmup):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        res[name] = ms
    line = {"op": args.op, "workload": w.name, "pairs": n, "block_bytes_k_plus_v": 2 * block_bytes,
            "steps": args.steps, "warmup": args.warmup}
    for name in names:
        gbs = moved / (res[name] * 1e-3) / 1e9
        line[name] = {"us": round(res[name] * 1e3, 2), "GBps": round(gbs, 1), "bound": bound,
                      "peak": peak, "frac": round(gbs / peak, 4) if peak else None}
    if args.op == "swap":
        for name, src, dst in (("memcpy_d2h", dev, big), ("memcpy_h2d", big, dev)):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                dst.copy_(src, non_blocking=True)
            torch.cuda.synchronize()
            dt_s = (time.perf_counter() - t0) / args.steps
            line[name + "_contiguous_GBps"] = round(big.numel() / dt_s / 1e9, 1)
    print(json.dumps(line), flush=True)


def bench_prepare(args):
    """Step inputs of --config from persistent state: the sequences sit in
    scattered slots of a 1,024-slot table; this step's new blocks (those past
    the blocks of the cached tokens) arrive as staged runs in page-locked host
    memory.  Times the two GPU calls with events, and, for scale, the same
    preparation done with vectorised NumPy on the host plus the upload of the
    whole table that the staged writes avoid."""
    import numpy as np
    import torch

    import workloads
    import paged_kv_cache_141_amd as pa

    w = workloads.make(args.config)
    R, S, B = 1024, w.num_seqs, w.block_size
    W = max(512, w.block_tables.shape[1])
    rng = np.random.default_rng(141)
    slot_of = rng.permutation(R)[:S].astype(np.int32)
    done = np.zeros(R, np.int32)
    done[slot_of] = w.seq_lens - w.query_lens
    table = np.zeros((R, W), np.int32)
    table[slot_of, :w.block_tables.shape[1]] = w.block_tables
    first_new = -(-(w.seq_lens - w.query_lens) // B)          # blocks already holding cached tokens
    last = -(-w.seq_lens // B)
    runs = [(int(slot_of[i]), int(first_new[i]), w.block_tables[i, first_new[i]:last[i]]) for i in range(S)
            if last[i] > first_new[i]]
    rows = torch.tensor([r[0] for r in runs], dtype=torch.int32).pin_memory()
    starts = torch.tensor([r[1] for r in runs], dtype=torch.int32).pin_memory()
    offs = torch.from_numpy(np.concatenate([[0], np.cumsum([len(r[2]) for r in runs])]).astype(np.int32)).pin_memory()
    vals = torch.from_numpy(np.concatenate([r[2] for r in runs]).astype(np.int32)).pin_memory()
    g_table = torch.from_numpy(table).cuda()
    g_idx = torch.from_numpy(slot_of).cuda()
    g_done = torch.from_numpy(done).cuda()
    g_sched = torch.from_numpy(w.query_lens.astype(np.int32)).cuda()
    stream = torch.cuda.current_stream()

    def gpu():
        pa.apply_block_table_writes(g_table, rows, starts, offs, vals)
        return pa.prepare_step(g_table, g_idx, g_done, g_sched, w.num_tokens, B)

    for _ in range(args.warmup):
        gpu()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        gpu()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    gpu_us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3

    def host():
        sched = w.query_lens.astype(np.int64)
        qsl = np.concatenate([[0], np.cumsum(sched)])
        base = done[slot_of].astype(np.int64)
        lens = base + sched
        tok_req = np.repeat(np.arange(S), sched)
        pos = base[tok_req] + (np.arange(w.num_tokens) - qsl[tok_req])
        slots = table[slot_of[tok_req], pos // B].astype(np.int64) * B + pos % B
        return qsl, lens, pos, slots, table[slot_of]

    for _ in range(3):
        host()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        host()
    host_us = (time.perf_counter() - t0) / args.steps * 1e6
    full = torch.from_numpy(table).pin_memory()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g_table.copy_(full, non_blocking=True)
    torch.cuda.synchronize()
    upload_us = (time.perf_counter() - t0) / args.steps * 1e6
    print(json.dumps({"op": "prepare", "workload": w.name, "persistent_slots": R, "table_width": W,
                      "requests": S, "tokens": w.num_tokens, "staged_runs": len(runs), "staged_values": int(vals.numel()),
                      "gpu_us": round(gpu_us, 2), "gpu_wall_us_per_step": round(wall * 1e6, 2), "bound": "latency",
                      "host_numpy_us": round(host_us, 2), "full_table_upload_us": round(upload_us, 2),
                      "full_table_bytes": int(table.nbytes)}), flush=True)


def bench_multistep(args):
    """Per-step time of --graph-steps decode steps of --config's batch: each
    step prepares its inputs from the per-slot state on the GPU, writes one
    new token per sequence, attends and commits.  Eager launches vs one
    replay of the captured graph (the state is restored before each run)."""
    import numpy as np
    import torch

    import workloads
    from workloads import device as wd
    from paged_kv_cache_141_amd.multistep import DecodeLoop

    w = workloads.make(args.config)
    N, R, B = args.graph_steps, w.num_seqs, w.block_size
    step = wd.stage(w, write_new=False)                     # context before the new token of each sequence
    W = w.block_tables.shape[1] + -(-N // B) + 1
    table = torch.full((R, W), int(w.spare_block), dtype=torch.int32, device="cuda")
    table[:, :w.block_tables.shape[1]] = torch.from_numpy(w.block_tables).cuda()
    done0 = torch.from_numpy((w.seq_lens - 1).astype(np.int32)).cuda()
    done = done0.clone()
    idx = torch.arange(R, dtype=torch.int32, device="cuda")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.q_dtype]
    sdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.src_dtype]
    gen = torch.Generator(device="cuda").manual_seed(141)
    q = torch.randn(N, R, w.num_q_heads, w.head_dim, device="cuda", generator=gen).to(tdt)
    key = torch.randn(N, R, w.num_kv_heads, w.head_dim, device="cuda", generator=gen).to(sdt)
    value = torch.randn(N, R, w.num_kv_heads, w.head_dim, device="cuda", generator=gen).to(sdt)
    loop = DecodeLoop(step.k_cache, step.v_cache, table, done, idx, q, key, value, B, w.scale,
                      int(w.max_seq_len) + N, w.k_scale, w.v_scale)
    stream = torch.cuda.current_stream()

    def timed(fn):
        ms = []
        for k in range(args.warmup + args.steps):
            done.copy_(done0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            if k >= args.warmup:
                ms.append(a.elapsed_time(b))
        return float(np.mean(ms)) * 1e3 / N

    eager_us = timed(loop.run)
    done.copy_(done0)
    g = loop.capture()
    graph_us = timed(g.replay)
    print(json.dumps({"op": "multistep", "workload": w.name, "graph_steps": N, "seqs": R,
                      "eager_us_per_step": round(eager_us, 2), "graph_us_per_step": round(graph_us, 2),
                      "speedup": round(eager_us / graph_us, 3), "steps": args.steps, "warmup": args.warmup}),
          flush=True)


def host_info():
    """CPU model, BLAS library and host memory of the machine the oracle runs on."""
    import numpy  # noqa: F401  (loads the BLAS that threadpool_info reports)
    from threadpoolctl import threadpool_info
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    ram = None
    try:
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                ram = round(int(line.split()[1]) / 2 ** 20, 1)
                break
    except OSError:
        pass
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    return {"cpu_model": model, "blas": ",".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in blas})),
            "host_ram_GiB": ram, "affinity_cpus": len(os.sched_getaffinity(0))}


def copy_ceiling(steps=10, nbytes=4 << 30):
    """A device-to-device copy of nbytes: the achievable HBM rate (read + write)."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_copied": nbytes, "GBps_read_plus_write": round(2 * nbytes / dt / 1e9, 1),
            "frac_of_peak": round(2 * nbytes / dt / 1e9 / HBM_PEAK_GBS, 4)}


def pct(xs, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(xs), q)), 4)


def measure_step(w, args, prefix=0, cpu_seconds=0.0):
    """Stage workload w, run --warmup untimed steps, then time --steps steps
    (cache write of the new tokens + attention).  Returns one record: wall and
    per-step event times, throughput, the kernel rooflines and, with a budget,
    the oracle's rate on a sample of the same workload."""
    import numpy as np
    import torch

    from workloads import accounting
    from workloads import device as wd
    import paged_kv_cache_141_amd as pa

    print(f"[bench] staging {w.name}: {json.dumps(w.summary())}", file=sys.stderr, flush=True)
    t_stage = time.perf_counter()
    step = wd.stage(w, write_new=False)
    if prefix:
        if not (w.shared_prefix_len and w.prefix_blocks_shared):
            raise SystemExit("--shared-prefix needs a workload whose sequences share prefix blocks")
        step.use_shared_prefix(prefix)
    torch.cuda.synchronize()
    print(f"[bench] staged in {time.perf_counter() - t_stage:.1f}s", file=sys.stderr, flush=True)

    kv_bytes = accounting.workload_kv_bytes(w)
    # the step's HBM share is priced on each physical block once (a prefix
    # whose blocks the tables share is read from HBM once, then from cache)
    step_unique_bytes = accounting.workload_kv_bytes(w, unique=True)
    stream = torch.cuda.current_stream()
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    # the chunk (prefill) kernel runs when a sequence has >= 65 (token, head) rows per kv head
    chunk_rows = w.query_lens.astype(np.int64) * w.group
    is_chunk = (chunk_rows >= 65) & (w.q_dtype != "f32")
    chunk_pairs = [(ev.create(), ev.create()) for _ in range(args.steps)] if is_chunk.any() else None
    prefix_pairs = [(ev.create(), ev.create()) for _ in range(args.steps)] if prefix else None
    whole = (ev.create(), ev.create())
    # A step is the cache write of its new tokens and its attention: one
    # pa_write_and_attend call (the write in the plan's launch), or, with
    # --separate-write, the two calls.
    joint = not args.separate_write
    run = step.bound_step() if joint else None     # the call's arguments marshalled once

    for _ in range(args.warmup):
        if joint:
            run()
        else:
            step.step()
    torch.cuda.synchronize()
    # The timed steps carry the events the kernel rooflines need (the library
    # records them around its kernels) and, with separate calls, a pair around
    # the cache write on every fourth step; each event costs the step a
    # little.  Per-step times are the periods between consecutive attention
    # kernels' starts (each spans one whole step: merge, cache write, plan).
    cw = {} if joint else {k: (ev.create(), ev.create()) for k in range(0, args.steps, 4)}
    t0 = time.perf_counter()
    ev.record(whole[0], stream)
    for k in range(args.steps):
        pa.set_attention_events(pairs[k][0], pairs[k][1])
        if chunk_pairs:
            pa.set_chunk_events(chunk_pairs[k][0], chunk_pairs[k][1])
        if prefix_pairs:
            pa.set_prefix_events(prefix_pairs[k][0], prefix_pairs[k][1])
        if joint:
            run()
            continue
        if k in cw:
            ev.record(cw[k][0], stream)
            step.write_new()
            ev.record(cw[k][1], stream)
        else:
            step.write_new()
        step.attend()
    ev.record(whole[1], stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pa.set_attention_events(None, None)
    pa.set_chunk_events(None, None)
    pa.set_prefix_events(None, None)

    step_s = (t1 - t0) / args.steps
    if args.steps > 1:
        step_ms = [ev.elapsed_ms(pairs[k][0], pairs[k + 1][0]) for k in range(args.steps - 1)]
    else:
        step_ms = [ev.elapsed_ms(whole[0], whole[1])]
    attn_ms = [ev.elapsed_ms(a, b) for a, b in pairs]
    chunk_ms = [ev.elapsed_ms(a, b) for a, b in chunk_pairs] if chunk_pairs else None
    prefix_ms = [ev.elapsed_ms(a, b) for a, b in prefix_pairs] if prefix_pairs else None
    cw_ms = [ev.elapsed_ms(a, b) for a, b in cw.values()]
    for a, b in pairs + list(cw.values()) + (chunk_pairs or []) + (prefix_pairs or []) + [whole]:
        ev.destroy(a), ev.destroy(b)
    attn_s = float(np.mean(attn_ms)) / 1e3
    # the decode kernel reads the KV of the sequences routed to it (all but chunk sequences)
    eb = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}[w.kv_dtype]
    # (with a shared prefix: the keys past it)
    decode_bytes = int(((w.seq_lens.astype(np.int64) - prefix) * ~is_chunk).sum()) * w.num_kv_heads * 2 * w.head_dim * eb
    # Blocks that several sequences' tables share are fetched from HBM once
    # and then served from cache: the HBM roofline prices the unique bytes
    # (the shared prefix once), and the logical bytes are reported beside it.
    unique_bytes = decode_bytes
    if w.shared_prefix_len and w.prefix_blocks_shared and not prefix:
        unique_bytes -= (int((~is_chunk).sum()) - 1) * w.shared_prefix_len * w.num_kv_heads * 2 * w.head_dim * eb
    achieved = unique_bytes / attn_s / 1e9
    # A step with prompt chunks (16-bit q, head dim <= 128) runs its decode and
    # chunk items in one fused launch: both event pairs then bracket that one
    # kernel, and each roofline is what its own work achieved over it.
    fused = bool(chunk_pairs) and w.head_dim <= 128
    main_kernel = "step_kernel" if fused else "attn_kernel"
    name = w.name + ("_cascade" if prefix else "")
    traffic = measured_traffic(name, main_kernel)

    rec = {
        "config": {"workload": name, "seqs": w.num_seqs, "query_tokens": w.num_tokens,
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "kv_dtype": w.kv_dtype, "q_dtype": w.q_dtype,
                   "context_tokens": int(w.seq_lens.sum()), "max_seq_len": w.max_seq_len,
                   "kv_bytes": kv_bytes},
        "ms_per_step": round(step_s * 1e3, 4),
        "ms_step_events": {"median": pct(step_ms, 50), "p10": pct(step_ms, 10), "p90": pct(step_ms, 90)},
        "kv_GBps": round(kv_bytes / step_s / 1e9, 2),
        "query_tokens_per_s": round(w.num_tokens / step_s, 1),
        "hbm_frac_step": round(step_unique_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "step_unique_kv_bytes": step_unique_bytes,
        "fragmentation": round(accounting.fragmentation(w), 5),
        "attention_kernel_us": round(attn_s * 1e6, 2),
        "attention_kernel_us_p10_p90": [round(pct(attn_ms, 10) * 1e3, 2), round(pct(attn_ms, 90) * 1e3, 2)],
        "attention_kernel_kv_bytes": decode_bytes,
        "attention_kernel_unique_kv_bytes": unique_bytes,
        "attention_kernel_logical_GBps": round(decode_bytes / attn_s / 1e9, 2),
        "step_calls": "pa_write_and_attend" if joint else "pa_reshape_and_cache + pa_attention" +
                      ("_shared_prefix" if prefix else ""),
        # with the joint call the write shares the plan's launch and has no time of its own
        "cache_write_us": round(float(np.mean(cw_ms)) * 1e3, 2) if cw_ms else None,
        "roofline": {"bound": "hbm", "kernel": main_kernel, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    if prefix_ms:
        # the prefix pass: every query row against every prefix key
        pflops = 4 * w.head_dim * w.num_q_heads * w.num_tokens * prefix
        tp = float(np.mean(prefix_ms)) / 1e3
        rec["config"]["shared_prefix_tokens"] = prefix
        rec["prefix_pass_us"] = round(tp * 1e6, 2)
        rec["roofline_prefix"] = {"bound": "mfma", "achieved": round(pflops / tp / 1e12, 2), "peak": 2500.0,
                                  "unit": "TFLOP/s", "frac": round(pflops / tp / 1e12 / 2500.0, 4),
                                  "flops": pflops, "prefix_kv_bytes": prefix * w.num_kv_heads * 2 * w.head_dim * eb,
                                  "traffic": measured_traffic(name, "chunk_kernel")}
    if chunk_ms:
        L = w.seq_lens.astype(np.int64)
        c = w.query_lens.astype(np.int64)
        pairs_chunk = int(((c * (L - c) + c * (c + 1) // 2) * is_chunk).sum())
        flops = 4 * w.head_dim * w.num_q_heads * pairs_chunk
        t = float(np.mean(chunk_ms)) / 1e3
        peak = 2500.0   # dense bf16/fp16 MFMA, TFLOP/s
        rec["chunk_kernel_us"] = round(t * 1e6, 2)
        rec["roofline_chunk"] = {"bound": "mfma", "kernel": "step_kernel" if fused else "chunk_kernel",
                                 "achieved": round(flops / t / 1e12, 2), "peak": peak,
                                 "unit": "TFLOP/s", "frac": round(flops / t / 1e12 / peak, 4),
                                 "flops": flops,
                                 "traffic": None if fused else measured_traffic(name, "chunk_kernel")}
        rec["fused_step_kernel"] = fused
        rec["config"]["chunk_tokens"] = int((c * is_chunk).sum())
    if cpu_seconds > 0:
        print(f"[bench] timing the CPU oracle on a sample of {name}", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, cpu_seconds)
    del step
    torch.cuda.empty_cache()
    return rec


# The other configurations, each one record inside the default line: GQA
# long-context decode (head dims 128 and 256), the mixed chunked-prefill step, the fp8 shared-prefix
# step at B = 16/32/64 through the block tables and through the shared-prefix
# (cascade) entry point, its private-copy twin, and the tiny decode step.
OTHER_CONFIGS = [
    ("gqa_long_decode", {}, False),
    ("gqa_long_decode", {"head_dim": 256}, False),
    ("mixed_chunked_prefill", {}, False),
    ("fp8_shared_prefix", {"block_size": 16}, False),
    ("fp8_shared_prefix", {"block_size": 32}, False),
    ("fp8_shared_prefix", {"block_size": 64}, False),
    ("fp8_shared_prefix", {"block_size": 16}, True),
    ("fp8_shared_prefix", {"block_size": 32}, True),
    ("fp8_shared_prefix", {"block_size": 64}, True),
    ("fp8_shared_prefix", {"block_size": 16, "placement": "private"}, False),
    ("tiny_decode", {}, False),
]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each sequence is independent, so the step shards by sequence across GPUs).", file=sys.stderr)
        sys.exit(2)
    if args.op == "prepare":
        return bench_prepare(args)
    if args.op == "multistep":
        return bench_multistep(args)
    if args.op != "step":
        return bench_block_copies(args)
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"calibrate_copy_bytes": n, "us_per_copy": round(dt * 1e6, 2),
                          "copy_GBps_read_plus_write": round(2 * n / dt / 1e9, 1)}), flush=True)
        return

    import workloads

    overrides = bool(args.block_size or args.placement or args.head_dim or args.kv_dtype or args.shared_prefix
                     or args.config != "llama7b_decode")
    kw = {}
    if args.block_size:
        kw["block_size"] = args.block_size
    if args.placement:
        kw["placement"] = args.placement
    if args.head_dim:
        kw["head_dim"] = args.head_dim
    if args.kv_dtype:
        kw["kv_dtype"] = args.kv_dtype
        if args.kv_dtype == "fp8_e4m3":
            kw.update(k_scale=workloads.generate.FP8_SCALE, v_scale=workloads.generate.FP8_SCALE)
    w = workloads.make(args.config, **kw)
    # overrides the configuration's name does not already carry go into it
    # (the measured-traffic records are keyed by workload name)
    if args.kv_dtype and args.config != "fp8_shared_prefix":
        w.name += f"_{args.kv_dtype}"
    if args.block_size and args.config != "fp8_shared_prefix":
        w.name += f"_B{args.block_size}"
    prefix = w.shared_prefix_len if args.shared_prefix else 0
    rec = measure_step(w, args, prefix, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": rec["kv_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": "synthetic",
    }
    line.update(rec)
    if line.get("cpu_baseline"):
        line["cpu_baseline"]["host"] = host_info()
    # the rest of the configurations (default run only), one record each
    if not overrides and not args.no_configs:
        line["copy_ceiling"] = copy_ceiling()
        recs = {}
        for name, ckw, casc in OTHER_CONFIGS:
            cw = workloads.make(name, **ckw)
            r = measure_step(cw, args, cw.shared_prefix_len if casc else 0, args.config_cpu_seconds)
            recs[r["config"]["workload"]] = r
        line["configs"] = recs
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Step inputs from persistent request state (oracle side) -- test infrastructure.

The llm-wiki "vLLM 0.25 Model Runner V2" article:
* "Redesign 1": an active request keeps a fixed persistent slot; a step
  names its requests through idx_mapping ("the first request of this batch
  is persistent slot 7") and the GPU gathers what it needs from those rows;
* "Redesign 3": the block table stays on the GPU; the host records changes
  as (row, start, value) runs, packs them into one staging buffer, and one
  kernel applies them;
* "Redesign 4": query_start_loc is the running sum of the per-request token
  counts, and positions, seq_lens and the slot mapping are built on the GPU.

Readings (the page gives no formulas): a request's persistent state is
num_computed (its tokens already in the cache) and its block-table row; a
step schedules num_scheduled tokens for each batch position; the new tokens
sit at positions num_computed .. num_computed + num_scheduled - 1, so
seq_len = num_computed + num_scheduled; a token's slot is its block id * B
plus its offset in the block (the slot encoding of ``oracle.cache``).  Where
an input leaves a value undefined (a token past the scheduled total, a
block past the table's width, a slot outside the table) the value is -1.
"""

from __future__ import annotations

import numpy as np


def apply_block_table_writes(table: np.ndarray, rows, starts, offsets, values) -> np.ndarray:
    """A new table with every run applied: row rows[k], columns starts[k] ..,
    values values[offsets[k]:offsets[k+1]].  Runs outside the table are skipped."""
    out = np.array(table, dtype=np.int32, copy=True)
    R, W = out.shape
    for k in range(len(rows)):
        r, s = int(rows[k]), int(starts[k])
        vals = np.asarray(values[int(offsets[k]):int(offsets[k + 1])], dtype=np.int32)
        if not (0 <= r < R) or s < 0:
            continue
        n = max(0, min(len(vals), W - s))
        out[r, s:s + n] = vals[:n]
    return out


def prepare_step(table: np.ndarray, idx_mapping, num_computed, num_scheduled, num_tokens: int,
                 block_size: int):
    """(query_start_loc, seq_lens, positions, slot_mapping, step_block_tables) of one step."""
    table = np.asarray(table, dtype=np.int64)
    R, W = table.shape
    idx = np.asarray(idx_mapping, dtype=np.int64)
    done = np.asarray(num_computed, dtype=np.int64)
    sched = np.asarray(num_scheduled, dtype=np.int64)
    qsl = np.zeros(len(idx) + 1, dtype=np.int64)
    seq_lens = np.zeros(len(idx), dtype=np.int64)
    positions = np.full(num_tokens, -1, dtype=np.int64)
    slots = np.full(num_tokens, -1, dtype=np.int64)
    step_tables = np.zeros((len(idx), W), dtype=np.int64)
    for b, s in enumerate(idx):
        ok = 0 <= s < R
        base = int(done[s]) if ok else 0
        qsl[b + 1] = qsl[b] + sched[b]
        seq_lens[b] = base + sched[b]
        if ok:
            step_tables[b] = table[s]
        for i in range(int(sched[b])):
            t = int(qsl[b]) + i
            if t >= num_tokens or not ok:
                continue
            p = base + i
            if p // block_size < W:
                positions[t] = p
                slots[t] = table[s, p // block_size] * block_size + p % block_size
    return (qsl.astype(np.int32), seq_lens.astype(np.int32), positions, slots, step_tables.astype(np.int32))

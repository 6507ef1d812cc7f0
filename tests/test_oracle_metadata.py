"""Pins for the step-input oracle (CPU only).

* the page's own example ("Redesign 1"): the request held in persistent slot
  7 is the first of the batch; its row is gathered, not moved;
* a simulated scheduler kept as plain Python lists of blocks per request
  (requests join, prefill in chunks, decode, finish; a block is taken only
  when the last one fills) -- the staged (row, start, values) writes must
  rebuild exactly those lists in the device-style table, and the step inputs
  must match positions and slots read straight off the lists;
* the seeded workload generator, which builds seq_lens, query_start_loc and
  the slot mapping of a step its own way;
* invariance: which persistent slot a request occupies does not change its
  step inputs.
"""

import numpy as np

import workloads
from oracle import metadata as M

B = 16


def test_page_example_slot_seven_is_first_in_batch():
    table = np.arange(10 * 4, dtype=np.int32).reshape(10, 4) + 100
    done = np.zeros(10, np.int32)
    done[7], done[2] = 20, 5
    qsl, lens, pos, slots, rows = M.prepare_step(table, [7, 2], done, [1, 3], 4, B)
    assert rows[0].tolist() == table[7].tolist() and rows[1].tolist() == table[2].tolist()
    assert qsl.tolist() == [0, 1, 4] and lens.tolist() == [21, 8]
    assert pos.tolist() == [20, 5, 6, 7]
    assert slots.tolist() == [table[7, 1] * B + 4, table[2, 0] * B + 5, table[2, 0] * B + 6, table[2, 0] * B + 7]


class Scheduler:
    """Plain-list model: per request its block list and cached-token count."""

    def __init__(self, max_reqs, max_blocks, num_blocks, rng):
        self.free_slots = list(range(max_reqs))
        self.free_blocks = list(rng.permutation(num_blocks))
        self.reqs = {}              # persistent slot -> [blocks, num_computed]
        self.W = max_blocks

    def join(self):
        s = self.free_slots.pop(0)
        self.reqs[s] = [[], 0]
        return s

    def finish(self, s):
        self.free_blocks.extend(self.reqs.pop(s)[0])
        self.free_slots.append(s)

    def schedule(self, s, n):
        """n more tokens for request s: the new blocks it needs, as one run."""
        blocks, done = self.reqs[s]
        need = -(-(done + n) // B) - len(blocks)
        new = [int(self.free_blocks.pop(0)) for _ in range(max(0, need))]
        start = len(blocks)
        blocks.extend(new)
        return (s, start, new) if new else None


def test_staged_writes_and_step_inputs_match_a_list_model():
    rng = np.random.default_rng(5)
    R, W, N = 12, 40, 600
    sch = Scheduler(R, W, N, rng)
    table = np.full((R, W), -7, np.int32)        # never read where no block was written
    for step in range(25):
        if len(sch.reqs) < R and rng.random() < 0.5:
            sch.join()
        if sch.reqs and rng.random() < 0.15:
            sch.finish(int(rng.choice(list(sch.reqs))))
        batch = [s for s in sch.reqs if rng.random() < 0.8]
        rng.shuffle(batch)
        counts = [int(rng.integers(1, 70)) if sch.reqs[s][1] == 0 or rng.random() < 0.2 else 1 for s in batch]
        runs = [r for r in (sch.schedule(s, n) for s, n in zip(batch, counts)) if r]
        if runs:
            rows = [r[0] for r in runs]
            starts = [r[1] for r in runs]
            offs = np.concatenate([[0], np.cumsum([len(r[2]) for r in runs])])
            vals = np.concatenate([r[2] for r in runs])
            table = M.apply_block_table_writes(table, rows, starts, offs, vals)
        for s, (blocks, _) in sch.reqs.items():
            assert table[s, :len(blocks)].tolist() == blocks
        done = np.zeros(R, np.int32)
        for s, (_, d) in sch.reqs.items():
            done[s] = d
        T = int(sum(counts))
        qsl, lens, pos, slots, rows_out = M.prepare_step(table, batch, done, counts, T, B)
        t = 0
        for b, (s, n) in enumerate(zip(batch, counts)):
            blocks, d = sch.reqs[s]
            assert lens[b] == d + n and qsl[b + 1] - qsl[b] == n
            for i in range(n):
                p = d + i
                assert pos[t] == p and slots[t] == blocks[p // B] * B + p % B
                t += 1
            assert rows_out[b].tolist() == table[s].tolist()
            sch.reqs[s][1] += n
        assert t == T and qsl[-1] == T


def test_reproduces_the_workload_generators_step():
    w = workloads.generate.random_mixed(3, num_decode=7, chunk_specs=[(0, 30), (40, 9)], max_decode_len=90,
                                        num_q_heads=4, num_kv_heads=2, head_dim=32, block_size=B, kv_dtype="bf16")
    R = w.num_seqs
    perm = np.random.default_rng(0).permutation(R + 3)[:R]    # persistent slots, scattered
    table = np.zeros((R + 3, w.block_tables.shape[1]), np.int32)
    table[perm] = w.block_tables
    done = np.zeros(R + 3, np.int32)
    done[perm] = w.seq_lens - w.query_lens
    qsl, lens, pos, slots, rows = M.prepare_step(table, perm, done, w.query_lens, w.num_tokens, w.block_size)
    assert qsl.tolist() == w.query_start_loc.tolist()
    assert lens.tolist() == w.seq_lens.tolist()
    assert (rows == w.block_tables).all()
    assert slots.tolist() == w.new_token_batch()[2].tolist()


def test_undefined_inputs_give_minus_one():
    table = np.arange(8, dtype=np.int32).reshape(2, 4)
    done = np.array([60, 0], np.int32)
    # request 0: positions 60..67 reach block 4 >= width 4; the step claims 12 tokens for 9 scheduled
    qsl, lens, pos, slots, _ = M.prepare_step(table, [0, 1], done, [8, 1], 12, B)
    assert pos[:4].tolist() == [60, 61, 62, 63] and pos[4:8].tolist() == [-1] * 4
    assert slots[4:8].tolist() == [-1] * 4 and pos[9:].tolist() == [-1] * 3 and slots[9:].tolist() == [-1] * 3
    # runs outside the table are skipped, partly outside are clipped
    t = M.apply_block_table_writes(table, [5, 1, 0], [0, 3, -1], [0, 1, 3, 4], [9, 8, 7, 6])
    assert t.tolist() == [[0, 1, 2, 3], [4, 5, 6, 8]]

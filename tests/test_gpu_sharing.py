"""Steps whose block tables share blocks (a common prefix reached through
the tables, the itwiki "vLLM" article, "Block sharing and copy-on-write"):
the plan finds the sharing and the decode kernel deals its items by XCD.
That changes only which wave takes which item, so every row is still
ordinary attention over the sequence's keys; each case is checked against
the fp64 oracle, and the plan's sharing word (workspace header word 8) is
checked for the steps that do and do not share blocks."""

import numpy as np
import pytest

import workloads
from oracle import codecs
from workloads import device as wd
from workloads.generate import build

from full_oracle import assert_close, attention, fill_pools, say

torch = pytest.importorskip("torch")
import paged_kv_cache_141_amd as pa  # noqa: E402,F401

pytestmark = pytest.mark.gpu

SHARE_WORD = 8


def sharing(step):
    return int(step.workspace[:64].view(torch.int32)[SHARE_WORD].item())


def test_sharing_word():
    # through the tables the fp8 shared-prefix step shares blocks; its
    # private-copy twin, the same step through the cascade (the decode reads
    # only the blocks past the prefix) and a plain decode step do not
    cases = [(workloads.make("fp8_shared_prefix", num_seqs=16), 0, 1),
             (workloads.make("fp8_shared_prefix", num_seqs=16, placement="private"), 0, 0),
             (workloads.make("fp8_shared_prefix", num_seqs=16), 8000, 0),
             (workloads.make("llama7b_decode", num_seqs=24), 0, 0)]
    for w, prefix, want in cases:
        step = wd.stage(w)
        if prefix:
            step.use_shared_prefix(prefix)
        step.attend()
        torch.cuda.synchronize()
        say(f"{w.name} prefix={prefix}: sharing word {sharing(step)}")
        assert sharing(step) == want, (w.name, prefix)


@pytest.mark.parametrize("hkv,G,kv,n", [(8, 4, "fp8_e4m3", 40), (1, 8, "bf16", 24), (2, 4, "f16", 30),
                                         (4, 2, "bf16", 33), (32, 1, "bf16", 12), (1, 1, "bf16", 2)])
def test_shared_tables_every_row(hkv, G, kv, n):
    # a prefix of whole blocks shared through the tables, then per sequence a
    # suffix and one to three query tokens; (1, 1, 2) is a step of two
    # sequences, which the plan does not look at (fewer than eight), and a
    # grid under eight waves, which keeps the single counter either way
    rng = np.random.default_rng([hkv, G, n])
    P = 16 * int(rng.integers(20, 300))
    ql = [int(x) for x in rng.integers(1, 4, size=n)]
    lens = [P + q + int(rng.integers(0, 700)) for q in ql]
    fp8 = kv == "fp8_e4m3"
    w = build("shared_tables", 700 + hkv + G + n, lens, ql, num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=128,
              block_size=16, kv_dtype=kv, q_dtype="bf16" if fp8 else kv, k_scale=2.0 ** -5 if fp8 else 1.0,
              v_scale=2.0 ** -5 if fp8 else 1.0, shared_prefix_len=P)
    step = wd.stage(w)
    out = step.attend()
    torch.cuda.synchronize()
    assert sharing(step) == (1 if n >= 8 else 0)
    got = codecs.decode(wd.to_host_bits(out), w.q_dtype)
    kp, vp = fill_pools(w)
    assert_close(w, got, attention(w, kp, vp), label=f"shared tables Hkv={hkv} G={G} {kv} n={n} P={P}")

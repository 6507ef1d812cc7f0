"""Every E4M3FN code through the attention kernels' fp8 widening, bit-exact.

A row whose only visible key is one position attends with weight 1, so its
output is that position's V row times v_scale, rounded to the q dtype.  With
v_scale = 1 every finite E4M3 value is exact in bf16 and f16, so the output
must equal the oracle's decoding of the codes bit for bit (the two NaN codes
give NaN).  Decode rows cover the decode kernel; the first row of a 65-token
prompt chunk (it sees only position 0) covers the chunk loop's widening,
which passes through LDS."""

import numpy as np
import pytest

from oracle import codecs

torch = pytest.importorskip("torch")
import paged_kv_cache_141_amd as pa  # noqa: E402

pytestmark = pytest.mark.gpu

B, D = 16, 128


def run(q_dtype, q_lens):
    """Sequence i: L = q_lens[i] tokens; position 0's V row holds codes
    128*i .. 128*i + 127 (i < 2).  Returns (GPU rows that see only position
    0, the codes they must reproduce)."""
    dev = "cuda"
    S = len(q_lens)
    N = S + 1
    nblk = -(-max(q_lens) // B)
    rng = np.random.default_rng(7)
    k = torch.from_numpy(rng.integers(0, 0x70, size=(N, 1, B, D), dtype=np.uint8)).to(dev)
    v = torch.from_numpy(rng.integers(0, 0x70, size=(N, 1, B, D), dtype=np.uint8))
    codes = np.arange(256, dtype=np.uint8).reshape(2, D)
    # sequence i: block i first, then blocks of the shared spare N - 1 (its
    # V codes are never a row's only key); position 0 of block i holds codes
    tables = np.full((S, nblk), N - 1, dtype=np.int32)
    for i in range(S):
        tables[i, 0] = i
        v[i, 0, 0, :] = torch.from_numpy(codes[i % 2])
    v = v.to(dev)
    qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(qsl[-1])
    qt = torch.randn(T, 1, D, dtype=torch.float32).to(dev).to({"bf16": torch.bfloat16, "f16": torch.float16}[q_dtype])
    out = pa.attention(qt, k, v, torch.from_numpy(tables).to(dev), torch.tensor(q_lens, dtype=torch.int32, device=dev),
                       torch.from_numpy(qsl).to(dev), 1.0 / np.sqrt(D), max_seq_len=max(q_lens),
                       max_query_len=max(q_lens))
    torch.cuda.synchronize()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    rows = bits[qsl[:-1], 0, :]                   # each sequence's first query sees position 0 only
    want = np.stack([codes[i % 2] for i in range(S)])
    return rows, want


@pytest.mark.parametrize("q_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("chunk", [False, True])
def test_every_code_widens_exactly(q_dtype, chunk):
    q_lens = [65, 65] if chunk else [1, 1]
    rows, codes = run(q_dtype, q_lens)
    ref = codecs.e4m3fn_to_f64(codes)
    enc = codecs.f32_to_bf16 if q_dtype == "bf16" else codecs.f32_to_f16
    want = enc(ref.astype(np.float32))
    got_f = codecs.decode(rows, q_dtype)
    nan = np.isnan(ref)
    assert nan.sum() == 2
    assert np.isnan(got_f[nan]).all()
    # values, not bits: the weighted sum starts from +0, so code 0x80 (-0)
    # comes out as +0, the same value
    bad = got_f[~nan] != codecs.decode(want, q_dtype)[~nan]
    assert not bad.any(), (f"{int(bad.sum())} codes widened wrong, e.g. code "
                           f"{int(codes[~nan][bad][0]):#04x}")
    assert np.array_equal(got_f[~nan], ref[~nan])

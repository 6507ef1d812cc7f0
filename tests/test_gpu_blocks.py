"""GPU parity of whole-block copies (pa_copy_blocks) against the oracle.

Byte-exact: the copy within one pool (copy-on-write), the swap out to a
page-locked host pool and back, and the copy-on-write step end to end (copy,
then write the next token into the copy, then attend), whose attention must
also match the oracle within the dtype tolerance.
"""

import ctypes
import sys

import numpy as np
import pytest

from oracle import attention as A
from oracle import blocks as BL
from oracle import cache as C
from oracle import codecs
from workloads import device as wd

torch = pytest.importorskip("torch")
import paged_kv_cache_141_amd as pa  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rand_pool(rng, n, H, B, D, kv):
    dt = {"bf16": np.uint16, "f32": np.uint32, "fp8_e4m3": np.uint8}[kv]
    hi = {"bf16": 2 ** 16, "f32": 2 ** 32, "fp8_e4m3": 2 ** 8}[kv]
    return (rng.integers(0, hi, size=(n, H, B, D), dtype=np.uint64).astype(dt),
            rng.integers(0, hi, size=(n, H, B, D), dtype=np.uint64).astype(dt))


TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8_e4m3": torch.uint8}


def to_dev(a, kv, device="cuda"):
    t = torch.from_numpy(a.view({"bf16": np.int16, "f32": np.int32, "fp8_e4m3": np.uint8}[kv]).copy())
    return t.view(TORCH_DT[kv]).to(device)


def bits(t):
    return wd.to_host_bits(t)


@pytest.mark.parametrize("kv,B,D", [("bf16", 16, 128), ("fp8_e4m3", 64, 128), ("f32", 32, 64)])
def test_copy_within_pool_bit_exact(kv, B, D):
    say("copy within pool", kv, B, D)
    rng = np.random.default_rng(7)
    kp, vp = rand_pool(rng, 40, 4, B, D, kv)
    m = np.array([[0, 20], [3, 21], [39, 22], [5, -1], [40, 23], [7, 24]], np.int64)  # two skipped
    ok, ov = BL.copy_blocks(kp, vp, kp, vp, m)
    gk, gv = to_dev(kp, kv), to_dev(vp, kv)
    pa.copy_blocks(gk, gv, gk, gv, torch.from_numpy(m).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(bits(gk), ok) and np.array_equal(bits(gv), ov)


def test_swap_out_to_pinned_host_and_back_bit_exact():
    rng = np.random.default_rng(8)
    kp, vp = rand_pool(rng, 64, 8, 16, 128, "bf16")
    hk0, hv0 = rand_pool(rng, 16, 8, 16, 128, "bf16")
    out = np.array([[10, 3], [11, 4], [40, 5], [2, 15]], np.int64)
    back = np.array([[3, 60], [4, 61], [5, 62], [15, 63]], np.int64)
    ek, ev = BL.copy_blocks(kp, vp, hk0, hv0, out)
    fk, fv = BL.copy_blocks(ek, ev, kp, vp, back)
    gk, gv = to_dev(kp, "bf16"), to_dev(vp, "bf16")
    hk = to_dev(hk0, "bf16", "cpu").pin_memory()
    hv = to_dev(hv0, "bf16", "cpu").pin_memory()
    say("swap: pinned", hk.is_pinned(), hv.is_pinned())
    pa.copy_blocks(gk, gv, hk, hv, torch.from_numpy(out).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(hk.view(torch.int16).numpy().view(np.uint16), ek)
    assert np.array_equal(hv.view(torch.int16).numpy().view(np.uint16), ev)
    pa.copy_blocks(hk, hv, gk, gv, torch.from_numpy(back).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(bits(gk), fk) and np.array_equal(bits(gv), fv)


def test_pageable_host_pool_is_refused():
    gk = torch.zeros(4, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    gv = torch.zeros(4, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    hk = torch.zeros(4, 2, 16, 64, dtype=torch.bfloat16)
    hv = torch.zeros(4, 2, 16, 64, dtype=torch.bfloat16)
    m = torch.tensor([[0, 1]], dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):
        pa.copy_blocks(gk, gv, hk, hv, m)
    # and through the C ABI directly: pageable memory is refused before any launch
    spec = pa.cache_spec(gk, gv)
    lib = pa.library()
    st = lib.pa_copy_blocks(ctypes.c_void_p(gk.data_ptr()), ctypes.c_void_p(gv.data_ptr()), ctypes.byref(spec),
                            ctypes.c_void_p(hk.data_ptr()), ctypes.c_void_p(hv.data_ptr()), ctypes.byref(spec),
                            ctypes.c_void_p(m.data_ptr()), 1, None)
    assert st == 4
    assert torch.count_nonzero(hk).item() == 0


def test_copy_on_write_step_end_to_end():
    """Two sequences share a 40-token prompt (blocks 3, 7, 5; block 5 half
    full).  Sequence b copies block 5 to block 9, then both write their next
    token and attend: pools byte-exact, attention within 1e-2 of the oracle."""
    rng = np.random.default_rng(9)
    H, Hq, D, B, P, N = 8, 32, 128, 16, 40, 12
    k = rng.standard_normal((P + 2, H, D)).astype(np.float32)
    v = rng.standard_normal((P + 2, H, D)).astype(np.float32)
    kb16, vb16 = codecs.f32_to_bf16(k), codecs.f32_to_bf16(v)
    q = codecs.f32_to_bf16(rng.standard_normal((2, Hq, D)).astype(np.float32))
    prompt_slots = np.array([[3, 7, 5][t // B] * B + t % B for t in range(P)], np.int64)
    tables = np.array([[3, 7, 5], [3, 7, 9]], np.int32)
    lens = np.array([P + 1, P + 1], np.int32)
    qsl = np.array([0, 1, 2], np.int32)
    scale = float(np.float32(1 / np.sqrt(D)))

    ok = np.full((N, H, B, D), 0x7FC0, np.uint16)
    ov = np.full((N, H, B, D), 0x7FC0, np.uint16)
    C.reshape_and_cache(ok, ov, kb16[:P], vb16[:P], "bf16", "bf16", prompt_slots, B)
    ok, ov = BL.copy_blocks(ok, ov, ok, ov, np.array([[5, 9]]))
    C.reshape_and_cache(ok, ov, kb16[P:], vb16[P:], "bf16", "bf16", np.array([5 * B + 8, 9 * B + 8]), B)
    ref = A.paged_attention(q, "bf16", ok, ov, "bf16", tables, lens, qsl, B, scale)

    def dev16(a):
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    gk = dev16(np.full((N, H, B, D), 0x7FC0, np.uint16))
    gv = dev16(np.full((N, H, B, D), 0x7FC0, np.uint16))
    pa.reshape_and_cache(dev16(kb16[:P]), dev16(vb16[:P]), gk, gv, torch.from_numpy(prompt_slots).cuda())
    pa.copy_blocks(gk, gv, gk, gv, torch.tensor([[5, 9]], dtype=torch.int64, device="cuda"))
    pa.reshape_and_cache(dev16(kb16[P:]), dev16(vb16[P:]), gk, gv,
                         torch.tensor([5 * B + 8, 9 * B + 8], dtype=torch.int64, device="cuda"))
    out = pa.attention(dev16(q), gk, gv, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                       torch.from_numpy(qsl).cuda(), scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits(gk), ok) and np.array_equal(bits(gv), ov)
    got = codecs.decode(bits(out), "bf16")
    err = np.abs(got - ref).max()
    say(f"copy-on-write step: max-abs err {err:.3e}")
    assert not np.isnan(got).any() and err <= 1e-2

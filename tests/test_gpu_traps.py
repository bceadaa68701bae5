"""Exact-zero tests for the causal and window traps ("FlashAttention
backward", section "The traps": a causal mask that leaks across the
diagonal).  A leak small enough to hide under the parity tolerance still
fails these, because each quantity below is exactly zero (or bit-identical)
in real arithmetic and in the kernels' arithmetic alike: every contribution
to it is a product with an exact zero, or never visited.

- Backward: with dO = 0 on every query row i >= r, key rows j >= r are seen
  only by those rows, so dK_j = dV_j = 0 exactly (causal).
- Forward: keys and values after row r do not reach rows i <= r, so O and L
  of those rows are bit-identical when K, V rows > r change (causal).
- Window: with dO non-zero on one row i only, dK and dV vanish outside that
  row's window [i - wl, i + wr], and dQ vanishes on every other row."""

import numpy as np
import pytest

from flashattention_backward_pass_fa_amd import binding as fa
from flashattention_backward_pass_fa_amd.inputs import make_tensors
from tests.gpu_cases import to_device, to_host

pytestmark = pytest.mark.gpu


def _dev(shape, dtype, seed):
    host = make_tensors(shape, dtype, seed)
    return {n: to_device(host[n], host.get(n + "_bits"), dtype) for n in ("q", "k", "v", "do")}


@pytest.mark.parametrize("deterministic", [True, False])
@pytest.mark.parametrize("B,H,N,d,dtype,r", [
    (1, 2, 700, 128, "bf16", 333),
    (2, 2, 517, 64, "bf16", 130),
    (1, 2, 400, 128, "f16", 64),
    (1, 1, 300, 40, "f32", 177),
])
def test_causal_backward_does_not_leak(B, H, N, d, dtype, r, deterministic):
    import torch
    print(f"\n[gpu] causal leak, backward: {B}x{H}x{N}x{d} {dtype} r={r} det={deterministic}", flush=True)
    t = _dev((B, H, N, d), dtype, 7 + r)
    o, lse = fa.forward(t["q"], t["k"], t["v"], causal=True)
    do = t["do"].clone()
    do[:, :, r:] = 0
    dq, dk, dv, _ = fa.backward(t["q"], t["k"], t["v"], o, do, lse, causal=True, deterministic=deterministic)
    torch.cuda.synchronize()
    for name, g in (("dk", dk), ("dv", dv)):
        tail = to_host(g)[:, :, r:]
        assert np.all(tail == 0), f"{name}: {int(np.count_nonzero(tail))} non-zero entries past row {r}"
    head = to_host(dv)[:, :, :r]
    assert np.count_nonzero(head) > 0  # the rows before r do carry gradient


@pytest.mark.parametrize("N,d,r", [(700, 128, 250), (517, 64, 64)])
def test_causal_forward_does_not_leak(N, d, r):
    import torch
    print(f"\n[gpu] causal leak, forward: N={N} d={d} r={r}", flush=True)
    t = _dev((1, 2, N, d), "bf16", 11 + r)
    o1, l1 = fa.forward(t["q"], t["k"], t["v"], causal=True)
    k2, v2 = t["k"].clone(), t["v"].clone()
    k2[:, :, r + 1:] = k2[:, :, r + 1:] * 3 + 1
    v2[:, :, r + 1:] = -v2[:, :, r + 1:]
    o2, l2 = fa.forward(t["q"], k2, v2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, :r + 1], o2[:, :, :r + 1])
    assert torch.equal(l1[:, :, :r + 1], l2[:, :, :r + 1])
    assert not torch.equal(o1[:, :, r + 1:], o2[:, :, r + 1:])


@pytest.mark.parametrize("deterministic", [True, False])
@pytest.mark.parametrize("N,d,i,wl,wr", [(600, 128, 300, 100, 37), (517, 64, 5, 0, 200), (700, 128, 650, 255, 0)])
def test_window_support_of_one_row(N, d, i, wl, wr, deterministic):
    import torch
    print(f"\n[gpu] window support: N={N} d={d} row {i} window ({wl}, {wr}) det={deterministic}", flush=True)
    t = _dev((1, 2, N, d), "bf16", 13 + i)
    kw = dict(window=(wl, wr))
    o, lse = fa.forward(t["q"], t["k"], t["v"], **kw)
    do = torch.zeros_like(t["do"])
    do[:, :, i] = t["do"][:, :, i]
    dq, dk, dv, _ = fa.backward(t["q"], t["k"], t["v"], o, do, lse, deterministic=deterministic, **kw)
    torch.cuda.synchronize()
    lo, hi = max(0, i - wl), min(N - 1, i + wr)
    outside = np.ones(N, dtype=bool)
    outside[lo:hi + 1] = False
    for name, g in (("dk", dk), ("dv", dv)):
        a = to_host(g)
        assert np.all(a[:, :, outside] == 0), f"{name} non-zero outside row {i}'s window"
        assert np.count_nonzero(a[:, :, lo:hi + 1]) > 0
    q_rows = to_host(dq)
    others = np.ones(N, dtype=bool)
    others[i] = False
    assert np.all(q_rows[:, :, others] == 0), "dQ non-zero on rows whose dO is zero"


_MANY_HEADS = {}


def _many_heads_inputs(shape):
    """Drawn once for both dQ modes (a 70000-head draw takes seconds)."""
    if shape not in _MANY_HEADS:
        _MANY_HEADS[shape] = make_tensors(shape, "bf16", 33)
    return _MANY_HEADS[shape]


@pytest.mark.parametrize("deterministic", [True, False])
def test_more_heads_than_a_16_bit_grid_dimension(deterministic):
    """B * H = 70000 workgroup columns (past 65535): sampled heads on both
    sides of 2^16 against the oracle."""
    import math
    import torch
    import oracle
    from tests.gpu_cases import assert_close
    B, H, N, d = 1, 70000, 8, 64
    print(f"\n[gpu] {B}x{H}x{N}x{d} bf16 causal det={deterministic}", flush=True)
    host = _many_heads_inputs((B, H, N, d))
    dev = {n: to_device(host[n], host.get(n + "_bits"), "bf16") for n in ("q", "k", "v", "do")}
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=True)
    dq, dk, dv, _ = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True,
                                deterministic=deterministic)
    torch.cuda.synchronize()
    spec = oracle.Spec(sm_scale=1.0 / math.sqrt(d), causal=True)
    for h in (0, 1, 40000, 65535, 65536, 69999):
        ref = oracle.head_backward(host["q"][0, h], host["k"][0, h], host["v"][0, h], host["do"][0, h],
                                   spec, 0, h)
        for name, got in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
            assert_close(f"{name}[h={h}]", to_host(got[0, h]), ref[name], "bf16")

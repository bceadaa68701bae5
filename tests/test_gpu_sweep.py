"""Seeded random sweep of small problems through the C ABI against the fp64
oracle: every flag combined with every other (dtype, head dim, unequal
lengths, varlen batches, causal, windows, dropout, sm_scale, dQ mode, and
[B, N, H, d] storage read and written through strides), so that an
interaction no hand-picked case covers still meets the bar."""

import math

import numpy as np
import pytest

import oracle
from flashattention_backward_pass_fa_amd import binding as fa
from flashattention_backward_pass_fa_amd.inputs import cumulative, make_tensors
from tests.gpu_cases import (TOL_BF16_FRO, TOL_BF16_MAX, assert_close, errors, to_device, to_host,
                             zero_floor)
from tests.rounding_cases import KNOWN, model_case

pytestmark = pytest.mark.gpu

N_CASES = 80
# configurations from a longer run of the same generator that once failed:
# 491, a 3-row dropout problem whose single-key row must give dQ = 0 (the
# kept weight was rounded with its 1 / (1 - p) factor, biasing D)
REGRESSIONS = [491]
# Configurations whose bars the method's own bf16 rounding already misses
# (single-key rows, near-cancelling D) are tests/rounding_cases.py's KNOWN:
# test_rounding_limited_configuration below runs each of them here and
# bounds the named tensor by MODEL_FACTOR times the rounding model's error.
# The model rounds at the method's points but not in the forward's order
# (its weights are taken against the row's final maximum, the forward's
# against a running one), and a tensor of a few values (three D values in
# 6936) then differs from it by up to ~20 %: measured 1.13 there, within
# 2 % on the others.
MODEL_FACTOR = 1.25


def _draw(i):
    """Configuration i of the sweep (its own seeded generator)."""
    r = np.random.default_rng(20260 + i)
    dtype = ["bf16", "bf16", "f16", "f32"][r.integers(4)]
    d = int(r.choice([64, 128])) if dtype != "f32" else int(r.integers(1, 129))
    varlen = bool(r.random() < 0.35)
    cfg = dict(dtype=dtype, d=d, H=int(r.integers(1, 4)), causal=bool(r.random() < 0.5),
               window=(int(r.choice([-1, -1, r.integers(0, 300)])),
                       int(r.choice([-1, -1, r.integers(0, 300)]))),
               p=float(r.choice([0.0, 0.0, 0.15])), det=bool(r.random() < 0.5),
               scale=float(r.uniform(0.3, 1.5)) / math.sqrt(d), varlen=varlen, seed=1000 + i)
    if varlen:
        nb = int(r.integers(1, 5))
        cfg["lq"] = [int(x) for x in r.integers(0, 400, size=nb)]
        cfg["lk"] = [int(x) if r.random() < 0.7 else cfg["lq"][j]
                     for j, x in enumerate(r.integers(0, 400, size=nb))]
        if max(cfg["lq"]) == 0:
            cfg["lq"][0] = 1
        if max(cfg["lk"]) == 0:
            cfg["lk"][0] = 1
    else:
        cfg["B"] = int(r.integers(1, 3))
        cfg["Nq"] = int(r.integers(1, 700))
        cfg["Nk"] = cfg["Nq"] if r.random() < 0.5 else int(r.integers(1, 700))
        # drawn last, so that the cases drawn before this option existed are unchanged
        cfg["bnhd"] = bool(r.random() < 0.35)
    return cfg


def _bnhd(t):
    """The same [B, H, N, d] values stored as [B, N, H, d]: a strided view."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def _kw(spec):
    return dict(sm_scale=spec.sm_scale, causal=spec.causal,
                window=(spec.window_left, spec.window_right), dropout_p=spec.dropout_p,
                seed=spec.seed, offset=spec.offset)


def run_configuration(c, spec):
    """GPU forward and backward of configuration c through the C ABI, and
    the oracle's result; returns (gpu outputs on the host, oracle, magnitudes)."""
    import torch
    H, d, dtype = c["H"], c["d"], c["dtype"]
    if c["varlen"]:
        cu_q, cu_k = cumulative(c["lq"]), cumulative(c["lk"])
        shapes = {"k": (int(cu_k[-1]), H, d), "v": (int(cu_k[-1]), H, d)}
        host = make_tensors((int(cu_q[-1]), H, d), dtype, c["seed"], shapes=shapes)
    else:
        shapes = {"k": (c["B"], H, c["Nk"], d), "v": (c["B"], H, c["Nk"], d)}
        host = make_tensors((c["B"], H, c["Nq"], d), dtype, c["seed"], shapes=shapes)
    dev = {n: to_device(host[n], host.get(n + "_bits"), dtype) for n in ("q", "k", "v", "do")}
    if c.get("bnhd"):
        dev = {n: _bnhd(t) for n, t in dev.items()}
    if c["varlen"]:
        cq, ck = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
        mq, mk = max(c["lq"]), max(c["lk"])
        o, lse = fa.forward_varlen(dev["q"], dev["k"], dev["v"], cq, ck, mq, mk, **_kw(spec))
        dq, dk, dv, delta = fa.backward_varlen(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, cq, ck,
                                               mq, mk, deterministic=c["det"], **_kw(spec))
        ref = oracle.varlen_backward(host["q"], host["k"], host["v"], host["do"], cu_q, cu_k, spec)
    else:
        o, lse = fa.forward(dev["q"], dev["k"], dev["v"], **_kw(spec))
        dq, dk, dv, delta = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse,
                                        deterministic=c["det"], **_kw(spec))
        ref = oracle.backward(host["q"], host["k"], host["v"], host["do"], spec)
    torch.cuda.synchronize()
    got = {n: to_host(t) for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv),
                                      ("delta", delta))}
    mags = {n: float(np.abs(host[n]).max()) if host[n].size else 0.0 for n in ("q", "k", "v", "do")}
    return got, ref, mags


def _query_rows(c):
    return max(c["lq"]) if c["varlen"] else c["Nq"]


def check_lse(got_l, want_l):
    valid = ~np.isnan(want_l)
    assert np.array_equal(np.isneginf(got_l[valid]), np.isneginf(want_l[valid]))
    live = valid & np.isfinite(want_l)
    if live.any():
        assert float(np.abs(got_l[live] - want_l[live]).max()) <= 1e-3
    return valid


@pytest.mark.parametrize("i", list(range(N_CASES)) + REGRESSIONS)
def test_random_configuration(i):
    c = _draw(i)
    print(f"\n[gpu] sweep {i}: {c}", flush=True)
    spec = oracle.Spec(sm_scale=c["scale"], causal=c["causal"], window_left=c["window"][0],
                       window_right=c["window"][1], dropout_p=c["p"], seed=77 + i, offset=i)
    got, ref, mags = run_configuration(c, spec)
    for name in ("o", "dq", "dk", "dv"):
        assert_close(name, got[name], ref[name], c["dtype"],
                     zero_floor(name, c["dtype"], c["d"], spec.sm_scale, mags, _query_rows(c), c["p"]))
    valid = check_lse(got["lse"], ref["lse"])
    assert_close("delta", got["delta"][valid], ref["delta"][valid], c["dtype"])


@pytest.mark.parametrize("i,c,names,reading", KNOWN, ids=[str(k[0]) for k in KNOWN])
def test_rounding_limited_configuration(i, c, names, reading):
    """A configuration whose `names` tensors the method's own bf16 rounding
    takes past the whole-tensor bars: every other tensor meets the bars, and
    each of `names` stays within MODEL_FACTOR times the rounding model's
    error (max and relative Frobenius, each bounded by the larger of the bar
    and that)."""
    print(f"\n[gpu] rounding-limited {i} ({names} {reading}): {c}", flush=True)
    spec, _, ref_m, model, mags = model_case(c, i)
    got, ref, _ = run_configuration(c, spec)
    valid = check_lse(got["lse"], ref["lse"])
    sel = {"delta": valid}
    for n in ("o", "dq", "dk", "dv", "delta"):
        g = got[n][sel[n]] if n in sel else got[n]
        r = ref[n][sel[n]] if n in sel else ref[n]
        if n not in names:
            assert_close(n, g, r, c["dtype"],
                         zero_floor(n, c["dtype"], c["d"], spec.sm_scale, mags, _query_rows(c), c["p"]))
            continue
        m = model[n][sel[n]] if n in sel else model[n]
        g_max, r_max, g_fro = errors(g, r)
        m_max, _, m_fro = errors(m, r)
        bar_max = TOL_BF16_MAX * r_max
        print(f"[gpu] {n}: max|err| {g_max:.4e} (model {m_max:.4e}, ratio {g_max / m_max:.3f}), "
              f"rel Frobenius {g_fro:.4e} (model {m_fro:.4e}, ratio {g_fro / m_fro:.3f})", flush=True)
        assert g_max <= max(bar_max, MODEL_FACTOR * m_max), (
            f"{n}: max|err| {g_max:.4e} > max(bar {bar_max:.4e}, {MODEL_FACTOR} x model {m_max:.4e})")
        assert g_fro <= max(TOL_BF16_FRO, MODEL_FACTOR * m_fro), (
            f"{n}: rel Frobenius {g_fro:.4e} > max(bar {TOL_BF16_FRO}, {MODEL_FACTOR} x model {m_fro:.4e})")

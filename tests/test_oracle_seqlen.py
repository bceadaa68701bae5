"""Pins of the oracle when queries and keys differ in number, and for packed
variable-length batches.

The alignment reading (the last query stands at the last key, so query i is
at key position i + Nk - Nq) is pinned to torch's own lower-right causal
bias (torch.nn.attention.bias.causal_lower_right), a library implementation
of that convention, through scaled_dot_product_attention and autograd in
fp64; windows, which torch has no lower-right form for, are pinned by
embedding the short problem in a square one (already pinned to torch) and by
finite differences.  Rows that see no key are pinned to torch's result for
them (O = 0, zero gradients) and to L = -inf.
"""

import math
import warnings

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st
from torch.nn.attention.bias import causal_lower_right

import oracle

SHAPES = [(1, 7), (5, 12), (12, 5), (7, 7), (9, 1), (3, 30)]


def _lower_right(nq, nk):
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")  # torch warns that nq > nk leaves rows empty
        return causal_lower_right(nq, nk)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("nq,nk", SHAPES)
def test_lower_right_causal_matches_torch(nq, nk):
    rng = np.random.default_rng(nq * 100 + nk)
    d = 8
    q, do = _rand(rng, nq, d), _rand(rng, nq, d)
    k, v = _rand(rng, nk, d), _rand(rng, nk, d)
    spec = oracle.Spec(sm_scale=0.7, causal=True)
    r = oracle.head_backward(q, k, v, do, spec)

    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    bias = _lower_right(nq, nk)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.view(1, 1, nq, d), tk.view(1, 1, nk, d), tv.view(1, 1, nk, d), attn_mask=bias,
        scale=0.7).view(nq, d)
    o.backward(torch.tensor(do))
    mask = bias._materialize(device="cpu").view(nq, nk)
    lse = torch.logsumexp(((tq @ tk.T) * 0.7).masked_fill(~mask, float("-inf")), dim=-1)

    np.testing.assert_allclose(r["o"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(r["lse"]), np.isneginf(lse.detach().numpy()))
    live = np.isfinite(r["lse"])
    np.testing.assert_allclose(r["lse"][live], lse.detach().numpy()[live], rtol=1e-12, atol=1e-12)
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(r[name], t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)


def test_rows_without_keys_are_empty_sums():
    # causal with nq > nk: the first nq - nk queries stand before key 0
    rng = np.random.default_rng(3)
    nq, nk, d = 10, 4, 5
    q, do = _rand(rng, nq, d), _rand(rng, nq, d)
    k, v = _rand(rng, nk, d), _rand(rng, nk, d)
    spec = oracle.Spec(sm_scale=0.5, causal=True)
    r = oracle.head_backward(q, k, v, do, spec)
    empty = nq - nk
    assert np.all(np.isneginf(r["lse"][:empty]))
    assert np.all(r["o"][:empty] == 0) and np.all(r["dq"][:empty] == 0)
    assert np.all(r["delta"][:empty] == 0)
    # the other rows are the square causal problem of the last nk queries
    sq = oracle.head_backward(q[empty:], k, v, do[empty:], spec)
    for name in ("o", "lse", "dq", "delta"):
        np.testing.assert_allclose(r[name][empty:], sq[name], rtol=1e-12, atol=1e-13)
    for name in ("dk", "dv"):
        np.testing.assert_allclose(r[name], sq[name], rtol=1e-12, atol=1e-13)


WINDOWS = [dict(causal=True), dict(window_left=2, window_right=1), dict(window_left=3),
           dict(window_right=0), dict(causal=True, window_left=4), dict()]


@pytest.mark.parametrize("mask", WINDOWS)
@pytest.mark.parametrize("nq,nk", [(3, 11), (6, 7), (1, 9)])
def test_short_queries_embed_in_the_square_problem(mask, nq, nk):
    """nq <= nk: query i behaves as query i + nk - nq of the nk x nk problem.

    The square problem's extra leading queries carry dO = 0, so they add
    nothing to dK and dV (their dS and P~^T dO vanish).
    """
    rng = np.random.default_rng(nq * 31 + nk)
    d = 4
    shift = nk - nq
    q_all, do_all = _rand(rng, nk, d), _rand(rng, nk, d)
    do_all[:shift] = 0.0
    k, v = _rand(rng, nk, d), _rand(rng, nk, d)
    spec = oracle.Spec(sm_scale=0.8, **mask)
    sq = oracle.head_backward(q_all, k, v, do_all, spec)
    r = oracle.head_backward(q_all[shift:], k, v, do_all[shift:], spec)
    for name in ("o", "lse", "dq", "delta"):
        np.testing.assert_allclose(r[name], sq[name][shift:], rtol=1e-12, atol=1e-13, err_msg=name)
    for name in ("dk", "dv"):
        np.testing.assert_allclose(r[name], sq[name], rtol=1e-12, atol=1e-13, err_msg=name)


@pytest.mark.parametrize("mask", [dict(window_left=2, window_right=1), dict(window_left=0),
                                  dict(causal=True, window_left=2), dict(window_right=2)])
def test_window_support_is_anchored_at_the_last_key(mask):
    """nq > nk: the last query sees the window around the last key; each row
    up sees the same window moved one key to the left."""
    nq, nk = 9, 4
    spec = oracle.Spec(sm_scale=0.3, **mask)
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, nq, 3), _rand(rng, nk, 3), _rand(rng, nk, 3)
    f = oracle.head_rows_forward(q, k, v, spec, 0, 0, np.arange(nq))
    p = np.zeros((nq, nk))
    p[:, f["lo"]:f["hi"]] = f["p"]
    wl = mask.get("window_left", -1)
    wr = 0 if mask.get("causal") else mask.get("window_right", -1)
    for t in range(nq):  # row nq - 1 - t
        centre = nk - 1 - t
        lo = 0 if wl < 0 else max(0, centre - wl)
        hi = nk - 1 if wr < 0 else min(nk - 1, centre + wr)
        expect = np.zeros(nk, dtype=bool)
        if lo <= hi:
            expect[lo:hi + 1] = True
        np.testing.assert_array_equal(p[nq - 1 - t] > 0, expect, err_msg=f"row {nq - 1 - t}")


def _f_value(q, k, v, do, spec):
    o, _ = oracle.head_forward(q, k, v, spec)
    return float((do * o).sum())


def _fd_grads(q, k, v, do, spec, h=1e-5):
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        for idx in np.ndindex(*g.shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (_f_value(*plus, do, spec) - _f_value(*minus, do, spec)) / (2 * h)
        grads.append(g)
    return grads


@settings(max_examples=25, deadline=None)
@given(nq=st.integers(1, 7), nk=st.integers(1, 7), d=st.integers(1, 3),
       mask=st.sampled_from(range(len(WINDOWS))), seed=st.integers(0, 2**31 - 1),
       p=st.sampled_from([0.0, 0.0, 0.3]))
def test_unequal_lengths_match_finite_differences(nq, nk, d, mask, seed, p):
    rng = np.random.default_rng(seed)
    q, do = _rand(rng, nq, d), _rand(rng, nq, d)
    k, v = _rand(rng, nk, d), _rand(rng, nk, d)
    spec = oracle.Spec(sm_scale=0.9, dropout_p=p, seed=seed, offset=3, **WINDOWS[mask])
    r = oracle.head_backward(q, k, v, do, spec)
    fq, fk, fv = _fd_grads(q, k, v, do, spec)
    for name, fd in (("dq", fq), ("dk", fk), ("dv", fv)):
        tol = 1e-7 * max(1.0, float(np.abs(fd).max()))
        assert float(np.abs(r[name] - fd).max()) <= tol, name


@pytest.mark.parametrize("nq,nk", [(5, 12), (12, 5)])
def test_unequal_dropout_matches_torch_with_fixed_mask(nq, nk):
    rng = np.random.default_rng(11)
    d = 6
    q, do = _rand(rng, nq, d), _rand(rng, nq, d)
    k, v = _rand(rng, nk, d), _rand(rng, nk, d)
    spec = oracle.Spec(sm_scale=0.6, causal=True, dropout_p=0.25, seed=99, offset=2)
    b, h = 1, 3
    r = oracle.head_backward(q, k, v, do, spec, b, h)
    z = torch.tensor(oracle.dropout_mask(spec, b, h, nq, nk), dtype=torch.float64)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = _lower_right(nq, nk)._materialize(device="cpu").view(nq, nk)
    s = ((tq @ tk.T) * 0.6).masked_fill(~mask, float("-inf"))
    live = mask.any(dim=1, keepdim=True)
    p = torch.where(live, torch.softmax(s.masked_fill(~live, 0.0), -1), 0.0)
    o = (p * z / 0.75) @ tv
    o.backward(torch.tensor(do))
    np.testing.assert_allclose(r["o"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(r[name], t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)


@pytest.mark.parametrize("mask", WINDOWS)
def test_unequal_gradient_invariants(mask):
    rng = np.random.default_rng(2)
    for nq, nk in ((6, 13), (13, 6)):
        q, do = _rand(rng, nq, 4), _rand(rng, nq, 4)
        k, v = _rand(rng, nk, 4), _rand(rng, nk, 4)
        r = oracle.head_backward(q, k, v, do, oracle.Spec(sm_scale=0.5, **mask))
        live = np.isfinite(r["lse"])
        np.testing.assert_allclose(r["dk"].sum(axis=0), 0.0, atol=1e-12)
        np.testing.assert_allclose(r["dv"].sum(axis=0), do[live].sum(axis=0), atol=1e-12)


def test_varlen_is_each_sequence_on_its_own():
    rng = np.random.default_rng(8)
    lens_q = [5, 0, 9, 1, 7]
    lens_k = [8, 3, 4, 1, 0]
    nh, d = 2, 4
    cu_q = np.concatenate([[0], np.cumsum(lens_q)])
    cu_k = np.concatenate([[0], np.cumsum(lens_k)])
    q, do = _rand(rng, cu_q[-1], nh, d), _rand(rng, cu_q[-1], nh, d)
    k, v = _rand(rng, cu_k[-1], nh, d), _rand(rng, cu_k[-1], nh, d)
    spec = oracle.Spec(sm_scale=0.4, causal=True, dropout_p=0.2, seed=5, offset=1)
    r = oracle.varlen_backward(q, k, v, do, cu_q, cu_k, spec)
    for b in range(len(lens_q)):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        for h in range(nh):
            if lens_q[b] == 0:
                assert np.all(r["dk"][ks, h] == 0) and np.all(r["dv"][ks, h] == 0)
                continue
            one = oracle.head_backward(q[qs, h], k[ks, h], v[ks, h], do[qs, h], spec, b, h)
            for name in ("dq", "o"):
                np.testing.assert_array_equal(r[name][qs, h], one[name])
            for name in ("dk", "dv"):
                np.testing.assert_array_equal(r[name][ks, h], one[name])
            np.testing.assert_array_equal(r["lse"][b, h, :lens_q[b]], one["lse"])
            assert np.all(np.isnan(r["lse"][b, h, lens_q[b]:]))
    # a sequence without keys: every row is empty
    assert np.all(np.isneginf(r["lse"][4, :, :lens_q[4]]))


def test_credited_flops_count_unequal_visible_pairs():
    spec = oracle.Spec(sm_scale=1.0, causal=True)
    # nq = 3 queries at key positions 5, 6, 7 of 8 keys: 6 + 7 + 8 pairs
    assert oracle.credited_flops(1, 1, 3, 2, spec, n_k=8) == 10 * 2 * (6 + 7 + 8)
    # nq = 8 queries over 3 keys: rows 5, 6, 7 see 1, 2, 3 keys
    assert oracle.credited_flops(1, 1, 8, 2, spec, n_k=3) == 10 * 2 * (1 + 2 + 3)


@pytest.mark.parametrize("nq,nk", SHAPES)
def test_key_columns_lower_right_causal_match_torch(nq, nk):
    """dK, dV of selected keys from the rows that see them, with the last
    query aligned to the last key, against torch's lower-right causal bias."""
    rng = np.random.default_rng(nq * 37 + nk)
    d = 5
    q, do = _rand(rng, nq, d), _rand(rng, nq, d)
    k, v = _rand(rng, nk, d), _rand(rng, nk, d)
    spec = oracle.Spec(sm_scale=0.6, causal=True)
    cols = np.unique(np.array([0, nk // 2, nk - 1]))
    r = oracle.head_columns_backward(q, k, v, do, spec, 0, 0, cols, chunk=3)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.view(1, 1, nq, d), tk.view(1, 1, nk, d), tv.view(1, 1, nk, d),
        attn_mask=_lower_right(nq, nk), scale=0.6).view(nq, d)
    o.backward(torch.tensor(do))
    np.testing.assert_allclose(r["dk"], tk.grad.numpy()[cols], rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(r["dv"], tv.grad.numpy()[cols], rtol=1e-9, atol=1e-11)

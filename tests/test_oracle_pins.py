"""Pins of the CPU oracle against things other than itself.

Each pin fixes the oracle to an outside fact: a library routine (torch fp64
scaled_dot_product_attention and autograd), central finite differences,
algebraic invariants of the softmax gradient, special cases with closed
forms, and the pages' printed worked numbers.  Together they fail on a
dropped term, a wrong sign, a wrong index or a transposed operand anywhere in
the oracle's forward or backward (test_oracle_mutations.py plants such
mistakes and checks that these pins catch them).
"""

import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle

torch.set_default_dtype(torch.float64)

MASKS = {
    "none": dict(),
    "causal": dict(causal=True),
    "window": dict(window_left=2, window_right=1),
    "window_left_only": dict(window_left=1),
    "causal_window": dict(causal=True, window_left=3),
}


def _spec(d, mask, **kw):
    return oracle.Spec(sm_scale=kw.pop("sm_scale", 1.0 / math.sqrt(d)), **MASKS[mask], **kw)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _torch_mask(n, spec):
    i = torch.arange(n).view(-1, 1)
    j = torch.arange(n).view(1, -1)
    ok = torch.ones(n, n, dtype=torch.bool)
    if spec.causal:
        ok &= j <= i
    if spec.window_left >= 0:
        ok &= j >= i - spec.window_left
    if spec.window_right >= 0:
        ok &= j <= i + spec.window_right
    return ok


def _torch_sdpa(q, k, v, spec):
    """torch's own attention on one head ([N, d] fp64 tensors)."""
    n = q.shape[0]
    q4, k4, v4 = (t.view(1, 1, n, -1) for t in (q, k, v))
    if spec.causal and spec.window_left < 0 and spec.window_right < 0:
        o = torch.nn.functional.scaled_dot_product_attention(
            q4, k4, v4, is_causal=True, scale=spec.sm_scale)
    else:
        o = torch.nn.functional.scaled_dot_product_attention(
            q4, k4, v4, attn_mask=_torch_mask(n, spec), scale=spec.sm_scale)
    return o.view(n, -1)


def _torch_explicit_dropout(q, k, v, spec, z):
    """Softmax attention with a fixed keep mask z, written with torch ops."""
    n = q.shape[0]
    s = (q @ k.T) * spec.sm_scale
    s = s.masked_fill(~_torch_mask(n, spec), float("-inf"))
    p = torch.softmax(s, dim=-1)
    return (p * z / (1.0 - spec.dropout_p)) @ v


def _f_value(q, k, v, do, spec, b=0, h=0):
    o, _ = oracle.head_forward(q, k, v, spec, b, h)
    return float((do * o).sum())


# ---------------------------------------------------------------- forward

@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("n,d", [(1, 4), (7, 3), (33, 16), (64, 8)])
def test_forward_matches_torch_sdpa(mask, n, d):
    rng = np.random.default_rng(n * 100 + d)
    q, k, v = (_rand(rng, n, d) for _ in range(3))
    spec = _spec(d, mask, sm_scale=0.37)
    o, lse = oracle.head_forward(q, k, v, spec)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    o_ref = _torch_sdpa(tq, tk, tv, spec).numpy()
    s = (tq @ tk.T) * spec.sm_scale
    s = s.masked_fill(~_torch_mask(n, spec), float("-inf"))
    lse_ref = torch.logsumexp(s, dim=-1).numpy()
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mask", list(MASKS))
def test_probability_rows_sum_to_one(mask):
    rng = np.random.default_rng(3)
    q, k, v = (_rand(rng, 40, 8) for _ in range(3))
    f = oracle.head_rows_forward(q, k, v, _spec(8, mask), 0, 0, np.arange(40))
    np.testing.assert_allclose(f["p"].sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert np.all(f["p"] >= 0)


def test_single_key_gives_value_row():
    rng = np.random.default_rng(4)
    q, k, v = (_rand(rng, 1, 5) for _ in range(3))
    spec = _spec(5, "none", sm_scale=0.8)
    o, lse = oracle.head_forward(q, k, v, spec)
    np.testing.assert_array_equal(o, v)
    assert lse[0] == pytest.approx(0.8 * float(q[0] @ k[0]), rel=1e-15)


@pytest.mark.parametrize("mask", list(MASKS))
def test_zero_keys_give_uniform_weights(mask):
    rng = np.random.default_rng(5)
    n, d = 12, 4
    q, v = _rand(rng, n, d), _rand(rng, n, d)
    k = np.zeros((n, d))
    spec = _spec(d, mask)
    f = oracle.head_rows_forward(q, k, v, spec, 0, 0, np.arange(n))
    ok = oracle.valid_mask(np.arange(n), np.arange(f["lo"], f["hi"]), spec)
    counts = ok.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(f["p"], ok / counts, atol=1e-15)
    np.testing.assert_allclose(f["lse"], np.log(counts[:, 0]), atol=1e-14)


def test_valid_mask_predicate_by_enumeration():
    spec = oracle.Spec(sm_scale=1.0, causal=True, window_left=2, window_right=5)
    ok = oracle.valid_mask(np.arange(9), np.arange(9), spec)
    for i in range(9):
        for j in range(9):
            assert ok[i, j] == (j <= i and j >= i - 2 and j <= i + 5)
    spec = oracle.Spec(sm_scale=1.0, window_left=1023, window_right=1023)
    ok = oracle.valid_mask([5000], np.arange(8192), spec)[0]
    # |i - j| < 1024: keys 3977 .. 6023
    assert ok.sum() == 2047 and ok[3977] and ok[6023] and not ok[3976] and not ok[6024]


# --------------------------------------------------------------- backward

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
@given(n=st.integers(1, 8), d=st.integers(1, 4), mask=st.sampled_from(list(MASKS)),
       scale=st.floats(0.2, 1.5), seed=st.integers(0, 2**31 - 1),
       p=st.sampled_from([0.0, 0.0, 0.3]))
def test_backward_matches_finite_differences(n, d, mask, scale, seed, p):
    rng = np.random.default_rng(seed)
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    spec = _spec(d, mask, sm_scale=scale, dropout_p=p, seed=seed, offset=7)
    r = oracle.head_backward(q, k, v, do, spec)
    fq, fk, fv = _fd_grads(q, k, v, do, spec)
    for name, fd in (("dq", fq), ("dk", fk), ("dv", fv)):
        tol = 1e-7 * max(1.0, float(np.abs(fd).max()))
        assert float(np.abs(r[name] - fd).max()) <= tol, name


@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("n,d", [(1, 8), (17, 8), (64, 16), (100, 32)])
def test_backward_matches_torch_autograd(mask, n, d):
    rng = np.random.default_rng(n + 1000 * d)
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    spec = _spec(d, mask, sm_scale=0.29)
    r = oracle.head_backward(q, k, v, do, spec, chunk=13)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    o = _torch_sdpa(tq, tk, tv, spec)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(r["o"], o.detach().numpy(), rtol=1e-12, atol=1e-12)
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(r[name], t.grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)


@pytest.mark.parametrize("mask", ["none", "causal", "window"])
def test_dropout_backward_matches_torch_autograd_with_fixed_mask(mask):
    rng = np.random.default_rng(11)
    n, d = 48, 8
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    spec = _spec(d, mask, dropout_p=0.25, seed=0x5EED, offset=3)
    r = oracle.head_backward(q, k, v, do, spec, b=1, h=2, chunk=10)
    z = torch.from_numpy(oracle.dropout_keep(spec.seed, spec.offset, 1, 2,
                                             np.arange(n), np.arange(n), 0.25).astype(np.float64))
    assert 0 < float(z.mean()) < 1
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    o = _torch_explicit_dropout(tq, tk, tv, spec, z)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(r["o"], o.detach().numpy(), rtol=1e-12, atol=1e-12)
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(r[name], t.grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)


def test_dropout_zero_probability_is_plain_attention():
    rng = np.random.default_rng(12)
    q, k, v, do = (_rand(rng, 20, 4) for _ in range(4))
    a = oracle.head_backward(q, k, v, do, _spec(4, "causal"))
    b = oracle.head_backward(q, k, v, do, _spec(4, "causal", dropout_p=0.0, seed=9))
    for name in ("dq", "dk", "dv", "o", "lse"):
        np.testing.assert_array_equal(a[name], b[name])


@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("p", [0.0, 0.2])
def test_gradient_invariants(mask, p):
    rng = np.random.default_rng(21)
    n, d = 50, 8
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    spec = _spec(d, mask, dropout_p=p, seed=5)
    rows = oracle.head_rows_backward(q, k, v, do, spec, 0, 0, np.arange(n))
    # softmax Jacobian rows sum to zero
    np.testing.assert_allclose(rows["ds"].sum(axis=1), 0.0, atol=1e-13)
    # D two ways: rowsum(dO * O) and sum_j P_ij dP_ij
    np.testing.assert_allclose(rows["delta"], (rows["p"] * rows["dp"]).sum(axis=1),
                               rtol=1e-12, atol=1e-13)
    r = oracle.head_backward(q, k, v, do, spec)
    # f is invariant under K_j -> K_j + c for all j  =>  sum_j dK_j = 0
    np.testing.assert_allclose(r["dk"].sum(axis=0), 0.0, atol=1e-12)
    if p == 0.0:
        # rows of P sum to 1  =>  sum_j dV_j = sum_i dO_i
        np.testing.assert_allclose(r["dv"].sum(axis=0), do.sum(axis=0), atol=1e-12)


def test_special_cases():
    rng = np.random.default_rng(31)
    # N = 1: dQ = dK = 0, dV = dO
    q, k, v, do = (_rand(rng, 1, 6) for _ in range(4))
    r = oracle.head_backward(q, k, v, do, _spec(6, "none"))
    np.testing.assert_allclose(r["dq"], 0.0, atol=1e-15)
    np.testing.assert_allclose(r["dk"], 0.0, atol=1e-15)
    np.testing.assert_array_equal(r["dv"], do)
    # all value rows equal: O does not depend on Q or K
    n, d = 30, 5
    q, k, do = (_rand(rng, n, d) for _ in range(3))
    v = np.tile(_rand(rng, 1, d), (n, 1))
    for mask in MASKS:
        r = oracle.head_backward(q, k, v, do, _spec(d, mask))
        np.testing.assert_allclose(r["dq"], 0.0, atol=1e-13)
        np.testing.assert_allclose(r["dk"], 0.0, atol=1e-13)
    # causal row 0 sees only key 0
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    r = oracle.head_backward(q, k, v, do, _spec(d, "causal"))
    np.testing.assert_allclose(r["dq"][0], 0.0, atol=1e-14)


def test_causal_boundary_has_no_leak():
    rng = np.random.default_rng(41)
    n, d, r_cut = 40, 6, 23
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    do[r_cut:] = 0.0
    for extra in ({}, {"dropout_p": 0.3, "seed": 2}):
        r = oracle.head_backward(q, k, v, do, _spec(d, "causal", **extra), chunk=7)
        assert np.all(r["dk"][r_cut:] == 0.0)
        assert np.all(r["dv"][r_cut:] == 0.0)
        assert np.abs(r["dk"][:r_cut]).max() > 0


def test_window_support():
    rng = np.random.default_rng(42)
    n, d, row = 40, 6, 17
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    do_one = np.zeros_like(do)
    do_one[row] = do[row]
    spec = _spec(d, "window")  # keys row-2 .. row+1
    r = oracle.head_backward(q, k, v, do_one, spec)
    support = np.zeros(n, dtype=bool)
    support[row - 2: row + 2] = True
    assert np.all(r["dk"][~support] == 0.0) and np.all(r["dv"][~support] == 0.0)
    assert np.all(np.abs(r["dv"][support]).sum(axis=1) > 0)


def test_chunking_is_exact_grouping():
    rng = np.random.default_rng(51)
    q, k, v, do = (_rand(rng, 2, 3, 45, 8) for _ in range(4))
    spec = _spec(8, "causal_window", dropout_p=0.1, seed=77)
    a = oracle.backward(q, k, v, do, spec)
    b = oracle.backward(q, k, v, do, spec, chunk=4)
    for name in a:
        np.testing.assert_allclose(a[name], b[name], rtol=1e-13, atol=1e-13)
    heads = [(1, 2)]
    c = oracle.backward(q, k, v, do, spec, heads=heads, chunk=16)
    np.testing.assert_allclose(c["dq"][1, 2], a["dq"][1, 2], atol=1e-13)
    assert np.all(c["dq"][0] == 0)


def test_credited_flops_counts_visible_pairs():
    spec = oracle.Spec(sm_scale=1.0, causal=True)
    assert oracle.credited_flops(1, 1, 4, 2, spec) == 10 * 2 * 10
    spec = oracle.Spec(sm_scale=1.0, window_left=1, window_right=1)
    assert oracle.credited_flops(2, 3, 5, 4, spec) == 10 * 4 * 13 * 6


# ------------------------------------------------- the pages' worked numbers

def _golden_rows(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    rows = []
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append([float(x) for x in line.split()])
    return rows


def test_memory_table_of_worked_numbers():
    for n, p_bytes, state_bytes, ratio in _golden_rows("memory_table.txt"):
        n = int(n)
        got_p = oracle.materialised_p_bytes(n, 2)
        got_state = oracle.saved_state_bytes(n, 128, 2)
        # the page prints two significant figures and rounds the ratio to N/d
        assert got_p == pytest.approx(p_bytes, rel=0.05)
        assert got_state == pytest.approx(state_bytes, rel=0.05)
        assert got_p / got_state == pytest.approx(ratio, rel=0.05)


def test_score_matrix_size_per_head():
    (n, bytes_per_head), = _golden_rows("score_matrix.txt")
    assert oracle.materialised_p_bytes(int(n), 4) == bytes_per_head


def test_closed_form_credited_flops_matches_enumeration():
    from flashattention_backward_pass_fa_amd.flops import credited_flops
    for n, causal, wl, wr in [(1, False, -1, -1), (37, True, -1, -1), (100, False, 7, 3),
                              (64, True, 10, -1), (90, False, -1, 0), (200, False, 1023, 1023)]:
        spec = oracle.Spec(sm_scale=1.0, causal=causal, window_left=wl, window_right=wr)
        assert credited_flops(2, 3, n, 16, causal, wl, wr) == oracle.credited_flops(2, 3, n, 16, spec)


def test_closed_form_credited_flops_matches_enumeration_unequal_lengths():
    from flashattention_backward_pass_fa_amd.flops import credited_flops
    for n, n_k, causal, wl, wr in [(3, 8, True, -1, -1), (8, 3, True, -1, -1), (50, 130, False, 7, 3),
                                   (130, 50, False, 10, -1), (64, 200, True, 20, -1), (9, 1, False, -1, 0)]:
        spec = oracle.Spec(sm_scale=1.0, causal=causal, window_left=wl, window_right=wr)
        assert (credited_flops(2, 3, n, 16, causal, wl, wr, n_k=n_k)
                == oracle.credited_flops(2, 3, n, 16, spec, n_k=n_k))


# ----------------------------------------------- selected key columns only

@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("p", [0.0, 0.3])
def test_key_columns_match_torch_autograd(mask, p):
    """dK, dV of a few keys, from only the rows that see them, against
    torch fp64 autograd of the whole problem (with the oracle's keep mask
    fixed when p > 0)."""
    rng = np.random.default_rng(31 + int(10 * p))
    n, d = 41, 6
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    spec = _spec(d, mask, sm_scale=0.43, dropout_p=p, seed=0x5EED, offset=2)
    cols = np.array([0, 5, 6, 23, 40])
    r = oracle.head_columns_backward(q, k, v, do, spec, 1, 3, cols, chunk=7)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    if p > 0:
        z = torch.from_numpy(oracle.dropout_keep(spec.seed, spec.offset, 1, 3, np.arange(n),
                                                 np.arange(n), p).astype(np.float64))
        o = _torch_explicit_dropout(tq, tk, tv, spec, z)
    else:
        o = _torch_sdpa(tq, tk, tv, spec)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(r["dk"], tk.grad.numpy()[cols], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(r["dv"], tv.grad.numpy()[cols], rtol=1e-10, atol=1e-11)

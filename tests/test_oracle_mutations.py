"""Plant plausible mistakes in the oracle (on the CPU) and check the pins fail.

Each mutant is the oracle's own source with one edit; it is loaded into a
copy of the oracle module, never into the real one.  A pin set that lets a
mutant through would be too weak to trust.
"""

import importlib.util
import inspect
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as attention

MUTANTS = {
    "drop_D_term": ("ds = f[\"p\"] * (dp - d_row[:, None])", "ds = f[\"p\"] * dp"),
    "sign_of_D": ("(dp - d_row[:, None])", "(dp + d_row[:, None])"),
    "dq_missing_scale": ("\"dq\": spec.sm_scale * (ds @ k[lo:hi])", "\"dq\": (ds @ k[lo:hi])"),
    "dk_transposed_ds": ("(ds.T @ q[rows])", "(ds @ q[rows])"),
    "dv_without_dropout": ("f[\"p_drop\"].T @ do[rows]", "f[\"p\"].T @ do[rows]"),
    "dp_without_dropout": ("dp = dp * f[\"z\"] / (1.0 - spec.dropout_p)", "dp = dp"),
    "dq_uses_v": ("(ds @ k[lo:hi])", "(ds @ v[lo:hi])"),
    "lse_without_max": ("lse[live] = m + np.log(ell)", "lse[live] = np.log(ell)"),
    "causal_off_by_one": ("ok &= j <= i", "ok &= j < i + 2"),
    "window_wrong_side": ("ok &= j >= i - spec.window_left", "ok &= j >= i - spec.window_left - 1"),
}

# Mistakes in the alignment of unequal query and key lengths
UNEQUAL_MUTANTS = {
    "shift_sign": ("shift = n - q.shape[0]", "shift = q.shape[0] - n"),
    "shift_left_out_of_mask": ("ok = valid_mask(rows, cols, spec, shift)",
                               "ok = valid_mask(rows, cols, spec)"),
    "shift_left_out_of_key_range": ("lo, hi = _key_range(rows, n, spec, shift)",
                                    "lo, hi = _key_range(rows, n, spec)"),
    "empty_rows_get_zero_lse": ("lse = np.full((len(rows), 1), -np.inf)",
                                "lse = np.full((len(rows), 1), 0.0)"),
}


# Mistakes in the selected-key-columns backward
COLUMN_MUTANTS = {
    "columns_only_rows_seeing_all": (".any(axis=1))[0]", ".all(axis=1))[0]"),
    "columns_dv_without_dropout": ("dv += p_drop.T @ do[rows]", "dv += p.T @ do[rows]"),
    "columns_dp_without_dropout": ("dp = dp * z / (1.0 - spec.dropout_p)", "dp = dp * z"),
    "columns_unscaled_dk": ("dk += spec.sm_scale * (ds.T @ q[rows])", "dk += (ds.T @ q[rows])"),
    # D from the selected keys only instead of the whole row
    "columns_local_D": ("d_row = (do[rows] * f[\"o\"]).sum(axis=1)\n        ds",
                        "d_row = (p * dp).sum(axis=1)\n        ds"),
}


def _load_mutant(old, new):
    src = inspect.getsource(attention)
    assert old in src, old
    src = src.replace(old, new)
    spec = importlib.util.spec_from_loader("oracle._mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__dict__["__package__"] = "oracle"
    sys.modules["oracle._mutant"] = mod
    exec(compile(src, "oracle/_mutant.py", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    """A compact run of the pins: torch autograd (with and without dropout)."""
    torch_dtype = torch.float64
    rng = np.random.default_rng(7)
    n, d = 24, 4
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    for kw in ({"causal": True}, {"window_left": 2, "window_right": 3},
               {"dropout_p": 0.3, "seed": 4}):
        sp = mod.Spec(sm_scale=0.6, **kw)
        r = mod.head_backward(q, k, v, do, sp)
        i = torch.arange(n).view(-1, 1)
        j = torch.arange(n).view(1, -1)
        ok = torch.ones(n, n, dtype=torch.bool)
        if sp.causal:
            ok &= j <= i
        if sp.window_left >= 0:
            ok &= j >= i - sp.window_left
        if sp.window_right >= 0:
            ok &= j <= i + sp.window_right
        tq, tk, tv = (torch.tensor(x, dtype=torch_dtype, requires_grad=True) for x in (q, k, v))
        s = ((tq @ tk.T) * sp.sm_scale).masked_fill(~ok, float("-inf"))
        p = torch.softmax(s, -1)
        if sp.dropout_p > 0:
            z = torch.tensor(oracle.dropout_keep(sp.seed, sp.offset, 0, 0, np.arange(n),
                                                 np.arange(n), sp.dropout_p), dtype=torch_dtype)
            p = p * z / (1 - sp.dropout_p)
        o = p @ tv
        o.backward(torch.tensor(do))
        for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
            if not np.allclose(r[name], t.grad.numpy(), rtol=1e-9, atol=1e-10):
                return False
        if not np.allclose(r["o"], o.detach().numpy(), rtol=1e-9, atol=1e-10):
            return False
    return True


def _unequal_pins_pass(mod):
    """A compact run of the unequal-length pin: torch's lower-right causal bias."""
    import warnings
    from torch.nn.attention.bias import causal_lower_right
    rng = np.random.default_rng(9)
    d = 4
    for nq, nk in ((5, 11), (11, 5)):
        q, do = rng.standard_normal((nq, d)), rng.standard_normal((nq, d))
        k, v = rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
        r = mod.head_backward(q, k, v, do, mod.Spec(sm_scale=0.6, causal=True))
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            bias = causal_lower_right(nq, nk)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(
            tq.view(1, 1, nq, d), tk.view(1, 1, nk, d), tv.view(1, 1, nk, d), attn_mask=bias,
            scale=0.6).view(nq, d)
        o.backward(torch.tensor(do))
        mask = bias._materialize(device="cpu").view(nq, nk)
        lse = torch.logsumexp(((tq @ tk.T) * 0.6).masked_fill(~mask, float("-inf")), -1)
        if not np.array_equal(np.isneginf(r["lse"]), np.isneginf(lse.detach().numpy())):
            return False
        live = np.isfinite(r["lse"])
        if not np.allclose(r["lse"][live], lse.detach().numpy()[live], rtol=1e-10):
            return False
        if not np.allclose(r["o"], o.detach().numpy(), rtol=1e-9, atol=1e-10):
            return False
        for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
            if not np.allclose(r[name], t.grad.numpy(), rtol=1e-9, atol=1e-10):
                return False
    return True


def _columns_pins_pass(mod):
    """A compact run of the key-columns pin: torch autograd columns of dK, dV."""
    rng = np.random.default_rng(13)
    n, d = 30, 6
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    cols = np.array([0, 3, 17, 29])
    for kw in ({"causal": True}, {"window_left": 4, "window_right": 2, "dropout_p": 0.3, "seed": 8}):
        sp = mod.Spec(sm_scale=0.7, **kw)
        r = mod.head_columns_backward(q, k, v, do, sp, 0, 0, cols, chunk=7)
        i = torch.arange(n).view(-1, 1)
        j = torch.arange(n).view(1, -1)
        ok = torch.ones(n, n, dtype=torch.bool)
        if sp.causal:
            ok &= j <= i
        if sp.window_left >= 0:
            ok &= (j >= i - sp.window_left) & (j <= i + sp.window_right)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        p = torch.softmax(((tq @ tk.T) * sp.sm_scale).masked_fill(~ok, float("-inf")), -1)
        if sp.dropout_p > 0:
            z = torch.tensor(oracle.dropout_keep(sp.seed, sp.offset, 0, 0, np.arange(n),
                                                 np.arange(n), sp.dropout_p), dtype=torch.float64)
            p = p * z / (1 - sp.dropout_p)
        (p @ tv).backward(torch.tensor(do))
        for name, t in (("dk", tk), ("dv", tv)):
            if not np.allclose(r[name], t.grad.numpy()[cols], rtol=1e-9, atol=1e-10):
                return False
    return True


def test_unmutated_oracle_passes_compact_pins():
    assert _pins_pass(_load_mutant("", ""))
    assert _unequal_pins_pass(_load_mutant("", ""))
    assert _columns_pins_pass(_load_mutant("", ""))


@pytest.mark.parametrize("name", list(COLUMN_MUTANTS))
def test_column_mutant_is_caught(name):
    old, new = COLUMN_MUTANTS[name]
    assert not _columns_pins_pass(_load_mutant(old, new)), name


@pytest.mark.parametrize("name", list(UNEQUAL_MUTANTS))
def test_unequal_length_mutant_is_caught(name):
    old, new = UNEQUAL_MUTANTS[name]
    assert not _unequal_pins_pass(_load_mutant(old, new)), name


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert not _pins_pass(_load_mutant(old, new)), name

"""The torch helpers of the binding check their tensors on the host before
anything reaches the C ABI (which sees raw pointers and cannot check sizes):
each mismatch below must raise ValueError without a GPU."""

import pytest
import torch

from flashattention_backward_pass_fa_amd import binding as fa

B, H, N, D = 2, 3, 40, 64


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _fixed():
    q = _t(B, H, N, D)
    return dict(q=q, k=_t(B, H, 50, D), v=_t(B, H, 50, D), o=_t(B, H, N, D), dout=_t(B, H, N, D),
                lse=_t(B, H, N, dtype=torch.float32))


def _backward(t, **kw):
    return fa.backward(t["q"], t["k"], t["v"], t["o"], t["dout"], t["lse"], causal=True, **kw)


def test_consistent_tensors_only_fail_for_being_on_the_host():
    with pytest.raises(ValueError, match="on a GPU"):
        _backward(_fixed())
    with pytest.raises(ValueError, match="on a GPU"):
        fa.forward(*(_fixed()[n] for n in ("q", "k", "v")))


@pytest.mark.parametrize("name,bad,match", [
    ("v", _t(B, H, 49, D), "same shape"),                      # V shorter than K
    ("k", _t(B, H, 50, 32), "same shape"),                     # K with another head dim than V
    ("o", _t(B, H, N - 1, D), "q's shape"),
    ("dout", _t(B, H + 1, N, D), "q's shape"),
    ("lse", _t(B, H, N - 1, dtype=torch.float32), "lse"),      # too short for the rows read
    ("lse", _t(B, H, N), "lse"),                               # wrong dtype
    ("o", _t(B, H, N, D, dtype=torch.float16), "dtype"),
    ("q", _t(B, H, N), "4-D"),
])
def test_backward_rejects(name, bad, match):
    t = _fixed()
    t[name] = bad
    if name == "k":
        t["v"] = _t(B, H, 50, D)
    with pytest.raises(ValueError, match=match):
        _backward(t)


def test_backward_rejects_mismatched_heads_between_q_and_k():
    t = _fixed()
    t["k"], t["v"] = _t(B, H + 1, 50, D), _t(B, H + 1, 50, D)
    with pytest.raises(ValueError, match="disagree"):
        _backward(t)


def test_float32_row_vectors_must_match_their_shape():
    """The check applied to a caller's lse and delta tensors."""
    cpu = torch.device("cpu")
    fa._check_f32(_t(B, H, N, dtype=torch.float32), "delta", (B, H, N), cpu)
    for bad in (_t(B, H, N - 1, dtype=torch.float32), _t(B, H, N), _t(B, H, 2 * N, dtype=torch.float32)[..., ::2]):
        with pytest.raises(ValueError, match="delta"):
            fa._check_f32(bad, "delta", (B, H, N), cpu)


def test_varlen_rejects_mismatched_packing():
    q = _t(70, H, D)
    k, v = _t(90, H, D), _t(89, H, D)
    with pytest.raises(ValueError, match="same shape"):
        fa._validate(q, k, v, varlen=True)
    with pytest.raises(ValueError, match="3-D"):
        fa._validate(_t(1, 70, H, D), _t(1, 90, H, D), _t(1, 90, H, D), varlen=True)
    with pytest.raises(ValueError, match="disagree"):
        fa._validate(q, _t(90, H, 32), _t(90, H, 32), varlen=True)


def test_missing_library_fails_loudly():
    """No fallback: a process whose library is not built gets an error on
    first use (run in a fresh interpreter, before anything is loaded)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import flashattention_backward_pass_fa_amd.binding as b\n"
            "try:\n    b.load_library('/nonexistent/libfa.so')\n"
            "except RuntimeError as e:\n    print('raised:', e)\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert "raised:" in out.stdout and "not built" in out.stdout, out.stdout + out.stderr

"""Plain fp64 attention forward and backward with S, P and dS materialised.

TEST INFRASTRUCTURE ONLY (part of the CPU oracle). It is slow on purpose and
shares no code with the GPU path; only tests, the smoke check and the CPU
baseline leg of the benchmark may call it.

Everything is computed from the definitions on the pages, in binary64:

  S = sm_scale * Q K^T, masked to -inf   "Lecture 7", section "The math" and
                                          "Mask behaviour"
  L_i = m_i + log l_i  (natural log)      "FlashAttention backward", section
                                          "What the forward left behind"
  P = exp(S - L)                          same section; "Lecture 7", "The
                                          recomputation trick"
  P~ = P * Z / (1 - p)  (dropout)         "Lecture 7", section "Dropout"
  O = P~ V
  dV = P~^T dO;  dP~ = dO V^T;  dP = dP~ * Z / (1 - p)
  D_i = sum_k dO_ik O_ik                  "FlashAttention backward", section
                                          "The gradients, and the one scalar
                                          that makes them local"
  dS = P * (dP - D)
  dQ = sm_scale * dS K;  dK = sm_scale * dS^T Q

The pages write the scale as 1/sqrt(d); a general sm_scale multiplies S and
the dQ/dK products in the same places.  Dropout is differentiated by the
chain rule through P~ (the pages do not derive it); the same D is correct
because sum_j P_ij dP_ij = sum_j P~_ij (dO_i . V_j) = dO_i . O_i.

Rows are processed in groups only to bound memory: every row always sees its
complete key row, and dK/dV are the plain sum of the per-row contributions.
Key columns that are masked for every row of a group are left out of that
group's products (their P is exactly 0).
"""

from dataclasses import dataclass

import numpy as np

from . import philox


@dataclass(frozen=True)
class Spec:
    """Flags of one attention call (same meaning as the library's fa_params)."""

    sm_scale: float
    causal: bool = False
    window_left: int = -1   # -1: unbounded; else keys j >= i - window_left
    window_right: int = -1  # -1: unbounded; else keys j <= i + window_right
    dropout_p: float = 0.0
    seed: int = 0
    offset: int = 0


def valid_mask(rows, cols, spec):
    """valid(i, j): key j is visible to query i ("Lecture 7", "Mask behaviour").

    Causal hides j > i; a window keeps i - window_left <= j <= i + window_right.
    """
    i = np.asarray(rows, dtype=np.int64).reshape(-1, 1)
    j = np.asarray(cols, dtype=np.int64).reshape(1, -1)
    ok = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if spec.causal:
        ok &= j <= i
    if spec.window_left >= 0:
        ok &= j >= i - spec.window_left
    if spec.window_right >= 0:
        ok &= j <= i + spec.window_right
    return ok


def _key_range(rows, n, spec):
    """Smallest [lo, hi) holding every key visible to at least one of rows."""
    r0, r1 = int(np.min(rows)), int(np.max(rows))
    lo, hi = 0, n
    if spec.causal:
        hi = min(hi, r1 + 1)
    if spec.window_left >= 0:
        lo = max(lo, r0 - spec.window_left)
    if spec.window_right >= 0:
        hi = min(hi, r1 + spec.window_right + 1)
    return lo, max(lo, hi)


def _row_groups(n, chunk):
    step = n if chunk is None else max(1, int(chunk))
    for start in range(0, n, step):
        yield np.arange(start, min(n, start + step))


def head_rows_forward(q, k, v, spec, b, h, rows):
    """Forward quantities of one head for the query rows `rows`.

    q, k, v: [N, d] arrays (any float dtype; widened to fp64).
    Returns a dict with the key range and the materialised S, P, Z, P~, O, L.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = k.shape[0]
    lo, hi = _key_range(rows, n, spec)
    cols = np.arange(lo, hi)
    ok = valid_mask(rows, cols, spec)
    s = spec.sm_scale * (q[rows] @ k[lo:hi].T)
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    ell = np.exp(s - m).sum(axis=1, keepdims=True)
    lse = m + np.log(ell)
    p = np.exp(s - lse)  # exactly 0 where the score is -inf
    if spec.dropout_p > 0.0:
        z = philox.dropout_keep(spec.seed, spec.offset, b, h, rows, cols, spec.dropout_p)
        p_drop = p * z / (1.0 - spec.dropout_p)
    else:
        z = None
        p_drop = p
    o = p_drop @ v[lo:hi]
    return {"lo": lo, "hi": hi, "s": s, "p": p, "z": z, "p_drop": p_drop,
            "o": o, "lse": lse[:, 0]}


def head_forward(q, k, v, spec, b=0, h=0, chunk=None):
    """O [N, d] and L [N] of one head."""
    n, dv = q.shape[0], v.shape[1]
    o = np.zeros((n, dv))
    lse = np.zeros(n)
    for rows in _row_groups(n, chunk):
        f = head_rows_forward(q, k, v, spec, b, h, rows)
        o[rows] = f["o"]
        lse[rows] = f["lse"]
    return o, lse


def head_rows_backward(q, k, v, do, spec, b, h, rows):
    """Backward quantities of one head for the query rows `rows`.

    Returns the forward dict of head_rows_forward extended with dP, D, dS and
    the rows' dQ plus their contributions to dK/dV over the key range.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    f = head_rows_forward(q, k, v, spec, b, h, rows)
    lo, hi = f["lo"], f["hi"]
    dp = do[rows] @ v[lo:hi].T
    if f["z"] is not None:
        dp = dp * f["z"] / (1.0 - spec.dropout_p)
    d_row = (do[rows] * f["o"]).sum(axis=1)
    ds = f["p"] * (dp - d_row[:, None])
    f.update({
        "dp": dp,
        "delta": d_row,
        "ds": ds,
        "dq": spec.sm_scale * (ds @ k[lo:hi]),
        "dk_part": spec.sm_scale * (ds.T @ q[rows]),
        "dv_part": f["p_drop"].T @ do[rows],
    })
    return f


def head_backward(q, k, v, do, spec, b=0, h=0, chunk=None):
    """dQ, dK, dV (and O, L, D) of one head, from the definitions above."""
    n = q.shape[0]
    dq = np.zeros((n, q.shape[1]))
    dk = np.zeros((n, k.shape[1]))
    dv = np.zeros((n, v.shape[1]))
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    delta = np.zeros(n)
    for rows in _row_groups(n, chunk):
        r = head_rows_backward(q, k, v, do, spec, b, h, rows)
        lo, hi = r["lo"], r["hi"]
        o[rows] = r["o"]
        lse[rows] = r["lse"]
        delta[rows] = r["delta"]
        dq[rows] = r["dq"]
        dk[lo:hi] += r["dk_part"]
        dv[lo:hi] += r["dv_part"]
    return {"dq": dq, "dk": dk, "dv": dv, "o": o, "lse": lse, "delta": delta}


def head_delta(o, do):
    """D_i = rowsum(dO * O) for given O and dO of one head ([N, d] each)."""
    return (np.asarray(do, dtype=np.float64) * np.asarray(o, dtype=np.float64)).sum(axis=1)


def forward(q, k, v, spec, heads=None, chunk=None):
    """O [B,H,N,d] and L [B,H,N] for all heads (or only the listed (b, h))."""
    bsz, nh, n, _ = q.shape
    o = np.zeros(q.shape[:3] + (v.shape[3],))
    lse = np.zeros((bsz, nh, n))
    for b, h in (heads if heads is not None else np.ndindex(bsz, nh)):
        o[b, h], lse[b, h] = head_forward(q[b, h], k[b, h], v[b, h], spec, b, h, chunk)
    return o, lse


def backward(q, k, v, do, spec, heads=None, chunk=None):
    """dQ, dK, dV, O, L, D for [B,H,N,d] inputs (all heads or the listed ones).

    Heads that are not listed are left at zero.
    """
    bsz, nh, n, d = q.shape
    out = {"dq": np.zeros((bsz, nh, n, d)), "dk": np.zeros((bsz, nh, n, d)),
           "dv": np.zeros((bsz, nh, n, v.shape[3])), "o": np.zeros((bsz, nh, n, v.shape[3])),
           "lse": np.zeros((bsz, nh, n)), "delta": np.zeros((bsz, nh, n))}
    for b, h in (heads if heads is not None else np.ndindex(bsz, nh)):
        r = head_backward(q[b, h], k[b, h], v[b, h], do[b, h], spec, b, h, chunk)
        for name in out:
            out[name][b, h] = r[name]
    return out


def dropout_mask(spec, b, h, n):
    """The full N x N keep mask Z of head (b, h) (uint8), for small N."""
    idx = np.arange(n)
    return philox.dropout_keep(spec.seed, spec.offset, b, h, idx, idx, spec.dropout_p)


def credited_flops(bsz, nh, n, d, spec):
    """10 * d per visible (b, h, i, j): the five N x N x d products of the backward."""
    visible = 0
    step = 4096
    for start in range(0, n, step):
        rows = np.arange(start, min(n, start + step))
        visible += int(valid_mask(rows, np.arange(n), spec).sum())
    return 10.0 * d * visible * bsz * nh


def saved_state_bytes(n, d, elem_bytes=2):
    """Per-head bytes of what the backward keeps: O (N x d) plus fp32 L and D.

    "FlashAttention backward", section "Worked numbers": the O(N d) state that
    replaces the materialised P.
    """
    return n * d * elem_bytes + n * 4 * 2


def materialised_p_bytes(n, elem_bytes=2):
    """Per-head bytes of a stored N x N probability matrix."""
    return n * n * elem_bytes

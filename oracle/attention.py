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
the dQ/dK products in the same places.

Queries and keys may differ in number (Nq, Nk).  The pages fix no alignment
for that case; this oracle aligns the last query with the last key, so query
i stands at key position i + Nk - Nq for the causal and window tests.  A row
that then sees no key has an empty softmax sum: L = log 0 = -inf, P = 0,
O = 0, and every gradient through it is 0.  Variable-length batches
(varlen_backward) are each sequence on its own, with its batch index b.
Dropout is differentiated by the chain rule through P~ (the pages do not
derive it); the same D is correct because
sum_j P_ij dP_ij = sum_j P~_ij (dO_i . V_j) = dO_i . O_i.

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


def valid_mask(rows, cols, spec, shift=0):
    """valid(i, j): key j is visible to query i ("Lecture 7", "Mask behaviour").

    Query i stands at key position i + shift (shift = Nk - Nq).  Causal hides
    keys after that position; a window keeps window_left keys before it and
    window_right keys after it.
    """
    i = np.asarray(rows, dtype=np.int64).reshape(-1, 1) + shift
    j = np.asarray(cols, dtype=np.int64).reshape(1, -1)
    ok = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if spec.causal:
        ok &= j <= i
    if spec.window_left >= 0:
        ok &= j >= i - spec.window_left
    if spec.window_right >= 0:
        ok &= j <= i + spec.window_right
    return ok


def _key_range(rows, n, spec, shift=0):
    """Smallest [lo, hi) holding every key visible to at least one of rows."""
    r0, r1 = int(np.min(rows)) + shift, int(np.max(rows)) + shift
    lo, hi = 0, n
    if spec.causal:
        hi = min(hi, r1 + 1)
    if spec.window_left >= 0:
        lo = max(lo, r0 - spec.window_left)
    if spec.window_right >= 0:
        hi = min(hi, r1 + spec.window_right + 1)
    lo = min(lo, n)
    return lo, max(lo, hi)


def _row_groups(n, chunk):
    step = n if chunk is None else max(1, int(chunk))
    for start in range(0, n, step):
        yield np.arange(start, min(n, start + step))


def head_rows_forward(q, k, v, spec, b, h, rows):
    """Forward quantities of one head for the query rows `rows`.

    q: [Nq, d], k, v: [Nk, d] arrays (any float dtype; widened to fp64).
    Returns a dict with the key range and the materialised S, P, Z, P~, O, L.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = k.shape[0]
    shift = n - q.shape[0]
    lo, hi = _key_range(rows, n, spec, shift)
    cols = np.arange(lo, hi)
    ok = valid_mask(rows, cols, spec, shift)
    s = spec.sm_scale * (q[rows] @ k[lo:hi].T)
    s = np.where(ok, s, -np.inf)
    # rows that see no key keep L = -inf and P = 0 (an empty sum)
    live = ok.any(axis=1)
    lse = np.full((len(rows), 1), -np.inf)
    p = np.zeros_like(s)
    if live.any():
        sl = s[live]
        m = sl.max(axis=1, keepdims=True)
        ell = np.exp(sl - m).sum(axis=1, keepdims=True)
        lse[live] = m + np.log(ell)
        p[live] = np.exp(sl - lse[live])  # exactly 0 where the score is -inf
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
    """O [Nq, d] and L [Nq] of one head."""
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
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
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


def head_columns_backward(q, k, v, do, spec, b, h, cols, chunk=None):
    """dK and dV of the key rows `cols` of one head ([len(cols), d] each).

    dK_j = sm_scale * sum_i dS_ij Q_i and dV_j = sum_i P~_ij dO_i, summed over
    every query row i that sees one of the keys ("Lecture 7", section "The
    math").  Each such row is taken whole: its L and O come from
    head_rows_forward over its complete key row, D_i = rowsum(dO_i * O_i)
    ("FlashAttention backward", section "The gradients, and the one scalar
    that makes them local") and dS = P * (dP - D).  The cost is that of the
    rows that see the keys, not of the whole head.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    cols = np.asarray(cols, dtype=np.int64)
    nq, n = q.shape[0], k.shape[0]
    shift = n - nq
    seeing = np.nonzero(valid_mask(np.arange(nq), cols, spec, shift).any(axis=1))[0]
    dk = np.zeros((len(cols), q.shape[1]))
    dv = np.zeros((len(cols), v.shape[1]))
    step = len(seeing) if chunk is None else max(1, int(chunk))
    for start in range(0, len(seeing), step):
        rows = seeing[start:start + step]
        f = head_rows_forward(q, k, v, spec, b, h, rows)
        ok = valid_mask(rows, cols, spec, shift) & np.isfinite(f["lse"])[:, None]
        s = spec.sm_scale * (q[rows] @ k[cols].T)
        p = np.zeros_like(s)
        p[ok] = np.exp((s - np.where(ok, f["lse"][:, None], 0.0))[ok])
        dp = do[rows] @ v[cols].T
        if spec.dropout_p > 0.0:
            z = philox.dropout_keep(spec.seed, spec.offset, b, h, rows, cols, spec.dropout_p)
            p_drop = p * z / (1.0 - spec.dropout_p)
            dp = dp * z / (1.0 - spec.dropout_p)
        else:
            p_drop = p
        d_row = (do[rows] * f["o"]).sum(axis=1)
        ds = p * (dp - d_row[:, None])
        dk += spec.sm_scale * (ds.T @ q[rows])
        dv += p_drop.T @ do[rows]
    return {"dk": dk, "dv": dv}


def forward(q, k, v, spec, heads=None, chunk=None):
    """O [B,H,Nq,d] and L [B,H,Nq] for all heads (or only the listed (b, h))."""
    bsz, nh, n, _ = q.shape
    o = np.zeros(q.shape[:3] + (v.shape[3],))
    lse = np.zeros((bsz, nh, n))
    for b, h in (heads if heads is not None else np.ndindex(bsz, nh)):
        o[b, h], lse[b, h] = head_forward(q[b, h], k[b, h], v[b, h], spec, b, h, chunk)
    return o, lse


def backward(q, k, v, do, spec, heads=None, chunk=None):
    """dQ, dK, dV, O, L, D for [B,H,Nq,d] queries and [B,H,Nk,d] keys/values.

    All heads or the listed ones; heads that are not listed are left at zero.
    """
    bsz, nh, n, d = q.shape
    out = {"dq": np.zeros((bsz, nh, n, d)), "dk": np.zeros(k.shape),
           "dv": np.zeros(v.shape), "o": np.zeros((bsz, nh, n, v.shape[3])),
           "lse": np.zeros((bsz, nh, n)), "delta": np.zeros((bsz, nh, n))}
    for b, h in (heads if heads is not None else np.ndindex(bsz, nh)):
        r = head_backward(q[b, h], k[b, h], v[b, h], do[b, h], spec, b, h, chunk)
        for name in out:
            out[name][b, h] = r[name]
    return out


def varlen_backward(q, k, v, do, cu_q, cu_k, spec, chunk=None):
    """The backward of a packed variable-length batch, one sequence at a time.

    q, do: [total_q, H, d]; k, v: [total_k, H, d]; sequence b owns rows
    cu_q[b]:cu_q[b+1] of q and cu_k[b]:cu_k[b+1] of k.  Returns packed O, dQ,
    dK, dV and L, D as [B, H, max query length] (NaN past each length).
    """
    bsz = len(cu_q) - 1
    nh = q.shape[1]
    max_q = max(int(cu_q[b + 1] - cu_q[b]) for b in range(bsz))
    out = {"dq": np.zeros(q.shape), "dk": np.zeros(k.shape), "dv": np.zeros(v.shape),
           "o": np.zeros(q.shape[:2] + (v.shape[2],)),
           "lse": np.full((bsz, nh, max_q), np.nan), "delta": np.full((bsz, nh, max_q), np.nan)}
    for b in range(bsz):
        qs, ks = slice(int(cu_q[b]), int(cu_q[b + 1])), slice(int(cu_k[b]), int(cu_k[b + 1]))
        nq = qs.stop - qs.start
        for h in range(nh):
            if nq == 0:
                continue
            r = head_backward(q[qs, h], k[ks, h], v[ks, h], do[qs, h], spec, b, h, chunk)
            for name in ("dq", "o"):
                out[name][qs, h] = r[name]
            for name in ("dk", "dv"):
                out[name][ks, h] = r[name]
            out["lse"][b, h, :nq] = r["lse"]
            out["delta"][b, h, :nq] = r["delta"]
    return out


def dropout_mask(spec, b, h, n, n_k=None):
    """The full Nq x Nk keep mask Z of head (b, h) (uint8), for small sizes."""
    return philox.dropout_keep(spec.seed, spec.offset, b, h, np.arange(n),
                               np.arange(n if n_k is None else n_k), spec.dropout_p)


def credited_flops(bsz, nh, n, d, spec, n_k=None):
    """10 * d per visible (b, h, i, j): the five N x N x d products of the backward."""
    n_k = n if n_k is None else n_k
    visible = 0
    step = 4096
    for start in range(0, n, step):
        rows = np.arange(start, min(n, start + step))
        visible += int(valid_mask(rows, np.arange(n_k), spec, n_k - n).sum())
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

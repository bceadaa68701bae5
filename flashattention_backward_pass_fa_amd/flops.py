"""Work accounting of the backward: credited FLOPs and algorithmic bytes.

Credited FLOPs are 10 d per visible (b, h, i, j): the backward's five
N x N x d products (S = Q K^T, dP = dO V^T, dV = P~^T dO, dK = dS^T Q,
dQ = dS K), 2 d FLOPs each ("FlashAttention backward", section "Worked
numbers": the backward costs about 2.5 times the forward's two products).
Algorithmic bytes are what the backward must move at least once: read Q, K,
V, dO, O (the last for D), L and D, write D, dQ, dK, dV.
"""

import numpy as np


def visible_pairs(n, causal=False, window_left=-1, window_right=-1, n_k=None):
    """Number of (i, j) with key j visible to query i, in closed form per row.

    n queries over n_k keys (default n); query i stands at key position
    i + n_k - n (the last query aligned with the last key).
    """
    n_k = n if n_k is None else n_k
    i = np.arange(n, dtype=np.int64) + (n_k - n)
    lo = np.zeros(n, dtype=np.int64)
    hi = np.full(n, n_k, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, i + 1)
    if window_left >= 0:
        lo = np.maximum(lo, i - window_left)
    if window_right >= 0:
        hi = np.minimum(hi, i + window_right + 1)
    return int(np.maximum(hi - lo, 0).sum())


def credited_flops(B, H, n, d, causal=False, window_left=-1, window_right=-1, n_k=None):
    return 10.0 * d * B * H * visible_pairs(n, causal, window_left, window_right, n_k)


def algorithmic_bytes(B, H, n, d, elem_bytes=2):
    """Reads of Q, K, V, dO, O, L, D; writes of D, dQ, dK, dV (no workspace)."""
    per_head = 8 * n * d * elem_bytes + 12 * n
    return float(B * H * per_head)


def tile_fraction(n, causal, window_left, window_right, br, bc):
    """Fraction of (br x bc) tiles that hold at least one visible pair."""
    live = 0
    total = 0
    for q0 in range(0, n, br):
        for k0 in range(0, n, bc):
            total += 1
            q1, k1 = min(n, q0 + br) - 1, min(n, k0 + bc) - 1
            dead = False
            if causal and k0 > q1:
                dead = True
            if window_left >= 0 and k1 < q0 - window_left:
                dead = True
            if window_right >= 0 and k0 > q1 + window_right:
                dead = True
            live += 0 if dead else 1
    return live / total

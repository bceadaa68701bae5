"""Configurations whose whole-tensor bf16 bars the method's own rounding
misses, and a model of that rounding.

The backward takes D_i = rowsum(dO o O) from the stored forward output O
("FlashAttention backward", section "The gradients, and the one scalar that
makes them local"), and dS = P o (dP - D) ("Lecture 7 — Backward Pass and
Validation", section "The math").  When a row sees a single key, dP_i and
D_i are one dot product computed two ways, so dS is zero in exact
arithmetic, and what the backward returns there is the rounding of O carried
through D.  A tensor whose exact value is built mostly from such rows (or
whose D is a near-cancelling sum) then has a relative error set by bf16's
unit roundoff, whatever the kernels do.

The model is the oracle with only the method's 16-bit rounding points added:
the forward's unnormalised weights and its stored O, and dS before the dQ and
dK products, each rounded to bf16 (round to nearest even); every sum stays in
fp64.  The GPU test of each configuration below checks every other tensor at
the stated bars and bounds each named tensor by a small multiple of the
model's error (test_gpu_sweep.MODEL_FACTOR).

Each configuration is written out in full.  Eight were drawn by the random
sweep's generator (index i: the generator's draw i, with dropout seed 77 + i
and offset i); two by variants of it with longer sequences and with packed
batches whose head count is a multiple of 8 (same seed rule).
"""

import numpy as np

import oracle
from oracle import attention as A
from flashattention_backward_pass_fa_amd.inputs import cumulative, make_tensors

# (index, configuration, tensors the rounding takes past their bars, which bar
# of the first).  Where a sequence's queries see a single key, that key's dK
# is a sum of the same rounding over the sequence's rows, so dK joins dQ.
KNOWN = [
    # 152 queries over a single key: that key's dK is zero exactly, and its
    # error (the O roundings summed over 152 rows) sets the dK maximum
    (3675, {"dtype": "bf16", "d": 128, "H": 2, "causal": False, "window": (-1, -1), "p": 0.15,
            "det": False, "scale": 0.0945639701433859, "varlen": True, "seed": 4675,
            "lq": [152, 271], "lk": [1, 95]}, ("dk",), "max"),
    # one query over 352 keys: a D of 0.002 from terms summing to 3.3
    (6936, {"dtype": "bf16", "d": 64, "H": 3, "causal": False, "window": (-1, -1), "p": 0.0,
            "det": True, "scale": 0.110950346886966, "varlen": True, "seed": 7936,
            "lq": [1], "lk": [352]}, ("delta",), "fro"),
    # 212 queries over 2 keys: two live rows per head, one of them single-key
    (19313, {"dtype": "bf16", "d": 128, "H": 2, "causal": True, "window": (54, 92), "p": 0.15,
             "det": False, "scale": 0.08276878638826188, "varlen": True, "seed": 20313,
             "lq": [212], "lk": [2]}, ("dq", "dk"), "fro"),
    # 262 queries over 2 keys, the same shape of problem
    (24832, {"dtype": "bf16", "d": 64, "H": 1, "causal": True, "window": (46, 212), "p": 0.15,
             "det": True, "scale": 0.12756641831735635, "varlen": True, "seed": 25832,
             "lq": [262], "lk": [2]}, ("dq", "dk"), "fro"),
    # one query over 316 keys
    (24551, {"dtype": "bf16", "d": 64, "H": 1, "causal": True, "window": (-1, 274), "p": 0.0,
             "det": True, "scale": 0.07881147684436546, "varlen": True, "seed": 25551,
             "lq": [1], "lk": [316]}, ("delta",), "max"),
    # 2 x 2, causal: the first row sees one key
    (24585, {"dtype": "bf16", "d": 64, "H": 1, "causal": True, "window": (-1, -1), "p": 0.15,
             "det": False, "scale": 0.04434036723118326, "varlen": False, "seed": 25585,
             "B": 2, "Nq": 2, "Nk": 2, "bnhd": False}, ("delta",), "fro"),
    # 2 x 2
    (26382, {"dtype": "bf16", "d": 64, "H": 1, "causal": False, "window": (-1, -1), "p": 0.0,
             "det": False, "scale": 0.048390318096789606, "varlen": True, "seed": 27382,
             "lq": [2], "lk": [2]}, ("dk",), "fro"),
    # a packed sequence of 52 queries over a single key
    (26888, {"dtype": "bf16", "d": 128, "H": 1, "causal": False, "window": (18, -1), "p": 0.15,
             "det": True, "scale": 0.05352565032580898, "varlen": True, "seed": 27888,
             "lq": [52, 99, 214, 372], "lk": [1, 284, 110, 266]}, ("dk",), "max"),
    # longer sequences: a packed batch with 479 queries over a single key
    (4711, {"dtype": "bf16", "d": 128, "H": 1, "causal": False, "window": (-1, -1), "p": 0.15,
            "det": False, "scale": 0.08996833498363563, "varlen": True, "seed": 5711,
            "lq": [1110, 479, 1743, 1653], "lk": [1110, 1, 1743, 1836]}, ("dq", "dk"), "max"),
    # eight heads, two sequences: 388 queries over a single key
    (307, {"dtype": "bf16", "d": 128, "H": 8, "causal": False, "window": (154, -1), "p": 0.15,
           "det": False, "scale": 0.11727776093365443, "varlen": True, "seed": 1307,
           "lq": [759, 388], "lk": [759, 1]}, ("dq", "dk"), "fro"),
]

# indices of KNOWN drawn by the committed sweep generator itself
FROM_SWEEP_GENERATOR = (3675, 6936, 19313, 24832, 24551, 24585, 26382, 26888)


def spec_of(c, i):
    """The oracle flags of configuration c with index i."""
    return oracle.Spec(sm_scale=c["scale"], causal=c["causal"], window_left=c["window"][0],
                       window_right=c["window"][1], dropout_p=c["p"], seed=77 + i, offset=i)


def host_inputs(c):
    """Seeded inputs of configuration c (packed [total, H, d] when varlen)."""
    H, d, dtype = c["H"], c["d"], c["dtype"]
    if c["varlen"]:
        cu_q, cu_k = cumulative(c["lq"]), cumulative(c["lk"])
        kv = (int(cu_k[-1]), H, d)
        return make_tensors((int(cu_q[-1]), H, d), dtype, c["seed"], shapes={"k": kv, "v": kv})
    kv = (c["B"], H, c["Nk"], d)
    return make_tensors((c["B"], H, c["Nq"], d), dtype, c["seed"], shapes={"k": kv, "v": kv})


def _bf16(x):
    """Round to bf16 (nearest even) through fp32, returned as fp64."""
    bits = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    bits = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def _model_head(q, k, v, do, spec, b, h):
    """dQ, dK and D of one sequence-head with bf16 rounding at the 16-bit
    operands and at the O store, everything else exact."""
    f = A.head_rows_backward(q, k, v, do, spec, b, h, np.arange(q.shape[0]))
    lo, hi = f["lo"], f["hi"]
    s = f["s"]
    seen = np.isfinite(s)
    live = seen.any(axis=1)
    m = np.where(live, np.max(np.where(seen, s, -np.inf), axis=1, initial=-np.inf), 0.0)
    e = np.where(seen, np.exp(s - m[:, None]), 0.0)  # weights before normalising, 1 at the max
    ell = np.where(live, e.sum(axis=1), 1.0)
    keep = f["z"] if f["z"] is not None else 1.0
    vv = np.asarray(v, np.float64)[lo:hi]
    o = _bf16(np.where(live[:, None], (_bf16(e * keep) @ vv) / ell[:, None] / (1.0 - spec.dropout_p), 0.0))
    d_row = (np.asarray(do, np.float64) * o).sum(axis=1)
    ds = _bf16(f["p"] * (f["dp"] - d_row[:, None]))
    dk = np.zeros(np.shape(k))
    dk[lo:hi] = spec.sm_scale * (ds.T @ np.asarray(q, np.float64))
    return {"dq": spec.sm_scale * (ds @ np.asarray(k, np.float64)[lo:hi]), "dk": dk, "delta": d_row}


def model_case(c, i):
    """The oracle's result and the rounding model's for configuration c, in
    the layouts the GPU tests compare, and the inputs' magnitudes."""
    assert c["dtype"] == "bf16"
    spec = spec_of(c, i)
    host = host_inputs(c)
    mags = {n: float(np.abs(host[n]).max()) for n in ("q", "k", "v", "do")}
    if not c["varlen"]:
        ref = oracle.backward(host["q"], host["k"], host["v"], host["do"], spec)
        model = {n: np.zeros(ref[n].shape) for n in ("dq", "dk", "delta")}
        for b in range(c["B"]):
            for h in range(c["H"]):
                r = _model_head(host["q"][b, h], host["k"][b, h], host["v"][b, h], host["do"][b, h], spec, b, h)
                for n in model:
                    model[n][b, h] = r[n]
        return spec, host, ref, model, mags
    cu_q, cu_k = cumulative(c["lq"]), cumulative(c["lk"])
    ref = oracle.varlen_backward(host["q"], host["k"], host["v"], host["do"], cu_q, cu_k, spec)
    model = {"dq": np.zeros(ref["dq"].shape), "dk": np.zeros(ref["dk"].shape),
             "delta": np.full(ref["delta"].shape, np.nan)}
    for b in range(len(cu_q) - 1):
        qs, ks = slice(int(cu_q[b]), int(cu_q[b + 1])), slice(int(cu_k[b]), int(cu_k[b + 1]))
        if qs.stop == qs.start:
            continue
        for h in range(c["H"]):
            r = _model_head(host["q"][qs, h], host["k"][ks, h], host["v"][ks, h], host["do"][qs, h], spec, b, h)
            model["dq"][qs, h] = r["dq"]
            model["dk"][ks, h] = r["dk"]
            model["delta"][b, h, :qs.stop - qs.start] = r["delta"]
    return spec, host, ref, model, mags


def query_rows(c):
    """Longest query sequence of configuration c (bounds a column sum of P)."""
    return max(c["lq"]) if c["varlen"] else c["Nq"]

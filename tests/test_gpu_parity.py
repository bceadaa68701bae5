"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small problems are compared element by element in full (they span several
tiles and a ragged tail).  The measured full-size workloads run in the
launch configuration the benchmark times, in both dQ modes: the training
shape is compared on every head, the larger two on a few full heads and on
sampled rows and keys of every head.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_cases import Case, compare, to_host, assert_close

pytestmark = pytest.mark.gpu


def _run_and_compare(case, deterministic=False, heads=None):
    print(f"\n[gpu] {case} deterministic={deterministic} heads={heads}", flush=True)
    host = case.host_inputs()
    dev = case.device_inputs(host)
    gpu = case.run_gpu(dev, deterministic=deterministic)
    ref = case.run_oracle(host, heads=heads)
    return compare(case, gpu, ref, heads=heads, names=("o", "delta", "dq", "dk", "dv"), host=host)


# ------------------------------------------------------- the five workloads

@pytest.mark.parametrize("deterministic", [False, True])
def test_tiny_fp32(deterministic):
    _run_and_compare(Case(1, 1, 128, 64, "f32", seed=1001), deterministic)


@pytest.mark.parametrize("deterministic", [False, True])
def test_small_causal_bf16(deterministic):
    _run_and_compare(Case(2, 4, 1024, 64, "bf16", causal=True, seed=1002), deterministic)


# The three large workloads, in both dQ modes, in the launch configuration
# the benchmark times.  The training shape is compared on every head in
# full.  The two larger ones are compared in full on a few heads, and on
# every head on samples the oracle can compute on their own: 16 random query
# rows (O, L, D, dQ of those rows; head_rows_backward takes each row whole)
# and a run of 8 consecutive keys (dK, dV of those keys, from every row that
# sees them; head_columns_backward).  A sample meets the same bars as a whole
# tensor, taken over the sampled values.
FULL_SIZE = {
    # name: (case, fully compared heads (None: all), last keys the sampled key runs start in)
    "train_causal": (Case(4, 16, 4096, 128, "bf16", causal=True, seed=1003), None, None),
    "window_dropout": (Case(2, 16, 8192, 64, "bf16", window=(1023, 1023), dropout_p=0.1, seed=1004),
                       [(0, 0), (1, 13), (0, 9), (1, 4)], None),
    # keys near the end: the rows that see them are few enough to take whole
    "long_causal": (Case(1, 8, 32768, 128, "bf16", causal=True, seed=1005), [(0, 5), (0, 2)], 2048),
}

_oracle_cache = {}


def _full_size_oracle(name):
    """Inputs and oracle result of a large workload, computed once for both modes."""
    if name not in _oracle_cache:
        _oracle_cache.clear()  # hold one workload at a time
        case, heads, _ = FULL_SIZE[name]
        host = case.host_inputs()
        _oracle_cache[name] = (host, case.run_oracle(host, heads=heads))
    return _oracle_cache[name]


def _sampled_rows_and_keys(case, host, gpu, key_window, seed):
    spec = case.spec()
    B, H, N, _ = case.shape
    rng = np.random.default_rng(seed)
    got = {n: to_host(gpu[n]) for n in ("o", "lse", "delta", "dq", "dk", "dv")}
    g = {n: [] for n in got}
    w = {n: [] for n in got}
    for b in range(B):
        for h in range(H):
            args = (host["q"][b, h], host["k"][b, h], host["v"][b, h], host["do"][b, h])
            rows = np.sort(rng.choice(N, 16, replace=False))
            r = oracle.head_rows_backward(*args, spec, b, h, rows)
            for n in ("o", "lse", "delta", "dq"):
                g[n].append(got[n][b, h][rows])
                w[n].append(r[n])
            lo = 0 if key_window is None else N - key_window
            j0 = int(rng.integers(lo, N - 8 + 1))
            cols = np.arange(j0, j0 + 8)
            c = oracle.head_columns_backward(*args, spec, b, h, cols, chunk=1024)
            for n in ("dk", "dv"):
                g[n].append(got[n][b, h][cols])
                w[n].append(c[n])
    for n in ("o", "delta", "dq", "dk", "dv"):
        assert_close(f"sampled {n}", np.concatenate(g[n]), np.concatenate(w[n]), case.dtype)
    lse_err = float(np.abs(np.concatenate(g["lse"]) - np.concatenate(w["lse"])).max())
    assert lse_err <= 1e-3, f"sampled lse: max|err| {lse_err:.3e}"


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("name", list(FULL_SIZE))
def test_full_size_workload(name, deterministic):
    case, heads, key_window = FULL_SIZE[name]
    print(f"\n[gpu] {name}: {case} deterministic={deterministic} heads={heads or 'all'}", flush=True)
    host, ref = _full_size_oracle(name)
    gpu = case.run_gpu(case.device_inputs(host), deterministic=deterministic)
    compare(case, gpu, ref, heads=heads, names=("o", "delta", "dq", "dk", "dv"), host=host)
    if heads is not None:
        _sampled_rows_and_keys(case, host, gpu, key_window, seed=case.seed + 17 * deterministic)


# ------------------------------------------- ragged shapes and every flag

RAGGED = [
    # (B, H, N, d, causal, window, p)
    (1, 2, 1, 64, False, (-1, -1), 0.0),
    (1, 2, 77, 64, True, (-1, -1), 0.0),
    (2, 1, 130, 128, False, (-1, -1), 0.0),
    (1, 3, 1000, 64, True, (-1, -1), 0.0),
    (1, 2, 1000, 128, False, (100, 37), 0.0),
    (1, 2, 515, 64, True, (200, -1), 0.0),
    (2, 2, 700, 128, False, (-1, 0), 0.0),
    (1, 2, 333, 64, False, (-1, -1), 0.25),
    (1, 2, 600, 128, True, (-1, -1), 0.1),
    (1, 1, 900, 64, False, (64, 64), 0.3),
    # head counts that are multiples of 8 with block counts padded to 4
    # (the launch-index remap): 6 -> 8 and 3 -> 4 blocks
    (2, 4, 700, 64, True, (-1, -1), 0.0),
    (1, 16, 300, 128, False, (40, 9), 0.1),
    # d = 64 with too many workgroups for the one-launch small-problem path
    # (2 * 16 heads x (8 + 4) blocks > 256): the two separate kernels
    (2, 16, 1000, 64, True, (-1, -1), 0.0),
]


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("B,H,N,d,causal,window,p", RAGGED)
def test_ragged_bf16(B, H, N, d, causal, window, p, deterministic):
    _run_and_compare(Case(B, H, N, d, "bf16", causal=causal, window=window, dropout_p=p,
                          seed=7 + N + d), deterministic)


# fp16: the same kernels compiled for fp16 (no workload on the pages uses it)
F16 = [
    (1, 2, 77, 64, True, (-1, -1), 0.0),
    (2, 2, 300, 128, True, (-1, -1), 0.0),
    (1, 2, 1000, 64, False, (100, 37), 0.0),
    (1, 2, 600, 128, True, (-1, -1), 0.1),
    (1, 1, 900, 64, False, (64, 64), 0.3),
]


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("B,H,N,d,causal,window,p", F16)
def test_ragged_fp16(B, H, N, d, causal, window, p, deterministic):
    rep = _run_and_compare(Case(B, H, N, d, "f16", causal=causal, window=window, dropout_p=p,
                                seed=11 + N + d), deterministic)
    print("[gpu] errors", {k: tuple(float(f"{x:.3g}") for x in v) for k, v in rep.items()}, flush=True)


@pytest.mark.parametrize("deterministic", [False, True])
def test_train_causal_fp16_sampled_heads(deterministic):
    rep = _run_and_compare(Case(4, 16, 4096, 128, "f16", causal=True, seed=1006), deterministic,
                           heads=[(0, 0), (3, 15)])
    print("[gpu] errors", {k: tuple(float(f"{x:.3g}") for x in v) for k, v in rep.items()}, flush=True)


@pytest.mark.parametrize("B,H,N,d,causal,window,p", [
    (1, 2, 1, 32, False, (-1, -1), 0.0),
    (2, 2, 100, 40, True, (-1, -1), 0.0),
    (1, 1, 257, 128, False, (30, 5), 0.2),
    (1, 2, 200, 64, True, (50, -1), 0.0),
])
def test_ragged_fp32(B, H, N, d, causal, window, p):
    _run_and_compare(Case(B, H, N, d, "f32", causal=causal, window=window, dropout_p=p, seed=3 + N))


def test_non_default_scale_and_strided_layout():
    """[B, N, H, d] storage (a transposed view) and sm_scale != 1/sqrt(d)."""
    import torch
    from flashattention_backward_pass_fa_amd import binding as fa
    case = Case(2, 3, 300, 64, "bf16", causal=True, seed=99, sm_scale=0.2)
    print(f"\n[gpu] strided {case}", flush=True)
    host = case.host_inputs()
    dev = case.device_inputs(host)
    # same values, stored as [B, N, H, d] and viewed back as [B, H, N, d]
    dev = {k: v.transpose(1, 2).contiguous().transpose(1, 2) for k, v in dev.items()}
    assert dev["q"].stride(2) == 3 * 64
    gpu = case.run_gpu(dev)
    ref = case.run_oracle(host)
    compare(case, gpu, ref, names=("o", "dq", "dk", "dv"))


def test_isolated_backward_from_oracle_forward():
    """Feed the oracle's O (rounded to bf16) and L into the GPU backward."""
    import torch
    case = Case(1, 4, 777, 128, "bf16", causal=True, seed=5)
    print(f"\n[gpu] isolation {case}", flush=True)
    host = case.host_inputs()
    dev = case.device_inputs(host)
    ref = case.run_oracle(host)
    o = torch.from_numpy(ref["o"].astype(np.float32)).to(torch.bfloat16).cuda()
    lse = torch.from_numpy(ref["lse"].astype(np.float32)).cuda()
    gpu = case.run_gpu(dev, o=o, lse=lse)
    for name in ("dq", "dk", "dv"):
        assert_close(name, to_host(gpu[name]), ref[name], "bf16")


@pytest.mark.parametrize("dtype,deterministic", [("bf16", True), ("f32", False), ("bf16", False)])
def test_preprocess_writes_workspace_only_in_atomic_mode(dtype, deterministic):
    """fa_bwd_preprocess zeroes dq_acc in atomic mode and leaves it alone otherwise.

    The buffer is full size in every case, so a wrong write lands in bounds and
    shows up as changed values."""
    import ctypes
    import torch
    from flashattention_backward_pass_fa_amd import binding as fa
    case = Case(1, 2, 96, 64, dtype, causal=True, seed=7)
    print(f"\n[gpu] preprocess workspace {case} deterministic={deterministic}", flush=True)
    dev = case.device_inputs(case.host_inputs())
    code = fa.FA_DTYPE_BF16 if dtype == "bf16" else fa.FA_DTYPE_F32
    params = fa.make_params(case.shape, code, causal=True, deterministic=deterministic)
    ws = torch.full((1 * 2 * 96 * 64,), 7.0, dtype=torch.float32, device="cuda")
    delta = torch.empty((1, 2, 96), dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    o = dev["q"]  # any [B, H, N, d] tensor stands in for O here
    assert fa.fa_bwd_preprocess(params, fa.tensor_arg(o), fa.tensor_arg(dev["do"]),
                                ctypes.c_void_p(delta.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                st) == 0
    torch.cuda.synchronize()
    used = fa.fa_bwd_workspace_bytes(params) > 0
    assert used == (dtype == "bf16" and not deterministic)
    assert torch.all(ws == (0.0 if used else 7.0)).item()


def test_longest_sequence_sampled_rows():
    """N = 2^21, the longest sequence the library takes, with a two-sided
    window (every row sees at most 251 keys).  Three row ranges [a, b) are
    checked against the oracle run on the sub-problem of rows and keys
    [a - wl, b + wr) (the window is translation-invariant, so those rows see
    the same keys there): O, L, dQ on [a, b), and dK, dV on the keys whose
    every visible query lies in [a, b), which the sub-problem sums whole."""
    import numpy as np
    import oracle
    from tests.gpu_cases import Case, to_host
    n, wl, wr = 1 << 21, 200, 50
    case = Case(1, 1, n, 64, "bf16", window=(wl, wr), seed=21)
    print(f"\n[gpu] longest {case}", flush=True)
    host = case.host_inputs()
    dev = case.device_inputs(host)
    gpu = case.run_gpu(dev, deterministic=True)
    got = {name: to_host(gpu[name])[0, 0] for name in ("o", "dq", "dk", "dv")}
    got_l = to_host(gpu["lse"])[0, 0]
    spec = case.spec()
    for a, b in ((0, 4096), (n // 2 - 2048, n // 2 + 2048), (n - 4096, n)):
        s0, e0 = max(0, a - wl), min(n, b + wr)
        sub = {name: host[name][0, 0, s0:e0] for name in ("q", "k", "v", "do")}
        r = oracle.head_backward(sub["q"], sub["k"], sub["v"], sub["do"], spec)
        for name in ("o", "dq"):
            assert_close(name, got[name][a:b], r[name][a - s0:b - s0], "bf16")
        assert float(np.abs(got_l[a:b] - r["lse"][a - s0:b - s0]).max()) <= 1e-3
        k0 = a + wr if a > 0 else 0
        k1 = b - wl if b < n else n
        for name in ("dk", "dv"):
            assert_close(name, got[name][k0:k1], r[name][k0 - s0:k1 - s0], "bf16")


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("dtype,d,causal,window", [
    ("bf16", 128, True, (-1, -1)),
    ("bf16", 64, False, (90, 30)),
    ("f16", 128, True, (-1, -1)),
    ("f32", 64, True, (-1, -1)),
])
def test_sharp_softmax(dtype, d, causal, window, deterministic):
    """sm_scale = 8/sqrt(d): scores with std ~ 8, nearly one-hot rows, so the
    exponentials span many orders of magnitude."""
    import math
    _run_and_compare(Case(2, 2, 700, d, dtype, causal=causal, window=window, seed=500 + d,
                          sm_scale=8.0 / math.sqrt(d)), deterministic)

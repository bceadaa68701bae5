"""fa_bwd_noalloc, the backward whose atomic-mode dQ workspace is the
library's static device array, against fa_bwd with a caller workspace.

Both are called through the C ABI on the same inputs, twice in a row with
the second problem smaller than the first (the array keeps the first call's
contents, which the second must clear).  dK and dV come from the same
kernels in the same order and must be identical; dQ is summed with fp32
atomics in an order that varies run to run, so it is held to the bf16 bars
against fa_bwd's dQ.  Deterministic mode (no workspace) must match fa_bwd
exactly.
"""

import ctypes

import numpy as np
import pytest

from flashattention_backward_pass_fa_amd import binding as fa
from tests.gpu_cases import Case, assert_close, to_host

pytestmark = pytest.mark.gpu

VOID = ctypes.c_void_p


def _both(case, deterministic, stream):
    """dQ, dK, dV from fa_bwd (caller workspace) and from fa_bwd_noalloc."""
    import torch
    host = case.host_inputs()
    dev = case.device_inputs(host)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], **case.kw())
    params = fa.make_params(case.shape, fa.FA_DTYPE_BF16, deterministic=deterministic, **case.kw())
    delta = torch.empty(case.shape[:3], dtype=torch.float32, device="cuda")
    ws_bytes = fa.fa_bwd_workspace_bytes(params)
    ws = torch.empty(max(1, ws_bytes // 4), dtype=torch.float32, device="cuda")
    ws_ptr = VOID(ws.data_ptr() if ws_bytes else 0)
    T = fa.tensor_arg
    st = VOID(stream.cuda_stream)
    assert fa.fa_bwd_preprocess(params, T(o), T(dev["do"]), VOID(delta.data_ptr()), ws_ptr, st) == 0
    ref = [torch.empty_like(dev["q"]) for _ in range(3)]
    assert fa.fa_bwd(params, T(dev["q"]), T(dev["k"]), T(dev["v"]), T(dev["do"]), VOID(lse.data_ptr()),
                     VOID(delta.data_ptr()), *(T(x) for x in ref), ws_ptr, st) == 0
    got = [torch.empty_like(dev["q"]) for _ in range(3)]
    assert fa.fa_bwd_noalloc(params, T(dev["q"]), T(dev["k"]), T(dev["v"]), T(dev["do"]),
                             VOID(lse.data_ptr()), VOID(delta.data_ptr()), *(T(x) for x in got), st) == 0
    stream.synchronize()
    return [to_host(x) for x in ref], [to_host(x) for x in got]


@pytest.mark.parametrize("deterministic", [False, True])
def test_noalloc_matches_fa_bwd_twice(deterministic):
    import torch
    stream = torch.cuda.current_stream()
    cases = [Case(2, 8, 1024, 128, "bf16", causal=True, seed=51),
             Case(1, 3, 333, 64, "bf16", window=(40, 17), dropout_p=0.1, seed=52)]
    for case in cases:
        print(f"\n[gpu] noalloc {case} deterministic={deterministic}", flush=True)
        ref, got = _both(case, deterministic, stream)
        for name, r, g in zip(("dq", "dk", "dv"), ref, got):
            assert np.isfinite(g).all(), name
            if deterministic or name != "dq":
                assert np.array_equal(r, g), name
            else:
                assert_close(name, g, r, "bf16")

"""The torch-facing helpers on a stream that is not torch's current one.

The helpers allocate their outputs and temporaries (atomic mode's fp32 dQ
workspace, D) with torch's caching allocator.  Passed `stream=`, they must
allocate on that stream: a temporary allocated on the current stream and
freed on return could be handed to the next current-stream allocation while
the kernels on the caller's stream still accumulate into it.
"""

import numpy as np
import pytest

from flashattention_backward_pass_fa_amd import binding as fa
from tests.gpu_cases import Case, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("deterministic", [False, True])
def test_backward_on_side_stream(deterministic):
    import torch
    case = Case(2, 8, 2048, 128, "bf16", causal=True, seed=41)
    print(f"\n[gpu] side stream: {case} deterministic={deterministic}", flush=True)
    host = case.host_inputs()
    dev = case.device_inputs(host)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], **case.kw())
    want = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, deterministic=deterministic,
                       **case.kw())
    torch.cuda.synchronize()
    params = fa.make_params(case.shape, fa.FA_DTYPE_BF16, deterministic=deterministic, **case.kw())
    ws_floats = max(1, fa.fa_bwd_workspace_bytes(params) // 4)
    side = torch.cuda.Stream()
    for _ in range(3):
        got = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, deterministic=deterministic,
                          stream=side, **case.kw())
        # current-stream work of the workspace's and D's sizes while the side
        # stream runs: it must not land in the side stream's memory
        junk = [torch.full((ws_floats,), float("nan"), device="cuda"),
                torch.full(case.shape[:3], float("nan"), device="cuda")]
        side.synchronize()
        torch.cuda.synchronize()
        del junk
        for name, g, w in zip(("dq", "dk", "dv", "delta"), got, want):
            g, w = to_host(g), to_host(w)
            assert np.isfinite(g).all(), name
            if deterministic or name != "dq":
                assert np.array_equal(g, w), name  # same kernels, same order
            else:
                # atomic mode: the order of the fp32 adds may differ run to run
                assert float(np.abs(g - w).max()) <= 2e-2 * float(np.abs(w).max()), name

"""moe_forward_noalloc (the entry point for callers that cannot allocate) against
moe_forward with a caller workspace, through the C ABI.

Both run the same kernels, so outputs and routing must be bit-identical; the
output is also checked against the fp64 oracle at the layer's tolerance.  Two
calls in a row, the second smaller, on each kernel path: the fixed scratch keeps
the first call's contents, which the second call must not depend on.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
from gpu_util import SMALL, check_forward, check_route, device_weights, log, moe_cfg, to_dev, y_to_f64

pytestmark = pytest.mark.gpu

# (workload, first T, second T): prefill then decode, decode then decode
CASES = [(2, 300, 40), (3, 64, 1), (5, 500, 130), (7, 300, 13)]


@pytest.mark.parametrize("cid,T1,T2", CASES)
def test_noalloc_matches_forward(cid, T1, T2):
    import mixture_experts_layer_03_amd as moe
    spec = SMALL[cid]
    L = synth.make_layer(spec)
    W = device_weights(L)
    cfg = moe_cfg(spec)
    for T in (T1, T2):
        x = synth.make_x(spec, T)
        xd = to_dev(x)
        log(f"no-alloc cfg{cid} {spec.name} T={T} ({cfg.kernel_path(T)} kernels)")
        assert cfg.workspace_size(T) <= moe._lib.NOALLOC_SCRATCH_BYTES
        y0, (i0, w0, c0) = moe.forward(xd, W, cfg, return_routing=True)
        y1, (i1, w1, c1) = moe.forward_noalloc(xd, W, cfg, return_routing=True)
        torch.cuda.synchronize()
        assert torch.equal(i0, i1) and torch.equal(w0, w1) and torch.equal(c0, c1), "routing differs"
        assert torch.equal(y0, y1), "outputs differ from moe_forward"
        check_route(spec, i1.cpu().numpy(), w1.cpu().numpy(), L, x)
        sf = check_forward(spec, y_to_f64(y1), i1.cpu().numpy(), L, x)
        log(f"  ok: bit-identical to moe_forward, max rel err {sf['max_rel']:.3e} against the oracle")


"""The persistent dW GEMM (one block per CU walking the tiles), plain and
pipelined (the next tile's first stages load while a tile stores), against
the one-tile-per-block launch: bitwise equal dW and dH, overwritten and
accumulated (each tile keeps its summation order).  The launch form is chosen
with STREAMBP_PERSISTENT_DW (0 one tile per block, 1 plain, 2 pipelined);
D = 200 is off the 256 tile grid, where the pipelined form falls back to the
plain one."""
import os

import numpy as np
import pytest
import torch

from tests.gpu_helpers import head, require_gpu, to_dev
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [dict(T=1100, D=512, V=50000, C=512), dict(T=2 * 1024 + 333, D=1024, V=151936, C=1024),
                                   dict(T=700, D=200, V=60003, C=256)])
def test_persistent_dw_bitwise(shape):
    require_gpu()
    wl = gen.SFT_9K.with_(**shape)
    print(f"[case] persistent_dw {shape}", flush=True)
    d = to_dev(gen.make_inputs(wl, 4))
    outs = []
    try:
        for flag in ("0", "1", "2"):
            os.environ["STREAMBP_PERSISTENT_DW"] = flag
            hd = head(wl.D, wl.V, wl.C, wl.dtype)
            base = torch.full((wl.V, wl.D), 0.25, device="cuda")
            loss, dH, dW, nv = hd.sft(d["H"], d["W"], d["y"])
            acc = base.clone()
            hd.sft(d["H"], d["W"], d["y"], dW=acc, accumulate=True)
            torch.cuda.synchronize()
            outs.append((dW.clone(), acc.clone(), dH.clone()))
    finally:
        os.environ.pop("STREAMBP_PERSISTENT_DW", None)
    (w0, a0, h0) = outs[0]
    for mode, (w1, a1, h1) in ((1, outs[1]), (2, outs[2])):
        nd = int((w0 != w1).sum()) + int((a0 != a1).sum())
        print(f"  mode {mode}: differing dW elements: {nd} of {2 * w0.numel()}", flush=True)
        if nd:
            idx = torch.nonzero(w0 != w1)
            print(f"  first differing (v, d): {idx[:8].tolist()}", flush=True)
        assert torch.equal(h0, h1)
        assert nd == 0

"""The SFT entry point that allocates nothing (static device scratch) against
the workspace entry point, through the C interface: two calls in a row on
one device, the second with fewer rows, each bitwise equal to
streambp_head_sft on the same inputs (same kernels, fixed summation orders)
and within the bf16 tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import streambp_oracle as O
from tests.gpu_helpers import TOL_BF16, head, np64, rel, require_gpu, to_dev
from workloads import gen

pytestmark = pytest.mark.gpu


def _run_both(hd, wl, seed):
    inp = gen.make_inputs(wl, seed)
    d = to_dev(inp)
    assert hd.workspace_bytes(wl.T, 1) <= hd.lib.streambp_head_workspace_bytes(hd._h, wl.T, 1)
    loss_a, dH_a, dW_a, nv_a = hd.sft(d["H"], d["W"], d["y"])
    torch.cuda.synchronize()
    dH_b = torch.full_like(dH_a, float("nan"))
    dW_b = torch.full_like(dW_a, float("nan"))
    loss_b = torch.full_like(loss_a, float("nan"))
    nv_b = torch.full_like(nv_a, -1)
    hd.sft_noalloc(d["H"], d["W"], d["y"], dH_b, dW_b, loss_b, nv_b)
    torch.cuda.synchronize()
    return inp, (loss_a, dH_a, dW_a, nv_a), (loss_b, dH_b, dW_b, nv_b)


def test_sft_noalloc_matches_workspace_entry_twice():
    require_gpu()
    from loss_head_amd import _capi
    big = gen.SFT_9K.with_(name="sft_bf16_t700_d512_v151936", T=700, D=512, V=151936, C=128)
    small = big.with_(name="sft_bf16_t300_d512_v151936", T=300)
    hd = head(big.D, big.V, big.C, big.dtype)
    need = hd.workspace_bytes(big.T, 1)
    print(f"[case] sft_noalloc T={big.T} then T={small.T}, D={big.D} V={big.V} C={big.C}; "
          f"workspace {need} of {_capi.STATIC_SCRATCH_BYTES} bytes", flush=True)
    assert need <= _capi.STATIC_SCRATCH_BYTES
    for wl, seed in ((big, 1), (small, 2)):
        inp, a, b = _run_both(hd, wl, seed)
        for x, y, name in zip(a, b, ("loss", "dH", "dW", "n_valid")):
            assert torch.equal(x, y), f"{wl.name}: {name} differs from the workspace entry point"
        ref = O.sft(inp.H, inp.W, inp.labels)
        assert int(b[3].item()) == ref.scan.n_valid
        e = (abs(b[0].item() - ref.loss) / abs(ref.loss), rel(np64(b[1]), ref.dH), rel(np64(b[2]), ref.dW))
        print(f"  {wl.name}: bitwise equal to streambp_head_sft; vs oracle loss/dH/dW {e[0]:.2e} {e[1]:.2e} "
              f"{e[2]:.2e}", flush=True)
        assert max(e) <= TOL_BF16


def test_sft_noalloc_rejects_calls_beyond_the_scratch():
    require_gpu()
    from loss_head_amd import HeadError
    wl = gen.SFT_9K.with_(T=64, D=256, V=151936, C=1024)   # C x V bf16 alone is 311 MB
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    d = to_dev(gen.make_inputs(wl, 0))
    dH = torch.empty((wl.T, wl.D), device="cuda")
    dW = torch.empty((wl.V, wl.D), device="cuda")
    loss = torch.empty(1, dtype=torch.float64, device="cuda")
    nv = torch.empty(1, dtype=torch.int64, device="cuda")
    with pytest.raises(HeadError, match="WORKSPACE_TOO_SMALL"):
        hd.sft_noalloc(d["H"], d["W"], d["y"], dH, dW, loss, nv)

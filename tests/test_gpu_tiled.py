"""GPU: the tiled logits operands (W and each chunk's H copied into 256 x 32
storage tiles, logits GEMM through the deeper k = 32 pipeline) give the same
results as the plain path, bit for bit: the same products are accumulated in
the same k order.  The plain path is checked against the fp64 oracle by the
parity tests; one case here also checks the tiled path against the oracle
directly."""
import numpy as np
import pytest
import torch

from oracle import streambp_oracle as O
from tests.gpu_helpers import TOL_BF16, head, np64, rel, require_gpu, to_dev
from workloads import gen

pytestmark = pytest.mark.gpu


def _case(name, **kw):
    print(f"[case] tiled {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _same(a, b):
    assert a.dtype == b.dtype and a.shape == b.shape
    assert torch.equal(a, b), f"max |diff| {(a.double() - b.double()).abs().max().item():.3e}"


SFT_SHAPES = [
    dict(T=333, D=200, V=1003, C=112),      # D off the 32-wide k tile, ragged vocabulary and tail chunk
    dict(T=1100, D=1024, V=20000, C=512),   # several token and vocabulary tiles
    dict(T=300, D=72, V=5003, C=300),       # fewer k-stages than the pipeline's depth
]


@pytest.mark.parametrize("shape", SFT_SHAPES, ids=lambda s: "T{T}_D{D}_V{V}_C{C}".format(**s))
@pytest.mark.parametrize("compact", [False, True], ids=["plain_loop", "compacted"])
def test_sft_tiled_equals_plain(shape, compact):
    require_gpu()
    _case("sft", compact=compact, **shape)
    wl = gen.SFT_9K.with_(mask="random", mask_frac=0.2, **shape)
    d = to_dev(gen.make_inputs(wl, 3))
    out = []
    for tiled in (False, True):
        hd = head(wl.D, wl.V, wl.C, wl.dtype, compact=compact, tiled=tiled)
        loss, dH, dW, nv = hd.sft(d["H"], d["W"], d["y"])
        torch.cuda.synchronize()
        assert int(hd.status.item()) == 0
        out.append((loss.clone(), dH.clone(), dW.clone(), nv.clone()))
    for a, b in zip(*out):
        _same(a, b)


def test_sft_tiled_against_oracle():
    require_gpu()
    wl = gen.SFT_9K.with_(T=600, D=520, V=8000, C=256)
    _case("sft_oracle", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = gen.make_inputs(wl, 1)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype, tiled=True)
    loss, dH, dW, _ = hd.sft(d["H"], d["W"], d["y"])
    torch.cuda.synchronize()
    ref = O.sft(inp.H, inp.W, inp.labels)
    assert abs(loss.item() - ref.loss) / abs(ref.loss) <= TOL_BF16
    assert rel(np64(dH), ref.dH) <= TOL_BF16 and rel(np64(dW), ref.dW) <= TOL_BF16


def test_grpo_and_ppo_tiled_equal_plain():
    require_gpu()
    wl = gen.PPO.with_(T=3 * 111, D=200, V=1003, C=100, n_seq=3)
    _case("grpo_ppo", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    old = torch.from_numpy(inp.logp_old.astype(np.float32)).cuda()
    ref = torch.from_numpy(inp.logp_ref.astype(np.float32)).cuda()
    out = []
    for tiled in (False, True):
        hd = head(wl.D, wl.V, wl.C, wl.dtype, tiled=tiled)
        g = [t.clone() for t in hd.grpo(d["H"], d["W"], d["y"], d["off"], d["adv"])]
        p = [t.clone() for t in hd.ppo(d["H"], d["W"], d["y"], d["off"], d["adv"], old, ref, 0.1, 0.2)]
        torch.cuda.synchronize()
        assert int(hd.status.item()) == 0
        out.append(g + p)
    for a, b in zip(*out):
        _same(a, b)


def test_dpo_tiled_equals_plain():
    require_gpu()
    wl = gen.DPO.with_(T=4 * 256, D=512, V=9000, C=256, n_seq=4)
    _case("dpo", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    out = []
    for tiled in (False, True):
        hd = head(wl.D, wl.V, wl.C, wl.dtype, tiled=tiled)
        res = [t.clone() for t in hd.dpo(d["H"], d["W"], d["y"], d["off"], d["ref"], 0.1)]
        torch.cuda.synchronize()
        assert int(hd.status.item()) == 0
        out.append(res)
    for a, b in zip(*out):
        _same(a, b)

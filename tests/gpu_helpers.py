"""Shared helpers of the GPU tests: upload seeded inputs, run the HIP path,
compare with the oracle."""
import numpy as np
import pytest
import torch

from workloads import gen

# Tolerances: relative Frobenius error against the fp64 oracle.
TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def head(D, V, C, dtype, compact=False, tiled=False):
    from loss_head_amd import Head  # raises if the HIP library is not built
    return Head(D, V, C, dtype, compact=compact, tiled_logits=tiled)


def to_dev(inp: gen.Inputs):
    dev = torch.device("cuda", 0)
    if inp.wl.dtype == "bf16":
        H = torch.from_numpy(inp.H.view(np.int16)).view(torch.bfloat16).to(dev)
        W = torch.from_numpy(inp.W.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        H = torch.from_numpy(inp.H).to(dev)
        W = torch.from_numpy(inp.W).to(dev)
    y = torch.from_numpy(inp.labels.astype(np.int32)).to(dev)
    off = torch.from_numpy(inp.offsets.astype(np.int32)).to(dev)
    out = dict(H=H, W=W, y=y, off=off)
    if inp.adv is not None:
        out["adv"] = torch.from_numpy(inp.adv.astype(np.float32)).to(dev)
    if inp.ref_logp is not None:
        out["ref"] = torch.from_numpy(np.asarray(inp.ref_logp, dtype=np.float64)).to(dev)
    return out


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def np64(t):
    return t.detach().double().cpu().numpy()


def loss_rel(got, want, scale):
    """|loss - loss*| / max(|loss*|, scale): the GRPO value can be near 0, so the
    scale includes sum_t |w_t logp_t|."""
    return abs(got - want) / max(abs(want), scale, 1e-300)

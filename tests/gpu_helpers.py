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


ROW_FACTOR = 2.0


def row_check(got, want, tol, what="", absval=None, row_scale=None):
    """Row-wise comparison, beside the whole-tensor Frobenius one.

    Every row's error ||got_r - want_r|| must be within ROW_FACTOR * tol
    times the row's size (the worst of hundreds of rows, against a tolerance
    stated for the whole tensor), rows that are exactly 0 in `want` must be
    exactly 0, and no element
    may be off by more than tol times its own size plus 0.1 of the row's rms
    size (a lost or stale element fails this even when the row's norm hides
    it).  The size of a row is ||want_r||, or larger where given:
    * `absval`: the product of the operands' absolute values, |G| |W| for dH
      and |G|^T |H| for dW (the standard componentwise bound of a product: a
      row that is a small difference of large terms carries the rounding of
      those terms, relative to them and not to the difference);
    * `row_scale` (per row): the size of a PPO row before the cancellation
      inside its weight (see ppo_row_scale).
    Returns the largest row error in those units."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    got2 = got.reshape(got.shape[0], -1)
    want2 = want.reshape(want.shape[0], -1)
    size = np.abs(want2)
    if absval is not None:
        size = np.maximum(size, np.asarray(absval, dtype=np.float64).reshape(size.shape))
    nrm = np.linalg.norm(want2, axis=1)
    zero = nrm == 0
    den = np.maximum(nrm, np.linalg.norm(size, axis=1))
    if row_scale is not None:
        den = np.maximum(den, np.asarray(row_scale, dtype=np.float64))
    assert np.all(got2[zero] == 0.0), f"{what}: rows that must be 0 are not"
    if (~zero).any():
        err = np.linalg.norm(got2[~zero] - want2[~zero], axis=1) / den[~zero]
        worst = int(np.argmax(err))
        assert err[worst] <= ROW_FACTOR * tol, f"{what}: row {np.nonzero(~zero)[0][worst]} rel err {err[worst]:.3e}"
        rms = (den[~zero] / np.sqrt(want2.shape[1]))[:, None]
        bad = np.abs(got2[~zero] - want2[~zero]) > tol * size[~zero] + 0.1 * rms
        assert not bad.any(), f"{what}: {int(bad.sum())} elements off, first at {np.argwhere(bad)[0]}"
        return float(err.max())
    return 0.0


def abs_products(H, W, labels, ref):
    """|G| |W| and |G|^T |H| (fp64) for an oracle result `ref` on small inputs,
    G the dlogits of the definition with the result's weights."""
    from oracle import streambp_oracle as O
    Hd, Wd = O.widen(H), O.widen(W)
    G = np.abs(O.grad_logits(O.logits(Hd, Wd), ref.lse, np.asarray(labels, dtype=np.int64), ref.scan.valid, ref.w))
    return G @ np.abs(Wd), G.T @ np.abs(Hd)


def ppo_row_scale(dH_want, ell, valid, adv_per_len, inv_len, logp_old, logp_ref, eps, beta_kl):
    """Per-row scale of a PPO dH row before cancellation: the row is w_t u_t
    with w_t = (slope of the surrogate) + (slope of the KL term); where the two
    nearly cancel, fp32 evaluation of w_t has a relative error far above fp32
    epsilon although each term is exact to it.  Scale = ||dH_t|| (|s1| + |s2|) / |w_t|."""
    ell = np.asarray(ell, dtype=np.float64)
    a = np.asarray(adv_per_len, dtype=np.float64)
    r = np.exp(ell - np.asarray(logp_old, dtype=np.float64))
    un, cl = r * a, np.clip(r, 1 - eps, 1 + eps) * a
    s1 = np.where(un <= cl, a * r, 0.0)
    s2 = np.zeros_like(ell) if logp_ref is None or beta_kl == 0 else \
        beta_kl * np.asarray(inv_len) * np.expm1(np.asarray(logp_ref, dtype=np.float64) - ell)
    w = s1 + s2
    nrm = np.linalg.norm(np.asarray(dH_want, dtype=np.float64).reshape(len(ell), -1), axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(valid & (w != 0), nrm * (np.abs(s1) + np.abs(s2)) / np.abs(w), 0.0)
    return sc


def kl_steps(T, seed=7):
    """Seeded steps logp_ref - logp for the off-policy tests: random sign,
    magnitude 0.25 + 0.5 |N(0,1)|, never near 0."""
    rng = np.random.default_rng(seed)
    return np.where(rng.random(T) < 0.5, -1.0, 1.0) * (0.25 + 0.5 * np.abs(rng.standard_normal(T)))

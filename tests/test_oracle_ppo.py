"""Pins of the oracle's off-policy clipped-surrogate head (PPO / off-policy
GRPO with a KL penalty) against facts that do not come from the oracle:
finite differences of its loss, torch fp64 autograd through an independent
writing of the objective, the on-policy reduction to GRPO, and closed forms
(fully clipped, KL at its minimum).  A planted mistake in the per-token terms
must fail at least one of them."""
import numpy as np
import pytest
import torch

from oracle import streambp_oracle as O

EPS = 0.2


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def _problem(seed, T=10, D=4, V=7, n_seq=3, masked=(1, 6)):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((T, D))
    W = rng.standard_normal((V, D))
    y = rng.integers(0, V, T)
    y[list(masked)] = O.IGNORE_INDEX
    off = np.linspace(0, T, n_seq + 1).astype(np.int64)
    adv = np.array([1.1, -0.8, 0.6])[:n_seq]
    ell = O.sft(H, W, y).logp                      # current log-probs of the labels
    # old log-probs a fixed step away, so that the ratio r = exp(logp - old)
    # takes the values e^0.6, e^0.05, e^-0.05, e^-0.6: clipped on either side
    # for one sign of A and inside the range otherwise, never near 1 +- EPS
    steps = np.array([-0.6, -0.05, 0.05, 0.6])
    old = ell - steps[np.arange(T) % 4]
    ref = ell + rng.standard_normal(T) * 0.5
    return H, W, y, off, adv, old, ref


def _torch_loss(H, W, y, off, adv, old, ref, eps, beta):
    """The same objective written with torch ops, fp64, for autograd."""
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    lp = torch.log_softmax(Ht @ Wt.T, dim=-1)
    yt = torch.tensor(y)
    valid = yt != -100
    tok = lp.gather(1, yt.clamp(min=0)[:, None])[:, 0]
    loss = torch.zeros((), dtype=torch.float64)
    for s in range(len(off) - 1):
        lo, hi = int(off[s]), int(off[s + 1])
        v = valid[lo:hi]
        n = int(v.sum())
        if n == 0:
            continue
        lt = tok[lo:hi][v]
        r = torch.exp(lt - torch.tensor(old[lo:hi])[v])
        surr = -torch.minimum(r * adv[s], torch.clamp(r, 1 - eps, 1 + eps) * adv[s])
        d = torch.tensor(ref[lo:hi])[v] - lt
        kl = torch.exp(d) - d - 1
        loss = loss + (surr.sum() + beta * kl.sum()) / n
    loss.backward()
    return loss.item(), Ht.grad.numpy(), Wt.grad.numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("beta", [0.0, 0.3])
def test_ppo_torch_autograd(seed, beta):
    H, W, y, off, adv, old, ref = _problem(seed)
    r = O.ppo(H, W, y, off, adv, old, ref, EPS, beta)
    loss, gH, gW = _torch_loss(H, W, y, off, adv, old, ref, EPS, beta)
    assert abs(r.loss - loss) <= 1e-12 * max(1.0, abs(loss))
    assert _rel(r.dH, gH) < 1e-12 and _rel(r.dW, gW) < 1e-12


@pytest.mark.parametrize("seed", [0, 1])
def test_ppo_finite_differences(seed):
    H, W, y, off, adv, old, ref = _problem(seed, T=8, n_seq=2, masked=(1, 5))
    beta = 0.3
    r = O.ppo(H, W, y, off, adv, old, ref, EPS, beta)
    f = lambda: O.ppo(H, W, y, off, adv, old, ref, EPS, beta).loss
    h = 1e-6
    for X, G in ((H, r.dH), (W, r.dW)):
        fd = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            x0 = X[idx]
            X[idx] = x0 + h
            fp = f()
            X[idx] = x0 - h
            fm = f()
            X[idx] = x0
            fd[idx] = (fp - fm) / (2 * h)
        assert _rel(G, fd) < 1e-6


def test_ppo_on_policy_reduces_to_grpo():
    # old = current log-probs (ratio exactly 1, inside the clip range) and no
    # KL: the gradient is on-policy GRPO's, and the surrogate's value is
    # -sum_s A_s over sequences with valid tokens
    H, W, y, off, adv, _, _ = _problem(3)
    g = O.grpo(H, W, y, off, adv)
    r = O.ppo(H, W, y, off, adv, g.logp, None, EPS, 0.0)
    np.testing.assert_allclose(r.dH, g.dH, rtol=1e-15, atol=0)
    np.testing.assert_allclose(r.dW, g.dW, rtol=1e-15, atol=0)
    want = -sum(adv[s] for s in range(len(off) - 1) if g.scan.seq_len[s] > 0)
    assert abs(r.loss - want) <= 1e-15 * abs(want)


def test_ppo_fully_clipped_has_zero_gradient():
    # every ratio beyond the binding side of the clip range (above 1+eps for
    # A > 0, below 1-eps for A < 0): the surrogate is flat, loss is
    # -sum clip(r) a
    H, W, y, off, adv, _, _ = _problem(4)
    ell = O.sft(H, W, y).logp
    sid = O.seq_index(off, len(y))
    old = np.where(adv[sid] > 0, ell - 1.0, ell + 1.0)
    r = O.ppo(H, W, y, off, adv, old, None, EPS, 0.0)
    assert np.all(r.dH == 0.0) and np.all(r.dW == 0.0)
    scan = O.scan_labels(y, W.shape[0], off)
    want = 0.0
    for t in np.nonzero(scan.valid)[0]:
        s = sid[t]
        a = adv[s] / scan.seq_len[s]
        want -= (1 + EPS if adv[s] > 0 else 1 - EPS) * a
    assert abs(r.loss - want) <= 1e-13 * abs(want)


def test_ppo_kl_at_its_minimum():
    # A = 0 and ref = current log-probs: the KL term and its slope vanish
    H, W, y, off, _, _, _ = _problem(5)
    ell = O.sft(H, W, y).logp
    r = O.ppo(H, W, y, off, np.zeros(3), ell, ell, EPS, 0.7)
    assert r.loss == 0.0
    assert np.all(r.dH == 0.0) and np.all(r.dW == 0.0)


def test_ppo_chunk_invariance():
    H, W, y, off, adv, old, ref = _problem(6, T=13, n_seq=3, masked=(0, 7))
    full = O.ppo(H, W, y, off, adv, old, ref, EPS, 0.4)
    for C in (1, 4, 12, 20):
        ch = O.ppo(H, W, y, off, adv, old, ref, EPS, 0.4, chunk=C)
        assert _rel(ch.dH, full.dH) < 1e-12 and _rel(ch.dW, full.dW) < 1e-12
        assert abs(ch.loss - full.loss) <= 1e-12 * abs(full.loss)


# planted mistakes ---------------------------------------------------------
_orig_terms = O.ppo_token_terms


def _max_instead_of_min(ell, valid, a, il, old, ref, eps, beta):
    r = np.exp(ell - old)
    u, c = r * a, np.clip(r, 1 - eps, 1 + eps) * a
    loss, w = _orig_terms(ell, valid, a, il, old, ref, eps, beta)
    takes_u = u >= c
    return loss, np.where(valid, np.where(takes_u, a * r, 0.0), 0.0) + (w - np.where(valid, np.where(u <= c, a * r, 0.0), 0.0))


def _clip_ignored(ell, valid, a, il, old, ref, eps, beta):
    loss, w = _orig_terms(ell, valid, a, il, old, ref, eps, beta)
    r = np.exp(ell - old)
    u, c = r * a, np.clip(r, 1 - eps, 1 + eps) * a
    return loss, w + np.where(valid & (u > c), a * r, 0.0)


def _kl_slope_sign(ell, valid, a, il, old, ref, eps, beta):
    loss, w = _orig_terms(ell, valid, a, il, old, ref, eps, beta)
    if ref is None or beta == 0.0:
        return loss, w
    d = ref - ell
    return loss, w - 2 * np.where(valid, beta * il * np.expm1(d), 0.0)


@pytest.mark.parametrize("mutant", [_max_instead_of_min, _clip_ignored, _kl_slope_sign])
def test_ppo_pins_catch_planted_mistakes(monkeypatch, mutant):
    monkeypatch.setattr(O, "ppo_token_terms", mutant)
    caught = 0
    for check in (lambda: test_ppo_torch_autograd(0, 0.3), lambda: test_ppo_fully_clipped_has_zero_gradient(),
                  lambda: test_ppo_torch_autograd(1, 0.0)):
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught >= 1

"""Pins of the CPU fp64 oracle against facts that do not come from the oracle.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, a transposed operand, a wrong normaliser) fails at least one:

* hand-worked examples (tests/golden/hand_cases.json);
* central finite differences of the oracle's loss against its gradients;
* PyTorch CPU fp64 autograd through library routines (cross_entropy,
  log_softmax, logsigmoid) -- an independent code base;
* closed forms: H = 0, W = 0, V = 1, all rows ignored, a constant logit shift,
  token permutation;
* each dlogits row sums to zero;
* results do not change with the chunk size (the method is exact);
* the DPO gradient equals -beta * sigma(-beta*Delta) * (grad S_chosen - grad S_rejected)
  with grad S taken from a different entry (GRPO weights).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import streambp_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")
LN2 = math.log(2.0)


def _val(s):
    if isinstance(s, (int, float)):
        return float(s)
    if s.endswith("*ln2"):
        return float(Fraction(s[:-4])) * LN2
    return float(Fraction(s))


def _arr(x):
    return np.array([[_val(v) for v in row] for row in x]) if isinstance(x[0], list) \
        else np.array([_val(v) for v in x])


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def _run(kind, H, W, y, offsets=None, adv=None, ref=None, beta=None, chunk=None):
    if kind == "sft":
        return O.sft(H, W, y, chunk=chunk)
    if kind == "grpo":
        return O.grpo(H, W, y, offsets, adv, chunk=chunk)
    return O.dpo(H, W, y, offsets, ref, beta, chunk=chunk)


# --------------------------------------------------------------------------
# hand-worked cases
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_cases(case):
    H = _arr(case["H"])
    W = _arr(case["W"])
    y = np.array(case["labels"])
    r = _run(case["kind"], H, W, y, case.get("offsets"), case.get("adv"),
             case.get("ref_logp"), case.get("beta"))
    want_loss = math.log(_val(case["loss_ln"])) if "loss_ln" in case else _val(case["loss"])
    assert abs(r.loss - want_loss) < 1e-14
    if "logp" in case:
        np.testing.assert_allclose(r.logp, _arr(case["logp"]), atol=1e-14)
    if "seq_logp" in case:
        np.testing.assert_allclose(r.seq_logp, _arr(case["seq_logp"]), atol=1e-14)
    Z = O.logits(O.widen(H), O.widen(W))
    G = O.grad_logits(Z, r.lse, y, r.scan.valid, r.w)
    np.testing.assert_allclose(G, _arr(case["G"]), atol=1e-14)
    np.testing.assert_allclose(r.dH, _arr(case["dH"]), atol=1e-14)
    np.testing.assert_allclose(r.dW, _arr(case["dW"]), atol=1e-14)


# --------------------------------------------------------------------------
# small random problems shared by the pins below
# --------------------------------------------------------------------------
def _problem(seed, T=8, D=4, V=7, n_seq=2, masked=(1, 5), scale=1.0):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((T, D)) * scale
    W = rng.standard_normal((V, D)) * scale
    y = rng.integers(0, V, T)
    y[list(masked)] = O.IGNORE_INDEX
    off = np.linspace(0, T, n_seq + 1).astype(np.int64)
    adv = rng.standard_normal(n_seq)
    ref = rng.standard_normal(n_seq) * 2.0
    return H, W, y, off, adv, ref


def _loss_fn(kind, y, off, adv, ref, beta):
    def f(H, W):
        return _run(kind, H, W, y, off, adv, ref, beta).loss
    return f


@pytest.mark.parametrize("kind", ["sft", "grpo", "dpo"])
@pytest.mark.parametrize("seed", [0, 1])
def test_finite_differences(kind, seed):
    H, W, y, off, adv, ref = _problem(seed, n_seq=2 if kind != "dpo" else 4)
    beta = 0.7
    r = _run(kind, H, W, y, off, adv, ref, beta)
    f = _loss_fn(kind, y, off, adv, ref, beta)
    h = 1e-6
    for X, G in ((H, r.dH), (W, r.dW)):
        fd = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + h
            fp = f(H, W)
            X[idx] = old - h
            fm = f(H, W)
            X[idx] = old
            fd[idx] = (fp - fm) / (2 * h)
        assert _rel(G, fd) < 1e-6, (kind, _rel(G, fd))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_torch_autograd_sft(seed):
    H, W, y, *_ = _problem(seed, T=12, D=5, V=9, masked=(0, 3, 4))
    r = O.sft(H, W, y)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(Ht @ Wt.T, torch.tensor(y), ignore_index=-100)
    loss.backward()
    assert abs(r.loss - loss.item()) <= 1e-12 * abs(loss.item())
    assert _rel(r.dH, Ht.grad.numpy()) < 1e-12
    assert _rel(r.dW, Wt.grad.numpy()) < 1e-12


@pytest.mark.parametrize("seed", [0, 1])
def test_torch_autograd_grpo(seed):
    H, W, y, off, adv, _ = _problem(seed, T=12, D=5, V=9, n_seq=3, masked=(0, 5))
    r = O.grpo(H, W, y, off, adv)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    lp = torch.log_softmax(Ht @ Wt.T, dim=-1)
    yt = torch.tensor(y)
    valid = yt != -100
    tok = lp.gather(1, yt.clamp(min=0)[:, None])[:, 0] * valid
    loss = torch.zeros((), dtype=torch.float64)
    for s in range(len(off) - 1):
        n = int(valid[off[s]:off[s + 1]].sum())
        if n:
            loss = loss - adv[s] / n * tok[off[s]:off[s + 1]].sum()
    loss.backward()
    assert abs(r.loss - loss.item()) <= 1e-12 * max(1.0, abs(loss.item()))
    assert _rel(r.dH, Ht.grad.numpy()) < 1e-12
    assert _rel(r.dW, Wt.grad.numpy()) < 1e-12
    np.testing.assert_allclose(r.logp, tok.detach().numpy(), atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("beta", [0.1, 2.0])
def test_torch_autograd_dpo(seed, beta):
    H, W, y, off, _, ref = _problem(seed, T=16, D=5, V=9, n_seq=4, masked=(0, 8))
    r = O.dpo(H, W, y, off, ref, beta)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    lp = torch.log_softmax(Ht @ Wt.T, dim=-1)
    yt = torch.tensor(y)
    valid = yt != -100
    tok = lp.gather(1, yt.clamp(min=0)[:, None])[:, 0] * valid
    S = torch.stack([tok[off[s]:off[s + 1]].sum() for s in range(4)])
    R = torch.tensor(ref)
    delta = (S[:2] - R[:2]) - (S[2:] - R[2:])
    loss = -torch.nn.functional.logsigmoid(beta * delta).mean()
    loss.backward()
    assert abs(r.loss - loss.item()) <= 1e-12 * max(1.0, abs(loss.item()))
    np.testing.assert_allclose(r.seq_logp, S.detach().numpy(), rtol=1e-13)
    assert _rel(r.dH, Ht.grad.numpy()) < 1e-12
    assert _rel(r.dW, Wt.grad.numpy()) < 1e-12


# --------------------------------------------------------------------------
# structural pins
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 3])
def test_dlogits_rows_sum_to_zero(seed):
    H, W, y, off, adv, _ = _problem(seed, T=20, D=6, V=11, n_seq=2, masked=(2, 3))
    r = O.grpo(H, W, y, off, adv)
    G = O.grad_logits(O.logits(H, W), r.lse, y, r.scan.valid, r.w)
    assert np.all(np.abs(G.sum(axis=1)) <= 1e-12 * np.abs(r.w).max())
    assert np.all(G[~r.scan.valid] == 0.0)


@pytest.mark.parametrize("kind", ["sft", "grpo", "dpo"])
def test_chunk_invariance(kind):
    T = 64
    H, W, y, off, adv, ref = _problem(5, T=T, D=8, V=13, n_seq=4, masked=(0, 7, 33, 63))
    full = _run(kind, H, W, y, off, adv, ref, 0.3)
    for C in (1, 3, 64, T - 1, T, T + 5):
        r = _run(kind, H, W, y, off, adv, ref, 0.3, chunk=C)
        assert abs(r.loss - full.loss) <= 1e-12 * max(1.0, abs(full.loss))
        assert _rel(r.dH, full.dH) < 1e-12
        assert _rel(r.dW, full.dW) < 1e-12
        np.testing.assert_allclose(r.logp, full.logp, atol=1e-12)


def test_dpo_closed_form_from_sequence_gradients():
    """grad L = sum_i -(beta/P) sigma(-beta Delta_i) (grad S_ci - grad S_ri); grad S_s is
    computed through the GRPO entry with weight +1 on the log-probs of sequence s
    (advantage -len_s on s, 0 elsewhere)."""
    H, W, y, off, _, ref = _problem(7, T=24, D=5, V=10, n_seq=6, masked=(0, 4, 13))
    beta = 0.25
    r = O.dpo(H, W, y, off, ref, beta)
    scan = O.scan_labels(y, W.shape[0], off)
    gS_H, gS_W = [], []
    for s in range(6):
        adv = np.zeros(6)
        adv[s] = -float(scan.seq_len[s])
        g = O.grpo(H, W, y, off, adv)
        assert abs(g.loss - r.seq_logp[s]) < 1e-12 * max(1, abs(r.seq_logp[s]))
        gS_H.append(g.dH)
        gS_W.append(g.dW)
    P = 3
    S = np.asarray(r.seq_logp)
    delta = (S[:P] - ref[:P]) - (S[P:] - ref[P:])
    sig = np.array([1 / (1 + math.exp(beta * d)) for d in delta])
    want_loss = np.mean([math.log1p(math.exp(-beta * d)) for d in delta])
    want_dH = sum(-(beta / P) * sig[i] * (gS_H[i] - gS_H[P + i]) for i in range(P))
    want_dW = sum(-(beta / P) * sig[i] * (gS_W[i] - gS_W[P + i]) for i in range(P))
    assert abs(r.loss - want_loss) < 1e-12
    assert _rel(r.dH, want_dH) < 1e-12
    assert _rel(r.dW, want_dW) < 1e-12


def test_dpo_saturated_sigmoid_is_finite():
    S = np.array([-1e5, 1e5, 0.0, 0.0])
    pairs = O.dpo_pairs(S, np.zeros(4), 0.1)
    assert np.all(np.isfinite(pairs.coef)) and math.isfinite(pairs.loss)
    assert pairs.coef[0] == pytest.approx(0.05)       # beta/P * sigma(+1e4)
    assert pairs.coef[1] == 0.0 or pairs.coef[1] < 1e-300
    assert pairs.loss == pytest.approx((1e4 + 0.0) / 2)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def test_zero_hidden_closed_form():
    rng = np.random.default_rng(11)
    T, D, V = 10, 4, 9
    H = np.zeros((T, D))
    W = rng.standard_normal((V, D))
    y = rng.integers(0, V, T)
    y[[2, 6]] = -100
    r = O.sft(H, W, y)
    valid = y != -100
    N = valid.sum()
    assert r.loss == pytest.approx(math.log(V), rel=1e-14)
    np.testing.assert_allclose(r.lse, np.full(T, math.log(V)), rtol=1e-14)
    np.testing.assert_allclose(r.logp[valid], -math.log(V), rtol=1e-14)
    want_dH = np.zeros((T, D))
    want_dH[valid] = (W.mean(axis=0)[None, :] - W[y[valid]]) / N
    assert _rel(r.dH, want_dH) < 1e-13
    assert np.all(r.dW == 0.0)
    # DPO sequence sums at H = 0: -len_s ln V
    off = np.array([0, 5, 10])
    p1 = O.dpo_logp(H, W, y, off)
    lens = [valid[0:5].sum(), valid[5:10].sum()]
    np.testing.assert_allclose(p1.seq_logp, [-lens[0] * math.log(V), -lens[1] * math.log(V)], rtol=1e-14)


def test_zero_weight_closed_form():
    rng = np.random.default_rng(12)
    T, D, V = 10, 4, 6
    H = rng.standard_normal((T, D))
    W = np.zeros((V, D))
    y = rng.integers(0, V, T)
    y[[1]] = -100
    off = np.array([0, 4, 10])
    adv = np.array([0.5, -1.5])
    r = O.grpo(H, W, y, off, adv)
    assert np.all(r.dH == 0.0)
    w = r.w
    want = np.tile((w[:, None] * H).sum(axis=0) / V, (V, 1))
    for t in range(T):
        if y[t] != -100:
            want[y[t]] -= w[t] * H[t]
    assert _rel(r.dW, want) < 1e-13
    # weights themselves: A_s/len_s on valid rows
    lens = [np.sum(y[0:4] != -100), np.sum(y[4:10] != -100)]
    want_w = np.array([(adv[0] / lens[0] if t < 4 else adv[1] / lens[1]) if y[t] != -100 else 0
                       for t in range(T)])
    np.testing.assert_allclose(w, want_w, rtol=1e-15)


def test_single_token_vocab_and_all_masked():
    rng = np.random.default_rng(13)
    H = rng.standard_normal((5, 3))
    r = O.sft(H, rng.standard_normal((1, 3)), np.zeros(5, dtype=np.int64))
    assert r.loss == 0.0 and np.all(r.dH == 0) and np.all(r.dW == 0)
    r = O.sft(H, rng.standard_normal((4, 3)), np.full(5, -100))
    assert r.loss == 0.0 and r.scan.n_valid == 0 and np.all(r.dH == 0) and np.all(r.dW == 0)


def test_constant_logit_shift():
    """Appending a ones column to H and a constant column c to W adds c to every
    logit; softmax, loss and the gradients on the original columns do not move.
    c = 1e4 would overflow exp without the max subtraction."""
    H, W, y, off, adv, _ = _problem(9, T=10, D=4, V=8, masked=(3,))
    r0 = O.grpo(H, W, y, off, adv)
    Hs = np.hstack([H, np.ones((10, 1))])
    Ws = np.hstack([W, np.full((8, 1), 1e4)])
    r1 = O.grpo(Hs, Ws, y, off, adv)
    assert abs(r1.loss - r0.loss) < 1e-9
    assert _rel(r1.dH[:, :4], r0.dH) < 1e-9
    assert _rel(r1.dW[:, :4], r0.dW) < 1e-9


def test_token_permutation():
    H, W, y, *_ = _problem(10, T=12, D=4, V=8, masked=(2, 9))
    perm = np.random.default_rng(0).permutation(12)
    r0 = O.sft(H, W, y)
    r1 = O.sft(H[perm], W, y[perm])
    assert abs(r1.loss - r0.loss) < 1e-13
    assert _rel(r1.dH, r0.dH[perm]) < 1e-13
    assert _rel(r1.dW, r0.dW) < 1e-13
    np.testing.assert_allclose(r1.logp, r0.logp[perm], atol=1e-14)


# --------------------------------------------------------------------------
# integer work
# --------------------------------------------------------------------------
def test_label_scan_integers():
    y = np.array([0, -100, 5, 6, -100, 3, 2, 1])
    s = O.scan_labels(y, 6, np.array([0, 3, 3, 8]), strict=False)
    assert s.valid.tolist() == [True, False, True, False, False, True, True, True]
    assert s.n_valid == 5
    assert s.seq_len.tolist() == [2, 0, 3]
    assert s.status == O.STATUS_LABEL_RANGE
    with pytest.raises(O.LabelError):
        O.scan_labels(y, 6)
    s = O.scan_labels(np.array([-100, 0, 5]), 6)
    assert s.status == O.STATUS_OK and s.n_valid == 2
    with pytest.raises(ValueError):
        O.scan_labels(np.array([1, 2]), 6, np.array([0, 3]))


def test_out_of_range_labels_are_ignored_in_lenient_mode():
    H, W, y, *_ = _problem(4, T=8, D=3, V=5, masked=())
    y2 = y.copy()
    y2[3] = 5       # out of range
    y2[6] = -7      # out of range
    ref = y.copy()
    ref[[3, 6]] = -100
    r = O.sft(H, W, y2, strict=False)
    r0 = O.sft(H, W, ref)
    assert r.scan.status == O.STATUS_LABEL_RANGE
    assert r.loss == r0.loss and np.array_equal(r.dH, r0.dH) and np.array_equal(r.dW, r0.dW)


def test_bf16_inputs_are_widened_exactly():
    bits = np.array([0x3F80, 0xC020, 0x0001, 0x7F7F], dtype=np.uint16)
    want = np.array([1.0, -2.5, 2.0 ** -133, 3.3895313892515355e38])
    np.testing.assert_array_equal(O.widen(bits), want)

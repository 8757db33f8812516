"""Pins of the oracle's sampled helpers (rows_lse_logp, rows_dH, all_lse,
cols_dW), which the full-size GPU tests evaluate on chosen rows and
vocabulary rows only.

Each helper restates the definition of the exact head ("StreamBP:
Memory-Efficient Exact Backpropagation ...", LM-head paragraph of the news
article; abstract: exact gradients) on a subset of rows, so on small shapes it
must agree with the whole-sequence oracle (itself pinned by finite
differences, torch autograd and closed forms in test_oracle_pins.py) and with
PyTorch's own fp64 routines.  The shapes carry ignored rows, out-of-range
labels (lenient mode), a vocabulary that is not a multiple of 8, several
sequences, unsorted and repeated sample indices, and bf16 bit-pattern inputs.
"""
import numpy as np
import pytest
import torch

from oracle import streambp_oracle as O
from workloads import gen

T, D, V, S = 23, 16, 37, 3
OFFSETS = np.array([0, 8, 15, 23])
ROWS = np.array([22, 0, 5, 7, 13, 3, 3, 14, 15])      # unsorted, repeated, ignored and out-of-range rows
COLS = np.array([36, 0, 9, 17, 17, 21])               # unsorted, repeated, V-1


def _case(seed, bf16):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((T, D)).astype(np.float32)
    W = (0.5 * rng.standard_normal((V, D))).astype(np.float32)
    y = rng.integers(0, V, T)
    y[[0, 5, 11]] = O.IGNORE_INDEX
    y[7] = V + 3          # out of range: ignored in lenient mode
    y[13] = -7
    y[[2, 4, 14]] = [9, 9, 17]   # sampled columns that are label targets, one twice
    adv = rng.standard_normal(S)
    if bf16:
        return gen.bf16_bits(H).reshape(T, D), gen.bf16_bits(W).reshape(V, D), y, adv
    return H, W, y, adv


def _torch_lse_logp(H, W, y):
    Z = torch.from_numpy(O.widen(H)) @ torch.from_numpy(O.widen(W)).T
    lse = torch.logsumexp(Z, dim=1)
    lp = torch.log_softmax(Z, dim=1)
    yt = torch.from_numpy(y)
    valid = (yt >= 0) & (yt < W.shape[0])
    ell = lp.gather(1, torch.where(valid, yt, 0)[:, None])[:, 0] * valid
    return lse.numpy(), ell.numpy()


def check_rows_lse_logp(seed, bf16):
    H, W, y, _ = _case(seed, bf16)
    lse, ell = O.rows_lse_logp(H, W, y, ROWS)
    full = O.sft(H, W, y, strict=False)
    np.testing.assert_allclose(lse, full.lse[ROWS], rtol=1e-13, atol=0)
    np.testing.assert_allclose(ell, full.logp[ROWS], rtol=1e-12, atol=1e-13)
    t_lse, t_ell = _torch_lse_logp(H, W, y)
    np.testing.assert_allclose(lse, t_lse[ROWS], rtol=1e-13, atol=0)
    np.testing.assert_allclose(ell, t_ell[ROWS], rtol=1e-12, atol=1e-13)
    assert np.all(ell[np.isin(ROWS, [0, 5, 7, 13])] == 0.0)


def check_rows_dH(seed, bf16):
    H, W, y, adv = _case(seed, bf16)
    full = O.grpo(H, W, y, OFFSETS, adv, strict=False)
    got = O.rows_dH(H, W, y, full.w, ROWS)
    np.testing.assert_allclose(got, full.dH[ROWS], rtol=1e-12, atol=1e-14)
    # and against torch autograd of the GRPO objective, independently of the oracle
    Ht = torch.tensor(O.widen(H), requires_grad=True)
    lp = torch.log_softmax(Ht @ torch.from_numpy(O.widen(W)).T, dim=1)
    yt = torch.from_numpy(y)
    valid = (yt >= 0) & (yt < V)
    tok = lp.gather(1, torch.where(valid, yt, 0)[:, None])[:, 0] * valid
    loss = torch.zeros((), dtype=torch.float64)
    for s in range(S):
        n = int(valid[OFFSETS[s]:OFFSETS[s + 1]].sum())
        if n:
            loss = loss - adv[s] / n * tok[OFFSETS[s]:OFFSETS[s + 1]].sum()
    loss.backward()
    np.testing.assert_allclose(got, Ht.grad.numpy()[ROWS], rtol=1e-12, atol=1e-14)
    assert np.all(got[np.isin(ROWS, [0, 5, 7, 13])] == 0.0)


def check_all_lse(seed, bf16):
    H, W, _, _ = _case(seed, bf16)
    want = torch.logsumexp(torch.from_numpy(O.widen(H)) @ torch.from_numpy(O.widen(W)).T, dim=1).numpy()
    for blk in (1, 5, T, 64):
        np.testing.assert_allclose(O.all_lse(H, W, row_block=blk), want, rtol=1e-13, atol=0)
    # a constant logit shift c moves every lse by exactly c (1e4 would overflow
    # exp without the max subtraction)
    Hs = np.hstack([O.widen(H), np.ones((T, 1))])
    Ws = np.hstack([O.widen(W), np.full((V, 1), 1e4)])
    np.testing.assert_allclose(O.all_lse(Hs, Ws, row_block=7) - 1e4, want, rtol=0, atol=1e-9)


def check_cols_dW(seed, bf16):
    H, W, y, adv = _case(seed, bf16)
    full = O.grpo(H, W, y, OFFSETS, adv, strict=False)
    got = O.cols_dW(H, W, y, full.w, full.lse, COLS)
    np.testing.assert_allclose(got, full.dW[COLS], rtol=1e-12, atol=1e-14)
    Wt = torch.tensor(O.widen(W), requires_grad=True)
    lp = torch.log_softmax(torch.from_numpy(O.widen(H)) @ Wt.T, dim=1)
    yt = torch.from_numpy(y)
    valid = (yt >= 0) & (yt < V)
    tok = lp.gather(1, torch.where(valid, yt, 0)[:, None])[:, 0] * valid
    loss = torch.zeros((), dtype=torch.float64)
    for s in range(S):
        n = int(valid[OFFSETS[s]:OFFSETS[s + 1]].sum())
        if n:
            loss = loss - adv[s] / n * tok[OFFSETS[s]:OFFSETS[s + 1]].sum()
    loss.backward()
    np.testing.assert_allclose(got, Wt.grad.numpy()[COLS], rtol=1e-12, atol=1e-14)


CHECKS = [check_rows_lse_logp, check_rows_dH, check_all_lse, check_cols_dW]


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__[6:])
def test_sampled_helper(check, seed, bf16):
    check(seed, bf16)

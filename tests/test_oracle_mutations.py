"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and check
that the pins catch each of them."""
import json

import numpy as np
import pytest

from oracle import streambp_oracle as O
from tests import test_oracle_pins as pins

_orig_grad = O.grad_logits
_orig_pairs = O.dpo_pairs
_orig_wsft = O.weights_sft
_orig_wgrpo = O.weights_grpo
_orig_lse = O.logsumexp_rows


def _no_onehot(Z, lse, labels, valid, w):
    G = np.exp(Z - lse[:, None])
    return G * np.where(valid, w, 0.0)[:, None]


def _flipped_sign(*a):
    return -_orig_grad(*a)


def _dpo_swapped(S, R, beta):
    p = _orig_pairs(S, R, beta)
    P = len(p.coef) // 2
    return O.DpoPairs(p.delta, p.loss, np.concatenate([p.coef[P:], p.coef[:P]]))


def _sft_over_T(scan):
    return np.where(scan.valid, 1.0 / scan.valid.shape[0], 0.0)


def _grpo_no_len(scan, offsets, adv):
    sid = O.seq_index(offsets, scan.valid.shape[0])
    return np.where(scan.valid, np.asarray(adv, dtype=np.float64)[sid], 0.0)


def _lse_no_log(Z):
    m = np.max(Z, axis=1)
    return m + np.sum(np.exp(Z - m[:, None]), axis=1) - 1.0


MUTATIONS = {
    "dropped_onehot": ("grad_logits", _no_onehot),
    "flipped_gradient_sign": ("grad_logits", _flipped_sign),
    "dpo_chosen_rejected_swapped": ("dpo_pairs", _dpo_swapped),
    "sft_mean_over_all_tokens": ("weights_sft", _sft_over_T),
    "grpo_missing_length": ("weights_grpo", _grpo_no_len),
    "lse_linearised": ("logsumexp_rows", _lse_no_log),
}


def _pin_suite():
    cases = json.load(open(pins.GOLDEN))["cases"]
    checks = [lambda c=c: pins.test_hand_cases(c) for c in cases]
    checks += [lambda: pins.test_torch_autograd_sft(0),
               lambda: pins.test_torch_autograd_grpo(0),
               lambda: pins.test_torch_autograd_dpo(0, 0.1),
               lambda: pins.test_zero_hidden_closed_form(),
               lambda: pins.test_zero_weight_closed_form(),
               lambda: pins.test_dlogits_rows_sum_to_zero(0)]
    return checks


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = 0
    for check in _pin_suite():
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake {name}"


def test_pins_pass_without_mutation():
    for check in _pin_suite():
        check()


# --------------------------------------------------------------------------
# the sampled helpers used by the full-size GPU tests, each with one
# plausible slip, against the pins of tests/test_oracle_sampled.py
# --------------------------------------------------------------------------
from tests import test_oracle_sampled as sampled  # noqa: E402

_orig_rows_lse_logp = O.rows_lse_logp
_orig_cols_dW = O.cols_dW


def _rows_logp_label_of_next_row(H, W, labels, rows, V_block=1 << 15):
    # the label of the following position (a missed next-token alignment)
    rows = np.asarray(rows)
    shifted = np.asarray(labels).copy()
    shifted[:-1] = shifted[1:]
    return _orig_rows_lse_logp(H, W, shifted, rows, V_block)


def _rows_dH_weight_by_sample_index(H, W, labels, w, rows):
    # the weight of sample k instead of token rows[k]
    rows = np.asarray(rows)
    Wd = O.widen(W)
    Hr = O.widen(np.asarray(H)[rows])
    y = np.asarray(labels, dtype=np.int64)[rows]
    valid = (y >= 0) & (y < Wd.shape[0])
    Z = O.logits(Hr, Wd)
    lse = O.logsumexp_rows(Z)
    G = O.grad_logits(Z, lse, y, valid, np.asarray(w, dtype=np.float64)[:len(rows)])
    return G @ Wd


def _all_lse_max_not_restored(H, W, row_block=512):
    # the max subtracted for stability is never added back
    Wd = O.widen(W)
    Hn = np.asarray(H)
    out = np.zeros(Hn.shape[0])
    for lo in range(0, Hn.shape[0], row_block):
        Z = O.logits(O.widen(Hn[lo:lo + row_block]), Wd)
        m = np.max(Z, axis=1)
        out[lo:lo + row_block] = np.log(np.sum(np.exp(Z - m[:, None]), axis=1))
    return out


def _cols_dW_onehot_by_position(H, W, labels, w, lse, cols):
    # the one-hot compares labels with the sample position, not the vocabulary id
    cols = np.asarray(cols)
    Hd = O.widen(H)
    Zc = Hd @ O.widen(np.asarray(W)[cols]).T
    y = np.asarray(labels, dtype=np.int64)
    G = np.exp(Zc - np.asarray(lse)[:, None]) - (y[:, None] == np.arange(len(cols))[None, :])
    G *= np.asarray(w, dtype=np.float64)[:, None]
    return G.T @ Hd


HELPER_MUTATIONS = {
    "rows_logp_label_of_next_row": ("rows_lse_logp", _rows_logp_label_of_next_row),
    "rows_dH_weight_by_sample_index": ("rows_dH", _rows_dH_weight_by_sample_index),
    "all_lse_max_not_restored": ("all_lse", _all_lse_max_not_restored),
    "cols_dW_onehot_by_position": ("cols_dW", _cols_dW_onehot_by_position),
}


def _sampled_suite():
    return [lambda f=f, s=s, b=b: f(s, b) for f in sampled.CHECKS for s in (0, 1) for b in (False, True)]


@pytest.mark.parametrize("name", sorted(HELPER_MUTATIONS))
def test_sampled_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = HELPER_MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = 0
    for check in _sampled_suite():
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake {name}"


def test_sampled_pins_pass_without_mutation():
    for check in _sampled_suite():
        check()

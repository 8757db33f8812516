"""CPU fp64 oracle for StreamBP's LM-head forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module; the product path never calls it.
It shares no code with the HIP library and imports nothing from it.

What it computes ("StreamBP: Memory-Efficient Exact Backpropagation for Long
Sequence Training of LLMs"):

* The method is exact (title and abstract): the chunked backward returns
  the same loss and gradients as ordinary backpropagation.  So the oracle is
  the plain definition: Z = H W^T over the whole sequence, a row-wise
  log-sum-exp, the per-token log-probability of the label, and
  dlogits = w_t (softmax(Z_t) - onehot(y_t)), dH = G W, dW = G^T H.
* LM-head paragraph (news article, LM-head paragraph): for SFT and GRPO the
  logits of different positions affect the objective independently, so the
  sequence is split into chunks and one chunk's loss gradient is formed at a
  time.  ``chunk=`` runs exactly that, accumulating dW over chunks.
* DPO paragraph (same article): the sigmoid couples the positions, but the
  logits gradient is still separable along the sequence once the sequence
  log-probabilities are known.  The oracle takes the two-pass reading: pass 1
  sums log-probabilities per sequence, pass 2 forms the per-token weights
  from the pair factor and runs the chunked backward.

Readings where the pages are silent (each one is listed with the others in
the design notes): labels are aligned to H rows, -100 means ignored, any
other label outside [0, V) is an error; SFT loss is the mean over valid
tokens of the call and is 0 with zero gradients when there are none; GRPO is
on-policy (ratio 1, no KL, no clipping) with weight -A_s/len_s on log pi,
len_s the number of valid tokens of sequence s, and its reported loss is
sum_t (-A_s/len_s) * logp_t; DPO averages softplus(-beta * Delta_i) over
pairs, sequences 0..P-1 are chosen and P..2P-1 rejected; the off-policy head
(PPO, listed among the objectives by the news article) is the clipped
surrogate -min(r a, clip(r, 1-eps, 1+eps) a) with r = exp(logp - logp_old),
a = A_s/len_s, plus beta_kl/len_s (exp(d) - d - 1), d = logp_ref - logp;
no bias, soft-cap, temperature or label smoothing.

Every function is fp64 numpy.  Inputs in bfloat16 arrive as uint16 bit
patterns and are widened exactly.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

IGNORE_INDEX = -100
# status codes of the library interface (0 = fine)
STATUS_OK = 0
STATUS_INVALID_ARGUMENT = 1
STATUS_LABEL_RANGE = 5


class LabelError(ValueError):
    pass


def widen(x: np.ndarray) -> np.ndarray:
    """Exact fp64 copy of an fp32 array, or of bfloat16 bit patterns (uint16):
    a bfloat16 is the top half of an IEEE binary32.  Large arrays are
    converted in blocks (fewer huge temporaries), which changes nothing in the
    values."""
    x = np.asarray(x)
    out = np.empty(x.shape, dtype=np.float64)
    src, dst = x.reshape(-1), out.reshape(-1)
    blk = 1 << 22

    def conv(lo):
        s = src[lo:lo + blk]
        if s.dtype == np.uint16:
            dst[lo:lo + blk] = (s.astype(np.uint32) << np.uint32(16)).view(np.float32)
        else:
            dst[lo:lo + blk] = s

    starts = range(0, src.size, blk)
    if len(starts) > 4:
        import concurrent.futures as cf
        import os
        with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(conv, starts))
    else:
        for lo in starts:
            conv(lo)
    return out


# --------------------------------------------------------------------------
# labels and segments (integer work; the device must match it bit for bit)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class LabelScan:
    valid: np.ndarray       # bool [T]
    n_valid: int            # number of valid tokens in the call
    seq_len: np.ndarray     # int64 [S]: valid tokens per sequence
    status: int


def scan_labels(labels: np.ndarray, V: int, offsets: Optional[np.ndarray] = None,
                strict: bool = True) -> LabelScan:
    """Validity of each position: a label counts when it lies in [0, V).
    -100 is ignored.  Any other value is an error (``strict``) or, as the
    library does, ignored with STATUS_LABEL_RANGE reported."""
    y = np.asarray(labels, dtype=np.int64)
    T = y.shape[0]
    in_range = (y >= 0) & (y < V)
    bad = ~in_range & (y != IGNORE_INDEX)
    status = STATUS_OK
    if bad.any():
        if strict:
            raise LabelError(f"{int(bad.sum())} labels outside [0,{V}) and not {IGNORE_INDEX}")
        status = STATUS_LABEL_RANGE
    if offsets is None:
        offsets = np.array([0, T])
    off = np.asarray(offsets, dtype=np.int64)
    if off[0] != 0 or off[-1] != T or np.any(np.diff(off) < 0):
        raise ValueError("offsets must start at 0, end at T and not decrease")
    seq_len = np.array([int(in_range[off[s]:off[s + 1]].sum()) for s in range(len(off) - 1)],
                       dtype=np.int64)
    return LabelScan(in_range, int(in_range.sum()), seq_len, status)


def seq_index(offsets: np.ndarray, T: int) -> np.ndarray:
    """Sequence id of every position."""
    off = np.asarray(offsets, dtype=np.int64)
    sid = np.empty(T, dtype=np.int64)
    for s in range(len(off) - 1):
        sid[off[s]:off[s + 1]] = s
    return sid


# --------------------------------------------------------------------------
# per-token weights in cross-entropy form: the loss gradient w.r.t. the
# logits of row t is w_t * (softmax(Z_t) - onehot(y_t))
# --------------------------------------------------------------------------
def weights_sft(scan: LabelScan) -> np.ndarray:
    """Mean cross-entropy over valid tokens: w_t = 1/N on valid rows."""
    w = np.zeros(scan.valid.shape[0])
    if scan.n_valid > 0:
        w[scan.valid] = 1.0 / scan.n_valid
    return w


def weights_grpo(scan: LabelScan, offsets: np.ndarray, adv: np.ndarray) -> np.ndarray:
    """On-policy GRPO: the objective weights log pi_t by -A_s/len_s, which is
    cross-entropy weight +A_s/len_s."""
    T = scan.valid.shape[0]
    sid = seq_index(offsets, T)
    adv = np.asarray(adv, dtype=np.float64)
    w = np.zeros(T)
    for t in range(T):
        s = sid[t]
        if scan.valid[t] and scan.seq_len[s] > 0:
            w[t] = adv[s] / scan.seq_len[s]
    return w


def sigmoid(x):
    """Logistic function, evaluated without overflow for either sign."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(x):
    """log(1 + e^x) without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


@dataclasses.dataclass
class DpoPairs:
    delta: np.ndarray   # [P]
    loss: float
    coef: np.ndarray    # [2P] cross-entropy weight of every sequence


def dpo_pairs(seq_logp: np.ndarray, ref_logp: np.ndarray, beta: float) -> DpoPairs:
    """Pairs (i, P+i): Delta_i = (S_ci - R_ci) - (S_ri - R_ri),
    loss = mean_i softplus(-beta Delta_i).  d loss / d S_ci = -(beta/P) sigma(-beta Delta_i)
    and the rejected side has the opposite sign; the cross-entropy weight of a
    sequence is minus that derivative."""
    S = np.asarray(seq_logp, dtype=np.float64)
    R = np.asarray(ref_logp, dtype=np.float64)
    assert S.shape == R.shape and S.shape[0] % 2 == 0
    P = S.shape[0] // 2
    delta = (S[:P] - R[:P]) - (S[P:] - R[P:])
    loss = float(np.mean(softplus(-beta * delta))) if P else 0.0
    f = (beta / P) * sigmoid(-beta * delta) if P else np.zeros(0)
    return DpoPairs(delta, loss, np.concatenate([f, -f]))


def weights_per_sequence(scan: LabelScan, offsets: np.ndarray, coef: np.ndarray) -> np.ndarray:
    T = scan.valid.shape[0]
    sid = seq_index(offsets, T)
    return np.where(scan.valid, np.asarray(coef, dtype=np.float64)[sid], 0.0)


# --------------------------------------------------------------------------
# one block of rows: logits, log-sum-exp, log-probs, logits gradient
# --------------------------------------------------------------------------
def logits(H: np.ndarray, W: np.ndarray) -> np.ndarray:
    return H @ W.T


def logsumexp_rows(Z: np.ndarray) -> np.ndarray:
    m = np.max(Z, axis=1)
    return m + np.log(np.sum(np.exp(Z - m[:, None]), axis=1))


def target_logp(Z: np.ndarray, lse: np.ndarray, labels: np.ndarray, valid: np.ndarray) -> np.ndarray:
    """log softmax(Z_t)[y_t] on valid rows, 0 elsewhere."""
    ell = np.zeros(Z.shape[0])
    rows = np.nonzero(valid)[0]
    ell[rows] = Z[rows, labels[rows]] - lse[rows]
    return ell


def grad_logits(Z: np.ndarray, lse: np.ndarray, labels: np.ndarray, valid: np.ndarray,
                w: np.ndarray) -> np.ndarray:
    """G_tv = w_t (exp(Z_tv - lse_t) - [v == y_t]); rows that are not valid are 0."""
    G = np.exp(Z - lse[:, None])
    rows = np.nonzero(valid)[0]
    G[rows, labels[rows]] -= 1.0
    G *= np.where(valid, w, 0.0)[:, None]
    return G


@dataclasses.dataclass
class Result:
    loss: float
    dH: Optional[np.ndarray]
    dW: Optional[np.ndarray]
    logp: np.ndarray            # per token, 0 on ignored rows
    lse: np.ndarray
    w: np.ndarray               # cross-entropy weights used in the backward
    scan: LabelScan
    seq_logp: Optional[np.ndarray] = None
    delta: Optional[np.ndarray] = None


def _chunks(T: int, chunk: Optional[int]):
    C = T if (chunk is None or chunk <= 0) else chunk
    return [(lo, min(T, lo + C)) for lo in range(0, T, max(C, 1))] if T else []


def _forward(Hd, Wd, y, valid, chunk):
    """log-sum-exp and target log-prob of every row, one chunk at a time."""
    T = Hd.shape[0]
    lse = np.zeros(T)
    ell = np.zeros(T)
    for lo, hi in _chunks(T, chunk):
        Z = logits(Hd[lo:hi], Wd)
        lse[lo:hi] = logsumexp_rows(Z)
        ell[lo:hi] = target_logp(Z, lse[lo:hi], y[lo:hi], valid[lo:hi])
    return lse, ell


def _backward(Hd, Wd, y, valid, w, chunk, want_grads=True):
    """Stream over chunks: logits, log-sum-exp, log-probs, G, dH rows and the
    dW contribution of each chunk, summed over chunks."""
    T, D = Hd.shape
    V = Wd.shape[0]
    lse = np.zeros(T)
    ell = np.zeros(T)
    dH = np.zeros((T, D)) if want_grads else None
    dW = np.zeros((V, D)) if want_grads else None
    for lo, hi in _chunks(T, chunk):
        Z = logits(Hd[lo:hi], Wd)
        lse[lo:hi] = logsumexp_rows(Z)
        ell[lo:hi] = target_logp(Z, lse[lo:hi], y[lo:hi], valid[lo:hi])
        if want_grads:
            G = grad_logits(Z, lse[lo:hi], y[lo:hi], valid[lo:hi], w[lo:hi])
            dH[lo:hi] = G @ Wd
            dW += G.T @ Hd[lo:hi]
    return lse, ell, dH, dW


def _prep(H, W, labels, V=None):
    Hd, Wd = widen(H), widen(W)
    y = np.asarray(labels, dtype=np.int64)
    assert Hd.ndim == 2 and Wd.ndim == 2 and Hd.shape[1] == Wd.shape[1] and y.shape[0] == Hd.shape[0]
    return Hd, Wd, y


def sft(H, W, labels, chunk: Optional[int] = None, strict: bool = True) -> Result:
    """SFT: loss = (1/N) sum over valid t of (lse_t - Z_{t,y_t})."""
    Hd, Wd, y = _prep(H, W, labels)
    scan = scan_labels(y, Wd.shape[0], strict=strict)
    w = weights_sft(scan)
    lse, ell, dH, dW = _backward(Hd, Wd, y, scan.valid, w, chunk)
    loss = float(-np.sum(w * ell))
    return Result(loss, dH, dW, ell, lse, w, scan)


def grpo(H, W, labels, offsets, adv, chunk: Optional[int] = None, strict: bool = True) -> Result:
    """On-policy GRPO head: loss = sum_t (-A_s/len_s) logp_t over valid tokens."""
    Hd, Wd, y = _prep(H, W, labels)
    scan = scan_labels(y, Wd.shape[0], offsets, strict=strict)
    w = weights_grpo(scan, offsets, adv)
    lse, ell, dH, dW = _backward(Hd, Wd, y, scan.valid, w, chunk)
    loss = float(-np.sum(w * ell))
    return Result(loss, dH, dW, ell, lse, w, scan)


def ppo_token_terms(ell: np.ndarray, valid: np.ndarray, adv_per_len: np.ndarray, inv_len: np.ndarray,
                    logp_old: np.ndarray, logp_ref: Optional[np.ndarray], eps: float, beta_kl: float):
    """Per-token loss terms and cross-entropy weights of the off-policy head.

    The news article lists PPO among the objectives StreamBP serves, and its
    LM-head paragraph needs only that each position's loss depends on that
    position's logits.  The objective itself is not written on the pages; the
    reading taken is the standard clipped surrogate with GRPO's per-sequence
    length normalisation and a per-token KL penalty:

        r_t   = exp(logp_t - logp_old_t)
        a_t   = A_s / len_s,  k_t = beta_kl / len_s
        L_t   = -min(r_t a_t, clip(r_t, 1-eps, 1+eps) a_t)
                + k_t (exp(d_t) - d_t - 1),   d_t = logp_ref_t - logp_t.

    dL_t/dlogp_t is -a_t r_t when the unclipped product is the minimum (ties
    included) and 0 when the clipped one is strictly smaller (then r_t lies
    outside the clip range, where the clipped term is flat), plus
    k_t (1 - exp(d_t)).  The cross-entropy weight is w_t = -dL_t/dlogp_t.
    Ignored rows have L_t = w_t = 0.  ``logp_ref`` may be None when
    beta_kl = 0."""
    ell = np.asarray(ell, dtype=np.float64)
    a = np.asarray(adv_per_len, dtype=np.float64)
    k = beta_kl * np.asarray(inv_len, dtype=np.float64)
    r = np.exp(ell - np.asarray(logp_old, dtype=np.float64))
    unclipped = r * a
    clipped = np.clip(r, 1.0 - eps, 1.0 + eps) * a
    takes_unclipped = unclipped <= clipped
    surrogate = -np.minimum(unclipped, clipped)
    d_surrogate = np.where(takes_unclipped, -a * r, 0.0)
    if logp_ref is None or beta_kl == 0.0:
        kl = np.zeros_like(ell)
        d_kl = np.zeros_like(ell)
    else:
        dref = np.asarray(logp_ref, dtype=np.float64) - ell
        kl = np.expm1(dref) - dref          # exp(d) - d - 1, accurate near d = 0
        d_kl = -np.expm1(dref)              # d/dlogp of exp(d) - d - 1
    loss_t = np.where(valid, surrogate + k * kl, 0.0)
    w = np.where(valid, -(d_surrogate + k * d_kl), 0.0)
    return loss_t, w


def ppo(H, W, labels, offsets, adv, logp_old, logp_ref=None, eps: float = 0.2, beta_kl: float = 0.0,
        chunk: Optional[int] = None, strict: bool = True) -> Result:
    """Off-policy clipped-surrogate head (PPO / off-policy GRPO with a KL
    penalty): loss = sum over valid t of L_t (see ``ppo_token_terms``).  Each
    chunk forms its logits, log-sum-exp and log-probs, then the per-token
    weights from those log-probs, then G, dH and its dW contribution."""
    Hd, Wd, y = _prep(H, W, labels)
    T, D = Hd.shape
    V = Wd.shape[0]
    scan = scan_labels(y, V, offsets, strict=strict)
    sid = seq_index(offsets, T)
    lens = scan.seq_len[sid] if T else np.zeros(0, dtype=np.int64)
    has = scan.valid & (lens > 0)
    adv = np.asarray(adv, dtype=np.float64)
    a = np.where(has, adv[sid] / np.maximum(lens, 1), 0.0) if T else np.zeros(0)
    inv_len = np.where(has, 1.0 / np.maximum(lens, 1), 0.0) if T else np.zeros(0)
    old = np.asarray(logp_old, dtype=np.float64)
    ref = None if logp_ref is None else np.asarray(logp_ref, dtype=np.float64)
    lse = np.zeros(T)
    ell = np.zeros(T)
    w = np.zeros(T)
    loss_t = np.zeros(T)
    dH = np.zeros((T, D))
    dW = np.zeros((V, D))
    for lo, hi in _chunks(T, chunk):
        Z = logits(Hd[lo:hi], Wd)
        lse[lo:hi] = logsumexp_rows(Z)
        ell[lo:hi] = target_logp(Z, lse[lo:hi], y[lo:hi], scan.valid[lo:hi])
        loss_t[lo:hi], w[lo:hi] = ppo_token_terms(
            ell[lo:hi], scan.valid[lo:hi], a[lo:hi], inv_len[lo:hi], old[lo:hi],
            None if ref is None else ref[lo:hi], eps, beta_kl)
        G = grad_logits(Z, lse[lo:hi], y[lo:hi], scan.valid[lo:hi], w[lo:hi])
        dH[lo:hi] = G @ Wd
        dW += G.T @ Hd[lo:hi]
    return Result(float(np.sum(loss_t)), dH, dW, ell, lse, w, scan)


def sequence_logp(ell: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    off = np.asarray(offsets, dtype=np.int64)
    return np.array([float(np.sum(ell[off[s]:off[s + 1]])) for s in range(len(off) - 1)])


def dpo_logp(H, W, labels, offsets, chunk: Optional[int] = None, strict: bool = True) -> Result:
    """DPO pass 1: S_s = sum of logp_t over the valid tokens of sequence s
    (a forward pass only; no gradients)."""
    Hd, Wd, y = _prep(H, W, labels)
    scan = scan_labels(y, Wd.shape[0], offsets, strict=strict)
    lse, ell = _forward(Hd, Wd, y, scan.valid, chunk)
    return Result(0.0, None, None, ell, lse, np.zeros_like(ell), scan,
                  seq_logp=sequence_logp(ell, offsets))


def dpo(H, W, labels, offsets, ref_logp, beta: float, chunk: Optional[int] = None,
        strict: bool = True) -> Result:
    """DPO head: pass 1 for the sequence log-probs, the pair factors, then the
    chunked backward with per-sequence weights."""
    Hd, Wd, y = _prep(H, W, labels)
    p1 = dpo_logp(H, W, labels, offsets, chunk, strict)
    pairs = dpo_pairs(p1.seq_logp, ref_logp, beta)
    w = weights_per_sequence(p1.scan, offsets, pairs.coef)
    lse, ell, dH, dW = _backward(Hd, Wd, y, p1.scan.valid, w, chunk)
    return Result(pairs.loss, dH, dW, ell, lse, w, p1.scan,
                  seq_logp=p1.seq_logp, delta=pairs.delta)


# --------------------------------------------------------------------------
# sampled evaluation at full size: the same definition on chosen rows only
# --------------------------------------------------------------------------
def rows_lse_logp(H, W, labels, rows: Sequence[int], V_block: int = 1 << 15):
    """lse_t and logp_t (label taken as valid if in range) for the given rows."""
    Wd = widen(W)
    Hr = widen(np.asarray(H)[np.asarray(rows)])
    y = np.asarray(labels, dtype=np.int64)[np.asarray(rows)]
    Z = logits(Hr, Wd)
    lse = logsumexp_rows(Z)
    valid = (y >= 0) & (y < Wd.shape[0])
    return lse, target_logp(Z, lse, y, valid)


def rows_dH(H, W, labels, w, rows: Sequence[int]) -> np.ndarray:
    """dH rows: G_t W with G_t from the definition; ``w`` is the full
    cross-entropy weight vector."""
    rows = np.asarray(rows)
    Wd = widen(W)
    Hr = widen(np.asarray(H)[rows])
    y = np.asarray(labels, dtype=np.int64)[rows]
    valid = (y >= 0) & (y < Wd.shape[0])
    Z = logits(Hr, Wd)
    lse = logsumexp_rows(Z)
    G = grad_logits(Z, lse, y, valid, np.asarray(w, dtype=np.float64)[rows])
    return G @ Wd


def all_lse(H, W, row_block: int = 512) -> np.ndarray:
    """lse of every row, computed block by block to bound memory (the same
    max-shifted log-sum-exp as logsumexp_rows, done in place on each block's
    own logits)."""
    Wd = widen(W)
    T = np.asarray(H).shape[0]
    out = np.zeros(T)
    for lo in range(0, T, row_block):
        Z = logits(widen(np.asarray(H)[lo:lo + row_block]), Wd)
        m = np.max(Z, axis=1)
        np.subtract(Z, m[:, None], out=Z)
        np.exp(Z, out=Z)
        out[lo:lo + row_block] = m + np.log(np.sum(Z, axis=1))
    return out


def cols_dW(H, W, labels, w, lse, cols: Sequence[int]) -> np.ndarray:
    """dW rows v in ``cols``: sum_t G_tv H_t, with G_tv = w_t (exp(Z_tv - lse_t) - [y_t == v])
    from the definition; ``lse`` is the full per-token log-sum-exp."""
    cols = np.asarray(cols)
    Hd = widen(H)
    Wc = widen(np.asarray(W)[cols])
    y = np.asarray(labels, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    Zc = Hd @ Wc.T                                      # [T, k]
    G = np.exp(Zc - np.asarray(lse)[:, None]) - (y[:, None] == cols[None, :])
    G *= w[:, None]
    return G.T @ Hd

"""GPU parity at the benchmark's full sizes.

* SFT, T=9000, D=2560, V=151936, C=1024 (the timed configuration, same
  launch path): the oracle computes every row's log-sum-exp in fp64, block by
  block; loss and n_valid are compared exactly / to tolerance, dH on sampled
  rows and dW on sampled vocabulary rows (chunk edges, tile edges, masked
  rows, V-1, label targets).
* GRPO (8 x 12288 tokens, D=4096) and DPO (4 pairs x 16384, D=5120) at full
  size through closed forms that hold at any size: with H = 0 every logit is 0,
  lse = ln V, logp = -ln V on valid rows, dH_t = w_t (mean_v W_v - W_{y_t}) and
  dW = 0; with W = 0, dH = 0 and dW_v = (1/V) sum_t w_t H_t - sum_{t: y_t = v} w_t H_t.
* GRPO, DPO and the long-context SFT (T = 2 x 8192 + 300, D = 5120, chunk
  sweep 2048 / 4096 / 8192) on their own seeded inputs, against the oracle's
  per-token log-sum-exp that tests/golden/make_fullsize_refs.py stores for
  exactly those inputs: losses, per-token logp, DPO sequence sums and pair
  factors, sampled dH rows and sampled dW vocabulary rows.
"""
import importlib.util
import math
import os

import numpy as np
import pytest
import torch

from oracle import streambp_oracle as O
from tests.gpu_helpers import TOL_BF16, head, loss_rel, np64, rel, require_gpu, row_check, to_dev
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _refs_module():
    spec = importlib.util.spec_from_file_location("make_fullsize_refs", os.path.join(GOLDEN, "make_fullsize_refs.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _stored_lse(name, inp):
    """The oracle's log-sum-exp of every valid row (tests/golden/make_fullsize_refs.py),
    checked to belong to these exact inputs; 0 on the other rows."""
    refs = _refs_module()
    z = np.load(refs.path(name))
    assert str(z["sha256"]) == refs.inputs_sha256(inp), f"{name}: stored oracle values are for other inputs"
    valid = (inp.labels >= 0) & (inp.labels < inp.wl.V)
    lse = np.zeros(inp.wl.T)
    lse[valid] = z["lse"].astype(np.float64)
    return lse


def _label_logits(inp, rows, block=8192):
    """fp64 Z[t, y_t] = H_t . W_{y_t} for the given rows, block by block."""
    out = np.zeros(len(rows))
    for lo in range(0, len(rows), block):
        r = rows[lo:lo + block]
        out[lo:lo + block] = np.einsum("td,td->t", O.widen(inp.H[r]), O.widen(inp.W[inp.labels[r]]))
    return out


def _oracle_logp(inp, lse):
    valid = np.nonzero((inp.labels >= 0) & (inp.labels < inp.wl.V))[0]
    logp = np.zeros(inp.wl.T)
    logp[valid] = _label_logits(inp, valid) - lse[valid]
    return logp


pytestmark = pytest.mark.gpu


def _case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def test_sft_9k_sampled_against_oracle():
    require_gpu()
    wl = gen.SFT_9K
    _case("sft_9k_full", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    loss, dH, dW, nv = hd.sft(d["H"], d["W"], d["y"])
    torch.cuda.synchronize()
    valid = inp.labels != -100
    N = int(valid.sum())
    assert int(nv.item()) == N == 8100
    print("  gpu done; oracle lse over all rows", flush=True)
    lse = O.all_lse(inp.H, inp.W, row_block=500)
    rows_v = np.nonzero(valid)[0]
    Hd = O.widen(inp.H[rows_v])
    zy = np.einsum("td,td->t", Hd, O.widen(inp.W[inp.labels[rows_v]]))
    ref_loss = float(np.sum(lse[rows_v] - zy) / N)
    assert abs(loss.item() - ref_loss) <= 1e-5 * abs(ref_loss), (loss.item(), ref_loss)
    w = valid / N
    rows = np.array([0, 1, 899, 900, 901, 1023, 1024, 2047, 2048, 4500, 8191, 8192, 8500, 8999])
    ref_dH = O.rows_dH(inp.H, inp.W, inp.labels, w, rows)
    got_dH = np64(dH[torch.from_numpy(rows).cuda()])
    e_dH = rel(got_dH, ref_dH)
    assert np.all(got_dH[:3] == 0.0)  # masked rows
    cols = np.unique(np.concatenate([[0, 1, 255, 256, 257, 75000, wl.V - 256, wl.V - 2, wl.V - 1],
                                     inp.labels[[900, 5000, 8999]]]))
    ref_dW = O.cols_dW(inp.H, inp.W, inp.labels, w, lse, cols)
    got_dW = np64(dW[torch.from_numpy(cols).cuda()])
    e_dW = rel(got_dW, ref_dW)
    print(f"  loss {abs(loss.item() - ref_loss) / abs(ref_loss):.2e} dH(sampled) {e_dH:.2e} "
          f"dW(sampled) {e_dW:.2e}", flush=True)
    assert e_dH <= TOL_BF16 and e_dW <= TOL_BF16


def _zero_hidden(wl, seed=0):
    inp = gen.make_inputs(wl, seed)
    inp.H = np.zeros_like(inp.H)
    return inp


def _wbar_minus_wy(W, labels, rows):
    """fp64 mean over vocabulary rows of W, minus W[y_t], for sampled rows."""
    Wd_sum = np.zeros(W.shape[1])
    for lo in range(0, W.shape[0], 16384):
        Wd_sum += O.widen(W[lo:lo + 16384]).sum(axis=0)
    wbar = Wd_sum / W.shape[0]
    out = np.zeros((len(rows), W.shape[1]))
    for k, t in enumerate(rows):
        if labels[t] != -100:
            out[k] = wbar - O.widen(W[labels[t]])
    return out


def test_grpo_full_size_zero_hidden_closed_form():
    require_gpu()
    wl = gen.GRPO
    _case("grpo_full_H0", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = _zero_hidden(wl)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    loss, logp, dH, dW = hd.grpo(d["H"], d["W"], d["y"], d["off"], d["adv"])
    torch.cuda.synchronize()
    scan = O.scan_labels(inp.labels, wl.V, inp.offsets)
    lnV = math.log(wl.V)
    want_loss = lnV * float(sum(float(inp.adv[s]) for s in range(wl.n_seq) if scan.seq_len[s] > 0))
    assert abs(loss.item() - want_loss) <= 1e-5 * max(1.0, abs(want_loss))
    lp = np64(logp)
    assert np.allclose(lp[scan.valid], -lnV, rtol=1e-6) and np.all(lp[~scan.valid] == 0)
    assert float(dW.abs().max()) == 0.0
    w = O.weights_grpo(scan, inp.offsets, inp.adv)
    rows = np.array([0, 3071, 3072, 3073, 12287, 12288 + 5000, 4 * 12288 + 3072, wl.T - 1])
    want = w[rows, None] * _wbar_minus_wy(inp.W, inp.labels, rows)
    got = np64(dH[torch.from_numpy(rows).cuda()])
    assert rel(got, want) <= TOL_BF16, rel(got, want)


def test_dpo_full_size_zero_hidden_closed_form():
    require_gpu()
    wl = gen.DPO
    _case("dpo_full_H0", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = _zero_hidden(wl)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    loss, seq, dH, dW = hd.dpo(d["H"], d["W"], d["y"], d["off"], d["ref"], wl.beta)
    torch.cuda.synchronize()
    scan = O.scan_labels(inp.labels, wl.V, inp.offsets)
    lnV = math.log(wl.V)
    want_seq = -scan.seq_len * lnV
    np.testing.assert_allclose(np64(seq), want_seq, rtol=1e-6)
    pairs = O.dpo_pairs(want_seq, inp.ref_logp, wl.beta)
    assert abs(loss.item() - pairs.loss) <= 1e-6 * max(1.0, abs(pairs.loss))
    assert float(dW.abs().max()) == 0.0
    w = O.weights_per_sequence(scan, inp.offsets, pairs.coef)
    rows = np.array([0, 4095, 4096, 16383, 16384 + 4096, 4 * 16384 + 5000, wl.T - 1])
    want = w[rows, None] * _wbar_minus_wy(inp.W, inp.labels, rows)
    got = np64(dH[torch.from_numpy(rows).cuda()])
    assert rel(got, want) <= TOL_BF16, rel(got, want)


def test_ppo_full_size_zero_hidden_closed_form():
    # H = 0: every logit is 0 and logp = -ln V on valid rows, so the oracle's
    # per-token terms at logp = -ln V give the weights exactly; then
    # dH_t = w_t (mean_v W_v - W_{y_t}) and dW = 0
    require_gpu()
    wl = gen.PPO
    _case("ppo_full_H0", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = _zero_hidden(wl)
    lnV = math.log(wl.V)
    steps = np.array([-0.6, -0.05, 0.05, 0.6])
    old = (-lnV - steps[np.arange(wl.T) % 4]).astype(np.float32)
    ref = (-lnV + 0.3 * np.cos(np.arange(wl.T))).astype(np.float32)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    loss, logp, dH, dW = hd.ppo(d["H"], d["W"], d["y"], d["off"], d["adv"], torch.from_numpy(old).cuda(),
                                torch.from_numpy(ref).cuda(), 0.2, wl.beta)
    torch.cuda.synchronize()
    scan = O.scan_labels(inp.labels, wl.V, inp.offsets)
    sid = O.seq_index(inp.offsets, wl.T)
    lens = scan.seq_len[sid]
    a = np.where(scan.valid, inp.adv[sid] / np.maximum(lens, 1), 0.0)
    il = np.where(scan.valid, 1.0 / np.maximum(lens, 1), 0.0)
    ell = np.where(scan.valid, -lnV, 0.0)
    loss_t, w = O.ppo_token_terms(ell, scan.valid, a, il, old, ref, 0.2, wl.beta)
    assert loss_rel(loss.item(), float(loss_t.sum()), float(np.abs(loss_t).sum())) <= 1e-5
    assert float(dW.abs().max()) == 0.0
    rows = np.array([0, 3071, 3072, 3073, 12287, 12288 + 5001, 4 * 12288 + 3074, wl.T - 1])
    want = w[rows, None] * _wbar_minus_wy(inp.W, inp.labels, rows)
    got = np64(dH[torch.from_numpy(rows).cuda()])
    assert rel(got, want) <= TOL_BF16, rel(got, want)


def test_sft_9k_compacted_sampled_against_oracle():
    # masked-row compaction at the benchmark size: loss exact to tolerance,
    # dH on sampled rows (ignored rows exactly 0), dW on sampled vocab rows
    require_gpu()
    wl = gen.SFT_9K
    _case("sft_9k_compacted", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype, compact=True)
    loss, dH, dW, nv = hd.sft(d["H"], d["W"], d["y"])
    torch.cuda.synchronize()
    valid = inp.labels != -100
    N = int(valid.sum())
    assert int(nv.item()) == N
    lse = O.all_lse(inp.H, inp.W, row_block=500)
    rows_v = np.nonzero(valid)[0]
    zy = np.einsum("td,td->t", O.widen(inp.H[rows_v]), O.widen(inp.W[inp.labels[rows_v]]))
    ref_loss = float(np.sum(lse[rows_v] - zy) / N)
    assert abs(loss.item() - ref_loss) <= 1e-5 * abs(ref_loss)
    w = valid / N
    rows = np.array([0, 899, 900, 1023, 1924, 1925, 4500, 8999])
    got_dH = np64(dH[torch.from_numpy(rows).cuda()])
    assert np.all(got_dH[:2] == 0.0)
    assert rel(got_dH, O.rows_dH(inp.H, inp.W, inp.labels, w, rows)) <= TOL_BF16
    cols = np.unique(np.concatenate([[0, 256, wl.V - 1], inp.labels[[900, 5000, 8999]]]))
    ref_dW = O.cols_dW(inp.H, inp.W, inp.labels, w, lse, cols)
    assert rel(np64(dW[torch.from_numpy(cols).cuda()]), ref_dW) <= TOL_BF16


def _zero_weight_dW_check(wl, kind):
    require_gpu()
    _case(f"{kind}_full_W0", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = gen.make_inputs(wl, 1)
    inp.W = np.zeros_like(inp.W)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    scan = O.scan_labels(inp.labels, wl.V, inp.offsets)
    if kind == "grpo":
        loss, logp, dH, dW = hd.grpo(d["H"], d["W"], d["y"], d["off"], d["adv"])
        w = O.weights_grpo(scan, inp.offsets, inp.adv)
    else:
        ref = torch.zeros(wl.n_seq, dtype=torch.float64, device="cuda")
        loss, seq, dH, dW = hd.dpo(d["H"], d["W"], d["y"], d["off"], ref, wl.beta)
        # every logit is 0, so S_s = -len_s ln V and Delta_i = 0 for equal lengths
        S = -scan.seq_len * math.log(wl.V)
        w = O.weights_per_sequence(scan, inp.offsets, O.dpo_pairs(S, np.zeros(wl.n_seq), wl.beta).coef)
    torch.cuda.synchronize()
    assert float(dH.abs().max()) == 0.0
    # sum_t w_t H_t in fp64, block by block
    acc = np.zeros(wl.D)
    for lo in range(0, wl.T, 8192):
        acc += (w[lo:lo + 8192, None] * O.widen(inp.H[lo:lo + 8192])).sum(axis=0)
    targets = inp.labels[scan.valid]
    cols = np.unique(np.concatenate([[0, wl.V - 1, 12345], targets[:6]]))
    want = np.tile(acc / wl.V, (len(cols), 1))
    for k, v in enumerate(cols):
        hit = np.nonzero(inp.labels == v)[0]
        if hit.size:
            want[k] -= (w[hit, None] * O.widen(inp.H[hit])).sum(axis=0)
    got = np64(dW[torch.from_numpy(cols).cuda()])
    assert rel(got, want) <= TOL_BF16, rel(got, want)


def test_grpo_full_size_zero_weight_closed_form():
    _zero_weight_dW_check(gen.GRPO, "grpo")


def test_dpo_full_size_zero_weight_closed_form():
    _zero_weight_dW_check(gen.DPO, "dpo")


# ---------------------------------------------------------------------------
# Full sizes with the benchmark's own seeded inputs (not degenerate ones): the
# oracle evaluates the definition row by row on sampled rows.  Ignored rows
# must come back exactly 0.


def _sampled_rows(wl, scan, extra=()):
    """Ignored rows, the first and last valid row of every sequence, rows at
    chunk edges and a few inside; sorted, unique."""
    rows = set(int(r) for r in extra)
    off = np.arange(wl.n_seq + 1) * (wl.T // wl.n_seq)
    for s in range(wl.n_seq):
        v = np.nonzero(scan.valid[off[s]:off[s + 1]])[0] + off[s]
        if v.size:
            rows.update((int(v[0]), int(v[-1]), int(v[v.size // 2])))
        rows.add(int(off[s]))  # a prompt (ignored) row
    for c in (1, 2, wl.T // wl.C - 1):
        rows.update((c * wl.C - 1, c * wl.C))
    return np.array(sorted(r for r in rows if 0 <= r < wl.T))


def _check_rows(rows, scan, got_dH, want_dH, got_logp=None, want_logp=None):
    ign = ~scan.valid[rows]
    assert ign.any() and (~ign).any()
    assert np.all(got_dH[ign] == 0.0)
    e_dH = rel(got_dH[~ign], want_dH[~ign])
    msg = f"  rows {len(rows)} dH(sampled) {e_dH:.2e}"
    ok = e_dH <= TOL_BF16
    if got_logp is not None:
        assert np.all(got_logp[ign] == 0.0)
        e_lp = rel(got_logp[~ign], want_logp[~ign])
        msg += f" logp(sampled) {e_lp:.2e}"
        ok = ok and e_lp <= TOL_BF16
    print(msg, flush=True)
    assert ok


def test_grpo_full_size_sampled_rows():
    # the benchmark's GRPO inputs at full size: loss and every token's logp
    # against the oracle's (from its stored per-token log-sum-exp), sampled dH
    # rows, and sampled dW vocabulary rows (label targets, tile and range edges)
    require_gpu()
    wl = gen.GRPO
    _case("grpo_full_sampled", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    loss, logp, dH, dW = hd.grpo(d["H"], d["W"], d["y"], d["off"], d["adv"])
    torch.cuda.synchronize()
    assert int(hd.status.item()) == 0
    scan = O.scan_labels(inp.labels, wl.V, inp.offsets)
    rows = _sampled_rows(wl, scan, extra=(5 * 12288 + 7001,))
    cols = np.unique(np.concatenate([[0, 255, 256, 75000, wl.V - 256, wl.V - 1],
                                     inp.labels[[3072, 12288 + 5000, wl.T - 1]]]))
    idx = torch.from_numpy(rows).cuda()
    got_dH, got_lp_rows, got_lp = np64(dH[idx]), np64(logp[idx]), np64(logp)
    got_dW = np64(dW[torch.from_numpy(cols).cuda()])
    got_loss = loss.item()
    del d, dH, dW, logp
    lse = _stored_lse(wl.name, inp)
    want_lp = _oracle_logp(inp, lse)
    w = O.weights_grpo(scan, inp.offsets, inp.adv)
    want_loss = float(-np.sum(w * want_lp))
    e_loss = loss_rel(got_loss, want_loss, float(np.sum(np.abs(w * want_lp))))
    e_lp = rel(got_lp, want_lp)
    assert np.all(got_lp[~scan.valid] == 0.0)
    want_dH = O.rows_dH(inp.H, inp.W, inp.labels, w, rows)
    _check_rows(rows, scan, got_dH, want_dH, got_lp_rows, want_lp[rows])
    want_dW = O.cols_dW(inp.H, inp.W, inp.labels, w, lse, cols)
    e_dW = rel(got_dW, want_dW)
    r_dW = row_check(got_dW, want_dW, TOL_BF16, "dW")
    print(f"  loss {e_loss:.2e} logp(all) {e_lp:.2e} dW(sampled) {e_dW:.2e} (worst row {r_dW:.2e})", flush=True)
    assert e_loss <= TOL_BF16 and e_lp <= TOL_BF16 and e_dW <= TOL_BF16


def test_ppo_full_size_sampled_rows():
    # the benchmark's behaviour and reference log-probs; rows whose ratio lies
    # within 1e-3 (in log) of a clip edge are left out: there the fp32 and
    # fp64 log-probs may take different branches of the min, and either is right
    require_gpu()
    wl = gen.PPO
    eps = 0.2
    _case("ppo_full_sampled", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    _, logp, dH, _ = hd.ppo(d["H"], d["W"], d["y"], d["off"], d["adv"], torch.from_numpy(inp.logp_old).cuda(),
                            torch.from_numpy(inp.logp_ref).cuda(), eps, wl.beta)
    torch.cuda.synchronize()
    assert int(hd.status.item()) == 0
    scan = O.scan_labels(inp.labels, wl.V, inp.offsets)
    rows = _sampled_rows(wl, scan, extra=(5 * 12288 + 7001, 6 * 12288 + 9000))
    _, ell = O.rows_lse_logp(inp.H, inp.W, inp.labels, rows)
    valid = scan.valid[rows]
    log_r = ell - inp.logp_old[rows].astype(np.float64)
    near = valid & (np.minimum(np.abs(log_r - math.log(1 - eps)), np.abs(log_r - math.log(1 + eps))) < 1e-3)
    rows, ell, valid = rows[~near], ell[~near], valid[~near]
    idx = torch.from_numpy(rows).cuda()
    got_dH, got_lp = np64(dH[idx]), np64(logp[idx])
    del d, dH, logp
    sid = O.seq_index(inp.offsets, wl.T)[rows]
    lens = np.maximum(scan.seq_len[sid], 1)
    a = np.where(valid, inp.adv[sid] / lens, 0.0)
    il = np.where(valid, 1.0 / lens, 0.0)
    _, w_rows = O.ppo_token_terms(ell, valid, a, il, inp.logp_old[rows], inp.logp_ref[rows], eps, wl.beta)
    w = np.zeros(wl.T)
    w[rows] = w_rows
    want_dH = O.rows_dH(inp.H, inp.W, inp.labels, w, rows)
    _check_rows(rows, scan, got_dH, want_dH, got_lp, ell)


def test_long_sft_full_size_sampled_rows():
    # T = 32768, D = 5120 (not RMS-normalised), 5% of positions ignored at random
    require_gpu()
    wl = gen.LONG
    _case("long_sft_full_sampled", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    _, dH, _, nv = hd.sft(d["H"], d["W"], d["y"])
    torch.cuda.synchronize()
    scan = O.scan_labels(inp.labels, wl.V, inp.offsets)
    assert int(nv.item()) == scan.n_valid == wl.T - 1638
    ign = np.nonzero(~scan.valid)[0]
    rows = np.unique(np.concatenate([_sampled_rows(wl, scan), ign[:3], ign[-2:], [wl.T - 1, 20000]]))
    got_dH = np64(dH[torch.from_numpy(rows).cuda()])
    del d, dH
    want_dH = O.rows_dH(inp.H, inp.W, inp.labels, O.weights_sft(scan), rows)
    _check_rows(rows, scan, got_dH, want_dH)


def test_dpo_full_size_rows_scale_per_sequence():
    # Full DPO needs every token's log-prob for the pair factors, which the
    # oracle cannot afford at this size.  What holds at any size: on the valid
    # rows of sequence s, dH_t = c_s u_t with u_t = (softmax_t - onehot(y_t)) W
    # (the oracle's row gradient at weight 1), c_s = (beta/P) sigma(-beta Delta_i)
    # on the chosen side of pair i and its negative on the rejected side, so
    # 0 <= c_i = -c_{P+i} <= beta/P.
    require_gpu()
    wl = gen.DPO
    _case("dpo_full_rows", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    _, _, dH, _ = hd.dpo(d["H"], d["W"], d["y"], d["off"], d["ref"], wl.beta)
    torch.cuda.synchronize()
    assert int(hd.status.item()) == 0
    scan = O.scan_labels(inp.labels, wl.V, inp.offsets)
    rows = _sampled_rows(wl, scan)
    got = np64(dH[torch.from_numpy(rows).cuda()])
    del d, dH
    u = O.rows_dH(inp.H, inp.W, inp.labels, scan.valid.astype(np.float64), rows)
    ign = ~scan.valid[rows]
    assert np.all(got[ign] == 0.0)
    sid = O.seq_index(inp.offsets, wl.T)[rows]
    P = wl.n_seq // 2
    c = np.zeros(wl.n_seq)
    fit = np.zeros_like(got)
    for s in range(wl.n_seq):
        m = (sid == s) & ~ign
        assert m.sum() >= 2
        c[s] = float(np.sum(got[m] * u[m]) / np.sum(u[m] * u[m]))
        fit[m] = c[s] * u[m]
    e = rel(got[~ign], fit[~ign])
    print(f"  rows {len(rows)} dH vs c_s u_t {e:.2e}; c = {np.array2string(c, precision=3)}", flush=True)
    assert e <= TOL_BF16
    bound = wl.beta / P
    assert np.all(c[:P] >= -1e-6 * bound) and np.all(c[:P] <= bound * (1 + TOL_BF16))
    assert np.all(np.abs(c[:P] + c[P:]) <= TOL_BF16 * bound)


def test_dpo_full_size_against_oracle():
    # The benchmark's DPO inputs at full size (4 pairs x 16384 tokens,
    # D = 5120): pass 1's fp64 sequence sums against the oracle's (every
    # valid token's logp from its stored log-sum-exp), the loss, and sampled
    # dH rows and dW vocabulary rows with the oracle's pair factors.
    require_gpu()
    wl = gen.DPO
    _case("dpo_full_oracle", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    loss, seq, dH, dW = hd.dpo(d["H"], d["W"], d["y"], d["off"], d["ref"], wl.beta)
    torch.cuda.synchronize()
    assert int(hd.status.item()) == 0
    scan = O.scan_labels(inp.labels, wl.V, inp.offsets)
    rows = _sampled_rows(wl, scan)
    cols = np.unique(np.concatenate([[0, 256, 99999, wl.V - 1], inp.labels[[4096, 16384 + 9000, wl.T - 1]]]))
    got_seq, got_loss = np64(seq), loss.item()
    got_dH = np64(dH[torch.from_numpy(rows).cuda()])
    got_dW = np64(dW[torch.from_numpy(cols).cuda()])
    del d, dH, dW
    lse = _stored_lse(wl.name, inp)
    want_seq = O.sequence_logp(_oracle_logp(inp, lse), inp.offsets)
    pairs = O.dpo_pairs(want_seq, inp.ref_logp, wl.beta)
    w = O.weights_per_sequence(scan, inp.offsets, pairs.coef)
    e_seq = rel(got_seq, want_seq)
    e_loss = loss_rel(got_loss, pairs.loss, 0.0)
    P = wl.n_seq // 2
    print(f"  seq {e_seq:.2e} (max |dS| {np.max(np.abs(got_seq - want_seq)):.3e}) loss {e_loss:.2e}; "
          f"beta*Delta {np.array2string(wl.beta * pairs.delta, precision=2)}; factors "
          f"{np.array2string(pairs.coef[:P], precision=3)}", flush=True)
    want_dH = O.rows_dH(inp.H, inp.W, inp.labels, w, rows)
    _check_rows(rows, scan, got_dH, want_dH)
    want_dW = O.cols_dW(inp.H, inp.W, inp.labels, w, lse, cols)
    e_dW = rel(got_dW, want_dW)
    r_dW = row_check(got_dW, want_dW, TOL_BF16, "dW")
    print(f"  dW(sampled) {e_dW:.2e} (worst row {r_dW:.2e})", flush=True)
    assert e_seq <= TOL_BF16 and e_loss <= TOL_BF16 and e_dW <= TOL_BF16


@pytest.mark.parametrize("C", [2048, 4096, 8192])
def test_long_sft_chunk_sweep_against_oracle(C):
    # The long-context SFT inputs (D = 5120, not RMS-normalised, 5% ignored at
    # random) at T = 2 * 8192 + 300, so that every chunk size of the sweep runs
    # two or more chunks and a ragged tail; the dW GEMM's K is C.  Loss and
    # n_valid against the oracle, sampled dH rows and dW vocabulary rows.
    require_gpu()
    refs = _refs_module()
    wl = refs.LONG_REDUCED.with_(C=C)
    _case("long_sft_sweep", T=wl.T, D=wl.D, V=wl.V, C=C)
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, C, wl.dtype)
    loss, dH, dW, nv = hd.sft(d["H"], d["W"], d["y"])
    torch.cuda.synchronize()
    scan = O.scan_labels(inp.labels, wl.V)
    assert int(nv.item()) == scan.n_valid
    ign = np.nonzero(~scan.valid)[0]
    rows = np.unique(np.concatenate([[0, C - 1, C, 2 * C - 1, 2 * C, wl.T - 1, 7777], ign[:2], ign[-2:]]))
    cols = np.unique(np.concatenate([[0, 255, 256, 123456, wl.V - 1], inp.labels[[C, 2 * C + 5, wl.T - 1]]]))
    cols = cols[cols >= 0]
    got_loss = loss.item()
    got_dH = np64(dH[torch.from_numpy(rows).cuda()])
    got_dW = np64(dW[torch.from_numpy(cols).cuda()])
    del d, dH, dW
    lse = _stored_lse(wl.name, inp)
    w = O.weights_sft(scan)
    want_loss = float(-np.sum(w * _oracle_logp(inp, lse)))
    e_loss = loss_rel(got_loss, want_loss, 0.0)
    want_dH = O.rows_dH(inp.H, inp.W, inp.labels, w, rows)
    want_dW = O.cols_dW(inp.H, inp.W, inp.labels, w, lse, cols)
    ok_rows = scan.valid[rows]
    assert np.all(got_dH[~ok_rows] == 0.0)
    e_dH, e_dW = rel(got_dH, want_dH), rel(got_dW, want_dW)
    r_dH, r_dW = row_check(got_dH, want_dH, TOL_BF16, "dH"), row_check(got_dW, want_dW, TOL_BF16, "dW")
    print(f"  loss {e_loss:.2e} dH(sampled) {e_dH:.2e} dW(sampled) {e_dW:.2e} (worst rows {r_dH:.2e} "
          f"{r_dW:.2e})", flush=True)
    assert e_loss <= TOL_BF16 and e_dH <= TOL_BF16 and e_dW <= TOL_BF16

"""GPU parity: the HIP path through the C interface against the fp64 oracle on
the same seeded inputs.  fp32 inputs must match to 1e-5 and bf16 inputs to
2e-2 relative Frobenius error; integer outputs must match exactly."""
import numpy as np
import pytest
import torch

from oracle import streambp_oracle as O
from tests.gpu_helpers import (TOL_BF16, TOL_F32, abs_products, head, kl_steps, loss_rel, np64, ppo_row_scale,
                               rel, require_gpu, row_check, to_dev)
from workloads import gen

pytestmark = pytest.mark.gpu


def _tol(wl):
    return TOL_F32 if wl.dtype == "f32" else TOL_BF16


def _print_case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _check_sft(wl, seed=0, C=None, compact=False):
    require_gpu()
    C = C or wl.C
    _print_case("sft", wl=wl.name, T=wl.T, D=wl.D, V=wl.V, C=C, seed=seed, compact=compact)
    inp = gen.make_inputs(wl, seed)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, C, wl.dtype, compact)
    loss, dH, dW, nv = hd.sft(d["H"], d["W"], d["y"])
    torch.cuda.synchronize()
    ref = O.sft(inp.H, inp.W, inp.labels)
    tol = _tol(wl)
    assert int(nv.item()) == ref.scan.n_valid
    assert int(hd.status.item()) == 0
    e_loss = loss_rel(loss.item(), ref.loss, 0.0)
    gH, gW = np64(dH), np64(dW)
    e_dH, e_dW = rel(gH, ref.dH), rel(gW, ref.dW)
    aH, aW = abs_products(inp.H, inp.W, inp.labels, ref)
    r_dH, r_dW = row_check(gH, ref.dH, tol, "dH", aH), row_check(gW, ref.dW, tol, "dW", aW)
    print(f"  loss {e_loss:.2e} dH {e_dH:.2e} dW {e_dW:.2e} (worst row dH {r_dH:.2e} dW {r_dW:.2e})", flush=True)
    assert e_loss <= tol and e_dH <= tol and e_dW <= tol
    return e_loss, e_dH, e_dW


@pytest.mark.parametrize("C", [200, 640, 832, 1024, 2048])
def test_bf16_dw_update_variants_accumulate(C):
    """The old dW tile is streamed in during the GEMM loop, one piece per
    segment of 2 or more k-stages of 32 rows; chunks of fewer than 16 stages
    are padded with zero rows.  The chunk lengths here give 7 (padded), 20,
    26, 32 and 64 stages and segments of 2 to 8; the last chunk (333 rows, 11
    stages; 133 rows at C = 200) is padded too.  D and V are off the 256 tile grid and the
    caller's dW is not zero: dW must come back as base + the oracle's
    gradient."""
    require_gpu()
    wl = gen.SFT_9K.with_(T=2 * C + 333, D=200, V=1003, C=C)
    _print_case("dw_variants", wl=wl.name, T=wl.T, D=wl.D, V=wl.V, C=C)
    inp = gen.make_inputs(wl, 5)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, C, wl.dtype)
    g = torch.Generator(device="cuda").manual_seed(7)
    base = torch.randn(wl.V, wl.D, device="cuda", generator=g) * 1e-2
    acc = base.clone()
    _, dH, _, _ = hd.sft(d["H"], d["W"], d["y"], dW=acc, accumulate=True)
    torch.cuda.synchronize()
    assert int(hd.status.item()) == 0
    ref = O.sft(inp.H, inp.W, inp.labels)
    e_dH, e_dW = rel(np64(dH), ref.dH), rel(np64(acc) - np64(base), ref.dW)
    print(f"  dH {e_dH:.2e} dW {e_dW:.2e}", flush=True)
    assert e_dH <= TOL_BF16 and e_dW <= TOL_BF16


def test_tiny_sft_f32():
    _check_sft(gen.TINY)


@pytest.mark.parametrize("C", [1, 37, 64, 255, 256, 300])
def test_tiny_sft_f32_chunk_sizes(C):
    _check_sft(gen.TINY.with_(T=256), C=C)


def test_f32_ragged_vocab_and_rows():
    # V not a multiple of the 64-wide tile nor of 8; T not a multiple of C
    _check_sft(gen.TINY.with_(T=203, V=1003, D=136, C=48))


def test_bf16_sft_reduced():
    wl = gen.SFT_9K.with_(T=600, D=512, V=8000, C=256)
    _check_sft(wl)


def test_bf16_sft_ragged_vocab():
    # V % 256 != 0 and V % 8 != 0: ragged vocab tile and padded logits rows
    _check_sft(gen.SFT_9K.with_(T=300, D=256, V=5003, C=128))


def test_bf16_sft_several_tiles_and_tail():
    # spans several 256-wide token and vocab tiles with a ragged tail chunk
    _check_sft(gen.SFT_9K.with_(T=1100, D=1024, V=20000, C=512))


@pytest.mark.parametrize("D,C", [(200, 112), (72, 45), (1000, 300)])
def test_bf16_sft_partial_k_stages(D, C):
    # D (the logits GEMM's K), the padded vocabulary (the dH GEMM's K) and the
    # chunk rows (the dW GEMM's K) all leave a partial last 32-wide k-stage
    _check_sft(gen.SFT_9K.with_(T=333, D=D, V=1003, C=C))


# More vocabulary tiles than CUs with a partial last round of tiles, the last
# vocabulary tile ragged (76763 = 299 x 256 + 219 rows) and D = 1000 leaving a
# partial last k-stage; chunks of one and two token tiles.
MANY_VTILES = dict(D=1000, V=76763)


def test_bf16_sft_many_vocab_tiles():
    # chunks of 512 (two token tiles) and 188 rows (one)
    _check_sft(gen.SFT_9K.with_(T=700, C=512, **MANY_VTILES))


def test_grpo_bf16_many_vocab_tiles():
    _grpo_case(gen.GRPO.with_(T=4 * 150, C=512, n_seq=4, **MANY_VTILES))


@pytest.mark.parametrize("fuse", [False, True], ids=["row_pass", "fused"])
def test_dpo_bf16_many_vocab_tiles(fuse):
    _dpo_case(gen.DPO.with_(T=4 * 150, C=256, n_seq=4, **MANY_VTILES), fuse=fuse)


@pytest.mark.parametrize("T,D,V,C,dtype", [(5, 8, 9, 3, "bf16"), (5, 8, 9, 3, "f32"), (1, 256, 97, 64, "bf16"),
                                           (257, 264, 250, 256, "bf16"), (257, 264, 250, 256, "f32")],
                         ids=["D8_V9_C3_bf16", "D8_V9_C3_f32", "T1_V97_bf16", "T257_V250_bf16", "T257_V250_f32"])
def test_sft_tiny_extremes(T, D, V, C, dtype):
    # the smallest feature width (one partial k-stage of 8), a vocabulary of
    # a single ragged tile, chunks of a few rows, a single token, and one row
    # past a whole token tile
    base = gen.TINY if dtype == "f32" else gen.SFT_9K
    _check_sft(base.with_(T=T, D=D, V=V, C=C, mask="random", mask_frac=0.2))


@pytest.mark.parametrize("T,D,V,C", [(5, 8, 9, 3), (1, 256, 97, 64), (257, 264, 250, 256)],
                         ids=["D8_V9_C3", "T1_V97", "T257_V250"])
def test_sft_tiny_extremes_compacted(T, D, V, C):
    # the same shapes with masked-row compaction (bf16): the chunk loop runs
    # over the valid rows only
    _check_sft(gen.SFT_9K.with_(T=T, D=D, V=V, C=C, mask="random", mask_frac=0.2), compact=True)


def empty_and_masked_sequences(inp):
    """Sequence 0 empty (equal offsets), sequence 1 with every label ignored,
    sequence 2 empty, the last one the rest (4 sequences)."""
    T = inp.labels.shape[0]
    inp.offsets = np.array([0, 0, T // 3, T // 3, T], dtype=np.int32)
    inp.labels = inp.labels.copy()
    inp.labels[: T // 3] = -100


def masked_sequence(inp):
    """Every label of sequence 1 ignored (its log-prob sum is exactly 0)."""
    inp.labels = inp.labels.copy()
    inp.labels[inp.offsets[1]:inp.offsets[2]] = -100


@pytest.mark.parametrize("compact", [False, True], ids=["plain", "compacted"])
def test_grpo_empty_and_masked_sequences(compact):
    _grpo_case(gen.GRPO.with_(T=300, D=256, V=3000, C=128, n_seq=4), compact=compact,
               edit=empty_and_masked_sequences)


def test_ppo_empty_and_masked_sequences():
    _ppo_case(gen.PPO.with_(T=300, D=256, V=3000, C=128, n_seq=4), edit=empty_and_masked_sequences)


@pytest.mark.parametrize("fuse", [False, True], ids=["row_pass", "fused"])
def test_dpo_masked_sequence(fuse):
    _dpo_case(gen.DPO.with_(T=4 * 75, D=256, V=3000, C=128, n_seq=4), fuse=fuse, edit=masked_sequence)


def _dirty(hd, wl):
    """Fill the head's workspace with NaN bit patterns (0xFF bytes) before a call."""
    ws, _ = hd.workspace(wl.T, wl.n_seq)
    ws.fill_(0xFF)
    torch.cuda.synchronize()


def _grpo_case(wl, seed=0, compact=False, dirty=False, edit=None):
    require_gpu()
    _print_case("grpo", wl=wl.name, T=wl.T, D=wl.D, V=wl.V, C=wl.C, compact=compact, dirty=dirty,
                edit=getattr(edit, "__name__", None))
    inp = gen.make_inputs(wl, seed)
    if edit is not None:
        edit(inp)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype, compact)
    if dirty:
        _dirty(hd, wl)
    loss, logp, dH, dW = hd.grpo(d["H"], d["W"], d["y"], d["off"], d["adv"])
    torch.cuda.synchronize()
    ref = O.grpo(inp.H, inp.W, inp.labels, inp.offsets, inp.adv)
    tol = _tol(wl)
    scale = float(np.sum(np.abs(ref.w * ref.logp)))
    e_loss = loss_rel(loss.item(), ref.loss, scale)
    e_lp = rel(np64(logp), ref.logp)
    gH, gW = np64(dH), np64(dW)
    e_dH, e_dW = rel(gH, ref.dH), rel(gW, ref.dW)
    aH, aW = abs_products(inp.H, inp.W, inp.labels, ref)
    r_dH, r_dW = row_check(gH, ref.dH, tol, "dH", aH), row_check(gW, ref.dW, tol, "dW", aW)
    print(f"  loss {e_loss:.2e} logp {e_lp:.2e} dH {e_dH:.2e} dW {e_dW:.2e} "
          f"(worst row dH {r_dH:.2e} dW {r_dW:.2e})", flush=True)
    assert max(e_loss, e_lp, e_dH, e_dW) <= tol
    # ignored rows report logp exactly 0
    assert np.all(np64(logp)[inp.labels == -100] == 0.0)


def test_grpo_f32():
    _grpo_case(gen.GRPO.with_(dtype="f32", T=4 * 96, D=128, V=3000, C=100, n_seq=4))


def test_grpo_bf16_reduced():
    _grpo_case(gen.GRPO.with_(T=4 * 320, D=512, V=9000, C=256, n_seq=4))


def _ppo_inputs(inp, steps=(-0.6, -0.05, 0.05, 0.6)):
    """Old log-probs a fixed step from the oracle's current ones, so the ratios
    land on both sides of the clip range and never near its edges; reference
    log-probs a seeded random step of at least 0.25 away.  (The KL term's
    slope, expm1(logp_ref - logp), is ill-conditioned in logp where the two
    nearly agree: fp32 log-probs would then give that slope a relative error
    of eps_fp32 * |lse| / |logp_ref - logp|.)"""
    cur = O.sft(inp.H, inp.W, inp.labels, strict=False).logp
    T = cur.shape[0]
    old = (cur - np.asarray(steps)[np.arange(T) % len(steps)]).astype(np.float32)
    ref = (cur + kl_steps(T)).astype(np.float32)
    return old, ref


def _ppo_case(wl, eps=0.2, beta=0.05, seed=0, compact=False, edit=None):
    require_gpu()
    _print_case("ppo", wl=wl.name, T=wl.T, D=wl.D, V=wl.V, C=wl.C, eps=eps, beta=beta, compact=compact,
                edit=getattr(edit, "__name__", None))
    inp = gen.make_inputs(wl, seed)
    if edit is not None:
        edit(inp)
    old, refl = _ppo_inputs(inp)
    d = to_dev(inp)
    t_old, t_ref = torch.from_numpy(old).cuda(), torch.from_numpy(refl).cuda()
    hd = head(wl.D, wl.V, wl.C, wl.dtype, compact)
    loss, logp, dH, dW = hd.ppo(d["H"], d["W"], d["y"], d["off"], d["adv"], t_old, t_ref if beta else None,
                                eps, beta)
    torch.cuda.synchronize()
    ref = O.ppo(inp.H, inp.W, inp.labels, inp.offsets, inp.adv, old, refl if beta else None, eps, beta)
    tol = _tol(wl)
    scale = float(np.sum(np.abs(ref.w * ref.logp)))
    e_loss = loss_rel(loss.item(), ref.loss, scale)
    e_lp = rel(np64(logp), ref.logp)
    gH, gW = np64(dH), np64(dW)
    e_dH, e_dW = rel(gH, ref.dH), rel(gW, ref.dW)
    sid = O.seq_index(inp.offsets, wl.T)
    lens = np.maximum(ref.scan.seq_len[sid], 1)
    sc = ppo_row_scale(ref.dH, ref.logp, ref.scan.valid, inp.adv[sid] / lens, 1.0 / lens, old,
                       refl if beta else None, eps, beta)
    aH, aW = abs_products(inp.H, inp.W, inp.labels, ref)
    r_dH, r_dW = row_check(gH, ref.dH, tol, "dH", aH, sc), row_check(gW, ref.dW, tol, "dW", aW)
    print(f"  loss {e_loss:.2e} logp {e_lp:.2e} dH {e_dH:.2e} dW {e_dW:.2e} "
          f"(worst row dH {r_dH:.2e} dW {r_dW:.2e})", flush=True)
    assert int(hd.status.item()) == 0
    assert max(e_loss, e_lp, e_dH, e_dW) <= tol


def test_ppo_f32():
    _ppo_case(gen.PPO.with_(dtype="f32", T=4 * 96, D=128, V=3000, C=100, n_seq=4))


def test_ppo_f32_no_kl():
    _ppo_case(gen.PPO.with_(dtype="f32", T=4 * 96, D=128, V=3000, C=100, n_seq=4), beta=0.0)


def test_ppo_bf16_reduced():
    _ppo_case(gen.PPO.with_(T=4 * 320, D=512, V=9000, C=256, n_seq=4))


def test_ppo_bf16_ragged():
    _ppo_case(gen.PPO.with_(T=3 * 111, D=200, V=1003, C=100, n_seq=3), eps=0.1, beta=0.2)


def test_ppo_on_policy_matches_grpo_on_gpu():
    # old log-probs equal to the current ones and no KL: the GPU's PPO
    # gradients are its GRPO gradients (ratio within rounding of 1)
    require_gpu()
    wl = gen.PPO.with_(T=4 * 128, D=256, V=4000, C=128, n_seq=4)
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    _, lp, dH_g, dW_g = hd.grpo(d["H"], d["W"], d["y"], d["off"], d["adv"])
    dH_g, dW_g = dH_g.clone(), dW_g.clone()
    _, _, dH_p, dW_p = hd.ppo(d["H"], d["W"], d["y"], d["off"], d["adv"], lp.clone(), None, 0.2, 0.0)
    torch.cuda.synchronize()
    assert rel(np64(dH_p), np64(dH_g)) <= 1e-6 and rel(np64(dW_p), np64(dW_g)) <= 1e-6


def _dpo_case(wl, seed=0, calibrate=True, compact=False, fuse=True, dirty=False, edit=None):
    require_gpu()
    _print_case("dpo", wl=wl.name, T=wl.T, D=wl.D, V=wl.V, C=wl.C, calibrate=calibrate, compact=compact, fuse=fuse,
                dirty=dirty, edit=getattr(edit, "__name__", None))
    inp = gen.make_inputs(wl, seed)
    if edit is not None:
        edit(inp)
    p1 = O.dpo_logp(inp.H, inp.W, inp.labels, inp.offsets)
    if calibrate:
        # reference log-probs set so that beta*Delta lies in [-2, 2] (sigmoid not saturated)
        P = wl.n_seq // 2
        target = np.linspace(-2.0, 2.0, P) / wl.beta
        ref = p1.seq_logp.copy()
        ref[:P] = p1.seq_logp[:P] - (p1.seq_logp[P:] - ref[P:]) - target
        inp.ref_logp = ref
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype, compact)
    if dirty:
        _dirty(hd, wl)
    loss, seq, dH, dW = hd.dpo(d["H"], d["W"], d["y"], d["off"], d["ref"], wl.beta, fuse=fuse)
    torch.cuda.synchronize()
    ref = O.dpo(inp.H, inp.W, inp.labels, inp.offsets, inp.ref_logp, wl.beta)
    tol = _tol(wl)
    e_seq = rel(np64(seq), ref.seq_logp)
    e_loss = loss_rel(loss.item(), ref.loss, 0.0)
    gH, gW = np64(dH), np64(dW)
    e_dH, e_dW = rel(gH, ref.dH), rel(gW, ref.dW)
    aH, aW = abs_products(inp.H, inp.W, inp.labels, ref)
    r_dH, r_dW = row_check(gH, ref.dH, tol, "dH", aH), row_check(gW, ref.dW, tol, "dW", aW)
    print(f"  seq {e_seq:.2e} loss {e_loss:.2e} dH {e_dH:.2e} dW {e_dW:.2e} "
          f"(worst row dH {r_dH:.2e} dW {r_dW:.2e})", flush=True)
    assert max(e_seq, e_loss, e_dH, e_dW) <= tol


@pytest.mark.parametrize("fuse", [False, True], ids=["row_pass", "fused"])
def test_dpo_bf16_ragged_pass2_variants(fuse):
    # pass 2 with the row pass, and with the gradient written by the logits
    # epilogue from pass 1's per-token log-sum-exp: ragged D, V and chunks
    _dpo_case(gen.DPO.with_(T=4 * 111, D=200, V=1003, C=100, n_seq=4), fuse=fuse)


def test_dpo_fused_pass2_matches_row_pass():
    # the two forms of pass 2 differ only in where the softmax is rounded
    # (fp32 logits in the epilogue, bf16 logits in the row pass)
    require_gpu()
    wl = gen.DPO.with_(T=4 * 256, D=512, V=9000, C=256, n_seq=4)
    _print_case("dpo_fused_vs_row_pass", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    d = to_dev(gen.make_inputs(wl, 4))
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    outs = []
    for fuse in (False, True):
        loss, seq, dH, dW = hd.dpo(d["H"], d["W"], d["y"], d["off"], d["ref"], wl.beta, fuse=fuse)
        torch.cuda.synchronize()
        outs.append((loss.clone(), seq.clone(), dH.clone(), dW.clone()))
    (l0, s0, h0, w0), (l1, s1, h1, w1) = outs
    assert torch.equal(l0, l1) and torch.equal(s0, s1)  # pass 1 and the pair factors are unchanged
    assert rel(np64(h1), np64(h0)) <= 1e-2 and rel(np64(w1), np64(w0)) <= 1e-2


def test_dpo_fused_pass2_compacted_matches_row_pass():
    # the same under masked-row compaction, where the epilogue reads the
    # per-token arrays through the row map and stops at the live row count:
    # a scattered mask, chunks of 64 valid rows, the last chunks empty
    require_gpu()
    wl = gen.DPO.with_(T=4 * 200, D=256, V=5003, C=64, n_seq=4, mask="random", mask_frac=0.3)
    _print_case("dpo_fused_vs_row_pass_compacted", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    d = to_dev(gen.make_inputs(wl, 5))
    hd = head(wl.D, wl.V, wl.C, wl.dtype, True)
    outs = []
    for fuse in (False, True):
        loss, seq, dH, dW = hd.dpo(d["H"], d["W"], d["y"], d["off"], d["ref"], wl.beta, fuse=fuse)
        torch.cuda.synchronize()
        outs.append((loss.clone(), seq.clone(), dH.clone(), dW.clone()))
    (l0, s0, h0, w0), (l1, s1, h1, w1) = outs
    assert torch.equal(l0, l1) and torch.equal(s0, s1)
    assert rel(np64(h1), np64(h0)) <= 1e-2 and rel(np64(w1), np64(w0)) <= 1e-2
    ignored = d["y"] < 0
    assert torch.count_nonzero(h1[ignored]) == 0  # dH rows of ignored tokens are zero


def test_dpo_token_lse_ignored_by_f32():
    # fp32 handles run pass 2 through the row pass whether or not pass 1's
    # log-sum-exp is passed: bitwise equal results
    require_gpu()
    wl = gen.DPO.with_(dtype="f32", T=4 * 96, D=128, V=2000, C=64, n_seq=4)
    _print_case("dpo_token_lse_ignored_f32")
    d = to_dev(gen.make_inputs(wl, 2))
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    outs = []
    for fuse in (False, True):
        res = hd.dpo(d["H"], d["W"], d["y"], d["off"], d["ref"], wl.beta, fuse=fuse)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in res])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_dpo_f32_calibrated():
    _dpo_case(gen.DPO.with_(dtype="f32", T=4 * 80, D=128, V=2000, C=64, n_seq=4))


def test_dpo_bf16_calibrated():
    _dpo_case(gen.DPO.with_(T=4 * 256, D=512, V=9000, C=256, n_seq=4))


def test_dpo_bf16_saturated_refs():
    _dpo_case(gen.DPO.with_(T=4 * 256, D=512, V=9000, C=256, n_seq=4), calibrate=False)


# masked-row compaction: the chunk loop over the valid rows only ------------
@pytest.mark.parametrize("shape", [dict(T=600, D=512, V=8000, C=256), dict(T=333, D=200, V=1003, C=112),
                                   dict(T=1100, D=1024, V=20000, C=512)])
def test_bf16_sft_compacted(shape):
    _check_sft(gen.SFT_9K.with_(**shape), compact=True)


def test_bf16_sft_compacted_random_mask():
    # a scattered 20% mask; chunks of 64 valid rows; the last chunks are empty
    _check_sft(gen.SFT_9K.with_(T=700, D=256, V=5003, C=64, mask="random", mask_frac=0.2), compact=True)


def test_grpo_bf16_compacted():
    _grpo_case(gen.GRPO.with_(T=4 * 320, D=512, V=9000, C=256, n_seq=4), compact=True)


def test_ppo_bf16_compacted():
    _ppo_case(gen.PPO.with_(T=3 * 111, D=200, V=1003, C=100, n_seq=3), eps=0.1, beta=0.2, compact=True)


@pytest.mark.parametrize("fuse", [False, True], ids=["row_pass", "fused"])
def test_dpo_bf16_compacted(fuse):
    _dpo_case(gen.DPO.with_(T=4 * 256, D=512, V=9000, C=256, n_seq=4), compact=True, fuse=fuse)


def test_dpo_bf16_compacted_ragged_fused():
    # ragged D, V and live rows per chunk, with the gradient from the epilogue
    _dpo_case(gen.DPO.with_(T=4 * 111, D=200, V=1003, C=100, n_seq=4), compact=True, fuse=True)


def test_compaction_matches_plain_loop_and_accumulates():
    # same call with and without compaction, accumulating into a given dW:
    # equal up to the fp32 summation order; dH rows of ignored tokens are 0
    require_gpu()
    wl = gen.SFT_9K.with_(T=900, D=256, V=6000, C=256, mask="random", mask_frac=0.3)
    inp = gen.make_inputs(wl, 2)
    d = to_dev(inp)
    dW0 = torch.randn(wl.V, wl.D, device="cuda") * 0.01
    outs = []
    for compact in (False, True):
        hd = head(wl.D, wl.V, wl.C, wl.dtype, compact)
        dW = dW0.clone()
        dH = torch.full((wl.T, wl.D), float("nan"), device="cuda")
        loss, dH, dW, nv = hd.sft(d["H"], d["W"], d["y"], dH=dH, dW=dW, accumulate=True)
        torch.cuda.synchronize()
        outs.append((loss.item(), np64(dH), np64(dW), int(nv.item())))
    (l0, h0, w0, n0), (l1, h1, w1, n1) = outs
    assert n0 == n1
    assert abs(l0 - l1) <= 1e-6 * abs(l0)
    assert rel(h1, h0) <= 1e-6 and rel(w1, w0) <= 1e-6
    assert np.all(h1[inp.labels == -100] == 0.0)


def test_compaction_all_ignored():
    require_gpu()
    wl = gen.SFT_9K.with_(T=300, D=256, V=3000, C=128)
    inp = gen.make_inputs(wl, 0)
    inp.labels[:] = -100
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype, True)
    dH = torch.full((wl.T, wl.D), 7.0, device="cuda")
    dW = torch.full((wl.V, wl.D), 7.0, device="cuda")
    loss, dH, dW, nv = hd.sft(d["H"], d["W"], d["y"], dH=dH, dW=dW)
    torch.cuda.synchronize()
    assert int(nv.item()) == 0 and loss.item() == 0.0
    assert float(dH.abs().max()) == 0.0 and float(dW.abs().max()) == 0.0


@pytest.mark.parametrize("compact", [False, True], ids=["plain_loop", "compacted"])
def test_nan_filled_workspace_does_not_leak(compact):
    """The workspace's contents are undefined between calls.  Every byte the
    chunk loop reads must be written by the same call first, or multiply a
    zero that stays exact: with compaction the dW GEMM reads the transposed
    tiles of a chunk's dense rows of H, whose rows past the device-side live
    count are written as zeros, and G reads zero there.  A workspace filled
    with NaN bit patterns before the call must not change any output, and
    outputs that are not accumulated into are overwritten whole."""
    require_gpu()
    wl = gen.SFT_9K.with_(T=700, D=320, V=5000, C=256, mask="random", mask_frac=0.3)
    print(f"[case] nan workspace compact={compact} T={wl.T} D={wl.D} V={wl.V} C={wl.C}", flush=True)
    inp = gen.make_inputs(wl, 4)
    d = to_dev(inp)
    ref = O.sft(inp.H, inp.W, inp.labels)
    hd = head(wl.D, wl.V, wl.C, wl.dtype, compact)
    ws, _ = hd.workspace(wl.T)
    ws.fill_(0xFF)  # 0xFFFF: a bf16 NaN; 0xFFFFFFFF: an fp32 NaN
    # outputs that are not accumulated into are overwritten whole, NaN or not
    dH0 = torch.full((wl.T, wl.D), float("nan"), device="cuda")
    dW0 = torch.full((wl.V, wl.D), float("nan"), device="cuda")
    torch.cuda.synchronize()
    loss, dH, dW, nv = hd.sft(d["H"], d["W"], d["y"], dH=dH0, dW=dW0)
    torch.cuda.synchronize()
    assert int(nv.item()) == ref.scan.n_valid
    assert bool(torch.isfinite(dH).all()) and bool(torch.isfinite(dW).all())
    assert abs(loss.item() - ref.loss) / abs(ref.loss) <= TOL_BF16
    assert rel(np64(dH), ref.dH) <= TOL_BF16 and rel(np64(dW), ref.dW) <= TOL_BF16


@pytest.mark.parametrize("compact", [False, True], ids=["plain_loop", "compacted"])
def test_grpo_nan_filled_workspace(compact):
    _grpo_case(gen.GRPO.with_(T=3 * 300, D=256, V=5000, C=256, n_seq=3), seed=2, compact=compact, dirty=True)


@pytest.mark.parametrize("compact", [False, True], ids=["plain_loop", "compacted"])
@pytest.mark.parametrize("fuse", [True, False], ids=["fused", "row_pass"])
def test_dpo_nan_filled_workspace(fuse, compact):
    _dpo_case(gen.DPO.with_(T=4 * 200, D=256, V=5000, C=192, n_seq=4), seed=3, compact=compact, fuse=fuse,
              dirty=True)

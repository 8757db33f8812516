"""Seeded input generators: determinism, mask structure, bfloat16 rounding."""
import numpy as np
import pytest
import torch

from workloads import gen


def test_same_seed_same_bits():
    a = gen.make_inputs(gen.TINY, seed=3)
    b = gen.make_inputs(gen.TINY, seed=3)
    c = gen.make_inputs(gen.TINY, seed=4)
    assert np.array_equal(a.H, b.H) and np.array_equal(a.W, b.W) and np.array_equal(a.labels, b.labels)
    assert not np.array_equal(a.H, c.H)


def test_block_streams_do_not_depend_on_length():
    # the first block of a long stream equals a short stream of the same tag
    n = gen._BLOCK + 100
    long = gen.normal_f32(1, 99, n)
    short = gen.normal_f32(1, 99, 1000)
    assert np.array_equal(long[:1000], short)


def test_mask_counts_and_positions():
    t = gen.make_labels(gen.TINY, 0)
    assert (t == -100).sum() == 51 and t.min() >= -100 and t.max() < gen.TINY.V
    s = gen.make_labels(gen.SFT_9K.with_(T=9000), 0)
    assert np.all(s[:900] == -100) and np.all(s[900:] >= 0)
    g = gen.GRPO.with_(T=8 * 64)
    y = gen.make_labels(g, 0)
    for i in range(8):
        seg = y[i * 64:(i + 1) * 64]
        assert np.all(seg[:16] == -100) and np.all(seg[16:] >= 0)
    lo = gen.make_labels(gen.LONG, 0)
    assert (lo == -100).sum() == 1638


def test_bf16_rounding_matches_torch():
    x = gen.normal_f32(5, 1, 100_000) * np.float32(37.0)
    # ties: exact halfway points between bf16 neighbours
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.bf16_bits(x), want)
    assert np.array_equal(gen.bf16_to_f32(gen.bf16_bits(x)),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_hidden_rows_are_rms_normalised():
    wl = gen.SFT_9K.with_(T=64, D=256, V=128, dtype="f32")
    h = gen.make_hidden(wl, 0)
    np.testing.assert_allclose(np.sqrt((h.astype(np.float64) ** 2).mean(axis=1)), 1.0, rtol=1e-5)


def test_dpo_reference_and_grpo_advantage():
    d = gen.make_inputs(gen.DPO.with_(T=8 * 64, D=16, V=32), 0)
    assert d.ref_logp.shape == (8,) and d.offsets.tolist() == list(range(0, 8 * 64 + 1, 64))
    # centred near -2 * (response length) = -2 * 48
    assert abs(d.ref_logp.mean() + 96) < 200
    g = gen.make_inputs(gen.GRPO.with_(T=8 * 64, D=16, V=32), 0)
    assert g.adv.shape == (8,) and g.adv.dtype == np.float32


def test_value_distribution_variants():
    # margin: valid rows' label logits rise by about the margin (before bf16
    # rounding of H exactly; after it within a few bf16 ulps of the margin);
    # shift: the last columns of H and W hold 1 and the constant
    base = gen.SFT_9K.with_(T=64, D=128, V=500, C=32)
    b = gen.make_inputs(base, 1)
    m = gen.make_inputs(base.with_(margin=12.0), 1)
    assert np.array_equal(b.W, m.W) and np.array_equal(b.labels, m.labels)
    rows = np.nonzero(b.labels != -100)[0]
    W = gen.bf16_to_f32(b.W).astype(np.float64)
    zb = np.einsum("td,td->t", gen.bf16_to_f32(b.H)[rows].astype(np.float64), W[b.labels[rows]])
    zm = np.einsum("td,td->t", gen.bf16_to_f32(m.H)[rows].astype(np.float64), W[b.labels[rows]])
    assert np.all(np.abs(zm - zb - 12.0) < 0.2)
    ign = np.nonzero(b.labels == -100)[0]
    assert np.array_equal(b.H[ign], m.H[ign])
    s = gen.make_inputs(base.with_(shift=1e4), 1)
    assert np.all(gen.bf16_to_f32(s.H)[:, -1] == 1.0)
    assert np.all(gen.bf16_to_f32(s.W)[:, -1] == np.float32(9984.0))  # 1e4 rounded to bf16
    assert np.array_equal(s.H[:, :-1], b.H[:, :-1]) and np.array_equal(s.W[:, :-1], b.W[:, :-1])

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

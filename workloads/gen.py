"""Seeded synthetic inputs for the chunked LM-head workloads.

This module is shared by the CPU oracle tests and by the GPU path (tests and
bench).  It draws random numbers and rounds them to the input precision; it
holds none of the head's arithmetic (no logits, softmax, loss or gradient).

Workload shapes follow StreamBP's LM-head setting ("StreamBP: Memory-Efficient
Exact Backpropagation for Long Sequence Training of LLMs", LM-head paragraph
and the Qwen3 experiments table): hidden states H[T,D], a head weight W[V,D]
in nn.Linear layout, labels aligned to H rows with -100 meaning "ignored".
V = 151936 and D in {2560, 4096, 5120} stand in for Qwen3-4B/8B/14B heads;
no trained weights or datasets are used.

Every array is produced block by block: block i of a stream uses
PCG64(SeedSequence([seed, stream_tag, i])), so the values do not depend on
the number of threads that generated them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Optional

import numpy as np

IGNORE_INDEX = -100
_BLOCK = 1 << 22  # elements per independent RNG block

# stream tags: one per drawn quantity, so that changing one array's size
# never shifts another array's values
_TAG_H, _TAG_W, _TAG_Y, _TAG_MASK, _TAG_ADV, _TAG_REF = 11, 12, 13, 14, 15, 16
_TAG_OLD, _TAG_TREF = 17, 18


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _rng(seed: int, tag: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, block])))


def normal_f32(seed: int, tag: int, n: int) -> np.ndarray:
    """n draws of N(0,1) as float32."""
    out = np.empty(n, dtype=np.float32)
    nblk = (n + _BLOCK - 1) // _BLOCK

    def fill(b):
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        _rng(seed, tag, b).standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nblk <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def uniform_int(seed: int, tag: int, n: int, high: int) -> np.ndarray:
    """n draws uniform over [0, high) as int32."""
    out = np.empty(n, dtype=np.int32)
    for b in range((n + _BLOCK - 1) // _BLOCK):
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        out[lo:hi] = _rng(seed, tag, b).integers(0, high, hi - lo, dtype=np.int64)
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the
    16-bit patterns as uint16.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).reshape(-1).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)

    def conv(lo):
        s = u[lo:lo + _BLOCK]
        r = (s >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += s
        r >>= np.uint32(16)
        out[lo:lo + _BLOCK] = r

    starts = range(0, u.size, _BLOCK)
    if len(starts) <= 1:
        for lo in starts:
            conv(lo)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(conv, starts))
    return out.reshape(np.shape(x))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One head workload.  ``kind`` is sft, grpo, ppo or dpo.

    For grpo/dpo the T tokens are ``n_seq`` packed sequences of equal length;
    in dpo the first n_seq/2 sequences are the chosen answers and the rest the
    rejected ones (pair i = (i, n_seq/2 + i)).
    """
    name: str
    kind: str
    dtype: str          # "f32" or "bf16": precision of H and W
    T: int
    D: int
    V: int
    C: int
    mask: str           # "random" (mask_frac of positions), "prefix" (first mask_frac), "prompt" (per sequence)
    mask_frac: float
    rms_norm_h: bool = False
    n_seq: int = 1
    beta: float = 0.1
    w_std: float = 0.02
    # value-distribution variants (parity cases, not benchmark workloads):
    # margin > 0 moves every valid row's label logit up by about `margin`
    # (a confident, peaked softmax); shift != 0 sets the last column of H to
    # 1 and the last column of W to `shift`, adding that constant to every
    # logit.
    margin: float = 0.0
    shift: float = 0.0

    @property
    def seq_len(self) -> int:
        return self.T // self.n_seq

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the LM-head benchmark.
TINY = Workload("tiny_sft_f32", "sft", "f32", T=256, D=256, V=4096, C=64,
                mask="random", mask_frac=0.20)
SFT_9K = Workload("sft_9k_bf16", "sft", "bf16", T=9000, D=2560, V=151936, C=1024,
                  mask="prefix", mask_frac=0.10, rms_norm_h=True)
GRPO = Workload("grpo_8x12288_bf16", "grpo", "bf16", T=8 * 12288, D=4096, V=151936, C=2048,
                mask="prompt", mask_frac=0.25, rms_norm_h=True, n_seq=8)
# Off-policy clipped-surrogate head at the GRPO shapes, KL coefficient 0.04.
PPO = Workload("ppo_8x12288_bf16", "ppo", "bf16", T=8 * 12288, D=4096, V=151936, C=2048,
               mask="prompt", mask_frac=0.25, rms_norm_h=True, n_seq=8, beta=0.04)
DPO = Workload("dpo_4pairs_16384_bf16", "dpo", "bf16", T=8 * 16384, D=5120, V=151936, C=2048,
               mask="prompt", mask_frac=0.25, rms_norm_h=True, n_seq=8, beta=0.1)
LONG = Workload("long_sft_32768_bf16", "sft", "bf16", T=32768, D=5120, V=151936, C=1024,
                mask="random", mask_frac=0.05)
ALL = {w.name: w for w in (TINY, SFT_9K, GRPO, PPO, DPO, LONG)}
LONG_CHUNKS = (512, 1024, 2048, 4096, 8192)


@dataclasses.dataclass
class Inputs:
    """Host copies of one workload's inputs.

    H, W are float32 arrays for dtype f32, uint16 bfloat16 bit patterns for
    bf16.  ``offsets`` has n_seq+1 entries.  ``adv`` (grpo) and ``ref_logp``
    (dpo) are per sequence."""
    wl: Workload
    H: np.ndarray
    W: np.ndarray
    labels: np.ndarray
    offsets: np.ndarray
    adv: Optional[np.ndarray] = None
    ref_logp: Optional[np.ndarray] = None
    logp_old: Optional[np.ndarray] = None   # ppo: per-token behaviour log-probs (float32)
    logp_ref: Optional[np.ndarray] = None   # ppo: per-token reference log-probs (float32)

    def H_f32(self) -> np.ndarray:
        return self.H if self.wl.dtype == "f32" else bf16_to_f32(self.H)

    def W_f32(self) -> np.ndarray:
        return self.W if self.wl.dtype == "f32" else bf16_to_f32(self.W)


def _hidden_f32(wl: Workload, seed: int) -> np.ndarray:
    h = normal_f32(seed, _TAG_H, wl.T * wl.D).reshape(wl.T, wl.D)
    if wl.rms_norm_h and wl.T > 0:
        # each row divided by its root-mean-square, in blocks to bound memory
        for lo in range(0, wl.T, 4096):
            blk = h[lo:lo + 4096]
            rms = np.sqrt(np.mean(blk.astype(np.float64) ** 2, axis=1, keepdims=True))
            rms[rms == 0] = 1.0
            blk /= rms.astype(np.float32)
    return h


def _round(wl: Workload, x: np.ndarray) -> np.ndarray:
    return x if wl.dtype == "f32" else bf16_bits(x)


def make_hidden(wl: Workload, seed: int) -> np.ndarray:
    return _round(wl, _hidden_f32(wl, seed))


def make_weight(wl: Workload, seed: int) -> np.ndarray:
    w = normal_f32(seed, _TAG_W, wl.V * wl.D).reshape(wl.V, wl.D)
    w *= np.float32(wl.w_std)
    if wl.shift:
        w[:, -1] = np.float32(wl.shift)
    return _round(wl, w)


def _peaked_hidden(wl: Workload, seed: int, W: np.ndarray, labels: np.ndarray) -> np.ndarray:
    """Hidden states whose valid rows point towards their label's weight row:
    h_t + margin * w_y / |w_y|^2 (w_y as stored), so the label logit rises by
    `margin` before h is rounded.  Only the input's value distribution
    changes."""
    h = _hidden_f32(wl, seed)
    Wf = W if wl.dtype == "f32" else bf16_to_f32(W)
    rows = np.nonzero((labels >= 0) & (labels < wl.V))[0]
    wy = Wf[labels[rows]].astype(np.float64)
    if wl.shift:
        wy[:, -1] = 0.0  # keep the constant column of H at 1
    nrm = np.maximum(np.sum(wy * wy, axis=1, keepdims=True), 1e-30)
    h[rows] += (wl.margin * wy / nrm).astype(np.float32)
    return h


def make_labels(wl: Workload, seed: int) -> np.ndarray:
    y = uniform_int(seed, _TAG_Y, wl.T, wl.V)
    if wl.mask == "random":
        k = int(round(wl.mask_frac * wl.T))
        pos = _rng(seed, _TAG_MASK, 0).permutation(wl.T)[:k]
        y[pos] = IGNORE_INDEX
    elif wl.mask == "prefix":
        y[: int(round(wl.mask_frac * wl.T))] = IGNORE_INDEX
    elif wl.mask == "prompt":
        L = wl.seq_len
        p = int(round(wl.mask_frac * L))
        for s in range(wl.n_seq):
            y[s * L: s * L + p] = IGNORE_INDEX
    elif wl.mask != "none":
        raise ValueError(wl.mask)
    return y


def make_offsets(wl: Workload) -> np.ndarray:
    assert wl.T % wl.n_seq == 0
    return (np.arange(wl.n_seq + 1, dtype=np.int64) * wl.seq_len).astype(np.int32)


def make_inputs(wl: Workload, seed: int = 0) -> Inputs:
    W = make_weight(wl, seed)
    y = make_labels(wl, seed)
    h = _peaked_hidden(wl, seed, W, y) if wl.margin else _hidden_f32(wl, seed)
    if wl.shift:
        h[:, -1] = 1.0
    inp = Inputs(wl, _round(wl, h), W, y, make_offsets(wl))
    if wl.kind in ("grpo", "ppo"):
        inp.adv = normal_f32(seed, _TAG_ADV, wl.n_seq).astype(np.float32)
    if wl.kind == "ppo":
        # per-token log-probs of the sampling and reference policies: normal
        # around the mean label log-prob of a V-way head with logit variance
        # about 1 (-ln V - 1/2), standard deviation 1
        centre = np.float32(-np.log(wl.V) - 0.5)
        inp.logp_old = normal_f32(seed, _TAG_OLD, wl.T) + centre
        inp.logp_ref = normal_f32(seed, _TAG_TREF, wl.T) + centre
    if wl.kind == "dpo":
        t_resp = wl.seq_len - int(round(wl.mask_frac * wl.seq_len))
        inp.ref_logp = (-2.0 * t_resp + 50.0 * normal_f32(seed, _TAG_REF, wl.n_seq)
                        .astype(np.float64))
    return inp

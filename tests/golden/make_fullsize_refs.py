"""Write the oracle's per-token log-sum-exp for full-size workloads.

The full-size GPU tests compare sampled outputs (loss, DPO sequence sums,
sampled dH rows and dW vocabulary rows) with the oracle.  Those need every
valid token's log-sum-exp over the whole vocabulary (dW_v sums over all
tokens), which takes the fp64 oracle minutes at these sizes; this script
computes it once, with the oracle alone, on the same seeded inputs the tests
regenerate, and stores it beside a hash of those inputs.

    python tests/golden/make_fullsize_refs.py [name ...]

Output: tests/golden/fullsize_lse_<name>.npz with
  lse      float32 [n_valid]  oracle log-sum-exp of the valid rows, in row order
           (the fp64 value rounded to fp32: at most 5e-7 off for |lse| < 16)
  sha256   hash of the inputs' bytes (H, W, labels, offsets)
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import streambp_oracle as O  # noqa: E402
from workloads import gen  # noqa: E402

# the long-context workload at a reduced length that spans two chunks and a
# ragged tail at the largest chunk of its sweep (8192)
LONG_REDUCED = gen.LONG.with_(name="long_sft_16684_bf16", T=2 * 8192 + 300)

WORKLOADS = {
    "grpo_8x12288_bf16": (gen.GRPO, 0),
    "dpo_4pairs_16384_bf16": (gen.DPO, 0),
    "long_sft_16684_bf16": (LONG_REDUCED, 0),
}


def inputs_sha256(inp) -> str:
    h = hashlib.sha256()
    for a in (inp.H, inp.W, inp.labels, inp.offsets):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def path(name: str) -> str:
    return os.path.join(HERE, f"fullsize_lse_{name}.npz")


def main(names):
    for name in names:
        wl, seed = WORKLOADS[name]
        t0 = time.time()
        inp = gen.make_inputs(wl, seed)
        valid = np.nonzero((inp.labels >= 0) & (inp.labels < wl.V))[0]
        print(f"{name}: {valid.size} valid rows of {wl.T}, D={wl.D}, V={wl.V}", flush=True)
        lse = O.all_lse(inp.H[valid], inp.W, row_block=512)
        np.savez(path(name), lse=lse.astype(np.float32), sha256=np.array(inputs_sha256(inp)))
        print(f"  wrote {path(name)} in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or list(WORKLOADS))

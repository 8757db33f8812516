"""The stored oracle values of the full-size GPU tests
(tests/golden/fullsize_lse_*.npz, written by tests/golden/make_fullsize_refs.py)
belong to the inputs the tests regenerate and agree with the oracle: the
input hash matches, and the stored log-sum-exp of sampled valid rows equals
the oracle's, recomputed here, to the fp32 rounding of the stored values."""
import importlib.util
import os

import numpy as np
import pytest

from oracle import streambp_oracle as O
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
spec = importlib.util.spec_from_file_location("make_fullsize_refs", os.path.join(GOLDEN, "make_fullsize_refs.py"))
refs = importlib.util.module_from_spec(spec)
spec.loader.exec_module(refs)


@pytest.mark.parametrize("name", sorted(refs.WORKLOADS))
def test_stored_lse_matches_the_oracle(name):
    wl, seed = refs.WORKLOADS[name]
    inp = gen.make_inputs(wl, seed)
    z = np.load(refs.path(name))
    assert str(z["sha256"]) == refs.inputs_sha256(inp)
    valid = np.nonzero((inp.labels >= 0) & (inp.labels < wl.V))[0]
    assert z["lse"].shape == (valid.size,)
    pick = np.unique(np.concatenate([[0, valid.size - 1], np.random.default_rng(0).integers(0, valid.size, 6)]))
    lse, _ = O.rows_lse_logp(inp.H, inp.W, inp.labels, valid[pick])
    np.testing.assert_allclose(z["lse"][pick].astype(np.float64), lse, rtol=0, atol=1e-6)

"""GPU: the sustained-MFMA probe (a measurement aid beside the head) launches
on the caller's stream, reports the flops of its launch and leaves no error
behind; its rate is bounded by the data-sheet peak."""
import ctypes

import pytest
import torch

from loss_head_amd import _capi
from tests.gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu

PEAK_BF16_TFLOPS = 2516.6


@pytest.mark.parametrize("changing", [0, 1])
def test_mfma_probe_runs_and_counts_flops(changing):
    require_gpu()
    print(f"[case] mfma probe changing={changing}", flush=True)
    lib = _capi.load()
    st = torch.cuda.current_stream()
    blocks, iters = 512, 400
    flops = ctypes.c_double(0.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    rc = lib.streambp_head_mfma_probe(blocks, iters, changing, ctypes.byref(flops), ctypes.c_void_p(st.cuda_stream))
    e1.record(st)
    e1.synchronize()
    assert rc == _capi.OK
    assert flops.value == blocks * 4 * iters * 8 * 2 * 32 * 32 * 16
    tflops = flops.value / (e0.elapsed_time(e1) * 1e-3) / 1e12
    assert 0 < tflops <= PEAK_BF16_TFLOPS * 1.02
    # the stream is usable afterwards
    x = torch.ones(1024, device="cuda")
    assert float(x.sum().item()) == 1024.0

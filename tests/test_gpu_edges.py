"""GPU edge cases: empty and fully ignored inputs, bad labels and offsets,
accumulation, chunk-size invariance, run-to-run determinism, HIP graph
capture of a call, two handles on two streams, and the per-kernel timer."""
import numpy as np
import pytest
import torch

from oracle import streambp_oracle as O
from tests.gpu_helpers import TOL_BF16, TOL_F32, head, np64, rel, require_gpu, to_dev
from workloads import gen

pytestmark = pytest.mark.gpu

SMALL_BF16 = gen.SFT_9K.with_(T=300, D=256, V=3000, C=128)
SMALL_F32 = gen.TINY.with_(T=100, D=64, V=500, C=32)


def _case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


@pytest.mark.parametrize("wl", [SMALL_F32, SMALL_BF16], ids=["f32", "bf16"])
def test_empty_input(wl):
    require_gpu()
    _case("empty", dtype=wl.dtype)
    inp = gen.make_inputs(wl.with_(T=0), 0)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    dW = torch.full((wl.V, wl.D), 7.0, device="cuda")
    loss, dH, dW2, nv = hd.sft(d["H"], d["W"], d["y"], dW=dW)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and nv.item() == 0 and dH.shape == (0, wl.D)
    assert torch.all(dW2 == 0)
    dW.fill_(7.0)
    hd.sft(d["H"], d["W"], d["y"], dW=dW, accumulate=True)
    assert torch.all(dW == 7.0)


@pytest.mark.parametrize("wl", [SMALL_F32, SMALL_BF16], ids=["f32", "bf16"])
def test_all_ignored(wl):
    require_gpu()
    _case("all_ignored", dtype=wl.dtype)
    inp = gen.make_inputs(wl, 0)
    inp.labels[:] = -100
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    loss, dH, dW, nv = hd.sft(d["H"], d["W"], d["y"])
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and nv.item() == 0
    assert torch.all(dH == 0) and torch.all(dW == 0)


@pytest.mark.parametrize("wl", [SMALL_F32, SMALL_BF16], ids=["f32", "bf16"])
def test_out_of_range_labels_flag_status_and_are_ignored(wl):
    require_gpu()
    _case("label_range", dtype=wl.dtype)
    inp = gen.make_inputs(wl, 1)
    bad = inp.labels.copy()
    bad[[3, 50, 99]] = [wl.V, -5, 2 ** 31 - 1]
    fixed = bad.copy()
    fixed[[3, 50, 99]] = -100
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    d = to_dev(inp)
    yb = torch.from_numpy(bad.astype(np.int32)).cuda()
    yf = torch.from_numpy(fixed.astype(np.int32)).cuda()
    with pytest.raises(Exception) as ei:
        hd.sft(d["H"], d["W"], yb)
    assert getattr(ei.value, "code", None) == 5
    lb, dHb, dWb, nvb = hd.sft(d["H"], d["W"], yb, check=False)
    torch.cuda.synchronize()
    assert int(hd.status.item()) == 5
    lf, dHf, dWf, nvf = hd.sft(d["H"], d["W"], yf)
    assert int(hd.status.item()) == 0
    assert nvb.item() == nvf.item() == int((fixed != -100).sum())
    assert lb.item() == lf.item() and torch.equal(dHb, dHf) and torch.equal(dWb, dWf)
    ref = O.sft(inp.H, inp.W, bad, strict=False)
    assert ref.scan.status == int(hd.status.item()) or ref.scan.status == 5


def test_bad_offsets_flag_status_and_zero_weights():
    require_gpu()
    wl = gen.GRPO.with_(T=4 * 64, D=256, V=3000, C=128, n_seq=4)
    _case("bad_offsets")
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    for off in ([0, 64, 32, 192, 256], [0, 64, 128, 192, 255], [1, 64, 128, 192, 256]):
        o = torch.tensor(off, dtype=torch.int32, device="cuda")
        loss, logp, dH, dW = hd.grpo(d["H"], d["W"], d["y"], o, d["adv"], check=False)
        torch.cuda.synchronize()
        assert int(hd.status.item()) == 1
        assert loss.item() == 0.0 and torch.all(dH == 0) and torch.all(dW == 0)


@pytest.mark.parametrize("wl", [SMALL_F32, SMALL_BF16], ids=["f32", "bf16"])
def test_accumulate_adds_to_dW(wl):
    require_gpu()
    _case("accumulate", dtype=wl.dtype)
    inp = gen.make_inputs(wl, 2)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    _, _, dW1, _ = hd.sft(d["H"], d["W"], d["y"])
    g = torch.Generator(device="cuda").manual_seed(11)
    base = torch.randn(wl.V, wl.D, device="cuda", generator=g)
    acc = base.clone()
    hd.sft(d["H"], d["W"], d["y"], dW=acc, accumulate=True)
    torch.cuda.synchronize()
    # each chunk's contribution is added to the running fp32 sum, so acc differs
    # from base + dW1 by a few fp32 roundings of |base| + |dW1| per chunk; the
    # bf16 path adds the old value partway through the chunk's products (the
    # streamed update), so a chunk may round twice
    n_chunks = -(-wl.T // wl.C)
    bound = 4 * (n_chunks + 1) * torch.finfo(torch.float32).eps * (base.abs() + dW1.abs())
    assert torch.all((acc - (base + dW1)).abs() <= bound)


@pytest.mark.parametrize("T,D,V,C", [(300, 256, 3000, 128), (333, 200, 1003, 112), (2100, 2560, 151936, 1024)],
                         ids=["small", "ragged_D200_V1003", "vocab_151936"])
def test_ignored_rows_leave_dW_bitwise(T, D, V, C):
    """Every label ignored: G = 0, so an accumulating call must leave every
    element of dW bitwise as it was (adding +0 to an fp32 sum is exact) and a
    write-only call must give exact zeros.  Unlike a norm-based comparison this
    sees a single wrong element anywhere in the V x D store path: at every
    vocabulary tile of the full-size head, and on feature and vocabulary
    edges that cut through a wave's tile (D = 200, V = 1003)."""
    require_gpu()
    _case("ignored_dW_bitwise", T=T, D=D, V=V, C=C)
    g = torch.Generator(device="cuda").manual_seed(17)
    H = torch.randn(T, D, device="cuda", generator=g).to(torch.bfloat16)
    W = (0.02 * torch.randn(V, D, device="cuda", generator=g)).to(torch.bfloat16)
    y = torch.full((T,), -100, dtype=torch.int32, device="cuda")
    hd = head(D, V, C, "bf16")
    base = torch.randn(V, D, device="cuda", generator=g)
    acc = base.clone()
    _, _, _, nv = hd.sft(H, W, y, dW=acc, accumulate=True)
    torch.cuda.synchronize()
    assert nv.item() == 0
    assert torch.equal(acc, base), int((acc != base).sum())
    _, dH, dW, _ = hd.sft(H, W, y)
    torch.cuda.synchronize()
    assert torch.all(dH == 0)
    assert torch.all(dW == 0), int((dW != 0).sum())


@pytest.mark.parametrize("wl", [SMALL_F32, SMALL_BF16], ids=["f32", "bf16"])
def test_bitwise_deterministic(wl):
    require_gpu()
    _case("determinism", dtype=wl.dtype)
    inp = gen.make_inputs(wl, 3)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    a = hd.sft(d["H"], d["W"], d["y"])
    a = [t.clone() for t in a]
    for _ in range(2):
        b = hd.sft(d["H"], d["W"], d["y"])
        for x, y in zip(a, b):
            assert torch.equal(x, y)


@pytest.mark.parametrize("wl", [SMALL_F32, SMALL_BF16], ids=["f32", "bf16"])
def test_chunk_size_invariance(wl):
    require_gpu()
    _case("chunk_invariance", dtype=wl.dtype)
    inp = gen.make_inputs(wl, 4)
    d = to_dev(inp)
    outs = []
    for C in (wl.C, 2 * wl.C, 77, wl.T, wl.T + 9):
        hd = head(wl.D, wl.V, C, wl.dtype)
        outs.append([np64(t) for t in hd.sft(d["H"], d["W"], d["y"])])
    tol = TOL_F32 if wl.dtype == "f32" else 1e-5
    for o in outs[1:]:
        assert abs(o[0][0] - outs[0][0][0]) <= tol * abs(outs[0][0][0])
        assert rel(o[1], outs[0][1]) <= tol
        assert rel(o[2], outs[0][2]) <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_vocab(dtype):
    require_gpu()
    _case("V=1", dtype=dtype)
    wl = (SMALL_F32 if dtype == "f32" else SMALL_BF16).with_(V=1, T=40)
    inp = gen.make_inputs(wl, 0)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    loss, dH, dW, nv = hd.sft(d["H"], d["W"], d["y"])
    torch.cuda.synchronize()
    assert nv.item() == int((inp.labels != -100).sum())
    assert abs(loss.item()) < 1e-6
    # with one vocabulary entry the softmax is exactly 1, so G = 0 in exact
    # arithmetic.  The bf16 path exponentiates the bf16-rounded logit against
    # the fp32 log-sum-exp: |G_t| <= w_t (exp(2^-8 |z_t|) - 1) (then rounded to
    # bf16), which bounds dH and dW.
    H = O.widen(inp.H)
    W = O.widen(inp.W)
    z = H @ W[0]
    valid = inp.labels != -100
    w = valid / max(1, valid.sum())
    slack = 0.0 if dtype == "f32" else 2.0 ** -8
    g = w * (np.exp(slack * np.abs(z)) - 1.0) * (1 + 2.0 ** -8) + 1e-12
    assert np.all(np.abs(np64(dH)) <= np.outer(g, np.abs(W[0])) * 1.01 + 1e-9)
    assert np.all(np.abs(np64(dW))[0] <= (g[:, None] * np.abs(H)).sum(axis=0) * 1.01 + 1e-9)


@pytest.mark.parametrize("wl,tiled", [(SMALL_BF16, False), (SMALL_BF16, True), (SMALL_F32, False)],
                         ids=["bf16", "bf16_tiled", "f32"])
def test_hip_graph_capture_and_replay(wl, tiled):
    # The call enqueues kernels only (no allocation, no memset), so it can be
    # captured into a HIP graph.  Replays, with unrelated eager work and
    # synchronisations between them, must give the eager result bit for bit.
    require_gpu()
    _case("graph", dtype=wl.dtype, T=wl.T, tiled=tiled)
    inp = gen.make_inputs(wl, 3)
    d = to_dev(inp)
    hd = head(wl.D, wl.V, wl.C, wl.dtype, tiled=tiled)
    dH = torch.empty(wl.T, wl.D, device="cuda")
    dW = torch.empty(wl.V, wl.D, device="cuda")
    loss_e, dH_e, dW_e, _ = hd.sft(d["H"], d["W"], d["y"], dH=dH, dW=dW)
    loss_e, dH_e, dW_e = loss_e.clone(), dH_e.clone(), dW_e.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            out = hd.sft(d["H"], d["W"], d["y"], dH=dH, dW=dW, check=False)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        dH.fill_(float("nan"))
        dW.fill_(float("nan"))
        junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[0], loss_e), rep
        assert torch.equal(dH, dH_e) and torch.equal(dW, dW_e), rep
        del junk


def test_two_handles_on_two_streams_at_once():
    """Two handles, each with its own workspace, called on two streams whose
    work may overlap: the library keeps no device state between calls, so
    each result equals the same call run alone, bit for bit."""
    require_gpu()
    wls = [gen.SFT_9K.with_(T=900, D=256, V=6000, C=256), gen.SFT_9K.with_(T=700, D=256, V=6000, C=128)]
    print("[case] two handles on two streams", flush=True)
    ins = [to_dev(gen.make_inputs(wl, 7 + i)) for i, wl in enumerate(wls)]
    alone = []
    for wl, d in zip(wls, ins):
        out = head(wl.D, wl.V, wl.C, wl.dtype).sft(d["H"], d["W"], d["y"])
        torch.cuda.synchronize()
        alone.append([t.clone() for t in out])
    hds = [head(wl.D, wl.V, wl.C, wl.dtype) for wl in wls]
    for hd, wl in zip(hds, wls):
        hd.workspace(wl.T)  # allocated before the streams fork
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [None, None]
    for rep in range(3):
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                outs[i] = hds[i].sft(ins[i]["H"], ins[i]["W"], ins[i]["y"], check=False)
    torch.cuda.synchronize()
    for i in (0, 1):
        assert int(hds[i].status.item()) == 0
        for a, b in zip(alone[i], outs[i]):
            assert torch.equal(a, b)


def test_kernel_timer_counts_launches_and_leaves_results_alone():
    """The per-kernel event timer: every launch of a call is counted under its
    kind with a positive time, the results stay bitwise those of an untimed
    call, and turning the timer off resets the totals."""
    require_gpu()
    wl = SMALL_BF16
    _case("timer", T=wl.T, D=wl.D, V=wl.V, C=wl.C)
    d = to_dev(gen.make_inputs(wl, 4))
    hd = head(wl.D, wl.V, wl.C, wl.dtype)
    ref = [t.clone() for t in hd.sft(d["H"], d["W"], d["y"])]
    torch.cuda.synchronize()
    hd.set_timing(True)
    calls = 2
    for _ in range(calls):
        out = [t.clone() for t in hd.sft(d["H"], d["W"], d["y"])]
        torch.cuda.synchronize()
        for a, b in zip(ref, out):
            assert torch.equal(a, b)
    kt = hd.kernel_times()
    n_chunks = -(-wl.T // wl.C)
    for k in ("tile_h", "tile_ht", "logits_lse", "rows_lse_dlogits", "dh_gemm", "dw_gemm"):
        assert kt[k][1] == calls * n_chunks and kt[k][0] > 0, (k, kt[k])
    for k in ("scan_labels", "loss_sum"):
        assert kt[k][1] == calls and kt[k][0] > 0, (k, kt[k])
    assert kt["dh_splitk_reduce"][1] in (0, calls * n_chunks)
    for k in ("dpo_pairs", "seq_sums", "gather_rows", "zero_dead_rows", "tile_w"):
        assert kt[k] == (0.0, 0), (k, kt[k])
    hd.set_timing(False)
    assert all(v == (0.0, 0) for v in hd.kernel_times().values())

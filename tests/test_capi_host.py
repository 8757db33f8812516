"""The C interface without a GPU: the library loads, exports exactly what the
header declares, and rejects bad arguments on the host before any device work."""
import ctypes
import os
import re
import subprocess

import pytest

from loss_head_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "streambp_head.h")


def header_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"STREAMBP_API\s+[\w\s\*]+?\b(streambp_head_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return _capi.load()


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("streambp_head_create", "streambp_head_sft", "streambp_head_grpo", "streambp_head_ppo",
              "streambp_head_dpo_logp", "streambp_head_dpo_bwd"):
        assert n in names
    assert set(names) == set(_capi.SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol(lib):
    for n in header_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _capi.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.split() and l.split()[-1].startswith("streambp")}
    assert exported == set(header_functions())


def test_library_is_built_for_gfx950():
    out = subprocess.run(["strings", _capi.LIB_PATH], capture_output=True, text=True).stdout
    assert "gfx950" in out


def test_version(lib):
    assert lib.streambp_head_version().startswith(b"streambp_head")


def _handle(lib, D=256, V=4096, C=64, dtype=_capi.BF16):
    h = ctypes.c_void_p()
    rc = lib.streambp_head_create(ctypes.byref(h), D, V, C, dtype, 0)
    return rc, h


def test_create_rejects_bad_shapes(lib):
    assert _handle(lib, D=0)[0] == _capi.ERR_INVALID_ARGUMENT
    assert _handle(lib, V=0)[0] == _capi.ERR_INVALID_ARGUMENT
    assert _handle(lib, C=0)[0] == _capi.ERR_INVALID_ARGUMENT
    assert _handle(lib, D=12)[0] == _capi.ERR_UNSUPPORTED
    assert _handle(lib, dtype=7)[0] == _capi.ERR_INVALID_ARGUMENT
    assert lib.streambp_head_create(None, 8, 8, 8, 0, 0) == _capi.ERR_INVALID_ARGUMENT


@pytest.fixture
def handle(lib):
    rc, h = _handle(lib, D=2560, V=151936, C=1024)
    if rc != 0:
        pytest.skip("handle creation needs the HIP runtime")
    yield h
    lib.streambp_head_destroy(h)


def test_workspace_is_order_chunk_times_vocab(lib, handle):
    ws0 = lib.streambp_head_workspace_bytes(handle, 0, 1)
    ws9k = lib.streambp_head_workspace_bytes(handle, 9000, 1)
    ws1m = lib.streambp_head_workspace_bytes(handle, 1_000_000, 1)
    zbuf = 1024 * 151936 * 2
    assert zbuf <= ws0 < zbuf * 1.5
    # only O(T) vectors grow with T: 20 bytes per token (weight, 1/len, logp,
    # fp64 loss term) plus alignment
    assert ws9k - ws0 <= 20 * 9000 + 5 * 256
    assert ws1m - ws0 <= 20 * 1_000_000 + 5 * 256
    assert lib.streambp_head_workspace_bytes(None, 10, 1) == 0


def _fake(addr=1 << 20):
    return ctypes.c_void_p(addr)


def test_host_argument_checks_need_no_device(lib, handle):
    T = 16
    ws_need = lib.streambp_head_workspace_bytes(handle, T, 1)
    P = _fake()
    args = dict(H=P, W=P, y=P, dH=P, dW=P, loss=P, nv=P, st=P, ws=_fake(1 << 30))

    def sft(**kw):
        a = dict(args, **kw)
        return lib.streambp_head_sft(handle, kw.get("T", T), a["H"], a["W"], a["y"], a["dH"], a["dW"], 0,
                                     a["loss"], a["nv"], a["st"], a["ws"], kw.get("nbytes", ws_need), None)

    assert sft(st=None) == _capi.ERR_INVALID_ARGUMENT
    assert b"status" in lib.streambp_head_last_error(handle)
    assert sft(dW=None) == _capi.ERR_INVALID_ARGUMENT
    assert sft(H=None) == _capi.ERR_INVALID_ARGUMENT
    assert sft(H=_fake((1 << 20) + 4)) == _capi.ERR_INVALID_ARGUMENT
    assert b"aligned" in lib.streambp_head_last_error(handle)
    assert sft(T=-1) == _capi.ERR_INVALID_ARGUMENT
    assert sft(ws=_fake((1 << 30) + 64)) == _capi.ERR_INVALID_ARGUMENT
    assert sft(nbytes=ws_need - 1) == _capi.ERR_WORKSPACE_TOO_SMALL
    assert b"needs" in lib.streambp_head_last_error(handle)

    # GRPO / DPO specific checks
    rc = lib.streambp_head_grpo(handle, T, P, P, P, None, 2, P, None, P, P, 0, P, P, args["ws"], 1 << 40, None)
    assert rc == _capi.ERR_INVALID_ARGUMENT  # NULL offsets
    rc = lib.streambp_head_grpo(handle, T, P, P, P, P, 0, P, None, P, P, 0, P, P, args["ws"], 1 << 40, None)
    assert rc == _capi.ERR_INVALID_ARGUMENT  # n_seq = 0
    rc = lib.streambp_head_dpo_bwd(handle, T, P, P, P, P, 3, P, P, 0.1, None, P, P, 0, P, P, args["ws"], 1 << 40, None)
    assert rc == _capi.ERR_INVALID_ARGUMENT  # odd n_seq
    assert b"even" in lib.streambp_head_last_error(handle)
    rc = lib.streambp_head_dpo_bwd(handle, T, P, P, P, P, 2, P, P, float("nan"), None, P, P, 0, P, P, args["ws"],
                                   1 << 40, None)
    assert rc == _capi.ERR_INVALID_ARGUMENT  # beta not finite
    rc = lib.streambp_head_dpo_logp(handle, T, P, P, P, P, 2, None, None, P, args["ws"], 1 << 40, None)
    assert rc == _capi.ERR_INVALID_ARGUMENT  # NULL seq_logp

    def ppo(adv=P, old=P, ref=P, eps=0.2, beta=0.1):
        return lib.streambp_head_ppo(handle, T, P, P, P, P, 2, adv, old, ref, eps, beta, None, P, P, 0, P, P,
                                     args["ws"], 1 << 40, None)
    assert ppo(adv=None) == _capi.ERR_INVALID_ARGUMENT
    assert ppo(old=None) == _capi.ERR_INVALID_ARGUMENT
    assert b"logp_old" in lib.streambp_head_last_error(handle)
    assert ppo(ref=None) == _capi.ERR_INVALID_ARGUMENT  # KL on without reference log-probs
    assert ppo(eps=-0.1) == _capi.ERR_INVALID_ARGUMENT
    assert ppo(eps=float("inf")) == _capi.ERR_INVALID_ARGUMENT
    assert ppo(beta=float("nan")) == _capi.ERR_INVALID_ARGUMENT


def test_row_compaction_option(lib):
    for dtype, want in ((_capi.F32, _capi.ERR_UNSUPPORTED), (_capi.BF16, 0)):
        h = ctypes.c_void_p()
        rc = lib.streambp_head_create(ctypes.byref(h), 256, 1000, 64, dtype, 0)
        if rc != 0:
            pytest.skip("handle creation needs the HIP runtime")
        try:
            before = lib.streambp_head_workspace_bytes(h, 500, 1)
            assert lib.streambp_head_set_row_compaction(h, 1) == want
            after = lib.streambp_head_workspace_bytes(h, 500, 1)
            if want == 0:
                # row indices (T x 4 B) and one chunk of dense H rows (C x D x 2 B)
                # more, besides the split-K slabs compaction always reduces through
                assert after >= before + 500 * 4 + 64 * 256 * 2
                assert lib.streambp_head_set_row_compaction(h, 0) == 0
                assert lib.streambp_head_workspace_bytes(h, 500, 1) == before
            else:
                assert b"bf16" in lib.streambp_head_last_error(h) and after == before
        finally:
            lib.streambp_head_destroy(h)
    assert lib.streambp_head_set_row_compaction(None, 1) == _capi.ERR_INVALID_ARGUMENT


def test_tiled_logits_option(lib):
    D, V, C = 200, 1003, 64
    for dtype, want in ((_capi.F32, _capi.ERR_UNSUPPORTED), (_capi.BF16, 0)):
        h = ctypes.c_void_p()
        rc = lib.streambp_head_create(ctypes.byref(h), D, V, C, dtype, 0)
        if rc != 0:
            pytest.skip("handle creation needs the HIP runtime")
        try:
            before = lib.streambp_head_workspace_bytes(h, 500, 1)
            assert lib.streambp_head_set_tiled_logits(h, 1) == want
            after = lib.streambp_head_workspace_bytes(h, 500, 1)
            if want == 0:
                # a bf16 copy of W in whole 256 x 32 tiles (a multiple of the
                # 256-byte workspace alignment); the tiled copy of a chunk of H
                # is part of every bf16 workspace
                cols = -(-D // 32) * 32
                w_tiles = -(-V // 256) * 256 * cols * 2
                assert after == before + w_tiles
                assert lib.streambp_head_set_tiled_logits(h, 0) == 0
                assert lib.streambp_head_workspace_bytes(h, 500, 1) == before
            else:
                assert b"bf16" in lib.streambp_head_last_error(h) and after == before
                assert lib.streambp_head_set_tiled_logits(h, 0) == 0  # disabling always succeeds
        finally:
            lib.streambp_head_destroy(h)
    assert lib.streambp_head_set_tiled_logits(None, 1) == _capi.ERR_INVALID_ARGUMENT


def test_mfma_probe_rejects_bad_sizes(lib):
    # checked before anything is launched, so no device is needed
    flops = ctypes.c_double(-1.0)
    for blocks, iters in ((0, 1), (-5, 1), (1 << 31, 1), (4, 0), (4, -1)):
        for changing in (0, 1):
            assert (lib.streambp_head_mfma_probe(blocks, iters, changing, ctypes.byref(flops), None)
                    == _capi.ERR_INVALID_ARGUMENT)
    assert flops.value == -1.0


def test_kernel_timer_interface(lib):
    """The per-kernel event timer's kinds and argument checks (no launches:
    a new handle reports zero totals)."""
    n = lib.streambp_head_kernel_kinds()
    names = [lib.streambp_head_kernel_name(k).decode() for k in range(n)]
    assert n == len(set(names)) and all(names)
    # the kinds the bench's roofline and flop accounting key on
    for k in ("logits_lse", "rows_lse_dlogits", "dh_gemm", "dh_splitk_reduce", "dw_gemm", "scan_labels"):
        assert k in names
    assert lib.streambp_head_kernel_name(n) == b"" and lib.streambp_head_kernel_name(-1) == b""
    assert lib.streambp_head_set_timing(None, 1) == _capi.ERR_INVALID_ARGUMENT
    assert lib.streambp_head_kernel_times(None, 0, None, None) == _capi.ERR_INVALID_ARGUMENT
    rc, h = _handle(lib, D=256, V=1000, C=64)
    if rc != 0:
        pytest.skip("handle creation needs the HIP runtime")
    try:
        ms, cnt = ctypes.c_double(-1.0), ctypes.c_int64(-1)
        for k in (-1, n):
            assert lib.streambp_head_kernel_times(h, k, ctypes.byref(ms), ctypes.byref(cnt)) == _capi.ERR_INVALID_ARGUMENT
        assert ms.value == -1.0 and cnt.value == -1  # untouched on error
        for enable in (1, 0):
            assert lib.streambp_head_set_timing(h, enable) == 0
            for k in range(n):
                assert lib.streambp_head_kernel_times(h, k, ctypes.byref(ms), ctypes.byref(cnt)) == 0
                assert ms.value == 0.0 and cnt.value == 0
        assert lib.streambp_head_kernel_times(h, 0, None, None) == 0  # output pointers may be NULL
    finally:
        lib.streambp_head_destroy(h)


def test_suggest_chunk(lib):
    C = ctypes.c_int64(-1)
    args = (2560, 151936, 9000, 1, _capi.BF16)
    # SFT-9k: C = 1024 needs about 379 MB of workspace, C = 2048 about 700 MB
    assert lib.streambp_head_suggest_chunk(*args, 400 << 20, ctypes.byref(C)) == 0 and C.value == 1024
    assert lib.streambp_head_suggest_chunk(*args, 10 << 30, ctypes.byref(C)) == 0 and C.value == 8192  # <= T
    assert lib.streambp_head_suggest_chunk(*args, 1 << 20, ctypes.byref(C)) == _capi.ERR_WORKSPACE_TOO_SMALL
    assert C.value == 0
    # the suggestion's workspace fits the budget and the next size up does not
    h = ctypes.c_void_p()
    budget = 900 << 20
    assert lib.streambp_head_suggest_chunk(*args, budget, ctypes.byref(C)) == 0
    for c, fits in ((C.value, True), (2 * C.value, False)):
        if lib.streambp_head_create(ctypes.byref(h), 2560, 151936, c, _capi.BF16, 0) != 0:
            pytest.skip("handle creation needs the HIP runtime")
        assert (lib.streambp_head_workspace_bytes(h, 9000, 1) <= budget) == fits
        lib.streambp_head_destroy(h)
    assert lib.streambp_head_suggest_chunk(12, 100, 10, 1, _capi.BF16, 1 << 30, ctypes.byref(C)) == _capi.ERR_UNSUPPORTED
    assert lib.streambp_head_suggest_chunk(*args, 1 << 30, None) == _capi.ERR_INVALID_ARGUMENT


def test_null_handle(lib):
    P = _fake()
    assert lib.streambp_head_sft(None, 1, P, P, P, P, P, 0, P, P, P, P, 1 << 30, None) == _capi.ERR_INVALID_ARGUMENT
    assert lib.streambp_head_destroy(None) == 0
    assert lib.streambp_head_last_error(None) == b"null handle"


def test_sft_noalloc_rejects_calls_beyond_the_static_scratch(lib, handle):
    # a host-side check made before the device is touched
    ws_need = lib.streambp_head_workspace_bytes(handle, 10 ** 7, 1)
    assert ws_need > _capi.STATIC_SCRATCH_BYTES
    P = _fake()
    rc = lib.streambp_head_sft_noalloc(handle, 10 ** 7, P, P, P, P, P, 0, P, P, P, None)
    assert rc == _capi.ERR_WORKSPACE_TOO_SMALL
    assert b"static scratch" in lib.streambp_head_last_error(handle)

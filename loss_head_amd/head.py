"""Python binding of the chunked LM-head library.

Argument marshalling only: tensors are checked, turned into device pointers,
and passed with torch's current HIP stream to the C interface in
include/streambp_head.h.  Every step of the computation runs in the HIP
kernels of libstreambp_head.so; there is no Python or CPU fallback.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _capi


class HeadError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_capi.STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


class DeviceStatusError(HeadError):
    """The device status word of a call was not OK (label out of range or
    malformed sequence offsets).  The outputs are still attached."""

    def __init__(self, code: int, outputs):
        super().__init__(code, "reported by the device")
        self.outputs = outputs


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, dev: torch.device, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != dev:
        raise ValueError(f"{name} must be on {dev}, not {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def suggest_chunk(D: int, V: int, T: int, budget_bytes: int, n_seq: int = 1, dtype: str = "bf16") -> int:
    """Largest chunk size (256 .. 16384, powers of two) whose workspace for T
    rows fits in budget_bytes; raises HeadError when none does."""
    lib = _capi.load()
    out = ctypes.c_int64(0)
    rc = lib.streambp_head_suggest_chunk(int(D), int(V), int(T), int(n_seq),
                                         _capi.BF16 if dtype == "bf16" else _capi.F32, int(budget_bytes),
                                         ctypes.byref(out))
    if rc != 0:
        raise HeadError(rc, f"suggest_chunk(D={D}, V={V}, T={T}, budget={budget_bytes})")
    return int(out.value)


class Head:
    """A head of width D over a vocabulary of V tokens, processed in chunks
    of ``chunk`` rows, with inputs in ``dtype`` ("bf16" or "f32").
    ``compact``: masked-row compaction; ``tiled_logits`` (bf16): the logits
    GEMM reads tiled copies of W and H (V*D bf16 more workspace)."""

    def __init__(self, D: int, V: int, chunk: int, dtype: str = "bf16", device=None, compact: bool = False,
                 tiled_logits: bool = False):
        self.lib = _capi.load()
        if dtype not in ("bf16", "f32"):
            raise ValueError(dtype)
        self.D, self.V, self.chunk, self.dtype = int(D), int(V), int(chunk), dtype
        self.torch_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None else
                                   torch.device(device).index or 0)
        h = ctypes.c_void_p()
        rc = self.lib.streambp_head_create(ctypes.byref(h), self.D, self.V, self.chunk,
                                           _capi.BF16 if dtype == "bf16" else _capi.F32, self.device.index)
        if rc != 0:
            raise HeadError(rc, f"streambp_head_create(D={D}, V={V}, chunk={chunk}, {dtype})")
        self._h = h
        self._ws: Optional[torch.Tensor] = None
        self._lse: Optional[torch.Tensor] = None  # per-token log-sum-exp between the DPO passes
        self.status = torch.zeros(1, dtype=torch.int32, device=self.device)
        if compact:
            self._check(self.lib.streambp_head_set_row_compaction(self._h, 1), "set_row_compaction")
        if tiled_logits:
            self._check(self.lib.streambp_head_set_tiled_logits(self._h, 1), "set_tiled_logits")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self.lib.streambp_head_destroy(h)
            self._h = None

    # -- workspace ----------------------------------------------------------
    def workspace_bytes(self, T: int, n_seq: int = 1) -> int:
        return int(self.lib.streambp_head_workspace_bytes(self._h, int(T), int(n_seq)))

    def workspace(self, T: int, n_seq: int = 1) -> Tuple[torch.Tensor, int]:
        """A device buffer of at least workspace_bytes(T, n_seq), kept between calls."""
        need = self.workspace_bytes(T, n_seq)
        if self._ws is None or self._ws.numel() < need + 256:
            self._ws = None
            self._ws = torch.empty(need + 256, dtype=torch.uint8, device=self.device)
        base = self._ws.data_ptr()
        return self._ws, (base + 255) // 256 * 256 - base

    def _ws_args(self, T, n_seq):
        ws, off = self.workspace(T, n_seq)
        return ws.data_ptr() + off, ws.numel() - off

    def _stream(self):
        return torch.cuda.current_stream(self.device).cuda_stream

    def _check(self, rc: int, what: str):
        if rc != 0:
            raise HeadError(rc, f"{what}: {self.lib.streambp_head_last_error(self._h).decode()}")

    def _check_inputs(self, H, W, labels):
        T = H.shape[0] if H.dim() == 2 else -1
        _need(H, "H", self.torch_dtype, self.device, (T, self.D))
        _need(W, "W", self.torch_dtype, self.device, (self.V, self.D))
        _need(labels, "labels", torch.int32, self.device, (T,))
        return T

    def _device_status(self, check: bool, outputs):
        if not check:
            return
        torch.cuda.current_stream(self.device).synchronize()
        code = int(self.status.item())
        if code != 0:
            raise DeviceStatusError(code, outputs)

    def _grads(self, T, dH, dW, accumulate):
        if dH is None:
            dH = torch.empty((T, self.D), dtype=torch.float32, device=self.device)
        if dW is None:
            if accumulate:
                raise ValueError("accumulate=True needs dW")
            dW = torch.empty((self.V, self.D), dtype=torch.float32, device=self.device)
        _need(dH, "dH", torch.float32, self.device, (T, self.D))
        _need(dW, "dW", torch.float32, self.device, (self.V, self.D))
        return dH, dW

    # -- per-kernel timing ---------------------------------------------------
    def set_timing(self, enable: bool):
        self._check(self.lib.streambp_head_set_timing(self._h, int(bool(enable))), "set_timing")

    def kernel_times(self):
        """{kernel kind: (total ms, launches)} since timing was enabled."""
        out = {}
        for k in range(self.lib.streambp_head_kernel_kinds()):
            ms, n = ctypes.c_double(), ctypes.c_int64()
            self._check(self.lib.streambp_head_kernel_times(self._h, k, ctypes.byref(ms), ctypes.byref(n)),
                        "kernel_times")
            out[self.lib.streambp_head_kernel_name(k).decode()] = (ms.value, n.value)
        return out

    # -- entry points -----------------------------------------------------
    def sft(self, H, W, labels, dH=None, dW=None, accumulate=False, check=True):
        """Returns (loss fp64 [1], dH fp32 [T,D], dW fp32 [V,D], n_valid int64 [1])."""
        T = self._check_inputs(H, W, labels)
        dH, dW = self._grads(T, dH, dW, accumulate)
        loss = torch.empty(1, dtype=torch.float64, device=self.device)
        n_valid = torch.empty(1, dtype=torch.int64, device=self.device)
        ws, nb = self._ws_args(T, 1)
        rc = self.lib.streambp_head_sft(self._h, T, _ptr(H), _ptr(W), _ptr(labels), _ptr(dH), _ptr(dW),
                                        int(bool(accumulate)), _ptr(loss), _ptr(n_valid), _ptr(self.status),
                                        ws, nb, self._stream())
        self._check(rc, "sft")
        out = (loss, dH, dW, n_valid)
        self._device_status(check, out)
        return out

    def sft_noalloc(self, H, W, labels, dH, dW, loss, n_valid, accumulate=False, check=True):
        """SFT through the entry point that allocates nothing: the workspace is
        the library's static device array, and every output is the caller's
        (dH fp32 [T,D], dW fp32 [V,D], loss fp64 [1], n_valid int64 [1])."""
        T = self._check_inputs(H, W, labels)
        _need(dH, "dH", torch.float32, self.device, (T, self.D))
        _need(dW, "dW", torch.float32, self.device, (self.V, self.D))
        _need(loss, "loss", torch.float64, self.device, (1,))
        _need(n_valid, "n_valid", torch.int64, self.device, (1,))
        rc = self.lib.streambp_head_sft_noalloc(self._h, T, _ptr(H), _ptr(W), _ptr(labels), _ptr(dH), _ptr(dW),
                                                int(bool(accumulate)), _ptr(loss), _ptr(n_valid), _ptr(self.status),
                                                self._stream())
        self._check(rc, "sft_noalloc")
        out = (loss, dH, dW, n_valid)
        self._device_status(check, out)
        return out

    def grpo(self, H, W, labels, offsets, adv, dH=None, dW=None, accumulate=False, want_logp=True,
             check=True):
        """Returns (loss fp64 [1], logp fp32 [T] or None, dH, dW)."""
        T = self._check_inputs(H, W, labels)
        S = offsets.numel() - 1
        _need(offsets, "offsets", torch.int32, self.device, (S + 1,))
        _need(adv, "adv", torch.float32, self.device, (S,))
        dH, dW = self._grads(T, dH, dW, accumulate)
        loss = torch.empty(1, dtype=torch.float64, device=self.device)
        logp = torch.empty(T, dtype=torch.float32, device=self.device) if want_logp else None
        ws, nb = self._ws_args(T, S)
        rc = self.lib.streambp_head_grpo(self._h, T, _ptr(H), _ptr(W), _ptr(labels), _ptr(offsets), S,
                                         _ptr(adv), _ptr(logp), _ptr(dH), _ptr(dW), int(bool(accumulate)),
                                         _ptr(loss), _ptr(self.status), ws, nb, self._stream())
        self._check(rc, "grpo")
        out = (loss, logp, dH, dW)
        self._device_status(check, out)
        return out

    def ppo(self, H, W, labels, offsets, adv, logp_old, logp_ref=None, eps=0.2, beta_kl=0.0, dH=None, dW=None,
            accumulate=False, want_logp=True, check=True):
        """Off-policy clipped-surrogate head: returns (loss fp64 [1], logp fp32 [T] or None, dH, dW)."""
        T = self._check_inputs(H, W, labels)
        S = offsets.numel() - 1
        _need(offsets, "offsets", torch.int32, self.device, (S + 1,))
        _need(adv, "adv", torch.float32, self.device, (S,))
        _need(logp_old, "logp_old", torch.float32, self.device, (T,))
        if logp_ref is not None:
            _need(logp_ref, "logp_ref", torch.float32, self.device, (T,))
        dH, dW = self._grads(T, dH, dW, accumulate)
        loss = torch.empty(1, dtype=torch.float64, device=self.device)
        logp = torch.empty(T, dtype=torch.float32, device=self.device) if want_logp else None
        ws, nb = self._ws_args(T, S)
        rc = self.lib.streambp_head_ppo(self._h, T, _ptr(H), _ptr(W), _ptr(labels), _ptr(offsets), S, _ptr(adv),
                                        _ptr(logp_old), _ptr(logp_ref), float(eps), float(beta_kl), _ptr(logp),
                                        _ptr(dH), _ptr(dW), int(bool(accumulate)), _ptr(loss), _ptr(self.status),
                                        ws, nb, self._stream())
        self._check(rc, "ppo")
        out = (loss, logp, dH, dW)
        self._device_status(check, out)
        return out

    def dpo_logp(self, H, W, labels, offsets, token_lse=None, check=True):
        """DPO pass 1: fp64 [n_seq] sums of per-token log-probs.  ``token_lse``
        (optional fp32 [T]) receives each token's log-sum-exp for pass 2."""
        T = self._check_inputs(H, W, labels)
        S = offsets.numel() - 1
        _need(offsets, "offsets", torch.int32, self.device, (S + 1,))
        if token_lse is not None:
            _need(token_lse, "token_lse", torch.float32, self.device, (T,))
        seq = torch.empty(S, dtype=torch.float64, device=self.device)
        ws, nb = self._ws_args(T, S)
        rc = self.lib.streambp_head_dpo_logp(self._h, T, _ptr(H), _ptr(W), _ptr(labels), _ptr(offsets), S,
                                             _ptr(seq), _ptr(token_lse), _ptr(self.status), ws, nb, self._stream())
        self._check(rc, "dpo_logp")
        self._device_status(check, (seq,))
        return seq

    def dpo_bwd(self, H, W, labels, offsets, seq_logp, ref_logp, beta, dH=None, dW=None,
                accumulate=False, token_lse=None, check=True):
        """DPO pass 2: returns (loss fp64 [1], dH, dW).  ``token_lse``: pass 1's
        per-token log-sum-exp (optional; lets the logits GEMM write the gradient)."""
        T = self._check_inputs(H, W, labels)
        S = offsets.numel() - 1
        _need(offsets, "offsets", torch.int32, self.device, (S + 1,))
        _need(seq_logp, "seq_logp", torch.float64, self.device, (S,))
        _need(ref_logp, "ref_logp", torch.float64, self.device, (S,))
        if token_lse is not None:
            _need(token_lse, "token_lse", torch.float32, self.device, (T,))
        dH, dW = self._grads(T, dH, dW, accumulate)
        loss = torch.empty(1, dtype=torch.float64, device=self.device)
        ws, nb = self._ws_args(T, S)
        rc = self.lib.streambp_head_dpo_bwd(self._h, T, _ptr(H), _ptr(W), _ptr(labels), _ptr(offsets), S,
                                            _ptr(seq_logp), _ptr(ref_logp), float(beta), _ptr(token_lse), _ptr(dH), _ptr(dW),
                                            int(bool(accumulate)), _ptr(loss), _ptr(self.status), ws, nb,
                                            self._stream())
        self._check(rc, "dpo_bwd")
        out = (loss, dH, dW)
        self._device_status(check, out)
        return out

    def dpo(self, H, W, labels, offsets, ref_logp, beta, dH=None, dW=None, accumulate=False, check=True,
            fuse=True):
        """Both DPO passes: returns (loss, seq_logp, dH, dW).  With ``fuse`` the
        per-token log-sum-exp of pass 1 is handed to pass 2."""
        lse = None
        if fuse:
            T = H.shape[0]
            if self._lse is None or self._lse.numel() < T:
                self._lse = torch.empty(max(T, 1), dtype=torch.float32, device=self.device)
            lse = self._lse[:T]
        seq = self.dpo_logp(H, W, labels, offsets, token_lse=lse, check=check)
        loss, dH, dW = self.dpo_bwd(H, W, labels, offsets, seq, ref_logp, beta, dH, dW, accumulate,
                                    token_lse=lse, check=check)
        return loss, seq, dH, dW

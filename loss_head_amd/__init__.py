"""MI355X (gfx950) library for StreamBP's sequence-chunked exact LM-head
forward and backward (SFT, on-policy GRPO, off-policy clipped surrogate,
two-pass DPO).

The computation lives in libstreambp_head.so (hand-written HIP) behind the C
interface of include/streambp_head.h; this package only marshals arguments.
"""
from .head import DeviceStatusError, Head, HeadError, suggest_chunk  # noqa: F401

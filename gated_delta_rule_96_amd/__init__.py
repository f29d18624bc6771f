"""MI355X-native Kimi Delta Attention (KDA) forward: chunked prefill, decay
preparation and decode step, served by hand-written gfx950 HIP kernels behind
the C-ABI library libkda.so (see include/kda.h).  The Python layer only
marshals torch tensors into that ABI."""

__all__ = ["synth"]

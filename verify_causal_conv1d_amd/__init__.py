"""libgdn: hand-written HIP (gfx950) kernels for the gated-delta-rule mixer.

The compute path lives in ``libgdn.so`` (C ABI, declared in ``include/libgdn.h``);
:mod:`verify_causal_conv1d_amd.gdn` marshals torch tensors into it.  Importing
this package loads nothing; the library is loaded on first use and a missing
library is an error, never a fallback.
"""
__all__ = ["gdn", "inputs"]

"""MI355X-native (gfx950) fused MXFP4 Mixture-of-Experts forward.

The compute path lives in the HIP library `libmoe_mxfp4.so` behind the C ABI
declared in include/moe_mxfp4.h; `binding` marshals torch tensors into it.
Importing this package does not load the library; `binding` does, and it
raises if the library is missing.
"""
__all__ = ["binding", "inputs"]

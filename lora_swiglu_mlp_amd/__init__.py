"""MI355X-native fused LoRA SwiGLU MLP (forward + backward).

The compute path is the HIP library ``liblora_mlp.so`` (gfx950 kernels behind a
C ABI, declared in ``include/lora_mlp.h``); :mod:`lora_swiglu_mlp_amd.abi` is the
thin ctypes binding over it. Importing this package loads nothing: the library
is opened on first use and a missing build is an error, never a fallback.
"""
__all__ = ["abi", "inputs"]

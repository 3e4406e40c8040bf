"""MI355X-native QLoRA linear layer: NF4 + double quantization codec and the
fused LoRA forward/backward, as hand-written HIP kernels for gfx950 behind a
C ABI (``include/qlora_nf4.h``).

The native library is loaded lazily by :mod:`bit_nf4_quantized_14_amd.capi`;
importing this package does not touch the GPU.
"""

__all__ = ["capi", "workloads"]

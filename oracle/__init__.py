"""Plain CPU oracle for the QLoRA linear layer (NF4 + double quantization +
fused LoRA forward/backward).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, tables or constant generators) and it
imports nothing from ``bit_nf4_quantized_14_amd``.

``oracle.codec_variants`` holds the FP4 / INT4 tables and the other ways of
storing the block constants (none, centered 8-bit); ``oracle.adamw8`` the
8-bit AdamW step on the adapters; ``oracle.dropout`` LoRA dropout with a
Philox4x32-10 mask.

Every function follows the passage of the source pages it cites; where the
pages are silent or garbled, the reading taken is stated in the function's
docstring.
"""

from .nf4_oracle import (  # noqa: F401
    BLOCK,
    GROUP,
    backward_f64,
    bf16_bits_to_f64,
    block_absmax,
    bf16_rne_bits,
    bf16_rne_from_f64,
    double_quantize,
    forward_f64,
    merge_f64,
    nf4_codes,
    nf4_dequantize,
    nf4_levels,
    nf4_quantize,
    nf4_thresholds,
    pack_nibbles,
    qlora_backward,
    qlora_forward,
    unpack_nibbles,
)

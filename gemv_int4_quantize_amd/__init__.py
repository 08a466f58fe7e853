"""MI355X-native weight-only int4 (W4A16) quantize-and-pack and mixed-precision matmul.

The compute lives in ``libw4a16.so`` (hand-written HIP for gfx950, C ABI in
``include/w4a16.h``); this package is its PyTorch binding.
"""

from ._lib import LIB_PATH, W4Desc, W4Error, lib  # noqa: F401
from .ops import (  # noqa: F401
    QuantizedWeight,
    dequantize,
    deserialize,
    load,
    empty_quantized,
    kernel_for,
    meta_shape,
    mm,
    mm_plan,
    mm_split,
    mode_id,
    quantize_fused,
    quantize_pack,
    quantize_pack_into,
    save,
    serialize,
)
from .layer import W4A16Linear, w4a16_linear  # noqa: F401

__version__ = "0.1.0"

"""fp9 routed-expert MoE FFN for MI355X (gfx950).

The compute path lives in libduckmoe.so (HIP kernels behind the C ABI declared
in include/duckmoe.h); this package is its ctypes binding plus the seeded
synthetic-input generator.  Build the library with
`python -m bit_moe_expert_fp9_amd.build`.
"""

from .duckmoe import (  # noqa: F401
    DuckMoeError,
    EXPORTS,
    LIB_PATH,
    Lane,
    Layer,
    LayerStruct,
    Stack,
    decode_fp9,
    expert_ffn,
    fp8_to_fp9_device,
    gemv_fp9,
    lib,
    moe_down,
    moe_gate_up,
    moe_layer,
    moe_layer_noalloc,
    moe_plan,
    moe_prefill,
    moe_stack,
    prefill_plan,
    quantize_fp9,
    quantize_fp9_device,
    read_probe,
    rms_normalize,
    status,
    strerror,
)
from . import synth  # noqa: F401

"""MACaQ online W4A4 linear layer for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libmacaq.so`` (hand-written HIP,
declared in ``include/macaq.h``); ``binding`` marshals torch tensors into it.
``inputs`` holds the seeded synthetic workloads. Submodules are imported on
use so that the input generators load without the HIP library.
"""

_BINDING_NAMES = {
    "MacaqError", "Layer", "Packed", "packed_codes_bytes", "packed_scales_bytes", "empty_grouped_weights", "expert",
    "calibrate", "make_multipliers", "prepare_weights", "prepare_layer", "quant_act",
    "linear", "linear_plain_gemm", "linear_grouped", "linear_workspace_size", "gemm_workspace_size",
    "linear_grouped_workspace_size", "load_library", "library_path",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)

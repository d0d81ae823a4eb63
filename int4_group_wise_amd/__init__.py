"""Group-wise 4-bit weight-only quantization and the W4A16 linear on MI355X.

The compute path is the HIP library ``libw4.so`` (C ABI declared in
``include/w4.h``); ``int4_group_wise_amd.w4`` is its thin Python binding.
Its names are re-exported here on first access, so importing the package (or
its ``workloads`` module) does not load the library.
"""
_EXPORTS = ("SYM", "ASYM", "ASYM_PACKED", "W4Error", "library_path", "load", "quantize_pack",
            "dequantize", "linear", "linear_workspace_bytes", "linear_noalloc", "linear_grad_input",
            "linear_grad_input_workspace_bytes", "lora_merge",
            "lora_merge_workspace_bytes", "PER_CHANNEL", "n_groups", "pack_zeros",
            "unpack_zeros", "q4_0_quantize", "q4_0_dequantize")


def __getattr__(name):
    if name in _EXPORTS:
        from . import w4
        return getattr(w4, name)
    raise AttributeError(name)

"""libcfz for AMD Instinct MI355X: the CompactFusion residual-compression codec
(fused residual + error feedback + group int4/int2 quantization, decode + base
update) and the rank-r subspace-iteration compressor, as hand-written HIP for
gfx950 behind a C ABI (``include/cfz.h``).  ``cfz`` is the ctypes binding.

The binding is imported on first use, not with the package, so that
``diffusion_activation_residual_amd.build`` can compile ``libcfz.so`` in a tree
where it does not exist yet.  Using any name of the binding without a built
library raises ImportError (there is no CPU fallback)."""
import importlib

_BINDING_NAMES = frozenset((
    "CfzError", "Receiver", "Sender", "LowrankSender", "LowrankReceiver", "cfz_abi_version",
    "cfz_codes_bytes", "cfz_compress", "cfz_compress_group", "cfz_decompress",
    "cfz_decompress_group", "cfz_lowrank", "cfz_lowrank_workspace_bytes", "cfz_scales_bytes",
    "cfz_state_create", "cfz_state_destroy", "cfz_state_resume", "cfz_state_steps",
    "cfz_status_string", "cfz_stream_copy"))


def __getattr__(name):
    if name == "cfz":
        return importlib.import_module(".cfz", __name__)
    if name in _BINDING_NAMES:
        return getattr(importlib.import_module(".cfz", __name__), name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")

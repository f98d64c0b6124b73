"""libcfz for AMD Instinct MI355X: the CompactFusion residual-compression codec
(fused residual + error feedback + group int4/int2 quantization, decode + base
update) and the rank-r subspace-iteration compressor, as hand-written HIP for
gfx950 behind a C ABI (``include/cfz.h``).  ``cfz`` is the ctypes binding."""
from . import cfz  # noqa: F401  (raises ImportError if libcfz.so is not built)
from .cfz import (CfzError, Receiver, Sender, cfz_abi_version, cfz_codes_bytes,  # noqa: F401
                  cfz_compress, cfz_compress_group, cfz_decompress,
                  cfz_decompress_group, cfz_lowrank, cfz_lowrank_workspace_bytes,
                  cfz_scales_bytes, cfz_state_create, cfz_state_destroy, cfz_state_resume,
                  cfz_state_steps, cfz_status_string, cfz_stream_copy)

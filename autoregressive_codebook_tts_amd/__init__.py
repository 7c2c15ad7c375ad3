"""MI355X (gfx950) batch-1 codebook-TTS decode: HIP kernels behind a C ABI (libhta.so)."""
from .hta import Hta, HtaError, lib, make_config, undelay, weights_to_device, workspace_bytes  # noqa: F401

"""MI355X (gfx950) FlashDecoder per-frame decode step.

Thin Python binding of libflashdec.so (include/flashdec.h and
include/flashdec_kernels.h).  It only marshals arguments: every step of the
decode runs in the library's HIP kernels.  Device buffers may be given as
integers (device addresses) or as objects with `data_ptr()` (torch tensors);
PyTorch is used by callers for device memory and streams only.

The library must be built first (`python -m transformer_latent_pixel_amd.build`);
importing this package without it raises, there is no fallback path.
"""
from .capi import (  # noqa: F401
    FD_OK, FD_ERR_INVALID_ARG, FD_ERR_UNSUPPORTED, FD_ERR_OOM, FD_ERR_DEVICE,
    FD_ERR_STATE, FD_MAX_WINDOW, KERNEL_KINDS, FdError, Decoder, config_check,
    exported_symbols, fdk_attention, fdk_attention_noalloc, fdk_gemm, fdk_layernorm,
    fdk_mfma_probe, lib_path,
    load_library, status_string,
)

"""MI355X (gfx950) lossless block speculative-decoding step: HIP kernels behind a C ABI
(include/dflash.h), loaded through a thin ctypes binding with the same names."""
from .binding import (DflashError, dflash_accept_resample, dflash_create, dflash_destroy,  # noqa: F401
                      dflash_device_status, dflash_draft_block, dflash_kv_alloc, dflash_kv_free,
                      dflash_kv_pool_bytes, dflash_last_error, dflash_verify_block, dflash_workspace_bytes)

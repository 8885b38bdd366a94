"""MI355X (gfx950) paged-FP8 MLA decode.

The compute path is the HIP library ``libmla_paged.so`` (sources in ``csrc/``,
C ABI in ``include/mla_paged.h``); ``binding`` marshals torch tensors into it.
Importing this package loads nothing: the library is opened on first use and
a missing library is an error, never a fallback.
"""

from .binding import (  # noqa: F401
    MlaError,
    lib_path,
    load_library,
    mla_abi_version,
    mla_append_kv_fp8,
    mla_decode_paged_bf16,
    mla_decode_paged_fp8,
    mla_decode_paged_fp8_noalloc,
    mla_decode_paged_fp8_plan,
    mla_decode_paged_fp8_ragged,
    mla_resolve_pages,
    new_workspace,
    workspace_bytes,
)

"""NVFP4 routed-expert MoE projection on AMD MI355X (gfx950).

A thin ctypes binding over libnvfp4moe.so (C ABI in include/nvfp4moe.h). This module
only marshals arguments: every step of the computation runs in the library's HIP
kernels. torch supplies device memory and the current stream. There is no fallback:
if the library is missing the import of the binding fails loudly.
"""
from .binding import (  # noqa: F401
    ACT,
    DTYPE,
    NVFP4Error,
    PreparedCall,
    PreparedHostCall,
    Proj,
    Q8Proj,
    FORMAT,
    ISA,
    host_isa,
    moe_decode_host,
    Layer,
    dequant,
    lib_path,
    linear,
    load_library,
    moe_decode,
    moe_decode_noalloc,
    moe_prefill,
    quant_rows_i8,
    quant_rows_nvfp4,
    route,
    router_topk,
    router_workspace_size,
    decode_workspace_size,
    prefill_workspace_size,
    route_workspace_size,
    prefill_workspace_region,
    check_decode_workspace,
    DECODE_ERROR_WORD,
    DECODE_SPIN_WORD,
    WS_REGION,
)

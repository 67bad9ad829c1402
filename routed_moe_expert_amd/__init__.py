"""Routed NVFP4 mixture-of-experts FFN for AMD MI355X (gfx950).

The compute lives in libmoe_nvfp4.so (hand-written HIP kernels behind a C ABI, declared in
include/moe_nvfp4.h). This package only marshals arguments to it; see binding.py.
"""
from .binding import (MOE_EINVAL, MOE_ELAUNCH, MOE_ESHAPE, MOE_EWS, MOE_KERNEL_BUCKET,
                      MOE_KERNEL_COMBINE, MOE_KERNEL_DN_DECODE, MOE_KERNEL_DN_PREFILL,
                      MOE_KERNEL_GU_DECODE, MOE_KERNEL_GU_PREFILL, MOE_KERNEL_NONE,
                      MOE_KERNEL_ROUTER, MOE_KERNEL_SCHEDULE, MOE_KPACK_ROWS, MOE_OK,
                      MOE_PATH_AUTO, MOE_PATH_DECODE, MOE_PATH_PREFILL, MOE_STATIC_WS_BYTES,
                      MoeError, bank, lib, moe_auto_path, moe_ffn_nvfp4, moe_ffn_nvfp4_static,
                      moe_ffn_nvfp4_ws, moe_kpack, moe_kpack_bytes, moe_layer_nvfp4,
                      moe_layer_nvfp4_ws, moe_profile_count, moe_profile_kernel, moe_route_bucket,
                      moe_route_bucket_ws, moe_router_topk, moe_status_str, with_kpack)

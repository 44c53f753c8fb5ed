"""MI355X (gfx950) Bailing/Ling mixture-of-experts FFN layer.

Hand-written HIP kernels behind a C ABI (include/moe.h), with this thin torch
binding for device memory and streams.  Build the library with
`python -m mixture_experts_layer_03_amd.build`.
"""
from ._lib import MoEError, lib
from .config import MoEConfig
from .layer import (MoEWeights, dense_mlp, dense_workspace_size, experts, forward, forward_noalloc,
                    host_tensor_to_device, permute, route, weights_from_host)

__all__ = ["MoEConfig", "MoEError", "MoEWeights", "dense_mlp", "dense_workspace_size", "experts", "forward", "forward_noalloc",
           "host_tensor_to_device", "lib",
           "permute", "route", "weights_from_host"]

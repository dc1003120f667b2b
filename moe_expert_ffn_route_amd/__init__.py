"""MI355X (gfx950) fused W8A8 MoE expert block.

The compute lives in libmoe_w8a8.so (hand-written HIP kernels behind the C ABI
of include/moe_w8a8.h); `binding` is its ctypes front end and `synth` draws
seeded synthetic inputs.
"""
from .binding import (Debug, Dims, MoeError, Runner, debug_buffers, dims_of_case, library, make_dims,  # noqa: F401
                      moe_w8a8_forward, moe_w8a8_forward_noalloc, moe_w8a8_pack_weights, moe_w8a8_pack_weights_mx,
                      moe_w8a8_packed_mx_bytes, moe_w8a8_read_probe, moe_w8a8_read_write_probe,
                      moe_w8a8_status_string, moe_w8a8_warm, moe_w8a8_workspace_size,
                      pack_weights, upload, MOE_PACK_GMM1, MOE_PACK_GMM2, MOE_WEIGHT_INT8, MOE_WEIGHT_MXFP4,
                      MOE_WEIGHT_PACKED, MOE_WEIGHT_ROW_MAJOR)

"""MI355X-native mixed-precision MoE layer (PagedWeight's fused MoE hot path).

The compute path is libmpb.so (HIP kernels for gfx950 behind the C ABI in
include/mpb.h); this package holds its build script and a thin ctypes binding.
"""
from . import _lib  # noqa: F401
from ._lib import (MPB_BF16, MPB_F16, moe_fused, moe_fused_workspace_bytes, MPB_PAGE_CPU, MPB_PAGE_GPU, MPB_PAGE_IN_TRANSFER, MpbError, moe_ffn, moe_ffn_workspace_bytes, moe_route,  # noqa: F401
                   moe_route_workspace_bytes, moe_routing_mass,
                   mpb_committed_bytes, mpb_dequant_block, mpb_dequant_block_image, mpb_get_committed_bits, mpb_init,
                   mpb_last_error, mpb_pack_block, mpb_pack_table, mpb_plane_page_bytes,
                   mpb_get_resident_planes, mpb_offload_pages, mpb_page_state, mpb_plan_step, mpb_reload_pages,
                   mpb_set_resident_planes, mpb_table_image_bytes, set_committed_bits)

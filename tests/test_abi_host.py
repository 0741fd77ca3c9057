"""C ABI checks that need no GPU: the library loads, exports every function
include/mpb.h declares, and its host-side validation rejects bad arguments
before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpb.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    from mixed_precision_bit_amd import _lib
    return _lib.lib()


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_route_workspace_bytes", "moe_ffn", "set_committed_bits", "mpb_init", "mpb_pack_block",
              "mpb_committed_bytes", "mpb_dequant_block", "mpb_last_error", "mpb_table_image_bytes",
              "mpb_pack_table", "moe_routing_mass", "mpb_offload_pages", "mpb_reload_pages", "mpb_page_state",
              "mpb_dequant_block_image"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_host_validation_without_device(L):
    from mixed_precision_bit_amd import _lib as M
    # nothing bound yet in this process
    assert L.set_committed_bits(0, 4) == -7
    assert L.mpb_offload_pages(0, 4, None, None, None, None, None) == -7
    assert L.mpb_reload_pages(0, 8, None, None, None, None, None) == -7
    assert L.mpb_page_state(0, 0) == -7
    assert L.mpb_get_resident_planes(0) == -7
    assert L.mpb_committed_bytes(None) == -7
    assert L.moe_ffn_workspace_bytes(16) == 0
    assert L.moe_fused_workspace_bytes(16) == 0
    one_ = ctypes.c_void_p(1)
    assert L.moe_fused(one_, 0, 4, one_, None, one_, one_, one_, one_, one_, one_, one_, 1 << 20, None) == -7
    assert "no layer bound" in M.mpb_last_error()
    d = M.LayerDesc(100, 128, 8, 0, 2)   # H not a multiple of 64
    assert L.mpb_init(ctypes.byref(d), ctypes.c_void_p(1), ctypes.c_void_p(1), None) == -2
    d = M.LayerDesc(256, 128, 8, 0, 9)   # K > E
    assert L.mpb_init(ctypes.byref(d), ctypes.c_void_p(1), ctypes.c_void_p(1), None) == -2
    assert L.mpb_init(None, None, None, None) == -1
    one = ctypes.c_void_p(1)
    assert L.moe_route(one, 2, one, None, 4, 256, 8, 2, one, one, one, 1 << 20, None) == -1   # dtype
    assert L.moe_route(one, 0, one, None, 4, 250, 8, 2, one, one, one, 1 << 20, None) == -2   # H % 64
    assert L.moe_route(one, 0, one, None, 4, 256, 8, 17, one, one, one, 1 << 20, None) == -2  # K
    assert L.moe_route(one, 0, one, None, 0, 256, 8, 2, one, one, one, 0, None) == 0          # T = 0
    r256 = lambda n: (n + 255) // 256 * 256
    # [8][4][8] fp64 parts and [8][8] router-row norms
    assert L.moe_route_workspace_bytes(4, 8) == r256(8 * (4 * 8 + 8) * 8)
    assert L.moe_route_workspace_bytes(4096, 128) == r256((4096 * 128 + 128) * 8)              # matrix-core path
    assert L.moe_route(one, 0, one, None, 4, 256, 8, 2, one, one, one, 255, None) == -5       # workspace
    assert L.moe_route(one, 0, one, None, 4, 256, 8, 2, one, one, None, 1 << 20, None) == -1  # null ws
    assert L.mpb_pack_block(one, 48, 128, (ctypes.c_void_p * 8)(*[1] * 8), None) == -2
    assert L.mpb_dequant_block((ctypes.c_void_p * 8)(*[1] * 8), one, 64, 128, 9, one, None) == -3
    assert L.mpb_plane_page_bytes(64, 128) == 64 * 128 // 8
    # table images: ceil(N/128) tiles of 256 * 2^b bytes
    assert M.mpb_table_image_bytes(0, 2816, 5) == 22 * 256 * 32
    assert M.mpb_table_image_bytes(1, 2048, 8) == 16 * 256 * 256
    assert M.mpb_table_image_bytes(1, 192, 3) == 2 * 256 * 8     # last tile half full
    assert L.mpb_table_image_bytes(0, 192, 3) == -2               # gate_up needs N % 128
    assert L.mpb_table_image_bytes(2, 256, 3) == -1               # kind
    assert L.mpb_table_image_bytes(1, 256, 9) == -3               # b
    assert L.mpb_pack_table(1, None, 256, 4, one, None) == -1
    pg = (ctypes.c_void_p * 8)(*[1] * 8)
    assert L.mpb_dequant_block_image(pg, one, 2, 256, 128, 4, one, None) == -1               # kind
    assert L.mpb_dequant_block_image(pg, one, 0, 192, 128, 4, one, None) == -2               # gate_up: N % 128
    assert L.mpb_dequant_block_image(pg, one, 1, 256, 128, 9, one, None) == -3               # b
    assert L.mpb_dequant_block_image(pg, None, 1, 256, 128, 4, one, None) == -1              # null image
    assert L.moe_routing_mass(one, one, 4, 0, 1, one, None) == -2     # E
    assert L.moe_routing_mass(one, one, 4, 8, 9, one, None) == -2     # K > E
    assert L.moe_routing_mass(one, one, 4, 8, 2, None, None) == -1    # null output


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits with status 2 and a
    message, before touching any device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in (r.stdout + r.stderr)

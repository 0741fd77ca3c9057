"""A MoE layer resident in device memory, driven through libmpb.

PyTorch provides the device allocations and the stream; packing, routing and
the expert FFN all run in the library's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as M

XDTYPE = {"f16": M.MPB_F16, "bf16": M.MPB_BF16}


def _dev(a: np.ndarray, device) -> torch.Tensor:
    """Raw copy of a numpy array to the device (uint32/uint16 kept as int32/int16 bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceLayer:
    """Packed pages, table images and pointer tables of one MoE layer.

    blocks: {i: (planes [8][N][Kd/32] uint32 canonical, luts list of 6
    [N][2**b] uint16)} for every i in 0..2(E+S)-1.
    q_dev: share an existing page table (e.g. several copies of one layer);
    by default a new one is created and bound with mpb_init.
    """

    def __init__(self, H, I, E, S, K, W_r, bias, q, blocks, device="cuda", q_dev=None, bind=True):
        self.H, self.I, self.E, self.S, self.K = H, I, E, S, K
        self.nb = 2 * (E + S)
        self.device = device
        self.W_r = torch.from_numpy(np.ascontiguousarray(W_r, np.float32)).to(device)
        self.bias = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias, np.float32)).to(device)
        self.pages, self.luts = [], []
        plane_ptrs, lut_ptrs = [], []
        for i in range(self.nb):
            planes, luts = blocks[i]
            N, W = planes.shape[1], planes.shape[2]
            Kd = 32 * W
            canon = _dev(planes, device)
            nwords = M.mpb_plane_page_bytes(N, Kd) // 4
            pg = [torch.empty(nwords, dtype=torch.int32, device=device) for _ in range(8)]
            M.mpb_pack_block(canon, N, Kd, pg)
            del canon
            kind = i % 2  # 0: gate_up, 1: down
            imgs = []
            for b in range(3, 9):
                lut = _dev(luts[b - 3], device)
                img = torch.empty(M.mpb_table_image_bytes(kind, N, b) // 2, dtype=torch.int16, device=device)
                M.mpb_pack_table(kind, lut, N, b, img)
                imgs.append(img)
                del lut
            self.pages.append(pg)
            self.luts.append(imgs)
            plane_ptrs += [p.data_ptr() for p in pg]
            lut_ptrs += [t.data_ptr() for t in imgs]
        self.planes_table = torch.tensor(plane_ptrs, dtype=torch.int64, device=device)
        self.luts_table = torch.tensor(lut_ptrs, dtype=torch.int64, device=device)
        if q_dev is None:
            q_dev = torch.empty(self.nb, dtype=torch.int32, device=device)
            if bind:
                M.mpb_init(H, I, E, S, K, q_dev, np.asarray(q, np.int32))
        self.q_dev = q_dev
        self.route_ws = None  # router logits scratch, sized by alloc_route
        torch.cuda.synchronize()

    @classmethod
    def from_synth(cls, layer, **kw):
        blocks = {i: (b.planes, b.luts) for i, b in layer.blocks.items()}
        return cls(layer.H, layer.I, layer.E, layer.S, layer.K, layer.W_r, layer.bias, layer.q, blocks, **kw)

    def weight_bytes(self):
        return sum(p.numel() * 4 for pg in self.pages for p in pg) + \
            sum(t.numel() * 2 for lt in self.luts for t in lt)

    # ---------------------------------------------------------------- calls
    def alloc_route(self, T):
        """Router outputs for T tokens; also sizes the router workspace for T."""
        idx = torch.empty((T, self.K), dtype=torch.int32, device=self.device)
        w = torch.empty((T, self.K), dtype=torch.float32, device=self.device)
        need = max(1, M.moe_route_workspace_bytes(T, self.E))
        if self.route_ws is None or self.route_ws.numel() < need:
            self.route_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return idx, w

    def alloc_ffn(self, T):
        out = torch.empty((T, self.H), dtype=torch.float32, device=self.device)
        ws = torch.empty(max(1, M.moe_ffn_workspace_bytes(T)), dtype=torch.uint8, device=self.device)
        return out, ws

    def alloc_fused(self, T):
        """Output and a zero-filled workspace for moe_fused (its counters must
        start at zero; each call leaves them zero)."""
        out = torch.empty((T, self.H), dtype=torch.float32, device=self.device)
        ws = torch.zeros(max(256, M.moe_fused_workspace_bytes(T)), dtype=torch.uint8, device=self.device)
        return out, ws

    def fused(self, X, xdtype, idx, w, out, ws, stream=None):
        M.moe_fused(X, XDTYPE[xdtype], self.W_r, self.bias, idx, w, self.planes_table, self.luts_table, self.q_dev,
                    out, ws, stream)

    def route(self, X, xdtype, idx, w, stream=None):
        M.moe_route(X, XDTYPE[xdtype], self.W_r, self.bias, self.K, idx, w, self.route_ws, stream)

    def ffn(self, X, xdtype, idx, w, out, ws, stream=None):
        M.moe_ffn(X, XDTYPE[xdtype], idx, w, self.planes_table, self.luts_table, self.q_dev, out, ws, stream)

    def forward(self, X, xdtype, stream=None):
        T = X.shape[0]
        idx, w = self.alloc_route(T)
        out, ws = self.alloc_ffn(T)
        self.route(X, xdtype, idx, w, stream)
        self.ffn(X, xdtype, idx, w, out, ws, stream)
        return idx, w, out

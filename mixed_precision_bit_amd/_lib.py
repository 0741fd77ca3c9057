"""ctypes binding of libmpb (include/mpb.h). Argument marshalling only: every
step of the layer runs in the library's HIP kernels. Functions keep the C
names; tensors are passed as device pointers, streams as raw HIP handles."""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmpb.so")

MPB_F16, MPB_BF16 = 0, 1
ERRORS = {-1: "MPB_E_ARG", -2: "MPB_E_SHAPE", -3: "MPB_E_RANGE", -4: "MPB_E_NOT_RESIDENT",
          -5: "MPB_E_WS", -6: "MPB_E_HIP", -7: "MPB_E_UNINIT", -8: "MPB_E_BUSY"}
MPB_PAGE_GPU, MPB_PAGE_CPU, MPB_PAGE_IN_TRANSFER = 0, 1, 2


class MpbError(RuntimeError):
    def __init__(self, name, code, msg):
        super().__init__(f"{name}: {ERRORS.get(code, code)}: {msg}")
        self.code = code


class LayerDesc(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("S", ctypes.c_int32), ("K", ctypes.c_int32)]


class PlannerParams(ctypes.Structure):
    _fields_ = [("n_buckets", ctypes.c_int32), ("bucket_frac", ctypes.c_double * 8), ("mu", ctypes.c_double * 8),
                ("floor", ctypes.c_int32 * 8), ("n_stages", ctypes.c_int32), ("stage_floor", ctypes.c_int32 * 6),
                ("eps", ctypes.c_double), ("alpha", ctypes.c_double), ("rho_min", ctypes.c_double),
                ("rho_max", ctypes.c_double), ("head_w", ((ctypes.c_double * 3) * 5) * 2),
                ("head_a", (ctypes.c_double * 5) * 2), ("head_c", (ctypes.c_double * 5) * 2),
                ("T_blk", ctypes.c_int64), ("F_blk", ctypes.c_int64), ("P_blk", ctypes.c_int64),
                ("B_kv", ctypes.c_int64)]


class PlanEntry(ctypes.Structure):
    _fields_ = [("i", ctypes.c_int32), ("from_", ctypes.c_int32), ("to", ctypes.c_int32),
                ("delta", ctypes.c_int64), ("damage", ctypes.c_double)]


class PlanSummary(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int64), ("triggered", ctypes.c_int32), ("stage", ctypes.c_int32),
                ("n_plan", ctypes.c_int32), ("pad", ctypes.c_int32), ("released", ctypes.c_int64),
                ("damage", ctypes.c_double), ("stage_released", ctypes.c_int64 * 6),
                ("stage_damage", ctypes.c_double * 6)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libmpb.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixed_precision_bit_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "mpb_init": (_I, [ctypes.POINTER(LayerDesc), _P, _P, _P]),
            "mpb_plane_page_bytes": (ctypes.c_size_t, [_I, _I]),
            "mpb_pack_block": (_I, [_P, _I, _I, _P, _P]),
            "moe_route": (_I, [_P, _I, _P, _P, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
            "moe_route_workspace_bytes": (_SZ, [_I, _I]),
            "moe_routing_mass": (_I, [_P, _P, _I, _I, _I, _P, _P]),
            "moe_ffn_workspace_bytes": (ctypes.c_size_t, [_I]),
            "moe_fused_workspace_bytes": (ctypes.c_size_t, [_I]),
            "moe_fused_counter_bytes": (ctypes.c_size_t, []),
            "moe_fused": (_I, [_P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
            "moe_ffn": (_I, [_P, _I, _I, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
            "moe_ffn_static": (_I, [_P, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
            "set_committed_bits": (_I, [_I, _I]),
            "mpb_committed_bytes": (ctypes.c_int64, [_P]),
            "mpb_get_committed_bits": (_I, [_I]),
            "mpb_dequant_block": (_I, [_P, _P, _I, _I, _I, _P, _P]),
            "mpb_table_image_bytes": (ctypes.c_int64, [_I, _I, _I]),
            "mpb_pack_table": (_I, [_I, _P, _I, _I, _P, _P]),
            "mpb_dequant_block_image": (_I, [_P, _P, _I, _I, _I, _I, _P, _P]),
            "mpb_set_resident_planes": (_I, [_I, _I]),
            "mpb_get_resident_planes": (_I, [_I]),
            "mpb_offload_pages": (_I, [_I, _I, _P, _P, _P, _P, _P]),
            "mpb_reload_pages": (_I, [_I, _I, _P, _P, _P, _P, _P]),
            "mpb_page_state": (_I, [_I, _I]),
            "mpb_plan_step": (_I, [ctypes.POINTER(LayerDesc), _P, _P, _P, _P, _P, ctypes.POINTER(PlannerParams),
                                   _P, ctypes.POINTER(PlanEntry), ctypes.POINTER(PlanSummary)]),
            "mpb_last_error": (ctypes.c_char_p, []),
            "mpb_set_kernel_events": (_I, [_P, _I]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _check(name, rc):
    if rc < 0:
        raise MpbError(name, rc, lib().mpb_last_error().decode())
    return rc


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _host_ptrs(ptrs):
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    return arr


def mpb_last_error() -> str:
    return lib().mpb_last_error().decode()


def mpb_init(H, I, E, S, K, q_dev: torch.Tensor, q_init, stream=None):
    import numpy as np
    q_init = np.ascontiguousarray(q_init, dtype=np.int32)
    d = LayerDesc(H, I, E, S, K)
    return _check("mpb_init", lib().mpb_init(ctypes.byref(d), _ptr(q_dev),
                                             q_init.ctypes.data_as(ctypes.c_void_p), _stream(stream)))


def mpb_plane_page_bytes(N, Kd) -> int:
    return lib().mpb_plane_page_bytes(N, Kd)


def mpb_pack_block(canon: torch.Tensor, N, Kd, pages, stream=None):
    arr = _host_ptrs([p.data_ptr() for p in pages])
    return _check("mpb_pack_block", lib().mpb_pack_block(_ptr(canon), N, Kd, arr, _stream(stream)))


def moe_route_workspace_bytes(T, E) -> int:
    return lib().moe_route_workspace_bytes(T, E)


def moe_route(X, x_dtype, W_router, bias, K, topk_idx, topk_w, ws, stream=None):
    T, H = X.shape
    E = W_router.shape[0]
    nbytes = ws.numel() * ws.element_size()
    return _check("moe_route", lib().moe_route(_ptr(X), x_dtype, _ptr(W_router), _ptr(bias), T, H, E, K,
                                               _ptr(topk_idx), _ptr(topk_w), _ptr(ws), nbytes, _stream(stream)))


def moe_routing_mass(topk_idx, topk_w, E, mass, stream=None):
    T, K = topk_idx.shape
    return _check("moe_routing_mass", lib().moe_routing_mass(_ptr(topk_idx), _ptr(topk_w), T, E, K, _ptr(mass),
                                                             _stream(stream)))


def moe_ffn_workspace_bytes(T) -> int:
    return lib().moe_ffn_workspace_bytes(T)


def moe_ffn(X, x_dtype, topk_idx, topk_w, planes_table, luts_table, q, out, ws, stream=None):
    T = X.shape[0]
    nbytes = ws.numel() * ws.element_size()
    return _check("moe_ffn", lib().moe_ffn(_ptr(X), x_dtype, T, _ptr(topk_idx), _ptr(topk_w),
                                           _ptr(planes_table), _ptr(luts_table), _ptr(q), _ptr(out),
                                           _ptr(ws), nbytes, _stream(stream)))


def moe_ffn_static(X, x_dtype, topk_idx, topk_w, planes_table, luts_table, q, out, stream=None):
    T = X.shape[0]
    return _check("moe_ffn_static", lib().moe_ffn_static(_ptr(X), x_dtype, T, _ptr(topk_idx), _ptr(topk_w),
                                                         _ptr(planes_table), _ptr(luts_table), _ptr(q), _ptr(out),
                                                         _stream(stream)))


def moe_fused_counter_bytes() -> int:
    return lib().moe_fused_counter_bytes()


def moe_fused_workspace_bytes(T) -> int:
    return lib().moe_fused_workspace_bytes(T)


def moe_fused(X, x_dtype, W_router, bias, topk_idx, topk_w, planes_table, luts_table, q, out, ws, stream=None):
    T = X.shape[0]
    nbytes = ws.numel() * ws.element_size()
    return _check("moe_fused", lib().moe_fused(_ptr(X), x_dtype, T, _ptr(W_router), _ptr(bias), _ptr(topk_idx),
                                               _ptr(topk_w), _ptr(planes_table), _ptr(luts_table), _ptr(q),
                                               _ptr(out), _ptr(ws), nbytes, _stream(stream)))


def set_committed_bits(i, b):
    return _check("set_committed_bits", lib().set_committed_bits(i, b))


def mpb_committed_bytes(touched=None) -> int:
    import numpy as np
    if touched is None:
        return _check("mpb_committed_bytes", lib().mpb_committed_bytes(None))
    t = np.ascontiguousarray(touched, dtype=np.uint8)
    return _check("mpb_committed_bytes", lib().mpb_committed_bytes(t.ctypes.data_as(ctypes.c_void_p)))


def mpb_get_committed_bits(i) -> int:
    return _check("mpb_get_committed_bits", lib().mpb_get_committed_bits(i))


def mpb_table_image_bytes(kind, N, b) -> int:
    return _check("mpb_table_image_bytes", lib().mpb_table_image_bytes(kind, N, b))


def mpb_pack_table(kind, lut, N, b, image, stream=None):
    return _check("mpb_pack_table", lib().mpb_pack_table(kind, _ptr(lut), N, b, _ptr(image), _stream(stream)))


def mpb_dequant_block(pages, lut, N, Kd, b, out, stream=None):
    arr = _host_ptrs([p.data_ptr() for p in pages[:b]])
    return _check("mpb_dequant_block", lib().mpb_dequant_block(arr, _ptr(lut), N, Kd, b, _ptr(out),
                                                               _stream(stream)))


def mpb_dequant_block_image(pages, image, kind, N, Kd, b, out, stream=None):
    arr = _host_ptrs([p.data_ptr() for p in pages[:b]])
    return _check("mpb_dequant_block_image", lib().mpb_dequant_block_image(arr, _ptr(image), kind, N, Kd, b,
                                                                           _ptr(out), _stream(stream)))


def mpb_set_kernel_events(events):
    """events: list of 5 raw hipEvent_t handles (ints), or [] to turn recording off."""
    if not events:
        return _check("mpb_set_kernel_events", lib().mpb_set_kernel_events(None, 0))
    return _check("mpb_set_kernel_events", lib().mpb_set_kernel_events(_host_ptrs(events), len(events)))


def mpb_set_resident_planes(i, r):
    return _check("mpb_set_resident_planes", lib().mpb_set_resident_planes(i, r))


def mpb_get_resident_planes(i) -> int:
    return _check("mpb_get_resident_planes", lib().mpb_get_resident_planes(i))


def _ptr_array(ts, n):
    """n pointers (0 where the entry is None or missing) from a list of tensors."""
    ptrs = [0] * n
    for k, t in enumerate(ts):
        if t is not None:
            ptrs[k] = t.data_ptr()
    return _host_ptrs(ptrs)


def mpb_offload_pages(i, r, host_planes, dev_planes, host_tables, dev_tables, copy_stream):
    """planes: lists of 8 tensors (plane pages 0..7), tables: lists of 6
    (table images of bitwidths 3..8); None where a page does not move."""
    return _check("mpb_offload_pages", lib().mpb_offload_pages(
        i, r, _ptr_array(host_planes, 8), _ptr_array(dev_planes, 8), _ptr_array(host_tables, 6),
        _ptr_array(dev_tables, 6), _stream(copy_stream)))


def mpb_reload_pages(i, r, host_planes, dev_planes, host_tables, dev_tables, copy_stream):
    return _check("mpb_reload_pages", lib().mpb_reload_pages(
        i, r, _ptr_array(host_planes, 8), _ptr_array(dev_planes, 8), _ptr_array(host_tables, 6),
        _ptr_array(dev_tables, 6), _stream(copy_stream)))


def mpb_page_state(i, p) -> int:
    return _check("mpb_page_state", lib().mpb_page_state(i, p))


def planner_params(P: dict) -> PlannerParams:
    """Pack a dict of planner parameters (the header's field names) into the C struct."""
    c = PlannerParams()
    c.n_buckets = len(P["bucket_frac"])
    for k in range(c.n_buckets):
        c.bucket_frac[k] = P["bucket_frac"][k]
        c.mu[k] = P["mu"][k]
        c.floor[k] = P["floor"][k]
    c.n_stages = len(P["stage_floor"])
    for k in range(c.n_stages):
        c.stage_floor[k] = P["stage_floor"][k]
    c.eps, c.alpha, c.rho_min, c.rho_max = P["eps"], P["alpha"], P["rho_min"], P["rho_max"]
    for u in range(2):
        for t in range(5):
            for j in range(3):
                c.head_w[u][t][j] = P["head_w"][u][t][j]
            c.head_a[u][t] = P["head_a"][u][t]
            c.head_c[u][t] = P["head_c"][u][t]
    c.T_blk, c.F_blk, c.P_blk, c.B_kv = P["T_blk"], P["F_blk"], P["P_blk"], P["B_kv"]
    return c


def mpb_plan_step(H, I, E, S, K, q, movable, sens, mass, phi, P: dict):
    """Host planner step. q [nb] int, movable [nb] bool or None, sens [nb][6]
    (b = 3..8), mass [E], phi [nb][3]. Returns (plan, summary, queue) with plan
    a list of (i, from, to, delta, damage), summary a dict and queue an
    [n_stages][nb] int32 array."""
    import numpy as np
    nb = 2 * (E + S)
    d = LayerDesc(H, I, E, S, K)
    q = np.ascontiguousarray(q, dtype=np.int32)
    mv = None if movable is None else np.ascontiguousarray(movable, dtype=np.uint8)
    sens = np.ascontiguousarray(sens, dtype=np.float64)
    mass = np.ascontiguousarray(mass, dtype=np.float64)
    phi = np.ascontiguousarray(phi, dtype=np.float64)
    assert q.shape == (nb,) and sens.shape == (nb, 6) and mass.shape == (E,) and phi.shape == (nb, 3)
    prm = planner_params(P)
    queue = np.zeros((prm.n_stages, nb), dtype=np.int32)
    plan = (PlanEntry * nb)()
    summ = PlanSummary()

    def vp(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    _check("mpb_plan_step", lib().mpb_plan_step(ctypes.byref(d), vp(q), vp(mv), vp(sens), vp(mass), vp(phi),
                                                ctypes.byref(prm), vp(queue), plan, ctypes.byref(summ)))
    entries = [(plan[k].i, plan[k].from_, plan[k].to, plan[k].delta, plan[k].damage) for k in range(summ.n_plan)]
    summary = {"D": summ.D, "triggered": bool(summ.triggered), "stage": summ.stage, "released": summ.released,
               "damage": summ.damage, "stage_released": list(summ.stage_released)[:prm.n_stages],
               "stage_damage": list(summ.stage_damage)[:prm.n_stages]}
    return entries, summary, queue

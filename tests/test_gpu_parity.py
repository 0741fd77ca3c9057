"""GPU parity: libmpb (through its C ABI) against the CPU oracle.

Bit-exact: dequantised weights (uint16 compare) and top-K expert indices.
Floating point: topk_w and out within |gpu - ref| <= 1e-3 + 1e-2 |ref| for
every element (the stated tolerance). The full-size decode and prefill layers
are checked on sampled tokens; the small and ragged layers on every element.
"""
import numpy as np
import pytest

import mpb_synth as S
import oracle as O
from helpers import assert_close, oracle_route, say, to_dev_x, tol_ratio

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_bit_amd  # noqa: F401  (fails loudly if libmpb.so is missing)


def M():
    from mixed_precision_bit_amd import _lib
    return _lib


_dev_layers = {}


def dev_layer(layer_cache, cfg):
    from mixed_precision_bit_amd.layer import DeviceLayer
    L = layer_cache(cfg)
    key = cfg
    if key not in _dev_layers:
        _dev_layers.clear()
        torch.cuda.empty_cache()
        _dev_layers[key] = DeviceLayer.from_synth(L)
    D = _dev_layers[key]
    # rebind this layer's page table and restore its initial bitwidths
    M().mpb_init(D.H, D.I, D.E, D.S, D.K, D.q_dev, L.q)
    return L, D


def run_layer(D, Xbits, xdtype):
    X = to_dev_x(Xbits)
    idx, w, out = D.forward(X, xdtype)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), out.cpu().numpy()


# ---------------------------------------------------------------- dequant
@pytest.mark.parametrize("N,Kd", [(64, 128), (256, 2048), (2816, 64)])
def test_dequant_bit_exact_all_bitwidths(N, Kd):
    blk = S.make_block(77, N + Kd, N, Kd)
    canon = torch.from_numpy(blk.planes.view(np.int32)).cuda()
    nw = M().mpb_plane_page_bytes(N, Kd) // 4
    pages = [torch.empty(nw, dtype=torch.int32, device="cuda") for _ in range(8)]
    M().mpb_pack_block(canon, N, Kd, pages)
    for b in S.BITS:
        lut = torch.from_numpy(blk.luts[b - 3].view(np.int16)).cuda()
        out = torch.empty((N, Kd), dtype=torch.int16, device="cuda")
        M().mpb_dequant_block(pages, lut, N, Kd, b, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint16)
        ref = O.dequant(blk.planes, blk.luts[b - 3], b).astype(np.float16).view(np.uint16)
        assert np.array_equal(got, ref), f"b={b}: {np.count_nonzero(got != ref)} mismatches"


@pytest.mark.parametrize("N,Kd,kind", [(256, 2048, 0), (2816, 64, 1), (192, 128, 1), (1408, 192, 0)])
def test_dequant_through_table_image_bit_exact(N, Kd, kind):
    """mpb_pack_table's image read the way the FFN kernels stage and index it
    (mpb_dequant_block_image) gives, bit for bit, the weights of the canonical
    tables ("PagedWeight" §3.1, Eq. 2) and of the oracle, at every bitwidth, for
    gate_up (kind 0: rows of the gate and up halves paired in a tile) and down
    (kind 1, with a last tile partly past N)."""
    blk = S.make_block(91, N + Kd + kind, N, Kd)
    canon = torch.from_numpy(blk.planes.view(np.int32)).cuda()
    nw = M().mpb_plane_page_bytes(N, Kd) // 4
    pages = [torch.empty(nw, dtype=torch.int32, device="cuda") for _ in range(8)]
    M().mpb_pack_block(canon, N, Kd, pages)
    for b in S.BITS:
        lut = torch.from_numpy(blk.luts[b - 3].view(np.int16)).cuda()
        img = torch.empty(M().mpb_table_image_bytes(kind, N, b) // 2, dtype=torch.int16, device="cuda")
        M().mpb_pack_table(kind, lut, N, b, img)
        out = torch.empty((N, Kd), dtype=torch.int16, device="cuda")
        M().mpb_dequant_block_image(pages, img, kind, N, Kd, b, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint16)
        ref = O.dequant(blk.planes, blk.luts[b - 3], b).astype(np.float16).view(np.uint16)
        assert np.array_equal(got, ref), f"b={b}: {np.count_nonzero(got != ref)} mismatches"


def test_pack_round_trip_integer_table():
    rng = np.random.default_rng(11)
    N, Kd = 96, 192
    codes = rng.integers(0, 256, size=(N, Kd), dtype=np.uint8)
    planes = S.codes_to_planes(codes)
    canon = torch.from_numpy(planes.view(np.int32)).cuda()
    nw = M().mpb_plane_page_bytes(N, Kd) // 4
    pages = [torch.empty(nw, dtype=torch.int32, device="cuda") for _ in range(8)]
    M().mpb_pack_block(canon, N, Kd, pages)
    lut = np.tile(np.arange(256) - 128.0, (N, 1)).astype(np.float16)
    out = torch.empty((N, Kd), dtype=torch.int16, device="cuda")
    M().mpb_dequant_block(pages, torch.from_numpy(lut.view(np.int16)).cuda(), N, Kd, 8, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.float16).astype(np.int64)
    assert np.array_equal(got, codes.astype(np.int64) - 128)
    # lower bitwidths read only the top planes: code >> (8-b) indexes the table
    for b in (3, 5, 7):
        lut_b = np.tile(np.arange(1 << b, dtype=np.float64), (N, 1)).astype(np.float16)
        M().mpb_dequant_block(pages, torch.from_numpy(lut_b.view(np.int16)).cuda(), N, Kd, b, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.float16).astype(np.int64)
        assert np.array_equal(got, codes.astype(np.int64) >> (8 - b))


# ---------------------------------------------------------------- routing
def route_ws(T, E):
    return torch.empty(max(1, M().moe_route_workspace_bytes(T, E)), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("cfg,T", [(0, None), (1, None), (2, None), (3, None), (4, None), (10, None), (11, None),
                                   (1, 4096)])
def test_route_bit_exact(cfg, T):
    """Top-K bit-exact, weights within tolerance. Config 3 (bf16) and config 1
    at 4096 tokens (fp16) take the matrix-core logits (>= 1024 16x16 tiles),
    the others the vector path."""
    c = S.layer_config(cfg)
    L = S.make_layer(cfg, blocks=[])
    Xb = S.make_tokens(cfg, T=T, seed=None if T is None else 8000 + T)
    say(f"route cfg{cfg}: T={Xb.shape[0]} H={c['H']} E={c['E']} K={c['K']}")
    X, z, r = oracle_route(L, Xb)
    W = torch.from_numpy(L.W_r).cuda()
    bias = None if L.bias is None else torch.from_numpy(L.bias).cuda()
    T = Xb.shape[0]
    idx = torch.empty((T, L.K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, L.K), dtype=torch.float32, device="cuda")
    ws = route_ws(T, L.E)
    M().moe_route(to_dev_x(Xb), 0 if c["xdtype"] == "f16" else 1, W, bias, L.K, idx, w, ws)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, z), f"{np.count_nonzero((gi != z).any(1))} tokens differ"
    assert_close(w.cpu().numpy(), r, f"cfg{cfg} topk_w")


def test_route_workspace_reused_across_calls_and_replays():
    """One router workspace serves calls of different sizes in a row and a
    captured graph's replays, each bit-identical to the first call and to the
    oracle's top-K."""
    c = S.layer_config(1)
    L = S.make_layer(1, blocks=[])
    Xb = S.make_tokens(1)
    T = Xb.shape[0]
    X, z, r = oracle_route(L, Xb)
    W = torch.from_numpy(L.W_r).cuda()
    Xd = to_dev_x(Xb)
    ws = route_ws(T, L.E)
    outs = []
    for n in (T, 37, T, 5, T):
        idx = torch.empty((n, L.K), dtype=torch.int32, device="cuda")
        w = torch.empty((n, L.K), dtype=torch.float32, device="cuda")
        M().moe_route(Xd[:n].contiguous(), 0, W, None, L.K, idx, w, ws)
        torch.cuda.synchronize()
        say(f"route call T={n}")
        assert np.array_equal(idx.cpu().numpy(), z[:n]), f"T={n}"
        outs.append((idx.cpu().numpy(), w.cpu().numpy()))
    for gi, gw in outs[1:]:
        n = gi.shape[0]
        assert np.array_equal(gw.view(np.uint32), outs[0][1][:n].view(np.uint32))
    assert_close(outs[0][1], r, "topk_w")
    idx = torch.full((T, L.K), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, L.K), dtype=torch.float32, device="cuda")
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            M().moe_route(Xd, 0, W, None, L.K, idx, w, ws, stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    for k in range(3):
        idx.fill_(-1)
        w.zero_()
        g.replay()
        torch.cuda.synchronize()
        say(f"route replay {k}")
        assert np.array_equal(idx.cpu().numpy(), z)
        assert np.array_equal(w.cpu().numpy().view(np.uint32), outs[0][1].view(np.uint32))


def test_route_ties_lowest_index():
    rng = np.random.default_rng(12)
    H, E, K, T = 256, 24, 6, 40
    Wr = (rng.standard_normal((E, H)) / 16).astype(np.float32)
    Wr[7] = Wr[3]
    Wr[19] = Wr[3]
    Wr[20] = Wr[11]
    Xb = rng.standard_normal((T, H)).astype(np.float16).view(np.uint16)
    X = S.f16_bits_to_f64(Xb)
    for Wt in (Wr, np.zeros_like(Wr)):
        z, r, _ = O.route(X, Wt, None, K)
        idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
        w = torch.empty((T, K), dtype=torch.float32, device="cuda")
        M().moe_route(to_dev_x(Xb), 0, torch.from_numpy(Wt).cuda(), None, K, idx, w, route_ws(T, E))
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), z)
        assert_close(w.cpu().numpy(), r, "tie topk_w")


@pytest.mark.parametrize("cfg", [1, 3])
def test_routing_mass_matches_eq1(cfg):
    """moe_routing_mass on the GPU router's output vs the oracle's Eq. 1 on the
    oracle's routing (same top-K, weights within fp32 rounding)."""
    c = S.layer_config(cfg)
    L = S.make_layer(cfg, blocks=[])
    Xb = S.make_tokens(cfg)
    T = Xb.shape[0]
    X, z, r = oracle_route(L, Xb)
    W = torch.from_numpy(L.W_r).cuda()
    bias = None if L.bias is None else torch.from_numpy(L.bias).cuda()
    idx = torch.empty((T, L.K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, L.K), dtype=torch.float32, device="cuda")
    M().moe_route(to_dev_x(Xb), 0 if c["xdtype"] == "f16" else 1, W, bias, L.K, idx, w, route_ws(T, L.E))
    mass = torch.empty(L.E, dtype=torch.float64, device="cuda")
    M().moe_routing_mass(idx, w, L.E, mass)
    m_ref = O.routing_mass(z, r, L.E)
    m = mass.cpu().numpy()
    assert abs(m.sum() - 1.0) < 1e-12
    assert_close(m, m_ref, f"cfg{cfg} routing mass")
    # out-of-range ids count in neither sum; an empty batch gives zeros
    idx2 = idx.clone()
    idx2[0, 0] = L.E
    M().moe_routing_mass(idx2, w, L.E, mass)
    z2 = z.copy()
    z2[0, 0] = L.E
    assert_close(mass.cpu().numpy(), O.routing_mass(z2, r, L.E), f"cfg{cfg} routing mass, one id out of range")
    M().moe_routing_mass(idx[:0], w[:0], L.E, mass)
    assert not mass.cpu().numpy().any()


# ---------------------------------------------------------------- FFN, every element
@pytest.mark.parametrize("cfg", [0, 10, 11])
def test_ffn_small_every_element(cfg, layer_cache):
    L, D = dev_layer(layer_cache, cfg)
    Xb = S.make_tokens(cfg)
    say(f"ffn cfg{cfg}: T={Xb.shape[0]} q={L.q.tolist()}")
    gi, gw, gout = run_layer(D, Xb, L.cfg["xdtype"])
    X, z, r = oracle_route(L, Xb)
    assert np.array_equal(gi, z)
    ref = O.moe_ffn(X, z, r, L)
    assert_close(gout, ref, f"cfg{cfg} out")


def test_ffn_qwen_decode_every_element(layer_cache):
    L, D = dev_layer(layer_cache, 1)
    Xb = S.make_tokens(1)
    say(f"ffn cfg1 full: T={Xb.shape[0]}")
    gi, gw, gout = run_layer(D, Xb, "f16")
    X, z, r = oracle_route(L, Xb)
    assert np.array_equal(gi, z)
    ref = O.moe_ffn(X, z, r, L)
    assert_close(gout, ref, "cfg1 out")


def test_ffn_refuses_batches_beyond_32bit_staging(layer_cache):
    """The FFN kernels stage activation and h rows with 32-bit byte offsets:
    a batch whose activations or h would span 4 GiB is refused on the host
    (MPB_E_SHAPE) before anything is enqueued."""
    L, D = dev_layer(layer_cache, 1)
    lib = M()
    tiny = torch.zeros(64, dtype=torch.int32, device="cuda")
    out = torch.zeros(64, dtype=torch.float32, device="cuda")
    T = 1 << 20   # 2^20 tokens of H = 2048: 4 GiB of fp16 activations
    rc = lib.lib().moe_ffn(lib._ptr(tiny), 0, T, lib._ptr(tiny), lib._ptr(tiny), lib._ptr(D.planes_table),
                           lib._ptr(D.luts_table), lib._ptr(D.q_dev), lib._ptr(out), lib._ptr(tiny), tiny.numel() * 4,
                           lib._stream(None))
    assert rc == -2, (rc, lib.mpb_last_error())
    assert "too large" in lib.mpb_last_error()
    torch.cuda.synchronize()


def test_ffn_deterministic_and_block_independent(layer_cache):
    L, D = dev_layer(layer_cache, 10)
    Xb = S.make_tokens(10)
    _, _, a = run_layer(D, Xb, "f16")
    gi, _, b = run_layer(D, Xb, "f16")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "two runs differ"
    # lower one routed gate_up block: only tokens routed to that expert change
    e = int(gi[0, 0])
    i = 2 * e
    newb = 3 if L.q[i] != 3 else 4
    M().set_committed_bits(i, newb)
    _, _, c = run_layer(D, Xb, "f16")
    routed = (gi == e).any(axis=1)
    assert np.array_equal(c[~routed].view(np.uint32), a[~routed].view(np.uint32))
    assert (c[routed] != a[routed]).any(axis=1).all()
    X, z, r = oracle_route(L, Xb)
    q2 = L.q.copy()
    q2[i] = newb
    assert_close(c, O.moe_ffn(X, z, r, L, q=q2), "after set_committed_bits")
    M().set_committed_bits(i, int(L.q[i]))


def test_set_committed_bits_is_stream_ordered(layer_cache):
    L, D = dev_layer(layer_cache, 0)
    Xb = S.make_tokens(0)
    X = to_dev_x(Xb)
    T = Xb.shape[0]
    idx, w = D.alloc_route(T)
    out1, ws1 = D.alloc_ffn(T)
    out2, ws2 = D.alloc_ffn(T)
    D.route(X, "f16", idx, w)
    q2 = L.q.copy()
    D.ffn(X, "f16", idx, w, out1, ws1)
    for i in range(L.n_blocks):          # enqueued behind the first FFN
        q2[i] = 8 if L.q[i] < 8 else 3
        M().set_committed_bits(i, int(q2[i]))
    D.ffn(X, "f16", idx, w, out2, ws2)
    torch.cuda.synchronize()
    Xf, z, r = oracle_route(L, Xb)
    assert_close(out1.cpu().numpy(), O.moe_ffn(Xf, z, r, L), "before commit")
    assert_close(out2.cpu().numpy(), O.moe_ffn(Xf, z, r, L, q=q2), "after commit")
    assert [M().mpb_get_committed_bits(i) for i in range(L.n_blocks)] == q2.tolist()


def _gated_stream(cycles=200_000_000):
    """A copy stream held back by a bounded spin kernel on another stream, so
    that work enqueued on it right now is still in flight a moment later."""
    gate, cs = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(gate):
        torch.cuda._sleep(cycles)
    ev = torch.cuda.Event()
    ev.record(gate)
    cs.wait_event(ev)
    return cs


def test_page_movement_offload_then_reload(layer_cache):
    """Offload lowers q_i first, then moves the pages above it (plane pages and
    the tables of the higher bitwidths) to the CPU; a reload brings them back
    and q_i rises only once they are GPU-resident (PagedWeight §3.1 after
    Eq. 3, §3.3 and Figure 4). After the offload the freed device memory is
    overwritten and the layer still matches the oracle; the reload goes into
    fresh device buffers."""
    L, D = dev_layer(layer_cache, 10)
    E_ = M().MpbError
    GPU, CPU, XFER = M().MPB_PAGE_GPU, M().MPB_PAGE_CPU, M().MPB_PAGE_IN_TRANSFER
    Xb = S.make_tokens(10)
    X, z, r = oracle_route(L, Xb)
    Xd = to_dev_x(Xb)
    T = Xb.shape[0]
    idx, w = D.alloc_route(T)
    out, ws = D.alloc_ffn(T)
    D.route(Xd, "f16", idx, w)
    e = int(z[0, 0])
    blocks = [2 * e, 2 * e + 1]          # both linear-blocks of a routed expert

    def pinned(t):
        return torch.empty(t.shape, dtype=t.dtype, pin_memory=True)

    keep_p = {i: [t.clone() for t in D.pages[i]] for i in blocks}
    keep_t = {i: [t.clone() for t in D.luts[i]] for i in blocks}
    hp = {i: [pinned(t) for t in D.pages[i]] for i in blocks}
    ht = {i: [pinned(t) for t in D.luts[i]] for i in blocks}
    q = L.q.copy()
    for i in blocks:
        M().set_committed_bits(i, 8)
        q[i] = 8
        with pytest.raises(E_) as ei:        # q_i must be lowered first
            M().mpb_offload_pages(i, 4, hp[i], D.pages[i], ht[i], D.luts[i], torch.cuda.Stream())
        assert ei.value.code == -4
    # ---- offload to 4 pages while an FFN at 8 bits is still enqueued
    D.ffn(Xd, "f16", idx, w, out, ws)
    for i in blocks:
        M().set_committed_bits(i, 4)
        q[i] = 4
    cs = _gated_stream()
    for i in blocks:
        M().mpb_offload_pages(i, 4, hp[i], D.pages[i], ht[i], D.luts[i], cs)
        assert M().mpb_get_resident_planes(i) == 4
        assert [M().mpb_page_state(i, p) for p in range(8)] == [GPU] * 4 + [XFER] * 4
        with pytest.raises(E_) as ei:
            M().set_committed_bits(i, 5)
        assert ei.value.code == -4
        with pytest.raises(E_) as ei:
            M().mpb_reload_pages(i, 8, hp[i], D.pages[i], ht[i], D.luts[i], cs)
        assert ei.value.code == -8
    cs.synchronize()
    for i in blocks:
        assert [M().mpb_page_state(i, p) for p in range(8)] == [GPU] * 4 + [CPU] * 4
        for p in range(4, 8):
            assert torch.equal(hp[i][p], keep_p[i][p].cpu()), f"offloaded plane {p} of block {i}"
            assert torch.equal(ht[i][p - 2], keep_t[i][p - 2].cpu()), f"offloaded table {p + 1} of block {i}"
            D.pages[i][p].fill_(0x5A5A5A5A)   # the freed memory is reused
            D.luts[i][p - 2].fill_(0x7E00)     # (a NaN pattern, were it ever read)
        assert torch.equal(D.luts[i][1], keep_t[i][1]), "the 4-bit table stays"
    torch.cuda.synchronize()
    q8 = q.copy()
    q8[blocks] = 8
    assert_close(out.cpu().numpy(), O.moe_ffn(X, z, r, L, q=q8), "FFN enqueued before the offload")
    D.ffn(Xd, "f16", idx, w, out, ws)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), O.moe_ffn(X, z, r, L, q=q), "after offload, memory reused")
    # ---- reload into fresh buffers; q_i rises only after the copies
    fp = {i: [None] * 4 + [torch.empty_like(D.pages[i][p]) for p in range(4, 8)] for i in blocks}
    ft = {i: [None] * 2 + [torch.empty_like(D.luts[i][t]) for t in range(2, 6)] for i in blocks}
    ptab, ttab = D.planes_table.clone(), D.luts_table.clone()
    for i in blocks:
        for p in range(4, 8):
            ptab[i * 8 + p] = fp[i][p].data_ptr()
            ttab[i * 6 + p - 2] = ft[i][p - 2].data_ptr()
    cs = _gated_stream()
    for i in blocks:
        M().mpb_reload_pages(i, 8, hp[i], fp[i], ht[i], ft[i], cs)
        assert [M().mpb_page_state(i, p) for p in range(8)] == [GPU] * 4 + [XFER] * 4
        with pytest.raises(E_) as ei:
            M().set_committed_bits(i, 6)
        assert ei.value.code == -4
    # an FFN at the committed 4 bits runs while the copies are in flight
    M().moe_ffn(Xd, 0, idx, w, ptab, ttab, D.q_dev, out, ws)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), O.moe_ffn(X, z, r, L, q=q), "during reload")
    cs.synchronize()
    for i in blocks:
        assert [M().mpb_page_state(i, p) for p in range(8)] == [GPU] * 8
        assert M().mpb_get_resident_planes(i) == 8
        M().set_committed_bits(i, 8)
    M().moe_ffn(Xd, 0, idx, w, ptab, ttab, D.q_dev, out, ws)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), O.moe_ffn(X, z, r, L, q=q8), "after reload at 8 bits")
    # restore the cached layer's buffers (later tests reuse it)
    for i in blocks:
        for p in range(8):
            D.pages[i][p].copy_(keep_p[i][p])
        for t in range(6):
            D.luts[i][t].copy_(keep_t[i][t])
    torch.cuda.synchronize()


# ---------------------------------------------------------------- full-size layers, sampled
def _coverage(L, z, T, tpi_gu, tpi_dn):
    """(token, expert) pairs of a batch and the FFN work items they form."""
    cnt = np.bincount(z.ravel(), minlength=L.E)
    cnt = np.concatenate([cnt, np.full(L.S, T)])
    pairs = int(cnt.sum())
    gu = int(sum((c + tpi_gu - 1) // tpi_gu for c in cnt))
    dn = int(sum((c + tpi_dn - 1) // tpi_dn for c in cnt))
    return pairs, gu, dn


def test_ffn_mixtral_decode_every_element(layer_cache):
    """The Mixtral-shaped decode layer (H 4096, I 14336, 8 experts, top-2, 128
    tokens, gate_up 4-bit / down 3-bit) at every output element: every token's
    two experts, every 32-token item (including the short second items of
    experts with more than 32 tokens) and every K range of the split down
    projection."""
    L, D = dev_layer(layer_cache, 2)
    Xb = S.make_tokens(2)
    T = Xb.shape[0]
    gi, gw, gout = run_layer(D, Xb, "f16")
    X, z, r = oracle_route(L, Xb)
    assert np.array_equal(gi, z)
    pairs, n_gu, n_dn = _coverage(L, z, T, 32, 32)
    say(f"ffn cfg2 full: T={T}, {pairs} (token, expert) pairs, {n_gu} gate_up / {n_dn} down items, "
        f"{T * L.H} outputs")
    ref = O.moe_ffn(X, z, r, L)
    assert_close(gout, ref, "cfg2 out")


def test_ffn_prefill_every_element(layer_cache):
    """The prefill-shaped layer (H 2816, I 704, 128 + 1 experts, top-8, 4096
    bf16 tokens, Zipf-skewed router bias) at every output element: every
    128-token gate_up item, including each expert's last, ragged one and all
    items of the largest group, and every 32-token down item."""
    L, D = dev_layer(layer_cache, 3)
    Xb = S.make_tokens(3)
    T = Xb.shape[0]
    gi, gw, gout = run_layer(D, Xb, "bf16")
    X, z, r = oracle_route(L, Xb)
    assert np.array_equal(gi, z)
    pairs, n_gu, n_dn = _coverage(L, z, T, 128, 32)
    cnt = np.bincount(z.ravel(), minlength=L.E)
    say(f"ffn cfg3 full: T={T}, {pairs} (token, expert) pairs, {n_gu} gate_up / {n_dn} down items, "
        f"largest group {cnt.max()} tokens, {int((cnt % 128 != 0).sum())} ragged last items, {T * L.H} outputs")
    ref = O.moe_ffn(X, z, r, L)
    assert_close(gout, ref, "cfg3 out")


# ---------------------------------------------------------------- bitwidth sweep
def test_planner_drives_commits_and_offloads(layer_cache):
    """The planner step (PagedWeight §3.2, Algorithm 1) fed with the routing
    mass the GPU computes for this batch (Eq. 1) selects a plan; applying it
    (lower q_i, then offload the pages above it, §3.3) releases exactly the
    planned bytes, and the layer at the planned bitwidths matches the oracle."""
    L, D = dev_layer(layer_cache, 1)
    Xb = S.make_tokens(1)
    X, z, r = oracle_route(L, Xb)
    Xd = to_dev_x(Xb)
    T = Xb.shape[0]
    idx, w = D.alloc_route(T)
    out, ws = D.alloc_ffn(T)
    D.route(Xd, "f16", idx, w)
    mass = torch.empty(L.E, dtype=torch.float64, device="cuda")
    M().moe_routing_mass(idx, w, L.E, mass)
    torch.cuda.synchronize()
    m = mass.cpu().numpy()
    sens = S.make_sensitivity(1, L.n_blocks)
    P, phi = S.make_planner_inputs(1, L.n_blocks, 20)
    plan, summ, _ = M().mpb_plan_step(L.H, L.I, L.E, L.S, L.K, L.q, None, sens[:, 3:9], m, phi, P)
    oplan, osumm, _ = O.plan_step(L.H, L.I, L.E, L.S, L.q, None, sens, m, phi, P)
    assert plan == oplan and summ == osumm
    assert summ["triggered"] and summ["released"] >= summ["D"] > 0 and plan
    say(f"  plan: stage {summ['stage']}, {len(plan)} blocks, {summ['released'] / 1e6:.2f} MB "
        f"for a target of {summ['D'] / 1e6:.2f} MB")
    before = M().mpb_committed_bytes()
    cs = torch.cuda.Stream()
    host = {}
    q = L.q.copy()
    for i, frm, to, delta, _ in plan:
        M().set_committed_bits(i, to)
        q[i] = to
        hp = [None] * to + [torch.empty(D.pages[i][p].shape, dtype=D.pages[i][p].dtype, pin_memory=True)
                            for p in range(to, 8)]
        ht = [None] * (to - 2) + [torch.empty(D.luts[i][t].shape, dtype=D.luts[i][t].dtype, pin_memory=True)
                                  for t in range(to - 2, 6)]
        host[i] = (hp, ht)
        M().mpb_offload_pages(i, to, hp, D.pages[i], ht, D.luts[i], cs)
    assert before - M().mpb_committed_bytes() == summ["released"]
    D.ffn(Xd, "f16", idx, w, out, ws)
    cs.synchronize()
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), O.moe_ffn(X, z, r, L, q=q), "at the planned bitwidths")
    for i, frm, to, delta, _ in plan:
        assert M().mpb_get_resident_planes(i) == to
        assert M().mpb_page_state(i, 7) == M().MPB_PAGE_CPU


def test_bitwidth_sweep_states(layer_cache):
    L, D = dev_layer(layer_cache, 1)   # the config-4 layer is the config-1 layer
    Xb = S.make_tokens(4)
    T = Xb.shape[0]
    X, z, r = oracle_route(L, Xb)
    s = S.make_sensitivity(4, L.n_blocks)
    states = [("initial", L.q.copy())]
    for f in (0.25, 0.5, 0.75):
        red, short = O.greedy_reductions(L, s, f)
        q = L.q.copy()
        for i, b2 in red:
            q[i] = b2
        states.append((f"lowered {int(f * 100)}% (short {short})", q))
    states.append(("all 8-bit", np.full(L.n_blocks, 8, np.int32)))
    wcache = {}
    Xd = to_dev_x(Xb)
    idx, w = D.alloc_route(T)
    out, ws = D.alloc_ffn(T)
    D.route(Xd, "f16", idx, w)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), z)
    prev = L.q.copy()
    for name, q in states:
        for i in np.nonzero(q != prev)[0]:
            M().set_committed_bits(int(i), int(q[i]))
        prev = q
        D.ffn(Xd, "f16", idx, w, out, ws)
        torch.cuda.synchronize()
        assert M().mpb_committed_bytes() == O.committed_bytes(L, q=q)
        ref = O.moe_ffn(X, z, r, L, q=q, wcache=wcache)
        r_ = tol_ratio(out.cpu().numpy(), ref)
        say(f"  state {name}: committed {O.committed_bytes(L, q=q) / 1e6:.1f} MB, max err/tol {r_:.4f}")
        assert r_ <= 1.0


# ---------------------------------------------------------------- edge cases
def test_edge_token_counts(layer_cache):
    L, D = dev_layer(layer_cache, 10)
    for T in (1, 33, 200):
        Xb = S.make_tokens(10, T=T, seed=5000 + T)
        _, _, gout = run_layer(D, Xb, "f16")
        X, z, r = oracle_route(L, Xb)
        assert_close(gout, O.moe_ffn(X, z, r, L), f"T={T}")
    X0 = torch.empty((0, L.H), dtype=torch.int16, device="cuda")
    idx, w = D.alloc_route(0)
    out, ws = D.alloc_ffn(0)
    D.route(X0, "f16", idx, w)
    D.ffn(X0, "f16", idx, w, out, ws)
    torch.cuda.synchronize()


def test_chunked_grouping_large_batch(layer_cache):
    """Batches with T*K at or above the chunked-grouping threshold (8192
    routed entries, chunks of 2048) group through the chunked path; a ragged
    last chunk and the shared experts included. Every output element is held
    to the oracle, and the one-launch path (single-pass grouping) agrees bit
    for bit."""
    L, D = dev_layer(layer_cache, 10)
    for T in (2731, 3000):     # T*K = 8193 (last chunk of 1 entry), 9000
        Xb = S.make_tokens(10, T=T, seed=7000 + T)
        say(f"chunked grouping: T={T}, T*K={T * L.K}")
        i1, w1, o1, i2, w2, o2, _ = _separate_and_fused(D, Xb, "f16")
        X, z, r = oracle_route(L, Xb)
        assert np.array_equal(i1, z)
        ref = O.moe_ffn(X, z, r, L)
        assert_close(o1, ref, f"T={T}")
        assert_close(o2, ref, f"T={T} fused")
        if not _wide(L, T):
            assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


def test_largest_batch_sampled(layer_cache):
    """A batch of 65536 tokens on the small layer: 131072 routed entries in 64
    grouping chunks, 128-token gate_up items, 4096-item down lists. Routing
    is compared for every token, outputs on a sample of tokens (the first,
    the last and every 1021st); the one-launch path agrees bit for bit."""
    L, D = dev_layer(layer_cache, 0)
    T = 65536
    Xb = S.make_tokens(0, T=T, seed=9000)
    say(f"largest batch: cfg0 T={T}")
    i1, w1, o1, i2, w2, o2, _ = _separate_and_fused(D, Xb, "f16")
    X, z, r = oracle_route(L, Xb)
    assert np.array_equal(i1, z)
    toks = np.unique(np.concatenate([np.arange(0, T, 1021), [T - 1]]))
    ref = O.moe_ffn(X[toks], z[toks], r[toks], L)
    assert_close(o1[toks], ref, f"T={T} sampled")
    assert_close(o2[toks], ref, f"T={T} sampled, fused")
    assert np.array_equal(i1, i2)
    if not _wide(L, T):
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


def test_bf16_beyond_fp16_range_every_element(layer_cache):
    """bf16 activations reach the fp16 matrix cores through a per-token
    power-of-two scale: tokens holding values far beyond the fp16 range
    (|x| up to ~4e6 and ~1e5) or far below its normal range (~1e-30) are held
    to the oracle at every element, like the ordinary tokens beside them, on
    both paths; the one-launch path agrees bit for bit."""
    L, D = dev_layer(layer_cache, 11)
    Xb = S.make_tokens(11).copy()
    for t, f in ((4, 1e6), (6, 3e4), (7, 1e-30)):
        Xb[t] = S.f32_to_bf16_bits((S.bf16_bits_to_f64(Xb[t]) * f).astype(np.float32))
    X, z, r = oracle_route(L, Xb)
    assert np.abs(X[4]).max() > 65504 and np.abs(X[6]).max() > 65504
    i1, w1, o1, i2, w2, o2, _ = _separate_and_fused(D, Xb, "bf16")
    assert np.array_equal(i1, z)
    ref = O.moe_ffn(X, z, r, L)
    say(f"  max |ref| of the large tokens: {np.abs(ref[4]).max():.3e}, {np.abs(ref[6]).max():.3e}")
    assert_close(o1, ref, "every token")
    for t in (4, 6, 7):
        assert_close(o1[t], ref[t], f"token {t}", guard=None)
    assert np.array_equal(i1, i2)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


def test_bf16_beyond_fp16_range_wide_groups(layer_cache):
    """The per-token power-of-two scale of bf16 activations beyond the fp16
    range in a batch whose large groups take the grouped-GEMM kernels
    (4000 tokens, Zipf-skewed router bias, H = I = 192: a ragged last row tile
    of the down projection and an odd number of 64-K steps): tokens holding
    values up to ~1e6 times their draw, and one far below the fp16 normal
    range, among ordinary ones, every output element against the oracle."""
    L, D = dev_layer(layer_cache, 11)
    T = 4000
    Xb = S.make_tokens(11, T=T, seed=8000 + T).copy()
    X0, z0, _ = oracle_route(L, Xb)
    cnt0 = np.bincount(z0.ravel(), minlength=L.E)
    wide0 = np.nonzero(cnt0 >= WIDE_FROM)[0]
    # scaled far up, a token goes to its unbiased best expert: take tokens whose
    # unbiased best expert is a large group, so that they stay in one
    best = np.argmax(X0 @ L.W_r.T, axis=1)
    cand = [int(t) for t in np.nonzero(np.isin(best, wide0))[0]]
    big = (cand[0], cand[len(cand) // 2], cand[-1])
    small = next(t for t in range(T) if t not in big and int(z0[t, 0]) in wide0)
    for t, f in zip(big + (small,), (1e6, 3e4, 1e5, 1e-30)):
        Xb[t] = S.f32_to_bf16_bits((S.bf16_bits_to_f64(Xb[t]) * f).astype(np.float32))
    X, z, r = oracle_route(L, Xb)
    assert all(np.abs(X[t]).max() > 65504 for t in big)
    cnt = np.bincount(z.ravel(), minlength=L.E)
    wide = set(np.nonzero(cnt >= WIDE_FROM)[0].tolist())
    assert _wide(L, T) and wide, "the batch must hold groups for the grouped-GEMM kernels"
    assert all(int(z[t, 0]) in wide for t in big + (small,)), "the scaled tokens must sit in wide groups"
    say(f"  wide groups {sorted(wide)}, sizes {sorted(cnt[list(wide)].tolist())}, scaled tokens {big + (small,)}")
    gi, _, gout = run_layer(D, Xb, "bf16")
    assert np.array_equal(gi, z)
    ref = O.moe_ffn(X, z, r, L)
    assert_close(gout, ref, "every token")
    for t in big + (small,):
        assert_close(gout[t], ref[t], f"token {t}", guard=None)


@pytest.mark.parametrize("cfg", [12, 13, 14, 15, 16])
def test_edge_shapes_every_element(cfg, layer_cache):
    """Extreme layer shapes, every element against the oracle on both paths:
    one expert with H = I = 64 (a single K half-chunk and row tile), more
    shared than routed experts with bf16 input and a router bias, top-16 of
    64 experts, 512 experts for a single token, and a layer whose few long
    down items are split over three K ranges (the last of odd length). The
    one-launch path agrees bit for bit."""
    L, D = dev_layer(layer_cache, cfg)
    Xb = S.make_tokens(cfg)
    xdtype = L.cfg["xdtype"]
    say(f"edge shape cfg{cfg} ({L.cfg['name']}): H={L.H} I={L.I} E={L.E} S={L.S} K={L.K} T={Xb.shape[0]}")
    i1, w1, o1, i2, w2, o2, _ = _separate_and_fused(D, Xb, xdtype)
    X, z, r = oracle_route(L, Xb)
    assert np.array_equal(i1, z)
    assert_close(w1, r, f"cfg{cfg} routing weights")
    assert_close(o1, O.moe_ffn(X, z, r, L), f"cfg{cfg} output")
    assert np.array_equal(i1, i2)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


@pytest.mark.parametrize("cfg,T", [(0, 400), (0, 1000), (11, 4000)])
def test_prefill_items_every_element(cfg, T, layer_cache):
    """Batches large enough for 128-token gate_up work items: every output
    element against the oracle, with group sizes ragged against 128 and
    hidden sizes 256 and 192 (even and uneven K halves)."""
    L, D = dev_layer(layer_cache, cfg)
    assert _prefill_items(L, T)
    Xb = S.make_tokens(cfg, T=T, seed=8000 + T)
    say(f"prefill items cfg{cfg}: T={T}")
    gi, _, gout = run_layer(D, Xb, L.cfg["xdtype"])
    X, z, r = oracle_route(L, Xb)
    assert np.array_equal(gi, z)
    assert_close(gout, O.moe_ffn(X, z, r, L), f"cfg{cfg} T={T}")


@pytest.mark.parametrize("T", [150, 600])
def test_edge_one_expert_takes_all_and_extreme_bitwidths(T, layer_cache):
    """One group of T tokens per routed expert (zero logits tie); T = 600
    takes 128-token gate_up items (4 full items and a ragged one)."""
    L, D = dev_layer(layer_cache, 10)
    Xb = S.make_tokens(10, T=T, seed=99)
    X = S.f16_bits_to_f64(Xb)
    # every token picks experts 0..K-1 (zero logits tie), one group of 150 tokens
    z = np.tile(np.arange(L.K), (T, 1))
    r = np.full((T, L.K), 1.0 / L.K)
    idx = torch.from_numpy(z.astype(np.int32)).cuda()
    w = torch.from_numpy(r.astype(np.float32)).cuda()
    out, ws = D.alloc_ffn(T)
    for qv in (3, 8):
        for i in range(L.n_blocks):
            M().set_committed_bits(i, qv)
        D.ffn(to_dev_x(Xb), "f16", idx, w, out, ws)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), O.moe_ffn(X, z, r, L, q=np.full(L.n_blocks, qv)), f"all q={qv}")


def test_edge_group_sizes_around_stage_switch(layer_cache):
    """Groups of 1, 6, 15, 16, 17, 32 and 33 tokens and a 40-token shared
    group: items of at most 16 tokens take the double-buffered activation
    stage, larger ones the single stage; both at every committed bitwidth of
    the layer, every output element against the oracle."""
    L, D = dev_layer(layer_cache, 10)
    T, K = 40, L.K
    sizes = [(0, 16), (1, 17), (2, 15), (3, 33), (4, 1), (5, 32)]
    ent = [e for e, n in sizes for _ in range(n)]
    ent += [6] * (T * K - len(ent))
    # entry j -> token j % T, slot j // T: a group spans < T entries, so no
    # token names an expert twice
    z = np.array(ent, dtype=np.int64).reshape(K, T).T.copy()
    assert all(len(set(row)) == K for row in z)
    rng = np.random.default_rng(123)
    r = rng.uniform(0.1, 1.0, (T, K))
    r /= r.sum(axis=1, keepdims=True)
    r = r.astype(np.float32).astype(np.float64)
    Xb = S.make_tokens(10, T=T, seed=321)
    X = S.f16_bits_to_f64(Xb)
    idx = torch.from_numpy(z.astype(np.int32)).cuda()
    w = torch.from_numpy(r.astype(np.float32)).cuda()
    out, ws = D.alloc_ffn(T)
    D.ffn(to_dev_x(Xb), "f16", idx, w, out, ws)
    torch.cuda.synchronize()
    counts = np.bincount(z.ravel(), minlength=L.E)
    assert sorted(counts[counts > 0].tolist()) == [1, 6, 15, 16, 17, 32, 33]
    assert_close(out.cpu().numpy(), O.moe_ffn(X, z, r, L), "group sizes 1..33")


def test_edge_out_of_range_expert_ids_contribute_nothing(layer_cache):
    L, D = dev_layer(layer_cache, 10)
    T = 20
    Xb = S.make_tokens(10, T=T, seed=7)
    X, z, r = oracle_route(L, Xb)
    zb = z.copy()
    zb[3, 1] = -1
    zb[8, 0] = L.E + 5
    idx = torch.from_numpy(zb.astype(np.int32)).cuda()
    w = torch.from_numpy(r.astype(np.float32)).cuda()
    out, ws = D.alloc_ffn(T)
    D.ffn(to_dev_x(Xb), "f16", idx, w, out, ws)
    torch.cuda.synchronize()
    rr = r.copy()
    rr[3, 1] = 0.0
    rr[8, 0] = 0.0
    zz = zb.copy()
    zz[3, 1] = 0
    zz[8, 0] = 0
    assert_close(out.cpu().numpy(), O.moe_ffn(X, zz, rr, L), "bad ids")


def test_abi_errors_after_init(layer_cache):
    L, D = dev_layer(layer_cache, 0)
    E = M().MpbError
    nb = L.n_blocks
    with pytest.raises(E) as ei:
        M().set_committed_bits(nb, 4)
    assert ei.value.code == -3
    with pytest.raises(E):
        M().set_committed_bits(0, 9)
    i = 1
    M().set_committed_bits(i, 4)
    M().mpb_set_resident_planes(i, 5)
    with pytest.raises(E) as ei:
        M().set_committed_bits(i, 6)   # planes 5..7 are not resident
    assert ei.value.code == -4
    M().set_committed_bits(i, 5)
    with pytest.raises(E) as ei:
        M().mpb_set_resident_planes(i, 4)  # offload must lower q_i first
    assert ei.value.code == -4
    M().mpb_set_resident_planes(i, 8)
    M().set_committed_bits(i, int(L.q[i]))
    Xb = S.make_tokens(0)
    idx, w = D.alloc_route(16)
    out, _ = D.alloc_ffn(16)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(E) as ei:
        D.ffn(to_dev_x(Xb), "f16", idx, w, out, small)
    assert ei.value.code == -5
    # a page table other than the bound one is refused (the host mirror that
    # sizes the kernels' table space describes the bound table only)
    _, ws = D.alloc_ffn(16)
    other = D.q_dev.clone()
    with pytest.raises(E) as ei:
        M().moe_ffn(to_dev_x(Xb), 0, idx, w, D.planes_table, D.luts_table, other, out, ws)
    assert ei.value.code == -1
    # a stream other than the bound one (and not under graph capture) is
    # refused: commits on the bound stream would not be ordered with it
    side = torch.cuda.Stream()
    with pytest.raises(E) as ei:
        M().moe_ffn(to_dev_x(Xb), 0, idx, w, D.planes_table, D.luts_table, D.q_dev, out, ws, side)
    assert ei.value.code == -1
    fo, fws = D.alloc_fused(16)
    with pytest.raises(E) as ei:
        M().moe_fused(to_dev_x(Xb), 0, D.W_r, D.bias, idx, w, D.planes_table, D.luts_table, D.q_dev, fo, fws, side)
    assert ei.value.code == -1
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg,T", [(10, None), (11, 4000)])
def test_graph_replay_matches_eager(cfg, T, layer_cache):
    """moe_route + moe_ffn captured in a HIP graph: every replay, with eager
    work and synchronisation in between, reproduces the eager result bitwise
    (a small batch, and a 4000-token bf16 batch whose large groups take the
    grouped-GEMM kernels)."""
    L, D = dev_layer(layer_cache, cfg)
    Xb = S.make_tokens(cfg, T=T, seed=None if T is None else 9100 + T)
    xdt = L.cfg["xdtype"]
    X = to_dev_x(Xb)
    T = Xb.shape[0]
    idx, w = D.alloc_route(T)
    out, ws = D.alloc_ffn(T)
    D.route(X, xdt, idx, w)
    D.ffn(X, xdt, idx, w, out, ws)
    torch.cuda.synchronize()
    eager = out.cpu().numpy().copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            D.route(X, xdt, idx, w)
            D.ffn(X, xdt, idx, w, out, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 16, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), f"replay {rep} differs"
        del junk


# ---------------------------------------------------------------- one fused launch
def _separate_and_fused(D, Xb, xdtype):
    X = to_dev_x(Xb)
    T = Xb.shape[0]
    idx, w = D.alloc_route(T)
    out, ws = D.alloc_ffn(T)
    D.route(X, xdtype, idx, w)
    D.ffn(X, xdtype, idx, w, out, ws)
    idx2, w2 = D.alloc_route(T)
    out2, ws2 = D.alloc_fused(T)
    D.fused(X, xdtype, idx2, w2, out2, ws2)
    torch.cuda.synchronize()
    return (idx.cpu().numpy(), w.cpu().numpy(), out.cpu().numpy(), idx2.cpu().numpy(), w2.cpu().numpy(),
            out2.cpu().numpy(), ws2)


WIDE_FROM = 96  # smallest group of the grouped-GEMM kernels (batches of >= 2048 tokens)


def _wide(L, T):
    """moe_ffn runs groups of at least 96 tokens through the grouped-GEMM
    kernels (weight tiles dequantised once per K step into LDS, 512 / 256
    tokens per workgroup) in batches of at least 2048 tokens; moe_fused keeps
    32-token items for every group, so the two agree bit for bit only below
    that size (both are held to the oracle either way)."""
    return T >= 2048


def _prefill_items(L, T):
    """moe_ffn takes 128-token gate_up work items (four 32-token chunks per
    dequantised weight operand) once a routed group holds 96 tokens on
    average."""
    return T * L.K // L.E >= 96


@pytest.mark.parametrize("cfg", [0, 10, 11, 1, 2, 3])
def test_fused_launch_equals_separate_calls(cfg, layer_cache):
    """moe_fused (one persistent launch, PagedWeight §3.3) gives bit for bit
    the routing and output of moe_route + moe_ffn, which the other tests hold
    to the oracle, where both take the same FFN kernels; at the prefill size
    (grouped-GEMM kernels for the large groups in moe_ffn) it is held to the
    oracle itself. The small layers are also checked against the oracle here.
    Its counters are back at zero after the call."""
    L, D = dev_layer(layer_cache, cfg)
    Xb = S.make_tokens(cfg)
    xdtype = L.cfg["xdtype"]
    say(f"fused cfg{cfg}: T={Xb.shape[0]}")
    i1, w1, o1, i2, w2, o2, ws2 = _separate_and_fused(D, Xb, xdtype)
    assert np.array_equal(i1, i2)
    assert np.array_equal(w1.view(np.uint32), w2.view(np.uint32))
    if _wide(L, Xb.shape[0]):
        X, z, r = oracle_route(L, Xb)
        assert_close(o2, O.moe_ffn(X, z, r, L), f"cfg{cfg} fused")
        assert_close(o1, o2.astype(np.float64), f"cfg{cfg} separate vs fused")
    else:
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)), \
            f"max |diff| {np.abs(o1.astype(np.float64) - o2).max()}"
    assert int(ws2[:M().moe_fused_counter_bytes()].count_nonzero()) == 0, "counters not reset"
    if cfg in (0, 10, 11):
        X, z, r = oracle_route(L, Xb)
        assert np.array_equal(i2, z)
        assert_close(o2, O.moe_ffn(X, z, r, L), f"cfg{cfg} fused")


def test_fused_launch_graph_replays_and_commits(layer_cache):
    """Captured in a HIP graph, every replay (with eager work and
    synchronisation in between) reproduces the eager result; after
    set_committed_bits the next replay follows the new bitwidths."""
    L, D = dev_layer(layer_cache, 10)
    Xb = S.make_tokens(10)
    X = to_dev_x(Xb)
    T = Xb.shape[0]
    idx, w = D.alloc_route(T)
    out, ws = D.alloc_fused(T)
    D.fused(X, "f16", idx, w, out, ws)
    torch.cuda.synchronize()
    eager = out.cpu().numpy().copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            D.fused(X, "f16", idx, w, out, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), eager.view(np.uint32)), f"replay {rep}"
        del junk
    # lower every block to 3 bits except the first routed expert, raised to the
    # highest bitwidth already committed (the captured table region's size)
    q2 = np.full(L.n_blocks, 3, np.int32)
    q2[0], q2[1] = int(L.q.max()), int(L.q.max())
    for i in range(L.n_blocks):
        M().set_committed_bits(i, int(q2[i]))
    g.replay()
    torch.cuda.synchronize()
    Xf, z, r = oracle_route(L, Xb)
    assert_close(out.cpu().numpy(), O.moe_ffn(Xf, z, r, L, q=q2), "fused replay after commits")
    assert int(ws[:M().moe_fused_counter_bytes()].count_nonzero()) == 0


def _tie_rows(T, n):
    """n tokens spread over the batch, the first and the last among them."""
    return np.unique(np.linspace(0, T - 1, n).round().astype(np.int64))


def _near_tie_x(T, H, j, xdt, rows, rng):
    """Positive activations; column j is the smallest subnormal (2^-24 in
    fp16, 2^-133 in bf16) in the given rows and 1.0 elsewhere, so a router
    weight one ulp apart decides a sub-ulp near-tie in those rows and a
    resolvable gap in the others."""
    xa = np.abs(rng.standard_normal((T, H))).astype(np.float32)
    if xdt == "f16":
        Xb = xa.astype(np.float16).view(np.uint16)
        one = np.float16(1.0).view(np.uint16)
    else:
        Xb = (xa.view(np.uint32) >> 16).astype(np.uint16)
        one = np.uint16(0x3F80)
    Xb[:, j] = one
    Xb[rows, j] = 1
    return np.ascontiguousarray(Xb)


def _near_tie_rows(Wr, a, b, j, up):
    """Router rows a and b equal except weight j of b, one ulp above or below."""
    rng = np.random.default_rng(Wr.shape[1])
    Wr[a] = (np.abs(rng.standard_normal(Wr.shape[1])) * 0.5 + 0.3).astype(np.float32)
    Wr[b] = Wr[a]
    Wr[b, j] = np.nextafter(Wr[a, j], np.float32(np.inf if up else -np.inf))


@pytest.mark.parametrize("H,E,T,K", [(256, 24, 40, 3), (1024, 24, 40, 3), (256, 64, 4096, 3),
                                     (320, 64, 33, 1), (320, 64, 33, 16), (256, 10, 40, 10)])
def test_route_sub_ulp_near_tie_exact_order(H, E, T, K):
    """Two router rows one ulp apart in one weight, met by the smallest fp16
    subnormal: their fp64 logits tie but the exact logits do not, and the
    top-K order must follow the exact ones ("PagedWeight" §2.1 ranks by the
    logits; the one-launch small-batch router, the vector logits path and the
    fp64 matrix-core path). The tokens of the other rows see a resolvable gap.
    K = 1 puts the tie between the winner and the runner-up, K = 16 fills
    every selection slot, E = K leaves no runner-up."""
    a, b, j = 5, 9, 17
    rng = np.random.default_rng(H + T + K)
    rows = _tie_rows(T, 8 if T > 64 else T)
    for up in (True, False):
        Wr = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
        _near_tie_rows(Wr, a, b, j, up)
        Xb = _near_tie_x(T, H, j, "f16", rows, rng)
        z, r, _ = O.route(S.f16_bits_to_f64(Xb), Wr, None, K)
        assert (z[:, 0] == (b if up else a)).all()
        if K > 1:
            assert (z[:, 1] == (a if up else b)).all()
        idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
        w = torch.empty((T, K), dtype=torch.float32, device="cuda")
        M().moe_route(to_dev_x(Xb), 0, torch.from_numpy(Wr).cuda(), None, K, idx, w, route_ws(T, E))
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        bad = int((got != z).any(axis=1).sum())
        say(f"H={H} E={E} T={T} ulp {'up' if up else 'down'}: {bad} of {T} tokens ordered differently")
        assert bad == 0
        assert_close(w.cpu().numpy(), r, "near-tie topk_w")


@pytest.mark.parametrize("H,E,T,K", [(256, 24, 40, 3), (1024, 24, 40, 4), (256, 64, 4096, 8), (64, 12, 9, 2)])
def test_route_non_finite_tokens(H, E, T, K):
    """Tokens holding an inf or a nan activation get K distinct expert ids in
    range (a nan logit ranks lowest, and such a token is ranked on its exact
    sums); the finite tokens of the same batch are routed as the oracle routes
    them (the vector, matrix-core and one-launch router paths)."""
    rng = np.random.default_rng(7 + H + T)
    Wr = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
    xa = rng.standard_normal((T, H)).astype(np.float16)
    bad = np.arange(0, T, 4)
    xa[bad[0::3], 5] = np.float16(np.inf)
    xa[bad[1::3], 7] = np.float16(-np.inf)
    xa[bad[2::3], 3] = np.float16(np.nan)
    Xb = np.ascontiguousarray(xa.view(np.uint16))
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    M().moe_route(to_dev_x(Xb), 0, torch.from_numpy(Wr).cuda(), None, K, idx, w, route_ws(T, E))
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert ((got >= 0) & (got < E)).all()
    assert all(len(set(row.tolist())) == K for row in got)
    good = np.setdiff1d(np.arange(T), bad)
    z, r, _ = O.route(S.f16_bits_to_f64(Xb[good]), Wr, None, K)
    assert np.array_equal(got[good], z)
    assert_close(w.cpu().numpy()[good], r, "finite tokens' topk_w")


@pytest.mark.parametrize("cfg", [10, 11])
def test_fused_non_finite_tokens_match_separate(cfg, layer_cache):
    """With inf and nan activations in some tokens, the one-launch path routes
    every token as moe_route does (ids and weights bit for bit, nan included)
    and gives the finite tokens the same outputs as moe_ffn."""
    L, D = dev_layer(layer_cache, cfg)
    xdt = L.cfg["xdtype"]
    Xb = np.array(S.make_tokens(cfg), copy=True)
    T = Xb.shape[0]
    bad = np.arange(1, T, 5)
    inf_bits, nan_bits = (0x7C00, 0x7E00) if xdt == "f16" else (0x7F80, 0x7FC0)
    Xb[bad[0::2], 3] = inf_bits
    Xb[bad[1::2], 6] = nan_bits
    i1, w1, o1, i2, w2, o2, _ = _separate_and_fused(D, Xb, xdt)
    assert ((i1 >= 0) & (i1 < L.E)).all()
    assert np.array_equal(i1, i2)
    assert np.array_equal(w1.view(np.uint32), w2.view(np.uint32))
    good = np.setdiff1d(np.arange(T), bad)
    assert np.isfinite(o1[good]).all()
    assert np.array_equal(o1[good].view(np.uint32), o2[good].view(np.uint32))


@pytest.mark.parametrize("cfg", [10, 11, 3])
def test_fused_sub_ulp_near_tie_exact_order(cfg, layer_cache):
    """The fused launch ranks near-tied experts by their exact logits too
    (router rows 1 and E-2, and their biases, equal but for one weight one ulp
    apart, met by the smallest subnormal activation in sampled tokens):
    vector-path logits in fp16 and in bf16, matrix-core logits with a bias."""
    L, D = dev_layer(layer_cache, cfg)
    H, E, K = D.H, D.E, D.K
    xdt = L.cfg["xdtype"]
    T = S.make_tokens(cfg).shape[0]
    rng = np.random.default_rng(4242 + cfg)
    a, b, j = 1, E - 2, 17
    Wr = np.array(L.W_r, np.float32, copy=True)
    _near_tie_rows(Wr, a, b, j, True)
    bias = None if L.bias is None else np.array(L.bias, np.float32, copy=True)
    if bias is not None:
        bias[b] = bias[a]
    Xb = _near_tie_x(T, H, j, xdt, _tie_rows(T, 8 if T > 64 else T), rng)
    z, r, _ = O.route(S.x_bits_to_f64(Xb, xdt), Wr, bias, K)
    assert (z[:, 0] == b).all()
    W0, b0 = D.W_r.clone(), None if D.bias is None else D.bias.clone()
    try:
        D.W_r.copy_(torch.from_numpy(Wr))
        if bias is not None:
            D.bias.copy_(torch.from_numpy(bias))
        say(f"fused near tie cfg{cfg}: T={T} H={H} E={E} K={K} {xdt}")
        i1, w1, _, i2, w2, _, _ = _separate_and_fused(D, Xb, xdt)
    finally:
        D.W_r.copy_(W0)
        if b0 is not None:
            D.bias.copy_(b0)
        torch.cuda.synchronize()
    assert int((i2 != z).any(axis=1).sum()) == 0, "fused order"
    assert int((i1 != z).any(axis=1).sum()) == 0, "separate order"
    assert_close(w2, r, f"cfg{cfg} near-tie fused topk_w")
    assert np.array_equal(w1.view(np.uint32), w2.view(np.uint32))

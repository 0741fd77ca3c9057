"""moe_ffn_static (the entry point for callers that cannot allocate) against
moe_ffn through the C ABI: two calls in a row on the same GPU, the second with
a smaller batch, each bit-identical to moe_ffn on the same inputs (the two
share their kernels; only the workspace differs). A batch whose workspace
exceeds the static array is refused on the host."""
import numpy as np
import pytest

import mpb_synth as S
from helpers import say, to_dev_x

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixed_precision_bit_amd  # noqa: F401


def _both(M, D, Xb, xdtype):
    xd = M.MPB_F16 if xdtype == "f16" else M.MPB_BF16
    X = to_dev_x(Xb)
    T = Xb.shape[0]
    idx, w = D.alloc_route(T)
    D.route(X, xdtype, idx, w)
    out, ws = D.alloc_ffn(T)
    M.moe_ffn(X, xd, idx, w, D.planes_table, D.luts_table, D.q_dev, out, ws)
    out_s = torch.full((T, D.H), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_ffn_static(X, xd, idx, w, D.planes_table, D.luts_table, D.q_dev, out_s)
    torch.cuda.synchronize()
    return out.cpu().numpy(), out_s.cpu().numpy()


@pytest.mark.parametrize("cfg,T1,T2", [(1, 64, 16), (10, 72, 9)])
def test_static_workspace_matches_moe_ffn(cfg, T1, T2):
    from mixed_precision_bit_amd import _lib as M
    from mixed_precision_bit_amd.layer import DeviceLayer
    L = S.make_layer(cfg)
    D = DeviceLayer.from_synth(L)
    Xb = S.make_tokens(cfg, T=T1)
    for T in (T1, T2):
        say(f"moe_ffn_static cfg{cfg} T={T}")
        ref, got = _both(M, D, Xb[:T], L.cfg["xdtype"])
        assert np.isfinite(got).all()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
            f"T={T}: {np.count_nonzero(got != ref)} elements differ"
    # a batch above the static limit is refused before anything is enqueued
    big = 4096 if cfg == 1 else 1 << 18
    X = torch.zeros((big, D.H), dtype=torch.int16, device="cuda")
    idx = torch.zeros((big, D.K), dtype=torch.int32, device="cuda")
    w = torch.zeros((big, D.K), dtype=torch.float32, device="cuda")
    out = torch.empty((big, D.H), dtype=torch.float32, device="cuda")
    with pytest.raises(M.MpbError) as ei:
        M.moe_ffn_static(X, M.MPB_F16, idx, w, D.planes_table, D.luts_table, D.q_dev, out)
    assert ei.value.code == -5 and "static scratch limit" in str(ei.value)
    torch.cuda.synchronize()

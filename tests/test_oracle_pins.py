"""Pins for the CPU oracle: each check ties the oracle to something other than
itself (the stored format, a library routine, a closed form, brute force, or
an invariant the PagedWeight pages state). CPU only."""
import math
import os

import numpy as np
import pytest
import scipy.special

import mpb_synth as S
import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def planes_to_codes(planes):
    """Codes from canonical planes via numpy's bit unpacking (library route)."""
    P, N, W = planes.shape
    codes = np.zeros((N, 32 * W), np.int64)
    for p in range(P):
        bits = np.unpackbits(np.ascontiguousarray(planes[p]).view(np.uint8), axis=1,
                             bitorder="little")
        codes |= bits.astype(np.int64) << (7 - p)
    return codes


def small_block(seed=7, N=64, Kd=128):
    return S.make_block(seed, 0, N, Kd)


# ---------------------------------------------------------------- P1 / P2
def test_p1_codes_planes_round_trip():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(48, 96), dtype=np.uint8)
    planes = S.codes_to_planes(codes)
    assert np.array_equal(O.unpack_indices(planes, 8), codes.astype(np.int64))
    assert np.array_equal(planes_to_codes(planes), codes.astype(np.int64))


@pytest.mark.parametrize("b", S.BITS)
def test_p2_index_is_top_b_bits(b):
    blk = small_block()
    codes = planes_to_codes(blk.planes)
    assert np.array_equal(O.unpack_indices(blk.planes, b), codes >> (8 - b))


def test_p2_single_element_msb_plane():
    # one set bit: element k=37 of row 3, plane 0 (the code MSB)
    planes = np.zeros((8, 4, 2), np.uint32)
    planes[0, 3, 1] = np.uint32(1 << 5)
    for b in S.BITS:
        idx = O.unpack_indices(planes, b)
        assert idx[3, 37] == 1 << (b - 1) and idx.sum() == 1 << (b - 1)
    assert O.unpack_index_scalar(planes, 3, 37, 8) == 128


# ---------------------------------------------------------------- P3
@pytest.mark.parametrize("b", S.BITS)
def test_p3_at_most_2b_values_per_row(b):
    blk = small_block(N=32, Kd=1024)
    W = O.dequant(blk.planes, blk.luts[b - 3], b)
    lut = blk.luts[b - 3].view(np.float16).astype(np.float64)
    for n in range(W.shape[0]):
        vals = np.unique(W[n])
        assert len(vals) <= 1 << b
        assert np.isin(vals, lut[n]).all()


def test_dequant_is_lut_of_code_prefix():
    blk = small_block()
    codes = planes_to_codes(blk.planes)
    for b in S.BITS:
        lut = blk.luts[b - 3].view(np.float16).astype(np.float64)
        ref = np.take_along_axis(lut, codes >> (8 - b), axis=1)
        assert np.array_equal(O.dequant(blk.planes, blk.luts[b - 3], b), ref)


# ---------------------------------------------------------------- P4
def test_p4_lowering_one_block_changes_only_it(layer_cache):
    L = layer_cache(0)
    X = S.x_bits_to_f64(S.make_tokens(0), "f16")
    z, r, _ = O.route(X, L.W_r, L.bias, L.K)
    base = O.moe_ffn(X, z, r, L)
    e = int(z[0, 0])
    for u in (0, 1):
        i = 2 * e + u
        q2 = L.q.copy()
        q2[i] = 3 if q2[i] != 3 else 4
        for j in range(L.n_blocks):
            if j != i:
                assert np.array_equal(O.dequant_block(L, j, int(q2[j])), O.dequant_block(L, j))
        out = O.moe_ffn(X, z, r, L, q=q2)
        routed = (z == e).any(axis=1)
        assert np.array_equal(out[~routed], base[~routed])
        assert not np.array_equal(out[routed], base[routed])


def test_p4_shared_block_changes_every_token(layer_cache):
    L = layer_cache(1)
    X = S.x_bits_to_f64(S.make_tokens(1, T=4), "f16")
    z, r, _ = O.route(X, L.W_r, L.bias, L.K)
    i = 2 * L.E + 1
    q2 = L.q.copy()
    q2[i] = 3 if q2[i] != 3 else 5
    a = O.moe_ffn_sampled(X, z, r, L, range(4), range(0, L.H, 97))
    b = O.moe_ffn_sampled(X, z, r, L, range(4), range(0, L.H, 97), q=q2)
    assert (np.abs(a - b) > 0).any(axis=1).all()


# ---------------------------------------------------------------- P5
@pytest.mark.parametrize("cfg", [0, 1])
def test_p5_routing_mass_sums_to_one(cfg, layer_cache):
    L = layer_cache(cfg)
    X = S.x_bits_to_f64(S.make_tokens(cfg), "f16")
    z, r, _ = O.route(X, L.W_r, L.bias, L.K)
    m = O.routing_mass(z, r, L.E)
    assert abs(m.sum() - 1.0) <= 1e-12 and (m >= 0).all()
    assert np.allclose(r.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    # the denominator of Eq. 1 is the token count when each token's weights sum to 1
    assert abs(r.sum() - X.shape[0]) <= 1e-9


# ---------------------------------------------------------------- P6
def test_p6_scalar_loops_match_vectorised(layer_cache):
    L = layer_cache(0)
    X = S.x_bits_to_f64(S.make_tokens(0), "f16")
    z, r, _ = O.route(X, L.W_r, L.bias, L.K)
    out = O.moe_ffn(X, z, r, L)
    toks = [0, 5]
    loops = np.array(O.moe_ffn_loops(X, z, r, L, toks))
    scale = np.abs(out[toks]).max()
    assert np.abs(loops - out[toks]).max() <= 1e-12 * scale


# ---------------------------------------------------------------- P7 special cases
def test_p7a_integer_lut_gives_integer_matmul():
    rng = np.random.default_rng(3)
    N, Kd = 64, 256
    codes = rng.integers(0, 256, size=(N, Kd), dtype=np.uint8)
    planes = S.codes_to_planes(codes)
    lut = np.tile(np.arange(256, dtype=np.float64) - 128, (N, 1)).astype(np.float16).view(np.uint16)
    W = O.dequant(planes, lut, 8)
    x = rng.integers(-4, 5, size=(5, Kd))
    a = np.asarray(x, np.float64) @ W.T
    ref = x.astype(np.int64) @ (codes.astype(np.int64) - 128).T
    assert np.array_equal(a, ref.astype(np.float64))


def test_p7b_constant_lut_row():
    blk = small_block(N=16, Kd=256)
    for b in (3, 6, 8):
        c = (np.arange(16) * 0.125 - 1.0)
        lut = np.repeat(c[:, None], 1 << b, axis=1).astype(np.float16).view(np.uint16)
        W = O.dequant(blk.planes, lut, b)
        x = np.random.default_rng(b).standard_normal(256)
        assert np.allclose(W @ x, c * x.sum(), rtol=1e-13, atol=1e-13)


def test_p7c_zero_router_ties_to_lowest_indices():
    X = np.random.default_rng(4).standard_normal((6, 64))
    for K in (1, 2, 5):
        z, r, _ = O.route(X, np.zeros((9, 64), np.float32), None, K)
        assert (z == np.arange(K)).all() and np.allclose(r, 1.0 / K)


def test_p7d_single_expert_is_dense_swiglu():
    rng = np.random.default_rng(5)
    H, I, T = 64, 32, 7
    cg = rng.integers(0, 256, size=(2 * I, H), dtype=np.uint8)
    cd = rng.integers(0, 256, size=(H, I), dtype=np.uint8)

    class L1:
        pass
    L = L1()
    L.H, L.I, L.E, L.S, L.K = H, I, 1, 0, 1
    L.q = np.array([5, 7], np.int32)
    lg = np.sort(rng.normal(0, 0.3, (2 * I, 32)), axis=1).astype(np.float16)
    ld = np.sort(rng.normal(0, 0.3, (H, 128)), axis=1).astype(np.float16)
    L.blocks = {0: S.Block(S.codes_to_planes(cg), [None, None, lg.view(np.uint16), None, None, None]),
                1: S.Block(S.codes_to_planes(cd), [None, None, None, None, ld.view(np.uint16), None])}
    X = rng.standard_normal((T, H))
    z, r, _ = O.route(X, np.ones((1, H), np.float32), None, 1)
    assert (z == 0).all() and np.allclose(r, 1)
    out = O.moe_ffn(X, z, r, L)
    Wg = np.take_along_axis(lg.astype(np.float64), cg.astype(np.int64) >> 3, axis=1)
    Wd = np.take_along_axis(ld.astype(np.float64), cd.astype(np.int64) >> 1, axis=1)
    a = X @ Wg.T
    g, u = a[:, :I], a[:, I:]
    ref = (g * scipy.special.expit(g) * u) @ Wd.T
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_p7e_zero_input_gives_zero(layer_cache):
    L = layer_cache(0)
    X = np.zeros((3, L.H))
    z, r, _ = O.route(X, L.W_r, L.bias, L.K)
    assert (O.moe_ffn(X, z, r, L) == 0).all()


# ---------------------------------------------------------------- routing vs library
@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_route_matches_full_softmax_then_renormalise(cfg, layer_cache):
    c = S.layer_config(cfg)
    L = layer_cache(0) if cfg == 0 else None
    rng = np.random.default_rng(cfg)
    E, H, K = c["E"], c["H"], c["K"]
    W = (rng.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32)
    bias = np.log(np.arange(1, E + 1) ** -1.1 / np.sum(np.arange(1, E + 1) ** -1.1)).astype(np.float32) \
        if c.get("bias") else None
    X = rng.standard_normal((32, H)).astype(np.float16).astype(np.float64)
    z, r, _ = O.route(X, W, bias, K)
    logits = X @ W.astype(np.float64).T + (0 if bias is None else bias.astype(np.float64))
    p = scipy.special.softmax(logits, axis=1)
    order = np.argsort(-p, axis=1, kind="stable")[:, :K]
    assert np.array_equal(z, order)
    pk = np.take_along_axis(p, order, axis=1)
    assert np.allclose(r, pk / pk.sum(axis=1, keepdims=True), rtol=1e-12, atol=0)
    del L


# ---------------------------------------------------------------- P8 ties
def test_p8_duplicate_router_rows_rank_lower_index_first():
    rng = np.random.default_rng(8)
    H, E, K = 128, 8, 3
    W = (rng.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32)
    W[5] = W[2]
    W[6] = W[2]
    X = rng.standard_normal((20, H)).astype(np.float16).astype(np.float64)
    z, _, _ = O.route(X, W, None, K)
    for t in range(20):
        pos = {e: j for j, e in enumerate(z[t])}
        present = [e for e in (2, 5, 6) if e in pos]
        assert [pos[e] for e in present] == sorted(pos[e] for e in present)
        if 5 in pos or 6 in pos:
            assert 2 in pos
        if 6 in pos:
            assert 5 in pos


def test_p8_near_tie_resolved_on_exact_logits():
    # rows 1 and 3 differ by one ulp in one weight: their float64 logits can
    # collide, the exact ones differ, and the larger exact logit must win
    H = 64
    rng = np.random.default_rng(9)
    W = np.zeros((4, H), np.float32)
    W[1] = np.abs(rng.standard_normal(H)).astype(np.float32)
    W[3] = W[1]
    W[3, 10] = np.nextafter(W[1, 10], np.float32(np.inf))
    X = np.abs(rng.standard_normal((1, H))).astype(np.float16).astype(np.float64)
    X[0, 10] = 1.0
    z, _, _ = O.route(X, W, None, 2)
    assert list(z[0]) == [3, 1]
    W[3, 10] = np.nextafter(W[1, 10], np.float32(-np.inf))
    z, _, _ = O.route(X, W, None, 2)
    assert list(z[0]) == [1, 3]


# ---------------------------------------------------------------- P9 bytes
def test_p9_block_bytes_equal_stored_arrays():
    blk = small_block(N=48, Kd=192)
    for b in S.BITS:
        stored = blk.planes[:b].nbytes + blk.luts[b - 3].nbytes
        assert O.block_bytes(48, 192, b) == stored
        for b2 in range(3, b):
            assert O.freed_bytes(48, 192, b, b2) == stored - blk.planes[:b2].nbytes - blk.luts[b2 - 3].nbytes


def test_p9_committed_bytes_difference_is_sum_of_deltas(layer_cache):
    L = layer_cache(1)
    s = S.make_sensitivity(4, L.n_blocks)
    red, _ = O.greedy_reductions(L, s, 0.25)
    q2 = L.q.copy()
    for i, b2 in red:
        q2[i] = b2
    d = sum(O.freed_bytes(*L.shape(i), int(L.q[i]), b2) for i, b2 in red)
    assert O.committed_bytes(L) - O.committed_bytes(L, q=q2) == d > 0


# ---------------------------------------------------------------- planner pieces
def test_eq4_eq8_damage():
    s = np.zeros((1, 9))
    s[0, 3:9] = [9, 5, 3, 2, 1, 0]
    assert O.global_damage(s, 0, 8, 5) == 3
    s2 = s.copy()
    s2[0, 5] = -1  # calibration noise: a lower bitwidth that scores better
    assert O.global_damage(s2, 0, 8, 5) == 0
    assert O.predicted_damage(0.0) == 1e-12
    assert O.predicted_damage(2.0, mu=3.0, eta=0.5) == 3.0


def test_greedy_sweep_properties(layer_cache):
    L = layer_cache(1)
    s = S.make_sensitivity(4, L.n_blocks)
    prev = set()
    for f in (0.25, 0.5, 0.75):
        red, short = O.greedy_reductions(L, s, f)
        chosen = {i for i, _ in red}
        assert prev <= chosen
        prev = chosen
        assert len(red) + short == math.ceil(f * 2 * L.E)
        for i, b2 in red:
            e = i // 2
            assert e < L.E
            assert (5 if L.hot[e] else 3) <= b2 < L.q[i]
    assert O.committed_bytes(L, q=np.full(L.n_blocks, 8)) > O.committed_bytes(L)


# ---------------------------------------------------------------- golden tables
def _table(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        if line.strip() and not line.startswith("#"):
            rows.append(line.split())
    return rows


def test_config_shapes_follow_table1():
    t1 = {r[0]: tuple(int(v) for v in r[1:]) for r in _table("table1_models.txt")}
    for cfg, model in ((1, "Qwen1.5-MoE-A2.7B"), (2, "Mixtral-8x7B-v0.1"), (3, "Gemma-4-26B-A4B")):
        c = S.CONFIGS[cfg]
        assert (c["E"], c["S"], c["K"]) == t1[model]


def test_headline_ratios_from_tables():
    t3 = _table("table3_throughput.txt")
    fp16 = [r for r in t3 if r[0] == "FP16"][0]
    uni = [r for r in t3 if r[0] == "Uniform"]
    pw = [r for r in t3 if r[0] == "PagedWeight"]
    assert round(float(pw[0][2]) / float(fp16[2]), 2) == 1.94
    drop1 = max(1 - float(p[2]) / float(u[2]) for p, u in zip(pw, uni))
    drop4 = max(1 - float(p[4]) / float(u[4]) for p, u in zip(pw, uni))
    assert round(100 * drop1, 1) == 3.3 and round(100 * drop4, 1) == 4.1
    t2 = {r[0]: (float(r[1]), float(r[2])) for r in _table("table2_longbench.txt")}
    assert t2["PagedWeight-10GB"][1] == t2["FP16"][1]
    assert round(100 * (1 - t2["PagedWeight-10GB"][0] / t2["FP16"][0]), 1) == 72.0
    assert round(100 * (t2["PagedWeight-10GB"][1] / t2["APL-3bit"][1] - 1), 1) == 39.3


# ---------------------------------------------------------------- generator
def test_generator_is_deterministic():
    a = S.make_layer(0)
    b = S.make_layer(0)
    for i in a.blocks:
        assert np.array_equal(a.blocks[i].planes, b.blocks[i].planes)
        for x, y in zip(a.blocks[i].luts, b.blocks[i].luts):
            assert np.array_equal(x, y)
    assert np.array_equal(S.make_tokens(3, T=8), S.make_tokens(3, T=8))
    assert np.array_equal(a.q, b.q) and np.array_equal(a.W_r, b.W_r)


def test_generator_recipe():
    L = S.make_layer(1, blocks=[0])
    assert L.q.min() >= 3 and L.q.max() <= 8 and L.hot.sum() == 12
    for e in np.nonzero(L.hot)[0]:
        assert L.q[2 * e] >= 5 and L.q[2 * e + 1] >= 5
    L2 = S.make_layer(2, blocks=[])
    assert (L2.q[0::2] == 4).all() and (L2.q[1::2] == 3).all()
    L3 = S.make_layer(3, blocks=[])
    p = np.exp(L3.bias.astype(np.float64))
    assert abs(p.sum() - 1) < 1e-5 and len(np.unique(L3.bias)) == 128
    bits = S.make_block(1, 0, 64, 4096).planes
    frac = np.unpackbits(bits.view(np.uint8)).mean()
    assert abs(frac - 0.5) < 0.01
    x = S.bf16_bits_to_f64(S.make_tokens(3, T=64))
    assert abs(x.std() - 1) < 0.05
    lut = S.make_block(2, 1, 512, 64).luts[5].view(np.float16).astype(np.float64)
    assert abs(lut.std() - 0.02) < 0.001 and (np.diff(lut, axis=1) >= 0).all()


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -9, -2.5e-3], np.float32)
    got = S.bf16_bits_to_f64(S.f32_to_bf16_bits(x))
    # neighbours of 1 in bf16 are 1 and 1+2^-7; halfway 1+2^-8 rounds to even (1.0)
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.0078125
    for v, g in zip(x, got):
        assert abs(g - v) <= abs(v) * 2 ** -8


# ---------------------------------------------------------------- Eq. 1 closed form
def test_routing_mass_closed_form_and_alignment():
    # [PW §2.1, Eq. 1] worked by hand: expert 0 gets .7 + .1, expert 1 gets
    # .4 + .9, expert 2 gets .3 + .6, over a total weight of 3
    z = np.array([[0, 2], [2, 1], [1, 0]])
    r = np.array([[.7, .3], [.6, .4], [.9, .1]])
    m = O.routing_mass(z, r, 3)
    assert np.allclose(m, [4 / 15, 13 / 30, 3 / 10], rtol=0, atol=1e-15)
    # a z/r misalignment (weights of the transposed entry order) moves the mass
    assert not np.allclose(O.routing_mass(z, r[:, ::-1], 3), m, rtol=0, atol=1e-6)
    # ids outside [0, E) name no routed expert: they leave both sums
    z2 = np.array([[0, -1], [2, 1], [1, 3]])
    r2 = np.array([[.7, .3], [.6, .4], [.9, .1]])
    assert np.allclose(O.routing_mass(z2, r2, 3), np.array([.7, 1.3, .6]) / 2.6, rtol=0, atol=1e-15)
    assert (O.routing_mass(np.full((2, 2), -1), np.ones((2, 2)), 3) == 0).all()
    assert (O.routing_mass(np.zeros((0, 2), np.int64), np.zeros((0, 2)), 3) == 0).all()


def test_routing_mass_brute_force_per_expert(layer_cache):
    # per-expert scalar loops over the (t, k) entries of a routed batch
    from fractions import Fraction
    L = layer_cache(1)
    X = S.x_bits_to_f64(S.make_tokens(1), "f16")
    z, r, _ = O.route(X, L.W_r, L.bias, L.K)
    m = O.routing_mass(z, r, L.E)
    tot = sum(Fraction(float(v)) for v in r.ravel())
    for e in range(L.E):
        num = sum((Fraction(float(r[t, k])) for t in range(z.shape[0]) for k in range(z.shape[1]) if z[t, k] == e),
                  Fraction(0))
        assert abs(m[e] - float(num / tot)) <= 1e-15


# ---------------------------------------------------------------- sampled FFN
@pytest.mark.parametrize("cfg", [0, 10, 13])
def test_moe_ffn_sampled_equals_full_layer(cfg, layer_cache):
    # the sampled evaluator is the full-size checker; hold it to moe_ffn (which
    # the scalar loops and the closed forms above pin) at every token and a
    # column sample that includes both ends
    L = layer_cache(cfg)
    Xb = S.make_tokens(cfg)
    X = S.x_bits_to_f64(Xb, L.cfg["xdtype"])
    z, r, _ = O.route(X, L.W_r, L.bias, L.K)
    full = O.moe_ffn(X, z, r, L)
    toks = np.arange(X.shape[0])
    cols = np.unique(np.r_[0, np.arange(1, L.H, 7), L.H - 1])
    samp = O.moe_ffn_sampled(X, z, r, L, toks, cols)
    scale = np.abs(full).max()
    assert np.abs(samp - full[np.ix_(toks, cols)]).max() <= 1e-12 * scale


def test_moe_ffn_sampled_equals_scalar_loops(layer_cache):
    L = layer_cache(0)
    X = S.x_bits_to_f64(S.make_tokens(0), "f16")
    z, r, _ = O.route(X, L.W_r, L.bias, L.K)
    loops = np.array(O.moe_ffn_loops(X, z, r, L, [3]))[0]
    cols = np.array([0, 17, 128, 255])
    samp = O.moe_ffn_sampled(X, z, r, L, [3], cols)[0]
    assert np.abs(samp - loops[cols]).max() <= 1e-12 * np.abs(loops).max()


# ---------------------------------------------------------------- greedy ranking
class _FakeLayer:
    """A layer stub carrying only what the greedy sweep reads."""

    def __init__(self, E, H, I, q, hot):
        self.E, self.S, self.H, self.I = E, 0, H, I
        self.q = np.array(q, np.int32)
        self.hot = np.array(hot, bool)
        self.n_blocks = 2 * E

    def shape(self, i):
        return (2 * self.I, self.H) if i % 2 == 0 else (self.H, self.I)


def test_greedy_reductions_hand_ranked():
    # [PW §3.2 "Planning objective"]: least predicted damage per released byte
    # first. Gate_up blocks are [64][64], down blocks [64][32], so by Eq. 3
    # M_gu^b = 512 b + 128 * 2^b and M_dn^b = 256 b + 128 * 2^b. Worked by hand:
    #   block 0 (q 8, floor 3): damage 8 - b'; best b' = 7, 1 / (36864 - 19968)
    #   block 1 (q 6, floor 3): damage .5/.6/10 at b' = 5/4/3; best b' = 4,
    #           0.6 / (9728 - 3072)
    #   block 2 (hot, q 6, floor 5): b' = 5 only, no damage: eps / 4608
    #   block 3 (hot, q 5 = floor): no candidate
    #   block 4 (q 4, floor 3): b' = 3, 0.2 / (4096 - 2560)
    #   block 5 (q 3 = floor): no candidate
    # ascending: 2 (2.2e-16), 0 (5.9e-5), 1 (9.0e-5), 4 (1.3e-4)
    L = _FakeLayer(3, 64, 32, [8, 6, 6, 5, 4, 3], [False, True, False])
    s = np.zeros((6, 9))
    s[0, 3:9] = [5, 4, 3, 2, 1, 0]
    s[1, 3:7] = [10, .6, .5, 0]
    s[4, 3:5] = [.2, 0]
    assert O.greedy_reductions(L, s, 0.25) == ([(2, 5), (0, 7)], 0)
    assert O.greedy_reductions(L, s, 0.50) == ([(2, 5), (0, 7), (1, 4)], 0)
    assert O.greedy_reductions(L, s, 0.75) == ([(2, 5), (0, 7), (1, 4), (4, 3)], 1)


def test_greedy_reductions_equal_scores_go_to_the_lower_block():
    L = _FakeLayer(2, 64, 32, [7, 3, 7, 3], [False, False])
    s = np.zeros((4, 9))
    s[0, 3:8] = [4, 3, 2, 1, 0]
    s[2] = s[0]
    assert O.greedy_reductions(L, s, 0.25) == ([(0, 6)], 0)
    assert O.greedy_reductions(L, s, 0.50) == ([(0, 6), (2, 6)], 0)


def test_greedy_reductions_against_enumeration(layer_cache):
    # every (block, b') pair of the config-1 layer enumerated: each chosen
    # block takes its least-score b', and no unchosen candidate scores below
    # a chosen one (so a reversed ranking fails)
    L = layer_cache(1)
    s = S.make_sensitivity(4, L.n_blocks)
    pairs = {}
    for i in range(2 * L.E):
        fl = 5 if L.hot[i // 2] else 3
        N, Kd = L.shape(i)
        for b2 in range(fl, int(L.q[i])):
            d = max(1e-12, max(s[i, b2] - s[i, int(L.q[i])], 0.0))
            pairs[(i, b2)] = d / (N * Kd * (int(L.q[i]) - b2) / 8 + N * (2 ** int(L.q[i]) - 2 ** b2) * 2)
    best = {}
    for (i, b2), sc in pairs.items():
        if i not in best or sc < best[i][0]:
            best[i] = (sc, b2)
    red, short = O.greedy_reductions(L, s, 0.5)
    chosen = {i for i, _ in red}
    assert short == 0 and len(red) == math.ceil(0.5 * 2 * L.E)
    for i, b2 in red:
        assert b2 == best[i][1]
    worst_in = max(best[i][0] for i in chosen)
    assert all(best[i][0] >= worst_in for i in best if i not in chosen)
    assert [i for i, _ in red] == sorted(chosen, key=lambda i: (best[i][0], i))

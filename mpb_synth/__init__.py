"""Seeded synthetic inputs for the mixed-precision MoE layer.

This module is shared by the tests, the benchmark and the smoke check. It holds
only input generation: random draws, rounding of those draws to the storage
dtypes, and the storage format of the Any-Precision weights (8-bit codes kept as
8 bit-planes). It performs none of the layer's arithmetic (no unpacking, no
lookup, no routing, no FFN); both the HIP path and the CPU oracle consume the
arrays it returns.

Storage format produced here (the canonical interchange format):

* ``planes[p][n][w]`` (uint32): plane 0 holds the most significant code bit
  (bit 7), plane 7 the least significant. Bit j of word w is the bit of element
  ``k = 32*w + j`` (least significant bit first), as in the Any-Precision
  bit-plane layout of PagedWeight §2.2 / §3.1, where a b-bit weight is read
  from a prefix of the planes.
* ``luts[b-3]`` (uint16, fp16 bits), shape ``[N][2**b]`` for b = 3..8: one
  centroid table per output row and bitwidth, sorted ascending.

Linear-blocks are numbered ``i = 2*e + u`` with u = 0 for gate_up (``[2I, H]``,
rows 0..I-1 gate, I..2I-1 up) and u = 1 for down (``[H, I]``); routed experts
0..E-1 come first, shared experts E..E+S-1 after them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BITS = tuple(range(3, 9))  # supported bitwidths B_i for every linear-block

# Workloads shaped like the evaluated models (PagedWeight §4, Table 1): the
# expert counts and top-K come from Table 1; hidden and intermediate sizes are
# the ones of the synthetic layers below.
CONFIGS = {
    0: dict(name="tiny", H=256, I=128, E=8, S=0, K=2, T=16, xdtype="f16",
            q_mode="uniform", bias=False, seed=1000),
    1: dict(name="qwen15moe_decode", H=2048, I=1408, E=60, S=4, K=4, T=64,
            xdtype="f16", q_mode="hot_floor", bias=False, seed=1001,
            hot_frac=0.2, hot_floor=5, zipf=1.1),
    2: dict(name="mixtral_decode", H=4096, I=14336, E=8, S=0, K=2, T=128,
            xdtype="f16", q_mode="fixed", q_gate_up=4, q_down=3, bias=False,
            seed=1002),
    3: dict(name="gemma4_prefill", H=2816, I=704, E=128, S=1, K=8, T=4096,
            xdtype="bf16", q_mode="uniform", bias=True, seed=1003, zipf=1.1),
    # the config-1 layer driven with 256 decode tokens through bitwidth states
    4: dict(name="qwen15moe_bitsweep", layer_of=1, T=256, xdtype="f16",
            seed=1004),
    # parity-only shapes: ragged row tiles (I % 128 != 0, H % 128 != 0), a
    # ragged token chunk, shared experts, and many empty experts
    10: dict(name="ragged_small", H=384, I=320, E=12, S=2, K=3, T=72, xdtype="f16",
             q_mode="uniform", bias=False, seed=1010),
    11: dict(name="sparse_bf16", H=192, I=192, E=40, S=0, K=1, T=9, xdtype="bf16",
             q_mode="uniform", bias=True, seed=1011, zipf=1.1),
    # parity-only extremes: the smallest dimensions (one half-chunk of K, one
    # row tile) with a single expert; more shared than routed experts; the
    # largest top-K; the largest expert count with one token
    12: dict(name="minimal", H=64, I=64, E=1, S=0, K=1, T=5, xdtype="f16",
             q_mode="uniform", bias=False, seed=1012),
    13: dict(name="shared_heavy", H=128, I=192, E=2, S=3, K=2, T=40, xdtype="bf16",
             q_mode="uniform", bias=True, seed=1013, zipf=1.1),
    14: dict(name="top16", H=320, I=128, E=64, S=0, K=16, T=33, xdtype="f16",
             q_mode="uniform", bias=False, seed=1014),
    15: dict(name="e512_one_token", H=64, I=64, E=512, S=0, K=8, T=1, xdtype="f16",
             q_mode="uniform", bias=False, seed=1015),
    # parity-only: few long items, so the down projection is split over K
    # ranges (49 half-chunks of 64 in three ranges, the last one odd)
    16: dict(name="split_k", H=192, I=3136, E=3, S=1, K=2, T=6, xdtype="f16",
             q_mode="uniform", bias=False, seed=1016),
}

LUT_STD = 0.02  # centroid draws ~ N(0, 0.02)

# SeedSequence stream ids
_S_TOKENS, _S_ROUTER, _S_BIAS, _S_Q, _S_HOT, _S_SENS, _S_PLAN = 1, 2, 3, 4, 5, 6, 7
_S_BLOCK = 100


def _rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *stream])))


def layer_config(cfg_id: int) -> dict:
    """The layer-defining config (config 4 reuses config 1's layer)."""
    c = CONFIGS[cfg_id]
    if "layer_of" in c:
        base = dict(CONFIGS[c["layer_of"]])
        base.update(T=c["T"], name=c["name"], token_seed=c["seed"])
        return base
    c = dict(c)
    c["token_seed"] = c["seed"]
    return c


def block_shape(H: int, I: int, i: int) -> tuple:
    """(N rows, Kd reduction) of linear-block i."""
    return (2 * I, H) if i % 2 == 0 else (H, I)


# ---------------------------------------------------------------- dtype helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def x_bits_to_f64(bits: np.ndarray, xdtype: str) -> np.ndarray:
    return f16_bits_to_f64(bits) if xdtype == "f16" else bf16_bits_to_f64(bits)


# ---------------------------------------------------------------- weight format
def codes_to_planes(codes: np.ndarray) -> np.ndarray:
    """8-bit codes [N][Kd] -> canonical planes [8][N][Kd/32] uint32 (format above)."""
    N, Kd = codes.shape
    assert Kd % 32 == 0
    out = np.empty((8, N, Kd // 32), dtype=np.uint32)
    for p in range(8):
        bits = (codes >> np.uint8(7 - p)) & np.uint8(1)
        packed = np.packbits(bits, axis=1, bitorder="little")  # [N][Kd/8] bytes
        out[p] = np.ascontiguousarray(packed).view("<u4")
    return out


@dataclasses.dataclass
class Block:
    planes: np.ndarray            # [8][N][Kd/32] uint32
    luts: list                    # 6 arrays [N][2**b] uint16 (fp16 bits), b = 3..8


def make_block(seed: int, i: int, N: int, Kd: int) -> Block:
    """Draw linear-block i: uniform 8-bit codes, stored as their 8 bit-planes.

    Uniform 8-bit codes are exactly 8 independent fair bits, so the plane words
    are drawn directly as uniform 32-bit integers (bit j of plane p's word w is
    bit 7-p of the code of element 32*w + j).
    """
    assert Kd % 32 == 0
    g = _rng(seed, _S_BLOCK, i)
    planes = g.integers(0, 1 << 32, size=(8, N, Kd // 32), dtype=np.uint32)
    luts = []
    for b in BITS:
        v = g.standard_normal(size=(N, 1 << b), dtype=np.float32) * np.float32(LUT_STD)
        v.sort(axis=1)  # rounding to fp16 is monotone, so the fp16 rows stay sorted
        luts.append(np.ascontiguousarray(v.astype(np.float16)).view(np.uint16))
    return Block(planes, luts)


def zipf_order(seed: int, stream: int, E: int) -> np.ndarray:
    """A seeded permutation: order[r] is the expert holding rank r+1."""
    return _rng(seed, stream).permutation(E)


@dataclasses.dataclass
class Layer:
    cfg: dict
    H: int
    I: int
    E: int
    S: int
    K: int
    W_r: np.ndarray               # [E][H] float32
    bias: Optional[np.ndarray]    # [E] float32 or None
    q: np.ndarray                 # [2(E+S)] int32 committed bitwidths
    hot: np.ndarray               # [E] bool (hot routing bucket), all False if unused
    blocks: dict                  # i -> Block (possibly a subset)

    @property
    def n_blocks(self) -> int:
        return 2 * (self.E + self.S)

    def shape(self, i: int) -> tuple:
        return block_shape(self.H, self.I, i)


def make_layer(cfg_id: int, blocks=None, seed=None) -> Layer:
    """Generate the layer of a config. ``blocks`` limits which blocks are built."""
    c = layer_config(cfg_id)
    seed = c["seed"] if seed is None else seed
    H, I, E, S, K = c["H"], c["I"], c["E"], c["S"], c["K"]
    nb = 2 * (E + S)
    W_r = (_rng(seed, _S_ROUTER).standard_normal((E, H)) / math.sqrt(H)).astype(np.float32)
    bias = None
    if c.get("bias"):
        order = zipf_order(seed, _S_BIAS, E)
        rank = np.empty(E, np.int64)
        rank[order] = np.arange(1, E + 1)
        p = rank.astype(np.float64) ** (-c["zipf"])
        p /= p.sum()
        bias = np.log(p).astype(np.float32)
    hot = np.zeros(E, dtype=bool)
    mode = c["q_mode"]
    if mode == "fixed":
        q = np.array([c["q_gate_up"], c["q_down"]] * (E + S), dtype=np.int32)
    else:
        q = _rng(seed, _S_Q).integers(3, 9, size=nb).astype(np.int32)
        if mode == "hot_floor":
            order = zipf_order(seed, _S_HOT, E)   # Zipf(1.1) mass decreases with rank
            n_hot = int(round(c["hot_frac"] * E))
            hot[order[:n_hot]] = True
            for e in np.nonzero(hot)[0]:
                q[2 * e] = max(q[2 * e], c["hot_floor"])
                q[2 * e + 1] = max(q[2 * e + 1], c["hot_floor"])
    ids = range(nb) if blocks is None else blocks
    blk = {}
    for i in ids:
        N, Kd = block_shape(H, I, i)
        blk[i] = make_block(seed, i, N, Kd)
    return Layer(c, H, I, E, S, K, W_r, bias, q, hot, blk)


def make_tokens(cfg_id: int, T: Optional[int] = None, seed=None) -> np.ndarray:
    """Activations X [T][H] as raw 16-bit storage (fp16 or bf16 bits)."""
    c = layer_config(cfg_id)
    T = c["T"] if T is None else T
    seed = c["token_seed"] if seed is None else seed
    x = _rng(seed, _S_TOKENS).standard_normal((T, c["H"]))
    if c["xdtype"] == "f16":
        return x.astype(np.float16).view(np.uint16)
    return f32_to_bf16_bits(x.astype(np.float32))


def make_sensitivity(cfg_id: int, n_blocks: int, seed=None) -> np.ndarray:
    """Synthetic sensitivity s_i^b, [n_blocks][9] (columns b = 3..8 used).

    s_i^8 = 0 and s_i^b = s_i^(b+1) + Exp(1): the damage score grows as the
    bitwidth falls (stands in for the calibrated Hessian scores of §2.2, Eq. 2).
    """
    c = layer_config(cfg_id)
    seed = c["token_seed"] if seed is None else seed
    d = _rng(seed, _S_SENS).exponential(1.0, size=(n_blocks, 5))
    s = np.zeros((n_blocks, 9))
    for j, b in enumerate(range(7, 2, -1)):
        s[:, b] = s[:, b + 1] + d[:, j]
    return s


def make_planner_inputs(cfg_id: int, n_blocks: int, F_blk: int, seed=None, P_blk: int = 0):
    """Synthetic planner observations and calibration results (stand-ins for
    the offline tables and runtime signals of §3.2).

    Returns (P, phi): P holds three routing buckets (hot 20% / next 30% / the
    rest with damage multipliers 4 / 2 / 1 and floors 5 / 4 / 3 bits), four
    bitwidth-floor stages 6, 5, 4, 3, prompt-residual heads with N(0, 0.3)
    weights and offsets and U(0.5, 1) confidences, alpha = 0.5, clip range
    [-1, 1], eps = 1e-12, a free-block threshold of 64 blocks, the given free
    and pending block counts, and a KV block of 16 tokens (K and V, fp16, H
    wide); phi [n_blocks][3] holds positive routed-input features (mean norm,
    RMS norm >= mean, max norm >= RMS) around 1.
    """
    c = layer_config(cfg_id)
    seed = c["token_seed"] if seed is None else seed
    g = _rng(seed, _S_PLAN)
    P = {"bucket_frac": [0.2, 0.5, 1.0], "mu": [4.0, 2.0, 1.0], "floor": [5, 4, 3],
         "stage_floor": [6, 5, 4, 3], "eps": 1e-12, "alpha": 0.5, "rho_min": -1.0, "rho_max": 1.0,
         "head_w": g.normal(0.0, 0.3, size=(2, 5, 3)).tolist(),
         "head_a": g.normal(0.0, 0.3, size=(2, 5)).tolist(),
         "head_c": g.uniform(0.5, 1.0, size=(2, 5)).tolist(),
         "T_blk": 64, "F_blk": int(F_blk), "P_blk": int(P_blk), "B_kv": 16 * 2 * c["H"] * 2}
    mean = g.uniform(0.8, 1.2, size=n_blocks)
    rms = mean * g.uniform(1.0, 1.2, size=n_blocks)
    mx = rms * g.uniform(1.2, 2.0, size=n_blocks)
    phi = np.stack([mean, rms, mx], axis=1)
    return P, phi

"""CPU oracle for the fused mixed-precision MoE layer of PagedWeight.

TEST INFRASTRUCTURE ONLY. This is the plain, slow, obviously correct reference
the HIP path is checked against. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the library and its
Python binding never do. It shares no code with the HIP path: it reads the
canonical storage produced by ``mpb_synth`` and nothing else.

Source: "PagedWeight: Efficient MoE LLM Serving with Dynamic Quality-Aware
Weight Quantization" (arXiv 2607.16184), cited below as [PW §x].

Arithmetic is float64 throughout. Every input value (fp16/bf16 activations,
fp32 router weights, fp16 centroids) is exactly representable in float64, and
every product of an activation with a router weight is exact in float64.

Readings where the pages leave a step open:
* bit j of plane word w belongs to element 32*w + j; plane 0 is the code MSB;
* the b-bit index is formed from the top b planes ([PW §2.2]: subsets of the
  bit-planes give the effective bitwidths);
* one centroid table per output row and bitwidth;
* the expert activation is SwiGLU, SiLU(gate) * up, gate rows first;
* routing: softmax over all experts, top-K with ties to the lowest expert
  index (ties decided on exact logits), renormalised over the K winners;
* shared experts are always on with weight 1;
* M_i^b counts the b planes plus the b-bit table only ([PW §3.1], Eq. 3).

Parity pins: tests/test_oracle_pins.py and tests/test_planner.py. Every
function here is pinned by at least one check that does not re-run it.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

BITS = tuple(range(3, 9))


# ----------------------------------------------------------------- O1 / O2
def unpack_indices(planes: np.ndarray, b: int) -> np.ndarray:
    """b-bit centroid indices from the top b bit-planes [PW §2.2, §3.1].

    idx[n][k] = sum_{p<b} bit_p(n, k) * 2**(b-1-p), where bit_p(n, k) is bit
    j = k mod 32 of word k//32 of plane p (evaluated for all j at once by
    broadcasting the 32 shifts).  planes: [>=b][N][W] uint32.
    """
    assert 3 <= b <= 8
    _, N, W = planes.shape
    j = np.arange(32, dtype=np.uint32)
    idx = np.zeros((N, W, 32), dtype=np.uint8)
    for p in range(b):
        bit = ((planes[p][:, :, None] >> j) & np.uint32(1)).astype(np.uint8)
        idx |= bit << np.uint8(b - 1 - p)
    return idx.reshape(N, 32 * W)


def dequant(planes: np.ndarray, lut_bits: np.ndarray, b: int) -> np.ndarray:
    """Dequantised weights W^[n][k] = LUT_b[n][idx_b[n][k]] in float64 [PW §2.2].

    lut_bits: [N][2**b] uint16 holding fp16 centroids of bitwidth b.
    """
    idx = unpack_indices(planes, b)
    lut = np.ascontiguousarray(lut_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    assert lut.shape == (planes.shape[1], 1 << b)
    return lut[np.arange(lut.shape[0])[:, None], idx]


def dequant_block(layer, i: int, b: int = None, rows=None) -> np.ndarray:
    """Dequantise linear-block i of an mpb_synth Layer at bitwidth b (default q_i)."""
    b = int(layer.q[i]) if b is None else b
    blk = layer.blocks[i]
    planes = blk.planes if rows is None else blk.planes[:, rows]
    lut = blk.luts[b - 3] if rows is None else blk.luts[b - 3][rows]
    return dequant(planes, lut, b)


# ----------------------------------------------------------------- O3 routing
_U = 2.0 ** -53


def router_logits(X: np.ndarray, W_r: np.ndarray, bias=None):
    """Router logits l = X W_r^T (+ bias) in float64 [PW §2.1], with an error bound.

    Returns (logits [T][E], bound [T][E]) where |logit - exact| <= bound.
    The bound is gamma_{H+1} * (sum_h |x_h w_eh| + |bias_e|) with a safety factor.
    """
    X = np.asarray(X, np.float64)
    W = np.asarray(W_r, np.float64)
    H = X.shape[1]
    L = X @ W.T
    A = np.abs(X) @ np.abs(W).T
    if bias is not None:
        b = np.asarray(bias, np.float64)
        L = L + b[None, :]
        A = A + np.abs(b)[None, :]
    g = (H + 2) * _U / (1 - (H + 2) * _U)
    return L, 2.0 * g * A + 1e-300


def _exact_logits(x: np.ndarray, W: np.ndarray, bias) -> list:
    """Exact rational logits for one token (every fp value is a dyadic rational)."""
    xs = [Fraction(float(v)) for v in x]
    out = []
    for e in range(W.shape[0]):
        s = sum((xs[h] * Fraction(float(W[e, h])) for h in range(len(xs))), Fraction(0))
        if bias is not None:
            s += Fraction(float(bias[e]))
        out.append(s)
    return out


def route(X: np.ndarray, W_r: np.ndarray, bias, K: int):
    """Top-K routing [PW §2.1]: softmax over all E experts, top-K, renormalise.

    The top-K order is the order of the exact logits, ties going to the lower
    expert index. Softmax is strictly increasing, so ranking probabilities and
    ranking logits agree; renormalising the top-K probabilities equals a softmax
    over the K winning logits (the full denominator cancels).
    Where the float64 logits cannot certify the order (a gap within the
    rounding bound), the token is re-ranked on exact rational logits.

    Returns z [T][K] int64 (descending), r [T][K] float64, logits [T][E].
    """
    X = np.asarray(X, np.float64)
    W = np.asarray(W_r, np.float64)
    T, E = X.shape[0], W.shape[0]
    assert 1 <= K <= E
    L, B = router_logits(X, W, bias)
    z = np.zeros((T, K), np.int64)
    r = np.zeros((T, K), np.float64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -L[t]))       # by (-logit, index)
        lo = L[t][order] - B[t][order]
        hi = L[t][order] + B[t][order]
        certified = all(lo[j] > hi[j + 1] for j in range(K - 1))
        if certified and K < E:
            certified = lo[K - 1] > hi[K:].max()
        if not certified:
            ex = _exact_logits(X[t], W, bias)
            order = np.array(sorted(range(E), key=lambda e: (-ex[e], e)))
        top = order[:K]
        z[t] = top
        lt = L[t][top]
        p = np.exp(lt - lt.max())
        r[t] = p / p.sum()
    return z, r, L


def routing_mass(z: np.ndarray, r: np.ndarray, E: int) -> np.ndarray:
    """Routing mass m_e of one layer [PW §2.1, Eq. 1]: sum_t sum_k r 1{z=e} / sum r.

    Both sums run over the (t, k) entries whose expert id lies in [0, E)
    (an id outside that range names no routed expert and carries no mass);
    a batch with no such entry has zero mass everywhere.
    """
    z = np.asarray(z).ravel()
    r = np.asarray(r, np.float64).ravel()
    keep = (z >= 0) & (z < E)
    num = np.zeros(E)
    np.add.at(num, z[keep], r[keep])
    den = r[keep].sum()
    return num / den if den > 0 else num


# ----------------------------------------------------------------- O4 FFN
def silu(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_ffn(Xe: np.ndarray, W_gu: np.ndarray, W_dn: np.ndarray) -> np.ndarray:
    """One expert on its tokens: gate_up, SiLU(gate)*up, down [PW §3.3].

    Xe [n][H]; W_gu [2I][H] (gate rows then up rows); W_dn [H][I] -> [n][H].
    """
    I = W_dn.shape[1]
    a = Xe @ W_gu.T
    h = silu(a[:, :I]) * a[:, I:]
    return h @ W_dn.T


def groups(z: np.ndarray, r: np.ndarray, E: int, S: int, T: int):
    """Token groups per expert: routed expert e gets its (t, r) pairs, each
    shared expert gets every token with weight 1."""
    for e in range(E + S):
        if e < E:
            rows, ks = np.nonzero(z == e)
            yield e, rows, r[rows, ks]
        else:
            yield e, np.arange(T), np.ones(T)


def moe_ffn(X: np.ndarray, z: np.ndarray, r: np.ndarray, layer, q=None, wcache=None) -> np.ndarray:
    """MoE layer output [PW §3.3]: out[t] = sum_k r_tk FFN_{z_tk}(x_t) + sum_s FFN_s(x_t).

    Weights are dequantised at each block's committed bitwidth q_i.
    """
    X = np.asarray(X, np.float64)
    T = X.shape[0]
    q = layer.q if q is None else q
    out = np.zeros((T, layer.H))
    for e, rows, w in groups(z, r, layer.E, layer.S, T):
        if len(rows) == 0:
            continue
        Wg = _weights(layer, 2 * e, int(q[2 * e]), wcache)
        Wd = _weights(layer, 2 * e + 1, int(q[2 * e + 1]), wcache)
        out[rows] += w[:, None] * expert_ffn(X[rows], Wg, Wd)
    return out


def moe_ffn_sampled(X, z, r, layer, tokens, cols, q=None) -> np.ndarray:
    """out[t][c] for t in tokens, c in cols (same definition as moe_ffn), for
    layers too large to dequantise whole: only the touched experts' gate_up
    blocks and the sampled rows of their down blocks are expanded, and each
    expert runs on the sampled tokens routed to it at once."""
    X = np.asarray(X, np.float64)
    q = layer.q if q is None else q
    tokens = np.asarray(tokens)
    cols = np.asarray(cols)
    out = np.zeros((len(tokens), len(cols)))
    for e in range(layer.E + layer.S):
        if e >= layer.E:
            js, ws = np.arange(len(tokens)), np.ones(len(tokens))
        else:
            js, ks = np.nonzero(z[tokens] == e)
            ws = r[tokens[js], ks]
        if len(js) == 0:
            continue
        Wg = dequant_block(layer, 2 * e, int(q[2 * e]))
        Wd = dequant_block(layer, 2 * e + 1, int(q[2 * e + 1]), rows=cols)
        out[js] += ws[:, None] * expert_ffn(X[tokens[js]], Wg, Wd)
        del Wg
    return out


def _weights(layer, i, b, wcache):
    if wcache is None:
        return dequant_block(layer, i, b)
    key = (i, b)
    if key not in wcache:
        wcache[key] = dequant_block(layer, i, b)
    return wcache[key]


# ----------------------------------------------------------------- byte table
def block_bytes(N: int, Kd: int, b: int) -> int:
    """M_i^b [PW §3.1]: GPU bytes of block i at b bits = b planes + the b-bit LUT."""
    return N * Kd * b // 8 + N * (1 << b) * 2


def freed_bytes(N: int, Kd: int, b: int, b2: int) -> int:
    """Delta_i^{b->b'} = M_i^b - M_i^b' for b' < b [PW §3.1, Eq. 3]."""
    assert b2 < b
    return block_bytes(N, Kd, b) - block_bytes(N, Kd, b2)


def committed_bytes(layer, q=None, touched=None) -> int:
    """sum_i M_i^{q_i}, optionally over the touched blocks only."""
    q = layer.q if q is None else q
    tot = 0
    for i in range(layer.n_blocks):
        if touched is not None and not touched[i]:
            continue
        N, Kd = layer.shape(i)
        tot += block_bytes(N, Kd, int(q[i]))
    return tot


# ----------------------------------------------------------------- planner pieces
def global_damage(s: np.ndarray, i: int, b: int, b2: int) -> float:
    """g_i^{b->b'} = max{s_i^b' - s_i^b, 0} [PW §3.2, Eq. 4]."""
    return max(s[i, b2] - s[i, b], 0.0)


def predicted_damage(g: float, mu: float = 1.0, eta: float = 1.0, eps: float = 1e-12) -> float:
    """d^ = max{eps, mu g eta} [PW §3.2, Eq. 8]."""
    return max(eps, mu * g * eta)


def greedy_reductions(layer, s: np.ndarray, frac: float, floor_hot: int = 5, eps: float = 1e-12):
    """Choose bitwidth reductions by predicted damage per released byte [PW §3.2,
    'Planning objective'], restricted to a block-count target.

    Candidates are routed blocks above their floor (3 bits, or floor_hot for
    blocks of hot-bucket experts, [PW §3.2 'Routing statistics']). Each block
    keeps its cheapest legal b' (score d^/Delta), blocks are ranked ascending
    (ties to the lower i), and the first ceil(frac * #routed blocks) are taken.
    Returns (list of (i, b'), shortfall).
    """
    q0 = layer.q
    cands = []
    for i in range(2 * layer.E):
        e = i // 2
        fl = floor_hot if layer.hot[e] else 3
        b = int(q0[i])
        if b <= fl:
            continue
        N, Kd = layer.shape(i)
        best = None
        for b2 in range(fl, b):
            sc = predicted_damage(global_damage(s, i, b, b2), eps=eps) / freed_bytes(N, Kd, b, b2)
            if best is None or sc < best[0]:
                best = (sc, b2)
        cands.append((best[0], i, best[1]))
    cands.sort(key=lambda c: (c[0], c[1]))
    want = math.ceil(frac * 2 * layer.E)
    take = cands[:want]
    return [(i, b2) for _, i, b2 in take], max(0, want - len(take))


# ----------------------------------------------------------------- planner step (Alg. 1)
# Readings where [PW §3.2] leaves a step open:
# * a step is a one-bit reduction b -> b-1 of one routed linear-block; a
#   block's steps are taken in order, so only its next step is available;
# * GreedySelect repeatedly takes the available step with the least predicted
#   damage per released byte (ties to the lower block index) until the
#   released bytes reach D;
# * the bitwidth-floor stages are global floors, highest first; a block's
#   floor in stage s is the larger of the stage floor and its bucket's floor;
#   relaxing the depth cap means moving to the next stage;
# * RefreshPlanQueue keeps the newest plan of each stage; SelectBestPlan takes
#   the first stage whose plan meets D, else the plan that releases the most
#   bytes (the largest safe reduction), ties to the earlier stage;
# * PressureTriggered means the current free-block count is at or below the
#   threshold; D uses the free count after the pending KV growth;
# * routing buckets split the experts, sorted by routing mass (descending,
#   ties to the lower expert index), at ceil(frac * E) boundaries;
# * only routed blocks whose pages may move are candidates; shared experts'
#   blocks never change.


def kv_target_bytes(T_blk: int, F_blk: int, B_kv: int) -> int:
    """D = max{0, T_blk + 1 - F_blk} * B_KV [PW §3.2, Eq. 7]."""
    return max(0, T_blk + 1 - F_blk) * B_kv


def prompt_residual(w, a: float, phi) -> float:
    """rho^ = w . phi + a, summed left to right [PW §3.2, Eq. 5]."""
    acc = 0.0
    for wj, pj in zip(w, phi):
        acc = acc + wj * pj
    return acc + a


def residual_multiplier(rho_hat: float, alpha: float, c: float, rho_min: float, rho_max: float) -> float:
    """eta = exp(alpha c clip(rho^, rho_min, rho_max)) [PW §3.2, Eq. 6]."""
    clipped = min(max(rho_hat, rho_min), rho_max)
    return math.exp(alpha * c * clipped)


def routing_buckets(mass: np.ndarray, fracs) -> np.ndarray:
    """Bucket of every expert [PW §3.2 'Routing statistics']: experts sorted by
    routing mass (hottest first, ties to the lower index); bucket k holds the
    ranks from ceil(fracs[k-1] E) up to ceil(fracs[k] E)."""
    E = len(mass)
    order = sorted(range(E), key=lambda e: (-mass[e], e))
    bucket = np.zeros(E, dtype=np.int64)
    lo = 0
    for k, f in enumerate(fracs):
        hi = min(E, math.ceil(f * E))
        for rank in range(lo, hi):
            bucket[order[rank]] = k
        lo = max(lo, hi)
    return bucket


def _step_damage(P, s, phi, i, b, bucket_mu):
    """d^ of the one-bit step (i, b -> b-1): Eq. 4, 5, 6 and 8."""
    u = i % 2
    t = b - 4                    # transition b -> b-1, b = 4..8
    g = max(s[i][b - 1] - s[i][b], 0.0)                                   # Eq. 4
    rho = prompt_residual(P["head_w"][u][t], P["head_a"][u][t], phi[i])  # Eq. 5
    eta = residual_multiplier(rho, P["alpha"], P["head_c"][u][t], P["rho_min"], P["rho_max"])  # Eq. 6
    return max(P["eps"], bucket_mu * g * eta)                              # Eq. 8


def plan_step(H, I, E, S, q, movable, s, mass, phi, P):
    """One planner step [PW §3.2, Algorithm 1] on a layer with E routed and S
    shared experts (block 2e+u: gate_up [2I][H] for u = 0, down [H][I]).

    q: committed bitwidths; movable: per block, whether its pages may move now
    (None = all); s: [n_blocks][9] sensitivity s_i^b (columns 3..8); mass: [E]
    routing mass (Eq. 1); phi: [n_blocks][3] routed-input features; P: the
    planner's parameters (buckets, stages, heads, Eq. 6 and 7 constants).
    Returns (plan, summary, queue): plan = [(i, q_i, d_i, Delta_i, damage)]
    when pressure is triggered (else []), queue = {stage: desired bitwidths}.
    """
    nb = 2 * (E + S)

    def shape(i):
        return (2 * I, H) if i % 2 == 0 else (H, I)

    D = kv_target_bytes(P["T_blk"], P["F_blk"] - P["P_blk"], P["B_kv"])   # bytes to release (Eq. 7)
    bucket = routing_buckets(mass, P["bucket_frac"])
    queue, stats = {}, []
    for st, sfloor in enumerate(P["stage_floor"]):                         # one candidate plan per stage
        # ScoreActions: floors of this stage; every step is scored lazily below
        cur = [int(x) for x in q]
        floor = [None] * nb
        for i in range(2 * E):
            if movable is None or movable[i]:
                floor[i] = max(sfloor, P["floor"][bucket[i // 2]])
        released, damage = 0, 0.0
        step_dmg = [0.0] * nb
        while released < D:                                                # GreedySelect
            best = None
            for i in range(2 * E):
                if floor[i] is None or cur[i] <= floor[i]:
                    continue
                N, Kd = shape(i)
                delta = block_bytes(N, Kd, cur[i]) - block_bytes(N, Kd, cur[i] - 1)
                d = _step_damage(P, s, phi, i, cur[i], P["mu"][bucket[i // 2]])
                ratio = d / delta
                if best is None or ratio < best[0]:
                    best = (ratio, i, delta, d)
            if best is None:
                break
            _, i, delta, d = best
            cur[i] -= 1
            released += delta
            damage += d
            step_dmg[i] += d
        queue[st] = cur                                                    # RefreshPlanQueue
        stats.append((released, damage, step_dmg))
    triggered = P["F_blk"] <= P["T_blk"]                                   # memory pressure
    pick = None
    for st in range(len(P["stage_floor"])):                                # SelectBestPlan
        if stats[st][0] >= D:
            pick = st
            break
    if pick is None:
        pick = max(range(len(stats)), key=lambda st: (stats[st][0], -st))
    plan = []
    if triggered:
        d_bits, step_dmg = queue[pick], stats[pick][2]
        for i in range(nb):
            if d_bits[i] != q[i]:
                N, Kd = shape(i)
                plan.append((i, int(q[i]), d_bits[i], block_bytes(N, Kd, int(q[i])) - block_bytes(N, Kd, d_bits[i]),
                             step_dmg[i]))
    summary = {"D": D, "triggered": triggered, "stage": pick if triggered else -1,
               "released": sum(e[3] for e in plan), "damage": sum(e[4] for e in plan),
               "stage_released": [x[0] for x in stats], "stage_damage": [x[1] for x in stats]}
    return plan, summary, queue


# ----------------------------------------------------------------- scalar loops
def unpack_index_scalar(planes, n: int, k: int, b: int) -> int:
    """O1 for one element, in plain Python integers."""
    v = 0
    for p in range(b):
        v = (v << 1) | ((int(planes[p][n][k >> 5]) >> (k & 31)) & 1)
    return v


def moe_ffn_loops(X, z, r, layer, tokens) -> list:
    """Brute-force scalar version of route-weighted FFN for a few tokens."""
    H, I = layer.H, layer.I
    res = []
    for t in tokens:
        x = [float(v) for v in X[t]]
        acc = [0.0] * H
        pairs = [(int(z[t][k]), float(r[t][k])) for k in range(z.shape[1])]
        pairs += [(layer.E + s, 1.0) for s in range(layer.S)]
        for e, w in pairs:
            gi, di = 2 * e, 2 * e + 1
            bg, bd = int(layer.q[gi]), int(layer.q[di])
            pg, lg = layer.blocks[gi].planes, layer.blocks[gi].luts[bg - 3].view(np.float16)
            pd, ld = layer.blocks[di].planes, layer.blocks[di].luts[bd - 3].view(np.float16)
            a = []
            for n in range(2 * I):
                s = 0.0
                for h in range(H):
                    s += float(lg[n][unpack_index_scalar(pg, n, h, bg)]) * x[h]
                a.append(s)
            hvec = [a[j] / (1.0 + math.exp(-a[j])) * a[I + j] for j in range(I)]
            for n in range(H):
                s = 0.0
                for j in range(I):
                    s += float(ld[n][unpack_index_scalar(pd, n, j, bd)]) * hvec[j]
                acc[n] += w * s
        res.append(acc)
    return res

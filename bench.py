#!/usr/bin/env python3
"""Benchmark of the mixed-precision MoE layer on one MI355X.

A step is one pass of the hot path over one batch: moe_route (router GEMV,
softmax, top-K) followed by moe_ffn (grouping, gate_up + SwiGLU, down,
weighted combine), reading every expert weight from its bit-planes and lookup
table at the block's committed bitwidth. The workload is the decode-shaped
layer shaped like Qwen1.5-MoE-A2.7B (PagedWeight §4, Table 1): H=2048,
I=1408, 60 routed + 4 shared experts, top-4, 64 tokens, per-block bitwidths
3..8 with the hot 20% of experts floored at 5 bits. Inputs are synthetic and
already resident in HBM when the timed region starts. R copies of the layer's
weights are rotated so the weight bytes streamed per rotation exceed 1 GB and
the 256 MB last-level cache cannot hold them.

Prints one JSON line (tokens/s, HBM GB/s of the step, a roofline entry for the
gate_up kernel timed with HIP events inside the timed region, and the CPU
oracle timed on a bounded sample on rank 0).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 MFMA
METRIC = "MoE-layer tokens/s and achieved HBM GB/s (% of peak) at mixed bitwidths"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ffn_qwen15moe_decode.md")
KERNEL_SRCS = ["k_ffn_decode.hip", "k_ffn_decode_df.hip", "k_ffn_kernels.h", "k_ffn_body.h", "mpb_device.h", "k_ffn_wide.hip"]


def _code_only(text):
    """C++ source without comments and blank lines (string literals kept), so
    that edits of comments leave the hash of the kernels' code unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return "\n".join(ln.rstrip() for ln in "".join(out).splitlines() if ln.strip())


def kernel_hash():
    """Hash of the FFN kernels' code (comments excluded): the traffic profile
    read into the bench line must have been taken of this code."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        with open(os.path.join(ROOT, "mixed_precision_bit_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def block_bytes(N, Kd, b):
    return N * Kd * b // 8 + N * (1 << b) * 2


def algorithmic_bytes(L, idx, T):
    """Bytes the method must move per step: touched blocks at q_i (planes +
    q_i-bit table), activations in, output out, router weights. Also the gate_up
    kernel's share (touched gate_up blocks + activations) and the down
    kernel's (touched down blocks; h is an intermediate)."""
    touched = np.zeros(L.E + L.S, bool)
    touched[np.unique(idx[(idx >= 0) & (idx < L.E)])] = True
    touched[L.E:] = True
    blocks_gu = sum(block_bytes(*L.shape(2 * e), int(L.q[2 * e])) for e in np.nonzero(touched)[0])
    blocks_dn = sum(block_bytes(*L.shape(2 * e + 1), int(L.q[2 * e + 1])) for e in np.nonzero(touched)[0])
    x_bytes = T * L.H * 2
    step = blocks_gu + blocks_dn + x_bytes + T * L.H * 4 + L.E * L.H * 4 + (4 * L.E if L.bias is not None else 0)
    return step, blocks_gu + x_bytes, blocks_dn, int(touched.sum())


def q_desc(c):
    if "q_gate_up" in c:
        return f"q_i {c['q_gate_up']} (gate_up) / {c['q_down']} (down)"
    if c.get("hot_floor"):
        return f"per-block q_i 3..8 (hot 20% floored at {c['hot_floor']})"
    return "per-block q_i 3..8"


def cpu_baseline(L, Xbits, n_tokens, min_s=10.0, max_s=30.0):
    """The oracle (route + FFN of every token, dequantising every touched
    block on each pass) timed on the host over whole passes of the first
    n_tokens tokens of the batch (all of it by default for batches of up to
    256 tokens, else 64), repeated until at least min_s seconds have passed
    (no pass starts after max_s)."""
    import oracle as O
    import mpb_synth as S
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), model)
    except OSError:
        pass
    T = Xbits.shape[0]
    n = min(T, n_tokens if n_tokens > 0 else (T if T <= 256 else 64))
    X = S.x_bits_to_f64(Xbits[:n], L.cfg["xdtype"])
    passes, t = 0, time.perf_counter()
    while True:
        z, r, _ = O.route(X, L.W_r, L.bias, L.K)
        O.moe_ffn(X, z, r, L)
        passes += 1
        dt = time.perf_counter() - t
        if dt >= min_s or dt * (passes + 1) / passes > max_s:
            break
    what = f"the whole {T}-token batch" if n == T else f"the first {n} of the {T} tokens"
    return {"value": round(passes * n / dt, 3), "unit": "tokens/s", "cores": int(cores), "cpu_model": model,
            "kind": "oracle",
            "sample": f"{what} of the same layer, {passes} pass(es) of route + FFN (every touched block "
                      f"dequantised on each pass), fp64 numpy, {dt:.1f} s"}


def page_movement(torch, M, L, D, replay, stream, ms_still, r=4):
    """Replays the captured steps again while a copy stream keeps offloading
    and reloading the pages above r (plane pages and the tables of bitwidths
    above r) of every block committed at <= r bits (PagedWeight §3.3,
    Figure 4: page I/O runs beside serving; no launch at q_i <= r reads those
    pages), and reports the step time with the copies running, against the
    same replay without them, and the copy rate."""
    blocks = [i for i in range(L.n_blocks) if L.q[i] <= r]

    def pinned(t):
        return torch.empty(t.shape, dtype=t.dtype, pin_memory=True)

    hp, ht, nbytes = {}, {}, {}
    for i in blocks:
        hp[i] = [None] * r + [pinned(D.pages[i][p]) for p in range(r, 8)]
        ht[i] = [None] * (r - 2) + [pinned(D.luts[i][t]) for t in range(r - 2, 6)]
        nbytes[i] = sum(D.pages[i][p].numel() * 4 + D.luts[i][p - 2].numel() * 2 for p in range(r, 8))
    cs = torch.cuda.Stream()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    moved, n_xfer = 0, 0
    c0.record(cs)
    s0.record(stream)
    replay()
    s1.record(stream)
    while not s1.query():
        for i in blocks:
            st = M.mpb_page_state(i, r)
            if st == M.MPB_PAGE_GPU:
                M.mpb_offload_pages(i, r, hp[i], D.pages[i], ht[i], D.luts[i], cs)
            elif st == M.MPB_PAGE_CPU:
                M.mpb_reload_pages(i, 8, hp[i], D.pages[i], ht[i], D.luts[i], cs)
            else:
                continue
            moved += nbytes[i]
            n_xfer += 1
    c1.record(cs)
    torch.cuda.synchronize()
    for i in blocks:             # leave every block resident again
        if M.mpb_page_state(i, r) == M.MPB_PAGE_CPU:
            M.mpb_reload_pages(i, 8, hp[i], D.pages[i], ht[i], D.luts[i], cs)
    cs.synchronize()
    ms_moving = s0.elapsed_time(s1) / replay.steps
    return {"blocks_moving": len(blocks), "pages_per_transfer": 8 - r, "transfers": n_xfer,
            "bytes_moved": int(moved), "copy_gbs": round(moved / (c0.elapsed_time(c1) * 1e-3) / 1e9, 1),
            "ms_per_step_still": round(ms_still, 5), "ms_per_step_moving": round(ms_moving, 5),
            "slowdown": round(ms_moving / ms_still - 1.0, 4)}


def planner_timing(torch, M, L, cfg, idx, w, steps, F_blk=20):
    """Times the routing-mass kernel (Eq. 1) on this batch and the host
    planner step (Algorithm 1) fed with its output, under KV pressure."""
    import mpb_synth as S
    mass = torch.empty(L.E, dtype=torch.float64, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    M.moe_routing_mass(idx, w, L.E, mass)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        M.moe_routing_mass(idx, w, L.E, mass)
    e1.record()
    torch.cuda.synchronize()
    m = mass.cpu().numpy()
    sens = S.make_sensitivity(cfg, L.n_blocks)[:, 3:9]
    P, phi = S.make_planner_inputs(cfg, L.n_blocks, F_blk)
    M.mpb_plan_step(L.H, L.I, L.E, L.S, L.K, L.q, None, sens, m, phi, P)
    times = []
    for _ in range(steps):
        t = time.perf_counter()
        plan, summ, _ = M.mpb_plan_step(L.H, L.I, L.E, L.S, L.K, L.q, None, sens, m, phi, P)
        times.append(time.perf_counter() - t)
    dt = float(np.median(times))  # host timings: the median is robust to scheduler noise
    return {"routing_mass_us": round(e0.elapsed_time(e1) * 1e3 / steps, 2),
            "plan_step_us": round(dt * 1e6, 1), "plan_blocks": len(plan), "target_bytes": summ["D"],
            "released_bytes": summ["released"], "stage": summ["stage"]}


def sweep_states(L, s, fracs=(0.25, 0.5, 0.75), floor_hot=5, eps=1e-12):
    """Bitwidth states of the sweep on the config-1 layer: the initial
    commitment; then, for each fraction f, the routed blocks with the least
    predicted damage per released byte lowered (PagedWeight §3.2 "Planning
    objective": damage max(eps, s_i^b' - s_i^q) of the drop q -> b' (Eq. 4, 8
    with unit multipliers) over the bytes it releases (Eq. 3)), each block to
    its best legal b' (floor 3 bits, 5 for hot-bucket experts), the first
    ceil(f x #routed blocks) of that ranking (ties to the lower block), so the
    lowered sets are nested; last, every block at 8 bits."""
    q0 = np.asarray(L.q, np.int64)
    best = []
    for i in range(2 * L.E):
        fl = floor_hot if L.hot[i // 2] else 3
        b = int(q0[i])
        N, Kd = L.shape(i)
        cands = [(max(eps, s[i, b2] - s[i, b]) / (block_bytes(N, Kd, b) - block_bytes(N, Kd, b2)), b2)
                 for b2 in range(fl, b)]
        if cands:
            sc, b2 = min(cands)
            best.append((sc, i, b2))
    best.sort()
    states = [("initial", q0.copy())]
    for f in fracs:
        q = q0.copy()
        for _, i, b2 in best[:int(np.ceil(f * 2 * L.E))]:
            q[i] = b2
        states.append((f"lowered {int(round(f * 100))}%", q))
    states.append(("all 8-bit", np.full(L.n_blocks, 8, np.int64)))
    return states


def run_sweep(torch, M, L, idx_host, step_fn, T, steps, warmup):
    """Times the step in every bitwidth state (eager launches, HIP events
    around the phases as in timed region 2). Launch order: for each state,
    warm-up steps, then `steps` timed ones."""
    import mpb_synth as S
    s = S.make_sensitivity(4, L.n_blocks)
    out = []
    prev = np.asarray(L.q, np.int64).copy()
    stream = torch.cuda.current_stream()
    k0 = 0
    for name, q in sweep_states(L, s):
        for i in np.nonzero(q != prev)[0]:
            M.set_committed_bits(int(i), int(q[i]))
        prev = q
        for k in range(warmup):
            step_fn(k0 + k)
        k0 += warmup
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
        for row in evs:
            for e in row:
                e.record(stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for k in range(steps):
            M.mpb_set_kernel_events([e.cuda_event for e in evs[k]])
            step_fn(k0 + k)
        M.mpb_set_kernel_events([])
        b.record(stream)
        torch.cuda.synchronize()
        k0 += steps
        ms = a.elapsed_time(b) / steps
        gu = float(np.mean([evs[k][1].elapsed_time(evs[k][2]) for k in range(steps)]))
        dn = float(np.mean([evs[k][5].elapsed_time(evs[k][6]) for k in range(steps)]))
        # blocks of the experts this batch touches (routed experts with tokens, every shared one)
        hit = np.zeros(L.E + L.S, bool)
        hit[np.unique(idx_host[(idx_host >= 0) & (idx_host < L.E)])] = True
        hit[L.E:] = True
        touched = np.repeat(hit, 2).astype(np.uint8)
        mb = int(M.mpb_committed_bytes(touched))
        gu_b = sum(block_bytes(*L.shape(2 * e), int(q[2 * e])) for e in np.nonzero(hit)[0])
        dn_b = mb - gu_b
        out.append({"state": name, "committed_bytes": mb, "gate_up_block_bytes": int(gu_b),
                    "down_block_bytes": int(dn_b), "ms_per_step": round(ms, 5),
                    "tokens_per_s": round(T / (ms * 1e-3), 1), "gate_up_us": round(gu * 1e3, 2),
                    "down_us": round(dn * 1e3, 2),
                    "gate_up_gbs": round((gu_b + T * L.H * 2) / (gu * 1e-3) / 1e9, 1),
                    "down_gbs": round(dn_b / (dn * 1e-3) / 1e9, 1),
                    "launches": [warmup, steps]})
    return out


def copy_calibration(torch, nbytes, steps):
    """Time a plain copy kernel (torch's device copy) of known size: the
    reference rocprofv3's FETCH_SIZE / WRITE_SIZE are scaled by, and the
    measured copy bandwidth of the device."""
    a = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    print(json.dumps({"copy_bytes": nbytes, "ms_per_copy": round(ms, 5),
                      "copy_gbs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--rotate", type=int, default=0, help="layer copies (0: enough for >= 1 GB)")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0: whole batch up to 256 tokens, else 64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only time a plain device-to-device copy of this many bytes (counter calibration)")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="launch the timed steps eagerly instead of replaying them as one HIP graph")
    ap.add_argument("--fused", action="store_true",
                    help="also time the same steps as one fused launch per step (moe_fused)")
    ap.add_argument("--plan", action="store_true",
                    help="also time the routing-mass kernel and the host planner step on this batch")
    ap.add_argument("--sweep", action="store_true",
                    help="config 4: also time the step in each bitwidth state (initial, 25/50/75%% of the routed "
                         "blocks lowered by damage per released byte, all 8-bit)")
    ap.add_argument("--page-movement", action="store_true",
                    help="also replay the steps while cold blocks' upper planes are offloaded and reloaded "
                         "on a copy stream, and report the slowdown")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this layer is measured at N=1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_bytes:
        copy_calibration(torch, args.copy_bytes, args.steps)
        return
    import mpb_synth as S
    from mixed_precision_bit_amd import _lib as M
    from mixed_precision_bit_amd.layer import DeviceLayer

    rank = int(os.environ.get("RANK", "0"))
    cfg = args.config
    c = S.layer_config(cfg)
    L = S.make_layer(cfg)
    Xbits = S.make_tokens(cfg)
    T = Xbits.shape[0]
    xdt = c["xdtype"]

    D0 = DeviceLayer.from_synth(L)
    wbytes = D0.weight_bytes()
    R = args.rotate or max(1, int(np.ceil(1.0e9 / (0.5 * wbytes))))
    layers = [D0] + [DeviceLayer.from_synth(L, q_dev=D0.q_dev) for _ in range(R - 1)]
    X = torch.from_numpy(Xbits.view(np.int16)).cuda()
    bufs = []
    for D in layers:
        idx, w = D.alloc_route(T)
        out, ws = D.alloc_ffn(T)
        bufs.append((idx, w, out, ws))
    stream = torch.cuda.current_stream()

    def step(k):
        D = layers[k % R]
        idx, w, out, ws = bufs[k % R]
        D.route(X, xdt, idx, w)        # on torch's current stream
        D.ffn(X, xdt, idx, w, out, ws)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    idx_host = bufs[0][0].cpu().numpy()
    step_bytes, gu_bytes, dn_bytes, n_touched = algorithmic_bytes(L, idx_host, T)

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # Timed region 1 (the headline): K steps. With --graph (default) the K
    # steps are captured once as a HIP graph, replayed once untimed, then
    # replayed inside the timed region.
    if args.graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for k in range(args.steps):
                    step(args.warmup + k)
        stream.wait_stream(cap)
        graph.replay()
        torch.cuda.synchronize()
        start.record(stream)
        graph.replay()
        end.record(stream)
    else:
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(args.steps):
            step(args.warmup + k)
        end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps

    # Timed region 2 (per-kernel times): the same K steps launched eagerly, with
    # moe_ffn recording HIP events on its stream before grouping, at the start
    # and end of the gate_up and down kernels (recorded by their launches),
    # before the combine and after it (event records inside a graph do not
    # order against its kernel nodes, so kernel times come from this pass).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    for row in evs:              # torch creates the HIP event on first record
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    start2, end2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start2.record(stream)
    for k in range(args.steps):
        M.mpb_set_kernel_events([e.cuda_event for e in evs[k]])
        step(args.warmup + k)
    M.mpb_set_kernel_events([])
    end2.record(stream)
    torch.cuda.synchronize()
    ms_eager = start2.elapsed_time(end2) / args.steps
    phase = np.array([[evs[k][j].elapsed_time(evs[k][j + 1]) for j in range(4)] for k in range(args.steps)])
    gu_ms = float(phase[:, 1].mean())
    dn_ms = float(np.mean([evs[k][5].elapsed_time(evs[k][6]) for k in range(args.steps)]))

    tok_s = T / (ms * 1e-3)
    step_gbs = step_bytes / (ms * 1e-3) / 1e9
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9
    # prefill-size groups make gate_up a dense contraction: report it against
    # the fp16 MFMA peak with its useful FLOPs (2 per multiply-add over the
    # grouped token rows), decode-size groups against HBM with its bytes
    n_rows = int(((idx_host >= 0) & (idx_host < L.E)).sum()) + T * L.S
    gu_flops = 2.0 * n_rows * (2 * L.I) * L.H
    prefill = T * L.K / L.E >= 96
    traffic = dn_traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tf = json.loads([ln for ln in open(TRAFFIC_FILE) if ln.strip().startswith("{")][-1])
        if tf.get("kernel_hash") == kernel_hash() and tf.get("workload") == c["name"]:
            traffic = tf.get("bytes_per_launch")
            dn_traffic = tf.get("down_bytes_per_launch")
    res = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{c['name']}: H={c['H']} I={c['I']} E={c['E']}+{c['S']} shared K={c['K']} "
                               f"T={T} x={xdt}, {q_desc(c)}",
                   "global_batch": T, "layer_copies_rotated": R, "touched_experts": n_touched,
                   "committed_weight_bytes": int(M.mpb_committed_bytes()),
                   "launch": "hip_graph" if args.graph else "eager",
                   "ms_per_step_eager": round(ms_eager, 5)},
        "hbm_gbs": round(step_gbs, 1),
        "hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "phase_ms": {"group": round(float(phase[:, 0].mean()), 5), "gate_up": round(gu_ms, 5),
                     "down": round(dn_ms, 5), "combine": round(float(phase[:, 3].mean()), 5)},
        "roofline": ({"kernel": "k_gate_up", "bound": "mfma", "achieved": round(gu_flops / (gu_ms * 1e-3) / 1e12, 1),
                      "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(gu_flops / (gu_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
                      "traffic": traffic, "algorithmic_flops_per_launch": gu_flops,
                      "hbm_gbs": round(gu_gbs, 1)} if prefill else
                     {"kernel": "k_gate_up", "bound": "hbm", "achieved": round(gu_gbs, 1),
                      "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                      "traffic": traffic, "algorithmic_bytes_per_launch": int(gu_bytes)}),
    }
    # the second FFN kernel, timed by its own launch events: down blocks' bytes
    # against HBM (prefill-size layers: its useful flops against the MFMA peak)
    dn_flops = 2.0 * n_rows * L.H * L.I
    res["roofline"]["k_down"] = (
        {"bound": "mfma", "achieved": round(dn_flops / (dn_ms * 1e-3) / 1e12, 1), "peak": MFMA_PEAK_TFLOPS,
         "unit": "TFLOP/s", "frac": round(dn_flops / (dn_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
         "algorithmic_flops_per_launch": dn_flops, "us": round(dn_ms * 1e3, 2)} if prefill else
        {"bound": "hbm", "achieved": round(dn_bytes / (dn_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(dn_bytes / (dn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": dn_traffic,
         "algorithmic_bytes_per_launch": int(dn_bytes), "us": round(dn_ms * 1e3, 2)})
    if args.fused:
        fb = [D.alloc_fused(T) for D in layers]

        def fstep(k):
            D = layers[k % R]
            idx, w = bufs[k % R][0], bufs[k % R][1]
            out, ws = fb[k % R]
            D.fused(X, xdt, idx, w, out, ws)

        for k in range(args.warmup):
            fstep(k)
        torch.cuda.synchronize()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        fg = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(fg, stream=cap):
                for k in range(args.steps):
                    fstep(args.warmup + k)
        stream.wait_stream(cap)
        fg.replay()
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        fg.replay()
        f1.record(stream)
        torch.cuda.synchronize()
        fms = f0.elapsed_time(f1) / args.steps
        res["fused"] = {"ms_per_step": round(fms, 5), "tokens_per_s": round(T / (fms * 1e-3), 1),
                        "launches_per_step": 1, "vs_separate": round(ms / fms, 4)}
    if args.plan:
        res["planner"] = planner_timing(torch, M, L, cfg, bufs[0][0], bufs[0][1], args.steps)
    if args.page_movement and args.graph:
        def replay():
            graph.replay()
        replay.steps = args.steps
        res["page_movement"] = page_movement(torch, M, L, D0, replay, stream, ms)
    if args.sweep:
        if cfg != 4:
            print("--sweep runs on config 4 (the bitwidth-change sweep)", file=sys.stderr)
            sys.exit(2)
        res["sweep"] = run_sweep(torch, M, L, idx_host, step, T, args.steps, max(1, args.warmup // 4))
    if rank == 0 and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(L, Xbits, args.cpu_tokens)
    if rank == 0:
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

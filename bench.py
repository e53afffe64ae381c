"""Benchmark of the MoE grouped-GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the hot path over one batch of synthetic input that
is already resident in HBM: routing (moegg_route) and the grouped GEMMs of
the workload.  The default workload is the Mixtral-shaped first MoE GEMM
(gate_up: T=4096 tokens, K=4096, N=28672, E=8, top-2, permute_x) with its
backward: route + forward + dX + dW.  Other workloads:
  fine    fine-grained down GEMM (T=8192, E=128, top-8, K=768, N=2048, Zipf
          routing): route + forward (permute_y + fuse_mul_post) + dX + dW
  decode  the same layer with T=64: route + forward (weights rotated over
          several copies so every step reads them from HBM)
  dual    two GEMM groups of different shapes in one launch
  tiny    T=128, K=256, N=512, E=8, top-2: route + forward

Prints ONE JSON line.  `value` is useful TFLOP/s over the whole step
(useful FLOPs = 2 * sum_e m_e * N * K per GEMM, actual rows only);
`roofline` describes the step's dominant kernel, timed with HIP events on
the stream the kernels run on; `cpu_baseline` is the plain CPU oracle timed
on a bounded sample of the same workload, route / fwd / dX / dW each on one
thread and on every core of the process's affinity mask.  With the default
workload the line also carries `configs`: the tiny layer, the dual-expert
groups, the fine-grained forward (permute_y + fuse_mul_post), its decode
slice and its backward, each timed the same way after the headline step.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import token_routing_amd as mg  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
BLOCK_M = 128


def _dev(t):
    return t.to("cuda", non_blocking=False).contiguous()


class Step:
    """A workload's kernels, resident inputs and per-kernel accounting."""

    def __init__(self, name):
        self.name = name
        self.kernels = []      # (label, fn, useful_flops, algorithmic_bytes)

    def add(self, label, fn, flops, nbytes):
        self.kernels.append((label, fn, float(flops), float(nbytes)))


def _useful(m_sizes, N, K):
    return 2.0 * float(np.sum(m_sizes)) * N * K


def build_layer_step(wl, dY_seed, with_bwd=True, rotate=1, extra_flags=0):
    """route + forward (+ dX + dW) of one routed grouped GEMM.

    extra_flags = GATED_SILU: the gate_up forward with the activation fused
    (output [S, N/2]); the backward is then not part of the step.
    """
    st = Step(wl.name)
    E, N, K = wl.W.shape
    S, T, topk = wl.S, wl.T, wl.topk
    flags = wl.flags | extra_flags
    out_cols = N // 2 if (flags & mg.GATED_SILU) else N
    ids = _dev(wl.ids)
    X = _dev(wl.X)
    Ws = [_dev(wl.W)]
    for i in range(1, rotate):
        Ws.append(Ws[0].clone())
    weights = _dev(wl.weights.reshape(-1))
    route_out = mg.moe_route(ids, E, BLOCK_M)
    ws = torch.empty(max(mg.route_workspace_bytes(S, E), 1), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    m_sizes = route_out["m_sizes"].cpu().numpy()
    nonempty = int((m_sizes > 0).sum())
    Y = torch.empty(S, out_cols, dtype=torch.bfloat16, device="cuda")
    it = {"i": 0}

    def route():
        mg.moe_route(ids, E, BLOCK_M, out=route_out, workspace=ws)

    def fwd():
        W = Ws[it["i"] % len(Ws)]
        it["i"] += 1
        mg.grouped_gemm_fwd(X, W, route_out["m_sizes"], route_out["gather"], weights, topk, flags,
                            Y=Y)

    x_rows = T if (flags & synth.PERMUTE_X) else S
    st.add("route", route, 0.0, S * 4 * 3 + E * 4 * 4)
    st.add("fwd", fwd, _useful(m_sizes, N, K),
           nonempty * N * K * 2 + x_rows * K * 2 + S * out_cols * 2 + S * 4 * 2)
    if with_bwd:
        bwd_flags = flags & (synth.PERMUTE_X | synth.PERMUTE_Y)
        dY = synth.normal_bf16((S, N), 0.01, synth.generator(dY_seed)).to("cuda")
        dX = torch.empty(S, K, dtype=torch.bfloat16, device="cuda")
        dW = torch.empty(E, N, K, dtype=torch.bfloat16, device="cuda")
        # under permute_x with room for X's rows in expert order (copied first)
        ws_bytes = (mg.dw_gather_workspace_bytes(T, topk, E, N, K)
                    if bwd_flags & synth.PERMUTE_X else mg.dw_workspace_bytes(T, topk, E, N, K))
        dw_ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None

        dx_bytes = mg.dx_workspace_bytes(T, topk, E, N, K)
        dx_ws = torch.empty(dx_bytes, dtype=torch.uint8, device="cuda") if dx_bytes else None

        def bwd_dx():
            # with rotated weights, not the copy the forward just read
            W = Ws[(it["i"] - 1 + len(Ws) // 2) % len(Ws)]
            mg.grouped_gemm_dX(dY, W, route_out["m_sizes"], route_out["gather"], topk,
                               bwd_flags, dX=dX, workspace=dx_ws, split=dx_ws is not None)

        def bwd_dw():
            mg.grouped_gemm_dW(X, dY, route_out["m_sizes"], route_out["gather"], topk, bwd_flags,
                               dW=dW, workspace=dw_ws, split=dw_ws is not None)

        st.add("dX", bwd_dx, _useful(m_sizes, N, K), S * N * 2 + nonempty * N * K * 2 + S * K * 2)
        st.add("dW", bwd_dw, _useful(m_sizes, N, K), S * N * 2 + x_rows * K * 2 + E * N * K * 2)
    st.m_sizes = m_sizes
    st.flags = flags
    st.inputs = wl
    st.dY_seed = dY_seed
    return st


def build_dual_step(wl):
    st = Step("dual")
    groups = [(_dev(x), _dev(w)) for x, w in wl.groups]
    outs = [torch.empty(x.shape[0], w.shape[1], dtype=torch.bfloat16, device="cuda")
            for x, w in groups]
    flops = sum(2.0 * x.shape[0] * x.shape[1] * w.shape[1] for x, w in groups)
    nbytes = sum((x.numel() + w.numel() + x.shape[0] * w.shape[1]) * 2 for x, w in groups)
    st.add("groups", lambda: mg.grouped_gemm_groups(groups, 0, outputs=outs), flops, nbytes)
    st.inputs = wl
    return st


def build_combine_step(wl, rotate=2):
    """Top-k combine after the fine-grained down projection (expert-sorted Y,
    scatter index and routing weights) and its backward with the weight
    gradient.  Y is rotated over `rotate` copies so that the 256 MB MALL does
    not hold it between steps."""
    st = Step("combine")
    S, T, N, k = wl.S, wl.T, wl.N, wl.topk
    ids = _dev(wl.ids)
    route_out = mg.moe_route(ids, wl.E, BLOCK_M)
    g = synth.generator(synth.SEEDS["combine_y"])
    Ys = [_dev(synth.normal_bf16((S, N), 1.0, g))]
    for _ in range(1, rotate):
        Ys.append(Ys[0].clone())
    dOut = _dev(synth.normal_bf16((T, N), 0.1, g))
    w = _dev(wl.weights.reshape(-1).contiguous())
    out = torch.empty(T, N, dtype=torch.bfloat16, device="cuda")
    dY = torch.empty(S, N, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty(S, dtype=torch.float32, device="cuda")
    it = {"f": 0, "b": 0}

    def fwd():
        Y = Ys[it["f"] % len(Ys)]
        it["f"] += 1
        mg.combine(Y, k, route_out["scatter"], w, out=out)

    def bwd():
        Y = Ys[it["b"] % len(Ys)]
        it["b"] += 1
        mg.combine_bwd(dOut, Y, k, route_out["scatter"], w, dY=dY, dw=dw)

    # useful FLOPs: one multiply-add per slot element (fwd); two per element (bwd)
    st.add("combine", fwd, 2.0 * S * N, S * N * 2 + S * 8 + T * N * 2)
    st.add("combine_bwd", bwd, 4.0 * S * N, T * N * 2 + S * N * 2 + S * 8 + S * N * 2 + S * 4)
    st.m_sizes = route_out["m_sizes"].cpu().numpy()
    st.inputs = wl
    return st


def make_step(name):
    if name == "mixtral":
        return build_layer_step(synth.mixtral(), dY_seed=synth.SEEDS["mixtral_bwd_dy"])
    if name == "mixtral_gated":
        return build_layer_step(synth.mixtral(), dY_seed=0, with_bwd=False,
                                extra_flags=mg.GATED_SILU)
    if name == "fine":
        return build_layer_step(synth.fine_bwd(), dY_seed=synth.SEEDS["fine_bwd_dy"])
    if name == "fine_fwd":
        return build_layer_step(synth.fine_down(), dY_seed=0, with_bwd=False)
    if name == "decode":
        return build_layer_step(synth.fine_decode(), dY_seed=0, with_bwd=False, rotate=4)
    if name == "decode_bwd":
        return build_layer_step(synth.fine_decode_bwd(), dY_seed=synth.SEEDS["fine_bwd_dy"],
                                rotate=4)
    if name == "tiny":
        return build_layer_step(synth.tiny(), dY_seed=0, with_bwd=False)
    if name == "dense":
        return build_layer_step(synth.dense(), dY_seed=0, with_bwd=False)
    if name == "dual":
        return build_dual_step(synth.dual())
    if name == "combine":
        return build_combine_step(synth.fine_down())
    raise SystemExit(f"unknown workload {name}")


WORKLOAD_DESC = {
    "mixtral": "Mixtral-shaped MoE gate_up grouped GEMM, T=4096 K=4096 N=28672 E=8 top-2, "
               "permute_x; step = route + fwd + dX + dW",
    "mixtral_gated": "Mixtral-shaped MoE gate_up grouped GEMM with the gated SiLU fused in the "
                     "epilogue, T=4096 K=4096 N=28672 (-> 14336) E=8 top-2, permute_x; "
                     "step = route + fwd",
    "fine": "fine-grained MoE down grouped GEMM, T=8192 E=128 top-8 K=768 N=2048 Zipf(1.2); "
            "training step = route + fwd(permute_y) + dX + dW (dY gathered on load)",
    "fine_fwd": "fine-grained MoE down grouped GEMM forward, T=8192 E=128 top-8 K=768 N=2048, "
                "permute_y + fuse_mul_post",
    "decode": "fine-grained MoE down grouped GEMM decode slice, T=64 E=128 top-8 K=768 N=2048, "
              "permute_y + fuse_mul_post",
    "decode_bwd": "decode-shaped backward of the fine-grained down GEMM, T=64 E=128 top-8 K=768 "
                  "N=2048; step = route + fwd(permute_y) + dX + dW",
    "dual": "asymmetric dual-expert GEMM: [512,1024]x[1024,2048] and [256,1024]x[1024,4096]",
    "dense": "the Mixtral gate_up FLOPs as one dense product through the grouped forward: "
             "X [8192,4096] times W^T, W [28672,4096] (one expert); the line also times the "
             "vendor GEMM (hipBLASLt via torch.matmul) on the same operands",
    "tiny": "tiny MoE grouped GEMM, T=128 K=256 N=512 E=8 top-2, permute_x",
    "combine": "top-k combine after the fine-grained down projection, T=8192 top-8 N=2048 "
               "(expert-sorted Y, routing weights) and its backward with the weight gradient",
}


def time_step(st, steps, warmup, min_warm_s=0.0):
    """Run `warmup` untimed steps (then more, doubling, until min_warm_s
    seconds have passed), then time `steps` steps with HIP events on the
    launch stream: per-kernel ms, step ms and wall seconds."""
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    batch, done = warmup, 0
    while batch > 0:
        for _ in range(batch):
            for _, fn, _, _ in st.kernels:
                fn()
        done += batch
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= min_warm_s:
            break
        batch = done
    nk = len(st.kernels)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        for i, (_, fn, _, _) in enumerate(st.kernels):
            fn()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.zeros(nk)
    total = 0.0
    for s in range(steps):
        for i in range(nk):
            per[i] += ev[s][i].elapsed_time(ev[s][i + 1])
        total += ev[s][0].elapsed_time(ev[s][nk])
    return per / steps, total / steps, wall


def kernel_source_sha(label=None):
    """sha256[:16] of the sources a kernel is built from (all kernels' when
    label is None): the shared headers plus the kernel's own file."""
    if label is None:
        own = ("gemm.hip", "route.hip", "combine.hip")
    elif label.startswith("combine"):
        own = ("combine.hip",)
    elif label.startswith("route"):
        own = ("route.hip",)
    else:
        own = ("gemm.hip",)
    h = hashlib.sha256()
    for f in own + ("common.h", "gemm_params.h"):
        with open(os.path.join(ROOT, "token_routing_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, label):
    """HBM bytes per launch from committed rocprofv3 counters, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{label}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_src_sha") != kernel_source_sha(label):
        return None
    return rec.get("bytes_per_launch")


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _run_threads(fn, parts):
    """fn(part) on one Python thread per part (the oracle's ctypes calls
    release the GIL, so the parts run on separate cores); wall seconds."""
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.perf_counter()
    if len(parts) == 1:
        fn(parts[0])
    else:
        with ThreadPoolExecutor(max_workers=len(parts)) as ex:
            list(ex.map(fn, parts))
    return time.perf_counter() - t0


def _oracle_leg(name, call, pool, flops_of, per_leg_s, cores, rng):
    """Time the unchanged oracle on random output rows of `pool`: one thread,
    then `cores` threads over disjoint row sets.  Each leg is sized to about
    per_leg_s seconds from a short calibration call.  Returns the two legs'
    rates (useful FLOP/s of the computed rows)."""
    pool = np.asarray(pool)
    cal = rng.choice(pool, size=min(2, pool.size), replace=False)
    t_cal = _run_threads(call, [cal])
    per_row = max(t_cal / cal.size, 1e-7)
    n1 = int(max(1, min(pool.size, per_leg_s / per_row)))
    legs = {}
    for leg, threads in (("single", 1), ("all_cores", cores)):
        n = min(pool.size, n1 * threads)
        rows = rng.choice(pool, size=n, replace=False)
        parts = [p for p in np.array_split(rows, threads) if p.size]
        dt = _run_threads(call, parts)
        fl = float(flops_of(rows))
        legs[leg] = {"rows": int(n), "threads": len(parts), "seconds": round(dt, 3),
                     "gflops": round(fl / dt / 1e9, 3)}
    return legs


def cpu_baseline(st, budget_s):
    """The CPU oracle, timed on the host cores on a bounded sample of the
    workload: each step of the path separately (route, fwd, dX, dW), once on
    one thread and once with one thread per core of sched_getaffinity over
    disjoint random output rows.  The oracle itself is unchanged (plain
    loops, one call per thread).  `value` is the step's useful FLOP/s at the
    all-cores rates: total useful FLOPs over the sum of each kernel's full
    time at its rate."""
    import oracle

    wl = st.inputs
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(0)
    labels = [k[0] for k in st.kernels]
    per_leg = budget_s / max(1, 2 * sum(1 for lab in labels if lab != "route"))
    out = {"kind": "oracle", "unit": "TFLOP/s", "cores": cores, "cpu_model": _cpu_model()}
    legs = {"single": {}, "all_cores": {}}
    full = {}
    if st.name == "combine":
        g = synth.generator(synth.SEEDS["combine_y"])
        Yb = synth.bits(synth.normal_bf16((wl.S, wl.N), 1.0, g))
        ref_route = oracle.route(wl.ids.numpy().reshape(-1), wl.E, BLOCK_M)
        sc = ref_route["scatter"]
        w = wl.weights.numpy().reshape(-1)
        k = wl.topk

        def call(tok):
            lo, hi = int(tok.min()), int(tok.max()) + 1
            oracle.combine(Yb, k, scatter=sc[lo * k:hi * k], weights=w[lo * k:hi * k],
                           num_tokens=hi - lo)
        # tokens in contiguous blocks (the combine takes a token range)
        blocks = np.arange(wl.T).reshape(-1, 64)
        r = _oracle_leg("combine", lambda b: [call(x) for x in blocks[b]], np.arange(len(blocks)),
                        lambda b: 2.0 * len(b) * 64 * k * wl.N, per_leg, cores, rng)
        for leg in legs:
            legs[leg]["combine"] = r[leg]
        full["combine"] = 2.0 * wl.S * wl.N
    elif st.name == "dual":
        for gi, (x, w) in enumerate(wl.groups):
            xb, wb = synth.bits(x), synth.bits(w)
            per_row = 2.0 * x.shape[1] * w.shape[1]
            r = _oracle_leg(f"group{gi}", lambda rows: oracle.dense_gemm_kn(xb[np.sort(rows)], wb),
                            np.arange(x.shape[0]), lambda rows: per_row * len(rows), per_leg, cores,
                            rng)
            for leg in legs:
                legs[leg][f"group{gi}"] = r[leg]
            full[f"group{gi}"] = per_row * x.shape[0]
    else:
        E, N, K = wl.W.shape
        ids = wl.ids.numpy().reshape(-1)
        reps, t0 = 0, time.perf_counter()
        while True:
            ref_route = oracle.route(ids, wl.E, BLOCK_M)
            reps += 1
            if time.perf_counter() - t0 >= 0.2:
                break
        t_route = (time.perf_counter() - t0) / reps
        for leg in legs:
            # one counting sort over all slots: not split over rows
            legs[leg]["route"] = {"rows": int(ids.size), "threads": 1, "seconds": round(t_route, 4),
                                  "note": "one stable counting sort over all slots"}
        Xb, Wb = synth.bits(wl.X), synth.bits(wl.W)
        gate = wl.weights.numpy().reshape(-1)
        ms, gather, topk, flags = ref_route["m_sizes"], ref_route["gather"], wl.topk, st.flags
        gated = bool(flags & mg.GATED_SILU)
        base_flags = flags & (synth.PERMUTE_X | synth.PERMUTE_Y | synth.FUSE_MUL_POST)
        row_fl = 2.0 * N * K
        if "dX" in labels or "dW" in labels:
            dYb = synth.bits(synth.normal_bf16((wl.S, N), 0.01, synth.generator(st.dY_seed)))
            bflags = flags & (synth.PERMUTE_X | synth.PERMUTE_Y)
        for lab in labels:
            if lab == "fwd":
                if gated:
                    call = lambda rows: oracle.grouped_gemm_fwd_gated(
                        Xb, Wb, ms, gather, topk, base_flags, rows=rows)
                else:
                    call = lambda rows: oracle.grouped_gemm_fwd(
                        Xb, Wb, ms, gather, gate, topk, base_flags, rows=rows)
                r = _oracle_leg(lab, call, np.arange(wl.S), lambda rows: row_fl * len(rows),
                                per_leg, cores, rng)
            elif lab == "dX":
                r = _oracle_leg(lab, lambda rows: oracle.grouped_gemm_dX(
                    dYb, Wb, ms, gather, topk, bflags, rows=rows), np.arange(wl.S),
                    lambda rows: row_fl * len(rows), per_leg, cores, rng)
            elif lab == "dW":
                live = np.nonzero(ms > 0)[0]
                pool = (live[:, None] * N + np.arange(N)[None, :]).reshape(-1)
                r = _oracle_leg(lab, lambda rows: oracle.grouped_gemm_dW(
                    Xb, dYb, ms, gather, topk, bflags, E, rows=rows), pool,
                    lambda rows: float(np.sum(2.0 * ms[np.asarray(rows) // N] * K)), per_leg,
                    cores, rng)
            else:
                continue
            for leg in legs:
                legs[leg][lab] = r[leg]
            full[lab] = _useful(ms, N, K)
    # each kernel's full-workload time at the leg's rate, and the step rate
    for leg in legs:
        tot = sum(full[k] / (legs[leg][k]["gflops"] * 1e9) for k in full)
        tot += legs[leg].get("route", {}).get("seconds", 0.0)
        legs[leg]["step_s_extrapolated"] = round(tot, 2)
        legs[leg]["tflops"] = round(sum(full.values()) / tot / 1e12, 6)
    out["value"] = legs["all_cores"]["tflops"]
    out["single"], out["all_cores"] = legs["single"], legs["all_cores"]
    out["sample"] = (f"random output rows of each kernel of the {st.name} step, each leg sized to "
                     f"~{per_leg:.1f} s (one thread, then {cores} threads over disjoint rows); "
                     "value = the step's useful FLOPs over the sum of each kernel's full time "
                     "at its all-cores rate")
    return out


def _time(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def vendor_reference(st, steps, warmup):
    """hipBLASLt (torch.matmul) on the same products, timed like a step: a
    reference point for the kernels, not part of the path.

    dense: one product X W^T.  Routed layer workloads: the products expert by
    expert (one torch.matmul per expert and kernel), on operands gathered
    into expert order beforehand (the gathers are not timed)."""
    wl = st.inputs
    if st.name == "dense":
        X = _dev(wl.X)
        Wt = _dev(wl.W[0]).t()
        ms = _time(lambda: torch.matmul(X, Wt), steps, warmup)
        flops = 2.0 * wl.T * wl.N * wl.K
        return {"kernel": "hipBLASLt via torch.matmul(X, W.t())", "ms": round(ms, 4),
                "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
    if not hasattr(st, "dY_seed"):
        return None                     # not a routed grouped-GEMM workload
    E, N, K = wl.W.shape
    route = mg.moe_route(_dev(wl.ids), E, BLOCK_M)
    torch.cuda.synchronize()
    off = route["offsets"].cpu().numpy()
    g = route["gather"].long()
    px = bool(wl.flags & synth.PERMUTE_X)
    py = bool(wl.flags & synth.PERMUTE_Y)
    X = _dev(wl.X)
    X = X[g // wl.topk] if px else X                        # expert order
    W = _dev(wl.W)
    out = {"kernel": "hipBLASLt via torch.matmul, one call per expert and product",
           "note": "operands gathered into expert order outside the timed region"}
    experts = [(e, int(off[e]), int(off[e + 1])) for e in range(E) if off[e + 1] > off[e]]
    flops = 2.0 * float(off[E]) * N * K
    Y = torch.empty(int(off[E]), N, dtype=torch.bfloat16, device="cuda")
    ms = _time(lambda: [torch.matmul(X[lo:hi], W[e].t(), out=Y[lo:hi]) for e, lo, hi in experts],
               steps, warmup)
    out["fwd"] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
    if any(lab == "dX" for lab, _, _, _ in st.kernels):
        dY = synth.normal_bf16((wl.S, N), 0.01, synth.generator(st.dY_seed)).to("cuda")
        dY = dY[g] if py else dY                              # expert order
        dX = torch.empty(int(off[E]), K, dtype=torch.bfloat16, device="cuda")
        dW = torch.empty(E, N, K, dtype=torch.bfloat16, device="cuda")
        ms = _time(lambda: [torch.matmul(dY[lo:hi], W[e], out=dX[lo:hi]) for e, lo, hi in experts],
                   steps, warmup)
        out["dX"] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
        ms = _time(lambda: [torch.matmul(dY[lo:hi].t(), X[lo:hi], out=dW[e])
                            for e, lo, hi in experts], steps, warmup)
        out["dW"] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
    return out


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters: each launch reads and writes nbytes."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": reps}), flush=True)
    return 0


KERNEL_LABELS = (("combine_fwd_kernel", "combine"), ("combine_bwd_kernel", "combine_bwd"),
                 ("fwd_kernel", "fwd"), ("dx_kernel", "dX"), ("dw_kernel", "dW"),
                 ("dw_small_kernel", "dW"),
                 ("dw_reduce_kernel", "dW_reduce"), ("gather_x_kernel", "dW_gather"),
                 ("tail_reduce_kernel", "tail_reduce"),
                 ("groups_kernel", "groups"), ("route_count", "route_count"),
                 ("route_scan", "route_scan"), ("route_scatter", "route_scatter"),
                 ("route_small", "route_small"), ("Cijk_", "vendor"))


def _label(kernel_name):
    for key, lab in KERNEL_LABELS:
        if key in kernel_name:
            return lab
    return None


def _counter_means(path, counter):
    """Mean counter value (KiB for FETCH_SIZE / WRITE_SIZE) per kernel label."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        lab = _label(r["Kernel_Name"])
        if lab is None and "elementwise" in r["Kernel_Name"]:
            lab = "copy"
        if lab:
            acc.setdefault(lab, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


MI355X_XCDS, MI355X_SIMDS = 8, 256 * 4


MI355X_MAX_GHZ = 2.4


def counter_lines(sq_dir, stat_rows):
    """Per-kernel MFMA utilisation and LDS bank conflicts from an SQ counter
    pass (SQ_VALU_MFMA_BUSY_CYCLES, SQ_LDS_IDX_ACTIVE, SQ_LDS_BANK_CONFLICT,
    GRBM_GUI_ACTIVE), all from the same run.

    GRBM_GUI_ACTIVE is summed over the 8 XCDs, so a kernel's busy cycles are
    GRBM_GUI_ACTIVE / 8; MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES over those
    cycles x 1024 SIMDs.  Those cycles over the kernel's average duration in
    the trace run give its clock.  For short kernels the GRBM window is longer
    than the kernel (the profiler's dispatch around it counts too), and the
    implied clock comes out above the chip's 2.4 GHz maximum: such a row is
    marked, and its MFMA busy is taken over duration x 2.4 GHz instead, the
    most cycles the kernel can have had, which makes it a lower bound."""
    import glob
    f = glob.glob(os.path.join(sq_dir, "*counter_collection.csv"))[0]
    names = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT",
             "GRBM_GUI_ACTIVE")
    means = {n: _counter_means(f, n) for n in names}
    dur = {}
    for r in stat_rows:
        lab = _label(r["Name"])
        if lab and lab not in dur:
            dur[lab] = float(r["AverageNs"])
    out = ["", "Counters (their own pass; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 "
           "SIMDs) with cycles = GRBM_GUI_ACTIVE / 8 XCDs; clock = those cycles / the trace run's "
           f"average duration; where that clock exceeds {MI355X_MAX_GHZ} GHz the GRBM window is "
           f"longer than the kernel, the row is marked, and MFMA busy uses duration x "
           f"{MI355X_MAX_GHZ} GHz, a lower bound):", "",
           "| kernel | MFMA busy | LDS bank conflicts / LDS active | clock GHz | cycles from |",
           "|---|---|---|---|---|"]
    for lab in ("fwd", "dX", "dW", "groups", "combine", "combine_bwd", "vendor"):
        g = means["GRBM_GUI_ACTIVE"].get(lab)
        if not g or lab not in dur:
            continue
        cyc = g / MI355X_XCDS
        ghz = cyc / dur[lab]
        src = "GRBM_GUI_ACTIVE / 8"
        busy_txt = None
        if ghz > MI355X_MAX_GHZ:
            cyc = dur[lab] * MI355X_MAX_GHZ
            src = f"invalid GRBM window ({ghz:.2f} GHz implied); duration x {MI355X_MAX_GHZ} GHz"
        busy = means["SQ_VALU_MFMA_BUSY_CYCLES"].get(lab, 0.0) / (cyc * MI355X_SIMDS)
        busy_txt = f"{100 * busy:.1f}%" if ghz <= MI355X_MAX_GHZ else f">= {100 * busy:.1f}%"
        act = means["SQ_LDS_IDX_ACTIVE"].get(lab, 0.0)
        conf = means["SQ_LDS_BANK_CONFLICT"].get(lab, 0.0) / act if act else 0.0
        clock = f"{ghz:.2f}" if ghz <= MI355X_MAX_GHZ else "-"
        out.append(f"| {lab} | {busy_txt} | {conf:.4f} | {clock} | {src} |")
    return out


def memory_lines(l2_dir, tcp_dir):
    """Per-kernel L2 hit rate (TCC_HIT_sum, TCC_MISS_sum) and mean L1 -> L2
    read latency (TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum), each
    pass in its own run."""
    import glob
    f2 = glob.glob(os.path.join(l2_dir, "*counter_collection.csv"))[0]
    fp = glob.glob(os.path.join(tcp_dir, "*counter_collection.csv"))[0]
    hit, miss = _counter_means(f2, "TCC_HIT_sum"), _counter_means(f2, "TCC_MISS_sum")
    ea = _counter_means(f2, "TCC_EA0_RDREQ_sum")
    lat, req = _counter_means(fp, "TCP_TCC_READ_REQ_LATENCY_sum"), _counter_means(fp, "TCP_TCC_READ_REQ_sum")
    out = ["", "L2 and L1 -> L2 counters (two more passes; per launch):", "",
           "| kernel | L1 -> L2 read requests | L2 hit rate | L2 -> fabric read requests | "
           "mean L1 -> L2 read latency (cycles) |", "|---|---|---|---|---|"]
    for lab in ("fwd", "dX", "dW", "groups", "vendor"):
        if lab in hit and lab in req and req[lab]:
            out.append(f"| {lab} | {req[lab]:.3g} | {hit[lab] / (hit[lab] + miss[lab]):.3f} | "
                       f"{ea.get(lab, 0.0):.3g} | {lat[lab] / req[lab]:.0f} |")
    return out


def summarize(prof_dir, workload, command):
    """Turn rocprofv3 CSV output under prof_dir (trace/, fetch/, write/,
    copy_FETCH_SIZE/, copy_WRITE_SIZE/) into profiles/ summaries: the kernel
    statistics table and, per GEMM kernel, calibrated HBM bytes per launch."""
    import csv
    import glob
    stats = glob.glob(os.path.join(prof_dir, "trace", "*kernel_stats.csv"))[0]
    rows = list(csv.DictReader(open(stats)))
    fetch = _counter_means(glob.glob(os.path.join(prof_dir, "fetch", "*counter_collection.csv"))[0],
                           "FETCH_SIZE")
    write = _counter_means(glob.glob(os.path.join(prof_dir, "write", "*counter_collection.csv"))[0],
                           "WRITE_SIZE")
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        f = glob.glob(os.path.join(prof_dir, f"copy_{c}", "*counter_collection.csv"))[0]
        import csv as _csv
        vals = sorted(float(r["Counter_Value"]) for r in _csv.DictReader(open(f))
                      if r["Counter_Name"] == c)
        cal[c] = (1 << 30) / 1024.0 / vals[len(vals) // 2]   # true KiB per counter KiB (median launch)
    sha = kernel_source_sha()
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    lines = [f"# rocprofv3 kernel statistics: {workload}", "",
             f"Workload: {WORKLOAD_DESC[workload]}", "",
             "Commands (from the repository root on the GPU box):", "",
             "```", *command.strip().splitlines(), "```", "",
             f"Kernel sources sha256[:16]: `{sha}`", "",
             "| kernel | calls | average ns | total % |", "|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{float(r['Percentage']):.2f} |")
    lines += ["", "HBM traffic per launch (FETCH_SIZE x {:.3f}, WRITE_SIZE x {:.3f}; factors from a "
              "1 GiB device copy read by the same counters):".format(cal["FETCH_SIZE"],
                                                                  cal["WRITE_SIZE"]), "",
              "| kernel | read MB | written MB |", "|---|---|---|"]
    for lab in ("fwd", "dX", "dW", "groups", "combine", "combine_bwd"):
        if lab in fetch and lab in write:
            rd = fetch[lab] * 1024 * cal["FETCH_SIZE"]
            wr = write[lab] * 1024 * cal["WRITE_SIZE"]
            lines.append(f"| {lab} | {rd / 1e6:.1f} | {wr / 1e6:.1f} |")
            json.dump({"kernel_src_sha": kernel_source_sha(lab), "workload": workload, "kernel": lab,
                       "bytes_per_launch": round(rd + wr), "read_bytes": round(rd),
                       "write_bytes": round(wr), "fetch_scale": cal["FETCH_SIZE"],
                       "write_scale": cal["WRITE_SIZE"]},
                      open(os.path.join(ROOT, "profiles", f"traffic_{lab}_{workload}.json"), "w"),
                      indent=1)
    sq_dir = os.path.join(prof_dir, "sq")
    if os.path.isdir(sq_dir):
        lines += counter_lines(sq_dir, rows)
    if os.path.isdir(os.path.join(prof_dir, "l2")) and os.path.isdir(os.path.join(prof_dir, "tcp")):
        lines += memory_lines(os.path.join(prof_dir, "l2"), os.path.join(prof_dir, "tcp"))
    out = os.path.join(ROOT, "profiles", f"kernels_{workload}.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)
    return 0


def kernel_breakdown(st, per):
    """Per kernel: ms, useful TFLOP/s, algorithmic GB/s, and the fraction of
    the MFMA peak, the HBM peak and the roofline (the larger of the two
    floors over the measured time)."""
    out = {}
    for i, (label, _, fl, nb) in enumerate(st.kernels):
        t = per[i] * 1e-3
        tf = fl / t / 1e12 if fl else 0.0
        gbs = nb / t / 1e9
        roof_t = max(fl / (PEAK_BF16_TFLOPS * 1e12), nb / (PEAK_HBM_GBS * 1e9))
        out[label] = {"ms": round(per[i], 4), "tflops": round(tf, 2), "gbs": round(gbs, 1),
                      "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
                      "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                      "bound": "mfma" if fl / (PEAK_BF16_TFLOPS * 1e12) >= nb / (PEAK_HBM_GBS * 1e9)
                      else "hbm",
                      "roofline_frac": round(roof_t / t, 4)}
    return out


# MI355X raises its clock over the first tens of milliseconds of load, so the
# short configurations warm up for at least this long.
CONFIG_MIN_WARMUP_S = 0.1

# Every configuration of the benchmark besides the headline one, timed in the
# default run: (key, workload, kernels reported, steps, warmup).
CONFIG_RUNS = (
    ("1_tiny", "tiny", ("route", "fwd"), 200, 50),
    ("2_dual", "dual", ("groups",), 200, 50),
    ("4_fine_fwd", "fine_fwd", ("route", "fwd"), 30, 10),
    ("4_decode", "decode", ("route", "fwd"), 200, 50),
    ("5_fine_bwd", "fine", ("dX", "dW"), 30, 10),
)


def run_configs():
    """Time the other configurations one after another, each on its own
    resident inputs (freed before the next)."""
    out = {}
    for key, workload, labels, steps, warmup in CONFIG_RUNS:
        print(f"config {key} ({workload})", file=sys.stderr, flush=True)
        st = make_step(workload)
        per, step_ms, _ = time_step(st, steps, warmup, min_warm_s=CONFIG_MIN_WARMUP_S)
        bd = kernel_breakdown(st, per)
        out[key] = {"workload": workload, "desc": WORKLOAD_DESC[workload], "steps": steps,
                    "step_ms": round(step_ms, 4),
                    "kernels": {lab: bd[lab] for lab in labels if lab in bd}}
        del st
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # MI355X raises its clock over the first tens of milliseconds of MFMA load:
    # 3 warmup steps of the gated gate_up forward time it 5% slower than 30.
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="mixtral", choices=sorted(WORKLOAD_DESC))
    ap.add_argument("--cpu-budget", type=float, default=24.0,
                    help="seconds of CPU oracle work for the baseline, over both legs (0 "
                         "disables)")
    ap.add_argument("--configs", action=argparse.BooleanOptionalAction, default=None,
                    help="also time the other configurations (tiny, dual, fine-grained forward, "
                         "decode slice, fine-grained backward) into a `configs` object; on by "
                         "default for the headline workload")
    ap.add_argument("--vendor", action="store_true",
                    help="also time hipBLASLt (torch.matmul) on the same products, expert by "
                         "expert (always on for --workload dense)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize", metavar="PROF_DIR",
                    help="write profiles/ summaries from rocprofv3 CSVs (no GPU needed)")
    ap.add_argument("--command-file", help="text of the profiling commands, for --summarize")
    args = ap.parse_args()
    if args.summarize:
        cmd = open(args.command_file).read() if args.command_file else "(not recorded)"
        return summarize(args.summarize, args.workload, cmd)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path is not sharded "
              "across GPUs", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.copy_calibration:
        return copy_calibration()
    mg.load_library()

    if args.configs is None:
        args.configs = args.workload == "mixtral"
    st = make_step(args.workload)
    per, step_ms, wall = time_step(st, args.steps, args.warmup)
    flops = sum(k[2] for k in st.kernels)
    value = flops / (step_ms * 1e-3) / 1e12

    breakdown = kernel_breakdown(st, per)
    dominant = max(range(len(st.kernels)), key=lambda i: per[i])
    label, _, fl, nb = st.kernels[dominant]
    t = per[dominant] * 1e-3
    mfma_bound = fl / (PEAK_BF16_TFLOPS * 1e12) >= nb / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        achieved, peak, unit = fl / t / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = nb / t / 1e9, PEAK_HBM_GBS, "GB/s"
    roofline = {"bound": "mfma" if mfma_bound else "hbm", "kernel": label,
                "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(args.workload, label)}

    vendor = (vendor_reference(st, args.steps, args.warmup)
              if args.workload == "dense" or args.vendor else None)
    cpu = cpu_baseline(st, args.cpu_budget) if args.cpu_budget > 0 else None
    del st
    torch.cuda.empty_cache()
    configs = run_configs() if args.configs else None
    line = {
        "metric": "MoE grouped-GEMM useful TFLOP/s (bf16) + % of MFMA/HBM roofline, fwd/dX/dW",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "desc": WORKLOAD_DESC[args.workload],
                   "block_m_route": BLOCK_M},
        "roofline": roofline, "cpu_baseline": cpu, "breakdown": breakdown,
        **({"vendor_reference": vendor} if vendor else {}),
        **({"configs": configs} if configs else {}),
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

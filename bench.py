#!/usr/bin/env python3
"""MoE-layer throughput of libmoe on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one moe_layer call through the C ABI: router top-k (logits given)
or router GEMM + top-k, permutation, gate/up + SiLU*mul, down + weighted
combine (and the gated shared expert when the workload has one), on one
batch of synthetic input already resident in HBM.  The default workload is
the single-token decode layer (T=1, H=6144, E=256, top-8, I=2048, int4 with
fp16 group-32 scales).  To keep the 256 MB Infinity Cache from serving the
weights, every expert stays resident and each step routes with a different
row of a 64-row pool of fresh logits (given-logit workloads), or rotates
through 4 independent weight sets (router workloads).

Prints one JSON line on stdout: the headline tokens/s, the dominant kernel's
roofline fraction (its duration measured with HIP events on the launch
stream through moe_layer_profiled), the per-stage device times of the
stages that ran, a "prefill" object with the same figures for the skewed
2048-token prefill (tiled weights, the library's AUTO path, the same steps
and warmup; the metric's MFMA half), and the CPU oracle's rate on a bounded
sample of the headline workload.  Details go to stderr.
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_synth as S  # noqa: E402

METRIC = "MoE-layer tokens/s at 1 GPU; decode HBM GB/s %, prefill MFMA % of peak"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_F16_PEAK_TFS = 2500.0  # MI355X dense fp16/bf16 MFMA
LOGIT_POOL = 64
WEIGHT_SETS = {"decode_batch": 4, "prefill_shared": 4}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """hipEvent_t handles through the HIP runtime (torch already loaded it)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def event(self) -> int:
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e: int, stream: int) -> None:
        assert self.L.hipEventRecord(e, stream) == 0

    def ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        assert self.L.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value

    # hipDeviceAttribute_t values (hip_runtime_api.h): peak shader and
    # memory clocks, in kHz
    ATTR_CLOCK_RATE, ATTR_MEMORY_CLOCK_RATE = 5, 60

    def attribute(self, attr: int, device: int = 0) -> int:
        v = ctypes.c_int()
        assert self.L.hipDeviceGetAttribute(ctypes.byref(v), attr, device) == 0
        return v.value


def counted_traffic(kernel: str, workload: str, gemm: bool, fmt: str = "int4",
                    layout: str = "rows"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/<workload>_<gemv|gemm>_hbm_counters.md), or None when
    there is none, it was taken for another weight layout, or the kernel
    sources changed since the counters were taken."""
    import hashlib
    if fmt != "int4":
        return None
    f = os.path.join(ROOT, "profiles", "%s_%s_hbm_counters.md" % (workload, "gemm" if gemm else "gemv"))
    if not os.path.exists(f):
        return None
    kv = {}
    for line in open(f):
        if ":" in line and not line.startswith(("#", "|", "`")):
            k_, v_ = line.split(":", 1)
            kv[k_.strip()] = v_.strip()
    h = hashlib.sha256()
    if gemm:
        srcs = ("gemm.hip",)
    else:
        srcs = ("topk.h", "gemv_impl.h", "gemv_tiled.hip" if layout == "tiled" else "gemv.hip")
    for src in ("device.h", "kernels.h") + srcs:
        h.update(open(os.path.join(ROOT, "quantized_expert_mlp_amd", "csrc", src), "rb").read())
    if kv.get("kernel") != kernel or kv.get("source_sha256") != h.hexdigest()[:16]:
        return None
    if kv.get("layout", "rows") != layout:
        return None
    return int(kv["traffic_bytes_per_launch"])


def router_bias(router: str, E: int):
    """Selection bias of the variant routers (None without one): N(0, 0.05)
    beside sigmoid scores, N(0, 1/E) beside softmax probabilities."""
    if not router.endswith("-bias"):
        return None
    sd = 0.05 if router.startswith("sigmoid") else 1.0 / E
    return (np.random.default_rng([E, 77]).standard_normal(E) * sd).astype(np.float32)


def routing_counts(logits: np.ndarray, k: int, top_p: float = 0.0, router: str = "softmax",
                   bias=None):
    """(distinct experts, slots) among the top-k picks of every row, for the
    byte and flop accounting; with 0 < top_p < 1, among the picks expert
    top-p keeps; for a variant router, the picks of its selection keys."""
    if router != "softmax":
        z = logits.astype(np.float64)
        if router.startswith("sigmoid"):
            key = 1.0 / (1.0 + np.exp(-z))
        else:
            key = np.exp(z - z.max(axis=1, keepdims=True))
            key /= key.sum(axis=1, keepdims=True)
        if bias is not None:
            key = key + bias.astype(np.float64)
        order = np.argsort(-key, axis=1, kind="stable")[:, :k]
        return len(np.unique(order)), order.size
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    if not 0.0 < top_p < 1.0:
        return len(np.unique(order)), order.size
    z = logits.astype(np.float64)
    P = np.exp(z - z.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    pk = np.take_along_axis(P, order, axis=1)
    kept = order[(np.cumsum(pk, axis=1) - pk) < top_p]
    return len(np.unique(kept)), kept.size


def stage_work(wl, T, U, gemm, fmt="int4", slots=None):
    """Algorithmic bytes and flops of the gate/up and down launches of one call.

    Counted: the touched experts' packed nibbles and group scales (fp16 for
    int4, one byte for MXFP4), activations in, hidden rows (fp16) out/in, y
    out.  Not counted: untouched experts.  On the MFMA path the shared
    expert's tiles run inside the routed launches, so its work is added to
    theirs."""
    H, I = wl.H, wl.I
    slots = T * wl.k if slots is None else slots
    act = 2
    sb = 1 if fmt == "mxfp4" else 2
    gu_w = U * 2 * (I * H // 2 + I * (H // 32) * sb)
    dn_w = U * (H * I // 2 + H * (I // 32) * sb)
    sh_gu = sh_dn = 0
    if wl.SI:
        sh_gu = 2 * (wl.SI * H // 2 + wl.SI * (H // 32) * sb) + T * H * 2 + T * wl.SI * act
        sh_dn = (H * wl.SI // 2 + H * (wl.SI // 32) * sb) + T * wl.SI * act + T * H * 4
    work = {
        "gate_up": {"bytes": gu_w + T * H * 2 + slots * I * act, "flops": 4.0 * slots * H * I},
        "down": {"bytes": dn_w + slots * I * act + T * H * 4, "flops": 2.0 * slots * H * I},
        "shared_gate_up": {"bytes": sh_gu, "flops": 4.0 * T * H * wl.SI},
        "shared_down": {"bytes": sh_dn, "flops": 2.0 * T * H * wl.SI},
    }
    if gemm:
        for routed, shared in (("gate_up", "shared_gate_up"), ("down", "shared_down")):
            for key in ("bytes", "flops"):
                work[routed][key] += work[shared][key]
                work[shared][key] = 0
    return work


def build_sets(wl, nsets, seed0=0, tiled=False, fmt="int4"):
    """Device-resident inputs; with tiled=True the planes are packed into the
    tiled layout once, as at weight-load time."""
    import torch

    import quantized_expert_mlp_amd as moe

    def pack(plane, N, K):
        q, s_ = plane
        dq, ds = torch.empty_like(q), torch.empty_like(s_)
        moe.moe_pack_weights((q, s_), q.numel() // (N * K // 2), N, K, (dq, ds),
                             format=moe.MOE_FORMAT_MXFP4 if fmt == "mxfp4" else moe.MOE_FORMAT_INT4)
        torch.cuda.synchronize()
        return dq, ds

    def dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()

    sets = []
    for r in range(nsets):
        inp = S.make_layer_inputs(wl, seed=seed0 + r, fmt=fmt)
        d = {
            "inp": inp,
            "x": dev(inp.x),
            "planes": {p: (dev(q), dev(s)) for p, (q, s) in inp.planes.items()},
            "w_router": None if inp.w_router is None else dev(inp.w_router),
            "shared": None if inp.shared is None else [
                (dev(inp.shared[p][0]), dev(inp.shared[p][1])) for p in S.PLANES],
            "shared_gate": None if inp.shared_gate is None else dev(inp.shared_gate),
        }
        if tiled:
            dims = {"gate": (wl.I, wl.H), "up": (wl.I, wl.H), "down": (wl.H, wl.I)}
            d["planes"] = {p: pack(pl, *dims[p]) for p, pl in d["planes"].items()}
            if d["shared"] is not None:
                sd = [(wl.SI, wl.H), (wl.SI, wl.H), (wl.H, wl.SI)]
                d["shared"] = [pack(pl, *nk) for pl, nk in zip(d["shared"], sd)]
        sets.append(d)
        inp.planes = None  # host copies no longer needed
    return sets


def cpu_baseline(wl, seconds_hint: float, fmt: str = "int4", router: str = "softmax", bias=None):
    """The oracle as it stands, on a bounded sample of the workload's tokens:
    a short first pass sizes the sample so the timed pass takes about
    `seconds_hint` seconds (decode: distinct logits rows for the same
    activation row; batches: a seeded subset of the token rows)."""
    import oracle
    threads = oracle.set_threads(min(16, os.cpu_count() or 1))
    inp = S.make_layer_inputs(wl, seed=0, fmt=fmt)
    if wl.logits == "router":
        logits_all = oracle.router_logits(inp.x, inp.w_router)
    else:
        logits_all = inp.logits
    gate = "sigmoid" if router.startswith("sigmoid") else "softmax"

    def run(n):
        if wl.T == 1:
            logits = S.draw_logits(S.Workload("pool", wl.wid, n, wl.H, wl.E, wl.k, wl.I, wl.SI,
                                              wl.logits, ""), seed=1000)
            x, rows = np.repeat(inp.x, n, axis=0), None
        else:
            logits, x = logits_all, inp.x
            rows = sorted(np.random.default_rng(7).choice(wl.T, n, replace=False).tolist())
        t0 = time.perf_counter()
        oracle.layer(x, logits, wl.k, inp.planes, inp.shared, inp.shared_gate, rows=rows,
                     fmt=fmt, gate=gate, bias=bias)
        return time.perf_counter() - t0

    cap = 64 * threads if wl.T == 1 else wl.T
    n0 = min(threads, cap)
    dt0 = run(n0)
    n = int(min(cap, max(n0, round(n0 * seconds_hint / max(dt0, 1e-6)))))
    dt = run(n)
    if wl.T == 1:
        sample = "%d decode tokens (distinct logits rows), %d threads" % (n, threads)
    else:
        sample = "%d of %d token rows, %d threads" % (n, wl.T, threads)
    # the same on one thread, on a sample sized for about a third of the time
    oracle.set_threads(1)
    dt1 = run(1)
    n1 = int(min(cap, max(1, round(seconds_hint / 3 / max(dt1, 1e-6)))))
    dt1 = run(n1)
    oracle.set_threads(threads)
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2),
            "single_thread": {"value": n1 / dt1, "unit": "tokens/s", "tokens": n1,
                              "seconds": round(dt1, 2)}}


def cpu_info():
    """The host's CPU count, the CPUs this process may run on, and the model."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count()
    return {"host_cpus": os.cpu_count(), "allowed_cpus": allowed, "cpu_model": model}


def measure(wl, args, layout, path_name, hip, steps, warmup, fold=False):
    """Time exactly `steps` moe_layer calls (after `warmup`) on workload wl,
    then the same calls through moe_layer_profiled for per-stage device time
    and the dominant kernel's roofline.  Returns a dict."""
    import torch

    import quantized_expert_mlp_amd as moe

    T = wl.T
    nsets = WEIGHT_SETS.get(wl.name, 1)
    log("workload %s: %s; %d weight set(s), layout %s" % (wl.name, wl.description, nsets, layout))
    t0 = time.perf_counter()
    tiled = layout == "tiled"
    mx = args.format == "mxfp4"
    sets = build_sets(wl, nsets, tiled=tiled, fmt=args.format)
    log("inputs resident in %.1f s" % (time.perf_counter() - t0))

    bias_np = router_bias(args.router, wl.E)
    bias = None if bias_np is None else torch.from_numpy(bias_np).cuda()
    rc = dict(top_p=args.top_p, router=args.router, bias=bias_np)

    # per-step inputs: logits pool (given-logit workloads) or weight-set rotation
    if wl.logits in ("given", "zipf"):
        pool_np = [S.draw_logits(wl, seed=100 + i) for i in range(LOGIT_POOL)] \
            if wl.T == 1 else [S.draw_logits(wl, seed=100 + i) for i in range(4)]
        pool = [torch.from_numpy(p).cuda() for p in pool_np]
        counts = [routing_counts(p, wl.k, **rc) for p in pool_np]
    else:
        pool_np, pool = None, None
        counts = []
        for s in sets:  # byte accounting only: which experts the router picks
            L = S.bf16_bits_to_f32(s["inp"].x) @ s["inp"].w_router.T
            counts.append(routing_counts(L, wl.k, **rc))
    touched = [c[0] for c in counts]
    nvar = len(pool) if pool is not None else len(sets)

    def shape(path):
        return moe.make_shape(T, wl.H, wl.E, wl.k, wl.I, wl.SI, path=path,
                              layout=moe.MOE_LAYOUT_TILED if tiled else moe.MOE_LAYOUT_ROWS,
                              format=moe.MOE_FORMAT_MXFP4 if mx else moe.MOE_FORMAT_INT4,
                              top_p=args.top_p,
                              score=moe.MOE_SCORE_SIGMOID if args.router.startswith("sigmoid")
                              else moe.MOE_SCORE_SOFTMAX, select_bias=bias)

    path = {"auto": moe.MOE_PATH_AUTO, "gemv": moe.MOE_PATH_GEMV, "gemm": moe.MOE_PATH_GEMM}[path_name]
    sh = shape(path)
    if moe.moe_workspace_bytes(sh) == 0:
        sys.exit("bench.py: workload %s is not served with --path %s --layout %s --format %s"
                 % (wl.name, path_name, layout, args.format))
    # the path AUTO takes: the GEMV's workspace holds no fp16 activation copy,
    # so AUTO sized like the GEMV (and the GEMV served) means the GEMV
    gemm = path_name == "gemm" or (path_name == "auto" and moe.moe_workspace_bytes(sh) !=
                                   moe.moe_workspace_bytes(shape(moe.MOE_PATH_GEMV)))
    nbytes = moe.moe_workspace_bytes(sh)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((T, wl.H), dtype=torch.float32, device="cuda")
    if fold:
        residual = torch.from_numpy(S.draw_residual(wl)).cuda()
        norm_w = torch.from_numpy(S.draw_norm_weight(wl)).cuda()
        x_next = torch.empty((T, wl.H), dtype=torch.int16, device="cuda")

    def call(i, events=None):
        s = sets[i % len(sets)] if pool is None else sets[0]
        lg = pool[i % len(pool)] if pool is not None else None
        wr = s["w_router"] if pool is None else None
        if fold and events is None:
            moe.moe_layer_residual_rmsnorm(sh, s["x"], lg, wr, s["planes"]["gate"],
                                           s["planes"]["up"], s["planes"]["down"], s["shared"],
                                           s["shared_gate"], residual, norm_w, 1e-6, x_next,
                                           None, None, ws, nbytes)
            return None
        args_ = (sh, s["x"], lg, wr, s["planes"]["gate"], s["planes"]["up"], s["planes"]["down"],
                 s["shared"], s["shared_gate"], y, None, None, None, ws, nbytes)
        if events is None:
            moe.moe_layer(*args_)
            return None
        return moe.moe_layer_profiled(*args_, events=events)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` layer calls; HIP events on the launch
    # stream between batches of `batch` calls give the spread over batches
    batch = max(1, min(20, steps))
    nb = steps // batch
    bev = [hip.event() for _ in range(nb + 1)]
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i % batch == 0 and i // batch < nb:
            hip.record(bev[i // batch], stream)
        call(i)
        if i + 1 == nb * batch:
            hip.record(bev[nb], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps
    tokens_per_s = T * steps / wall
    per_call = np.array([hip.ms(bev[j], bev[j + 1]) * 1e3 / batch for j in range(nb)])
    timing = {"batch_calls": batch, "batches": nb,
              "median_us_per_call": round(float(np.median(per_call)), 3),
              "p10_us_per_call": round(float(np.percentile(per_call, 10)), 3),
              "p90_us_per_call": round(float(np.percentile(per_call, 90)), 3)}

    # ---- per-stage device time (HIP events on the launch stream); with
    # fold these come from moe_layer_profiled, whose kernels are the folded
    # step's except the final norm launch.  Only stages whose kernels ran.
    ev = [[hip.event() for _ in range(2 * len(moe.STAGES))] for _ in range(steps)]
    ran = set()
    for i in range(steps):
        ran.update(call(i, ev[i]))
    torch.cuda.synchronize()
    stage_ms = {name: 0.0 for name in moe.STAGES[1:] if name in ran}
    for i in range(steps):
        for j, name in enumerate(moe.STAGES):
            if name in stage_ms:
                stage_ms[name] += hip.ms(ev[i][2 * j], ev[i][2 * j + 1])
    for k_ in stage_ms:
        stage_ms[k_] /= steps
    U = float(np.mean([touched[i % nvar] for i in range(steps)]))
    kept_slots = float(np.mean([counts[i % nvar][1] for i in range(steps)]))
    work = stage_work(wl, T, U, gemm, args.format, kept_slots)
    dom = max((s_ for s_ in ("gate_up", "down", "shared_gate_up", "shared_down") if s_ in stage_ms),
              key=lambda s_: stage_ms[s_])
    dur_s = stage_ms[dom] * 1e-3
    # The roof the kernel is held to: the MFMA peak when its arithmetic
    # intensity reaches half the ridge point (peak flops / peak bytes, about
    # 312 flop/byte), else HBM bandwidth (the GEMV, and the MFMA path at
    # decode-sized batches, where each expert's weights serve a few rows).
    ridge = MFMA_F16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    mfma_bound = gemm and work[dom]["flops"] >= 0.5 * ridge * work[dom]["bytes"]
    if mfma_bound:
        achieved = work[dom]["flops"] / dur_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFS, 4)}
    else:
        achieved = work[dom]["bytes"] / dur_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["kernel"] = dom
    roof["kernel_us"] = round(stage_ms[dom] * 1e3, 3)
    roof["algorithmic_bytes"] = int(work[dom]["bytes"])
    roof["algorithmic_flops"] = int(work[dom]["flops"])
    roof["intensity_flop_per_byte"] = round(work[dom]["flops"] / work[dom]["bytes"], 1)
    roof["traffic"] = counted_traffic(dom, wl.name, gemm, args.format, layout)
    layer_bytes = sum(w_["bytes"] for w_ in work.values())
    layer_flops = sum(w_["flops"] for w_ in work.values())
    log("stage device time (us): " + ", ".join("%s %.2f" % (k_, v * 1e3)
                                                for k_, v in stage_ms.items()))
    log("touched experts per call %.1f; layer: %.2f us/step wall, %.1f GB/s, %.1f TFLOP/s"
        % (U, ms_per_step * 1e3, layer_bytes / (ms_per_step * 1e-3) / 1e9,
           layer_flops / (ms_per_step * 1e-3) / 1e12))
    log("dominant kernel %s: %.2f us, %s" % (dom, stage_ms[dom] * 1e3, roof))
    del sets, pool, ws
    torch.cuda.empty_cache()
    return {
        "ms_per_step": ms_per_step, "tokens_per_s": tokens_per_s, "gemm": gemm, "timing": timing,
        "stage_us": {k_: round(v * 1e3, 3) for k_, v in stage_ms.items()},
        "roofline": roof, "nvar": nvar, "pool": pool_np is not None,
        "layer": {"touched_experts": round(U, 1),
                  "tflops": round(layer_flops / (ms_per_step * 1e-3) / 1e12, 1),
                  "gbs": round(layer_bytes / (ms_per_step * 1e-3) / 1e9, 1)},
    }


def fold_router_chain(wl, args, hip, steps, warmup):
    """The decode layer chained through its residual step, two ways, each
    step a full layer: (a) the step's own router GEMM launch from w_router
    (moe_layer_residual_rmsnorm with w_router), (b) the router folded into the
    previous step's norm launch (next_w_router), its logits the given logits
    of the next step.  Returns ms/step of both."""
    import torch

    import quantized_expert_mlp_amd as moe

    sets = build_sets(wl, 1)
    s = sets[0]
    W = torch.from_numpy(np.random.default_rng([wl.wid, 92]).normal(
        0.0, 0.02, (wl.E, wl.H)).astype(np.float32)).cuda()
    sh = moe.make_shape(wl.T, wl.H, wl.E, wl.k, wl.I, wl.SI)
    nbytes = moe.moe_workspace_bytes(sh)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    residual = torch.from_numpy(S.draw_residual(wl)).cuda()
    norm_w = torch.from_numpy(S.draw_norm_weight(wl)).cuda()
    x = [s["x"].clone(), s["x"].clone()]
    lg = [torch.from_numpy(S.draw_logits(wl, seed=100)).cuda(),
          torch.empty((wl.T, wl.E), dtype=torch.float32, device="cuda")]
    P = s["planes"]

    def step_unfused(i):
        moe.moe_layer_residual_rmsnorm(sh, x[i % 2], None, W, P["gate"], P["up"], P["down"],
                                       s["shared"], s["shared_gate"], residual, norm_w, 1e-6,
                                       x[(i + 1) % 2], None, None, ws, nbytes)

    def step_folded(i):
        moe.moe_layer_residual_rmsnorm(sh, x[i % 2], lg[i % 2], None, P["gate"], P["up"],
                                       P["down"], s["shared"], s["shared_gate"], residual, norm_w,
                                       1e-6, x[(i + 1) % 2], None, None, ws, nbytes,
                                       next_w_router=W, next_E=wl.E, next_logits=lg[(i + 1) % 2])

    out = {}
    for name, fn in (("own_router_launch", step_unfused), ("router_folded_into_norm", step_folded)):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        out[name] = round((time.perf_counter() - t0) * 1e3 / steps, 5)
        log("fold chain %s: %.2f us/step" % (name, out[name] * 1e3))
    return out


def read_probe(hip, sizes=(113_246_208, 1 << 30), widths=(1024, 2048, 4096, 8192)):
    """Best streaming-read rate of moe_debug_read_probe over sizes and
    launch widths (the practical HBM read ceiling for the decode GEMVs)."""
    import torch

    import quantized_expert_mlp_amd as moe

    buf = torch.randint(0, 1 << 30, (1 << 28,), dtype=torch.int32, device="cuda")  # 1 GiB
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    rows = []
    for nbytes in sizes:
        for wgs in widths:
            for _ in range(5):
                moe.moe_debug_read_probe(buf, nbytes, wgs, sink)
            e = [hip.event() for _ in range(2)]
            best = None
            for _ in range(20):
                hip.record(e[0], st.cuda_stream)
                moe.moe_debug_read_probe(buf, nbytes, wgs, sink)
                hip.record(e[1], st.cuda_stream)
                torch.cuda.synchronize()
                ms = hip.ms(e[0], e[1])
                best = ms if best is None else min(best, ms)
            rows.append({"bytes": nbytes, "workgroups": wgs, "best_us": round(best * 1e3, 2),
                         "gbs": round(nbytes / (best * 1e-3) / 1e9, 1)})
            log("read probe %d bytes, %d workgroups: %.2f us, %.1f GB/s"
                % (nbytes, wgs, best * 1e3, rows[-1]["gbs"]))
    del buf
    torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="decode", choices=list(S.WORKLOADS))
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "gemm"],
                    help="expert-MLP path (auto: the library's choice)")
    ap.add_argument("--layout", default="tiled", choices=["rows", "tiled"],
                    help="weight plane layout (tiled: packed once with moe_pack_weights, as at "
                         "weight-load time, served by both expert paths; rows: the planes as "
                         "drawn)")
    ap.add_argument("--format", default="int4", choices=["int4", "mxfp4"],
                    help="expert weight format (mxfp4: e2m1 nibbles, ue8m0 exponent per 32 "
                         "inputs)")
    ap.add_argument("--fold", action="store_true",
                    help="time the layer with its combine folded into the residual add + "
                         "RMSnorm (moe_layer_residual_rmsnorm) instead of moe_layer")
    ap.add_argument("--top-p", type=float, default=0.0,
                    help="expert top-p after the top-k (0 < p < 1; default off)")
    ap.add_argument("--router", default="softmax",
                    choices=["softmax", "sigmoid", "softmax-bias", "sigmoid-bias"],
                    help="router: the plain softmax top-k, or a variant (sigmoid scores "
                         "and/or a seeded selection bias)")
    ap.add_argument("--prefill-workload", default="prefill_skewed",
                    choices=[w for w in S.WORKLOADS if w.startswith("prefill")],
                    help="the prefill workload timed beside a decode headline (the metric's "
                         "prefill half), with --prefill-layout weights through AUTO")
    ap.add_argument("--prefill-layout", default="tiled", choices=["rows", "tiled"])
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (HBM counter calibration)")
    ap.add_argument("--fold-router", action="store_true",
                    help="only time the layer chained through its residual step with its own "
                         "router GEMM launch against the router folded into the previous "
                         "step's norm launch, and print both")
    ap.add_argument("--probe-read", action="store_true",
                    help="only run the streaming-read probe (moe_debug_read_probe) and print "
                         "its rates")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_expert_mlp_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        # A copy of known size: its FETCH_SIZE / WRITE_SIZE counters give the
        # scale between counter readings and bytes moved.
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d x 256 MiB" % max(1, args.steps))
        return
    moe.lib()
    hip = Hip()
    if args.probe_read:
        print(json.dumps({"probe": "moe_debug_read_probe", "rows": read_probe(hip)}), flush=True)
        return
    if args.router != "softmax" and 0.0 < args.top_p < 1.0:
        sys.exit("bench.py: --top-p applies to the plain softmax router only")
    if args.fold_router:
        wl = S.WORKLOADS[args.workload]
        print(json.dumps({"fold_router_chain": wl.name, "steps": args.steps,
                          "ms_per_step": fold_router_chain(wl, args, hip, args.steps,
                                                           args.warmup)}), flush=True)
        return

    wl = S.WORKLOADS[args.workload]
    m = measure(wl, args, args.layout, args.path, hip, args.steps, args.warmup, fold=args.fold)
    gemm = m["gemm"]
    mx = args.format == "mxfp4"
    # an HBM-bound line is also held to this box's streaming-read probe
    probe = None
    if m["roofline"]["bound"] == "hbm":
        best = max(read_probe(hip, sizes=(113_246_208,), widths=(2048, 4096)),
                   key=lambda r: r["gbs"])
        probe = {"kernel": "moe_debug_read_probe", "bytes": best["bytes"],
                 "workgroups": best["workgroups"], "gbs": best["gbs"]}
        m["roofline"]["probe_gbs"] = best["gbs"]
        m["roofline"]["frac_of_probe"] = round(m["roofline"]["achieved"] / best["gbs"], 4)
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "arch": props.gcnArchName,
              "compute_units": props.multi_processor_count,
              "sclk_peak_mhz": hip.attribute(Hip.ATTR_CLOCK_RATE) // 1000,
              "mclk_peak_mhz": hip.attribute(Hip.ATTR_MEMORY_CLOCK_RATE) // 1000}

    prefill = None
    if not args.no_prefill and not wl.name.startswith("prefill"):
        pw = S.WORKLOADS[args.prefill_workload]
        pm = measure(pw, args, args.prefill_layout, "auto", hip, args.steps, args.warmup)
        prefill = {
            "workload": pw.name, "description": pw.description,
            "layout": args.prefill_layout, "path": "auto",
            "expert_path": "grouped fp16 MFMA GEMM" if pm["gemm"] else "streaming GEMV",
            "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(pm["ms_per_step"], 5),
            "tokens_per_s": round(pm["tokens_per_s"], 1),
            "layer": pm["layer"], "roofline": pm["roofline"], "stage_us": pm["stage_us"],
            "timing": pm["timing"],
        }

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds, args.format, args.router,
                           router_bias(args.router, wl.E))
        cpu.update(cpu_info())
        log("cpu oracle: %s" % cpu)

    out = {
        "metric": METRIC,
        "value": round(m["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if gemm or mx else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "T": wl.T, "H": wl.H,
                   "E": wl.E, "k": wl.k, "I": wl.I, "SI": wl.SI,
                   "weights": ("mxfp4: e2m1, ue8m0 exponent per 32 inputs" if mx
                               else "int4 offset-binary, fp16 scale per 32 inputs"),
                   "layout": args.layout,
                   "path": args.path,
                   "top_p": args.top_p if 0.0 < args.top_p < 1.0 else None,
                   "router": args.router,
                   "step": ("layer + residual add + RMSnorm (moe_layer_residual_rmsnorm)"
                            if args.fold else "layer (moe_layer)"),
                   "expert_path": "grouped fp16 MFMA GEMM" if gemm else
                   "streaming %s GEMV" % args.format,
                   "input_rotation": ("%d logits rows" % m["nvar"]) if m["pool"]
                   else ("%d weight sets" % m["nvar"])},
        "roofline": m["roofline"],
        "timing": m["timing"],
        "hbm_probe": probe,
        "device": device,
        "stage_us": m["stage_us"],
        "layer": m["layer"],
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

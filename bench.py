#!/usr/bin/env python3
"""Benchmark of the LatentMoE MXFP4 (w4a16) layer on one MI355X.

One step = one lmoe_forward over one batch: router, top-k, grouping, routed
experts, shared experts, combine. Headline: K3-shaped batch-1 decode (T=1,
L=3584, E=896 resident experts, k=16, I=2048, two shared experts), reported as
algorithmic HBM GB/s. Each decode step takes the next of 64 distinct tokens and
the next of 4 device copies of the dense (router + shared) weights, so neither
the routed experts nor the dense weights are served from the 256 MB last-level
cache across steps. A same-token, same-weights figure is reported separately as
"warm". The prefill chunk (T=4096) is measured too and reported as bf16 MFMA
TFLOP/s in the "prefill" object.

Algorithmic work (only what the layer must move or compute):
  bytes = D*3*L*I*17/32 + S*3*L*Is*2 + 2*L*E + 4*T*L     (D = distinct experts)
  flops = 6*L*I*T*k + 6*L*Is*T*S + 2*T*L*E

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0     # dense fp8 MFMA (an FP8 x FP4 product runs at the fp8 rate)
FP4_PEAK_TFLOPS = 10100.0    # dense fp4 MFMA
# quantised activations of the routed experts (lmoe_exec.act_format):
# workload-name suffix -> (act format name, MFMA peak of its routed GEMMs)
ACT_SUFFIX = {"_a8": ("e4m3", FP8_PEAK_TFLOPS), "_a4": ("e2m1", FP4_PEAK_TFLOPS)}
N_TOKENS = 64
N_REPLICAS = 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
HOLD_MS = 30.0               # spin the GPU this long while the host enqueues


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# HIP events (ctypes on the HIP runtime torch already loaded)
# ---------------------------------------------------------------------------
class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self) -> int:
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return e.value

    def record(self, ev: int, stream: int) -> None:
        rc = self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a: int, b: int) -> float:
        self.lib.hipEventSynchronize(ctypes.c_void_p(b))
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)


# ---------------------------------------------------------------------------
# Work model
# ---------------------------------------------------------------------------
def algorithmic(d, D: int, logits_given: bool):
    L, I, E, T, k, S, Is = d.L, d.I, d.E, d.T, d.k, d.S, d.Is
    fp4_row = 17.0 / 32.0  # bytes per MXFP4 weight: half a byte + one byte per 32
    st_bytes = {
        "router": 0 if logits_given else 2 * L * E + 2 * T * L,
        "topk": 0, "permute": 0,
        "gate_up": D * 2 * I * L * fp4_row + 2 * T * L,
        "down": D * L * I * fp4_row,
        "shared_gate_up": S * 2 * Is * L * 2 + (2 * T * L if S else 0),
        "shared_down": S * L * Is * 2,
        "combine": 2 * T * L,
    }
    st_flops = {
        "router": 0 if logits_given else 2 * T * L * E,
        "topk": 0, "permute": 0,
        "gate_up": 4 * L * I * T * k, "down": 2 * L * I * T * k,
        "shared_gate_up": 4 * L * Is * T * S, "shared_down": 2 * L * Is * T * S,
        "combine": 0,
    }
    total_bytes = D * 3 * L * I * fp4_row + S * 3 * L * Is * 2 + \
        (0 if logits_given else 2 * L * E) + 4 * T * L
    total_flops = 6 * L * I * T * k + 6 * L * Is * T * S + (0 if logits_given else 2 * T * L * E)
    return total_bytes, total_flops, st_bytes, st_flops


# Kernel that does each stage's work (names as rocprofv3 reports them).
STAGE_KERNEL = {
    "router": "router_kernel", "topk": "topk_kernel", "permute": "permute_kernel",
    "combine": "combine_kernel",
}


def stage_kernel(stage: str, large: bool, sh_large: bool, d=None, logits_given=False) -> str:
    if stage == "topk" and d is not None:
        # one wave per token when the router leaves one partial sum per
        # logit, one workgroup per token when it splits K (small T)
        tok = 128 if d.T > 512 else 64
        tiles = -(-d.E // 64) * -(-d.T // tok)
        target = 256 if tok == 128 else 512
        ks = 1 if logits_given else max(1, min(d.L // 32, -(-target // tiles)))
        return f"topk_kernel<{'false' if ks == 1 else 'true'}>"
    if stage == "permute" and d is not None and d.T > 512:
        return "chunk_scan_kernel"
    if stage == "router" and d is not None:
        return f"router_kernel<{128 if d.T > 512 else 64}>"
    if stage in STAGE_KERNEL:
        return STAGE_KERNEL[stage]
    kind = {"gate_up": ("true", "true"), "down": ("false", "true"),
            "shared_gate_up": ("true", "false"), "shared_down": ("false", "false")}[stage]
    if stage.startswith("shared") and not sh_large:
        # bf16 16-row tiles for the shared experts of up to 64 tokens
        return f"gemm_small_kernel<{kind[0]}>"
    # the large MXFP4 kernel stages whole exponent rows in LDS when K/32 is a
    # multiple of 16 and at most 112 (third template argument)
    K = None if d is None else {"gate_up": d.L, "down": d.I}.get(stage)
    win = K is not None and (K // 32) % 16 == 0 and K // 32 <= 112
    return f"gemm_large_kernel<{kind[0]}, {kind[1]}, {str(win).lower()}>"


# The source files a kernel is compiled from: its own file and the headers
# every kernel file includes. Counter traffic is kept per kernel, keyed to a
# hash of these files, so a change elsewhere does not discard it.
KERNEL_SOURCES = {
    "decode_kernel": "decode.hip",
    "decode_multi_kernel": "decode_multi.hip",
    "gemm_packed": "packed.hip",
    "pack_": "packed.hip",
    "quantize_act": "packed.hip",
    "read_stream": "experts.hip",
    "mfma_rate": "measure.hip",
    "gemm_large": "experts.hip",
    "gemm_small": "experts.hip",
    "router_kernel": "route.hip",
    "topk_kernel": "route.hip",
    "chunk_": "route.hip",
    "permute_kernel": "route.hip",
    "combine_kernel": "experts.hip",
    "dense_": "dense.hip",
    "rmsnorm": "dense.hip",
}


def sources_sha(kernel: str = None) -> str:
    """Hash of the kernel's source files (all of csrc when kernel is None)."""
    csrc = os.path.join(ROOT, "mxfp4_latent_mixture_amd", "csrc")
    names = sorted(os.listdir(csrc))
    if kernel is not None:
        own = [f for k, f in KERNEL_SOURCES.items() if kernel.startswith(k)]
        names = [n for n in names if n.endswith(".h") or n in own]
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def kernel_short_name(name: str) -> str:
    """rocprofv3's kernel name without 'void', namespace and arguments."""
    return name.replace("void ", "").replace("lmoe::", "").split("(")[0]


def traffic_from(pmc_dir: str, workload: str) -> dict:
    """Merge into profiles/pmc_traffic.json the HBM bytes per dispatch of the
    kernels in two rocprofv3 --pmc runs of this bench with --calib-copy-mib
    1024: <pmc_dir>/fetch (FETCH_SIZE) and <pmc_dir>/write (WRITE_SIZE), each
    holding a *_counter_collection.csv. Each kernel's figure is its mean
    FETCH_SIZE and WRITE_SIZE (KiB) scaled by what the same counters read for
    the 1 GiB device copy, filed under `workload` (the single-token kernel
    always under decode), and keyed to a hash of the kernel's sources."""
    import csv
    import glob

    def read(tag):
        acc = {}
        for path in glob.glob(os.path.join(pmc_dir, tag, "*counter_collection.csv")):
            with open(path) as f:
                for r in csv.DictReader(f):
                    acc.setdefault(kernel_short_name(r["Kernel_Name"]), []).append(
                        float(r["Counter_Value"]))
        return acc

    f, w = read("fetch"), read("write")
    copy = [k for k in f if "copyBuffer" in k]
    if not copy:
        raise SystemExit("no device copy in the counter runs: run the bench with "
                         "--calib-copy-mib 1024")
    cal_f, cal_w = max(f[copy[0]]), max(w[copy[0]])
    fs, ws = round(1048576.0 / cal_f, 4), round(1048576.0 / cal_w, 4)
    try:
        with open(TRAFFIC_FILE) as fh:
            out = json.load(fh)
    except (OSError, ValueError):
        out = {}
    out["calibration"] = {"copy_bytes_each_way": 1 << 30, "fetch_kib": cal_f,
                          "write_kib": cal_w, "fetch_scale": fs, "write_scale": ws}
    kernels = out.setdefault("kernels", {})
    for k in sorted(f):
        if not any(k.startswith(p) for p in KERNEL_SOURCES) or k not in w:
            continue
        fk = sum(f[k]) / len(f[k])
        wk = sum(w[k]) / len(w[k])
        tag = "decode" if k == FUSED_KERNEL else workload
        if not isinstance(kernels.get(k), dict) or "traffic_bytes" in kernels.get(k, {}):
            kernels[k] = {}
        kernels[k][tag] = {"sources_sha": sources_sha(k), "dispatches": len(f[k]),
                           "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                           "traffic_bytes": int(round((fk * fs + wk * ws) * 1024))}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
    return out


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` in `workload` from the committed PMC
    summary, or None when absent or taken on different sources of that
    kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(kernel, {}).get(workload)
    if k is None or k.get("sources_sha") != sources_sha(kernel):
        return None
    return k.get("traffic_bytes")


# ---------------------------------------------------------------------------
# Device setup
# ---------------------------------------------------------------------------
def upload(a: np.ndarray, dev):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


def setup(name: str, dev, n_tokens: int = 1, replicas: int = 1, lm=None, packed=False):
    """Inputs resident on the device. packed: the routed experts repacked once
    by lmoe_pack_weights (as at model load; not part of any timed step)."""
    import torch
    from workloads import get_workload, gen_x, gen_router, gen_experts, gen_shared, gen_logits
    w = get_workload(name)
    t0 = time.time()
    ex = gen_experts(w)
    weights = {k: upload(v, dev) for k, v in ex.items()}
    del ex
    if packed:
        pk = {k: torch.empty(n, dtype=torch.uint8, device=dev)
              for k, n in lm.packed_sizes(w.dims).items()}
        lm.pack_weights(w.dims, weights, pk)
        torch.cuda.synchronize()
        weights = pk
    dense = []
    rw = upload(gen_router(w), dev)
    sh = {k: upload(v, dev) for k, v in gen_shared(w).items()}
    for r in range(replicas):
        dense.append({"router_w": rw if r == 0 else rw.clone(),
                      **{k: (v if r == 0 else v.clone()) for k, v in sh.items()}})
    xs = gen_x(w.with_T(max(w.dims.T, n_tokens)))
    x = upload(xs, dev)
    logits = upload(gen_logits(w), dev) if w.logits_given else None
    log(f"{name}: inputs generated and resident in {time.time() - t0:.1f}s")
    return w, weights, dense, x, logits


def hold_cycles(hip, stream, ms_target: float) -> int:
    """Argument of torch.cuda._sleep that spins the GPU for about ms_target."""
    import torch
    e0, e1 = hip.event(), hip.event()
    n = 1 << 20
    hip.record(e0, stream)
    torch.cuda._sleep(n)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    per = max(hip.elapsed_ms(e0, e1), 1e-3) / n
    return int(ms_target / per)


def routing_buffers(d, dev):
    import torch
    return {
        "topk_idx": torch.empty((d.T, d.k), dtype=torch.int32, device=dev),
        "counts": torch.empty((d.E,), dtype=torch.int32, device=dev),
    }


def run_case(lm, hip, name, dev, steps, warmup, rotate: bool, traced_steps: int,
             packed: bool = False, path=None, act: str = "bf16"):
    """Time `steps` layer calls; returns a dict of measurements. packed: the
    tile-packed routed experts and lmoe_forward_packed (shared experts on a
    second stream of the bench's own). path: lmoe_forward_ex with that path
    choice (PATH_GROUPED or PATH_FUSED), likewise with the bench's stream."""
    import torch
    n_tok = N_TOKENS if rotate else 1
    reps = N_REPLICAS if rotate else 1
    w = __import__("workloads").get_workload(name)
    T = w.dims.T
    # rotating calls take T rows at a time from a pool of n_tok * T rows
    w, experts, dense, x_pool, logits = setup(name, dev, n_tok * T, reps, lm, packed)
    own = packed or path is not None
    side = torch.cuda.Stream() if own else None
    fork, join = (hip.event(), hip.event()) if own else (None, None)

    act_code = {"bf16": lm.ACT_BF16, "e4m3": lm.ACT_E4M3, "e2m1": lm.ACT_E2M1}[act]

    def fwd(d, xi, wi, lg, r, out, ws, events=None):
        if packed and events is not None:
            lm.forward_packed(d, xi, wi, lg, r, out, ws, stage_events=events, act=act_code)
        elif packed:
            lm.forward_packed(d, xi, wi, lg, r, out, ws, side.cuda_stream, fork, join,
                              act=act_code)
        elif path is not None and events is not None:
            lm.forward_ex(d, xi, wi, lg, r, out, ws, stage_events=events, path=path)
        elif path is not None:
            lm.forward_ex(d, xi, wi, lg, r, out, ws, side.cuda_stream, fork, join, path=path)
        elif events is not None:
            lm.forward_traced(d, xi, wi, lg, r, out, ws, events)
        else:
            lm.forward(d, xi, wi, lg, r, out, ws)
    d = w.dims
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    out = torch.empty((T, d.L), dtype=torch.int16, device=dev)
    rbuf = routing_buffers(d, dev)
    stream = torch.cuda.current_stream().cuda_stream

    def args(i):
        if rotate:
            xi = x_pool[(i % n_tok) * T: (i % n_tok + 1) * T]
            wi = {**experts, **dense[i % reps]}
        else:
            xi = x_pool[:T]
            wi = {**experts, **dense[0]}
        r = {"logits": logits} if w.logits_given else None
        return xi, wi, r

    # distinct experts per step (untimed)
    D = []
    for i in range(n_tok):
        xi, wi, r = args(i)
        rr = dict(rbuf)
        if r:
            rr.update(r)
        fwd(d, xi, wi, w.logits_given, rr, out, ws)
        D.append(int((rbuf["counts"] > 0).sum().item()))
    D_mean = float(np.mean(D))

    pre = [args(i) for i in range(max(steps, warmup, traced_steps, 1))]
    for i in range(warmup):
        xi, wi, r = pre[i % len(pre)]
        fwd(d, xi, wi, w.logits_given, r, out, ws)
    torch.cuda.synchronize()

    # The GPU is held in a spin kernel while the host enqueues, so the timed
    # region measures back-to-back execution, not the host's launch rate.
    sleep_cycles = hold_cycles(hip, stream, HOLD_MS)
    e0, e1 = hip.event(), hip.event()

    def timed(calls):
        torch.cuda._sleep(sleep_cycles)
        hip.record(e0, stream)
        t = time.perf_counter()
        for c in calls:
            c()
        enq = time.perf_counter() - t
        hip.record(e1, stream)
        torch.cuda.synchronize()
        return hip.elapsed_ms(e0, e1), enq * 1e3

    def call(i):
        xi, wi, r = pre[i]
        return lambda: fwd(d, xi, wi, w.logits_given, r, out, ws)

    tot_ms, enq_ms = timed([call(i) for i in range(steps)])
    ms = tot_ms / steps
    if enq_ms > HOLD_MS + tot_ms:
        log(f"{name}: host enqueue ({enq_ms:.1f} ms) outran the hold; GPU time may include gaps")

    warm_ms = None
    if rotate:  # the same token and weights every step
        warm_ms = timed([call(0) for _ in range(steps)])[0] / steps

    # per-stage times from events the library records at stage boundaries
    evs = [[hip.event() for _ in range(lm.NUM_STAGE_EVENTS)] for _ in range(traced_steps)]

    def traced(i):
        xi, wi, r = pre[i]
        return lambda: fwd(d, xi, wi, w.logits_given, r, out, ws, evs[i])

    timed([traced(i) for i in range(traced_steps)])
    stage_ms = {s: 0.0 for s in lm.STAGES[1:]}
    for i in range(traced_steps):
        for j in range(1, lm.NUM_STAGE_EVENTS):
            stage_ms[lm.STAGES[j]] += hip.elapsed_ms(evs[i][j - 1], evs[i][j]) / traced_steps
    traced_total = sum(stage_ms.values())

    del experts, dense, x_pool, ws, out
    torch.cuda.empty_cache()
    return {"w": w, "D": D_mean, "ms": ms, "enqueue_ms": enq_ms / steps, "warm_ms": warm_ms,
            "stage_ms": stage_ms, "traced_ms": traced_total, "packed": packed, "path": path,
            "act": act}


# The single-token path is one kernel; the library records every stage event
# right after it, so its whole time lands on the first stage. So is the path
# of 2..16 tokens.
FUSED_KERNEL = "decode_kernel"
FUSED_KERNELS = {"fused_decode": FUSED_KERNEL, "fused_multi": "decode_multi_kernel"}


def taken_path(res, lm) -> str:
    """The implementation a measured call took."""
    w = res["w"]
    d = w.dims
    if res.get("packed") or res.get("path") == lm.PATH_GROUPED:
        return "grouped"
    if res.get("path") == lm.PATH_FUSED and not w.logits_given:
        if d.T == 1:
            return lm.path_name(d, False)
        if 2 <= d.T <= 16 and d.T * d.k <= 256 and max(d.L, d.I, d.Is) <= 4096:
            return "fused_multi"
    return lm.path_name(d, w.logits_given)


def kernel_units(res, lm):
    """(kernel, algorithmic bytes, flops, seconds) per launched kernel."""
    d = res["w"].dims
    logits_given = res["w"].logits_given
    tb, tf, sb, sf = algorithmic(d, res["D"], logits_given)
    path = taken_path(res, lm)
    if path in FUSED_KERNELS:
        # one kernel does the whole layer: the layer's bytes (the tokens are
        # read once, though three stages count them). Every timed step is one
        # launch of it, back to back, so the events around the timed region
        # give its average launch; the events a traced call records around
        # the kernel add 2-5 us of their own.
        return [(FUSED_KERNELS[path], tb, tf, res["ms"] * 1e-3)]
    large = True  # routed groups of every size take the large kernel
    sh_large = d.T > 64
    act = res.get("act", "bf16")
    if act == "bf16":
        # second template argument: K a multiple of the 128-value chunk
        ka = lambda K: "true" if K % 128 == 0 else "false"
        packed_kernel = {"gate_up": f"gemm_packed_kernel<true, {ka(d.L)}>",
                         "down": f"gemm_packed_kernel<false, {ka(d.I)}>"}
    else:
        f8 = "true" if act == "e4m3" else "false"
        # MXFP4 activations with K a multiple of 256 up to 4096: the
        # pair-copy kernel
        a4 = lambda K: act == "e2m1" and K % 256 == 0 and K <= 4096
        packed_kernel = {
            "gate_up": ("gemm_packed_a4_kernel<true>" if a4(d.L)
                        else f"gemm_packed_q_kernel<true, {f8}>"),
            "down": ("gemm_packed_a4_kernel<false>" if a4(d.I)
                     else f"gemm_packed_q_kernel<false, {f8}>")}
    return [((packed_kernel.get(s) if res.get("packed") else None)
             or stage_kernel(s, large, sh_large, d, logits_given), sb[s], sf[s],
             res["stage_ms"][s] * 1e-3)
            for s in sb if res["stage_ms"][s] > 0]


def read_ceiling(lm, hip, dev, gib: int = 4, reps: int = 10):
    """The plain HBM read rate of this GPU: lmoe_debug_read_stream over a
    `gib` GiB buffer (every byte read once with 16-byte loads), best over a
    few grid sizes, median of `reps` timed reads each."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    buf = torch.zeros(gib << 30, dtype=torch.uint8, device=dev)
    best, by_grid = None, {}
    for blocks in (256, 512, 1024, 2048, 4096, 8192):
        sink = torch.empty(blocks, dtype=torch.int32, device=dev)
        lm.debug_read_stream(buf, sink, blocks)
        times = []
        for _ in range(reps):
            e0, e1 = hip.event(), hip.event()
            hip.record(e0, stream)
            lm.debug_read_stream(buf, sink, blocks)
            hip.record(e1, stream)
            times.append(hip.elapsed_ms(e0, e1))
        ms = float(np.median(times))
        gbs = buf.numel() / (ms * 1e-3) / 1e9
        by_grid[str(blocks)] = round(gbs, 1)
        if best is None or gbs > best["gb_s"]:
            best = {"gb_s": round(gbs, 1), "workgroups": blocks, "bytes": buf.numel(),
                    "kernel": "read_stream_kernel"}
    best["gb_s_by_workgroups"] = by_grid
    del buf
    torch.cuda.empty_cache()
    return best


def mfma_ceiling(lm, hip, dev, reps: int = 5):
    """The bf16 MFMA rate this GPU sustains under full load:
    lmoe_debug_mfma_rate (every wave issuing independent 32x32x16 bf16 MFMAs
    on random register operands), median of `reps` timed launches at each of
    a few grid sizes; the best is the ceiling."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    iters = 4096
    best, by_grid = None, {}
    for blocks in (512, 1024, 2048):
        sink = torch.empty(blocks, dtype=torch.int32, device=dev)
        lm.debug_mfma_rate(iters, sink, blocks)
        times = []
        for _ in range(reps):
            e0, e1 = hip.event(), hip.event()
            hip.record(e0, stream)
            lm.debug_mfma_rate(iters, sink, blocks)
            hip.record(e1, stream)
            times.append(hip.elapsed_ms(e0, e1))
        ms = float(np.median(times))
        flops = blocks * 4 * iters * 8 * 32768
        tfl = flops / (ms * 1e-3) / 1e12
        by_grid[str(blocks)] = round(tfl, 1)
        if best is None or tfl > best["tflop_s"]:
            best = {"tflop_s": round(tfl, 1), "workgroups": blocks, "flops": flops,
                    "frac_of_peak": round(tfl / BF16_PEAK_TFLOPS, 4),
                    "kernel": "mfma_rate_kernel"}
    best["tflop_s_by_workgroups"] = by_grid
    return best


def stage_us(res, lm):
    """Per-stage times in us from the traced calls; on the single-token path
    one kernel runs every stage, so only that kernel's average launch (the
    untraced timed region) is reported."""
    path = taken_path(res, lm)
    if path in FUSED_KERNELS:
        return {FUSED_KERNELS[path]: round(res["ms"] * 1e3, 2)}
    return {k: round(v * 1e3, 1) for k, v in res["stage_ms"].items()}


def traffic_workload(res) -> str:
    """The workload name the PMC summary files a run under: the workload,
    plus _a8 / _a4 for quantised activations (as `--extra` names them)."""
    suffix = {a: suf for suf, (a, _) in ACT_SUFFIX.items()}.get(res.get("act", "bf16"), "")
    return res["w"].name + suffix


def roofline_for(res, bound: str, lm):
    """Roofline of the kernel with the longest average launch."""
    units = [u for u in kernel_units(res, lm) if (u[1] if bound == "hbm" else u[2]) > 0]
    kernel, nbytes, flops, sec = max(units, key=lambda u: u[3])
    if bound == "hbm":
        achieved, peak, unit = nbytes / sec / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        mfma_peak = {"bf16": BF16_PEAK_TFLOPS, "e4m3": FP8_PEAK_TFLOPS,
                     "e2m1": FP4_PEAK_TFLOPS}[res.get("act", "bf16")]
        if not kernel.startswith("gemm_packed"):   # the bf16 kernels of the same layer
            mfma_peak = BF16_PEAK_TFLOPS
        achieved, peak, unit = flops / sec / 1e12, mfma_peak, "TFLOP/s"
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(kernel, traffic_workload(res)),
            "kernel": kernel, "kernel_us": round(sec * 1e6, 2),
            "algorithmic_bytes": round(nbytes), "algorithmic_flops": round(flops)}


def host_cpu():
    """(usable cores, CPU model) of this host."""
    try:
        cores = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return cores, model


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(max_tokens: int, budget_s: float):
    """The oracle as it stands, on decode tokens of the same layer, host cores:
    tokens are run one at a time until `budget_s` seconds of work or
    `max_tokens` tokens."""
    import oracle as O
    from workloads import get_workload, gen_x, gen_router, gen_expert, gen_shared
    w = get_workload("decode")
    d = w.dims
    xs = gen_x(w.with_T(max_tokens))
    rw = gen_router(w)
    sh = gen_shared(w)
    cache = {}

    def expert(e):  # generated outside the timed work
        return cache[e]

    sec, n = 0.0, 0
    while n < max_tokens and sec < budget_s:
        x = xs[n:n + 1]
        for e in O.topk_select(O.router_logits(x, rw), d.k).ravel().tolist():
            if e not in cache:
                cache[e] = gen_expert(w, e)
        t0 = time.perf_counter()
        lgt = O.router_logits(x, rw)
        it = O.topk_select(lgt, d.k)
        wt = O.softmax_selected(lgt, it)
        O.forward_tokens(x, it, wt, expert, sh, d.L, d.I)
        sec += time.perf_counter() - t0
        n += 1
    tb, _, _, _ = algorithmic(d, d.k, False)
    cores, model = host_cpu()
    return {"value": round(tb * n / sec / 1e9, 4), "unit": "GB/s", "cores": blas_threads(),
            "host_cores": cores, "cpu_model": model, "kind": "oracle",
            "sample": f"{n} decode tokens (T=1 each: router, top-16 of 896, 16 MXFP4 experts "
                      f"+ 2 bf16 shared, float64 numpy oracle), {sec:.1f} s of oracle work"}


def cpu_baseline_prefill(n_experts: int, n_tokens: int):
    """The oracle on the prefill chunk (T=4096), from a sample scaled linearly:
    routing (router logits, top-k, softmax, grouping) timed on every token;
    the routed experts timed on n_experts seeded experts with all of their
    routes (dequantisation plus the GLU over those rows, the oracle's
    per-expert work) and scaled by E / n_experts; the shared experts and the
    combine timed on n_tokens tokens and scaled by T / n_tokens."""
    import oracle as O
    from workloads import get_workload, gen_x, gen_router, gen_expert, gen_shared
    w = get_workload("prefill")
    d = w.dims
    x = gen_x(w)
    rw = gen_router(w)
    sh = gen_shared(w)
    t0 = time.perf_counter()
    lg = O.router_logits(x, rw)
    idx = O.topk_select(lg, d.k)
    wt = O.softmax_selected(lg, idx)
    O.permute_routes(idx, d.E)
    t_route = time.perf_counter() - t0
    rng = np.random.default_rng(7)
    experts = sorted(int(e) for e in rng.choice(d.E, size=n_experts, replace=False))
    x64 = O.f64_from_bf16(x)
    t_exp = 0.0
    for e in experts:
        ex = gen_expert(w, e)                         # generation is not timed
        rows, _ = np.nonzero(idx == e)
        t0 = time.perf_counter()
        gate = O.dequant_mxfp4(ex["gate_q"], ex["gate_s"], d.I, d.L)
        up = O.dequant_mxfp4(ex["up_q"], ex["up_s"], d.I, d.L)
        down = O.dequant_mxfp4(ex["down_q"], ex["down_s"], d.L, d.I)
        O.glu_ffn(x64[rows], gate, up, down)
        t_exp += time.perf_counter() - t0
    toks = np.arange(n_tokens)
    t0 = time.perf_counter()
    ysh = np.stack([O.glu_ffn(x64[toks], O.f64_from_bf16(sh["sh_gate"][s]),
                              O.f64_from_bf16(sh["sh_up"][s]),
                              O.f64_from_bf16(sh["sh_down"][s]))[1] for s in range(d.S)])
    O.combine(np.zeros((n_tokens, d.k, d.L)), wt[toks], ysh)
    t_tok = time.perf_counter() - t0
    est = t_route + t_exp * d.E / n_experts + t_tok * d.T / n_tokens
    _, tf, _, _ = algorithmic(d, d.E, False)
    cores, model = host_cpu()
    return {"value": round(tf / est / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(),
            "host_cores": cores, "cpu_model": model, "kind": "oracle",
            "estimated_s": round(est, 2),
            "sample": f"prefill T=4096 float64 numpy oracle: routing timed on all 4096 tokens "
                      f"({t_route:.1f} s); routed experts timed on {n_experts} seeded experts "
                      f"with all their routes ({t_exp:.1f} s), scaled by {d.E}/{n_experts}; "
                      f"shared experts and combine timed on {n_tokens} tokens ({t_tok:.1f} s), "
                      f"scaled by {d.T}/{n_tokens}"}


# Further workloads reported on request (--extra): the other configurations of
# the layer, the expert width the pages' per-expert size implies, and one
# GPU's share of the layer split eight ways. Decode-sized ones are HBM-bound
# and rotate tokens like the headline case; the rest are rated against MFMA.
EXTRA = ("batched_decode", "skewed", "decode_i3072", "prefill_i3072", "decode_tp8",
         "prefill_a4", "batched_decode_a8", "skewed_a4")
# reported by default: the other graded configurations, the page-implied
# expert width at decode, and the pages' quantised-activation precisions
# (MXFP4 activations at prefill, FP8 at batched decode)
DEFAULT_EXTRA = "batched_decode,skewed,decode_i3072,prefill_a4,batched_decode_a8"


def extra_case(lm, hip, name, dev, steps, packed: bool, path=None):
    from workloads import get_workload
    act, mfma_peak = "bf16", BF16_PEAK_TFLOPS
    for suf, (a, pk) in ACT_SUFFIX.items():
        if name.endswith(suf):   # quantised activations: packed experts only
            name, act, mfma_peak, packed = name[: -len(suf)], a, pk, True
    d = get_workload(name).dims
    hbm = d.T <= 64
    # single tokens take the one-kernel path on row-major experts
    packed = packed and d.T > 1 and path is None
    res = run_case(lm, hip, name, dev, steps if hbm else max(3, steps // 20), 3, rotate=hbm,
                   traced_steps=5, packed=packed, path=path, act=act)
    tb, tf, _, _ = algorithmic(d, res["D"], res["w"].logits_given)
    sec = res["ms"] * 1e-3
    # with quantised activations the routed GEMMs' MFMA ridge (fp8 625, fp4
    # 1262 flop/byte at 8 TB/s) is far above the layer's intensity even at
    # prefill: their roofline is HBM's
    bound = "hbm" if hbm or (act != "bf16" and
                             tf / tb < mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)) else "mfma"
    out = {"T": d.T, "L": d.L, "E": d.E, "k": d.k, "I": d.I, "S": d.S, "Is": d.Is,
           "distinct_experts": round(res["D"], 1), "ms_per_step": round(res["ms"], 5),
           "gb_s": round(tb / sec / 1e9, 1), "tflop_s": round(tf / sec / 1e12, 2),
           "algorithmic_bytes": round(tb), "algorithmic_flops": round(tf),
           "layout": "packed" if packed else "row-major",
           "path": taken_path(res, lm),
           "act_format": act,
           "roofline": roofline_for(res, bound, lm),
           "stage_us": stage_us(res, lm)}
    out["frac_of_peak"] = round(out["gb_s"] / HBM_PEAK_GBS if bound == "hbm"
                                else out["tflop_s"] / mfma_peak, 4)
    log(f"{name}: {res['ms']:.4f} ms/step, {out['gb_s']} GB/s, {out['tflop_s']} TFLOP/s")
    return out


# Decode of a few tokens per call: the fused multi-token kernel against the
# grouped kernels on the same row-major experts (lmoe_forward_ex with each
# path choice) and on tile-packed experts (lmoe_forward_packed), at each T;
# all stream the D distinct experts' weights. `auto` is what lmoe_forward
# takes for that shape.
BLOCKS = ("block_decode", "block_batched", "block_prefill")
DEFAULT_BLOCKS = "block_decode,block_prefill"


def block_algorithmic(d, D: int):
    """Algorithmic bytes and flops of the MoE block's input step, tail and
    the whole block (input step + the layer without shared experts + tail):
    every weight read once, the activations in and out once."""
    T, H, L, E, SI = d.T, d.H, d.L, d.E, d.S * d.Is
    n_in = E + L + 2 * SI
    inp_b = 2 * H * n_in + 2 * T * H + 4 * T * E + 2 * T * L + 2 * T * SI
    inp_f = 2 * T * H * n_in
    tail_b = 2 * H * (L + SI) + 2 * T * (L + SI) + 2 * L + 4 * T * H
    tail_f = 2 * T * H * (L + SI)
    lay = type(d)(T=T, L=L, E=E, k=d.k, I=d.I, S=0, Is=0)
    lb, lf, _, _ = algorithmic(lay, D, True)
    return {"input": (inp_b, inp_f), "tail": (tail_b, tail_f),
            "block": (inp_b + lb + tail_b, inp_f + lf + tail_f)}


def block_case(lm, hip, name, dev, steps):
    """The MoE block around the layer (lmoe_moe_input, lmoe_moe_tail,
    lmoe_block_forward), timed with HIP events on the launch stream. Up to 64
    tokens the calls rotate over 2 copies of the block's dense weights and 64
    tokens' inputs, so weights are read from HBM each step, as in serving."""
    import torch
    from workloads import get_workload, gen_block, gen_experts
    w = get_workload(name)
    d = w.dims
    T, SI = d.T, d.S * d.Is
    rotate = T <= 64
    n_tok = N_TOKENS if rotate else 1
    reps = 2 if rotate else 1
    t0 = time.time()
    ex = gen_experts(w)
    experts = {k: upload(v, dev) for k, v in ex.items()}
    del ex
    b = gen_block(w.with_T(T * n_tok))
    dense = [{k: upload(b[k], dev) for k in ("w_in", "norm_w", "w_up", "w_sd")}]
    for _ in range(reps - 1):
        dense.append({k: v.clone() for k, v in dense[0].items()})
    u_pool, res_pool = upload(b["u"], dev), upload(b["residual"], dev)
    del b
    log(f"{name}: inputs generated and resident in {time.time() - t0:.1f}s")
    ws = torch.zeros(lm.block_workspace_bytes(d), dtype=torch.uint8, device=dev)
    logits = torch.empty((T, d.E), dtype=torch.float32, device=dev)
    x = torch.empty((T, d.L), dtype=torch.int16, device=dev)
    h = torch.empty((T, max(SI, 1)), dtype=torch.int16, device=dev)
    routed = torch.empty((T, d.L), dtype=torch.int16, device=dev)
    out = torch.empty((T, d.H), dtype=torch.int16, device=dev)
    r = {"logits": logits, "counts": torch.empty((d.E,), dtype=torch.int32, device=dev)}
    stream = torch.cuda.current_stream().cuda_stream

    def rows(i, pool):
        j = i % n_tok
        return pool[j * T:(j + 1) * T]

    def f_input(i):
        dw = dense[i % reps]
        return lambda: lm.moe_input(d, rows(i, u_pool), dw["w_in"], logits, x, h, ws)

    def f_tail(i):
        dw = dense[i % reps]
        return lambda: lm.moe_tail(d, routed, h, dw["norm_w"], dw["w_up"], dw["w_sd"],
                                   rows(i, res_pool), out, ws)

    def f_block(i):
        dw = dense[i % reps]
        return lambda: lm.block_forward(d, rows(i, u_pool), rows(i, res_pool), dw, experts, r,
                                        out, ws)

    # distinct experts per step (untimed), and a routed result for the tail
    D = []
    for i in range(n_tok):
        f_block(i)()
        D.append(int((r["counts"] > 0).sum().item()))
    routed.copy_(x)
    sleep_cycles = hold_cycles(hip, stream, HOLD_MS)
    e0, e1 = hip.event(), hip.event()
    n = steps if rotate else max(3, steps // 20)

    def timed(make):
        for i in range(2):
            make(i)()
        calls = [make(i) for i in range(n)]
        torch.cuda.synchronize()
        torch.cuda._sleep(sleep_cycles)
        hip.record(e0, stream)
        for c in calls:
            c()
        hip.record(e1, stream)
        torch.cuda.synchronize()
        return hip.elapsed_ms(e0, e1) / n

    alg = block_algorithmic(d, float(np.mean(D)))
    out_d = {"T": T, "H": d.H, "L": d.L, "E": d.E, "k": d.k, "I": d.I, "S": d.S, "Is": d.Is,
             "distinct_experts": round(float(np.mean(D)), 1), "steps": n}
    for leg, make, kernel in (("input", f_input, "dense_gemm_kernel"),
                              ("tail", f_tail, "dense_gemm_kernel"),
                              ("block", f_block, None)):
        ms = timed(make)
        nb, nf = alg[leg]
        sec = ms * 1e-3
        hbm = nf / nb < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        e = {"us": round(ms * 1e3, 2), "gb_s": round(nb / sec / 1e9, 1),
             "tflop_s": round(nf / sec / 1e12, 2), "algorithmic_bytes": round(nb),
             "algorithmic_flops": round(nf)}
        if kernel:   # the leg's GEMMs (and their K-split finish) as one unit
            ach = nb / sec / 1e9 if hbm else nf / sec / 1e12
            peak = HBM_PEAK_GBS if hbm else BF16_PEAK_TFLOPS
            e["roofline"] = {"bound": "hbm" if hbm else "mfma", "achieved": round(ach, 2),
                             "peak": peak, "unit": "GB/s" if hbm else "TFLOP/s",
                             "frac": round(ach / peak, 4), "kernel": kernel,
                             "traffic": measured_traffic(kernel, name)}
        out_d[leg] = e
        log(f"{name} {leg}: {ms * 1e3:.1f} us, {e['gb_s']} GB/s, {e['tflop_s']} TFLOP/s")
    del experts, dense, u_pool, res_pool, ws
    torch.cuda.empty_cache()
    return out_d


SMALL_T = (2, 4, 8, 16)


def small_t_sweep(lm, hip, dev, steps):
    from workloads import get_workload
    out = {}
    cross = None
    for T in SMALL_T:
        name = f"decode_t{T}"
        legs = {"fused": extra_case(lm, hip, name, dev, steps, False, lm.PATH_FUSED),
                "grouped": extra_case(lm, hip, name, dev, steps, False, lm.PATH_GROUPED),
                "grouped_packed": extra_case(lm, hip, name, dev, steps, True)}
        faster = min(legs, key=lambda k: legs[k]["ms_per_step"])
        out[name] = {**legs, "faster": faster,
                     "auto": lm.path_name(get_workload(name).dims, False)}
        if cross is None and legs["grouped"]["ms_per_step"] < legs["fused"]["ms_per_step"]:
            cross = T
    out["first_T_grouped_faster"] = cross
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-experts", type=int, default=40,
                    help="experts the prefill oracle sample times")
    ap.add_argument("--extra", default=DEFAULT_EXTRA,
                    help="comma-separated further workloads to report, 'all', or 'none': "
                         + ", ".join(EXTRA))
    ap.add_argument("--block", default=DEFAULT_BLOCKS,
                    help="MoE-block workloads to report (input step, tail, whole block): "
                         + ", ".join(BLOCKS) + ", or 'none'")
    ap.add_argument("--no-small-t", action="store_true",
                    help="skip the 2..16-token decode sweep (fused kernel against the "
                         "grouped path)")
    ap.add_argument("--layout", default="packed", choices=("packed", "row-major"),
                    help="routed-expert layout of the multi-token cases (single tokens run "
                         "the one-kernel path on row-major experts)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the plain HBM read and sustained MFMA ceiling measurements")
    ap.add_argument("--traffic-from", default="",
                    help="merge into profiles/pmc_traffic.json the FETCH_SIZE / WRITE_SIZE "
                         "counter runs in this directory (subfolders fetch/ and write/) and exit")
    ap.add_argument("--traffic-workload", default="prefill",
                    help="workload the --traffic-from runs measured (the single-token "
                         "kernel is always filed under decode)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this size (PMC calibration)")
    args = ap.parse_args()
    if args.traffic_from:
        out = traffic_from(args.traffic_from, args.traffic_workload)
        for k, v in out["kernels"].items():
            for wl, e in v.items():
                print(f"{k} [{wl}]: {e['traffic_bytes']} bytes per dispatch")
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this layer is measured on a single MI355X "
              f"(asked for --gpus {args.gpus}); multi-GPU sharding is not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mxfp4_latent_mixture_amd as lm
    dev = torch.device("cuda:0")
    hip = Hip()

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"calibration copy of {n} bytes done")
        del a, b

    ceiling = mceil = None
    if not args.no_ceiling:
        ceiling = read_ceiling(lm, hip, dev)
        log(f"plain HBM read ceiling: {ceiling['gb_s']} GB/s ({ceiling['workgroups']} workgroups)")
        mceil = mfma_ceiling(lm, hip, dev)
        log(f"sustained bf16 MFMA rate: {mceil['tflop_s']} TFLOP/s "
            f"({mceil['workgroups']} workgroups)")
    dec = run_case(lm, hip, "decode", dev, args.steps, args.warmup, rotate=True,
                   traced_steps=min(args.steps, 50))
    d = dec["w"].dims
    tb, tf, _, _ = algorithmic(d, dec["D"], False)
    value = tb / (dec["ms"] * 1e-3) / 1e9
    log(f"decode: {dec['ms'] * 1e3:.1f} us/step, {value:.0f} GB/s; warm "
        f"{dec['warm_ms'] * 1e3:.1f} us; stages {stage_us(dec, lm)}")
    result = {
        "metric": "MoE-layer HBM GB/s at T=1 (K3 LatentMoE decode, MXFP4 w4a16)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "K3 LatentMoE decode: T=1, L=3584, E=896 resident MXFP4 experts, "
                               "k=16, I=2048, 2 bf16 shared experts (Is=2048), seed 1; "
                               "64 rotating tokens, 4 rotating copies of router+shared weights",
                   "tokens": d.T, "latent": d.L, "experts": d.E, "top_k": d.k,
                   "intermediate": d.I, "shared": d.S},
        "roofline": {**roofline_for(dec, "hbm", lm),
                     **({"read_ceiling_gb_s": ceiling["gb_s"],
                         "frac_of_read_ceiling": round(value / ceiling["gb_s"], 4)}
                        if ceiling else {})},
        "hbm_read_ceiling": ceiling,
        "mfma_ceiling": mceil,
        "algorithmic_bytes_per_step": round(tb),
        "warm_gb_s": round(tb / (dec["warm_ms"] * 1e-3) / 1e9, 2),
        "stage_us": stage_us(dec, lm),
    }
    if not args.no_prefill:
        pf = run_case(lm, hip, "prefill", dev, args.prefill_steps, 2, rotate=False,
                      traced_steps=min(args.prefill_steps, 5), packed=args.layout == "packed")
        pd = pf["w"].dims
        ptb, ptf, _, _ = algorithmic(pd, pf["D"], False)
        tfl = ptf / (pf["ms"] * 1e-3) / 1e12
        log(f"prefill: {pf['ms']:.3f} ms/step, {tfl:.1f} TFLOP/s; stages {stage_us(pf, lm)}")
        result["prefill"] = {
            "metric": "MoE-layer bf16 MFMA TFLOP/s at T=4096",
            "value": round(tfl, 2), "unit": "TFLOP/s", "ms_per_step": round(pf["ms"], 4),
            "steps": args.prefill_steps, "frac_of_peak": round(tfl / BF16_PEAK_TFLOPS, 4),
            "gb_s": round(ptb / (pf["ms"] * 1e-3) / 1e9, 1),
            "workload": "K3 LatentMoE prefill chunk: T=4096, same layer, seed 3",
            "layout": args.layout,
            "roofline": roofline_for(pf, "mfma", lm),
            "stage_us": stage_us(pf, lm),
        }
        if mceil:
            rf = result["prefill"]["roofline"]
            rf["mfma_ceiling_tflop_s"] = mceil["tflop_s"]
            rf["frac_of_mfma_ceiling"] = round(rf["achieved"] / mceil["tflop_s"], 4)
            result["prefill"]["frac_of_mfma_ceiling"] = round(tfl / mceil["tflop_s"], 4)
    if args.extra and args.extra != "none":
        names = EXTRA if args.extra == "all" else tuple(args.extra.split(","))
        result["extra"] = {}
        for n in names:
            packed = args.layout == "packed"
            if n.endswith("_rowmajor"):
                n, packed = n[: -len("_rowmajor")], False
                result["extra"][n + "_rowmajor"] = extra_case(lm, hip, n, dev, args.steps, False)
            else:
                result["extra"][n] = extra_case(lm, hip, n, dev, args.steps, packed)
    if args.block and args.block != "none":
        result["block"] = {n: block_case(lm, hip, n, dev, args.steps)
                           for n in args.block.split(",")}
    if not args.no_small_t:
        result["decode_small_t"] = small_t_sweep(lm, hip, dev, max(20, args.steps // 2))
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args.cpu_tokens, args.cpu_seconds)
        if "prefill" in result:
            result["prefill"]["cpu_baseline"] = cpu_baseline_prefill(args.cpu_experts, 512)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

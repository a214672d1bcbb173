"""Helpers shared by the GPU tests: moving seeded inputs to the device, running
the HIP path through the binding, and the parity bounds."""
from __future__ import annotations

import sys
import time
from typing import Dict, Optional

import numpy as np

import oracle as O
from workloads import Workload

WEIGHT_KEYS = ("router_w", "gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s",
               "sh_gate", "sh_up", "sh_down")


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dev):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


def upload(inp: Dict[str, np.ndarray], dev) -> Dict[str, object]:
    out = {}
    for k in WEIGHT_KEYS + ("x", "logits"):
        if k in inp:
            out[k] = to_dev(inp[k], dev)
    return out


def alloc_routing(d, dev) -> Dict[str, object]:
    import torch
    R = d.T * d.k
    return {
        "logits": torch.empty((d.T, d.E), dtype=torch.float32, device=dev),
        "topk_idx": torch.empty((d.T, d.k), dtype=torch.int32, device=dev),
        "topk_w": torch.empty((d.T, d.k), dtype=torch.float32, device=dev),
        "counts": torch.empty((d.E,), dtype=torch.int32, device=dev),
        "offsets": torch.empty((d.E + 1,), dtype=torch.int32, device=dev),
        "perm": torch.empty((R,), dtype=torch.int32, device=dev),
        "inv_perm": torch.empty((R,), dtype=torch.int32, device=dev),
    }


def run_forward(lm, w: Workload, dev_inp: Dict[str, object], routing: Optional[dict] = None):
    """Run lmoe_forward; returns (out bf16 bits numpy, routing dict of numpy)."""
    import torch
    d = w.dims
    dev = dev_inp["x"].device
    if routing is None:
        routing = alloc_routing(d, dev)
    if w.logits_given:
        routing["logits"] = dev_inp["logits"]
    out = torch.empty((d.T, d.L), dtype=torch.int16, device=dev)
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    lm.forward(d, dev_inp["x"], dev_inp, w.logits_given, routing, out, ws)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in routing.items()}
    return out.cpu().numpy().view(np.uint16), res


def out_bound(ref64: np.ndarray, rms: Optional[float] = None) -> np.ndarray:
    """Element-wise bound for a bf16 output against the float64 reference:
    1e-2 * rms(ref) for the arithmetic, plus half a bf16 ulp for the final
    rounding to bf16 that the output format itself imposes."""
    if rms is None:
        rms = float(np.sqrt(np.mean(ref64 ** 2)))
    tol = 1e-2 * rms
    mag = np.maximum(np.abs(ref64) + tol, np.finfo(np.float64).tiny)
    e = np.floor(np.log2(mag)).astype(np.int64)
    return tol + np.ldexp(1.0, e - 8)


def check_out(got_bits: np.ndarray, ref64: np.ndarray, what: str, rms: Optional[float] = None):
    got = O.f64_from_bf16(got_bits)
    if rms is None:
        rms = float(np.sqrt(np.mean(ref64 ** 2)))
    bound = out_bound(ref64, rms)
    err = np.abs(got - ref64)
    bad = np.nonzero(~(err <= bound))
    rel_rms = float(np.sqrt(np.mean((got - ref64) ** 2)) / rms)
    log(f"{what}: max|err|/rms={err.max() / rms:.3e} rms(err)/rms={rel_rms:.3e}")
    assert bad[0].size == 0, (
        f"{what}: {bad[0].size} outputs out of bound; first at {tuple(b[0] for b in bad)}: "
        f"got {got[bad][0]!r} ref {ref64[bad][0]!r} bound {bound[bad][0]!r}")
    # the pages report stage RMS relative errors around 1e-3; bf16 output
    # rounding alone contributes ~1.1e-3
    assert rel_rms < 3e-3, f"{what}: rms error {rel_rms:.3e}"


def logits_bound(x_bits: np.ndarray, wr_bits: np.ndarray) -> np.ndarray:
    """Worst-case fp32 summation bound on |gpu_logit - oracle_logit| per (t, e):
    (L + 2) * 2^-24 * sum_l |x w| plus the final rounding of the oracle."""
    ax = np.abs(O.f64_from_bf16(x_bits))
    aw = np.abs(O.f64_from_bf16(wr_bits))
    L = ax.shape[1]
    s = ax @ aw.T
    return (L + 2) * 2.0 ** -24 * s + 2.0 ** -24 * s


def check_routing_against_oracle(gpu_idx: np.ndarray, gpu_logits: np.ndarray,
                                 ref_logits: np.ndarray, bound: np.ndarray, k: int, what: str):
    """GPU logits within the summation bound; the GPU's selected set equals the
    oracle's wherever the oracle's top-k boundary gap exceeds twice the bound,
    and elsewhere every GPU choice is a valid top-k choice within the bound.
    Returns the boolean mask of tokens whose sets agree."""
    g64, r64 = gpu_logits.astype(np.float64), ref_logits.astype(np.float64)
    both_nan = np.isnan(g64) & np.isnan(r64)
    d = np.where(both_nan, 0.0, np.abs(g64 - r64))
    assert np.all(d <= bound), f"{what}: logits off by {np.nanmax(d - bound):.3e} beyond bound"
    ref_idx = O.topk_select(ref_logits, k)
    same = np.array([set(a) == set(b) for a, b in zip(gpu_idx.tolist(), ref_idx.tolist())])
    lg = ref_logits.astype(np.float64)
    srt = -np.sort(-np.nan_to_num(lg, nan=-np.inf), axis=1)
    for t in np.nonzero(~same)[0]:
        tb = bound[t].max()
        gap = srt[t, k - 1] - srt[t, k] if lg.shape[1] > k else np.inf
        assert gap <= 2 * tb, f"{what}: token {t} routed differently with a clear gap {gap:.3e}"
        kth = srt[t, k - 1]
        assert np.all(lg[t, gpu_idx[t]] >= kth - 2 * tb), f"{what}: token {t} invalid choice"
    log(f"{what}: routing sets agree on {same.sum()}/{same.size} tokens")
    return same

"""Seeded generation of the layer's inputs.

Every tensor is drawn from its own numpy generator keyed by
(workload seed, tensor id, sub-index), so any slice (one expert's weights, the
activations alone) can be regenerated independently and identically by the
oracle, the GPU tests and the bench.

Byte layouts produced here (the layout the layer consumes):
  x          bf16 bits, uint16 [T][L]            N(0, x_std)
  router_w   bf16 bits, uint16 [E][L]            N(0, router_std)
  gate_q     uint8 [E][I][L/2]   E2M1 codes, element 2m in the low nibble of byte m
  gate_s     uint8 [E][I][L/32]  E8M0 exponents, one per 32 consecutive inputs
  up_q/up_s  same shapes as gate
  down_q     uint8 [E][L][I/2], down_s uint8 [E][L][I/32]
  sh_gate    bf16 bits, uint16 [S][Is][L]        N(0, shared_std)
  sh_up      same
  sh_down    bf16 bits, uint16 [S][L][Is]
  logits     float32 [T][E]  (given-logits workloads only)

MoE block workloads (dims.H > 0), all bf16 bits:
  u          uint16 [T][H]                      N(0, 1), the normalised MoE input
  residual   uint16 [T][H]                      N(0, 1)
  w_in       uint16 [E + L + 2 S Is][H]         router rows N(0, router_std),
             latent rows N(0, 1/sqrt(H)), then per shared expert its gate and
             up rows N(0, shared_std) interleaved in groups of 16 (16 gate
             rows, then the 16 up rows of the same columns)
  norm_w     uint16 [L]                         N(1, 0.1), the routed RMSNorm weight
  w_up       uint16 [H][L]                      N(0, 1/sqrt(L))
  w_sd       uint16 [H][S Is]                   N(0, shared_std), the shared
             experts' down matrices side by side along the input dimension

Codes are uniform over all 16 E2M1 values, which makes every byte uniform over
0..255. Normal samples are drawn in float64 and rounded to nearest-even bf16.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Iterable, Optional

import numpy as np

from .configs import Workload

# Tensor ids: part of each generator's key.
TID_X = 1
TID_ROUTER = 2
TID_EXPERT = 3     # gate/up/down codes and scales of one expert
TID_SH_GATE = 9
TID_SH_UP = 10
TID_SH_DOWN = 11
TID_LOGITS = 12
TID_U = 13
TID_RESIDUAL = 14
TID_W_IN = 15      # sub 0 router rows, 1 latent rows, 2 + 2 s / 3 + 2 s gate / up of expert s
TID_NORM_W = 16
TID_W_UP = 17
TID_W_SD = 18


def _rng(seed: int, tid: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tid), int(sub)]))


def _normal_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 samples -> bf16 bit patterns, round to nearest even.

    Input sampling only: samples are finite and far above the bf16 normal
    minimum (or exactly zero), so only the normal-range case is needed.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                      # v = m * 2**e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0)                  # 8 significant bits, ties to even
    r = np.ldexp(q, e - 8).astype(np.float32)   # exact: 8-bit significand
    bits = r.view(np.uint32) >> np.uint32(16)
    return bits.astype(np.uint16)


def gen_x(w: Workload) -> np.ndarray:
    d = w.dims
    v = _rng(w.seed, TID_X).normal(0.0, w.x_std, size=(d.T, d.L))
    return _normal_to_bf16_bits(v)


def gen_router(w: Workload) -> np.ndarray:
    d = w.dims
    v = _rng(w.seed, TID_ROUTER).normal(0.0, w.router_std, size=(d.E, d.L))
    return _normal_to_bf16_bits(v)


def _scales(rng: np.random.Generator, w: Workload, n: int) -> np.ndarray:
    kind = w.scales[0]
    if kind == "uniform":
        lo, hi = int(w.scales[1]), int(w.scales[2])
        return rng.integers(lo, hi + 1, size=n, dtype=np.int64).astype(np.uint8)
    if kind == "normal":
        mean, std = float(w.scales[1]), float(w.scales[2])
        v = np.rint(rng.normal(mean, std, size=n))
        return np.clip(v, 0, 254).astype(np.uint8)
    raise ValueError(f"unknown scale distribution {w.scales!r}")


def gen_expert(w: Workload, e: int) -> Dict[str, np.ndarray]:
    """Codes and scales of routed expert e (gate, up, down)."""
    d = w.dims
    L, I = d.L, d.I
    rng = _rng(w.seed, TID_EXPERT, e)
    n_gu = I * L // 2
    n_d = L * I // 2
    codes = rng.integers(0, 256, size=2 * n_gu + n_d, dtype=np.uint8)
    sc = _scales(rng, w, 2 * (I * L // 32) + L * I // 32)
    ns = I * L // 32
    return {
        "gate_q": codes[:n_gu].reshape(I, L // 2),
        "up_q": codes[n_gu:2 * n_gu].reshape(I, L // 2),
        "down_q": codes[2 * n_gu:].reshape(L, I // 2),
        "gate_s": sc[:ns].reshape(I, L // 32),
        "up_s": sc[ns:2 * ns].reshape(I, L // 32),
        "down_s": sc[2 * ns:].reshape(L, I // 32),
    }


def gen_experts(w: Workload, experts: Optional[Iterable[int]] = None,
                threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Stacked [E][...] arrays for all experts (or the listed ones, in order)."""
    d = w.dims
    ids = list(range(d.E)) if experts is None else [int(e) for e in experts]
    n = len(ids)
    L, I = d.L, d.I
    out = {
        "gate_q": np.empty((n, I, L // 2), np.uint8),
        "up_q": np.empty((n, I, L // 2), np.uint8),
        "down_q": np.empty((n, L, I // 2), np.uint8),
        "gate_s": np.empty((n, I, L // 32), np.uint8),
        "up_s": np.empty((n, I, L // 32), np.uint8),
        "down_s": np.empty((n, L, I // 32), np.uint8),
    }

    def fill(slot: int) -> None:
        t = gen_expert(w, ids[slot])
        for key, arr in t.items():
            out[key][slot] = arr

    nthreads = threads or min(16, os.cpu_count() or 1)
    if n <= 2 or nthreads <= 1:
        for s in range(n):
            fill(s)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, range(n)))
    return out


def gen_shared(w: Workload) -> Dict[str, np.ndarray]:
    d = w.dims
    S, Is, L = d.S, d.Is, d.L
    g = _rng(w.seed, TID_SH_GATE).normal(0.0, w.shared_std, size=(S, Is, L))
    u = _rng(w.seed, TID_SH_UP).normal(0.0, w.shared_std, size=(S, Is, L))
    dn = _rng(w.seed, TID_SH_DOWN).normal(0.0, w.shared_std, size=(S, L, Is))
    return {
        "sh_gate": _normal_to_bf16_bits(g),
        "sh_up": _normal_to_bf16_bits(u),
        "sh_down": _normal_to_bf16_bits(dn),
    }


def gen_logits(w: Workload) -> np.ndarray:
    """Given router logits, float32 [T][E].

    l[t,e] = fp32(n[t,e] + b_e) with n ~ N(0,1) and a Zipf-shaped expert bias
    b_e = -s * ln(rank_e), ranks a seeded permutation of 1..E. A seeded
    tie_frac of the tokens then get tie_group distinct experts whose logits
    are all set to fp32(max_row + 1.0): an exact tie straddling the top-k
    boundary.
    """
    d = w.dims
    rng = _rng(w.seed, TID_LOGITS)
    ranks = rng.permutation(d.E) + 1
    bias = -w.zipf_s * np.log(ranks.astype(np.float64))
    n = rng.normal(0.0, 1.0, size=(d.T, d.E))
    lg = (n + bias[None, :]).astype(np.float32)
    n_tie = int(round(w.tie_frac * d.T))
    g = min(w.tie_group, d.E)
    if n_tie > 0 and g > 1:
        toks = rng.choice(d.T, size=n_tie, replace=False)
        for t in np.sort(toks):
            grp = rng.choice(d.E, size=g, replace=False)
            top = np.float64(lg[t].max())
            lg[t, grp] = np.float32(top + 1.0)
    return lg


def gen_all(w: Workload, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Every input of the layer for workload w (host arrays)."""
    out = {"x": gen_x(w), "router_w": gen_router(w)}
    out.update(gen_experts(w, threads=threads))
    out.update(gen_shared(w))
    if w.logits_given:
        out["logits"] = gen_logits(w)
    return out


def gen_block(w: Workload) -> Dict[str, np.ndarray]:
    """The MoE block's own inputs and weights (dims.H > 0); the routed
    experts come from gen_expert / gen_experts as for the layer."""
    d = w.dims
    T, H, L, E, S, Is = d.T, d.H, d.L, d.E, d.S, d.Is
    assert H > 0 and Is % 16 == 0
    u = _rng(w.seed, TID_U).normal(0.0, 1.0, size=(T, H))
    res = _rng(w.seed, TID_RESIDUAL).normal(0.0, 1.0, size=(T, H))
    rows = [_rng(w.seed, TID_W_IN, 0).normal(0.0, w.router_std, size=(E, H)),
            _rng(w.seed, TID_W_IN, 1).normal(0.0, 1.0 / np.sqrt(H), size=(L, H))]
    for s in range(S):
        g = _rng(w.seed, TID_W_IN, 2 + 2 * s).normal(0.0, w.shared_std, size=(Is, H))
        v = _rng(w.seed, TID_W_IN, 3 + 2 * s).normal(0.0, w.shared_std, size=(Is, H))
        # 16 gate rows, then the 16 up rows of the same columns
        rows.append(np.stack([g.reshape(Is // 16, 16, H), v.reshape(Is // 16, 16, H)],
                             axis=1).reshape(2 * Is, H))
    w_in = np.concatenate(rows, axis=0)
    return {
        "u": _normal_to_bf16_bits(u),
        "residual": _normal_to_bf16_bits(res),
        "w_in": _normal_to_bf16_bits(w_in),
        "norm_w": _normal_to_bf16_bits(_rng(w.seed, TID_NORM_W).normal(1.0, 0.1, size=L)),
        "w_up": _normal_to_bf16_bits(
            _rng(w.seed, TID_W_UP).normal(0.0, 1.0 / np.sqrt(L), size=(H, L))),
        "w_sd": _normal_to_bf16_bits(
            _rng(w.seed, TID_W_SD).normal(0.0, w.shared_std, size=(H, S * Is))),
    }

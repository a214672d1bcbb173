"""GPU parity of the MoE block around the layer (TokenSpeed sections 4.2-4.4
and 6) through the C ABI: lmoe_moe_input, lmoe_moe_tail and
lmoe_block_forward against the oracle's moe_input, moe_tail and
block_forward.

Bounds, all derived from the arithmetic:
  - router scores (fp32 outputs of the input GEMM): within the fp32 summation
    bound (H + 2) 2^-24 sum |u w| of the exact value, whatever the order the
    K splits and MFMA tiles add in;
  - bf16 outputs of a GEMM (latent rows, shared activations): a bf16
    rounding of some value within the kernel's evaluation error of the exact
    one, so bit-equal to the exact value rounded unless that error reaches a
    rounding midpoint;
  - the tail's output: half a bf16 ulp for its rounding, the fp32 summation
    bound of the up-projection, and one ulp of every normalised element or
    shared partial whose rounding may have gone the other way (their evaluation
    error reaches a midpoint), carried through the up-projection;
  - the whole block: the tail's bound on the oracle's intermediates plus the
    layer's 1e-2 rms carried through the normalisation, and an rms error
    below 3e-3, with the routing the GPU took checked bit for bit against the
    oracle's routing steps on the GPU's own router scores.
"""
import numpy as np
import pytest

import oracle as O
from workloads import get_workload, gen_block, gen_experts

from lmoe_testutil import (log, to_dev, alloc_routing, logits_bound,
                           check_routing_exact, check_routing_against_oracle)

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
EXPERT_KEYS = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")


@pytest.fixture(scope="module")
def lm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mxfp4_latent_mixture_amd as lm
    return lm


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


def _ulp(v):
    """bf16 spacing at |v| (the normal range)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def _bits_np(t):
    return t.cpu().numpy().view(np.uint16)


def check_bf16_rounding(got_bits, ref64, err, what):
    """got is a bf16 rounding of some value within err of the exact ref64:
    bf16(ref64 - err) <= got <= bf16(ref64 + err) (rounding is monotone), so
    it equals bf16(ref64) unless the evaluation error reaches a rounding
    midpoint. Returns how many differ from bf16(ref64)."""
    want = O.bf16_from_f64(ref64)
    diff = got_bits != want
    n = int(diff.sum())
    if n:
        g = O.f64_from_bf16(got_bits[diff])
        lo = O.f64_from_bf16(O.bf16_from_f64(ref64[diff] - err[diff]))
        hi = O.f64_from_bf16(O.bf16_from_f64(ref64[diff] + err[diff]))
        bad = ~((g >= lo) & (g <= hi))
        assert not bad.any(), (
            f"{what}: {int(bad.sum())} of {diff.size} values outside the rounding of their "
            f"error interval; first got {g[bad][0]!r} exact {ref64[diff][bad][0]!r} "
            f"err bound {err[diff][bad][0]!r}")
    log(f"{what}: bf16 values exact on {diff.size - n}/{diff.size}, {n} within the evaluation "
        f"error of a rounding midpoint")
    return n


def _block_on_device(w, dev, inp):
    return {k: to_dev(inp[k], dev) for k in ("u", "residual", "w_in", "norm_w", "w_up", "w_sd")}


def run_input(lm, dev, w, binp, rows=None):
    """lmoe_moe_input on the GPU, checked against the oracle on every row or
    on `rows`."""
    import torch
    d = w.dims
    SI = d.S * d.Is
    db = _block_on_device(w, dev, binp)
    logits = torch.empty((d.T, d.E), dtype=torch.float32, device=dev)
    x = torch.empty((d.T, d.L), dtype=torch.int16, device=dev)
    h = torch.empty((d.T, max(SI, 1)), dtype=torch.int16, device=dev)
    ws = torch.zeros(lm.block_workspace_bytes(d), dtype=torch.uint8, device=dev)
    lm.moe_input(d, db["u"], db["w_in"], logits, x, h if SI else None, ws)
    torch.cuda.synchronize()
    rows = np.arange(d.T) if rows is None else np.asarray(rows)
    g_lg, g_x = logits.cpu().numpy()[rows], _bits_np(x)[rows]
    g_h = _bits_np(h)[rows][:, :SI]
    u = binp["u"][rows]
    ref = O.moe_input(u, binp["w_in"], d.E, d.L, d.S, d.Is)
    # the fp32 summation bound of every column, and the GLU's propagated one
    au, aw = np.abs(O.f64_from_bf16(u)), np.abs(O.f64_from_bf16(binp["w_in"]))
    s = au @ aw.T
    err = (d.H + 2) * U * s
    lb = logits_bound(u, binp["w_in"][:d.E])
    dl = np.abs(g_lg.astype(np.float64) - ref["logits"].astype(np.float64))
    assert np.all(dl <= lb), f"{w.name}: router scores beyond the fp32 bound"
    check_bf16_rounding(g_x, ref["z"][:, d.E:d.E + d.L], err[:, d.E:d.E + d.L],
                        f"{w.name} latent rows")
    if SI:
        gr, ur = O.shared_gate_up_rows(d.E, d.L, d.S, d.Is)
        g64 = np.concatenate([ref["z"][:, gr[s_]] for s_ in range(d.S)], axis=1)
        v64 = np.concatenate([ref["z"][:, ur[s_]] for s_ in range(d.S)], axis=1)
        dg = np.concatenate([err[:, gr[s_]] for s_ in range(d.S)], axis=1)
        dv = np.concatenate([err[:, ur[s_]] for s_ in range(d.S)], axis=1)
        with np.errstate(over="ignore", invalid="ignore"):
            sig = 1.0 / (1.0 + np.exp(-g64))
            silu = g64 * sig
            dsilu = sig * (1.0 + g64 * (1.0 - sig))
        hv = silu * v64
        herr = np.abs(dsilu * v64) * dg + np.abs(silu) * dv + 8 * U * np.abs(hv)
        check_bf16_rounding(g_h, hv, herr, f"{w.name} shared activations")
    return {"logits": logits, "x": x, "h": h, "ws": ws, "db": db}


def tail_bound(routed, h, gamma, w_up, w_sd, resid, ref):
    """Per-element bound on |gpu - out64| for the tail (see the module
    docstring)."""
    T, L = routed.shape
    r = O.f64_from_bf16(routed)
    wu = np.abs(O.f64_from_bf16(w_up))
    n = O.f64_from_bf16(ref["n"])
    # normalised elements: exact value, its fp32 evaluation error (sum of L
    # squares, mean, sqrt, reciprocal, two products), and flips
    ms = np.mean(r * r, axis=1, keepdims=True)
    n64 = r / np.sqrt(ms + 1e-6) * O.f64_from_bf16(gamma)[None, :]
    nerr = (L + 16) * U * np.abs(n64)
    mid_n = np.abs(np.abs(n64 - n) - _ulp(n64) / 2) <= nerr
    allow = (np.where(mid_n, _ulp(n64), 0.0)) @ wu.T
    sh = O.f64_from_bf16(ref["sh"])
    if h.shape[1]:
        sh64 = O.f64_from_bf16(h) @ O.f64_from_bf16(w_sd).T
        sherr = (h.shape[1] + 2) * U * (np.abs(O.f64_from_bf16(h)) @ np.abs(O.f64_from_bf16(w_sd)).T)
        mid_s = np.abs(np.abs(sh64 - sh) - _ulp(sh64) / 2) <= sherr
        allow = allow + np.where(mid_s, _ulp(sh64), 0.0)
    acc = np.abs(n) @ wu.T
    res = np.abs(O.f64_from_bf16(resid))
    base = (L + 2) * U * acc + 4 * U * (acc + np.abs(sh) + res)
    return _ulp(ref["out64"]) / 2 + base + allow


def run_tail(lm, dev, w, binp, rng, rows=None):
    import torch
    d = w.dims
    SI = d.S * d.Is
    routed = O.bf16_from_f64(rng.normal(0.0, 0.3, size=(d.T, d.L)))
    h = O.bf16_from_f64(rng.normal(0.0, 1.0, size=(d.T, SI)))
    db = _block_on_device(w, dev, binp)
    out = torch.empty((d.T, d.H), dtype=torch.int16, device=dev)
    ws = torch.zeros(lm.block_workspace_bytes(d), dtype=torch.uint8, device=dev)
    lm.moe_tail(d, to_dev(routed, dev), to_dev(h, dev) if SI else None, db["norm_w"], db["w_up"],
                db["w_sd"] if SI else None, db["residual"], out, ws)
    torch.cuda.synchronize()
    rows = np.arange(d.T) if rows is None else np.asarray(rows)
    got = O.f64_from_bf16(_bits_np(out)[rows])
    ref = O.moe_tail(routed[rows], h[rows], binp["norm_w"], binp["w_up"], binp["w_sd"],
                     binp["residual"][rows])
    bound = tail_bound(routed[rows], h[rows], binp["norm_w"], binp["w_up"], binp["w_sd"],
                       binp["residual"][rows], ref)
    err = np.abs(got - ref["out64"])
    rms = float(np.sqrt(np.mean(ref["out64"] ** 2)))
    bad = np.nonzero(~(err <= bound))
    log(f"{w.name} tail: max|err|/rms={err.max() / rms:.3e}, "
        f"rms(err)/rms={np.sqrt(np.mean(err ** 2)) / rms:.3e}, max err/bound "
        f"{np.max(err / bound):.3f}")
    assert bad[0].size == 0, (f"{w.name} tail: {bad[0].size} outputs out of bound, first at "
                              f"{tuple(b[0] for b in bad)}: got {got[bad][0]!r} "
                              f"ref {ref['out64'][bad][0]!r} bound {bound[bad][0]!r}")


SMALL = ["block_tiny", "block_ragged"]


@pytest.mark.parametrize("name", SMALL + ["block_decode", "block_batched"])
def test_moe_input_every_token(lm, dev, name):
    w = get_workload(name)
    run_input(lm, dev, w, gen_block(w))


def test_moe_input_prefill_sampled(lm, dev):
    w = get_workload("block_prefill")
    T = w.dims.T
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(T - 64, T),
                                     rng.choice(T, 128, replace=False)]))
    run_input(lm, dev, w, gen_block(w), rows)


@pytest.mark.parametrize("name", SMALL + ["block_decode", "block_batched"])
def test_moe_tail_every_token(lm, dev, name):
    w = get_workload(name)
    run_tail(lm, dev, w, gen_block(w), np.random.default_rng(7))


def test_moe_tail_prefill_sampled(lm, dev):
    w = get_workload("block_prefill")
    T = w.dims.T
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(T - 64, T),
                                     rng.choice(T, 128, replace=False)]))
    run_tail(lm, dev, w, gen_block(w), np.random.default_rng(9), rows)


@pytest.mark.parametrize("T", [65, 300, 600])
def test_input_and_tail_k3_ragged_tiles(lm, dev, T):
    """Token counts that take 64- and 128-row tiles with K splits and a
    ragged last row tile."""
    from dataclasses import replace
    w0 = get_workload("block_decode")
    w = replace(w0, name=f"block_k3_t{T}", dims=replace(w0.dims, T=T))
    b = gen_block(w)
    run_input(lm, dev, w, b)
    run_tail(lm, dev, w, b, np.random.default_rng(11))


def test_moe_tail_without_shared_experts(lm, dev):
    from dataclasses import replace
    w0 = get_workload("block_ragged")
    w = replace(w0, name="block_ragged_s0", dims=replace(w0.dims, S=0, Is=0))
    run_tail(lm, dev, w, gen_block(w), np.random.default_rng(10))


def run_block(lm, dev, w, experts_all=True):
    """lmoe_block_forward against the oracle on every token."""
    import torch
    d = w.dims
    binp = gen_block(w)
    db = _block_on_device(w, dev, binp)
    log(f"{w.name}: generating the routed experts (E={d.E})")
    ex = gen_experts(w)
    dex = {k: to_dev(ex[k], dev) for k in EXPERT_KEYS}
    if d.E > 64:
        del ex
    r = alloc_routing(d, dev)
    out = torch.empty((d.T, d.H), dtype=torch.int16, device=dev)
    ws = torch.zeros(lm.block_workspace_bytes(d), dtype=torch.uint8, device=dev)
    lm.block_forward(d, db["u"], db["residual"], db, dex, r, out, ws)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in r.items()}
    got = _bits_np(out)
    del dex
    torch.cuda.empty_cache()
    # routing: the GPU scores against the oracle's, then the oracle's routing
    # steps on the GPU's own scores bit for bit
    ref_in = O.moe_input(binp["u"], binp["w_in"], d.E, d.L, d.S, d.Is)
    check_routing_against_oracle(res["topk_idx"], res["logits"], ref_in["logits"],
                                 logits_bound(binp["u"], binp["w_in"][:d.E]), d.k, w.name)
    check_routing_exact(res, res["logits"], d.k, f"{w.name} (on the GPU scores)")
    if d.E > 64:
        used = np.unique(res["topk_idx"])
        sub = gen_experts(w, used)
        full = {k: np.zeros((d.E,) + sub[k].shape[1:], np.uint8) for k in EXPERT_KEYS}
        for k in EXPERT_KEYS:
            full[k][used] = sub[k]
        ex = full
    ref = O.block_forward(binp["u"], binp["residual"], binp["w_in"], ex, binp["norm_w"],
                          binp["w_up"], binp["w_sd"], d.E, d.L, d.S, d.Is, d.k,
                          logits=res["logits"])
    # the tail's own bound on the oracle's intermediates, plus the layer's
    # 1e-2 rms carried through the normalisation (its gain 1 / rms(routed)
    # times the up-projection's row norm is about one on the workloads)
    o64 = ref["out64"]
    rms = float(np.sqrt(np.mean(o64 ** 2)))
    bound = tail_bound(ref["routed"]["out"], ref["input"]["h"], binp["norm_w"], binp["w_up"],
                       binp["w_sd"], binp["residual"], ref["tail"]) + 1e-2 * rms
    g64 = O.f64_from_bf16(got)
    err = np.abs(g64 - o64)
    rel_rms = float(np.sqrt(np.mean(err ** 2)) / rms)
    bad = np.nonzero(~(err <= bound))
    log(f"{w.name} block T={d.T}: max|err|/rms={err.max() / rms:.3e} rms(err)/rms={rel_rms:.3e} "
        f"max err/bound {np.max(err / bound):.3f}")
    assert bad[0].size == 0, (f"{w.name} block: {bad[0].size} outputs out of bound, first at "
                              f"{tuple(b[0] for b in bad)}: got {g64[bad][0]!r} "
                              f"ref {o64[bad][0]!r} bound {bound[bad][0]!r}")
    assert rel_rms < 3e-3, f"{w.name} block: rms error {rel_rms:.3e}"


@pytest.mark.parametrize("name", SMALL)
def test_block_forward_small(lm, dev, name):
    run_block(lm, dev, get_workload(name))


def test_block_forward_k3_decode(lm, dev):
    run_block(lm, dev, get_workload("block_decode"))


def test_block_forward_k3_width_few_experts(lm, dev):
    """The K3 widths (H = 7168, L = 3584, I = Is = 2048) with 64 experts, so
    the oracle runs every token; 300 tokens put several row tiles in the
    dense GEMMs and groups of about 75 routes per expert."""
    from dataclasses import replace
    w0 = get_workload("block_decode")
    w = replace(w0, name="block_k3w", dims=replace(w0.dims, T=300, E=64, k=16))
    run_block(lm, dev, w)

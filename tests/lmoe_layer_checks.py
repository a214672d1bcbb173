"""Whole-layer parity checks shared by the GPU test files: one call through
the C ABI (row-major experts with lmoe_forward, or tile-packed experts with
lmoe_pack_weights + lmoe_forward_packed) against the float64 oracle.

Routing: with given logits the oracle's selection, weights and grouping must
match bit for bit (weights within the derived softmax bound); with computed
logits the GPU logits must lie within the fp32 summation bound of the oracle's,
the oracle's routing steps applied to the GPU's own logits must reproduce the
GPU's routing bit for bit, and the selected sets must agree wherever the
boundary gap is clear. Outputs: within 1e-2 * rms + half a bf16 ulp of the
oracle run on the routing the GPU took, plus the h-rounding allowance where
that alone fails (lmoe_testutil)."""
from __future__ import annotations

import numpy as np

import oracle as O
from workloads import gen_all, gen_expert
from workloads.configs import Workload

from lmoe_testutil import (log, upload, alloc_routing, run_forward, check_out, logits_bound,
                           check_routing_against_oracle, check_routing_exact, flip_allowance_fn)

EXPERT_KEYS = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")


def full_small(lm, dev, w: Workload, packed: bool = False, act: str = "bf16"):
    """Every token of a layer small enough for the whole oracle (act: the
    routed experts' activation format, packed path only)."""
    d = w.dims
    inp = gen_all(w)
    dinp = upload(inp, dev)
    act_code = {"bf16": lm.ACT_BF16, "e4m3": lm.ACT_E4M3, "e2m1": lm.ACT_E2M1}[act]
    got, r = run_forward(lm, w, dinp, packed=packed, act=act_code)
    what = f"{w.name}{' packed' if packed else ''}{'' if act == 'bf16' else ' ' + act}"
    if w.logits_given:
        lg = inp["logits"]
        check_routing_exact(r, lg, d.k, what)
    else:
        ref_lg = O.router_logits(inp["x"], inp["router_w"])
        same = check_routing_against_oracle(r["topk_idx"], r["logits"], ref_lg,
                                            logits_bound(inp["x"], inp["router_w"]), d.k, what)
        assert same.mean() >= 0.9
        lg = r["logits"]
        check_routing_exact(r, lg, d.k, f"{what} (on the GPU logits)")
    ref = O.forward(inp["x"], None, inp, inp, d.k, logits=lg, act=act)
    get = lambda e: {key: inp[key][e] for key in EXPERT_KEYS}
    check_out(got, ref["out64"], f"{what} T={d.T}",
              allowance_fn=flip_allowance_fn(inp["x"], ref["idx"], ref["w"], get, inp, d.L, d.I,
                                             act=act))
    return got


def check_full_routing(w: Workload, inp, r):
    """Routing checks of a full-size call; returns the (idx, weights) the
    outputs are compared with and the mask of tokens whose sets agree with the
    oracle's own logits."""
    d = w.dims
    if w.logits_given:
        lg = inp["logits"]
        check_routing_exact(r, lg, d.k, w.name)
        same = np.ones(d.T, bool)
    else:
        log(f"{w.name}: oracle logits")
        ref_lg = O.router_logits(inp["x"], inp["router_w"])
        same = check_routing_against_oracle(r["topk_idx"], r["logits"], ref_lg,
                                            logits_bound(inp["x"], inp["router_w"]), d.k,
                                            w.name)
        assert same.mean() >= 0.99
        lg = r["logits"]
        check_routing_exact(r, lg, d.k, f"{w.name} (on the GPU logits)")
    idx = O.topk_select(lg, d.k)
    return idx, O.softmax_selected(lg, idx), same


def full_size(lm, dev, w: Workload, n_sample, packed: bool = False):
    """A full-size workload: routing on every token, outputs on sampled tokens
    (and one tied token when logits are given)."""
    import torch
    d = w.dims
    log(f"{w.name}: generating inputs (T={d.T}, E={d.E}, L={d.L}, I={d.I})")
    inp = gen_all(w)
    dinp = upload(inp, dev)
    for key in EXPERT_KEYS:
        del inp[key]                      # experts are regenerated per expert below
    log(f"{w.name}: running the layer{' (packed)' if packed else ''}")
    got, r = run_forward(lm, w, dinp, packed=packed)
    del dinp
    torch.cuda.empty_cache()
    idx, wts, same = check_full_routing(w, inp, r)
    rng = np.random.default_rng(99)
    cand = np.nonzero(same)[0]
    toks = list(rng.choice(cand, size=min(n_sample, cand.size), replace=False))
    if w.logits_given:
        tied = [t for t in cand if (inp["logits"][t] == inp["logits"][t].max()).sum() > d.k]
        toks = sorted(set(toks[: max(1, n_sample - 1)]) | {tied[0]})
    toks = sorted(int(t) for t in toks)
    log(f"{w.name}: oracle on tokens {toks}")
    get = lambda e: gen_expert(w, e)
    o64, _ = O.forward_tokens(inp["x"], idx, wts, get, inp, d.L, d.I, toks)
    check_out(got[toks], o64, f"{w.name} sampled tokens", rows=np.array(toks),
              allowance_fn=flip_allowance_fn(inp["x"], idx, wts, get, inp, d.L, d.I))


def every_token_isolated(lm, dev, w: Workload, packed: bool = False, path=None, act: str = "bf16"):
    """Every token at full size. The workload runs with its real router,
    routing and shapes, but every expert outside a kept set has all gate codes
    zero, so its routes give h = bf16(silu(0) u) = 0 and y = 0: each output is
    then the kept experts' weighted partials plus the shared experts, which the
    oracle computes for all T tokens at the cost of the kept experts alone.
    Kept: the hottest expert (every one of its tokens checked, over all of its
    row tiles), the coldest non-empty one, and ones whose groups just pass a
    96- and a 128-route row tile."""
    import torch
    d = w.dims
    log(f"{w.name}: generating inputs (T={d.T}, E={d.E}, L={d.L}, I={d.I})")
    inp = gen_all(w)
    dinp = upload(inp, dev)
    for key in EXPERT_KEYS:
        del inp[key]
    # routing first (it does not read the expert weights)
    r0 = alloc_routing(d, dev)
    if w.logits_given:
        r0["logits"] = dinp["logits"]
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    lm.route(d, dinp["x"], dinp["router_w"], w.logits_given, r0, ws)
    torch.cuda.synchronize()
    counts = r0["counts"].cpu().numpy()
    order = np.argsort(-counts, kind="stable")
    keep = {int(order[0]), int(order[np.nonzero(counts[order] > 0)[0][-1]])}
    for lo, hi in ((96, 120), (128, 160)):
        past = np.nonzero((counts > lo) & (counts <= hi))[0]
        if past.size:
            keep.add(int(past[0]))
    keep = sorted(keep)
    log(f"{w.name}: kept experts {keep} with {counts[keep].tolist()} routes")
    mask = torch.ones(d.E, dtype=torch.bool, device=dev)
    mask[keep] = False
    dinp["gate_q"].view(d.E, -1)[mask] = 0
    act_code = {"bf16": lm.ACT_BF16, "e4m3": lm.ACT_E4M3, "e2m1": lm.ACT_E2M1}[act]
    got, r = run_forward(lm, w, dinp, packed=packed, path=path, act=act_code)
    del dinp, ws
    torch.cuda.empty_cache()
    idx0 = r0["topk_idx"].cpu().numpy()
    if lm.path_name(d, w.logits_given) == "grouped" and path in (None, lm.PATH_GROUPED):
        assert np.array_equal(r["topk_idx"], idx0)
    else:
        # the fused decode kernels compute the logits in another order: the
        # kept set may differ on a near tie, never much
        assert (r["topk_idx"] == idx0).all(axis=1).mean() >= 0.9
    idx, wts, _ = check_full_routing(w, inp, r)
    x64 = O.f64_from_bf16(inp["x"])
    y = np.zeros((d.T, d.k, d.L), np.float64)
    for e in keep:
        ex = gen_expert(w, e)
        rows, slots = np.nonzero(idx == e)
        gate = O.dequant_mxfp4(ex["gate_q"], ex["gate_s"], d.I, d.L)
        up = O.dequant_mxfp4(ex["up_q"], ex["up_s"], d.I, d.L)
        down = O.dequant_mxfp4(ex["down_q"], ex["down_s"], d.L, d.I)
        _, y[rows, slots] = O.glu_ffn(x64[rows], gate, up, down, act)
    ysh = np.stack([O.glu_ffn(x64, O.f64_from_bf16(inp["sh_gate"][s]),
                              O.f64_from_bf16(inp["sh_up"][s]),
                              O.f64_from_bf16(inp["sh_down"][s]))[1] for s in range(d.S)])
    o64, _ = O.combine(y, wts, ysh)
    del y
    check_out(got, o64, f"{w.name}{' packed' if packed else ''}"
              f"{'' if act == 'bf16' else ' ' + act} every token ({len(keep)} experts kept)",
              allowance_fn=flip_allowance_fn(inp["x"], idx, wts, lambda e: gen_expert(w, e), inp,
                                             d.L, d.I, experts=set(keep), act=act))

"""GPU parity of the single-token decode path (one persistent kernel) against
the CPU oracle, including its dependency counters being left at zero and
back-to-back calls reusing one workspace."""
import numpy as np
import pytest

import oracle as O
from workloads import gen_all, gen_x, get_workload
from workloads.configs import Dims, Workload

from lmoe_testutil import (log, upload, alloc_routing, check_out, logits_bound,
                           check_routing_against_oracle, check_routing_exact,
                           flip_allowance_fn)

pytestmark = pytest.mark.gpu

CTR_BYTES = 256 << 10  # LMOE_COUNTER_BYTES
ERROR_SLOT = 1040  # int32 slot of the abandoned-wait count


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


def _expert(inp, e):
    return {key: inp[key][e] for key in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")}


def _run_tokens(lm, dev, w: Workload, n_tokens: int):
    """n_tokens consecutive T=1 calls on one zero-filled workspace; each output
    checked against the oracle; the counter block must be all zero after."""
    import torch
    d = w.dims
    assert d.T == 1
    assert lm.path_name(d) == "fused_decode"
    inp = gen_all(w)
    dinp = upload(inp, dev)
    xs = gen_x(w.with_T(n_tokens))
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    for t in range(n_tokens):
        x = torch.from_numpy(xs[t:t + 1].view(np.int16).copy()).to(dev)
        r = alloc_routing(d, dev)
        out = torch.empty((1, d.L), dtype=torch.int16, device=dev)
        lm.forward(d, x, dinp, False, r, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint16)
        res = {k: v.cpu().numpy() for k, v in r.items()}
        ref_lg = O.router_logits(xs[t:t + 1], inp["router_w"])
        check_routing_against_oracle(res["topk_idx"], res["logits"], ref_lg,
                                     logits_bound(xs[t:t + 1], inp["router_w"]), d.k,
                                     f"{w.name} token {t}")
        # the oracle's routing on the GPU's own logits: bit-exact, and the
        # output against the oracle on that routing
        check_routing_exact(res, res["logits"], d.k, f"{w.name} token {t} (GPU logits)")
        ref = O.forward(xs[t:t + 1], None, inp, inp, d.k, logits=res["logits"])
        check_out(got, ref["out64"], f"{w.name} token {t}",
                  allowance_fn=flip_allowance_fn(xs[t:t + 1], ref["idx"], ref["w"],
                                                 lambda e: _expert(inp, e), inp, d.L, d.I))
    ctr = ws[:CTR_BYTES].view(torch.int32).cpu().numpy()
    assert ctr[ERROR_SLOT] == 0, "a dependency wait timed out"
    assert not ctr.any(), f"counters left non-zero at {np.nonzero(ctr)[0][:8]}"
    # the same count through the C ABI's readout
    count = torch.full((1,), -1, dtype=torch.int32, device=dev)
    lm.wait_errors(ws, count)
    torch.cuda.synchronize()
    assert int(count.item()) == 0


@pytest.mark.parametrize("name,dims,scales", [
    ("tiny1", Dims(T=1, L=256, E=32, k=4, I=128, S=2, Is=128), ("uniform", 120, 130)),
    ("ragged1", Dims(T=1, L=416, E=48, k=6, I=352, S=2, Is=224), ("uniform", 118, 132)),
    ("odd_experts", Dims(T=1, L=544, E=37, k=5, I=160, S=1, Is=96), ("uniform", 118, 132)),
    ("no_shared", Dims(T=1, L=320, E=64, k=8, I=256, S=0, Is=0), ("uniform", 118, 132)),
    ("k1", Dims(T=1, L=256, E=16, k=1, I=64, S=3, Is=64), ("uniform", 118, 132)),
    ("wide_k", Dims(T=1, L=288, E=1024, k=32, I=96, S=1, Is=4096), ("uniform", 118, 132)),
    ("many_shared", Dims(T=1, L=320, E=40, k=4, I=160, S=3, Is=1600), ("uniform", 118, 132)),
])
def test_fused_decode_shapes(lm, dev, name, dims, scales):
    _run_tokens(lm, dev, Workload(name, 40 + len(name), dims, scales=scales), 3)


def _tied_router(inp, d):
    """Router rows with exact logit ties: groups of four identical rows, the
    strongest row copied onto experts 5, 69, 133 and 197 (one lane of the
    selecting wave holds all four), a NaN row and an all-zero row."""
    wr = inp["router_w"].copy()
    for g in range(8, 48, 4):
        wr[g + 1:g + 4] = wr[g]
    top = int(np.argmax(O.router_logits(inp["x"], wr)[0]))
    for e in (5, 69, 133, 197):
        wr[e] = wr[top]
    wr[50] = 0x7FC0                    # bf16 NaN: logit NaN
    wr[51] = 0                         # logit +0
    return wr


def test_fused_decode_router_ties_and_nan(lm, dev):
    """Selection inside the fused kernel on exact logit ties (lower expert
    index first), one lane winning four times, a NaN logit (ordered after
    every number) and an all-zero row (logit +0); the oracle decides."""
    import torch
    d = Dims(T=1, L=256, E=256, k=10, I=128, S=1, Is=64)
    w = Workload("ties1", 61, d, scales=("uniform", 118, 132))
    inp = gen_all(w)
    wr = _tied_router(inp, d)
    inp["router_w"] = wr
    dinp = upload(inp, dev)
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    r = alloc_routing(d, dev)
    out = torch.empty((1, d.L), dtype=torch.int16, device=dev)
    lm.forward(d, dinp["x"], dinp, False, r, out, ws)
    torch.cuda.synchronize()
    ref = O.forward(inp["x"], wr, inp, inp, d.k)
    assert {5, 69, 133, 197} <= set(ref["idx"][0].tolist())
    res = {k: v.cpu().numpy() for k, v in r.items()}
    lg = res["logits"][0]
    assert np.isnan(lg[50]) and lg[51] == 0.0
    for r0 in (1, 2, 3):                                 # the ties are exact on the GPU
        assert np.array_equal(lg[8 + r0:48:4], lg[8:48:4])
    assert lg[5] == lg[69] == lg[133] == lg[197]
    assert np.array_equal(res["topk_idx"], ref["idx"])
    check_routing_exact(res, lg[None, :], d.k, "ties1 (GPU logits)")
    check_out(out.cpu().numpy().view(np.uint16), ref["out64"], "ties1",
              allowance_fn=flip_allowance_fn(inp["x"], ref["idx"], ref["w"],
                                             lambda e: _expert(inp, e), inp, d.L, d.I))
    assert not ws[:CTR_BYTES].view(torch.int32).cpu().numpy().any()


def _crowded_router(inp, d):
    """Router rows that put the 128 largest logits on experts e with
    e % 64 < 32 (four per lane of the selecting wave), arranged so that lane
    31 holds the four smallest of them: the k-th largest lane maximum is then
    reached by 125 keys, more than the wave has lanes. Each such logit is one
    exact product: x[0] = 1 and the row's only nonzero entry is its first."""
    x = inp["x"].copy()
    x[0, 0] = 0x3F80                       # bf16 1.0
    wr = inp["router_w"].copy()
    lanes = [l for l in range(32) if l != 31] + [31]
    experts = [l + 64 * i for l in lanes for i in range(4)]
    for r, e in enumerate(experts):        # values 127.5, 127, ..., 64
        v = np.float32(128.0 - 0.5 * (r + 1))
        wr[e] = 0
        wr[e, 0] = np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16
    return x, wr


def test_fused_decode_router_crowded_lanes(lm, dev):
    """Selection when the largest logits crowd into a few lanes of the
    selecting wave (the threshold admits more keys than the wave has lanes);
    the oracle decides."""
    import torch
    d = Dims(T=1, L=256, E=256, k=32, I=128, S=1, Is=64)
    w = Workload("crowd1", 67, d, scales=("uniform", 118, 132))
    inp = gen_all(w)
    x, wr = _crowded_router(inp, d)
    inp["x"], inp["router_w"] = x, wr
    dinp = upload(inp, dev)
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    r = alloc_routing(d, dev)
    out = torch.empty((1, d.L), dtype=torch.int16, device=dev)
    lm.forward(d, dinp["x"], dinp, False, r, out, ws)
    torch.cuda.synchronize()
    ref = O.forward(x, wr, inp, inp, d.k)
    lg = O.router_logits(x, wr)[0]
    assert np.sum(lg >= 64.0) == 128 and np.max(np.delete(lg, np.flatnonzero(lg >= 64.0))) < 64.0
    res = {k: v.cpu().numpy() for k, v in r.items()}
    assert np.array_equal(res["topk_idx"], ref["idx"])
    check_routing_exact(res, res["logits"], d.k, "crowd1 (GPU logits)")
    check_out(out.cpu().numpy().view(np.uint16), ref["out64"], "crowd1",
              allowance_fn=flip_allowance_fn(x, ref["idx"], ref["w"],
                                             lambda e: _expert(inp, e), inp, d.L, d.I))
    assert not ws[:CTR_BYTES].view(torch.int32).cpu().numpy().any()


def test_fused_decode_k3_back_to_back(lm, dev):
    w = get_workload("decode")
    log("decode: 4 consecutive K3 tokens on one workspace")
    _run_tokens(lm, dev, w, 4)


@pytest.mark.parametrize("T", [1, 3, 16])
def test_given_logits_take_the_fused_kernels(lm, dev, T):
    """Given logits (ties straddling the top-k boundary, a NaN, -inf) on the
    one-kernel paths: the router items publish them instead of computing
    them. Routing bit-exact against the oracle's steps on the same logits,
    outputs against the oracle, counters zero after, the logits untouched."""
    import torch
    w = Workload(f"given{T}", 51, Dims(T=T, L=256, E=32, k=4, I=128, S=2, Is=128),
                 scales=("uniform", 120, 130), logits_given=True, tie_frac=0.5, tie_group=6)
    d = w.dims
    assert lm.path_name(d, True) == ("fused_decode" if T == 1 else "fused_multi")
    inp = gen_all(w)
    inp["logits"][0, 5] = np.nan
    inp["logits"][-1, 7] = -np.inf
    dinp = upload(inp, dev)
    r = alloc_routing(d, dev)
    r["logits"] = dinp["logits"]
    out = torch.empty((T, d.L), dtype=torch.int16, device=dev)
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    lm.forward(d, dinp["x"], dinp, True, r, out, ws)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in r.items()}
    assert np.array_equal(res["logits"].view(np.uint32), inp["logits"].view(np.uint32))
    check_routing_exact(res, inp["logits"], d.k, f"given logits T={T}")
    ref = O.forward(inp["x"], None, inp, inp, d.k, logits=inp["logits"])
    check_out(out.cpu().numpy().view(np.uint16), ref["out64"], f"given logits T={T}",
              allowance_fn=flip_allowance_fn(inp["x"], ref["idx"], ref["w"],
                                             lambda e: _expert(inp, e), inp, d.L, d.I))
    ctr = ws[:CTR_BYTES].view(torch.int32).cpu().numpy()
    assert not ctr.any(), f"counters left non-zero at {np.nonzero(ctr)[0][:8]}"

"""GPU parity of the 2..16-token decode path (one persistent kernel, one
token per MFMA row, the routes of all tokens grouped by expert inside the
launch) against the CPU oracle: the GPU logits within the fp32 summation
bound, the oracle's routing on the GPU's own logits bit for bit (indices,
counts, offsets, perm, inv_perm; weights within the derived softmax bound),
every token's output, the counter block left at zero and no abandoned wait,
and calls of different T back to back on one workspace."""
import numpy as np
import pytest

import oracle as O
from workloads import gen_all, gen_expert, gen_x, get_workload
from workloads.configs import Dims, Workload

from lmoe_testutil import (log, upload, alloc_routing, check_out, logits_bound,
                           check_routing_against_oracle, check_routing_exact,
                           flip_allowance_fn)
from lmoe_layer_checks import check_full_routing, every_token_isolated

pytestmark = pytest.mark.gpu

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


def _expert(inp, e):
    return {key: inp[key][e] for key in EXPERT_KEYS}


def _check_counters(lm, ws):
    """The counter block is all zero after a call, and no wait was abandoned
    (read through the C ABI)."""
    import torch
    n = lm.COUNTER_BYTES
    ctr = ws[:n].view(torch.int32).cpu().numpy()
    assert ctr[1040] == 0, "a dependency wait timed out"
    assert not ctr.any(), f"counters left non-zero at {np.nonzero(ctr)[0][:8]}"
    count = torch.full((1,), -1, dtype=torch.int32, device=ws.device)
    lm.wait_errors(ws, count)
    torch.cuda.synchronize()
    assert int(count.item()) == 0


def _call(lm, dev, d, x, dinp, ws, router_w=None):
    import torch
    r = alloc_routing(d, dev)
    out = torch.empty((d.T, d.L), dtype=torch.int16, device=dev)
    w = dinp if router_w is None else {**dinp, "router_w": router_w}
    lm.forward(d, x, w, False, r, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16), {k: v.cpu().numpy() for k, v in r.items()}


def _check_call(got, res, xs, inp, d, what, wr=None):
    """Routing and every token's output of one call against the oracle."""
    wr = inp["router_w"] if wr is None else wr
    ref_lg = O.router_logits(xs, wr)
    check_routing_against_oracle(res["topk_idx"], res["logits"], ref_lg,
                                 logits_bound(xs, wr), d.k, what)
    check_routing_exact(res, res["logits"], d.k, f"{what} (GPU logits)")
    ref = O.forward(xs, None, inp, inp, d.k, logits=res["logits"])
    check_out(got, ref["out64"], what,
              allowance_fn=flip_allowance_fn(xs, ref["idx"], ref["w"],
                                             lambda e: _expert(inp, e), inp, d.L, d.I))


SHAPES = [
    # every expert taken by several tokens (groups of up to 16 rows)
    ("tiny_t2", Dims(T=2, L=256, E=32, k=4, I=128, S=2, Is=128)),
    ("tiny_t16", Dims(T=16, L=256, E=32, k=4, I=128, S=2, Is=128)),
    ("dense_t16", Dims(T=16, L=320, E=20, k=16, I=96, S=1, Is=64)),
    # a ragged last output block (L % 64 == 32), odd expert count
    ("ragged_t5", Dims(T=5, L=416, E=48, k=6, I=352, S=2, Is=224)),
    ("odd_t7", Dims(T=7, L=544, E=37, k=5, I=160, S=1, Is=96)),
    ("no_shared_t9", Dims(T=9, L=320, E=64, k=8, I=256, S=0, Is=0)),
    ("k1_t13", Dims(T=13, L=256, E=16, k=1, I=64, S=3, Is=64)),
    # T * k at the limit of the grouping tables, E at its limit
    ("max_routes", Dims(T=8, L=288, E=1024, k=32, I=96, S=1, Is=4096)),
    # the widest tokens: the LDS holds 16 rows of 4096
    ("wide_t16", Dims(T=16, L=4096, E=40, k=16, I=512, S=1, Is=4096)),
]


@pytest.mark.parametrize("name,dims", SHAPES, ids=[s[0] for s in SHAPES])
def test_multi_decode_shapes(lm, dev, name, dims):
    import torch
    w = Workload(name, 70 + len(name), dims, scales=("uniform", 118, 132))
    d = w.dims
    assert lm.path_name(d) == "fused_multi"
    log(f"{name}: T={d.T} L={d.L} E={d.E} k={d.k} I={d.I} S={d.S} Is={d.Is}")
    inp = gen_all(w)
    dinp = upload(inp, dev)
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    got, res = _call(lm, dev, d, dinp["x"], dinp, ws)
    _check_call(got, res, inp["x"], inp, d, name)
    _check_counters(lm, ws)


def test_multi_decode_back_to_back(lm, dev):
    """T = 16, 3, 11, 2 on one workspace (each call must leave the counters
    as the next expects them), then the first call again: same bits."""
    import torch
    base = Dims(T=16, L=416, E=48, k=6, I=352, S=2, Is=224)
    w = Workload("b2b", 91, base, scales=("uniform", 118, 132))
    inp = gen_all(w)
    dinp = upload(inp, dev)
    xs = inp["x"]
    ws = torch.zeros(lm.workspace_bytes(base), dtype=torch.uint8, device=dev)
    first = None
    for T in (16, 3, 11, 2, 16):
        d = Dims(T=T, L=base.L, E=base.E, k=base.k, I=base.I, S=base.S, Is=base.Is)
        x = dinp["x"][:T].contiguous()
        got, res = _call(lm, dev, d, x, dinp, ws)
        if first is None:
            first = got
            _check_call(got, res, xs[:T], inp, d, f"b2b T={T}")
        elif T == 16:
            assert np.array_equal(got, first), "same call, different bits"
        else:
            _check_call(got, res, xs[:T], inp, d, f"b2b T={T}")
        _check_counters(lm, ws)


def test_multi_decode_router_ties_and_nan(lm, dev):
    """Exact logit ties (groups of identical router rows, the strongest row
    of token 0 copied onto four experts held by one lane of the selecting
    wave), a NaN row (ordered after every number) and an all-zero row (logit
    +0), for every token; the oracle's selection on the GPU logits decides."""
    import torch
    d = Dims(T=6, L=256, E=256, k=8, I=128, S=1, Is=128)
    w = Workload("ties_m", 93, d, scales=("uniform", 118, 132))
    inp = gen_all(w)
    wr = inp["router_w"].copy()
    for g in range(8, 48, 4):
        wr[g + 1:g + 4] = wr[g]
    top = int(np.argmax(O.router_logits(inp["x"], wr)[0]))
    for e in (5, 69, 133, 197):
        wr[e] = wr[top]
    wr[50] = 0x7FC0                    # bf16 NaN: logit NaN
    wr[51] = 0                         # logit +0
    inp["router_w"] = wr
    dinp = upload(inp, dev)
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    got, res = _call(lm, dev, d, dinp["x"], dinp, ws)
    lg = res["logits"]
    assert np.isnan(lg[:, 50]).all() and (lg[:, 51] == 0.0).all()
    for r0 in (1, 2, 3):                                 # the ties are exact on the GPU
        assert np.array_equal(lg[:, 8 + r0:48:4], lg[:, 8:48:4])
    assert (lg[:, 5] == lg[:, 69]).all() and (lg[:, 69] == lg[:, 133]).all()
    assert (lg[:, 133] == lg[:, 197]).all()
    ref = O.forward(inp["x"], None, inp, inp, d.k, logits=lg)
    assert {5, 69, 133, 197} <= set(ref["idx"][0].tolist())
    check_routing_exact(res, lg, d.k, "ties_m (GPU logits)")
    check_out(got, ref["out64"], "ties_m",
              allowance_fn=flip_allowance_fn(inp["x"], ref["idx"], ref["w"],
                                             lambda e: _expert(inp, e), inp, d.L, d.I))
    _check_counters(lm, ws)


def test_multi_decode_router_crowded_lanes(lm, dev):
    """Selection when the largest logits crowd into a few lanes of the
    selecting wave (the threshold admits more keys than the wave has lanes,
    and the round-by-round selection decides), for four tokens at once: each
    of those logits is one exact product (x[t][0] = 1, the row's only nonzero
    entry its first)."""
    import torch
    d = Dims(T=4, L=256, E=256, k=16, I=128, S=1, Is=64)
    w = Workload("crowd_m", 94, d, scales=("uniform", 118, 132))
    inp = gen_all(w)
    x = inp["x"].copy()
    x[:, 0] = 0x3F80
    wr = inp["router_w"].copy()
    lanes = [l for l in range(32) if l != 31] + [31]
    for r, e in enumerate(l + 64 * i for l in lanes for i in range(4)):
        v = np.float32(128.0 - 0.5 * (r + 1))
        wr[e] = 0
        wr[e, 0] = np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16
    inp["x"], inp["router_w"] = x, wr
    dinp = upload(inp, dev)
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    got, res = _call(lm, dev, d, dinp["x"], dinp, ws)
    lg = res["logits"]
    check_routing_exact(res, lg, d.k, "crowd_m (GPU logits)")
    ref = O.forward(x, None, inp, inp, d.k, logits=lg)
    assert np.array_equal(res["topk_idx"], ref["idx"])
    check_out(got, ref["out64"], "crowd_m",
              allowance_fn=flip_allowance_fn(x, ref["idx"], ref["w"],
                                             lambda e: _expert(inp, e), inp, d.L, d.I))
    _check_counters(lm, ws)


def test_multi_decode_path_limits(lm):
    """The fused multi-token kernel can run from 2 to 16 tokens while T * k
    <= 256 and the widths fit; lmoe_forward takes it while the weight stream
    of min(E, T k) experts stays under LMOE_FUSED_MULTI_BYTES (Kimi-K3: two
    and three tokens), the grouped path beyond."""
    K3 = (3584, 896, 16, 2048, 2, 2048)
    for T in (2, 3):
        assert lm.path_name((T,) + K3) == "fused_multi"
    for T in (4, 5, 16, 17):
        assert lm.path_name((T,) + K3) == "grouped"
    # given logits take the same paths: the router items publish them
    assert lm.path_name((2,) + K3, True) == "fused_multi"
    assert lm.path_name((16,) + K3, True) == "grouped"
    small = (256, 32, 4, 128, 2, 128)
    for T in (2, 9, 16):
        assert lm.path_name((T,) + small) == "fused_multi"
    assert lm.path_name((17,) + small) == "grouped"
    assert lm.path_name((9, 288, 1024, 32, 96, 1, 96)) == "grouped"      # T * k > 256
    assert lm.path_name((8, 288, 1024, 32, 96, 1, 96)) == "fused_multi"
    assert lm.path_name((2, 8192, 896, 16, 2048, 2, 2048)) == "grouped"  # L too wide
    assert lm.path_name((2, 3584, 896, 16, 4128, 2, 2048)) == "grouped"  # I too wide


@pytest.mark.parametrize("T", [2, 4])
def test_full_multi_decode(lm, dev, T):
    """K3 decode with T tokens in one call on the fused kernel (seed 1's first
    T tokens; T = 4 through lmoe_forward_ex's path choice): routing on every
    token, and every token's output with the real experts."""
    import torch
    w = get_workload("decode").with_T(T, f"decode_t{T}")
    d = w.dims
    assert lm.path_name(d) == ("fused_multi" if T == 2 else "grouped")
    log(f"{w.name}: generating inputs")
    inp = gen_all(w)
    dinp = upload(inp, dev)
    for key in EXPERT_KEYS:
        del inp[key]
    r = alloc_routing(d, dev)
    out = torch.empty((d.T, d.L), dtype=torch.int16, device=dev)
    ws = torch.zeros(lm.workspace_bytes(d), dtype=torch.uint8, device=dev)
    lm.forward_ex(d, dinp["x"], dinp, False, r, out, ws, path=lm.PATH_FUSED)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    res = {k: v.cpu().numpy() for k, v in r.items()}
    _check_counters(lm, ws)
    del dinp, ws
    torch.cuda.empty_cache()
    idx, wts, _ = check_full_routing(w, inp, res)
    toks = list(range(d.T))
    log(f"{w.name}: oracle on every token ({len(np.unique(idx))} experts)")
    get = lambda e: gen_expert(w, e)
    o64, _ = O.forward_tokens(inp["x"], idx, wts, get, inp, d.L, d.I, toks)
    check_out(got, o64, f"{w.name} every token", rows=np.array(toks),
              allowance_fn=flip_allowance_fn(inp["x"], idx, wts, get, inp, d.L, d.I))


@pytest.mark.parametrize("T", [8, 16])
def test_full_multi_decode_every_token_isolated(lm, dev, T):
    """K3 decode with 8 and 16 tokens on the fused kernel (chosen through
    lmoe_forward_ex): every token's output with all but a few experts
    silenced (their gate codes zero), so the oracle covers every token at
    the cost of the kept experts."""
    w = get_workload("decode").with_T(T, f"decode_t{T}")
    every_token_isolated(lm, dev, w, path=lm.PATH_FUSED)
